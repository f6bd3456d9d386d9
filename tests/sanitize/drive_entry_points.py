"""Drives every device entry point of the host-only sanitizer build of the
library (kernel launchers replaced by tests/sanitize/launch_stub.cpp) with
host buffers of exactly the documented sizes, allocated one by one so that
AddressSanitizer sees each buffer's end.  The stub launchers touch every
region the kernels would read or write; an entry point that hands a launcher
a region past its buffer, or two overlapping regions, fails the run.

Run by tests/test_host_sanitized.py in a process with the sanitizer runtime
preloaded and AREA_LIBRARY pointing at the sanitized library."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.modules["torch"] = None  # the host library needs no torch; keep it out of this process

import resolution_diffusion_transformer_amd as A  # noqa: E402
import workloads as W  # noqa: E402

libc = ctypes.CDLL(None)
libc.posix_memalign.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_size_t]
libc.free.argtypes = [ctypes.c_void_p]
live = []


def alloc(nbytes):
    """nbytes of host memory, 256-byte aligned, ending exactly at its size."""
    ptr = ctypes.c_void_p()
    assert libc.posix_memalign(ctypes.byref(ptr), 256, max(int(nbytes), 1)) == 0
    ctypes.memset(ptr, 0, max(int(nbytes), 1))
    live.append(ptr.value)
    return ptr.value


def release():
    while live:
        libc.free(live.pop())


def ok(rc, what):
    if rc != 0:
        raise SystemExit(f"{what}: status {rc}: {A.lib().area_last_error().decode()}")


def drive(name, p):
    L = A.lib()
    c = p.c()
    ref = ctypes.byref(c)
    ok(L.area_validate(ref), f"{name} validate")
    B, H, D, T, N = p.B, p.H, p.D, p.T, p.Gh * p.Gw
    seq = B * H * (T + N) * D * 2
    q, k, v, out = alloc(seq), alloc(seq), alloc(seq), alloc(seq)
    C = 16
    lat = alloc(C * N * 4)
    E, Eq = alloc(N // 4 * 4), alloc(N // 4 * 4)
    steps = p.p1_steps + p.p2_steps
    infos = [A.area_step_info(p, s) for s in range(steps)]
    # full attention and the text pass
    nf = L.area_workspace_bytes(ref, A.OP_FULL)
    ok(L.area_full_attn(ref, q, k, v, out, alloc(nf), nf, None), f"{name} full")
    ok(L.area_text_attn(ref, q, k, v, out, alloc(nf), nf, None), f"{name} text")
    # Phase I: every pooling factor of the ramp, and f = 1
    nc = L.area_workspace_bytes(ref, A.OP_COARSE)
    for f in sorted({st["f"] for st in infos if st["phase"] == A.PHASE_COARSE} | {1}):
        M = T + (p.Gh // f) * (p.Gw // f)
        kp, vp = alloc(B * H * M * D * 4), alloc(B * H * M * D * 4)
        ok(L.area_pool_kv(ref, f, k, v, kp, vp, None), f"{name} pool f={f}")
        ok(L.area_coarse_attn(ref, f, q, kp, vp, out, alloc(nc), nc, None), f"{name} coarse f={f}")
    # Phase II: map, plan, bridge and windowed attention of every window step
    ok(L.area_dwt_detail(ref, C, lat, E, Eq, None), f"{name} dwt")
    words = L.area_plan_words(ref)
    npl, nw = L.area_workspace_bytes(ref, A.OP_PLAN), L.area_workspace_bytes(ref, A.OP_WINDOW)
    for s, st in enumerate(infos):
        if st["phase"] != A.PHASE_WINDOW:
            continue
        plan, wsum = alloc(words * 4), alloc(N * 4)
        br = alloc(B * H * st["R"] * 4) if st["R"] > 0 else None
        ok(L.area_window_plan(ref, s, Eq, k, plan, wsum, br, alloc(npl), npl, None), f"{name} plan step {s}")
        ok(L.area_window_attn(ref, s, plan, wsum, br, q, k, v, out, alloc(nw), nw, None), f"{name} window step {s}")
    # the per-step driver over the whole schedule, one workspace
    ns = L.area_workspace_bytes(ref, A.OP_STEP)
    ws = alloc(ns)
    for s in range(steps):
        ok(L.area_attn_step(ref, s, C, lat, q, k, v, out, ws, ns, None), f"{name} step {s}")
        ok(L.area_attn_step(ref, s, 0, None, q, k, v, out, ws, ns, None), f"{name} step {s} without latent")
    release()
    print(f"[sanitize] {name}: {steps} steps, every entry point ok", flush=True)


def main():
    cases = [(n, A.problem_for(W.get(n))) for n in ("tiny-32", "tiny-32-text", "flux-2048")]
    cases.append(("tiny-32 pages' knobs", A.problem_for(W.get("tiny-32"), **W.PAGES_KNOBS)))
    cases.append(("96x64 native 20, pages' knobs",
                  A.Problem(B=1, H=2, D=64, Gh=96, Gw=64, native_h=20, native_w=20, p1_steps=4, p2_steps=5,
                            w_start=0, w_min=8, halo=0, halo_max=8, bridge_rho_num=1, bridge_rho_den=2, seed=3)))
    cases.append(("30x34 batch 2, text", A.Problem(B=2, H=3, D=128, Gh=30, Gw=34, native_h=15, native_w=17, T=5,
                                                    p1_steps=2, p2_steps=3, w_start=16, w_min=8, halo=2,
                                                    bridge_k=12, seed=9)))
    cases.append(("gated 64x64", A.Problem(B=1, H=2, D=128, Gh=64, Gw=64, native_h=64, native_w=64, p1_steps=2,
                                           p2_steps=2, w_start=32, w_min=16)))
    for name, p in cases:
        drive(name, p)
    print("[sanitize] all entry points ok", flush=True)


if __name__ == "__main__":
    main()
