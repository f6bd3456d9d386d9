"""Benchmark of the AReA attention path on one MI355X.

One bench step is one pass of the whole hot path for one attention layer of
the FLUX.1-shaped 6144x6144 workload (384x384 tokens, 24 heads, head dim
128): every denoising step of the schedule -- 8 coarse steps (pool + coarse
attention over the pooling ramp) and 20 window steps (Haar map, window plan
with bridge, windowed attention with blending) -- plus one uniform full
attention call at the same shape, the baseline of the speedup.

The reported value is AReA attention milliseconds per denoising step (the
schedule's time divided by its 28 steps), timed over K bench steps after W
warm-up steps with inputs already resident in HBM.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--ablation]

--ablation prints, instead of the bench line, the schedule's time with the
quadrant splits, the Halo or the bridge turned off, at a fixed smallest
window, and at the pages' own knob values (first window from the cost rule,
seeded Halo widths up to 8, bridge of (w/2)^2 tokens), each against the same
full-attention baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AReA attn ms/step + % bf16 MFMA peak, FLUX-shape 6144²; speedup vs full attn"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def new(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        self.pool.append(ev.value)
        return ev.value

    def elapsed(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)


class Schedule:
    """One problem's buffers, algorithmic work and timed pass over the whole
    schedule (coarse steps, window steps and optionally one full call)."""

    def __init__(self, A, wl, p, q, k, v, lat, out, ev):
        import torch
        self.A, self.wl, self.p, self.q, self.k, self.v, self.lat, self.out, self.ev = A, wl, p, q, k, v, lat, out, ev
        A.area_validate(p)
        dev = q.device
        B, H, N, D = p.B, p.H, p.N, p.D
        ws_bytes = max(A.area_workspace_bytes(p, op) for op in (A.OP_FULL, A.OP_COARSE, A.OP_PLAN, A.OP_WINDOW))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.plan = torch.zeros(A.area_plan_words(p), dtype=torch.int32, device=dev)
        self.wsum = torch.empty(N, dtype=torch.int32, device=dev)
        self.n_steps = p.p1_steps + p.p2_steps
        self.sched = [A.area_step_info(p, s) for s in range(self.n_steps)]
        r_max = max([st["R"] for st in self.sched] + [0])
        self.bridge_buf = torch.empty(B * H * r_max, dtype=torch.int32, device=dev) if r_max > 0 else None
        self.energy = torch.empty((p.Gh // 2, p.Gw // 2), dtype=torch.float32, device=dev)
        self.energy_q = torch.empty((p.Gh // 2, p.Gw // 2), dtype=torch.int32, device=dev)
        fs = sorted({st["f"] for st in self.sched if st["phase"] == A.PHASE_COARSE})
        self.kpv = {f: (torch.empty((B, H, N // (f * f), D), dtype=torch.float32, device=dev),
                        torch.empty((B, H, N // (f * f), D), dtype=torch.float32, device=dev)) for f in fs}

    def bridge(self, s):
        """The step's bridge-index view [B, H, R_s] of the shared buffer (None without a bridge)."""
        R = self.sched[s]["R"]
        if R == 0 or self.bridge_buf is None:
            return None
        return self.bridge_buf[:self.p.B * self.p.H * R].view(self.p.B, self.p.H, R)

    @staticmethod
    def _tev():
        import torch
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def window_plan(self, s):
        A, p = self.A, self.p
        A.area_dwt_detail(p, self.lat, self.energy, self.energy_q)
        A.area_window_plan(p, s, self.energy_q, self.k, self.plan, self.wsum, self.bridge(s), self.ws)

    def one_pass(self, rec, full=True):
        """Enqueue the whole hot path once; rec collects (kind, step, events)."""
        A, p, ev, tev = self.A, self.p, self.ev, self._tev
        for s, st in enumerate(self.sched):
            if st["phase"] == A.PHASE_COARSE:
                f = st["f"]
                kp, vp = self.kpv[f]
                e0 = tev()
                A.area_pool_kv(p, f, self.k, self.v, kp, vp)
                e1 = tev()
                a0, a1 = ev.new(), ev.new()
                A.area_set_attn_events(a0, a1)
                A.area_coarse_attn(p, f, self.q, kp, vp, self.out, self.ws)
                A.area_set_attn_events(None, None)
                e2 = tev()
                rec.append(("coarse", s, (e0, e1, e2, a0, a1)))
            else:
                e0 = tev()
                A.area_dwt_detail(p, self.lat, self.energy, self.energy_q)
                e1 = tev()
                br = self.bridge(s)
                A.area_window_plan(p, s, self.energy_q, self.k, self.plan, self.wsum, br, self.ws)
                e2 = tev()
                a0, a1 = ev.new(), ev.new()
                A.area_set_attn_events(a0, a1)
                A.area_window_attn(p, s, self.plan, self.wsum, br, self.q, self.k, self.v, self.out, self.ws)
                A.area_set_attn_events(None, None)
                e3 = tev()
                rec.append(("window", s, (e0, e1, e2, e3, a0, a1)))
        if full:
            e0 = tev()
            a0, a1 = ev.new(), ev.new()
            A.area_set_attn_events(a0, a1)
            A.area_full_attn(p, self.q, self.k, self.v, self.out, self.ws)
            A.area_set_attn_events(None, None)
            e1 = tev()
            rec.append(("full", -1, (e0, e1, a0, a1)))

    def count(self):
        """Algorithmic FLOPs per step (deterministic: plans depend only on the
        inputs) and the (query, key) pairs of every window step."""
        A, p = self.A, self.p
        D, BH, N, Gw = p.D, p.B * p.H, p.N, p.Gw
        flops, win_pairs = {}, {}
        for s, st in enumerate(self.sched):
            if st["phase"] == A.PHASE_COARSE:
                flops[s] = 4.0 * D * BH * N * (N // (st["f"] ** 2))
                continue
            self.window_plan(s)
            pl = self.plan.cpu().numpy()
            nwin = int(pl[0])
            recs = pl[A.PLAN_HEADER:A.PLAN_HEADER + A.PLAN_REC * nwin].reshape(nwin, A.PLAN_REC)
            brt = self.bridge(s)
            if brt is not None:
                br = brt.cpu().numpy().reshape(BH, -1)
                by, bx = br // Gw, br % Gw
            pairs = 0
            for r in recs:
                qy0, qx0, qh, qw, ky0, kx0, kh, kw = (int(x) for x in r[:8])
                nkv = kh * kw * BH
                if brt is not None:
                    inside = (by >= ky0) & (by < ky0 + kh) & (bx >= kx0) & (bx < kx0 + kw)
                    nkv += int((~inside).sum())
                pairs += qh * qw * nkv
            win_pairs[s] = pairs
            flops[s] = 4.0 * D * pairs
        self.flops, self.win_pairs = flops, win_pairs
        self.full_flops = 4.0 * D * BH * float(N) * N
        return flops

    def summarize(self, recs, K):
        """Per-phase times averaged over K passes."""
        A, ev = self.A, self.ev
        agg = {k_: 0.0 for k_ in ("pool", "coarse_call", "coarse_kernel", "dwt", "plan", "window_call",
                                   "window_kernel", "full_call", "full_kernel")}
        per_step = {}
        parts = {}  # step -> summed component times over the K passes
        for kind, s, e in recs:
            if kind == "coarse":
                e0, e1, e2, a0, a1 = e
                t_pool, t_call, t_ker = e0.elapsed_time(e1), e1.elapsed_time(e2), ev.elapsed(a0, a1)
                agg["pool"] += t_pool
                agg["coarse_call"] += t_call
                agg["coarse_kernel"] += t_ker
                per_step.setdefault(s, []).append(t_pool + t_call)
                c = parts.setdefault(s, {"pool_ms": 0.0, "attn_call_ms": 0.0, "kernel_ms": 0.0})
                c["pool_ms"] += t_pool
                c["attn_call_ms"] += t_call
                c["kernel_ms"] += t_ker
            elif kind == "window":
                e0, e1, e2, e3, a0, a1 = e
                t_dwt, t_plan, t_call = e0.elapsed_time(e1), e1.elapsed_time(e2), e2.elapsed_time(e3)
                t_ker = ev.elapsed(a0, a1)
                agg["dwt"] += t_dwt
                agg["plan"] += t_plan
                agg["window_call"] += t_call
                agg["window_kernel"] += t_ker
                per_step.setdefault(s, []).append(t_dwt + t_plan + t_call)
                c = parts.setdefault(s, {"dwt_ms": 0.0, "plan_bridge_ms": 0.0, "attn_call_ms": 0.0, "kernel_ms": 0.0})
                c["dwt_ms"] += t_dwt
                c["plan_bridge_ms"] += t_plan
                c["attn_call_ms"] += t_call
                c["kernel_ms"] += t_ker
            else:
                e0, e1, a0, a1 = e
                agg["full_call"] += e0.elapsed_time(e1)
                agg["full_kernel"] += ev.elapsed(a0, a1)
        for k_ in agg:
            agg[k_] /= K
        # one entry per schedule step: its components (ms, averaged over the
        # passes; attn_call includes the kernel) and the attention kernel's rate
        self.step_detail = []
        for s in sorted(parts):
            st = self.sched[s]
            d = {"step": s}
            if st["phase"] == A.PHASE_COARSE:
                d["phase"], d["f"] = "coarse", st["f"]
            else:
                d["phase"], d["w"] = "window", st["w"]
            for k_, v_ in parts[s].items():
                d[k_] = round(v_ / K, 3)
            d["kernel_tflops"] = round(self.flops[s] / (d["kernel_ms"] * 1e-3) / 1e12, 1) if d["kernel_ms"] > 0 else None
            self.step_detail.append(d)
        area_ms = agg["pool"] + agg["coarse_call"] + agg["dwt"] + agg["plan"] + agg["window_call"]
        return agg, per_step, area_ms


def tflops(fl, ms):
    return fl / (ms * 1e-3) / 1e12 if ms > 0 else 0.0


# every configured workload besides the headline one is measured in the same
# run, with fewer timed passes
OTHER_CONFIGS = ["tiny-32", "flux-2048", "flux-4096", "qwen-6144x2048"]


def measure(A, W, wl, dev, ev, steps, warmup, calibrate=False):
    """Time `steps` passes of the workload's whole schedule (plus one full
    attention call each) after `warmup` passes; returns (schedule, metrics)."""
    import torch
    p = A.problem_for(wl)
    log(f"[bench] generating {wl.name} inputs on the GPU")
    q, k, v = W.make_qkv(wl, device="cuda", dtype="bf16")
    lat = torch.from_numpy(W.make_latent(wl)).to(dev)
    out = torch.empty_like(q)
    sc = Schedule(A, wl, p, q, k, v, lat, out, ev)
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: counting algorithmic work")
    flops = sc.count()
    sched, n_steps = sc.sched, sc.n_steps
    if calibrate:
        # one elementwise kernel with a unique name: reads 512 MiB, writes 512 MiB
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        log("[bench] calibration kernel (bitwise_not): 512 MiB read, 512 MiB written")
        del src, dst
    log(f"[bench] {wl.name}: warmup x{warmup}")
    for _ in range(warmup):
        sc.one_pass([])
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: timing x{steps}")
    recs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        sc.one_pass(recs)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps

    agg, per_step, area_ms = sc.summarize(recs, steps)
    BH, N, D = wl.B * wl.H, wl.N, wl.D
    n_coarse = sum(1 for st in sched if st["phase"] == A.PHASE_COARSE)
    n_win = n_steps - n_coarse
    coarse_fl = sum(flops[s] for s in flops if sched[s]["phase"] == A.PHASE_COARSE)
    win_fl = sum(flops[s] for s in flops if sched[s]["phase"] == A.PHASE_WINDOW)
    full_ms = agg["full_call"]
    # pooling bytes (mean mode): read K and V (bf16), write pooled K and V (fp32)
    pool_bytes = sum(2 * BH * N * D * 2 + 2 * BH * (N // sched[s]["f"] ** 2) * D * 4
                     for s in range(n_steps) if sched[s]["phase"] == A.PHASE_COARSE)
    dwt_bytes = n_win * (wl.C * N * 4 + (N // 4) * 8)
    p1_ms = agg["pool"] + agg["coarse_call"]
    p2_ms = agg["dwt"] + agg["plan"] + agg["window_call"]
    m = {
        "area_ms_per_step": area_ms / n_steps,
        "wall_ms_per_pass": wall_ms,
        "full_ms": full_ms,
        "full_tflops": tflops(sc.full_flops, agg["full_kernel"]),
        "area_tflops": tflops(coarse_fl + win_fl, area_ms),
        "phases": {
            "phase1_ms_per_step": p1_ms / max(n_coarse, 1),
            "phase2_ms_per_step": p2_ms / max(n_win, 1),
            "pool_ms_per_call": agg["pool"] / max(n_coarse, 1),
            "coarse_ms_per_call": agg["coarse_call"] / max(n_coarse, 1),
            "coarse_kernel_tflops": tflops(coarse_fl, agg["coarse_kernel"]),
            "dwt_ms_per_call": agg["dwt"] / max(n_win, 1),
            "plan_ms_per_call": agg["plan"] / max(n_win, 1),
            "window_ms_per_call": agg["window_call"] / max(n_win, 1),
            "window_kernel_tflops": tflops(win_fl, agg["window_kernel"]),
            "window_kernel_avg_ms": agg["window_kernel"] / max(n_win, 1),
            "phase1_tflops": tflops(coarse_fl, p1_ms),
            "phase2_tflops": tflops(win_fl, p2_ms),
            "pool_gbs": pool_bytes / (agg["pool"] * 1e-3) / 1e9 if agg["pool"] > 0 else 0.0,
            "dwt_gbs": dwt_bytes / (agg["dwt"] * 1e-3) / 1e9 if agg["dwt"] > 0 else 0.0,
            # per-phase speedups: full attention over one Phase I step (pool + coarse) and over
            # one Phase II step (DWT map + plan + windowed attention), averaged over each phase
            "speedup_phase1": full_ms * n_coarse / p1_ms if p1_ms > 0 else None,
            "speedup_phase2": full_ms * n_win / p2_ms if p2_ms > 0 else None,
            "per_step_ms": [round(sum(per_step[s]) / len(per_step[s]), 3) for s in sorted(per_step)],
            "per_step": sc.step_detail,
            "schedule_tflop": (coarse_fl + win_fl) / 1e12,
        },
        "n_coarse": n_coarse, "n_win": n_win, "steps": steps, "warmup": warmup,
        "tensors": (p, q, k, v, lat), "flops": flops,
    }
    return sc, m


def rounded(d):
    return {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in d.items()}


def config_summary(wl, m, cpu):
    """The per-config record of the bench line: per-phase ms/step, TFLOP/s and
    fractions of the bf16 MFMA peak, speedups over full attention, and the
    oracle's time on the host."""
    ph = m["phases"]
    return {
        "grid": [wl.Gh, wl.Gw], "heads": wl.H, "head_dim": wl.D, "steps": m["steps"],
        "coarse_steps": m["n_coarse"], "window_steps": m["n_win"],
        "area_ms_per_step": round(m["area_ms_per_step"], 4),
        "full_attn_ms": round(m["full_ms"], 4),
        "full_attn_tflops": round(m["full_tflops"], 1),
        "full_attn_frac": round(m["full_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "speedup_vs_full": round(m["full_ms"] / m["area_ms_per_step"], 3),
        "speedup_phase1": round(ph["speedup_phase1"], 3) if ph["speedup_phase1"] else None,
        "speedup_phase2": round(ph["speedup_phase2"], 3) if ph["speedup_phase2"] else None,
        "phase1_ms_per_step": round(ph["phase1_ms_per_step"], 4),
        "phase2_ms_per_step": round(ph["phase2_ms_per_step"], 4),
        "phase1_tflops": round(ph["phase1_tflops"], 1), "phase1_frac": round(ph["phase1_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "phase2_tflops": round(ph["phase2_tflops"], 1), "phase2_frac": round(ph["phase2_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "coarse_kernel_tflops": round(ph["coarse_kernel_tflops"], 1),
        "coarse_kernel_frac": round(ph["coarse_kernel_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "window_kernel_tflops": round(ph["window_kernel_tflops"], 1),
        "window_kernel_frac": round(ph["window_kernel_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "area_tflops": round(m["area_tflops"], 1), "area_frac": round(m["area_tflops"] / PEAK_MFMA_TFLOPS, 4),
        "pool_gbs": round(ph["pool_gbs"], 1), "pool_frac_hbm": round(ph["pool_gbs"] / PEAK_HBM_GBS, 4),
        "per_step_ms": ph["per_step_ms"],
        "cpu_oracle": cpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="flux-6144")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configured workloads (each is timed in the same run by default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one elementwise kernel over 512 MiB before the warm-up (known "
                         "traffic, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the bench line, print one JSON line with the AReA schedule timed "
                         "as configured and with splits, halo or bridge turned off, and at fixed w=64")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the AReA path runs on one GPU (no sharding across GPUs is implemented); --gpus must be 1"}))
        sys.exit(2)

    import torch

    import resolution_diffusion_transformer_amd as A
    import workloads as W

    if not os.path.exists(A.library_path()):
        from resolution_diffusion_transformer_amd import _build
        _build.build(verbose=False)
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    A.lib()
    dev = torch.device("cuda:0")
    wl = W.get(args.workload)
    ev = HipEvents()

    if args.ablation:
        p = A.problem_for(wl)
        q, k, v = W.make_qkv(wl, device="cuda", dtype="bf16")
        lat = torch.from_numpy(W.make_latent(wl)).to(dev)
        sc = Schedule(A, wl, p, q, k, v, lat, torch.empty_like(q), ev)
        run_ablation(A, wl, sc, args)
        return

    sc, m = measure(A, W, wl, dev, ev, args.steps, args.warmup, calibrate=args.copy_calibration)
    agg_win_ms = m["phases"]["window_kernel_avg_ms"]
    win_tflops = m["phases"]["window_kernel_tflops"]

    # ---- the matrix-core rate this GPU sustains (register-only MFMA stream) and a plain
    # read+write stream rate (torch's elementwise bitwise_not over 1 GiB in, 1 GiB out), for context
    mfma_measured = A.area_measure_mfma_peak()
    copy_gbs = 0.0
    if not args.copy_calibration:  # under the counters, the calibration kernel must stay the only one of its name
        cp_in = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cp_out = torch.empty_like(cp_in)
        torch.bitwise_not(cp_in, out=cp_out)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            torch.bitwise_not(cp_in, out=cp_out)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 5 * 2 * cp_in.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del cp_in, cp_out

    # ---- CPU oracle baseline on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        p, q, k, v, lat = m["tensors"]
        cpu = cpu_baseline(wl, q, k, v, lat, sc.sched, m["flops"], sc.win_pairs, sc.full_flops,
                           coarse_rows=wl.N, rows=8192, full_rows=4096)
    headline = config_summary(wl, m, None)

    # ---- every other configured workload, measured in the same run
    configs = {}
    if not args.no_configs:
        del sc
        m.pop("tensors")
        torch.cuda.empty_cache()
        for name in OTHER_CONFIGS:
            if name == wl.name:
                continue
            cwl = W.get(name)
            csc, cm = measure(A, W, cwl, dev, ev, max(1, min(args.steps, 3)), 1)
            ccpu = None
            if not args.no_cpu_baseline:
                p_, q_, k_, v_, lat_ = cm["tensors"]
                ccpu = cpu_baseline(cwl, q_, k_, v_, lat_, csc.sched, cm["flops"], csc.win_pairs, csc.full_flops,
                                    coarse_rows=2048, rows=2048, full_rows=1024)
            configs[name] = config_summary(cwl, cm, ccpu)
            del csc, cm
            torch.cuda.empty_cache()

    ph = m["phases"]
    result = {
        "metric": METRIC,
        "value": round(m["area_ms_per_step"], 4),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["wall_ms_per_pass"], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": wl.name, "grid": [wl.Gh, wl.Gw], "batch": wl.B, "heads": wl.H, "head_dim": wl.D,
                   "coarse_steps": m["n_coarse"], "window_steps": m["n_win"], "pool": "mean",
                   "halo": wl.halo, "bridge_k": wl.bridge_k, "io": "bf16"},
        "area_tflops": round(m["area_tflops"], 2),
        "area_pct_mfma_peak": round(100.0 * m["area_tflops"] / PEAK_MFMA_TFLOPS, 2),
        "full_attn_ms": round(m["full_ms"], 3),
        "full_attn_tflops": round(m["full_tflops"], 2),
        "speedup_vs_full": round(m["full_ms"] / m["area_ms_per_step"], 3),
        "phases": rounded(ph),
        "roofline": {
            "kernel": "attn_kernel (windowed)",
            "bound": "mfma",
            "achieved": round(win_tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(win_tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": measured_traffic(wl.name),
            "launches_per_step": m["n_win"],
            "avg_launch_ms": round(agg_win_ms, 4),
        },
        "cpu_baseline": cpu,
        "measured_peak": {
            "what": "register-only v_mfma_f32_32x32x16_f16 stream on this GPU (area_measure_mfma_peak)",
            "mfma_tflops": round(mfma_measured, 1),
            "window_kernel_frac": round(win_tflops / mfma_measured, 4) if mfma_measured > 0 else None,
            "full_attn_frac": round(m["full_tflops"] / mfma_measured, 4) if mfma_measured > 0 else None,
            "copy_gbs": round(copy_gbs, 1) if copy_gbs > 0 else None,
            "pool_frac_of_copy": round(ph["pool_gbs"] / copy_gbs, 4) if copy_gbs > 0 else None,
        },
        "configs": dict({wl.name: dict(headline, note="the headline workload above")}, **configs),
    }
    print(json.dumps(result), flush=True)


def run_ablation(A, wl, base, args):
    """Attention-time ablations of the AReA schedule (quadrant splits off,
    Halo off, bridge off, fixed smallest window, the other Phase I pooling
    modes) and the pages' own knob values, each against the same
    full-attention baseline; prints one JSON line."""
    import torch
    import workloads as W
    variants = [("as configured", {}), ("no quadrant splits", {"split_num": 0}), ("no halo", {"halo": 0}),
                ("no bridge", {"bridge_k": 0}), (f"fixed w={wl.w_min}", {"w_start": wl.w_min}),
                ("pooling: block centre", {"pool_mode": A.POOL_CENTER}),
                ("pooling: medoid", {"pool_mode": A.POOL_MEDOID}),
                ("pooling: random", {"pool_mode": A.POOL_RANDOM}),
                ("pages' knobs (w_start rule, seeded Halo <= 8, bridge (w/2)^2)", dict(W.PAGES_KNOBS))]
    rows = []
    full_ms = None
    for name, over in variants:
        sc = base if not over else Schedule(A, wl, A.problem_for(wl, **over), base.q, base.k, base.v, base.lat,
                                            base.out, base.ev)
        log(f"[ablation] {name}")
        flops = sc.count()
        for _ in range(args.warmup):
            sc.one_pass([], full=full_ms is None)
        torch.cuda.synchronize()
        recs = []
        for _ in range(args.steps):
            sc.one_pass(recs, full=full_ms is None)
        torch.cuda.synchronize()
        agg, _, area_ms = sc.summarize(recs, args.steps)
        if full_ms is None:
            full_ms = agg["full_call"]
        win_fl = sum(flops[s_] for s_ in flops if sc.sched[s_]["phase"] == A.PHASE_WINDOW)
        rows.append({"variant": name, "overrides": over,
                     "ms_per_step": round(area_ms / sc.n_steps, 4),
                     "speedup_vs_full": round(full_ms * sc.n_steps / area_ms, 3),
                     "schedule_tflop": round(sum(flops.values()) / 1e12, 2),
                     "window_kernel_tflops": round(tflops(win_fl, agg["window_kernel"]), 1)})
        if sc is not base:
            del sc
            torch.cuda.empty_cache()
    print(json.dumps({"ablation": rows, "workload": wl.name, "full_attn_ms": round(full_ms, 3),
                      "steps": args.steps, "warmup": args.warmup, "unit": "ms/step"}), flush=True)


def measured_traffic(workload):
    """HBM bytes per launch of the windowed attention kernel from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on
    the current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_window_{workload}_traffic.md")
    src = os.path.join(ROOT, "resolution_diffusion_transformer_amd", "csrc", "k_attn.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k_, v_ = line.split(":", 1)
            fields[k_.strip().lstrip("-* ").strip("`")] = v_.strip().strip("`")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("k_attn.hip sha256") != sha:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, q, k, v, lat, sched, flops, win_pairs, full_flops, coarse_rows, rows, full_rows):
    """The float64 NumPy oracle on head 0 of the workload, timed on the host:
    the Phase I step at the first pooling factor, Phase II steps 0, 1 and
    S-1 (Haar map, plan, bridge and windowed attention) and full attention,
    each on a bounded sample of query rows (coarse_rows, rows, full_rows;
    all rows when the grid is smaller).  Each attention call is timed twice,
    with one row and with the sample: the one-row time is the call's fixed
    part (the key rotation of the head), counted once per head; the rest is
    scaled by algorithmic FLOPs to all rows and heads.  Map and plan time is
    counted once per step, pooling and bridge once per head.  Unsampled steps
    take the seconds per FLOP of their phase's nearest sample."""
    import numpy as np
    import resolution_diffusion_transformer_amd as A
    from oracle import area_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    H = wl.B * wl.H
    N, D = wl.N, wl.D
    log(f"[bench] cpu baseline ({wl.name}): oracle on head 0, sampled query rows")
    qh = q[:, :1].float().cpu().numpy().astype(np.float64)
    kh = k[:, :1].float().cpu().numpy().astype(np.float64)
    vh = v[:, :1].float().cpu().numpy().astype(np.float64)
    latn = lat.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(7))
    O.attention(qh[0, 0, :1024], kh[0, 0, :1024], vh[0, 0, :1024])  # BLAS thread warm-up, untimed

    def pick(n):
        return np.arange(N) if n >= N else np.sort(rng.choice(N, size=n, replace=False))

    def two_times(fn, r):
        """(fixed seconds, seconds of the sample beyond the fixed part)"""
        t0 = time.perf_counter()
        fn(r[:1])
        t1 = time.perf_counter()
        fn(r)
        t2 = time.perf_counter()
        return t1 - t0, max((t2 - t1) - (t1 - t0), 1e-9), t2 - t0

    coarse = [s for s, st in enumerate(sched) if st["phase"] == A.PHASE_COARSE]
    window = [s for s, st in enumerate(sched) if st["phase"] == A.PHASE_WINDOW]
    detail, measured = [], 0.0
    est_ms = {}
    # Phase I at the first pooling factor: pooling of the whole head, attention of the sampled rows
    if coarse:
        s = coarse[0]
        f = sched[s]["f"]
        r = pick(coarse_rows)
        t0 = time.perf_counter()
        kp, vp = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta)
        t_pool = time.perf_counter() - t0
        t_fix, t_var, t_all = two_times(lambda rr: O.coarse_attention(qh, kp, vp, wl.Gh, wl.Gw, f, wl.rope_theta,
                                                                      rows=rr), r)
        measured += t_pool + t_all
        per_flop = t_var / (4.0 * D * max(len(r) - 1, 1) * (N // (f * f)))
        for c in coarse:
            est_ms[c] = 1e3 * (H * (t_pool + t_fix) + per_flop * flops[c])
        detail.append({"step": s, "phase": "coarse", "f": f, "rows": int(len(r)), "measured_s": round(t_pool + t_all, 3),
                       "est_ms_all_heads": round(est_ms[s], 1)})
    # Phase II steps 0, 1 and S-1
    win_rate = []
    for s in sorted({window[0], window[min(1, len(window) - 1)], window[-1]}) if window else []:
        t = s - wl.p1_steps
        w = sched[s]["w"]
        R = sched[s]["R"]
        r = pick(rows)
        t0 = time.perf_counter()
        Eq = O.energy_fixed(O.detail_energy(latn))
        plan = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq)
        t1 = time.perf_counter()
        br = O.bridge_select(kh[0, 0], R, wl.Gh, wl.Gw) if R > 0 else None
        t2 = time.perf_counter()
        brr = None if br is None else br[None, None]
        t_fix, t_var, t_all = two_times(lambda rr: O.window_attention(qh, kh, vh, plan, brr, wl.Gh, wl.Gw,
                                                                      wl.rope_theta, rows=rr), r)
        measured += (t2 - t0) + t_all
        sel = np.zeros(N, dtype=bool)
        sel[r[1:]] = True  # the rows beyond the one-row call
        sel[r[0]] = False
        pairs = 0
        for win in plan.windows:
            nsel = int(sel[O.window_query_indices(win, wl.Gw)].sum())
            if nsel:
                pairs += nsel * len(O.window_key_indices(win, wl.Gw, br))
        per_flop = t_var / (4.0 * D * max(pairs, 1))
        win_rate.append((s, per_flop, t1 - t0, (t2 - t1) + t_fix))
        est_ms[s] = 1e3 * ((t1 - t0) + H * ((t2 - t1) + t_fix) + per_flop * flops[s])
        detail.append({"step": s, "phase": "window", "w": w, "rows": int(len(r)),
                       "measured_s": round((t2 - t0) + t_all, 3), "est_ms_all_heads": round(est_ms[s], 1)})
    for s in window:
        if s in est_ms:
            continue
        _, per_flop, t_plan, t_head = min(win_rate, key=lambda e: abs(e[0] - s))
        est_ms[s] = 1e3 * (t_plan + H * t_head + per_flop * flops[s])
    # full attention: sampled rows of head 0, scaled to every row and head
    r = pick(full_rows)
    t_fix, t_var, t_all = two_times(lambda rr: O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta, rows=rr), r)
    measured += t_all
    full_ms = 1e3 * (H * t_fix + t_var * full_flops / (4.0 * D * max(len(r) - 1, 1) * N))
    ms_per_step = sum(est_ms.values()) / max(len(est_ms), 1)
    return {"value": round(ms_per_step, 1), "unit": "ms/step", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"float64 NumPy oracle on head 0 of {H}: Phase I step at f0 ({min(coarse_rows, N)} query "
                       f"rows), Phase II steps 0, 1 and S-1 ({min(rows, N)} sampled query rows each, with the step's "
                       f"Haar map, plan and bridge), full attention ({min(full_rows, N)} rows); a one-row call gives "
                       f"each call's fixed part (counted per head), the rest is scaled by FLOPs to all {N} rows and "
                       f"{H} heads; unsampled steps take their phase's seconds per FLOP; {len(est_ms)} steps"),
            "sample_seconds": round(measured, 2),
            "steps": detail,
            "full_attn_ms_est": round(full_ms, 1),
            "full_attn_note": (f"head 0, {min(full_rows, N)} of {N} query rows timed, scaled to all rows and x{H} "
                               f"heads (extrapolated)"),
            "speedup_vs_full_oracle": round(full_ms / ms_per_step, 3) if ms_per_step > 0 else None}


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
