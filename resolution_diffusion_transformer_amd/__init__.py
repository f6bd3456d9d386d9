"""Python binding of libarea.so, the MI355X (gfx950) AReA attention library.

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI declared in include/area.h.  PyTorch supplies
device memory and the current HIP stream.  The functions carry the C names.

If the shared library is missing this module raises on first use; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

__all__ = [
    "AreaError", "Problem", "lib", "library_path", "exported_symbols",
    "area_validate", "area_step_info", "area_f0", "area_base_windows", "area_workspace_bytes",
    "area_plan_words", "area_pool_kv", "area_coarse_attn", "area_dwt_detail",
    "area_window_plan", "area_window_plan_static", "area_window_attn", "area_full_attn", "area_text_attn", "area_attn_step",
    "area_set_attn_events",
    "POOL_MEAN", "POOL_CENTER", "POOL_MEDOID", "POOL_RANDOM", "PHASE_FULL", "PHASE_COARSE", "PHASE_WINDOW",
    "OP_FULL", "OP_COARSE", "OP_PLAN", "OP_WINDOW", "OP_STEP", "PLAN_HEADER", "PLAN_REC",
]

POOL_MEAN, POOL_CENTER, POOL_MEDOID, POOL_RANDOM = 0, 1, 2, 3
PHASE_FULL, PHASE_COARSE, PHASE_WINDOW = 0, 1, 2
OP_FULL, OP_COARSE, OP_PLAN, OP_WINDOW, OP_STEP = 0, 1, 2, 3, 4
PLAN_HEADER, PLAN_REC = 16, 10

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("AREA_LIBRARY", os.path.join(_HERE, "libarea.so"))


class AreaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"AReA status {status}: {detail}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("Gh", ctypes.c_int32), ("Gw", ctypes.c_int32),
                ("native_h", ctypes.c_int32), ("native_w", ctypes.c_int32),
                ("T", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("p1_steps", ctypes.c_int32), ("f0", ctypes.c_int32), ("f_min", ctypes.c_int32),
                ("pool_mode", ctypes.c_int32), ("p2_steps", ctypes.c_int32),
                ("w_start", ctypes.c_int32), ("w_min", ctypes.c_int32), ("halo", ctypes.c_int32),
                ("bridge_k", ctypes.c_int32), ("split_num", ctypes.c_int32),
                ("split_den", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("halo_max", ctypes.c_int32), ("bridge_rho_num", ctypes.c_int32),
                ("bridge_rho_den", ctypes.c_int32)]


class _Step(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int32), ("f", ctypes.c_int32), ("w", ctypes.c_int32),
                ("ny", ctypes.c_int32), ("nx", ctypes.c_int32), ("jit_y", ctypes.c_int32),
                ("jit_x", ctypes.c_int32), ("max_windows", ctypes.c_int32),
                ("q_total", ctypes.c_int64), ("R", ctypes.c_int32),
                ("bridge_rh", ctypes.c_int32), ("bridge_rw", ctypes.c_int32)]


@dataclass
class Problem:
    """Mirror of area_problem (include/area.h)."""
    B: int
    H: int
    D: int
    Gh: int
    Gw: int
    native_h: int
    native_w: int
    T: int = 0
    rope_theta: float = 10000.0
    p1_steps: int = 8
    f0: int = 0
    f_min: int = 2
    pool_mode: int = POOL_MEAN
    p2_steps: int = 0
    w_start: int = 0
    w_min: int = 0
    halo: int = 0
    bridge_k: int = 0
    split_num: int = 1
    split_den: int = 2
    seed: int = 0
    halo_max: int = 0
    bridge_rho_num: int = 0
    bridge_rho_den: int = 1

    def c(self) -> _Problem:
        return _Problem(self.B, self.H, self.D, self.Gh, self.Gw, self.native_h, self.native_w,
                        self.T, self.rope_theta, self.p1_steps, self.f0, self.f_min, self.pool_mode,
                        self.p2_steps, self.w_start, self.w_min, self.halo, self.bridge_k,
                        self.split_num, self.split_den, self.seed & ((1 << 64) - 1),
                        self.halo_max, self.bridge_rho_num, self.bridge_rho_den)

    @property
    def N(self) -> int:
        return self.Gh * self.Gw

    @property
    def L(self) -> int:
        """Rows per sequence: T text tokens, then the image tokens."""
        return self.T + self.Gh * self.Gw


_LIB = None

_SIGS = {
    "area_validate": (ctypes.c_int, [ctypes.c_void_p]),
    "area_step_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "area_f0": (ctypes.c_int, [ctypes.c_void_p]),
    "area_base_windows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]),
    "area_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int]),
    "area_plan_words": (ctypes.c_size_t, [ctypes.c_void_p]),
    "area_set_attn_events": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "area_measure_mfma_peak": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
    "area_phase1_steps_for_sigma": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_double,
                                                   ctypes.POINTER(ctypes.c_int)]),
    "area_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "area_last_error": (ctypes.c_char_p, []),
    "area_pool_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 5),
    "area_coarse_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 5
                         + [ctypes.c_size_t, ctypes.c_void_p]),
    "area_dwt_detail": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 4),
    "area_window_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 6
                         + [ctypes.c_size_t, ctypes.c_void_p]),
    "area_window_plan_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 6),
    "area_window_attn": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 8
                         + [ctypes.c_size_t, ctypes.c_void_p]),
    "area_full_attn": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5
                       + [ctypes.c_size_t, ctypes.c_void_p]),
    "area_text_attn": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5
                       + [ctypes.c_size_t, ctypes.c_void_p]),
    "area_attn_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6
                       + [ctypes.c_size_t, ctypes.c_void_p]),
}


def lib():
    """Load libarea.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m resolution_diffusion_transformer_amd._build`")
        try:  # let torch load its HIP runtime first so the process holds one copy
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def exported_symbols():
    return sorted(_SIGS)


def _check(rc: int):
    if rc < 0:
        raise AreaError(rc, lib().area_last_error().decode())
    return rc


def _pp(p: Problem):
    s = p.c()
    return s, ctypes.byref(s)


def area_validate(p: Problem) -> int:
    s, ref = _pp(p)
    return _check(lib().area_validate(ref))


def area_f0(p: Problem) -> int:
    s, ref = _pp(p)
    return _check(lib().area_f0(ref))


def area_step_info(p: Problem, step: int) -> dict:
    s, ref = _pp(p)
    out = _Step()
    _check(lib().area_step_info(ref, step, ctypes.byref(out)))
    return {k: getattr(out, k) for k, _ in _Step._fields_}


def area_base_windows(p: Problem, step: int):
    import numpy as np
    s, ref = _pp(p)
    cap = 64 * 64
    buf = (ctypes.c_int32 * (4 * cap))()
    n = _check(lib().area_base_windows(ref, step, buf, cap))
    return np.frombuffer(buf, dtype=np.int32, count=4 * n).reshape(n, 4).copy()


def area_workspace_bytes(p: Problem, op: int) -> int:
    s, ref = _pp(p)
    return int(lib().area_workspace_bytes(ref, op))


def area_plan_words(p: Problem) -> int:
    s, ref = _pp(p)
    return int(lib().area_plan_words(ref))


def area_set_attn_events(ev_begin: Optional[int], ev_end: Optional[int]) -> int:
    """Record the given hipEvent_t handles around each attention kernel
    launched by this thread (None, None to stop)."""
    return _check(lib().area_set_attn_events(ev_begin, ev_end))


# ----------------------------------------------------------- device calls --

def area_phase1_steps_for_sigma(sigmas, sigma_star: float) -> int:
    """Number of leading denoising steps whose noise level is above sigma_star
    (Phase I); host only."""
    vals = [float(x) for x in sigmas]
    arr = (ctypes.c_double * max(len(vals), 1))(*vals)
    out = ctypes.c_int(0)
    _check(lib().area_phase1_steps_for_sigma(arr, len(vals), float(sigma_star), ctypes.byref(out)))
    return int(out.value)


def area_measure_mfma_peak() -> float:
    """Sustained fp16/bf16 matrix-core rate of the current device in TFLOP/s
    (register-only MFMA stream; synchronises the current stream)."""
    torch = _torch()
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    out = ctypes.c_double(0.0)
    _check(lib().area_measure_mfma_peak(ctypes.c_void_p(sink.data_ptr()), ctypes.byref(out), _stream()))
    return float(out.value)


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _need(t, dtype, shape, name):
    torch = _torch()
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t) -> int:
    """Size in bytes of a device buffer tensor (0 for None)."""
    return 0 if t is None else t.numel() * t.element_size()


def workspace(p: Problem, op: int, device="cuda"):
    """A device workspace tensor of the size the library asks for (or None)."""
    torch = _torch()
    n = area_workspace_bytes(p, op)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def area_pool_kv(p: Problem, f: int, k, v, kp=None, vp=None):
    torch = _torch()
    shp = (p.B, p.H, p.L, p.D)
    _need(k, torch.bfloat16, shp, "k")
    _need(v, torch.bfloat16, shp, "v")
    M = p.T + ((p.Gh // f) * (p.Gw // f) if f > 0 else 0)
    kp = torch.empty((p.B, p.H, M, p.D), dtype=torch.float32, device=k.device) if kp is None else kp
    vp = torch.empty((p.B, p.H, M, p.D), dtype=torch.float32, device=k.device) if vp is None else vp
    _need(kp, torch.float32, (p.B, p.H, M, p.D), "kp")
    _need(vp, torch.float32, (p.B, p.H, M, p.D), "vp")
    s, ref = _pp(p)
    _check(lib().area_pool_kv(ref, f, _ptr(k), _ptr(v), _ptr(kp), _ptr(vp), _stream()))
    return kp, vp


def area_coarse_attn(p: Problem, f: int, q, kp, vp, out=None, ws=None):
    torch = _torch()
    _need(q, torch.bfloat16, (p.B, p.H, p.L, p.D), "q")
    M = p.T + ((p.Gh // f) * (p.Gw // f) if f > 0 else 0)
    _need(kp, torch.float32, (p.B, p.H, M, p.D), "kp")
    _need(vp, torch.float32, (p.B, p.H, M, p.D), "vp")
    out = torch.empty_like(q) if out is None else out
    _need(out, torch.bfloat16, (p.B, p.H, p.L, p.D), "out")
    ws = workspace(p, OP_COARSE, q.device) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_coarse_attn(ref, f, _ptr(q), _ptr(kp), _ptr(vp), _ptr(out), _ptr(ws),
                                  _nbytes(ws), _stream()))
    return out


def area_dwt_detail(p: Problem, latent, energy=None, energy_q=None):
    torch = _torch()
    C = latent.shape[0]
    _need(latent, torch.float32, (C, p.Gh, p.Gw), "latent")
    hw = (p.Gh // 2, p.Gw // 2)
    energy = torch.empty(hw, dtype=torch.float32, device=latent.device) if energy is None else energy
    energy_q = torch.empty(hw, dtype=torch.int32, device=latent.device) if energy_q is None else energy_q
    _need(energy, torch.float32, hw, "energy")
    _need(energy_q, torch.int32, hw, "energy_q")
    s, ref = _pp(p)
    _check(lib().area_dwt_detail(ref, C, _ptr(latent), _ptr(energy), _ptr(energy_q), _stream()))
    return energy, energy_q


def area_window_plan(p: Problem, step: int, energy_q, k, plan=None, wsum=None, bridge_idx=None, ws=None):
    torch = _torch()
    src = energy_q if energy_q is not None else k
    dev = src.device if src is not None else torch.device("cuda")
    if energy_q is not None:
        _need(energy_q, torch.int32, (p.Gh // 2, p.Gw // 2), "energy_q")
    if k is not None:
        _need(k, torch.bfloat16, (p.B, p.H, p.L, p.D), "k")
    words = area_plan_words(p)
    plan = torch.zeros(words, dtype=torch.int32, device=dev) if plan is None else plan
    wsum = torch.empty(p.N, dtype=torch.int32, device=dev) if wsum is None else wsum
    R = area_step_info(p, step)["R"]
    use_bridge = k is not None and R > 0
    if use_bridge and bridge_idx is None:
        bridge_idx = torch.empty((p.B, p.H, R), dtype=torch.int32, device=dev)
    _need(plan, torch.int32, (words,), "plan")
    _need(wsum, torch.int32, (p.N,), "wsum")
    if use_bridge:
        _need(bridge_idx, torch.int32, (p.B, p.H, R), "bridge_idx")
    ws = workspace(p, OP_PLAN, dev) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_window_plan(ref, step, _ptr(energy_q), _ptr(k), _ptr(plan), _ptr(wsum),
                                  _ptr(bridge_idx) if use_bridge else None, _ptr(ws),
                                  _nbytes(ws), _stream()))
    return plan, wsum, (bridge_idx if use_bridge else None)


def area_window_plan_static(p: Problem, step: int, energy_q, k, plan=None, wsum=None, bridge_idx=None):
    """area_window_plan with the library's static device scratch (no workspace)."""
    torch = _torch()
    src = energy_q if energy_q is not None else k
    dev = src.device if src is not None else torch.device("cuda")
    if energy_q is not None:
        _need(energy_q, torch.int32, (p.Gh // 2, p.Gw // 2), "energy_q")
    if k is not None:
        _need(k, torch.bfloat16, (p.B, p.H, p.L, p.D), "k")
    words = area_plan_words(p)
    plan = torch.zeros(words, dtype=torch.int32, device=dev) if plan is None else plan
    wsum = torch.empty(p.N, dtype=torch.int32, device=dev) if wsum is None else wsum
    R = area_step_info(p, step)["R"]
    use_bridge = k is not None and R > 0
    if use_bridge and bridge_idx is None:
        bridge_idx = torch.empty((p.B, p.H, R), dtype=torch.int32, device=dev)
    _need(plan, torch.int32, (words,), "plan")
    _need(wsum, torch.int32, (p.N,), "wsum")
    if use_bridge:
        _need(bridge_idx, torch.int32, (p.B, p.H, R), "bridge_idx")
    s, ref = _pp(p)
    _check(lib().area_window_plan_static(ref, step, _ptr(energy_q), _ptr(k), _ptr(plan), _ptr(wsum),
                                         _ptr(bridge_idx) if use_bridge else None, _stream()))
    return plan, wsum, (bridge_idx if use_bridge else None)


def area_window_attn(p: Problem, step: int, plan, wsum, bridge_idx, q, k, v, out=None, ws=None):
    torch = _torch()
    shp = (p.B, p.H, p.L, p.D)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, shp, nm)
    _need(plan, torch.int32, (area_plan_words(p),), "plan")
    _need(wsum, torch.int32, (p.N,), "wsum")
    if bridge_idx is not None:
        _need(bridge_idx, torch.int32, (p.B, p.H, area_step_info(p, step)["R"]), "bridge_idx")
    out = torch.empty_like(q) if out is None else out
    _need(out, torch.bfloat16, shp, "out")
    ws = workspace(p, OP_WINDOW, q.device) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_window_attn(ref, step, _ptr(plan), _ptr(wsum), _ptr(bridge_idx), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                  _nbytes(ws), _stream()))
    return out


def area_text_attn(p: Problem, q, k, v, out=None, ws=None):
    """Text-query rows (0 .. T-1) of out: dense attention over all T + N keys."""
    torch = _torch()
    shp = (p.B, p.H, p.L, p.D)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, shp, nm)
    out = torch.empty_like(q) if out is None else out
    _need(out, torch.bfloat16, shp, "out")
    ws = workspace(p, OP_FULL, q.device) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_text_attn(ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                _nbytes(ws), _stream()))
    return out


def area_attn_step(p: Problem, step: int, latent, q, k, v, out=None, ws=None):
    """One denoising step's attention along the schedule (full, pooled
    coarse, or windowed with plan and bridge); latent [C, Gh, Gw] fp32 feeds
    the detail map of window steps (None: no quadrant splits)."""
    torch = _torch()
    shp = (p.B, p.H, p.L, p.D)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, shp, nm)
    C = 0
    if latent is not None:
        C = latent.shape[0]
        _need(latent, torch.float32, (C, p.Gh, p.Gw), "latent")
    out = torch.empty_like(q) if out is None else out
    _need(out, torch.bfloat16, shp, "out")
    ws = workspace(p, OP_STEP, q.device) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_attn_step(ref, step, C, _ptr(latent), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                _nbytes(ws), _stream()))
    return out


def area_full_attn(p: Problem, q, k, v, out=None, ws=None):
    torch = _torch()
    shp = (p.B, p.H, p.L, p.D)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, shp, nm)
    out = torch.empty_like(q) if out is None else out
    _need(out, torch.bfloat16, shp, "out")
    ws = workspace(p, OP_FULL, q.device) if ws is None else ws
    s, ref = _pp(p)
    _check(lib().area_full_attn(ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                _nbytes(ws), _stream()))
    return out


def problem_for(wl, **over) -> Problem:
    """Problem for a workloads.Workload (sizes and knobs), with overrides."""
    kw = dict(B=wl.B, H=wl.H, D=wl.D, Gh=wl.Gh, Gw=wl.Gw, native_h=wl.native_h,
              native_w=wl.native_w, rope_theta=wl.rope_theta, p1_steps=wl.p1_steps, f0=0,
              f_min=wl.f_min, pool_mode=POOL_MEAN, p2_steps=wl.p2_steps, w_start=wl.w_start,
              w_min=wl.w_min, halo=wl.halo, bridge_k=wl.bridge_k, seed=wl.seed, T=getattr(wl, "T", 0))
    kw.update(over)
    return Problem(**kw)
