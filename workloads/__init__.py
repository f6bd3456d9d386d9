"""Seeded synthetic workloads for the adaptive receptive-field attention path.

This module only describes problem sizes and draws random inputs.  It holds
none of the method's arithmetic (no RoPE, pooling, wavelet, window plan or
attention), so both the HIP path and the CPU oracle can take their inputs
from it without sharing any computation.

Workload shapes follow the FLUX.1 and Qwen-Image settings discussed in
"AReA: Adaptive Receptive-Field Attention for Efficient High-Resolution
Diffusion Transformers" (ai.info summary, Main Findings: 6144^2 speedups) and
the repository README (base resolution paragraph: 1024 px for FLUX.1, 1328 px
native for Qwen-Image with windows down to 1024 px).  One token is one 16 px
patch, so FLUX.1's native grid is 64x64 tokens.

Input recipe (the same for every workload):
  * Q, K, V: per (tensor, batch, head, channel) an N(0,1) image on the token
    grid, blurred with a separable Gaussian (sigma 3 tokens, radius 12,
    reflect boundary, taps normalised to sum 1), divided by the blurred
    field's theoretical std (the sum of squared taps) so it is unit-variance
    again, plus 0.3 * N(0,1) white noise.  Laid out [B, H, Gh*Gw, D] with
    token n = y*Gw + x.  bf16 workloads round once to bf16.
  * DWT latent [C=16, Gh, Gw] fp32: smooth regions are per-channel linear
    gradients a*y/Gh + b*x/Gw + c with a, b, c ~ N(0,1); textured regions are
    that gradient plus N(0,1).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_qkv", "make_latent",
           "gaussian_taps", "SEED_Q", "SEED_K", "SEED_V", "SEED_LATENT"]

SEED_Q, SEED_K, SEED_V, SEED_LATENT = 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    Gh: int
    Gw: int
    native_h: int
    native_w: int
    dtype: str            # "fp32" or "bf16": precision of the Q/K/V handed to the path
    p1_steps: int         # coarse-attention (Phase I) steps
    f_min: int
    p2_steps: int         # windowed (Phase II) steps
    w_start: int
    w_min: int
    halo: int
    bridge_k: int
    latent_kind: str      # which smooth/textured layout the DWT latent has
    C: int = 16
    rope_theta: float = 10000.0
    seed: int = 0         # plan seed (window-boundary jitter)
    T: int = 0            # text tokens ahead of the image tokens in every sequence

    @property
    def N(self) -> int:
        return self.Gh * self.Gw


WORKLOADS = {
    # 32x32 token grid, native 16x16: f = 2 gives 256 pooled keys.
    "tiny-32": Workload("tiny-32", B=1, H=2, D=64, Gh=32, Gw=32, native_h=16, native_w=16,
                        dtype="fp32", p1_steps=8, f_min=2, p2_steps=4, w_start=16, w_min=8,
                        halo=1, bridge_k=16, latent_kind="tiny_patches"),
    # FLUX.1 at 2048^2: 128x128 tokens, native 64x64.
    "flux-2048": Workload("flux-2048", B=1, H=24, D=128, Gh=128, Gw=128, native_h=64, native_w=64,
                          dtype="bf16", p1_steps=8, f_min=2, p2_steps=8, w_start=128, w_min=64,
                          halo=4, bridge_k=256, latent_kind="half_columns"),
    # FLUX.1 at 4096^2: 256x256 tokens.
    "flux-4096": Workload("flux-4096", B=1, H=24, D=128, Gh=256, Gw=256, native_h=64, native_w=64,
                          dtype="bf16", p1_steps=8, f_min=2, p2_steps=16, w_start=128, w_min=64,
                          halo=4, bridge_k=256, latent_kind="half_columns"),
    # FLUX.1 at 6144^2: 384x384 tokens (147456), 30% smooth latent.
    "flux-6144": Workload("flux-6144", B=1, H=24, D=128, Gh=384, Gw=384, native_h=64, native_w=64,
                          dtype="bf16", p1_steps=8, f_min=2, p2_steps=20, w_start=192, w_min=64,
                          halo=4, bridge_k=512, latent_kind="smooth30_columns"),
    # Qwen-Image at 6144x2048: 384x128 tokens, native 1328 px = 83 tokens.
    "qwen-6144x2048": Workload("qwen-6144x2048", B=1, H=24, D=128, Gh=384, Gw=128, native_h=83,
                               native_w=83, dtype="bf16", p1_steps=20, f_min=2, p2_steps=16,
                               w_start=128, w_min=64, halo=4, bridge_k=256,
                               latent_kind="row_bands32"),
    # Joint text + image sequences: the tiny grid with 8 text tokens, and FLUX.1 at
    # 2048^2 with the 512 text tokens of its T5 prompt encoding.
    "tiny-32-text": Workload("tiny-32-text", B=1, H=2, D=64, Gh=32, Gw=32, native_h=16, native_w=16,
                             dtype="fp32", p1_steps=8, f_min=2, p2_steps=4, w_start=16, w_min=8,
                             halo=1, bridge_k=16, latent_kind="tiny_patches", T=8),
    "flux-2048-text": Workload("flux-2048-text", B=1, H=24, D=128, Gh=128, Gw=128, native_h=64, native_w=64,
                               dtype="bf16", p1_steps=8, f_min=2, p2_steps=8, w_start=128, w_min=64,
                               halo=4, bridge_k=256, latent_kind="half_columns", T=512),
}


# The pages' own Phase II knob values, as problem overrides: the first window
# from the cost rule (w_start 0), Halo widths drawn per window up to 8, and a
# bridge of (w/2)^2 tokens at window side w.
PAGES_KNOBS = dict(w_start=0, halo_max=8, bridge_rho_num=1, bridge_rho_den=2)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def gaussian_taps(sigma: float = 3.0, radius: int = 12) -> np.ndarray:
    t = np.arange(-radius, radius + 1, dtype=np.float64)
    w = np.exp(-0.5 * (t / sigma) ** 2)
    return w / w.sum()


def _smooth_noise(n_img: int, Gh: int, Gw: int, gen, device, chunk: int = 1024):
    """[n_img, Gh, Gw] float32 unit-variance blurred field + 0.3 white noise."""
    import torch
    import torch.nn.functional as F
    taps = gaussian_taps()
    r = (len(taps) - 1) // 2
    norm = float((taps ** 2).sum())  # std of the 2-D blurred unit field
    kt = torch.tensor(taps, dtype=torch.float32, device=device)
    out = torch.empty((n_img, Gh, Gw), dtype=torch.float32, device=device)
    for s in range(0, n_img, chunk):
        e = min(n_img, s + chunk)
        x = torch.randn((e - s, 1, Gh, Gw), generator=gen, device=device, dtype=torch.float32)
        x = F.pad(x, (0, 0, r, r), mode="reflect")
        x = F.conv2d(x, kt.view(1, 1, -1, 1))
        x = F.pad(x, (r, r, 0, 0), mode="reflect")
        x = F.conv2d(x, kt.view(1, 1, 1, -1))
        x = x[:, 0] / norm
        x += 0.3 * torch.randn(x.shape, generator=gen, device=device, dtype=torch.float32)
        out[s:e] = x
    return out


def make_qkv(wl: Workload, device: str = "cpu", dtype: Optional[str] = None, seed: int = 0):
    """Return (q, k, v) torch tensors [B, H, T + N, D] on `device`: T text
    tokens (iid N(0,1) rows, their own stream) ahead of the N image tokens.

    dtype "bf16" rounds to torch.bfloat16; "fp32" keeps float32.  The draw is
    reproducible per (device type, seed, workload)."""
    import torch
    dtype = dtype or wl.dtype
    outs = []
    for which in (SEED_Q, SEED_K, SEED_V):
        gen = torch.Generator(device=device)
        gen.manual_seed(seed * 1000003 + which)
        f = _smooth_noise(wl.B * wl.H * wl.D, wl.Gh, wl.Gw, gen, device)
        f = f.view(wl.B, wl.H, wl.D, wl.N).transpose(2, 3).contiguous()
        if wl.T > 0:
            gt = torch.Generator(device=device)
            gt.manual_seed(seed * 1000003 + which + 100)
            t = torch.randn((wl.B, wl.H, wl.T, wl.D), generator=gt, device=device, dtype=torch.float32)
            f = torch.cat([t, f], dim=2)
            del t
        outs.append(f.to(torch.bfloat16) if dtype == "bf16" else f)
        del f
    return tuple(outs)


def _gradient(C: int, Gh: int, Gw: int, rng) -> np.ndarray:
    a, b, c = rng.standard_normal((3, C))
    y = np.arange(Gh, dtype=np.float64)[:, None] / Gh
    x = np.arange(Gw, dtype=np.float64)[None, :] / Gw
    return a[:, None, None] * y + b[:, None, None] * x + c[:, None, None]


def textured_mask(wl: Workload) -> np.ndarray:
    """Boolean [Gh, Gw]: True where the latent carries N(0,1) texture."""
    m = np.zeros((wl.Gh, wl.Gw), dtype=bool)
    if wl.latent_kind == "tiny_patches":
        m[4:12, 4:12] = True
        m[18:26, 16:24] = True
    elif wl.latent_kind == "half_columns":
        m[:, wl.Gw // 2:] = True
    elif wl.latent_kind == "smooth30_columns":
        s = int(round(0.3 * wl.Gw / 2)) * 2  # even split column: 116 at 384
        m[:, s:] = True
    elif wl.latent_kind == "row_bands32":
        for r0 in range(0, wl.Gh, 64):
            m[r0 + 32:r0 + 64, :] = True
    else:
        raise ValueError(wl.latent_kind)
    return m


def make_latent(wl: Workload, seed: int = 0) -> np.ndarray:
    """DWT input [C, Gh, Gw] float32 (numpy PCG64, seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed * 1000003 + SEED_LATENT))
    g = _gradient(wl.C, wl.Gh, wl.Gw, rng)
    tex = rng.standard_normal((wl.C, wl.Gh, wl.Gw))
    m = textured_mask(wl)
    lat = g + np.where(m[None], tex, 0.0)
    return lat.astype(np.float32)


def random_small_qkv(B, H, N, D, seed=0, scale=1.0):
    """Plain iid N(0, scale^2) fp32 tensors (numpy) for tiny property tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return tuple((scale * rng.standard_normal((B, H, N, D))).astype(np.float32) for _ in range(3))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (a >> 16) & 1
    a = (a + 0x7FFF + lsb) & 0xFFFF0000
    return a.astype(np.uint32).view(np.float32)
