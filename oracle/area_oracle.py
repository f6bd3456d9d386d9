"""CPU oracle for adaptive receptive-field attention (AReA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its binding) never calls it and shares no code with it.

Everything here is the plain definition written out: float64 NumPy, one
library matmul per attention block, Python loops where the method iterates
over windows or cells.  Plan decisions (pooling ramp, window sizes, tiling,
jitter, quadrant splits, bridge choice, blend weights) are integers or
fixed-order float64, so a second implementation that follows the same steps
reproduces them bit for bit.

Sources (page titles, sections):
  [blog]    "AReA: atención training-free para generar más allá de la
            resolución nativa de FLUX.1", section "Las dos fases de AReA"
            (Fase I, Fase II) and "Cómo entra en tu pipeline".
  [summary] "AReA: Adaptive Receptive-Field Attention for Efficient
            High-Resolution Diffusion Transformers" (ai.info AI summary),
            section "Methodology in Plain English" (Phase I, Phase II,
            Scheduling the switch) and "Main Findings".
  [readme]  AReA GitHub wiki / README: introduction (Phase I / Phase II
            bullets), base-resolution paragraph, canvas-rules paragraph,
            repository layout.

Where the pages leave a step open, the reading taken is marked READING and
named (R1...R23); each is one small function here.

Text tokens (READING R20, [summary] Phase I: pooling leaves the text
tokens alone, so a query's key set is the T text keys plus the N/f^2
pooled image keys): with T > 0 the
token sequence is T text tokens first, then the Gh*Gw image tokens in
row-major order.  Text tokens sit at RoPE position (0, 0) (no rotation),
join every key set of both phases whole, and text queries attend densely to
all T + N keys (text_attention).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

MASK64 = (1 << 64) - 1

# ----------------------------------------------------------------------------
# RoPE on a 2-D token grid
# ----------------------------------------------------------------------------


def rope_inv_freq(D: int, theta: float) -> np.ndarray:
    """READING R1: two-axis RoPE.  The first D/2 channels encode the row y, the
    last D/2 the column x; within an axis half, channel pair (2k, 2k+1) turns
    by pos * theta^(-2k/(D/2)) for k < D/4.  The pages only state that the
    RoPE frequencies are kept intact with no extrapolation ([blog] TL;DR and
    "El problema"; [summary] Phase I: queries and pooled keys share one
    coordinate system)."""
    if D % 4:
        raise ValueError("head dim must be a multiple of 4 for two-axis RoPE")
    half = D // 2
    k = np.arange(half // 2, dtype=np.float64)
    return theta ** (-2.0 * k / half)


def apply_rope_2d(x: np.ndarray, ypos: np.ndarray, xpos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate x[..., n, D] at per-token positions (ypos[n], xpos[n]) (float64)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    inv = rope_inv_freq(D, theta)
    out = np.empty_like(x)
    for axis, pos in ((0, np.asarray(ypos, np.float64)), (1, np.asarray(xpos, np.float64))):
        ang = pos[:, None] * inv[None, :]            # [n, D/4]
        c, s = np.cos(ang), np.sin(ang)
        base = axis * (D // 2)
        a = x[..., base + 0:base + D // 2:2]        # even channel of each pair
        b = x[..., base + 1:base + D // 2:2]        # odd channel
        out[..., base + 0:base + D // 2:2] = a * c - b * s
        out[..., base + 1:base + D // 2:2] = a * s + b * c
    return out


def grid_positions(Gh: int, Gw: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row-major token grid: token n sits at (n // Gw, n % Gw)."""
    n = np.arange(Gh * Gw)
    return n // Gw, n % Gw


def token_positions(Gh: int, Gw: int, T: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Positions of the joint sequence: T text tokens at (0, 0) (READING R20),
    then the image grid."""
    y, x = grid_positions(Gh, Gw)
    z = np.zeros(T, dtype=y.dtype)
    return np.concatenate([z, y]), np.concatenate([z, x])


# ----------------------------------------------------------------------------
# Dense attention (the speedup baseline, and the inner step of both phases)
# ----------------------------------------------------------------------------


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              key_mask: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(q k^T / sqrt(D)) v for already-rotated q [.., nq, D] and k, v
    [.., nk, D] (READING R2: the usual 1/sqrt(D) scale).  key_mask [nq, nk]
    (True = keep) restricts each query's key set."""
    D = q.shape[-1]
    s = (np.asarray(q, np.float64) @ np.swapaxes(np.asarray(k, np.float64), -1, -2)) / math.sqrt(D)
    if key_mask is not None:
        s = np.where(key_mask, s, -np.inf)
    return softmax_rows(s) @ np.asarray(v, np.float64)


def full_attention(q, k, v, Gh: int, Gw: int, theta: float,
                   rows: Optional[np.ndarray] = None, T: int = 0) -> np.ndarray:
    """Uniform full attention over all tokens with RoPE at native grid
    positions: the baseline AReA replaces ([summary] Overview and Main
    Findings: speedups are quoted against full attention).  q, k, v are
    un-rotated [B, H, T + N, D]; `rows` optionally restricts the output
    queries (indices into the joint sequence)."""
    y, x = token_positions(Gh, Gw, T)
    kr = apply_rope_2d(k, y, x, theta)
    if rows is None:
        rows = np.arange(T + Gh * Gw)
    qr = apply_rope_2d(np.asarray(q)[..., rows, :], y[rows], x[rows], theta)
    return attention(qr, kr, v)


def text_attention(q, k, v, Gh: int, Gw: int, theta: float, T: int) -> np.ndarray:
    """READING R20: text queries take the dense path in every phase, over
    all T + N keys at native positions; [B, H, T, D]."""
    return full_attention(q, k, v, Gh, Gw, theta, rows=np.arange(T), T=T)


# ----------------------------------------------------------------------------
# Phase I: pooled keys/values and cross-scale coarse attention
# ----------------------------------------------------------------------------

POOL_MEAN, POOL_CENTER, POOL_MEDOID, POOL_RANDOM = 0, 1, 2, 3
POOL_STREAM = 0x504F4F4C  # "POOL": random pooling draws from its own SplitMix64 stream


def pool_tokens(t: np.ndarray, Gh: int, Gw: int, f: int, mode: int) -> np.ndarray:
    """One token per f x f block of the grid ([blog] Fase I; [summary]
    Phase I; [readme] Phase I bullet).  READING R3: mean = average of the f^2
    tokens of the block; center = the token at offset (f//2, f//2) inside the
    block.  t is [..., N, D] with row-major tokens; the result is
    [..., (Gh/f)*(Gw/f), D], block (by, bx) at index by*(Gw/f) + bx."""
    if Gh % f or Gw % f:
        raise ValueError("pooling factor must divide both grid sides")
    t = np.asarray(t, np.float64)
    lead = t.shape[:-2]
    D = t.shape[-1]
    g = t.reshape(lead + (Gh // f, f, Gw // f, f, D))
    if mode == POOL_MEAN:
        p = g.mean(axis=(-4, -2))
    elif mode == POOL_CENTER:
        c = f // 2
        p = g[..., :, c, :, c, :]
    else:
        raise ValueError("pool mode")
    return p.reshape(lead + ((Gh // f) * (Gw // f), D))


def block_tokens(Gw: int, f: int, by: int, bx: int) -> np.ndarray:
    """Token indices of block (by, bx), row-major inside the block: in-block
    offset o is token (by*f + o // f, bx*f + o % f)."""
    o = np.arange(f * f)
    return (by * f + o // f) * Gw + (bx * f + o % f)


def pool_random_offset(seed: int, f: int, block: int) -> int:
    """READING R21 of random pooling ([blog] "Cómo entra en tu pipeline": the
    tunable pooling takes subsample / mean / medoid / random, and the seed
    controls random pooling; [summary] Main Findings: random pooling in the
    representative ablation).  One in-block offset per (pooling factor,
    block), the same for every batch, head, K and V:
    splitmix64(seed ^ POOL_STREAM, 1 + f * 2^32 + block) mod f^2."""
    return int(splitmix64(seed ^ POOL_STREAM, 1 + f * (1 << 32) + block) % (f * f))


def medoid_offset(kb: np.ndarray) -> int:
    """READING R22 of medoid pooling (same passages as R21): the medoid of a
    block is its token whose key has the smallest sum of Euclidean distances
    to the block's keys (un-rotated), ties to the smaller in-block offset.
    kb is [f*f, D] in in-block order.  float64 in a fixed order, so a second
    implementation that follows it decides the same way: per pair the
    squared differences summed over d ascending, the square root, then the
    sum over the other token i ascending."""
    kb = np.asarray(kb, np.float64)
    n, D = kb.shape
    diff = kb[:, None, :] - kb[None, :, :]          # [i, j, d]
    s = np.zeros((n, n))
    for d in range(D):                              # d ascending, one rounding per step
        s = s + diff[:, :, d] * diff[:, :, d]
    dist = np.sqrt(s)
    total = np.zeros(n)
    for i in range(n):                              # other token i ascending
        total = total + dist[i, :]
    return int(np.argmin(total))                    # first minimum: the smaller offset


def pool_offsets(k: np.ndarray, Gh: int, Gw: int, f: int, mode: int, seed: int = 0) -> np.ndarray:
    """In-block offset of the representative token of every block, for the
    single-token modes (center, medoid, random): [..., (Gh/f)*(Gw/f)] int.
    Medoid decides per leading index (batch, head) on that head's keys."""
    k = np.asarray(k, np.float64)
    lead = k.shape[:-2]
    nb = (Gh // f) * (Gw // f)
    out = np.zeros(lead + (nb,), np.int64)
    for b in range(nb):
        by, bx = divmod(b, Gw // f)
        if mode == POOL_CENTER:
            out[..., b] = (f // 2) * f + f // 2
        elif mode == POOL_RANDOM:
            out[..., b] = pool_random_offset(seed, f, b)
        elif mode == POOL_MEDOID:
            toks = block_tokens(Gw, f, by, bx)
            for idx in np.ndindex(*lead):
                out[idx + (b,)] = medoid_offset(k[idx][toks])
        else:
            raise ValueError("pool mode")
    return out


def pool_kv(k, v, Gh: int, Gw: int, f: int, mode: int, theta: float, T: int = 0, seed: int = 0):
    """Pooled keys (rotated at integer coarse positions (by, bx)) and pooled
    values (never rotated).  Keys are pooled before rotation so that the
    pooled key carries the coarse-grid position ([summary] Phase I: pooled
    keys sit on the (W/f) x (H/f) grid).  Mean averages the block; the other
    modes take one token of the block, the same token for K and V (its
    offset from pool_offsets; medoid chooses it on the keys).  With T text
    tokens, the T text keys (position (0, 0): unrotated) and values come
    first, unpooled ([summary] Phase I: pooling applies to image tokens
    only)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    ki, vi = k[..., T:, :], v[..., T:, :]
    if mode == POOL_MEAN:
        kp = pool_tokens(ki, Gh, Gw, f, mode)
        vp = pool_tokens(vi, Gh, Gw, f, mode)
    else:
        off = pool_offsets(ki, Gh, Gw, f, mode, seed)
        nb = off.shape[-1]
        bys, bxs = np.divmod(np.arange(nb), Gw // f)
        tok = (bys * f + off // f) * Gw + (bxs * f + off % f)  # [..., nb] token per block
        kp = np.take_along_axis(ki, tok[..., None], axis=-2)
        vp = np.take_along_axis(vi, tok[..., None], axis=-2)
    by, bx = grid_positions(Gh // f, Gw // f)
    kp = apply_rope_2d(kp, by, bx, theta)
    return np.concatenate([k[..., :T, :], kp], axis=-2), np.concatenate([v[..., :T, :], vp], axis=-2)


def coarse_attention(q, kp_rot, vp, Gh: int, Gw: int, f: int, theta: float,
                     rows: Optional[np.ndarray] = None, T: int = 0) -> np.ndarray:
    """Every full-resolution image query attends to all pooled keys (and the
    T text keys that pool_kv put first); its RoPE position is its grid
    coordinate divided by f so that queries and pooled keys share one
    coordinate system ([summary] Phase I).  Cost is N (T + N/f^2) query-key
    pairs.  `rows` are image-token indices; image token n is row T + n of q."""
    y, x = grid_positions(Gh, Gw)
    if rows is None:
        rows = np.arange(Gh * Gw)
    rows = np.asarray(rows)
    qr = apply_rope_2d(np.asarray(q)[..., T + rows, :], y[rows] / f, x[rows] / f, theta)
    return attention(qr, kp_rot, vp)


# ----------------------------------------------------------------------------
# Schedules
# ----------------------------------------------------------------------------


def common_divisors(a: int, b: int, lo: int = 1) -> List[int]:
    g = math.gcd(a, b)
    return [d for d in range(max(1, lo), g + 1) if g % d == 0]


def nearest_divisor_num(Gh: int, Gw: int, f_min: int, num: int, den: int) -> int:
    """Common divisor d >= f_min of (Gh, Gw) nearest to num/den, ties to the
    larger d; exact integer comparison |d*den - num|."""
    best, bestd = None, None
    for d in common_divisors(Gh, Gw, f_min):
        dist = abs(d * den - num)
        if best is None or dist < bestd or (dist == bestd and d > best):
            best, bestd = d, dist
    if best is None:
        raise ValueError("grid sides share no factor >= f_min")
    return best


def f0_for(Gh: int, Gw: int, native_h: int, native_w: int, f_min: int) -> int:
    """READING R5: the first pooling factor matches the native grid ([summary]
    Phase I: f = 4 at 4096^2 where 256x256 tokens map to the native 64x64;
    [readme] base-resolution paragraph).  f0 = common divisor >= f_min of
    (Gh, Gw) nearest to the larger of Gh/native_h and Gw/native_w, ties to
    the larger divisor.  Compared exactly as fractions."""
    # larger ratio of the two axes, kept as a fraction num/den
    if Gh * native_w >= Gw * native_h:
        num, den = Gh, native_h
    else:
        num, den = Gw, native_w
    return nearest_divisor_num(Gh, Gw, f_min, num, den)


def pooling_ramp(Gh: int, Gw: int, f0: int, f_min: int, steps: int) -> List[int]:
    """READING R4 of the Phase I ramp ([blog] Fase I, worked example for a
    256x256 grid; [summary] Phase I): f goes linearly from f0 to f_min over
    the Phase I steps, x_t = f0 + (f_min - f0) * t / (P - 1), each value
    snapped to the nearest common divisor (>= f_min) of the grid sides, ties
    to the larger divisor.  Exact rational arithmetic."""
    if steps <= 0:
        return []
    if steps == 1:
        return [nearest_divisor_num(Gh, Gw, f_min, f0, 1)]
    P1 = steps - 1
    return [nearest_divisor_num(Gh, Gw, f_min, f0 * P1 + (f_min - f0) * t, P1) for t in range(steps)]


def window_sizes(w_start: int, w_min: int, steps: int) -> List[int]:
    """READING R6 of the Phase II shrink ([blog] Fase II; [summary] Phase II:
    windows shrink geometrically from w_start to w_min): r_t = w_start *
    (w_min / w_start)^(t / (S - 1)) in float64, rounded to the nearest even
    integer (ties up) so that quadrants stay integral."""
    out = []
    for t in range(steps):
        if steps == 1:
            r = float(w_start)
        else:
            r = w_start * math.pow(w_min / w_start, t / (steps - 1))
        out.append(2 * int(math.floor(r / 2.0 + 0.5)))
    return out


def w_start_auto(Gh: int, Gw: int, w_min: int) -> int:
    """READING R7 of the first Phase II window ([summary] Phase II: the
    first window is the biggest one whose windowed attention costs less than
    one pass of full attention, near 70% of the grid's longer side; [blog]
    Fase II gives the same rule): the largest even w in [w_min, max(Gh, Gw)] whose base tiling
    costs fewer (query, key) pairs than full attention, each window attending
    to itself: sum over the R8 windows of (min(w, Gh) * min(w, Gw))^2 <
    (Gh * Gw)^2.  w_min when no larger size qualifies."""
    N = Gh * Gw
    best = w_min
    for w in range(w_min, max(Gh, Gw) + 1):
        if w % 2:
            continue
        n = len(base_starts(Gh, w)) * len(base_starts(Gw, w))
        if n * (min(w, Gh) * min(w, Gw)) ** 2 < N * N:
            best = w
    return best


# ----------------------------------------------------------------------------
# Window tiling
# ----------------------------------------------------------------------------


def base_starts(G: int, w: int) -> List[int]:
    """READING R8 of the even base tiling ([summary] Phase II: overlap is
    spread evenly): n = ceil(G / w) windows per axis (1 if w >= G), starts
    b_i = round_half_up(i (G - w) / (n - 1)), so b_0 = 0 and the last window
    ends at G."""
    if w >= G:
        return [0]
    n = -(-G // w)
    return [(2 * i * (G - w) + (n - 1)) // (2 * (n - 1)) for i in range(n)]


def splitmix64(seed: int, k: int) -> int:
    """k-th output (k >= 1) of the SplitMix64 generator of Steele, Lea and
    Flood (OOPSLA 2014) started from `seed`: state advances by the golden
    gamma 0x9E3779B97F4A7C15, then the variant-13 finalizer mixes it."""
    z = (seed + k * 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def jitter_offset(starts: Sequence[int], w: int, seed: int, step: int, axis: int) -> int:
    """READING R9 of the per-step boundary shift ([blog] Fase II; [summary]
    Phase II: window boundaries move randomly between steps; [blog] "Cómo
    entra en tu pipeline": the seed drives the border jitter).  One offset o
    per (step, axis) in [-J, J], J = floor(min overlap / 2), drawn as
    splitmix64(seed, 2*step + axis + 1) mod (2J + 1) - J; applied to interior
    windows only.  No shift with two or fewer windows."""
    n = len(starts)
    if n <= 2:
        return 0
    gap = max(starts[i + 1] - starts[i] for i in range(n - 1))
    ov = w - gap
    J = ov // 2 if ov > 0 else 0
    if J == 0:
        return 0
    return int(splitmix64(seed, 2 * step + axis + 1) % (2 * J + 1)) - J


def axis_windows(G: int, w: int, seed: int, step: int, axis: int) -> Tuple[List[Tuple[int, int]], int]:
    """[(start, length)] along one axis after the shift, and the shift."""
    L = min(w, G)
    b = base_starts(G, w)
    o = jitter_offset(b, L, seed, step, axis)
    out = []
    for i, s in enumerate(b):
        if 0 < i < len(b) - 1:
            s += o
        out.append((s, L))
    return out, o


def detail_energy(latent: np.ndarray) -> np.ndarray:
    """READING R10: single-level orthonormal 2-D Haar transform per channel
    on 2x2 blocks (a b / c d) of the latent on the token grid ([summary]
    Phase II: a wavelet map of the hidden state gauges how much fine detail
    each region holds; [readme] Phase II bullet).  Detail energy per 2x2 cell:
        E = sum over channels (in order) of ((LH^2 + HL^2) + HH^2)
    with LH = (a - b + c - d)/2, HL = (a + b - c - d)/2, HH = (a - b - c + d)/2.
    Float64, each operation in the order written."""
    x = np.asarray(latent, dtype=np.float64)
    C, Gh, Gw = x.shape
    if Gh % 2 or Gw % 2:
        raise ValueError("grid sides must be even for the Haar map")
    a = x[:, 0::2, 0::2]
    b = x[:, 0::2, 1::2]
    c = x[:, 1::2, 0::2]
    d = x[:, 1::2, 1::2]
    E = np.zeros((Gh // 2, Gw // 2), dtype=np.float64)
    for ch in range(C):
        lh = (((a[ch] - b[ch]) + c[ch]) - d[ch]) * 0.5
        hl = (((a[ch] + b[ch]) - c[ch]) - d[ch]) * 0.5
        hh = (((a[ch] - b[ch]) - c[ch]) + d[ch]) * 0.5
        E = E + ((lh * lh + hl * hl) + hh * hh)
    return E


def haar_forward(latent: np.ndarray):
    """(LL, LH, HL, HH) subbands of the orthonormal Haar step (same formulas
    as detail_energy; LL = (a + b + c + d)/2)."""
    x = np.asarray(latent, dtype=np.float64)
    a = x[:, 0::2, 0::2]
    b = x[:, 0::2, 1::2]
    c = x[:, 1::2, 0::2]
    d = x[:, 1::2, 1::2]
    ll = (((a + b) + c) + d) * 0.5
    lh = (((a - b) + c) - d) * 0.5
    hl = (((a + b) - c) - d) * 0.5
    hh = (((a - b) - c) + d) * 0.5
    return ll, lh, hl, hh


def haar_inverse(ll, lh, hl, hh):
    a = (ll + lh + hl + hh) * 0.5
    b = (ll - lh + hl - hh) * 0.5
    c = (ll + lh - hl - hh) * 0.5
    d = (ll - lh - hl + hh) * 0.5
    C, h, w = ll.shape
    x = np.empty((C, 2 * h, 2 * w))
    x[:, 0::2, 0::2] = a
    x[:, 0::2, 1::2] = b
    x[:, 1::2, 0::2] = c
    x[:, 1::2, 1::2] = d
    return x


def energy_fixed(E: np.ndarray) -> np.ndarray:
    """READING R11: fixed-point copy E_q = min(round_half_even(E * 2^16),
    2^31 - 1) as int32, so every later sum is an exact integer."""
    q = np.rint(np.asarray(E, np.float64) * 65536.0)
    q = np.minimum(q, 2147483647.0)
    return q.astype(np.int64).astype(np.int32)


@dataclass
class Window:
    qy0: int
    qx0: int
    qh: int
    qw: int
    ky0: int
    kx0: int
    kh: int
    kw: int
    parent: int
    quadrant: int      # -1: not split; 0..3 = TL, TR, BL, BR

    def as_tuple(self):
        return (self.qy0, self.qx0, self.qh, self.qw, self.ky0, self.kx0, self.kh, self.kw,
                self.parent, self.quadrant)


@dataclass
class Plan:
    step: int
    w: int
    ny: int
    nx: int
    jit_y: int
    jit_x: int
    halo: int
    windows: List[Window] = field(default_factory=list)
    wsum: Optional[np.ndarray] = None       # int32 [Gh*Gw]

    def records(self) -> np.ndarray:
        return np.array([w.as_tuple() for w in self.windows], dtype=np.int32).reshape(-1, 10)


def window_score(Eq: np.ndarray, y0: int, x0: int, h: int, w: int) -> int:
    """Sum over the window's tokens (y, x) of E_q[y // 2, x // 2] (exact)."""
    ys = np.arange(y0, y0 + h) // 2
    xs = np.arange(x0, x0 + w) // 2
    return int(np.asarray(Eq, np.int64)[np.ix_(ys, xs)].sum())


def halo_rect(y0, x0, h, w, delta, Gh, Gw):
    """READING R14: the Halo dilates the window by delta tokens on every side,
    clipped to the grid ([blog] Fase II; [summary] Phase II)."""
    ky0 = max(0, y0 - delta)
    kx0 = max(0, x0 - delta)
    ky1 = min(Gh, y0 + h + delta)
    kx1 = min(Gw, x0 + w + delta)
    return ky0, kx0, ky1 - ky0, kx1 - kx0


HALO_STREAM = 0x48414C4F  # "HALO": Halo widths use their own SplitMix64 stream


def halo_width(seed: int, step: int, base: int, quadrant: int, halo_max: int) -> int:
    """READING R18 of the randomised Halo ([blog] Fase II: a Halo of up to
    delta_max = 8 patches; [blog] "Cómo entra en tu pipeline": the seed
    controls the Halo widths; [summary] Phase II: delta_max set to 8): every
    window of every step (a quadrant is a window of its own) draws its width
    uniformly from 1..halo_max, as
    1 + splitmix64(seed ^ HALO_STREAM, 1 + (step * 4096 + base) * 5 + quadrant + 1) mod halo_max,
    with base the row-major index of its base window and quadrant -1 for an
    unsplit window."""
    k = 1 + (step * 4096 + base) * 5 + (quadrant + 1)
    return 1 + int(splitmix64(seed ^ HALO_STREAM, k) % halo_max)


def bridge_size(w: int, rho_num: int, rho_den: int) -> int:
    """READING R19 ([summary] Phase II: each window gains R = (rho w_t)^2
    bridge tokens, rho = 0.5; [blog] Fase II, same): R_t = round_half_up(rho *
    w_t)^2 with w_t the step's scheduled window side (one bridge set per step,
    shared by its windows and quadrants)."""
    side = (2 * rho_num * w + rho_den) // (2 * rho_den)
    return side * side


def tent(L: int) -> np.ndarray:
    """READING R15: centre weight along one axis, min(u + 1, L - u)."""
    u = np.arange(L)
    return np.minimum(u + 1, L - u).astype(np.int64)


def window_plan(Gh: int, Gw: int, w: int, halo: int, seed: int, step: int,
                Eq: Optional[np.ndarray], split_num: int = 1, split_den: int = 2,
                halo_max: int = 0) -> Plan:
    """Phase II window list for one step ([summary] Phase II; [readme]
    repository layout: tiling covers base tiling, DWT map, splits, Halo and
    merge weights).

    Base windows (R8 tiling, R9 shift) in row-major order; a window whose
    mean detail is below split_num/split_den of the grid's mean detail is
    replaced in place by its four quadrants TL, TR, BL, BR (READING R12:
    split iff den * S_w * N < num * S_tot * |Q_w| with S the integer sums of
    E_q over tokens).  Each window then gets its Halo rectangle (width
    `halo`, or a seeded width per window from halo_width when halo_max > 0)
    and its tent weights accumulate into wsum."""
    N = Gh * Gw
    ys, oy = axis_windows(Gh, w, seed, step, 0)
    xs, ox = axis_windows(Gw, w, seed, step, 1)
    plan = Plan(step=step, w=w, ny=len(ys), nx=len(xs), jit_y=oy, jit_x=ox, halo=halo)
    S_tot = window_score(Eq, 0, 0, Gh, Gw) if Eq is not None else 0
    parent = 0
    for (y0, h) in ys:
        for (x0, wd) in xs:
            rects = [(y0, x0, h, wd, -1)]
            if Eq is not None and h >= 2 and wd >= 2:
                S_w = window_score(Eq, y0, x0, h, wd)
                if split_den * S_w * N < split_num * S_tot * (h * wd):
                    h1, w1 = h // 2, wd // 2
                    rects = [(y0, x0, h1, w1, 0), (y0, x0 + w1, h1, wd - w1, 1),
                             (y0 + h1, x0, h - h1, w1, 2), (y0 + h1, x0 + w1, h - h1, wd - w1, 3)]
            for (ry, rx, rh, rw, quad) in rects:
                delta = halo_width(seed, step, parent, quad, halo_max) if halo_max > 0 else halo
                ky0, kx0, kh, kw = halo_rect(ry, rx, rh, rw, delta, Gh, Gw)
                plan.windows.append(Window(ry, rx, rh, rw, ky0, kx0, kh, kw, parent, quad))
            parent += 1
    wsum = np.zeros((Gh, Gw), dtype=np.int64)
    for win in plan.windows:
        wsum[win.qy0:win.qy0 + win.qh, win.qx0:win.qx0 + win.qw] += np.outer(tent(win.qh), tent(win.qw))
    plan.wsum = wsum.reshape(-1).astype(np.int32)
    return plan


# ----------------------------------------------------------------------------
# Global-KV bridge
# ----------------------------------------------------------------------------


def bridge_cells(R: int, Gh: int, Gw: int) -> Tuple[int, int]:
    """READING R13 (spatial spread, [summary] Phase II): the bridge takes one
    token from each cell of an r_h x r_w grid of R = r_h * r_w cells.  Among
    the factor pairs of R with r_h <= Gh and r_w <= Gw, the cells are the
    most nearly square in tokens: a cell is (Gh / r_h) x (Gw / r_w) tokens, so
    its elongation is max(Gh r_w, Gw r_h) / min(Gh r_w, Gw r_h), compared
    exactly as integer cross products; equal elongations go to the smaller
    r_h (fewer, taller cell rows).  No pair fits: ValueError."""
    best = None
    for rh in range(1, R + 1):
        if R % rh:
            continue
        rw = R // rh
        if rh > Gh or rw > Gw:
            continue
        a, b = Gh * rw, Gw * rh           # cell height : cell width = a : b
        hi, lo = max(a, b), min(a, b)
        if best is None or hi * best[1] < best[0] * lo:
            best = (hi, lo, rh, rw)
    if best is None:
        raise ValueError("no r_h x r_w = R cell grid fits the token grid")
    return best[2], best[3]


K_MEAN_CLAMP = 2.0 ** 28   # keys saturate here inside the mean-key sum only
BRIDGE_CHUNK = 1024         # rows per exact int64 partial sum


def bridge_scores(kbh: np.ndarray) -> np.ndarray:
    """Deviation of every key from the head's global mean key ([summary]
    Phase II: bridge tokens are chosen by their deviation from the global
    mean key).  READING R13: kbh [N, D] un-rotated keys.  The mean is exact:
    keys (saturated at +-2^28) in fixed point round_half_even(k * 2^24)
    summed as integers, the sum T rounded once to float64, then
    mu_d = T / (2^24 * N) in one float64 division.  The score is
    s_j = sum over d ascending of (k_jd - mu_d)^2 in float64 (no fused
    multiply-add)."""
    k = np.asarray(kbh, dtype=np.float64)
    N, D = k.shape
    # Keys enter the mean saturated at +-2^28 (so |kq| <= 2^52 and any 1024
    # rows sum exactly in int64); the total over all rows is an exact
    # integer T, converted to float64 once (rounded to nearest) as
    # hi * 2^32 + lo with hi = floor(T / 2^32), both parts exact in float64.
    kq = np.rint(np.clip(k, -K_MEAN_CLAMP, K_MEAN_CLAMP) * 16777216.0).astype(np.int64)
    pad = (-N) % BRIDGE_CHUNK
    chunks = np.concatenate([kq, np.zeros((pad, D), np.int64)]).reshape(-1, BRIDGE_CHUNK, D).sum(axis=1)
    mu = np.empty(D, dtype=np.float64)
    for d in range(D):
        T = sum(int(x) for x in chunks[:, d])  # exact (Python integers)
        mu[d] = (float(T >> 32) * 4294967296.0 + float(T & 0xFFFFFFFF)) / (16777216.0 * N)
    s = np.zeros(N, dtype=np.float64)
    for d in range(D):
        t = k[:, d] - mu[d]
        s = s + t * t
    return s


def bridge_select(kbh: np.ndarray, R: int, Gh: int, Gw: int) -> np.ndarray:
    """R bridge token indices for one (batch, head): the highest-scoring
    token of each cell (ties to the smaller index), sorted ascending."""
    s = bridge_scores(kbh)
    rh, rw = bridge_cells(R, Gh, Gw)
    out = []
    for a in range(rh):
        y0, y1 = a * Gh // rh, (a + 1) * Gh // rh
        for c in range(rw):
            x0, x1 = c * Gw // rw, (c + 1) * Gw // rw
            best, bi = None, -1
            for y in range(y0, y1):
                row = s[y * Gw + x0:y * Gw + x1]
                j = int(np.argmax(row))      # first maximum = smallest index
                if best is None or row[j] > best:
                    best, bi = row[j], y * Gw + x0 + j
            out.append(bi)
    return np.sort(np.array(out, dtype=np.int32))


def bridge_all(k: np.ndarray, R: int, Gh: int, Gw: int) -> np.ndarray:
    """[B, H, R] int32 bridge indices, one set per (batch, head)."""
    B, H = k.shape[:2]
    out = np.zeros((B, H, R), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            out[b, h] = bridge_select(k[b, h], R, Gh, Gw)
    return out


# ----------------------------------------------------------------------------
# Phase II: windowed attention with Halo, bridge and centre-weighted blending
# ----------------------------------------------------------------------------


def window_key_indices(win: Window, Gw: int, bridge: Optional[np.ndarray]) -> np.ndarray:
    """Keys of one window: its Halo rectangle, plus the bridge tokens that
    lie outside that rectangle (the bridge brings tokens from the rest of
    the grid; no key appears twice)."""
    ys = np.arange(win.ky0, win.ky0 + win.kh)
    xs = np.arange(win.kx0, win.kx0 + win.kw)
    rect = (ys[:, None] * Gw + xs[None, :]).reshape(-1)
    if bridge is None or len(bridge) == 0:
        return rect
    by, bx = np.asarray(bridge) // Gw, np.asarray(bridge) % Gw
    outside = ~((by >= win.ky0) & (by < win.ky0 + win.kh) & (bx >= win.kx0) & (bx < win.kx0 + win.kw))
    return np.concatenate([rect, np.asarray(bridge)[outside]])


def window_query_indices(win: Window, Gw: int) -> np.ndarray:
    ys = np.arange(win.qy0, win.qy0 + win.qh)
    xs = np.arange(win.qx0, win.qx0 + win.qw)
    return (ys[:, None] * Gw + xs[None, :]).reshape(-1)


def window_attention(q, k, v, plan: Plan, bridge: Optional[np.ndarray], Gh: int, Gw: int,
                     theta: float, rows: Optional[np.ndarray] = None, T: int = 0) -> np.ndarray:
    """Phase II output [B, H, len(rows), D] (float64) for image tokens `rows`.

    Each window's queries attend to the window's keys (Halo rectangle plus
    outside bridge tokens, plus the T text keys, READING R20) with RoPE at
    native grid positions; the outputs of the windows covering a token are
    averaged with the windows' tent weights (READING R15 of the
    centre-weighted blend, [summary] Phase II).  q, k, v are [B, H, T + N, D]
    with image token n at row T + n; bridge holds image-token indices."""
    q = np.asarray(q, np.float64)[..., T:, :]
    kt = np.asarray(k, np.float64)[..., :T, :]
    vt = np.asarray(v, np.float64)[..., :T, :]
    k = np.asarray(k, np.float64)[..., T:, :]
    v = np.asarray(v, np.float64)[..., T:, :]
    B, H, N, D = q.shape
    y, x = grid_positions(Gh, Gw)
    kr = apply_rope_2d(k, y, x, theta)
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    pos_of = -np.ones(N, dtype=np.int64)
    pos_of[rows] = np.arange(len(rows))
    acc = np.zeros((B, H, len(rows), D))
    for win in plan.windows:
        qi = window_query_indices(win, Gw)
        sel = pos_of[qi] >= 0
        if not np.any(sel):
            continue
        qi = qi[sel]
        wt = np.outer(tent(win.qh), tent(win.qw)).reshape(-1)[sel].astype(np.float64)
        qr = apply_rope_2d(q[..., qi, :], y[qi], x[qi], theta)
        for b in range(B):
            for h in range(H):
                ki = window_key_indices(win, Gw, None if bridge is None else bridge[b, h])
                o = attention(qr[b, h], np.concatenate([kt[b, h], kr[b, h, ki]]),
                              np.concatenate([vt[b, h], v[b, h, ki]]))
                acc[b, h, pos_of[qi]] += wt[:, None] * o
    ws = plan.wsum[rows].astype(np.float64)
    if np.any(ws <= 0):
        raise ValueError("a requested token is covered by no window")
    return acc / ws[None, None, :, None]


# ----------------------------------------------------------------------------
# Canvas gating and the per-step phase
# ----------------------------------------------------------------------------

PHASE_FULL, PHASE_COARSE, PHASE_WINDOW = 0, 1, 2


def canvas_check(Gh: int, Gw: int, native_h: int, native_w: int, f_min: int = 2) -> int:
    """[readme] canvas-rules paragraph and [blog] "Cómo entra en tu
    pipeline": a canvas no larger than the native one runs the model's own
    (full) attention; a larger one needs patch counts along the two sides
    with a common factor >= 2, because Phase I pools square f x f blocks.  Returns PHASE_FULL for the gated case and
    -1 when the grid cannot be pooled, else PHASE_COARSE."""
    if Gh <= native_h and Gw <= native_w:
        return PHASE_FULL
    if math.gcd(Gh, Gw) < max(2, f_min):
        return -1
    return PHASE_COARSE


def step_phases(p1_steps: int, p2_steps: int) -> List[int]:
    """READING R16: a fixed count of coarse steps, then the window steps
    ([summary] Scheduling the switch: 8 steps for FLUX.1, 20 for
    Qwen-Image).  phase1_steps_for_sigma turns a sampler's noise levels and
    a threshold sigma* into that count."""
    return [PHASE_COARSE] * p1_steps + [PHASE_WINDOW] * p2_steps


def phase1_steps_for_sigma(sigmas: Sequence[float], sigma_star: float) -> int:
    """READING R23 ([summary] Scheduling the switch and [readme] sigma*
    paragraph: the switch from Phase I to Phase II is a noise level sigma*,
    not a step count): Phase I runs the leading steps whose noise level is
    above sigma*; the first step at or below sigma* starts Phase II, and
    every later step stays there."""
    n = 0
    for s in sigmas:
        if not s > sigma_star:
            break
        n += 1
    return n
