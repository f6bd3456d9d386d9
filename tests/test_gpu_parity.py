"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small workloads are compared element by element; the full-size FLUX.1
workloads on sampled outputs the oracle computes one by one.  Plans, blend
weight sums and bridge indices must match bit for bit; attention outputs
within max-abs 2e-2 and mean-abs 2e-3 (bf16 inputs and outputs against the
float64 oracle fed the same bf16-rounded inputs)."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import resolution_diffusion_transformer_amd as A
import workloads as W
from oracle import area_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3
# pooled keys and values are fp32; keys carry the fp32 rotation's error (angles
# up to ~400 rad rounded to fp32: a few 1e-5 relative)
POOLED_MAX, POOLED_MEAN = 1e-3, 1e-4


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


def assert_close(got, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    say(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= max_abs, (what, err.max())
    assert err.mean() <= mean_abs, (what, err.mean())


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def inputs(name, device):
    wl = W.get(name)
    q, k, v = W.make_qkv(wl, device=device, dtype="bf16")
    return wl, q.cuda(), k.cuda(), v.cuda()


# ------------------------------------------------------------ tiny, dense --

@pytest.fixture(scope="module")
def tiny():
    wl, q, k, v = inputs("tiny-32", "cpu")
    return wl, q, k, v, to_host(q), to_host(k), to_host(v)


def test_full_attention_tiny(tiny):
    wl, q, k, v, qh, kh, vh = tiny
    p = A.problem_for(wl)
    out = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    ref = O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta)
    assert_close(to_host(out), ref, "full tiny")


@pytest.mark.parametrize("mode", [A.POOL_MEAN, A.POOL_CENTER, A.POOL_MEDOID, A.POOL_RANDOM])
@pytest.mark.parametrize("f", [1, 2, 4])
def test_pool_and_coarse_tiny(tiny, mode, f):
    wl, q, k, v, qh, kh, vh = tiny
    p = A.problem_for(wl, pool_mode=mode, seed=11)
    kp, vp = A.area_pool_kv(p, f, k, v)
    out = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    kp_ref, vp_ref = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, mode, wl.rope_theta, seed=11)
    if mode != A.POOL_MEAN:
        # one token per block, the same as the oracle's: the pooled V rows are the chosen
        # tokens' values, bit for bit
        np.testing.assert_array_equal(vp.cpu().numpy(), vp_ref.astype(np.float32), f"vp tokens f={f} mode={mode}")
    # pooled tensors are fp32: the block sum and one division, keys turned by an fp32
    # (cos, sin) of fp32 angles
    assert_close(to_host(kp), kp_ref, f"kp f={f} mode={mode}", max_abs=POOLED_MAX, mean_abs=POOLED_MEAN)
    assert_close(to_host(vp), vp_ref, f"vp f={f} mode={mode}", max_abs=POOLED_MAX, mean_abs=POOLED_MEAN)
    ref = O.coarse_attention(qh, kp_ref, vp_ref, wl.Gh, wl.Gw, f, wl.rope_theta)
    assert_close(to_host(out), ref, f"coarse f={f} mode={mode}")


@pytest.fixture(scope="module")
def grid48():
    """A 48 x 48 grid (native 16 x 16), so that the odd factor 3 and the
    factor 6 of the 6144^2 pooling ramp can be checked element by element."""
    wl = W.Workload("grid-48", B=1, H=2, D=128, Gh=48, Gw=48, native_h=16, native_w=16, dtype="bf16",
                    p1_steps=4, f_min=2, p2_steps=0, w_start=16, w_min=8, halo=1, bridge_k=16,
                    latent_kind="tiny_patches")
    q, k, v = W.make_qkv(wl, device="cpu", dtype="bf16")
    return wl, q.cuda(), k.cuda(), v.cuda(), to_host(q), to_host(k), to_host(v)


@pytest.mark.parametrize("mode", [A.POOL_MEAN, A.POOL_CENTER, A.POOL_MEDOID, A.POOL_RANDOM])
@pytest.mark.parametrize("f", [3, 6])
def test_pool_and_coarse_odd_factors(grid48, mode, f):
    # f = 3: query positions y/3, x/3 are not binary fractions, so the (cos, sin)
    # table built with divisor 3 is exercised; f = 6 pools 6 x 6 blocks
    wl, q, k, v, qh, kh, vh = grid48
    say(f"grid-48 f={f} mode={mode}")
    p = A.problem_for(wl, pool_mode=mode, seed=5)
    assert A.area_f0(p) == 3
    kp, vp = A.area_pool_kv(p, f, k, v)
    out = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    kp_ref, vp_ref = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, mode, wl.rope_theta, seed=5)
    assert_close(to_host(kp), kp_ref, f"kp f={f} mode={mode}", max_abs=POOLED_MAX, mean_abs=POOLED_MEAN)
    assert_close(to_host(vp), vp_ref, f"vp f={f} mode={mode}", max_abs=POOLED_MAX, mean_abs=POOLED_MEAN)
    ref = O.coarse_attention(qh, kp_ref, vp_ref, wl.Gh, wl.Gw, f, wl.rope_theta)
    assert_close(to_host(out), ref, f"grid-48 coarse f={f} mode={mode}")


def test_coarse_f1_equals_full_on_gpu(tiny):
    wl, q, k, v, *_ = tiny
    p = A.problem_for(wl, pool_mode=A.POOL_CENTER)
    kp, vp = A.area_pool_kv(p, 1, k, v)
    a = A.area_coarse_attn(p, 1, q, kp, vp)
    b = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    # identical inputs after one rounding of the rotated keys: equal up to bf16 rounding
    assert_close(to_host(a), to_host(b), "coarse(f=1) vs full", max_abs=1e-2, mean_abs=1e-3)


# ------------------------------------------------------------ tiny, Phase II --

def test_dwt_detail_bit_exact():
    for name in ("tiny-32", "flux-2048", "flux-6144", "qwen-6144x2048"):
        wl = W.get(name)
        lat = W.make_latent(wl)
        p = A.problem_for(wl)
        E, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
        torch.cuda.synchronize()
        E_ref = O.detail_energy(lat)
        Eq_ref = O.energy_fixed(E_ref)
        assert np.array_equal(Eq.cpu().numpy(), Eq_ref), name
        np.testing.assert_array_equal(E.cpu().numpy(), E_ref.astype(np.float32))


def plan_records(plan_t):
    pl = plan_t.cpu().numpy()
    nwin = int(pl[0])
    return pl[:A.PLAN_HEADER], pl[A.PLAN_HEADER:A.PLAN_HEADER + A.PLAN_REC * nwin].reshape(nwin, A.PLAN_REC)


def check_plan_step(wl, p, step, Eq_dev, Eq_ref, k_dev, k_host, heads=None):
    t = step - wl.p1_steps
    w = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)[t]
    plan, wsum, br = A.area_window_plan(p, step, Eq_dev, k_dev)
    torch.cuda.synchronize()
    ref = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq_ref)
    hdr, recs = plan_records(plan)
    assert hdr[A.PLAN_HEADER - 16 + 0] == len(ref.windows)
    assert (hdr[1], hdr[2], hdr[3], hdr[4], hdr[5], hdr[6], hdr[7]) == \
        (t, w, ref.ny, ref.nx, ref.jit_y, ref.jit_x, wl.halo)
    np.testing.assert_array_equal(recs, ref.records())
    np.testing.assert_array_equal(wsum.cpu().numpy(), ref.wsum)
    br_ref = None
    if br is not None:
        bh = br.cpu().numpy()
        hs = range(wl.H) if heads is None else heads
        br_ref = np.zeros_like(bh)
        for h in hs:
            br_ref[0, h] = O.bridge_select(k_host[0, h], wl.bridge_k, wl.Gh, wl.Gw)
            np.testing.assert_array_equal(bh[0, h], br_ref[0, h], err_msg=f"bridge head {h}")
    return plan, wsum, br, ref, br_ref


def test_window_plan_and_attention_tiny(tiny):
    wl, q, k, v, qh, kh, vh = tiny
    p = A.problem_for(wl)
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    for t in range(wl.p2_steps):
        step = wl.p1_steps + t
        plan, wsum, br, ref, br_ref = check_plan_step(wl, p, step, Eq, Eq_ref, k, kh)
        out = A.area_window_attn(p, step, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        o_ref = O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta)
        assert_close(to_host(out), o_ref, f"window tiny step {t} (w={ref.w}, {len(ref.windows)} windows)")


def test_window_whole_grid_equals_full_gpu(tiny):
    # a single window covering the grid, with a bridge: every bridge token is
    # inside the Halo rectangle, so the result is full attention
    wl, q, k, v, qh, kh, vh = tiny
    p = A.problem_for(wl, p2_steps=1, w_start=wl.Gh, w_min=wl.Gh)
    plan, wsum, br = A.area_window_plan(p, wl.p1_steps, None, k)
    out = A.area_window_attn(p, wl.p1_steps, plan, wsum, br, q, k, v)
    full = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    hdr, recs = plan_records(plan)
    assert hdr[0] == 1
    assert torch.equal(out, full)


def test_window_no_bridge_no_split_tiny(tiny):
    wl, q, k, v, qh, kh, vh = tiny
    p = A.problem_for(wl, bridge_k=0, halo=0)
    step = wl.p1_steps + 2
    plan, wsum, br = A.area_window_plan(p, step, None, None)
    assert br is None
    out = A.area_window_attn(p, step, plan, wsum, None, q, k, v)
    torch.cuda.synchronize()
    t = 2
    w = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)[t]
    ref = O.window_plan(wl.Gh, wl.Gw, w, 0, wl.seed, t, None)
    o_ref = O.window_attention(qh, kh, vh, ref, None, wl.Gh, wl.Gw, wl.rope_theta)
    assert_close(to_host(out), o_ref, "window tiny no bridge/split")


@pytest.fixture(scope="module")
def one_head16():
    """One head on a 16 x 16 grid: full and coarse attention are a single work
    item and each window step has a handful, fewer than the 8 per-XCD shares
    of the persistent attention kernel, so most work-groups find every share
    empty and leave."""
    wl = W.Workload("one-head-16", B=1, H=1, D=128, Gh=16, Gw=16, native_h=8, native_w=8, dtype="bf16",
                    p1_steps=2, f_min=2, p2_steps=2, w_start=8, w_min=6, halo=1, bridge_k=4,
                    latent_kind="half_columns")
    q, k, v = W.make_qkv(wl, device="cpu", dtype="bf16")
    return wl, q.cuda(), k.cuda(), v.cuda(), to_host(q), to_host(k), to_host(v)


def test_fewer_items_than_xcd_shares(one_head16):
    wl, q, k, v, qh, kh, vh = one_head16
    p = A.problem_for(wl)
    out = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    assert_close(to_host(out), O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta), "one head full (1 item)")
    f = 2
    kp, vp = A.area_pool_kv(p, f, k, v)
    out = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    kp_ref, vp_ref = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, A.POOL_MEAN, wl.rope_theta)
    assert_close(to_host(out), O.coarse_attention(qh, kp_ref, vp_ref, wl.Gh, wl.Gw, f, wl.rope_theta),
                 "one head coarse (1 item)")
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    for t in range(wl.p2_steps):
        step = wl.p1_steps + t
        plan, wsum, br, ref, br_ref = check_plan_step(wl, p, step, Eq, Eq_ref, k, kh)
        out = A.area_window_attn(p, step, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        o_ref = O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta)
        assert_close(to_host(out), o_ref, f"one head window step {t} ({len(ref.windows)} windows)")


# ------------------------------------------------- flux-2048, full size ----

@pytest.fixture(scope="module")
def flux2048():
    say("generating flux-2048 inputs on the GPU")
    wl, q, k, v = inputs("flux-2048", "cuda")
    return wl, q, k, v, to_host(q), to_host(k), to_host(v)


def sample_rows(wl, n=96, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, wl.Gw - 1, wl.N - 1, wl.N - wl.Gw, (wl.Gh // 2) * wl.Gw + wl.Gw // 2]
    return np.unique(np.concatenate([fixed, rng.integers(0, wl.N, n)]))


def test_full_attention_2048_sampled(flux2048):
    wl, q, k, v, qh, kh, vh = flux2048
    p = A.problem_for(wl)
    out = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    rows = sample_rows(wl)
    oh = to_host(out)
    for h in (0, 7, 23):
        ref = O.full_attention(qh[:, h:h + 1], kh[:, h:h + 1], vh[:, h:h + 1], wl.Gh, wl.Gw,
                               wl.rope_theta, rows=rows)
        assert_close(oh[:, h:h + 1, rows], ref, f"full 2048 head {h}")


def test_coarse_2048_sampled(flux2048):
    wl, q, k, v, qh, kh, vh = flux2048
    p = A.problem_for(wl)
    f = A.area_f0(p)
    kp, vp = A.area_pool_kv(p, f, k, v)
    out = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    rows = sample_rows(wl)
    oh = to_host(out)
    for h in (0, 23):
        kp_ref, vp_ref = O.pool_kv(kh[:, h:h + 1], vh[:, h:h + 1], wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta)
        assert_close(to_host(kp)[:, h:h + 1], kp_ref, f"kp 2048 head {h}")
        ref = O.coarse_attention(qh[:, h:h + 1], kp_ref, vp_ref, wl.Gh, wl.Gw, f, wl.rope_theta, rows=rows)
        assert_close(oh[:, h:h + 1, rows], ref, f"coarse 2048 head {h}")


def test_window_2048_every_step(flux2048):
    wl, q, k, v, qh, kh, vh = flux2048
    p = A.problem_for(wl)
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    rows = sample_rows(wl, 64, seed=3)
    for t in range(wl.p2_steps):
        step = wl.p1_steps + t
        heads = [0, 11, 23] if t in (0, 1, wl.p2_steps - 1) else [5]
        plan, wsum, br, ref, br_ref = check_plan_step(wl, p, step, Eq, Eq_ref, k, kh, heads=heads)
        if t not in (0, 1, wl.p2_steps - 1):
            continue
        out = A.area_window_attn(p, step, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        oh = to_host(out)
        for h in heads:
            o_ref = O.window_attention(qh[:, h:h + 1], kh[:, h:h + 1], vh[:, h:h + 1], ref,
                                       br_ref[:, h:h + 1], wl.Gh, wl.Gw, wl.rope_theta, rows=rows)
            assert_close(oh[:, h:h + 1, rows], o_ref, f"window 2048 step {t} head {h}")


def test_measured_mfma_peak_is_plausible():
    # register-only MFMA stream: below the published 2.5 PF (the clock under load is below
    # nominal), and far above what any memory-bound kernel could reach
    t = A.area_measure_mfma_peak()
    assert 500.0 < t < 2600.0, t


@pytest.mark.parametrize("mode", [A.POOL_MEDOID, A.POOL_RANDOM])
def test_single_token_pooling_2048(flux2048, mode):
    # 128 x 128 grid, D = 128, f = 2 and 4: the chosen token of every block of two heads
    # equals the oracle's (medoid decides in float64 in the same order as the oracle)
    wl, q, k, v, qh, kh, vh = flux2048
    p = A.problem_for(wl, pool_mode=mode, seed=5)
    for f in (2, 4):
        kp, vp = A.area_pool_kv(p, f, k, v)
        torch.cuda.synchronize()
        got = vp.cpu().numpy()
        for h in (0, 13):
            _, vp_ref = O.pool_kv(kh[:, h:h + 1], vh[:, h:h + 1], wl.Gh, wl.Gw, f, mode, wl.rope_theta, seed=5)
            np.testing.assert_array_equal(got[:, h:h + 1], vp_ref.astype(np.float32), f"f={f} head {h}")


# ------------------------------------------------ running-maximum moves --

@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_running_maximum_moves(direction):
    """Scores that climb along the key sequence make every later tile exceed
    the running maximum by far more than 8 log2 units (a lane's P sum above
    2^8), so the rescale path (O and l rescaled, P recomputed, pending scores
    and accumulator start moved) runs on almost every tile; falling scores
    keep the first tile's maximum.  The ramp sits on the lowest-frequency rotation pair of the row
    half, which RoPE barely turns on a 32 x 32 grid: q carries 8 there, k the
    ramp 0 .. 256 (about 23 log2 units per 64-key tile)."""
    wl = W.get("tiny-32")
    p = A.problem_for(wl)
    q, k, v = W.make_qkv(wl, device="cpu", dtype="bf16")
    N, D = wl.N, wl.D
    ch = D // 2 - 2
    j = torch.arange(N, dtype=torch.float32)
    ramp = 256.0 * (j if direction == "rising" else (N - 1 - j)) / N
    q[..., ch] = 8.0
    q[..., ch + 1] = 0.0
    k[..., ch] = ramp.to(torch.bfloat16)
    k[..., ch + 1] = 0.0
    # the outputs nearly copy single value rows here, so their bf16 rounding
    # sets the error floor: halve V (exact in bf16) to keep clear of the bound
    v = v * 0.5
    qh, kh, vh = to_host(q), to_host(k), to_host(v)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    full = A.area_full_attn(p, q, k, v)
    f = A.area_step_info(p, 0)["f"]
    kp, vp = A.area_pool_kv(p, f, k, v)
    co = A.area_coarse_attn(p, f, q, kp, vp)
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    s = wl.p1_steps
    plan, wsum, br = A.area_window_plan(p, s, Eq, k)
    win = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
    torch.cuda.synchronize()
    assert_close(to_host(full), O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta),
                 f"full attention, {direction} scores")
    kpr, vpr = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta)
    assert_close(to_host(co), O.coarse_attention(qh, kpr, vpr, wl.Gh, wl.Gw, f, wl.rope_theta),
                 f"coarse attention f={f}, {direction} scores")
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    w0 = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)[0]
    ref = O.window_plan(wl.Gh, wl.Gw, w0, wl.halo, wl.seed, 0, Eq_ref)
    br_ref = O.bridge_all(kh, wl.bridge_k, wl.Gh, wl.Gw)
    np.testing.assert_array_equal(br.cpu().numpy(), br_ref)
    assert_close(to_host(win), O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta),
                 f"window attention w={w0}, {direction} scores")
