"""GPU parity at the full FLUX.1 / Qwen-Image sizes, in the configuration
bench.py times, plus edge cases (ragged key counts, batch > 1, block-centre
pooling).

Full-size outputs are checked on sampled tokens the oracle computes one by
one (including window seams, overlap bands and tokens of split windows);
window plans and blend-weight sums are compared bit for bit at every Phase II
step, bridge indices on sampled heads."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import resolution_diffusion_transformer_amd as A
import workloads as W
from oracle import area_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def say(*a):
    print("[gpu-fullsize]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


def close(got, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    say(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} (n={err.size})")
    assert err.max() <= max_abs and err.mean() <= mean_abs, what


def head(t, h):
    return t[:, h:h + 1].float().cpu().numpy().astype(np.float64)


def rows_for(wl, plan, n_random=48, seed=0):
    """Random tokens plus window corners, seam/overlap tokens and the first
    token of every quadrant of a split window."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = set(rng.integers(0, wl.N, n_random).tolist())
    pick |= {0, wl.Gw - 1, wl.N - wl.Gw, wl.N - 1}
    if plan is not None:
        for win in plan.windows[::max(1, len(plan.windows) // 12)]:
            pick.add(win.qy0 * wl.Gw + win.qx0)
            y1, x1 = win.qy0 + win.qh - 1, win.qx0 + win.qw - 1
            pick.add(y1 * wl.Gw + x1)
        cov = np.zeros((wl.Gh, wl.Gw), dtype=np.int32)
        for win in plan.windows:
            cov[win.qy0:win.qy0 + win.qh, win.qx0:win.qx0 + win.qw] += 1
        ov = np.flatnonzero(cov.reshape(-1) > 1)      # tokens blended from several windows
        if len(ov):
            pick |= set(rng.choice(ov, min(16, len(ov)), replace=False).tolist())
    return np.array(sorted(pick))


FULLSIZE = ["flux-4096", "flux-6144", "qwen-6144x2048"]


@pytest.fixture(scope="module", params=FULLSIZE)
def big(request):
    wl = W.get(request.param)
    say(f"generating {wl.name} on the GPU")
    q, k, v = W.make_qkv(wl, device="cuda", dtype="bf16")
    yield wl, q, k, v
    del q, k, v
    torch.cuda.empty_cache()


def test_full_attention_sampled(big):
    wl, q, k, v = big
    p = A.problem_for(wl)
    out = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    rows = rows_for(wl, None)
    for h in (0, wl.H - 1):
        ref = O.full_attention(head(q, h), head(k, h), head(v, h), wl.Gh, wl.Gw, wl.rope_theta, rows=rows)
        close(head(out, h)[:, :, rows], ref, f"{wl.name} full head {h}")


def test_coarse_attention_sampled(big):
    """Every distinct pooling factor of the workload's ramp with mean pooling,
    as bench.py times it (6144^2: f = 6, 4, 3, 2), and the last factor with
    block-centre pooling."""
    wl, q, k, v = big
    p_mean = A.problem_for(wl, pool_mode=A.POOL_MEAN)
    ramp = [A.area_step_info(p_mean, s)["f"] for s in range(wl.p1_steps)]
    cases = [(f, A.POOL_MEAN) for f in sorted(set(ramp), reverse=True)] + [(ramp[-1], A.POOL_CENTER)]
    rows = rows_for(wl, None, seed=1)
    for f, mode in cases:
        say(f"{wl.name} coarse f={f} mode={mode}")
        p = A.problem_for(wl, pool_mode=mode)
        kp, vp = A.area_pool_kv(p, f, k, v)
        out = A.area_coarse_attn(p, f, q, kp, vp)
        torch.cuda.synchronize()
        for h in (3, wl.H - 2):
            kpr, vpr = O.pool_kv(head(k, h), head(v, h), wl.Gh, wl.Gw, f, mode, wl.rope_theta)
            close(head(kp, h), kpr, f"{wl.name} pooled keys f={f} mode={mode} head {h}", 1e-3, 1e-4)
            ref = O.coarse_attention(head(q, h), kpr, vpr, wl.Gh, wl.Gw, f, wl.rope_theta, rows=rows)
            close(head(out, h)[:, :, rows], ref, f"{wl.name} coarse f={f} mode={mode} head {h}")
        del kp, vp, out


def test_window_steps(big):
    wl, q, k, v = big
    p = A.problem_for(wl)
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    assert np.array_equal(Eq.cpu().numpy(), Eq_ref)
    heads = (1, wl.H // 2)
    br_ref = {h: O.bridge_select(head(k, h)[0, 0], wl.bridge_k, wl.Gh, wl.Gw) for h in heads}
    sizes = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)
    check_attn = {0, 1, wl.p2_steps - 1}
    for t, w in enumerate(sizes):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq_ref)
        pl = plan.cpu().numpy()
        nwin = int(pl[0])
        assert nwin == len(ref.windows), (wl.name, t)
        np.testing.assert_array_equal(pl[16:16 + 10 * nwin].reshape(nwin, 10), ref.records())
        np.testing.assert_array_equal(wsum.cpu().numpy(), ref.wsum)
        b = br.cpu().numpy()
        for h in heads:
            np.testing.assert_array_equal(b[0, h], br_ref[h], err_msg=f"{wl.name} step {t} bridge head {h}")
        if t not in check_attn:
            continue
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        rows = rows_for(wl, ref, seed=10 + t)
        for h in heads:
            o_ref = O.window_attention(head(q, h), head(k, h), head(v, h), ref, br_ref[h][None, None],
                                       wl.Gh, wl.Gw, wl.rope_theta, rows=rows)
            close(head(out, h)[:, :, rows], o_ref,
                  f"{wl.name} window step {t} (w={w}, {nwin} windows, {int(pl[9])} split) head {h}")


# ----------------------------------------------------------- edge cases --

def small_problem(Gh, Gw, H=2, B=1, D=64, **kw):
    wl = W.Workload("edge", B=B, H=H, D=D, Gh=Gh, Gw=Gw, native_h=Gh // 2, native_w=Gw // 2,
                    dtype="bf16", p1_steps=2, f_min=2, p2_steps=3, w_start=kw.get("w_start", 16),
                    w_min=kw.get("w_min", 8), halo=kw.get("halo", 2), bridge_k=kw.get("bridge_k", 8),
                    latent_kind="half_columns")
    return wl, A.problem_for(wl)


@pytest.mark.parametrize("Gh,Gw", [(30, 34), (18, 50)])
def test_ragged_key_counts_dense(Gh, Gw):
    # N = 1020 and 900 are not multiples of the 64-key tile; f = 2 gives 255 / 225 pooled keys
    wl, p = small_problem(Gh, Gw)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=5))
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    out = A.area_full_attn(p, q, k, v)
    kp, vp = A.area_pool_kv(p, 2, k, v)
    co = A.area_coarse_attn(p, 2, q, kp, vp)
    torch.cuda.synchronize()
    close(out.float().cpu().numpy(), O.full_attention(qh, kh, vh, Gh, Gw, wl.rope_theta), f"full {Gh}x{Gw}")
    kpr, vpr = O.pool_kv(kh, vh, Gh, Gw, 2, O.POOL_MEAN, wl.rope_theta)
    close(co.float().cpu().numpy(), O.coarse_attention(qh, kpr, vpr, Gh, Gw, 2, wl.rope_theta), f"coarse {Gh}x{Gw}")


@pytest.mark.parametrize("Gh,Gw", [(4, 10), (8, 8), (8, 16), (10, 14), (12, 16), (10, 20), (16, 20), (20, 28)])
def test_short_key_sets_one_to_three_tiles(Gh, Gw):
    # key sets of 1, 2 and 3 64-key tiles, whole and ragged, through both orders of the item's last
    # steps (full attention: N = 40 .. 560 keys, 1 to 9 tiles; coarse f = 2: 10 .. 140 pooled keys)
    # (iid inputs: the smooth-noise generator's blur needs grids of 13 or more per side)
    wl, p = small_problem(Gh, Gw, D=128, w_start=4, w_min=2, halo=1, bridge_k=2)
    q, k, v = (torch.from_numpy(t).to(torch.bfloat16).cuda()
               for t in W.random_small_qkv(wl.B, wl.H, Gh * Gw, wl.D, seed=8))
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    out = A.area_full_attn(p, q, k, v)
    kp, vp = A.area_pool_kv(p, 2, k, v)
    co = A.area_coarse_attn(p, 2, q, kp, vp)
    torch.cuda.synchronize()
    close(out.float().cpu().numpy(), O.full_attention(qh, kh, vh, Gh, Gw, wl.rope_theta), f"full {Gh}x{Gw}")
    kpr, vpr = O.pool_kv(kh, vh, Gh, Gw, 2, O.POOL_MEAN, wl.rope_theta)
    close(co.float().cpu().numpy(), O.coarse_attention(qh, kpr, vpr, Gh, Gw, 2, wl.rope_theta), f"coarse {Gh}x{Gw}")


def test_batch_two_windowed():
    wl, p = small_problem(32, 48, H=3, B=2, D=128, w_start=20, w_min=12, halo=2, bridge_k=12)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=6))
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    sizes = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)
    for t, w in enumerate(sizes):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq_ref)
        br_ref = O.bridge_all(kh, wl.bridge_k, wl.Gh, wl.Gw)
        np.testing.assert_array_equal(br.cpu().numpy(), br_ref)
        o_ref = O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta)
        close(out.float().cpu().numpy(), o_ref, f"batch 2 window step {t} (w={w})")


def test_max_windows_per_axis():
    # w = 2 on a 128 x 128 grid: 64 base windows per axis, the most a step may
    # have; windows over the smooth half split into 1 x 1 quadrants, giving
    # 10240 records (2048 whole windows, 8192 quadrants) with one-token queries
    # and 4 x 4 Halo rectangles plus the bridge.
    wl, p = small_problem(128, 128, H=2, D=64, w_start=4, w_min=2, halo=1, bridge_k=16)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=7))
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    sizes = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)
    assert sizes[-1] == 2 and A.area_step_info(p, wl.p1_steps + 2)["ny"] == 64
    br_ref = O.bridge_all(kh, wl.bridge_k, wl.Gh, wl.Gw)
    for t, w in enumerate(sizes):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq_ref)
        pl = plan.cpu().numpy()
        nwin = int(pl[0])
        assert nwin == len(ref.windows), t
        np.testing.assert_array_equal(pl[16:16 + 10 * nwin].reshape(nwin, 10), ref.records())
        np.testing.assert_array_equal(wsum.cpu().numpy(), ref.wsum)
        np.testing.assert_array_equal(br.cpu().numpy(), br_ref)
        o_ref = O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta)
        close(out.float().cpu().numpy(), o_ref, f"64 windows per axis, step {t} (w={w}, {len(ref.windows)} records)")


def test_repeated_calls_are_deterministic():
    wl = W.get("tiny-32")
    p = A.problem_for(wl)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16"))
    lat = torch.from_numpy(W.make_latent(wl)).cuda()
    _, Eq = A.area_dwt_detail(p, lat)
    s = wl.p1_steps + 2
    outs = []
    for _ in range(3):
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        outs.append((plan.clone(), wsum.clone(), br.clone(), A.area_window_attn(p, s, plan, wsum, br, q, k, v)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a, b)


# ------------------------------------------------ ablation knob settings --
# The attention-time ablations of bench.py --ablation (quadrant splits off,
# Halo off, bridge off, fixed smallest window) run the same kernels on plans
# the oracle builds from the same knobs.

ABLATIONS = {"no_splits": dict(split_num=0), "no_halo": dict(halo=0), "no_bridge": dict(bridge_k=0),
             "fixed_w": dict(w_start=None)}


@pytest.fixture(scope="module")
def mid():
    wl = W.get("flux-4096")
    say(f"generating {wl.name} on the GPU (ablations)")
    q, k, v = W.make_qkv(wl, device="cuda", dtype="bf16")
    lat = W.make_latent(wl)
    yield wl, q, k, v, lat
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", sorted(ABLATIONS))
def test_ablation_knobs(mid, name):
    wl, q, k, v, lat = mid
    over = dict(ABLATIONS[name])
    if "w_start" in over:
        over["w_start"] = wl.w_min
    p = A.problem_for(wl, **over)
    halo = over.get("halo", wl.halo)
    R = over.get("bridge_k", wl.bridge_k)
    split_num = over.get("split_num", 1)
    w_start = over.get("w_start", wl.w_start)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    heads = (2, wl.H - 1)
    br_ref = {h: O.bridge_select(head(k, h)[0, 0], R, wl.Gh, wl.Gw) for h in heads} if R > 0 else None
    sizes = O.window_sizes(w_start, wl.w_min, wl.p2_steps)
    for t in (0, wl.p2_steps - 1):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, sizes[t], halo, wl.seed, t, Eq_ref, split_num=split_num)
        pl = plan.cpu().numpy()
        nwin = int(pl[0])
        assert nwin == len(ref.windows), (name, t)
        np.testing.assert_array_equal(pl[16:16 + 10 * nwin].reshape(nwin, 10), ref.records())
        np.testing.assert_array_equal(wsum.cpu().numpy(), ref.wsum)
        if R == 0:
            assert br is None
        else:
            b = br.cpu().numpy()
            for h in heads:
                np.testing.assert_array_equal(b[0, h], br_ref[h], err_msg=f"{name} bridge head {h}")
        rows = rows_for(wl, ref, n_random=32, seed=40 + t)
        for h in heads:
            o_ref = O.window_attention(head(q, h), head(k, h), head(v, h), ref,
                                       br_ref[h][None, None] if R > 0 else None,
                                       wl.Gh, wl.Gw, wl.rope_theta, rows=rows)
            close(head(out, h)[:, :, rows], o_ref, f"{wl.name} ablation {name} step {t} (w={sizes[t]}) head {h}")


# --------------------------------------------------- the pages' knob values --
# First window from the cost rule, seeded Halo widths up to 8 per window and a
# bridge of (w/2)^2 tokens at window side w.

def test_window_steps_pages_knobs(big):
    wl, q, k, v = big
    p = A.problem_for(wl, **W.PAGES_KNOBS)
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    w0 = O.w_start_auto(wl.Gh, wl.Gw, wl.w_min)
    sizes = O.window_sizes(w0, wl.w_min, wl.p2_steps)
    heads = (0, wl.H - 3)
    check_attn = {0, 1, wl.p2_steps - 1}
    say(f"{wl.name}: pages' knobs, w_start {w0}, bridge {O.bridge_size(sizes[0], 1, 2)} .. "
        f"{O.bridge_size(sizes[-1], 1, 2)}")
    for t, w in enumerate(sizes):
        s = wl.p1_steps + t
        R = O.bridge_size(w, 1, 2)
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, w, 0, wl.seed, t, Eq_ref, halo_max=8)
        pl = plan.cpu().numpy()
        nwin = int(pl[0])
        assert nwin == len(ref.windows), (wl.name, t)
        np.testing.assert_array_equal(pl[16:16 + 10 * nwin].reshape(nwin, 10), ref.records())
        np.testing.assert_array_equal(wsum.cpu().numpy(), ref.wsum)
        assert tuple(br.shape) == (wl.B, wl.H, R)
        if t not in check_attn:
            continue
        br_ref = {h: O.bridge_select(head(k, h)[0, 0], R, wl.Gh, wl.Gw) for h in heads}
        b = br.cpu().numpy()
        for h in heads:
            np.testing.assert_array_equal(b[0, h], br_ref[h], err_msg=f"{wl.name} step {t} bridge head {h}")
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        rows = rows_for(wl, ref, seed=70 + t)
        for h in heads:
            o_ref = O.window_attention(head(q, h), head(k, h), head(v, h), ref, br_ref[h][None, None],
                                       wl.Gh, wl.Gw, wl.rope_theta, rows=rows)
            close(head(out, h)[:, :, rows], o_ref,
                  f"{wl.name} pages' knobs step {t} (w={w}, R={R}, {nwin} windows) head {h}")
