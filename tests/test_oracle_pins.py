"""Pins for the CPU oracle: each test checks it against something other than
itself -- values the pages print, closed forms, library routines, brute force
on tiny inputs and invariants -- so that a dropped term, a wrong sign or index
or a transposed operand anywhere in it fails here."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import area_oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------- RoPE ----

def test_rope_identity_at_origin():
    x = rng(1).standard_normal((3, 5, 16))
    z = np.zeros(5)
    np.testing.assert_array_equal(O.apply_rope_2d(x, z, z, 10000.0), x)


def test_rope_preserves_norm():
    x = rng(2).standard_normal((7, 64))
    y = rng(3).integers(0, 400, 7).astype(float)
    xx = rng(4).integers(0, 400, 7).astype(float)
    r = O.apply_rope_2d(x, y, xx, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_relative_positions_2d():
    # <R(p) q, R(p') k> depends on p - p' only, separately along both axes.
    g = rng(5)
    q, k = g.standard_normal((2, 1, 32))
    base = O.apply_rope_2d(q, [3.0], [5.0], 100.0) @ O.apply_rope_2d(k, [1.0], [9.0], 100.0).T
    for dy, dx in [(7, 0), (0, 11), (13, -2), (0.5, 2.25)]:
        s = O.apply_rope_2d(q, [3 + dy], [5 + dx], 100.0) @ O.apply_rope_2d(k, [1 + dy], [9 + dx], 100.0).T
        np.testing.assert_allclose(s, base, rtol=1e-11, atol=1e-12)
    # and it does change when only one side moves
    s = O.apply_rope_2d(q, [4.0], [5.0], 100.0) @ O.apply_rope_2d(k, [1.0], [9.0], 100.0).T
    assert abs(s - base).max() > 1e-3


def test_rope_axis_layout_closed_form():
    # D = 8: channels 0..3 follow the row, 4..7 the column; pair k of an axis
    # half turns by pos * theta^(-2k/4).  Hand-worked with theta = 10000:
    # frequencies 1 and 10000^(-1/2) = 0.01.
    e = np.eye(8)
    r = O.apply_rope_2d(e, np.full(8, 1.0), np.zeros(8), 10000.0)
    # row position 1: pair (0,1) turns by 1 rad, pair (2,3) by 0.01 rad; column half untouched
    np.testing.assert_allclose(r[0, :2], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    np.testing.assert_allclose(r[1, :2], [-math.sin(1.0), math.cos(1.0)], rtol=1e-15)
    np.testing.assert_allclose(r[2, 2:4], [math.cos(0.01), math.sin(0.01)], rtol=1e-15)
    np.testing.assert_array_equal(r[4:, 4:], np.eye(4))
    r = O.apply_rope_2d(e, np.zeros(8), np.full(8, 2.0), 10000.0)
    np.testing.assert_array_equal(r[:4, :4], np.eye(4))
    np.testing.assert_allclose(r[4, 4:6], [math.cos(2.0), math.sin(2.0)], rtol=1e-15)
    np.testing.assert_allclose(r[6, 6:8], [math.cos(0.02), math.sin(0.02)], rtol=1e-15)


# ------------------------------------------------------------ attention ----

def test_attention_matches_library_sdpa():
    g = rng(6)
    q, k, v = (g.standard_normal((2, 3, n, 16)) for n in (9, 13, 13))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(O.attention(q, k, v), ref, rtol=1e-12, atol=1e-13)


def test_attention_two_keys_closed_form():
    # q = a e0, keys +e0 and -e0: weight of the first key is sigmoid(2a/sqrt(D))
    D, a = 16, 3.0
    q = np.zeros((1, D)); q[0, 0] = a
    k = np.zeros((2, D)); k[0, 0] = 1.0; k[1, 0] = -1.0
    v = np.array([[1.0] + [0] * (D - 1), [0.0] * D])
    p = 1.0 / (1.0 + math.exp(-2 * a / math.sqrt(D)))
    np.testing.assert_allclose(O.attention(q, k, v)[0, 0], p, rtol=1e-14)


def test_softmax_rows_sum_to_one():
    s = rng(7).standard_normal((50, 300)) * 20
    p = O.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-13)
    assert (p >= 0).all()


def test_constant_values_give_constant_output():
    g = rng(8)
    q, k = g.standard_normal((2, 2, 64, 32))
    v = np.tile(g.standard_normal(32), (2, 64, 1))
    out = O.full_attention(q, k, v, 8, 8, 10000.0)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=1e-12)


def test_full_attention_brute_force_loops():
    # explicit per-(query, key) loops, exp and normalisation
    g = rng(9)
    Gh, Gw, D = 3, 4, 8
    q, k, v = (g.standard_normal((1, 1, Gh * Gw, D)) for _ in range(3))
    y, x = O.grid_positions(Gh, Gw)
    qr = O.apply_rope_2d(q, y, x, 50.0)[0, 0]
    kr = O.apply_rope_2d(k, y, x, 50.0)[0, 0]
    out = O.full_attention(q, k, v, Gh, Gw, 50.0)[0, 0]
    for i in range(Gh * Gw):
        s = [sum(qr[i, d] * kr[j, d] for d in range(D)) / math.sqrt(D) for j in range(Gh * Gw)]
        m = max(s)
        e = [math.exp(t - m) for t in s]
        z = sum(e)
        o = [sum(e[j] * v[0, 0, j, d] for j in range(Gh * Gw)) / z for d in range(D)]
        np.testing.assert_allclose(out[i], o, rtol=1e-12, atol=1e-13)


def test_full_attention_row_subset():
    g = rng(10)
    q, k, v = (g.standard_normal((1, 2, 36, 8)) for _ in range(3))
    rows = np.array([0, 5, 35, 17])
    np.testing.assert_allclose(O.full_attention(q, k, v, 6, 6, 1e4, rows=rows),
                               O.full_attention(q, k, v, 6, 6, 1e4)[..., rows, :], rtol=1e-13)


# -------------------------------------------------------------- pooling ----

def test_pool_mean_is_avg_pool2d():
    g = rng(11)
    Gh, Gw, f, D = 12, 18, 3, 5
    t = g.standard_normal((2, 3, Gh * Gw, D))
    img = torch.from_numpy(t).reshape(6, Gh, Gw, D).permute(0, 3, 1, 2)
    ref = torch.nn.functional.avg_pool2d(img, f).permute(0, 2, 3, 1).reshape(2, 3, -1, D).numpy()
    np.testing.assert_allclose(O.pool_tokens(t, Gh, Gw, f, O.POOL_MEAN), ref, rtol=1e-13)


@pytest.mark.parametrize("f", [2, 3, 4, 6])
def test_pool_center_is_strided_slice(f):
    g = rng(12)
    Gh, Gw, D = 12, 24, 4
    t = g.standard_normal((1, 1, Gh * Gw, D))
    img = t.reshape(Gh, Gw, D)
    c = f // 2
    ref = img[c::f, c::f].reshape(1, 1, -1, D)
    np.testing.assert_array_equal(O.pool_tokens(t, Gh, Gw, f, O.POOL_CENTER), ref)


def test_pool_f1_is_identity():
    t = rng(13).standard_normal((1, 2, 20, 4))
    for mode in (O.POOL_MEAN, O.POOL_CENTER):
        np.testing.assert_array_equal(O.pool_tokens(t, 4, 5, 1, mode), t)


def test_pool_kv_center_takes_the_strided_slice_token():
    # pool_kv picks single tokens through in-block offsets; for center that must be the
    # strided-slice token of pool_tokens, rotated at the coarse position
    g = rng(15)
    Gh, Gw, f, D = 12, 18, 3, 8
    k, v = g.standard_normal((2, 1, 2, Gh * Gw, D))
    kp, vp = O.pool_kv(k, v, Gh, Gw, f, O.POOL_CENTER, 1e4)
    by, bx = O.grid_positions(Gh // f, Gw // f)
    np.testing.assert_array_equal(vp, O.pool_tokens(v, Gh, Gw, f, O.POOL_CENTER))
    np.testing.assert_array_equal(kp, O.apply_rope_2d(O.pool_tokens(k, Gh, Gw, f, O.POOL_CENTER), by, bx, 1e4))


def test_medoid_of_collinear_keys_is_the_median():
    # keys t_i * u on a line: the sum of |t_i - t_j| is smallest at the median of t
    g = rng(16)
    for f in (3, 5):
        t = g.permutation(f * f).astype(np.float64) * 0.37 - 2.0
        u = g.standard_normal(6)
        kb = t[:, None] * u[None, :]
        assert O.medoid_offset(kb) == int(np.argsort(t)[(f * f) // 2])


def test_medoid_matches_library_distances():
    # independent of the oracle's loops: scipy's pairwise Euclidean distances, summed per
    # candidate, argmin (random keys make ties impossible in practice)
    from scipy.spatial.distance import cdist
    g = rng(17)
    for f in (2, 3, 4, 6):
        kb = g.standard_normal((f * f, 16))
        assert O.medoid_offset(kb) == int(np.argmin(cdist(kb, kb).sum(axis=0)))


def test_medoid_invariances_and_majority():
    g = rng(18)
    kb = g.standard_normal((9, 5))
    j = O.medoid_offset(kb)
    assert O.medoid_offset(kb + g.standard_normal(5)) == j          # translation
    assert O.medoid_offset(3.0 * kb) == j                           # scale
    maj = np.repeat(kb[4:5], 9, axis=0)
    maj[[0, 8]] = kb[[0, 8]] * 5.0                                 # 7 of 9 keys identical
    assert O.medoid_offset(maj) == 1                                # smallest offset holding it
    assert O.medoid_offset(kb[:1]) == 0                             # one token


def test_random_pool_offsets():
    f, nb = 4, 6000
    offs = np.array([O.pool_random_offset(7, f, b) for b in range(nb)])
    assert offs.min() >= 0 and offs.max() < f * f
    counts = np.bincount(offs, minlength=f * f)
    # uniform over the f^2 offsets: every count within 5 sigma of nb / f^2
    mu = nb / (f * f)
    assert np.all(np.abs(counts - mu) < 5 * np.sqrt(mu))
    assert [O.pool_random_offset(7, f, b) for b in range(20)] == list(offs[:20])
    assert [O.pool_random_offset(8, f, b) for b in range(20)] != list(offs[:20])
    assert O.pool_random_offset(7, 1, 3) == 0
    # the draw is the POOL stream of SplitMix64 at counter 1 + f * 2^32 + block
    assert O.pool_random_offset(7, f, 5) == O.splitmix64(7 ^ 0x504F4F4C, 1 + f * (1 << 32) + 5) % (f * f)


def test_single_token_pooling_shares_the_token_between_k_and_v():
    # medoid chooses on K; V takes the same token: with V = K the pooled V is the
    # un-rotated pooled K, and with f = 1 every mode is the identity
    g = rng(19)
    Gh, Gw, D = 6, 6, 8
    k = g.standard_normal((1, 2, Gh * Gw, D))
    for mode in (O.POOL_MEDOID, O.POOL_RANDOM):
        off = O.pool_offsets(k, Gh, Gw, 3, mode, seed=3)
        kp, vp = O.pool_kv(k, k, Gh, Gw, 3, mode, 1e4, seed=3)
        by, bx = O.grid_positions(2, 2)
        np.testing.assert_allclose(kp, O.apply_rope_2d(vp, by, bx, 1e4), rtol=0, atol=0)
        k1, v1 = O.pool_kv(k, k, Gh, Gw, 1, mode, 1e4, seed=3)
        y, x = O.grid_positions(Gh, Gw)
        np.testing.assert_array_equal(v1, k)
    # medoid decides per head: the two heads' offsets come from their own keys
    off = O.pool_offsets(k, Gh, Gw, 3, O.POOL_MEDOID)
    for h in range(2):
        for b in range(4):
            by, bx = divmod(b, 2)
            assert off[0, h, b] == O.medoid_offset(k[0, h][O.block_tokens(Gw, 3, by, bx)])


def test_coarse_f1_equals_full_attention():
    g = rng(14)
    Gh, Gw, D = 6, 8, 16
    q, k, v = (g.standard_normal((1, 2, Gh * Gw, D)) for _ in range(3))
    for mode in (O.POOL_MEAN, O.POOL_CENTER):
        kp, vp = O.pool_kv(k, v, Gh, Gw, 1, mode, 1e4)
        np.testing.assert_allclose(O.coarse_attention(q, kp, vp, Gh, Gw, 1, 1e4),
                                   O.full_attention(q, k, v, Gh, Gw, 1e4), rtol=1e-12, atol=1e-13)


def test_pooled_key_count_and_cost():
    for c in gold("phase_costs.json")["cases"]:
        Gh, Gw, f = c["Gh"], c["Gw"], c["f"]
        t = np.zeros((1, 1, Gh * Gw, 4))
        assert O.pool_tokens(t, Gh, Gw, f, O.POOL_MEAN).shape[-2] == c["pooled_keys"]
        # query-key pairs are 1/f^2 of full attention
        assert Fraction(Gh * Gw * c["pooled_keys"], (Gh * Gw) ** 2) == Fraction(1, f * f)


def test_coarse_positions_put_block_on_key():
    # A query at the top-left token of block (by, bx) has RoPE position
    # (by, bx), exactly the pooled key's: their rotated dot product equals
    # the un-rotated one.
    g = rng(15)
    Gh, Gw, f, D = 8, 8, 2, 16
    q = g.standard_normal((1, 1, Gh * Gw, D))
    k = g.standard_normal((1, 1, Gh * Gw, D))
    kp, _ = O.pool_kv(k, k, Gh, Gw, f, O.POOL_MEAN, 1e4)
    kp_raw = O.pool_tokens(k, Gh, Gw, f, O.POOL_MEAN)
    y, x = O.grid_positions(Gh, Gw)
    for by, bx in [(0, 0), (1, 3), (3, 2)]:
        n = (by * f) * Gw + bx * f
        qr = O.apply_rope_2d(q[0, 0, [n]], y[[n]] / f, x[[n]] / f, 1e4)
        j = by * (Gw // f) + bx
        np.testing.assert_allclose(qr @ kp[0, 0, j], q[0, 0, n] @ kp_raw[0, 0, j], rtol=1e-11)


# ------------------------------------------------------------ schedules ----

def test_ramp_worked_example_from_pages():
    g = gold("ramp_worked_example.json")
    f0 = O.f0_for(g["Gh"], g["Gw"], g["native_h"], g["native_w"], g["f_min"])
    assert f0 == g["f0"]
    assert O.pooling_ramp(g["Gh"], g["Gw"], f0, g["f_min"], g["steps"]) == g["ramp"]


def test_ramp_readings_that_fail_the_example_are_rejected():
    # The worked example separates rounding rules: snapping by floor or by
    # ceil does not reproduce it, nearest does.
    xs = [4 + (2 - 4) * t / 7 for t in range(8)]
    assert [2 if x < 4 else 4 for x in xs] != [4, 4, 4, 4, 2, 2, 2, 2]       # floor
    assert [4 if x > 2 else 2 for x in xs] != [4, 4, 4, 4, 2, 2, 2, 2]       # ceil


@pytest.mark.parametrize("name,f0", [("tiny-32", 2), ("flux-2048", 2), ("flux-4096", 4),
                                     ("flux-6144", 6), ("qwen-6144x2048", 4)])
def test_first_pooling_factor_per_workload(name, f0):
    wl = W.get(name)
    assert O.f0_for(wl.Gh, wl.Gw, wl.native_h, wl.native_w, wl.f_min) == f0


def test_ramp_endpoints_and_monotone():
    for G in (96, 128, 256, 384, 512):
        for f0 in O.common_divisors(G, G, 2)[:6]:
            for P in (1, 2, 5, 8, 20):
                r = O.pooling_ramp(G, G, f0, 2, P)
                assert r[0] == f0 and len(r) == P
                if P > 1:
                    assert r[-1] == 2
                assert all(a >= b for a, b in zip(r, r[1:]))
                assert all(G % f == 0 for f in r)


def test_window_sizes_endpoints_monotone_even():
    for ws, wm, S in [(192, 64, 20), (128, 64, 16), (128, 64, 8), (16, 8, 4), (100, 64, 3)]:
        w = O.window_sizes(ws, wm, S)
        assert w[0] == ws and w[-1] == wm and len(w) == S
        assert all(a >= b for a, b in zip(w, w[1:]))
        assert all(x % 2 == 0 for x in w)


def test_w_start_rule_is_about_seventy_percent():
    g = gold("w_start_rule.json")
    for G in g["grid_sides"]:
        def cost(w):
            return sum(1 for _ in O.base_starts(G, w)) ** 2 * (w * w) ** 2
        wmax = max(w for w in range(1, G) if cost(w) < G ** 4)
        assert g["fraction_low"] <= wmax / G <= g["fraction_high"], (G, wmax)


def test_w_start_auto_closed_form_on_square_grids():
    # On a G x G grid the R8 tiling has ceil(G/w)^2 windows of w^2 tokens (w < G), so the
    # rule "cheaper than one full pass" is ceil(G/w)^2 * w^4 < G^4; the largest even such w
    # is the first window, about 70% of the side for the configured grids.
    for G in (64, 128, 256, 384, 512):
        want = max(w for w in range(2, G, 2) if math.ceil(G / w) ** 2 * w ** 4 < G ** 4)
        assert O.w_start_auto(G, G, 8) == want
        if G >= 128:   # the configured grids; even sizes are coarser on small grids
            assert 0.69 <= want / G <= 0.71
    assert [O.w_start_auto(G, G, 8) for G in (128, 256, 384)] == [90, 180, 270]


def test_w_start_auto_counts_pairs_of_the_actual_tiling():
    # a non-square grid: enumerate the step's windows (no Halo, no splits) and count
    # (query, key) pairs directly; the chosen w passes, the next even size does not.
    Gh, Gw = 384, 128
    w = O.w_start_auto(Gh, Gw, 64)

    def pairs(ws):
        plan = O.window_plan(Gh, Gw, ws, 0, 0, 0, None)
        return sum(win.qh * win.qw * win.kh * win.kw for win in plan.windows)

    assert pairs(w) < (Gh * Gw) ** 2 <= pairs(w + 2)
    assert w == 270   # the longer side's 70%
    # a minimum above every qualifying size is kept
    assert O.w_start_auto(64, 64, 64) == 64


def test_halo_widths_seeded_uniform_in_range():
    draws = [O.halo_width(3, t, b, q, 8) for t in range(20) for b in range(60) for q in range(-1, 4)]
    assert min(draws) == 1 and max(draws) == 8
    counts = np.bincount(draws, minlength=9)[1:]
    exp = len(draws) / 8
    assert np.all(np.abs(counts - exp) < 0.15 * exp), counts
    # deterministic, and a different seed gives a different sequence
    assert draws == [O.halo_width(3, t, b, q, 8) for t in range(20) for b in range(60) for q in range(-1, 4)]
    assert draws != [O.halo_width(4, t, b, q, 8) for t in range(20) for b in range(60) for q in range(-1, 4)]
    # its own stream: not the jitter draws of the same seed
    assert O.halo_width(0, 0, 0, -1, 1 << 30) - 1 != O.splitmix64(0, 1) % (1 << 30)


def test_random_halo_rects():
    wl = W.get("tiny-32")
    Eq = O.energy_fixed(O.detail_energy(W.make_latent(wl)))
    for step, w in enumerate([16, 12, 10, 8]):
        plan = O.window_plan(wl.Gh, wl.Gw, w, 0, 11, step, Eq, halo_max=8)
        widths = set()
        for win in plan.windows:
            d = O.halo_width(11, step, win.parent, win.quadrant, 8)
            widths.add(d)
            assert 1 <= d <= 8
            assert (win.ky0, win.kx0, win.kh, win.kw) == O.halo_rect(win.qy0, win.qx0, win.qh, win.qw, d,
                                                                     wl.Gh, wl.Gw)
        if len(plan.windows) > 4:
            assert len(widths) > 1
        # delta_max = 1 is the fixed Halo of width 1
        fixed = O.window_plan(wl.Gh, wl.Gw, w, 1, 11, step, Eq)
        one = O.window_plan(wl.Gh, wl.Gw, w, 0, 11, step, Eq, halo_max=1)
        np.testing.assert_array_equal(fixed.records(), one.records())


def test_bridge_size_per_step():
    for w in range(2, 400, 2):
        assert O.bridge_size(w, 1, 2) == (w // 2) ** 2          # rho = 0.5 on even sides
    assert O.bridge_size(192, 1, 2) == 9216 and O.bridge_size(64, 1, 2) == 1024
    assert O.bridge_size(5, 1, 2) == 9                           # round half up: 2.5 -> 3
    assert O.bridge_size(10, 1, 3) == 9                          # 3.33 -> 3


def test_base_tiling_properties():
    for G in range(8, 70):
        for w in range(2, G + 3):
            b = O.base_starts(G, w)
            L = min(w, G)
            assert b[0] == 0 and b[-1] + L == G
            assert len(b) == max(1, -(-G // w))
            assert all(0 <= b[i + 1] - b[i] <= L for i in range(len(b) - 1))
            if G % w == 0:
                assert b == list(range(0, G, w))


def test_splitmix64_published_vectors():
    g = gold("splitmix64_vectors.json")
    assert [O.splitmix64(g["seed"], k) for k in range(1, 6)] == [int(s) for s in g["outputs"]]


def test_jitter_keeps_coverage_for_every_offset():
    # brute force over all offsets in [-J, J]: every token stays covered and
    # every window stays inside the grid
    for G in range(10, 60, 3):
        for w in range(4, G, 3):
            b = O.base_starts(G, w)
            if len(b) <= 2:
                continue
            gap = max(b[i + 1] - b[i] for i in range(len(b) - 1))
            J = max(0, (w - gap) // 2)
            for o in range(-J, J + 1):
                s = [x + (o if 0 < i < len(b) - 1 else 0) for i, x in enumerate(b)]
                cov = np.zeros(G, int)
                for x in s:
                    assert 0 <= x and x + w <= G
                    cov[x:x + w] += 1
                assert (cov >= 1).all(), (G, w, o)


def test_jitter_range_and_variation():
    b = O.base_starts(384, 182)
    offs = {O.jitter_offset(b, 182, 0, step, 0) for step in range(40)}
    J = (182 - max(b[1] - b[0], b[2] - b[1])) // 2
    assert all(-J <= o <= J for o in offs) and len(offs) > 10


# ----------------------------------------------------------------- Haar ----

def test_haar_perfect_reconstruction():
    x = rng(16).standard_normal((3, 10, 14))
    np.testing.assert_allclose(O.haar_inverse(*O.haar_forward(x)), x, rtol=0, atol=1e-14)


def test_haar_parseval_and_energy_is_detail_bands():
    x = rng(17).standard_normal((4, 8, 12))
    ll, lh, hl, hh = O.haar_forward(x)
    np.testing.assert_allclose((x ** 2).sum(), (ll ** 2 + lh ** 2 + hl ** 2 + hh ** 2).sum(), rtol=1e-13)
    np.testing.assert_allclose(O.detail_energy(x), (lh ** 2 + hl ** 2 + hh ** 2).sum(0), rtol=1e-13)


def test_haar_linear_ramp_closed_form():
    # x = a*y + b*x + c: LH = -b, HL = -a, HH = 0 in every cell, so E = a^2 + b^2
    Gh, Gw = 8, 6
    a, b, c = 0.75, -1.25, 0.5
    yy, xx = np.meshgrid(np.arange(Gh), np.arange(Gw), indexing="ij")
    lat = (a * yy + b * xx + c)[None]
    ll, lh, hl, hh = O.haar_forward(lat)
    np.testing.assert_allclose(lh, -b, atol=1e-14)
    np.testing.assert_allclose(hl, -a, atol=1e-14)
    np.testing.assert_allclose(hh, 0.0, atol=1e-14)
    np.testing.assert_allclose(O.detail_energy(lat), a * a + b * b, rtol=1e-14)


def test_haar_white_noise_mean_energy():
    C = 16
    x = rng(18).standard_normal((C, 256, 256))
    E = O.detail_energy(x)
    # three orthonormal detail bands of unit-variance noise: E[E] = 3C
    assert abs(E.mean() - 3 * C) < 0.1


def test_energy_fixed_point():
    E = np.array([[0.0, 1.0, 2.5 / 65536, 3.5 / 65536], [1e9, 1e-7, 0.5, 32767.99999]])
    q = O.energy_fixed(E)
    assert q.dtype == np.int32
    assert q.tolist() == [[0, 65536, 2, 4], [2147483647, 0, 32768, 2147483647]]


# --------------------------------------------------------- window plan ----

def _tiny_plan(step, w, seed=0):
    wl = W.get("tiny-32")
    Eq = O.energy_fixed(O.detail_energy(W.make_latent(wl)))
    return wl, O.window_plan(wl.Gh, wl.Gw, w, wl.halo, seed, step, Eq), Eq


def test_plan_splits_smooth_windows_only():
    wl = W.get("flux-4096")
    m = W.textured_mask(wl)
    Eq = O.energy_fixed(O.detail_energy(W.make_latent(wl)))
    for step, w in enumerate(O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)):
        plan = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, step, Eq)
        parents = {}
        for win in plan.windows:
            parents.setdefault(win.parent, []).append(win)
        for p, ws in parents.items():
            if len(ws) == 4:
                y0 = ws[0].qy0; x0 = ws[0].qx0
                h = ws[0].qh + ws[2].qh; wd = ws[0].qw + ws[1].qw
            else:
                y0, x0, h, wd = ws[0].qy0, ws[0].qx0, ws[0].qh, ws[0].qw
            frac = m[y0:y0 + h, x0:x0 + wd].mean()
            if frac == 0:
                assert len(ws) == 4
            if frac > 0.6:
                assert len(ws) == 1


def test_plan_quadrants_tile_parent():
    for step, w in enumerate([16, 12, 10, 8]):
        wl, plan, Eq = _tiny_plan(step, w)
        byp = {}
        for win in plan.windows:
            byp.setdefault(win.parent, []).append(win)
        for ws in byp.values():
            if len(ws) == 4:
                assert [x.quadrant for x in ws] == [0, 1, 2, 3]
                cov = np.zeros((wl.Gh, wl.Gw), int)
                for x in ws:
                    cov[x.qy0:x.qy0 + x.qh, x.qx0:x.qx0 + x.qw] += 1
                assert cov.max() == 1
                assert cov.sum() == (ws[0].qh + ws[2].qh) * (ws[0].qw + ws[1].qw)


def test_plan_halo_and_wsum_brute_force():
    for step, w in enumerate([16, 12, 10, 8]):
        wl, plan, Eq = _tiny_plan(step, w, seed=7)
        ws = np.zeros((wl.Gh, wl.Gw), int)
        for win in plan.windows:
            for yy in range(win.qy0, win.qy0 + win.qh):
                for xx in range(win.qx0, win.qx0 + win.qw):
                    uy, ux = yy - win.qy0, xx - win.qx0
                    ws[yy, xx] += min(uy + 1, win.qh - uy) * min(ux + 1, win.qw - ux)
            assert win.ky0 == max(0, win.qy0 - wl.halo)
            assert win.ky0 + win.kh == min(wl.Gh, win.qy0 + win.qh + wl.halo)
            assert win.kx0 == max(0, win.qx0 - wl.halo)
            assert win.kx0 + win.kw == min(wl.Gw, win.qx0 + win.qw + wl.halo)
        np.testing.assert_array_equal(plan.wsum.reshape(wl.Gh, wl.Gw), ws)
        assert (ws > 0).all()


# --------------------------------------------------------------- bridge ----

def test_bridge_mean_is_exact():
    k = W.bf16_round(rng(19).standard_normal((1000, 8)).astype(np.float32)).astype(np.float64)
    kq = np.rint(k * 2 ** 24).astype(np.int64)
    s = O.bridge_scores(k)
    # recompute the score of token 0 with an exactly rounded mean (Fractions)
    N = k.shape[0]
    mu = [float(Fraction(int(kq[:, d].sum()), 2 ** 24 * N)) for d in range(8)]
    acc = 0.0
    for d in range(8):
        t = k[0, d] - mu[d]
        acc = acc + t * t
    assert s[0] == acc


def test_bridge_mean_saturates_and_stays_exact_beyond_int64():
    """Keys enter the mean saturated at +-2^28: 40000 equal keys of 2^40 (a
    fixed-point total of 40000 * 2^52 > 2^63) have the exact mean 2^28, so
    every score is (2^40 - 2^28)^2 summed over channels; for mixed magnitudes
    the mean is the exact integer total of the saturated fixed-point keys,
    rounded once to float64 (Python's correctly rounded int -> float),
    divided by 2^24 N."""
    N, D = 40000, 4
    k = np.full((N, D), 2.0 ** 40)
    s = O.bridge_scores(k)
    assert (s == D * (2.0 ** 40 - 2.0 ** 28) ** 2).all()
    g = rng(24)
    k = W.bf16_round((g.standard_normal((3000, D)) * 10.0 ** g.integers(-7, 12, (3000, D))).astype(np.float32))
    k = k.astype(np.float64)
    kq = np.rint(np.clip(k, -2.0 ** 28, 2.0 ** 28) * 2 ** 24).astype(np.int64)
    s = O.bridge_scores(k)
    for j in (0, 17, 2999):
        acc = 0.0
        for d in range(D):
            mu = float(sum(int(x) for x in kq[:, d])) / (2.0 ** 24 * 3000)
            t = k[j, d] - mu
            acc = acc + t * t
        assert s[j] == acc


def test_bridge_selection_brute_force():
    g = rng(20)
    for (Gh, Gw, R) in [(16, 16, 16), (12, 20, 6), (32, 32, 16), (24, 8, 8)]:
        k = g.standard_normal((Gh * Gw, 8))
        k[5] = k[6]  # a tie inside a cell
        idx = O.bridge_select(k, R, Gh, Gw)
        s = O.bridge_scores(k)
        rh, rw = O.bridge_cells(R, Gh, Gw)
        assert rh * rw == R
        expect = []
        for a in range(rh):
            for c in range(rw):
                cell = [y * Gw + x for y in range(a * Gh // rh, (a + 1) * Gh // rh)
                        for x in range(c * Gw // rw, (c + 1) * Gw // rw)]
                order = sorted(cell, key=lambda j: (-s[j], j))
                expect.append(order[0])
        assert idx.tolist() == sorted(expect)
        assert len(set(idx.tolist())) == R


def test_bridge_cells_golden():
    """Hand-worked cell grids (tests/golden/bridge_cells.json), including the
    non-square Qwen grid where the most nearly square cells are 12 x 16
    tokens, and a bridge size with no fitting grid."""
    g = gold("bridge_cells.json")
    for c in g["cases"]:
        if c["rh"] is None:
            with pytest.raises(ValueError):
                O.bridge_cells(c["R"], c["Gh"], c["Gw"])
            continue
        assert O.bridge_cells(c["R"], c["Gh"], c["Gw"]) == (c["rh"], c["rw"]), c["note"]


def test_bridge_cells_most_square_brute_force():
    """The cell grid minimises the cells' elongation over every factor pair
    of R that fits the grid, measured here as |log(cell height / cell
    width)| with exact fractions (an independent formulation), equal
    elongations going to the fewest cell rows."""
    g = rng(23)
    for _ in range(400):
        Gh, Gw = int(g.integers(2, 200)), int(g.integers(2, 200))
        R = int(g.integers(1, 600))
        pairs = [(a, R // a) for a in range(1, R + 1) if R % a == 0 and a <= Gh and R // a <= Gw]
        if not pairs:
            with pytest.raises(ValueError):
                O.bridge_cells(R, Gh, Gw)
            continue

        def elong(pr):
            ratio = Fraction(Gh, pr[0]) / Fraction(Gw, pr[1])
            return max(ratio, 1 / ratio)

        best = min(elong(pr) for pr in pairs)
        expect = min(pr for pr in pairs if elong(pr) == best)
        assert O.bridge_cells(R, Gh, Gw) == expect, (Gh, Gw, R)


def test_bridge_cells_partition_the_grid():
    """Every image token lies in exactly one cell, and cell sides differ by at
    most one token along each axis."""
    for (Gh, Gw, R) in [(384, 128, 256), (384, 384, 512), (12, 20, 6), (30, 34, 15)]:
        rh, rw = O.bridge_cells(R, Gh, Gw)
        owner = -np.ones((Gh, Gw), dtype=np.int64)
        hs, ws = set(), set()
        for a in range(rh):
            y0, y1 = a * Gh // rh, (a + 1) * Gh // rh
            hs.add(y1 - y0)
            for c in range(rw):
                x0, x1 = c * Gw // rw, (c + 1) * Gw // rw
                ws.add(x1 - x0)
                assert (owner[y0:y1, x0:x1] < 0).all()
                owner[y0:y1, x0:x1] = a * rw + c
        assert (owner >= 0).all()
        assert max(hs) - min(hs) <= 1 and max(ws) - min(ws) <= 1


def test_bridge_prefers_outliers():
    k = rng(21).standard_normal((16 * 16, 8)) * 0.1
    k[37] += 5.0
    idx = O.bridge_select(k, 4, 16, 16)
    assert 37 in idx.tolist()


# -------------------------------------------------- windowed attention ----

def test_whole_grid_window_equals_full_attention_any_bridge():
    g = rng(22)
    Gh, Gw, D = 8, 8, 16
    q, k, v = (g.standard_normal((1, 2, Gh * Gw, D)) for _ in range(3))
    plan = O.window_plan(Gh, Gw, Gh, 2, 0, 0, None)
    assert len(plan.windows) == 1
    full = O.full_attention(q, k, v, Gh, Gw, 1e4)
    for R in (0, 4, 16):
        br = O.bridge_all(k, R, Gh, Gw) if R else None
        np.testing.assert_allclose(O.window_attention(q, k, v, plan, br, Gh, Gw, 1e4), full,
                                   rtol=1e-12, atol=1e-13)


def test_window_attention_brute_force_key_sets():
    # Per token: the windows covering it, each with its explicit key set
    # (Halo rectangle, plus bridge tokens outside it), blended by tent weights.
    wl = W.get("tiny-32")
    g = rng(23)
    Gh, Gw, D = wl.Gh, wl.Gw, 16
    q, k, v = (g.standard_normal((1, 1, Gh * Gw, D)) for _ in range(3))
    Eq = O.energy_fixed(O.detail_energy(W.make_latent(wl)))
    plan = O.window_plan(Gh, Gw, 12, 1, 3, 1, Eq)
    br = O.bridge_all(k, 16, Gh, Gw)
    rows = np.array([0, 1, 33, 100, 200, 511, 512, 700, 1023, 15 * 32 + 15])
    out = O.window_attention(q, k, v, plan, br, Gh, Gw, 1e4, rows=rows)[0, 0]
    y, x = O.grid_positions(Gh, Gw)
    kr = O.apply_rope_2d(k[0, 0], y, x, 1e4)
    for r, p in enumerate(rows):
        py, px = divmod(int(p), Gw)
        qr = O.apply_rope_2d(q[0, 0, [p]], [py], [px], 1e4)[0]
        num = np.zeros(D)
        den = 0
        for win in plan.windows:
            if not (win.qy0 <= py < win.qy0 + win.qh and win.qx0 <= px < win.qx0 + win.qw):
                continue
            keys = set()
            for yy in range(win.ky0, win.ky0 + win.kh):
                for xx in range(win.kx0, win.kx0 + win.kw):
                    keys.add(yy * Gw + xx)
            keys |= set(int(t) for t in br[0, 0])
            keys = sorted(keys)
            s = np.array([qr @ kr[j] for j in keys]) / math.sqrt(D)
            e = np.exp(s - s.max())
            o = (e[:, None] * v[0, 0, keys]).sum(0) / e.sum()
            uy, ux = py - win.qy0, px - win.qx0
            wt = min(uy + 1, win.qh - uy) * min(ux + 1, win.qw - ux)
            num += wt * o
            den += wt
        np.testing.assert_allclose(out[r], num / den, rtol=1e-11, atol=1e-12)


def test_window_constant_values():
    g = rng(24)
    Gh = Gw = 16
    q, k = g.standard_normal((2, 1, 2, Gh * Gw, 8))
    v = np.tile(g.standard_normal(8), (1, 2, Gh * Gw, 1))
    plan = O.window_plan(Gh, Gw, 6, 1, 0, 2, None)
    out = O.window_attention(q, k, v, plan, O.bridge_all(k, 4, Gh, Gw), Gh, Gw, 1e4)
    np.testing.assert_allclose(out, v, rtol=1e-12)


def test_single_cover_token_gets_its_window_output():
    g = rng(25)
    Gh = Gw = 16
    q, k, v = (g.standard_normal((1, 1, Gh * Gw, 8)) for _ in range(3))
    plan = O.window_plan(Gh, Gw, 8, 1, 0, 0, None)   # 2x2 non-overlapping windows
    assert len(plan.windows) == 4
    # no overlaps: every token's weight sum is its own window's tent weight
    np.testing.assert_array_equal(plan.wsum.reshape(2, 8, 2, 8).transpose(0, 2, 1, 3),
                                  np.broadcast_to(np.outer(O.tent(8), O.tent(8)), (2, 2, 8, 8)))
    out = O.window_attention(q, k, v, plan, None, Gh, Gw, 1e4)[0, 0]
    win = plan.windows[3]
    qi = O.window_query_indices(win, Gw)
    ki = O.window_key_indices(win, Gw, None)
    y, x = O.grid_positions(Gh, Gw)
    ref = O.attention(O.apply_rope_2d(q[0, 0, qi], y[qi], x[qi], 1e4),
                      O.apply_rope_2d(k[0, 0, ki], y[ki], x[ki], 1e4), v[0, 0, ki])
    np.testing.assert_allclose(out[qi], ref, rtol=1e-12)


# ---------------------------------------------------------------- canvas ----

def test_canvas_rules_from_pages():
    for c in gold("canvas_rules.json")["cases"]:
        r = O.canvas_check(c["Gh"], c["Gw"], c["native"], c["native"])
        expect = {"full": O.PHASE_FULL, "area": O.PHASE_COARSE, "reject": -1}[c["expect"]]
        assert r == expect, c


def test_step_phases_counts():
    assert O.step_phases(8, 20) == [1] * 8 + [2] * 20


# ------------------------------------------------------------ text tokens ----
# READING R20: T text tokens first, at RoPE position (0, 0), left out of pooling and windowing,
# keys of every key set; text queries attend densely to all T + N keys.

def _text_inputs(T, Gh, Gw, D=16, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [rng.standard_normal((1, 2, T + Gh * Gw, D)) for _ in range(3)]


def test_text_phase1_key_count_from_pages():
    # [summary] Phase I: text keys skip the pooling, so every image query sees T + N/f^2 keys
    T, Gh, Gw, f = 5, 8, 12, 2
    q, k, v = _text_inputs(T, Gh, Gw)
    kp, vp = O.pool_kv(k, v, Gh, Gw, f, O.POOL_MEAN, 10000.0, T=T)
    assert kp.shape[-2] == vp.shape[-2] == T + Gh * Gw // f ** 2
    np.testing.assert_array_equal(kp[..., :T, :], k[..., :T, :])     # text keys unrotated, unpooled
    np.testing.assert_array_equal(vp[..., :T, :], v[..., :T, :])


def test_text_zero_queries_average_their_key_sets():
    # q = 0 makes every score equal, so each output is the plain mean of its key set's values
    T, Gh, Gw, f = 4, 8, 8, 2
    _, k, v = _text_inputs(T, Gh, Gw, seed=1)
    q = np.zeros_like(k)
    full = O.full_attention(q, k, v, Gh, Gw, 10000.0, T=T)
    np.testing.assert_allclose(full, np.broadcast_to(v.mean(axis=-2, keepdims=True), full.shape), atol=1e-12)
    np.testing.assert_allclose(O.text_attention(q, k, v, Gh, Gw, 10000.0, T), full[..., :T, :], atol=1e-12)
    kp, vp = O.pool_kv(k, v, Gh, Gw, f, O.POOL_MEAN, 10000.0, T=T)
    co = O.coarse_attention(q, kp, vp, Gh, Gw, f, 10000.0, T=T)
    np.testing.assert_allclose(co, np.broadcast_to(vp.mean(axis=-2, keepdims=True), co.shape), atol=1e-12)
    plan = O.window_plan(Gh, Gw, 4, 1, 0, 0, None)
    wo = O.window_attention(q, k, v, plan, None, Gh, Gw, 10000.0, T=T)
    acc = np.zeros_like(wo)
    for win in plan.windows:
        ki = O.window_key_indices(win, Gw, None)
        m = np.concatenate([v[..., :T, :], v[..., T + ki, :]], axis=-2).mean(axis=-2)
        wt = np.outer(O.tent(win.qh), O.tent(win.qw)).reshape(-1)
        for j, n in enumerate(O.window_query_indices(win, Gw)):
            acc[..., n, :] += wt[j] * m
    np.testing.assert_allclose(wo, acc / plan.wsum[None, None, :, None], atol=1e-12)


def test_text_brute_force_tiny():
    # direct double loops over explicit key lists, rotating each token at its own position
    T, Gh, Gw, f, D, th = 3, 4, 6, 2, 8, 100.0
    q, k, v = _text_inputs(T, Gh, Gw, D=D, seed=2)
    ys, xs = O.token_positions(Gh, Gw, T)

    def rot(t, y, x):
        return O.apply_rope_2d(t[None, None, None, :], np.array([y]), np.array([x]), th)[0, 0, 0]

    def softmax_out(qv, keys, vals):
        s = np.array([qv @ kk for kk in keys]) / math.sqrt(D)
        e = np.exp(s - s.max())
        return (e[:, None] * np.array(vals)).sum(0) / e.sum()

    b, h = 0, 1
    kr = [rot(k[b, h, i], ys[i], xs[i]) for i in range(T + Gh * Gw)]
    # full attention and text queries
    full = O.full_attention(q, k, v, Gh, Gw, th, T=T)
    for i in (0, T - 1, T, T + 7, T + Gh * Gw - 1):
        want = softmax_out(rot(q[b, h, i], ys[i], xs[i]), kr, list(v[b, h]))
        np.testing.assert_allclose(full[b, h, i], want, rtol=1e-10, atol=1e-12)
    # coarse: image query n at (y/f, x/f) against text keys + block-mean keys at block positions
    kp, vp = O.pool_kv(k, v, Gh, Gw, f, O.POOL_MEAN, th, T=T)
    co = O.coarse_attention(q, kp, vp, Gh, Gw, f, th, T=T)
    keys = [k[b, h, i] for i in range(T)]
    vals = [v[b, h, i] for i in range(T)]
    for by in range(Gh // f):
        for bx in range(Gw // f):
            blk = [T + (by * f + a) * Gw + bx * f + c for a in range(f) for c in range(f)]
            keys.append(rot(np.mean([k[b, h, i] for i in blk], axis=0), by, bx))
            vals.append(np.mean([v[b, h, i] for i in blk], axis=0))
    for n in (0, 5, Gh * Gw - 1):
        y, x = divmod(n, Gw)
        want = softmax_out(rot(q[b, h, T + n], y / f, x / f), keys, vals)
        np.testing.assert_allclose(co[b, h, n], want, rtol=1e-10, atol=1e-12)
    # window: text keys + the window's Halo rectangle
    plan = O.window_plan(Gh, Gw, 4, 1, 0, 0, None)
    wo = O.window_attention(q, k, v, plan, None, Gh, Gw, th, T=T)
    for n in (0, 9, Gh * Gw - 1):
        y, x = divmod(n, Gw)
        acc, wsum = 0.0, 0
        for win in plan.windows:
            if not (win.qy0 <= y < win.qy0 + win.qh and win.qx0 <= x < win.qx0 + win.qw):
                continue
            ki = list(range(T)) + [T + i for i in O.window_key_indices(win, Gw, None)]
            o = softmax_out(rot(q[b, h, T + n], y, x), [kr[i] for i in ki], [v[b, h, i] for i in ki])
            w = min(y - win.qy0 + 1, win.qh - (y - win.qy0)) * min(x - win.qx0 + 1, win.qw - (x - win.qx0))
            acc, wsum = acc + w * o, wsum + w
        np.testing.assert_allclose(wo[b, h, n], acc / wsum, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------ sigma switch --

def test_phase1_steps_for_sigma():
    # linear schedule sigma_t = 1 - t / n: the steps above sigma* are t < n (1 - sigma*)
    n = 28
    sig = [1.0 - t / n for t in range(n)]
    for s_star in (0.86, 0.9, 0.93, 0.96):
        assert O.phase1_steps_for_sigma(sig, s_star) == math.ceil(n * (1.0 - s_star) - 1e-12)
    assert O.phase1_steps_for_sigma(sig, 1.5) == 0            # sigma* above every level
    assert O.phase1_steps_for_sigma(sig, -1.0) == n           # below every level
    assert O.phase1_steps_for_sigma(sig, sig[3]) == 3         # a level equal to sigma* is Phase II
    assert O.phase1_steps_for_sigma([0.99, 0.8, 0.97], 0.9) == 1   # no switching back
    assert O.phase1_steps_for_sigma([], 0.9) == 0
