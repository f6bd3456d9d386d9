"""CPU tests of the C ABI: the library loads and exports every declared
symbol, its host-side schedule and tiling match the oracle bit for bit, and
invalid requests are rejected before anything is launched."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import resolution_diffusion_transformer_amd as A
import workloads as W
from oracle import area_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(A.library_path()):
        from resolution_diffusion_transformer_amd import _build
        _build.build(verbose=False)
    A.lib()


def declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            txt = open(os.path.join(inc, fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(area_[a-z0-9_]+)\s*\(", txt))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_symbols()
    for must in ["area_pool_kv", "area_coarse_attn", "area_dwt_detail", "area_window_plan",
                 "area_window_attn", "area_full_attn", "area_validate", "area_step_info",
                 "area_workspace_bytes"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(A.library_path())
    missing = [n for n in declared_symbols() if not hasattr(L, n)]
    assert not missing, missing
    assert set(declared_symbols()) == set(A.exported_symbols())


def prob(name, **over):
    return A.problem_for(W.get(name), **over)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_schedule_matches_oracle(name):
    wl = W.get(name)
    p = prob(name)
    assert A.area_validate(p) == 0
    f0 = O.f0_for(wl.Gh, wl.Gw, wl.native_h, wl.native_w, wl.f_min)
    assert A.area_f0(p) == f0
    ramp = O.pooling_ramp(wl.Gh, wl.Gw, f0, wl.f_min, wl.p1_steps)
    ws = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)
    for s in range(wl.p1_steps):
        info = A.area_step_info(p, s)
        assert info["phase"] == A.PHASE_COARSE and info["f"] == ramp[s]
    for t in range(wl.p2_steps):
        s = wl.p1_steps + t
        info = A.area_step_info(p, s)
        ys, oy = O.axis_windows(wl.Gh, ws[t], wl.seed, t, 0)
        xs, ox = O.axis_windows(wl.Gw, ws[t], wl.seed, t, 1)
        assert info["phase"] == A.PHASE_WINDOW
        assert (info["w"], info["ny"], info["nx"], info["jit_y"], info["jit_x"]) == \
            (ws[t], len(ys), len(xs), oy, ox)
        bw = A.area_base_windows(p, s)
        expect = [(y0, x0, h, w) for (y0, h) in ys for (x0, w) in xs]
        assert [tuple(r) for r in bw.tolist()] == expect


def test_schedule_matches_oracle_random_problems():
    rnd = random.Random(1234)
    for _ in range(300):
        Gh = 2 * rnd.randint(8, 200)
        Gw = 2 * rnd.randint(8, 200)
        nat = rnd.randint(4, min(Gh, Gw))
        wmin = 2 * rnd.randint(1, 40)
        wst = wmin + 2 * rnd.randint(0, 100)
        P1, S = rnd.randint(0, 12), rnd.randint(0, 24)
        seed = rnd.getrandbits(64)
        p = A.Problem(B=1, H=1, D=64, Gh=Gh, Gw=Gw, native_h=nat, native_w=nat, p1_steps=P1,
                      p2_steps=S, w_start=wst, w_min=wmin, halo=2, seed=seed)
        try:
            A.area_validate(p)
        except A.AreaError:
            continue
        if Gh <= nat and Gw <= nat:
            for s in range(P1 + S):
                assert A.area_step_info(p, s)["phase"] == A.PHASE_FULL
            continue
        f0 = O.f0_for(Gh, Gw, nat, nat, 2)
        assert A.area_f0(p) == f0
        ramp = O.pooling_ramp(Gh, Gw, f0, 2, P1)
        wsz = O.window_sizes(wst, wmin, S)
        for s in range(P1):
            assert A.area_step_info(p, s)["f"] == ramp[s]
        for t in range(S):
            info = A.area_step_info(p, P1 + t)
            ys, oy = O.axis_windows(Gh, wsz[t], seed, t, 0)
            xs, ox = O.axis_windows(Gw, wsz[t], seed, t, 1)
            assert (info["w"], info["jit_y"], info["jit_x"]) == (wsz[t], oy, ox)
            bw = A.area_base_windows(p, P1 + t)
            assert [tuple(r) for r in bw.tolist()] == [(y0, x0, h, w) for (y0, h) in ys for (x0, w) in xs]


def test_gated_canvas_keeps_full_attention():
    p = A.Problem(B=1, H=2, D=128, Gh=64, Gw=64, native_h=64, native_w=64, p1_steps=8, p2_steps=4,
                  w_start=64, w_min=32)
    assert A.area_validate(p) == 0
    for s in range(12):
        assert A.area_step_info(p, s)["phase"] == A.PHASE_FULL
    assert A.area_workspace_bytes(p, A.OP_WINDOW) == 0
    # fp16 key rows and V^T tiles (N is a multiple of 64), the two layouts of
    # the (cos, sin) table of 64 positions x D/4 frequencies, one exponent per
    # (head, 64-key tile) for K and for V, and the range words (a flag per
    # head, 8 work counters, the scaled-item count and list of up to N/256
    # items per head),
    # each region rounded up to 256 bytes
    up = lambda x: (x + 255) // 256 * 256
    BH, tiles = p.B * p.H, p.N // 64
    expect = (2 * BH * p.N * p.D * 2 + 2 * 64 * (p.D // 4) * 8 + 2 * up(BH * tiles * 4)
              + up((BH + 9 + BH * (p.N // 256)) * 4))
    assert A.area_workspace_bytes(p, A.OP_FULL) == expect


@pytest.mark.parametrize("over,status", [
    (dict(D=96), -3), (dict(T=4), 0), (dict(T=-1), -1), (dict(Gh=127), -2), (dict(Gh=130, Gw=126), 0),
    (dict(Gh=2 * 67, Gw=2 * 71), 0),               # both even: they share the factor 2
    (dict(w_start=60, w_min=64), -2), (dict(w_min=63), -2), (dict(bridge_k=3 * 1024 * 1024), -2),
    (dict(pool_mode=7), -1), (dict(split_den=0), -1), (dict(halo=-1), -1), (dict(B=0), -1),
    (dict(f0=5), -2), (dict(rope_theta=-1.0), -1),
    (dict(Gh=65538, Gw=2), -3),                     # a grid side above 65536 (RoPE table rows)
    (dict(Gh=65536, Gw=16, p2_steps=0), 0),         # the largest side, Phase I only
])
def test_validation_statuses(over, status):
    p = prob("flux-2048", **over)
    if status == 0:
        assert A.area_validate(p) == 0
    else:
        with pytest.raises(A.AreaError) as e:
            A.area_validate(p)
        assert e.value.status == status


def test_odd_factor_grid_rejected():
    # grid sides sharing no factor >= 2 (README canvas rules); even sides always share 2,
    # so use f_min = 3 to ask for a factor the sides do not share
    p = A.Problem(B=1, H=1, D=64, Gh=2 * 67, Gw=2 * 71, native_h=64, native_w=64, f_min=3)
    with pytest.raises(A.AreaError) as e:
        A.area_validate(p)
    assert e.value.status == -2


def test_device_calls_reject_bad_arguments_before_launch():
    L = A.lib()
    p = prob("flux-2048").c()
    fake = ctypes.c_void_p(0x1000)
    # NULL tensors
    assert L.area_full_attn(ctypes.byref(p), None, fake, fake, fake, fake, 1 << 40, None) == -1
    assert L.area_pool_kv(ctypes.byref(p), 2, fake, None, fake, fake, None) == -1
    # pooling factor that does not divide the grid
    assert L.area_pool_kv(ctypes.byref(p), 3, fake, fake, fake, fake, None) == -2
    # workspace too small / missing / misaligned
    assert L.area_full_attn(ctypes.byref(p), fake, fake, fake, fake, fake, 16, None) == -4
    assert L.area_full_attn(ctypes.byref(p), fake, fake, fake, fake, None, 1 << 40, None) == -4
    assert L.area_full_attn(ctypes.byref(p), fake, fake, fake, fake, ctypes.c_void_p(0x1008), 1 << 40, None) == -4
    # a coarse step index given to a window call
    assert L.area_window_plan(ctypes.byref(p), 0, fake, fake, fake, fake, fake, fake, 1 << 40, None) == -1
    assert L.area_window_attn(ctypes.byref(p), 99, fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None) == -1
    assert b"Phase II" in L.area_last_error() or b"step" in L.area_last_error()
    assert L.area_validate(None) == -1
    assert L.area_strerror(-4) == b"workspace missing or too small"


def test_workspace_sizes():
    p = prob("flux-6144")
    up = lambda x: (x + 255) // 256 * 256
    BH = p.B * p.H
    tok = BH * p.N * p.D * 2
    tab = 2 * max(p.Gh, p.Gw) * (p.D // 4) * 8                 # (cos, sin) tables
    exps = 2 * up(BH * (p.N // 64) * 4)                        # per-tile exponents of K and V
    words = up((BH + 9 + BH * (p.N // 256)) * 4)               # range flags, scaled-item list
    # fp16 key rows + V^T tiles + tables + exponents + range words; coarse
    # attention has the same layout (pooled keys down to f = 1)
    assert A.area_workspace_bytes(p, A.OP_FULL) == 2 * tok + tab + exps + words
    assert A.area_workspace_bytes(p, A.OP_COARSE) == A.area_workspace_bytes(p, A.OP_FULL)
    # window workspace covers the table, gathered k and V^T tiles, and the fp32
    # outputs of the largest step
    wl = W.get("flux-6144")
    qmax = max(len(O.axis_windows(wl.Gh, w, 0, t, 0)[0]) * len(O.axis_windows(wl.Gw, w, 0, t, 1)[0])
               * min(w, wl.Gh) * min(w, wl.Gw)
               for t, w in enumerate(O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)))
    assert A.area_workspace_bytes(p, A.OP_WINDOW) >= tab + qmax * p.B * p.H * p.D * 4
    assert A.area_plan_words(p) == A.PLAN_HEADER + A.PLAN_REC * 4 * 36


def test_step_workspace_covers_every_phase():
    for name in ("tiny-32", "flux-2048", "flux-6144", "qwen-6144x2048"):
        p = prob(name)
        wl = W.get(name)
        step = A.area_workspace_bytes(p, A.OP_STEP)
        # window steps: energy map, plan, weight sums, bridge indices, then the larger
        # of the plan and attention workspaces
        win_min = max(A.area_workspace_bytes(p, A.OP_PLAN), A.area_workspace_bytes(p, A.OP_WINDOW))
        win_min += 4 * A.area_plan_words(p) + 4 * p.N + 2 * 4 * (p.N // 4) + 4 * p.B * p.H * p.bridge_k
        assert step >= win_min
        # coarse steps: pooled K and V at the ramp's smallest factor, then the coarse workspace
        f_small = min(A.area_step_info(p, s)["f"] for s in range(wl.p1_steps))
        pooled = 2 * p.B * p.H * (p.N // f_small ** 2) * p.D * 2
        assert step >= pooled + A.area_workspace_bytes(p, A.OP_COARSE)
    # a canvas at or below native keeps full attention: the step needs the full workspace
    g = prob("tiny-32", native_h=32, native_w=32)
    assert A.area_workspace_bytes(g, A.OP_STEP) == A.area_workspace_bytes(g, A.OP_FULL)


def test_step_rejects_bad_arguments_before_launch():
    L = A.lib()
    p = prob("flux-2048").c()
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    # NULL q, step out of range, latent with C < 1, workspace missing / too small
    assert L.area_attn_step(ctypes.byref(p), 0, 0, None, None, fake, fake, fake, fake, big, None) == -1
    assert L.area_attn_step(ctypes.byref(p), 10 ** 6, 0, None, fake, fake, fake, fake, fake, big, None) == -1
    assert L.area_attn_step(ctypes.byref(p), 0, 0, fake, fake, fake, fake, fake, fake, big, None) == -1
    assert L.area_attn_step(ctypes.byref(p), 0, 0, None, fake, fake, fake, fake, None, big, None) == -4
    assert L.area_attn_step(ctypes.byref(p), 9, 16, fake, fake, fake, fake, fake, fake, 64, None) == -4


@pytest.mark.parametrize("name", ["tiny-32", "flux-2048", "flux-4096", "flux-6144", "qwen-6144x2048"])
def test_schedule_at_pages_knobs_matches_oracle(name):
    wl = W.get(name)
    p = prob(name, **W.PAGES_KNOBS)
    w0 = O.w_start_auto(wl.Gh, wl.Gw, wl.w_min)
    sizes = O.window_sizes(w0, wl.w_min, wl.p2_steps)
    for t, w in enumerate(sizes):
        st = A.area_step_info(p, wl.p1_steps + t)
        assert st["w"] == w, (name, t)
        assert st["R"] == O.bridge_size(w, 1, 2), (name, t)
        assert (st["bridge_rh"], st["bridge_rw"]) == O.bridge_cells(st["R"], wl.Gh, wl.Gw), (name, t)
    # configured knobs: fixed bridge at every window step, none on coarse steps
    q = prob(name)
    assert all(A.area_step_info(q, wl.p1_steps + t)["R"] == wl.bridge_k for t in range(wl.p2_steps))
    assert A.area_step_info(q, 0)["R"] == 0


def test_pages_knob_validation():
    ok = prob("flux-2048", **W.PAGES_KNOBS)
    A.area_validate(ok)
    for over, status in [(dict(bridge_rho_num=1, bridge_rho_den=0), -1), (dict(halo_max=-1), -1),
                         (dict(bridge_rho_num=-1), -1), (dict(w_start=63), -2)]:
        with pytest.raises(A.AreaError) as e:
            A.area_validate(prob("flux-2048", **over))
        assert e.value.status == status, over
    # a bridge whose cell grid cannot fit the image is rejected before anything runs
    with pytest.raises(A.AreaError) as e:
        A.area_validate(prob("tiny-32", bridge_rho_num=4, bridge_rho_den=1))
    assert e.value.status == -2


def test_phase1_steps_for_sigma_matches_oracle():
    g = np.random.default_rng(21)
    for _ in range(50):
        n = int(g.integers(0, 40))
        sig = np.sort(g.random(n))[::-1]
        s_star = float(g.random())
        assert A.area_phase1_steps_for_sigma(sig, s_star) == O.phase1_steps_for_sigma(list(sig), s_star)
    L = A.lib()
    out = ctypes.c_int(-7)
    arr = (ctypes.c_double * 2)(0.9, 0.5)
    assert L.area_phase1_steps_for_sigma(arr, 2, 0.7, ctypes.byref(out)) == 0 and out.value == 1
    assert L.area_phase1_steps_for_sigma(None, 2, 0.7, ctypes.byref(out)) == -1
    assert L.area_phase1_steps_for_sigma(arr, -1, 0.7, ctypes.byref(out)) == -1
    assert L.area_phase1_steps_for_sigma(arr, 2, float("nan"), ctypes.byref(out)) == -1
    assert L.area_phase1_steps_for_sigma(arr, 2, 0.7, None) == -1


def test_bridge_cell_grid_matches_oracle():
    """The library's bridge cell grid (area_step_info) against the oracle's
    reading, for every workload and for random grids and bridge sizes."""
    for name in ("tiny-32", "flux-2048", "flux-4096", "flux-6144", "qwen-6144x2048"):
        wl = W.get(name)
        st = A.area_step_info(prob(name), wl.p1_steps)
        assert (st["bridge_rh"], st["bridge_rw"]) == O.bridge_cells(wl.bridge_k, wl.Gh, wl.Gw), name
    rnd = random.Random(77)
    checked = 0
    while checked < 200:
        Gh, Gw = 2 * rnd.randint(4, 200), 2 * rnd.randint(4, 200)
        R = rnd.randint(1, 2000)
        p = A.Problem(B=1, H=1, D=64, Gh=Gh, Gw=Gw, native_h=4, native_w=4, p1_steps=0, p2_steps=1,
                      w_start=8, w_min=8, halo=1, bridge_k=R)
        try:
            ref = O.bridge_cells(R, Gh, Gw)
        except ValueError:
            with pytest.raises(A.AreaError):
                A.area_validate(p)
            continue
        try:
            A.area_validate(p)
        except A.AreaError:
            continue  # rejected for another reason (for example a cell row wider than 4096)
        st = A.area_step_info(p, 0)
        assert (st["bridge_rh"], st["bridge_rw"]) == ref, (Gh, Gw, R)
        checked += 1
