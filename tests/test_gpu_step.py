"""GPU tests of area_attn_step, the per-step entry point: for every step of
the schedule its output is bit-identical to calling the individual entry
points in the order the schedule names (pool + coarse attention, or Haar
map + plan + windowed attention), with and without the latent; a canvas at
or below native size runs full attention at every step; and one coarse and
one window step are checked against the oracle."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import resolution_diffusion_transformer_amd as A
import workloads as W
from oracle import area_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-step]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


def composed(p, s, lat, q, k, v):
    st = A.area_step_info(p, s)
    if st["phase"] == A.PHASE_FULL:
        return A.area_full_attn(p, q, k, v)
    if st["phase"] == A.PHASE_COARSE:
        kp, vp = A.area_pool_kv(p, st["f"], k, v)
        return A.area_coarse_attn(p, st["f"], q, kp, vp)
    eq = A.area_dwt_detail(p, lat)[1] if lat is not None else None
    plan, wsum, br = A.area_window_plan(p, s, eq, k)
    return A.area_window_attn(p, s, plan, wsum, br, q, k, v)


@pytest.mark.parametrize("name", ["tiny-32", "flux-2048"])
@pytest.mark.parametrize("with_latent", [True, False])
def test_step_equals_composed_calls(name, with_latent):
    wl = W.get(name)
    p = A.problem_for(wl)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=3))
    lat = torch.from_numpy(W.make_latent(wl)).cuda() if with_latent else None
    ws = A.workspace(p, A.OP_STEP, q.device)
    for s in range(wl.p1_steps + wl.p2_steps):
        say(f"{name} step {s} latent={with_latent}")
        got = A.area_attn_step(p, s, lat, q, k, v, ws=ws)
        ref = composed(p, s, lat, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (name, s)


def test_gated_canvas_runs_full_attention():
    wl = W.get("tiny-32")
    p = A.problem_for(wl, native_h=wl.Gh, native_w=wl.Gw)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=4))
    full = A.area_full_attn(p, q, k, v)
    for s in (0, wl.p1_steps + wl.p2_steps - 1):
        assert torch.equal(A.area_attn_step(p, s, None, q, k, v), full)


def test_step_against_oracle():
    wl = W.get("tiny-32")
    p = A.problem_for(wl)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=5))
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k, v))
    latn = W.make_latent(wl)
    lat = torch.from_numpy(latn).cuda()
    s_c = 0
    f = A.area_step_info(p, s_c)["f"]
    got = A.area_attn_step(p, s_c, lat, q, k, v).float().cpu().numpy()
    kpr, vpr = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta)
    ref = O.coarse_attention(qh, kpr, vpr, wl.Gh, wl.Gw, f, wl.rope_theta)
    err = np.abs(got - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    t = wl.p2_steps - 1
    s_w = wl.p1_steps + t
    got = A.area_attn_step(p, s_w, lat, q, k, v).float().cpu().numpy()
    w = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)[t]
    plan = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, O.energy_fixed(O.detail_energy(latn)))
    ref = O.window_attention(qh, kh, vh, plan, O.bridge_all(kh, wl.bridge_k, wl.Gh, wl.Gw), wl.Gh, wl.Gw,
                             wl.rope_theta)
    err = np.abs(got - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
