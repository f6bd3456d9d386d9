"""GPU parity of joint text + image sequences (T > 0): text tokens first, at
position (0, 0), left out of the pooling, in every key set; text queries dense over all
T + N keys.  Elementwise on the tiny grid with 8 text tokens, sampled rows on
FLUX.1 2048^2 with 512 text tokens; plans and bridges bit-exact; the
per-step driver equals the composed calls."""
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
    print("[gpu-text]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), what
    say(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} (n={err.size})")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, what


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def setup(name, seed=3):
    wl = W.get(name)
    p = A.problem_for(wl)
    q, k, v = (t.to(torch.bfloat16).cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16", seed=seed))
    return wl, p, q, k, v


def test_tiny_text_all_phases_elementwise():
    wl, p, q, k, v = setup("tiny-32-text")
    T = wl.T
    qh, kh, vh = host(q), host(k), host(v)
    out = A.area_full_attn(p, q, k, v)
    close(host(out), O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta, T=T), "tiny full (text + image rows)")
    txt = A.area_text_attn(p, q, k, v)
    close(host(txt)[:, :, :T], O.text_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta, T), "tiny text rows")
    for s in (0, wl.p1_steps - 1):
        f = A.area_step_info(p, s)["f"]
        kp, vp = A.area_pool_kv(p, f, k, v)
        co = A.area_coarse_attn(p, f, q, kp, vp)
        torch.cuda.synchronize()
        kpr, vpr = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta, T=T)
        close(host(kp), kpr, f"tiny pooled keys f={f} (text rows first)")
        close(host(co)[:, :, T:], O.coarse_attention(qh, kpr, vpr, wl.Gh, wl.Gw, f, wl.rope_theta, T=T),
              f"tiny coarse f={f} image rows")
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    br_ref = O.bridge_all(kh[:, :, T:], wl.bridge_k, wl.Gh, wl.Gw)
    for t, w in enumerate(O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, w, wl.halo, wl.seed, t, Eq_ref)
        nwin = int(plan[0].item())
        np.testing.assert_array_equal(plan.cpu().numpy()[16:16 + 10 * nwin].reshape(nwin, 10), ref.records())
        np.testing.assert_array_equal(br.cpu().numpy(), br_ref)
        close(host(out)[:, :, T:], O.window_attention(qh, kh, vh, ref, br_ref, wl.Gh, wl.Gw, wl.rope_theta, T=T),
              f"tiny window step {t} image rows")


def test_flux2048_text_sampled():
    wl, p, q, k, v = setup("flux-2048-text")
    T, N = wl.T, wl.N
    rng = np.random.Generator(np.random.PCG64(5))
    img_rows = np.array(sorted(set(rng.integers(0, N, 40).tolist()) | {0, N - 1}))
    txt_rows = np.array([0, 1, T // 2, T - 1])
    heads = (0, wl.H - 1)

    def hd(t, h, rows=None):
        # only the rows a call writes: the rest of an output tensor is never initialised
        t = t[:, h:h + 1] if rows is None else t[:, h:h + 1, torch.as_tensor(rows, device=t.device)]
        return t.float().cpu().numpy().astype(np.float64)

    full = A.area_full_attn(p, q, k, v)
    txt = A.area_text_attn(p, q, k, v)
    f = A.area_step_info(p, 0)["f"]
    kp, vp = A.area_pool_kv(p, f, k, v)
    co = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    for h in heads:
        qh, kh, vh = hd(q, h), hd(k, h), hd(v, h)
        rows = np.concatenate([txt_rows, T + img_rows])
        close(hd(full, h, rows), O.full_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta, rows=rows, T=T),
              f"2048 full rows (text and image) head {h}")
        close(hd(txt, h, np.arange(T)), O.text_attention(qh, kh, vh, wl.Gh, wl.Gw, wl.rope_theta, T),
              f"2048 text rows head {h}")
        kpr, vpr = O.pool_kv(kh, vh, wl.Gh, wl.Gw, f, O.POOL_MEAN, wl.rope_theta, T=T)
        close(hd(co, h, T + img_rows), O.coarse_attention(qh, kpr, vpr, wl.Gh, wl.Gw, f, wl.rope_theta,
                                                                rows=img_rows, T=T),
              f"2048 coarse f={f} image rows head {h}")
    lat = W.make_latent(wl)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    sizes = O.window_sizes(wl.w_start, wl.w_min, wl.p2_steps)
    for t in (0, wl.p2_steps - 1):
        s = wl.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, s, Eq, k)
        out = A.area_window_attn(p, s, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        ref = O.window_plan(wl.Gh, wl.Gw, sizes[t], wl.halo, wl.seed, t, Eq_ref)
        for h in heads:
            kh = hd(k, h)
            brh = O.bridge_select(kh[0, 0, T:], wl.bridge_k, wl.Gh, wl.Gw)
            np.testing.assert_array_equal(br.cpu().numpy()[0, h], brh)
            close(hd(out, h, T + img_rows),
                  O.window_attention(hd(q, h), kh, hd(v, h), ref, brh[None, None], wl.Gh, wl.Gw, wl.rope_theta,
                                     rows=img_rows, T=T),
                  f"2048 window step {t} image rows head {h}")


def test_step_with_text_equals_composed_calls():
    wl, p, q, k, v = setup("tiny-32-text", seed=4)
    lat = torch.from_numpy(W.make_latent(wl)).cuda()
    ws = A.workspace(p, A.OP_STEP, q.device)
    for s in range(wl.p1_steps + wl.p2_steps):
        got = A.area_attn_step(p, s, lat, q, k, v, ws=ws)
        st = A.area_step_info(p, s)
        ref = torch.empty_like(q)
        if st["phase"] == A.PHASE_COARSE:
            kp, vp = A.area_pool_kv(p, st["f"], k, v)
            A.area_coarse_attn(p, st["f"], q, kp, vp, out=ref)
        else:
            eq = A.area_dwt_detail(p, lat)[1]
            plan, wsum, br = A.area_window_plan(p, s, eq, k)
            A.area_window_attn(p, s, plan, wsum, br, q, k, v, out=ref)
        A.area_text_attn(p, q, k, v, out=ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), s
