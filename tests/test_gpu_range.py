"""GPU parity for inputs far outside fp16's range.

The attention operands are fp16, whose largest value is 65504 while bf16
inputs reach 3e38.  Each 64-key tile of K and of V, and each query row, is
stored at its own power-of-two scale (1 for magnitudes in [2^-8, 2^15)) and
the attention kernel undoes nonzero scales in fp32.  Every head below sits in
another magnitude regime; its output, divided by the factor its V was
multiplied by, must match the float64 oracle (fed the same bf16 inputs,
divided the same way) within the usual max-abs 2e-2 and mean-abs 2e-3, with
no inf or NaN.  Large keys are paired with small queries (and the other way
round) so that the scores keep their usual size: a score of 1e5 log2 units
would make the softmax hinge on differences far below fp16's resolution of
the score, an ill-conditioned case no 16-bit operand format can serve.

Heads: 0 unscaled; 1 V x 1e5; 2 K x 1e5 with Q x 1e-5; 3 V x 1e-6; 4 K x 1e-6
with Q x 1e6; 5 the value rows of the top quarter of the grid x 3e4 (tiles of
very different scales in one key set) and the key rows of the bottom quarter
x 1e-6; 6 every other query row x 1e-6 (rows of one wave at different
scales); 7 K x 1e12 with Q x 1e-12 (the bridge's fixed-point key sum
saturates each key at 2^28, so its integer total stays exact)."""
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
    print("[gpu-range]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


WL = W.Workload("range-32", B=1, H=8, D=128, Gh=32, Gw=32, native_h=16, native_w=16, dtype="bf16",
                p1_steps=2, f_min=2, p2_steps=3, w_start=16, w_min=8, halo=1, bridge_k=16,
                latent_kind="tiny_patches")
V_SCALE = [1.0, 1e5, 1.0, 1e-6, 1.0, 3e4, 1.0, 1.0]   # the largest factor applied to each head's V


@pytest.fixture(scope="module")
def scaled_inputs():
    q, k, v = (t.float() for t in W.make_qkv(WL, device="cpu", dtype="fp32", seed=21))
    y = torch.arange(WL.N) // WL.Gw
    v[0, 1] *= 1e5
    k[0, 2] *= 1e5
    q[0, 2] *= 1e-5
    v[0, 3] *= 1e-6
    k[0, 4] *= 1e-6
    q[0, 4] *= 1e6
    v[0, 5, y < WL.Gh // 4] *= 3e4
    k[0, 5, y >= 3 * WL.Gh // 4] *= 1e-6
    q[0, 6, 1::2] *= 1e-6
    k[0, 7] *= 1e12
    q[0, 7] *= 1e-12
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    host = [t.float().numpy().astype(np.float64) for t in (q, k, v)]
    return (q.cuda(), k.cuda(), v.cuda()), host


def check(got, ref, what):
    got = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    for h in range(WL.H):
        err = np.abs(got[:, h] - ref[:, h]) / V_SCALE[h]
        say(f"{what} head {h}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} (after / {V_SCALE[h]:g})")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, h)


def test_full_attention_any_range(scaled_inputs):
    (q, k, v), (qh, kh, vh) = scaled_inputs
    p = A.problem_for(WL)
    out = A.area_full_attn(p, q, k, v)
    torch.cuda.synchronize()
    check(out, O.full_attention(qh, kh, vh, WL.Gh, WL.Gw, WL.rope_theta), "full")


@pytest.mark.parametrize("mode", [A.POOL_MEAN, A.POOL_CENTER])
def test_coarse_attention_any_range(scaled_inputs, mode):
    (q, k, v), (qh, kh, vh) = scaled_inputs
    p = A.problem_for(WL, pool_mode=mode)
    f = 2
    kp, vp = A.area_pool_kv(p, f, k, v)
    out = A.area_coarse_attn(p, f, q, kp, vp)
    torch.cuda.synchronize()
    kpr, vpr = O.pool_kv(kh, vh, WL.Gh, WL.Gw, f, mode, WL.rope_theta)
    check(out, O.coarse_attention(qh, kpr, vpr, WL.Gh, WL.Gw, f, WL.rope_theta), f"coarse mode={mode}")


def test_window_attention_any_range(scaled_inputs):
    (q, k, v), (qh, kh, vh) = scaled_inputs
    p = A.problem_for(WL)
    lat = W.make_latent(WL)
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(lat).cuda())
    Eq_ref = O.energy_fixed(O.detail_energy(lat))
    sizes = O.window_sizes(WL.w_start, WL.w_min, WL.p2_steps)
    br_ref = O.bridge_all(kh, WL.bridge_k, WL.Gh, WL.Gw)
    for t in (0, WL.p2_steps - 1):
        step = WL.p1_steps + t
        plan, wsum, br = A.area_window_plan(p, step, Eq, k)
        out = A.area_window_attn(p, step, plan, wsum, br, q, k, v)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(br.cpu().numpy(), br_ref)
        ref = O.window_plan(WL.Gh, WL.Gw, sizes[t], WL.halo, WL.seed, t, Eq_ref)
        check(out, O.window_attention(qh, kh, vh, ref, br_ref, WL.Gh, WL.Gw, WL.rope_theta), f"window step {t}")


def test_in_range_heads_take_the_plain_path(scaled_inputs):
    # the unscaled head's output does not depend on the other heads' ranges:
    # it equals a run where every head is unscaled, bit for bit
    (q, k, v), _ = scaled_inputs
    p = A.problem_for(WL)
    a = A.area_full_attn(p, q, k, v)
    q1, k1, v1 = (t[:, :1].repeat(1, WL.H, 1, 1).contiguous() for t in (q, k, v))
    b = A.area_full_attn(p, q1, k1, v1)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b[:, 0])
