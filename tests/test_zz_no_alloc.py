"""The allocation-free plan call (area_window_plan_static) against the
workspace call (area_window_plan), through the C ABI: plans, blend-weight
sums and bridge indices must be identical, bit for bit, on two calls in a
row, the second on a smaller problem (the static scratch keeps the first
call's contents, which must not leak into the second)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import resolution_diffusion_transformer_amd as A
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-no-alloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


def _case(name, step_offset):
    wl = W.get(name)
    p = A.problem_for(wl)
    q, k, v = W.make_qkv(wl, device="cuda", dtype="bf16")
    _, Eq = A.area_dwt_detail(p, torch.from_numpy(W.make_latent(wl)).cuda())
    step = wl.p1_steps + step_offset
    a = A.area_window_plan(p, step, Eq, k)
    b = A.area_window_plan_static(p, step, Eq, k)
    torch.cuda.synchronize()
    for x, y, what in zip(a, b, ("plan", "wsum", "bridge")):
        assert (x is None) == (y is None), what
        if x is not None:
            np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=f"{name} {what}")
    say(f"{name} step {step}: plan, wsum and bridge equal ({int(a[0][0].item())} windows)")


def test_static_scratch_plan_equals_workspace_plan_twice():
    # 6144^2 (3.6 MB of bridge partial sums in the scratch), then the 32x32
    # grid, much smaller, on the same scratch
    _case("flux-6144", 1)
    _case("tiny-32", 2)


def test_static_scratch_rejects_a_plan_beyond_its_size():
    wl = W.get("flux-6144")
    p = A.problem_for(wl, B=8)  # 8 x 24 heads: about 28 MB of partial sums
    assert A.area_workspace_bytes(p, A.OP_PLAN) > (16 << 20)
    k = torch.empty((p.B, p.H, p.L, p.D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AreaError) as e:
        A.area_window_plan_static(p, wl.p1_steps, None, k)
    assert e.value.status == -4
