"""HIP graph capture of whole attention steps.

The library's device calls only enqueue kernels on the caller's stream: no
allocation, no memset, no synchronisation.  A caller can therefore capture a
step (Haar map, plan, bridge, gather, attention, blend; or pooling and coarse
attention) into a graph once and replay it.  Each replay here follows eager
work on the same buffers and must reproduce the eager output bit for bit."""
import sys

import pytest

torch = pytest.importorskip("torch")

import resolution_diffusion_transformer_amd as A
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-graph]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


@pytest.mark.parametrize("name", ["tiny-32", "flux-2048"])
def test_step_graph_replays_match_eager(name):
    wl = W.get(name)
    p = A.problem_for(wl)
    q, k, v = (t.cuda() for t in W.make_qkv(wl, device="cpu", dtype="bf16"))
    lat = torch.from_numpy(W.make_latent(wl)).cuda()
    ws = A.workspace(p, A.OP_STEP)
    for s in (0, wl.p1_steps - 1, wl.p1_steps, wl.p1_steps + wl.p2_steps - 1):
        say(f"{name} step {s}: phase {A.area_step_info(p, s)['phase']}")
        eager = A.area_attn_step(p, s, lat, q, k, v, ws=ws).clone()
        out = torch.empty_like(q)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture, as torch asks
            A.area_attn_step(p, s, lat, q, k, v, out=out, ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            A.area_attn_step(p, s, lat, q, k, v, out=out, ws=ws)
        torch.cuda.synchronize()
        for r in range(3):
            out.zero_()
            # eager use of the same workspace between replays
            A.area_attn_step(p, (s + 1) % (wl.p1_steps + wl.p2_steps), lat, q, k, v, ws=ws)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), (name, s, r)
        del g
