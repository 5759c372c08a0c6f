"""attn_fwd under HIP graph capture (GPU).

The library allocates nothing, never synchronises and only enqueues one
kernel on the caller's stream, so a caller may capture it in a graph. Each
kernel layout is captured once with preallocated outputs, and the graph is
replayed several times with eager work and synchronisations between the
replays; every replay must reproduce the eager result bit for bit (the
kernels are deterministic)."""
import pytest
import torch

from workloads import DEFAULT_SCALE, make_random

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def daf():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dense_attention_forward_amd as m
    m.lib()  # raises if the library is missing
    return m


@pytest.mark.parametrize("variant", [1, 2, 4])  # TILE128, PAIR256, PAIR128
def test_graph_replays_match_eager(daf, variant):
    print(f"case graph capture, variant={variant}", flush=True)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in make_random(1, 4, 1024, 128, seed=77, outlier_frac=0.01))
    o_ref, lse_ref = daf.forward(q, k, v, DEFAULT_SCALE, variant=variant)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # capture from a side stream, as torch recommends
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            daf.forward(q, k, v, DEFAULT_SCALE, out=o, lse=lse, variant=variant)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        o.fill_(float("nan"))  # eager work between the replays
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager result"
        assert torch.equal(lse, lse_ref), f"replay {rep}: LSE differs from the eager result"
