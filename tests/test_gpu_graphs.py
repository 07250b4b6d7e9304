"""attn_prefill captured in a HIP graph (torch.cuda.graph) and replayed: a
stream under capture launches without work tickets, so the replays run
items bound to workgroups, and every replay must equal, bit for bit, the
eager call (which takes tickets when the launch is heavy).  Replays are
interleaved with eager launches and synchronisations, and inputs are
rewritten in place between replays."""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


CASES = {
    # 65 tiles x 32 heads = 2080 items: eager launches take tickets
    "causal-heavy": (np.array([0, 8320]), 32, 2, 128, "causal"),
    # 3152 items at head_dim 128: 32-key tiles
    "window-many": (np.cumsum([0, 8000, 7001, 0, 5000, 4575, 1, 130]), 16, 2, 128, ("window", 64)),
    "small-d72": (np.array([0, 300, 301, 777]), 8, 8, 72, "full"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    import torch

    import long_context_attention_prefill_amd as lcap

    cu, hq, hkv, d, mask = CASES[name]
    cu_l = [int(x) for x in cu]
    inputs = [W.draw_qkv(cu, hq, hkv, d, W.BF16, 1.0, seed=90 + s) for s in range(2)]
    dev = [[G.to_device(x, "bf16") for x in trio] for trio in inputs]
    q, k, v = (t.clone() for t in dev[0])
    scale = 1 / math.sqrt(d)
    want = [lcap.attn_prefill(*trio, cu_l, mask=mask, scale=scale) for trio in dev]
    torch.cuda.synchronize()

    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on the capture stream first
        lcap.attn_prefill(q, k, v, cu_l, mask=mask, scale=scale, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        lcap.attn_prefill(q, k, v, cu_l, mask=mask, scale=scale, out=out)
    torch.cuda.synchronize()

    for rep in range(4):
        src = dev[rep % 2]
        q.copy_(src[0])
        k.copy_(src[1])
        v.copy_(src[2])
        out.fill_(float("nan"))
        graph.replay()
        eager = lcap.attn_prefill(*src, cu_l, mask=mask, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(out, want[rep % 2]), f"{name}: replay {rep} differs from the eager call"
        assert torch.equal(eager, want[rep % 2]), f"{name}: eager call {rep} differs"
