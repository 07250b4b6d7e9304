"""Heavy causal launches with work tickets (workgroups past the first wave
claim items from a per-stream device counter).  Which workgroup computes an
item does not change its arithmetic, so the output must equal, bit for bit,
that of launches too small to take tickets (the same heads, a quarter at a
time); repeated launches on one stream check that each launch leaves its
counters at zero, and launches interleaved on two streams that streams keep
separate counters.  A few rows are also checked against the fp64 oracle."""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

# 65 query tiles of 128 rows x 32 heads = 2080 items, over twice the 512
# workgroup slots of a 256-CU device; a quarter of the heads (520 items) is not
N, HQ, HKV, D = 8320, 32, 2, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


def _inputs(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = W.round_to(rng.standard_normal((N, HQ, D)), W.BF16)
    k = W.round_to(rng.standard_normal((N, HKV, D)), W.BF16)
    v = W.round_to(rng.standard_normal((N, HKV, D)), W.BF16)
    return q, k, v


def _by_quarters(tq, tk, tv):
    """The same attention as four launches of 8 query heads (one KV head each)."""
    import torch

    import long_context_attention_prefill_amd as lcap

    parts = []
    for j in range(4):
        hk = (8 * j) // (HQ // HKV)
        parts.append(lcap.attn_prefill(tq[:, 8 * j:8 * j + 8].contiguous(), tk[:, hk:hk + 1].contiguous(),
                                       tv[:, hk:hk + 1].contiguous(), [0, N], mask="causal"))
    return torch.cat(parts, dim=1)


def test_tickets_match_small_launches_and_oracle(orc):
    import torch

    import long_context_attention_prefill_amd as lcap

    q, k, v = _inputs(91)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    want = _by_quarters(tq, tk, tv)
    outs = [lcap.attn_prefill(tq, tk, tv, [0, N], mask="causal") for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, want), "a ticketed launch differs from the per-quarter launches"
    rows = np.repeat(np.array([0, 1, 127, 128, 4000, N - 1]), 4)
    heads = np.tile(np.array([0, 15, 16, 31]), 6)
    ref = orc.attention_rows(q, k, v, np.array([0, N]), "causal", 1 / math.sqrt(D), rows, heads)
    got = outs[0].double().cpu().numpy()
    assert G.max_err(got[rows, heads], ref) <= G.TOL["bf16"]


def test_tickets_on_two_streams():
    import torch

    import long_context_attention_prefill_amd as lcap

    ins = [_inputs(92), _inputs(93)]
    dev = [[G.to_device(x, "bf16") for x in trio] for trio in ins]
    want = [_by_quarters(*d) for d in dev]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = [[], []]
    for _ in range(3):
        for i, s in enumerate((s1, s2)):
            got[i].append(lcap.attn_prefill(*dev[i], [0, N], mask="causal", stream=s))
    s1.synchronize()
    s2.synchronize()
    torch.cuda.synchronize()
    for i in range(2):
        for o in got[i]:
            assert torch.equal(o, want[i]), f"stream {i + 1}: output differs from the per-quarter launches"


def test_tickets_between_other_launches():
    """Heavy, small and non-causal launches alternate on one stream."""
    import torch

    import long_context_attention_prefill_amd as lcap

    q, k, v = _inputs(94)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    want = _by_quarters(tq, tk, tv)
    small = lcap.attn_prefill(tq[:300].contiguous(), tk[:300].contiguous(), tv[:300].contiguous(), [0, 300],
                              mask="causal")
    full = lcap.attn_prefill(tq[:1000].contiguous(), tk[:1000].contiguous(), tv[:1000].contiguous(), [0, 1000],
                             mask="full")
    torch.cuda.synchronize()
    for _ in range(2):
        a = lcap.attn_prefill(tq, tk, tv, [0, N], mask="causal")
        b = lcap.attn_prefill(tq[:300].contiguous(), tk[:300].contiguous(), tv[:300].contiguous(), [0, 300],
                              mask="causal")
        c = lcap.attn_prefill(tq[:1000].contiguous(), tk[:1000].contiguous(), tv[:1000].contiguous(),
                              [0, 1000], mask="full")
        torch.cuda.synchronize()
        assert torch.equal(a, want)
        assert torch.equal(b, small)
        assert torch.equal(c, full)
