"""Calls with more sequences than one launch holds, against the fp64 oracle.

The library splits a prefill or kv batch into launches of at most 64
sequences, and a decode batch likewise; each launch writes its own output
rows.  These cases put 70 to 150 sequences of mixed lengths (empty, single
token, ragged, several tiles) into one call, so the split, the sequences'
order inside each launch (longest first) and the row bookkeeping across
launches are all exercised.  Tolerances as in the other parity tests (max abs
2e-2 bf16, 1e-4 fp32; log-sum-exp 2^-7 bf16).
"""
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


def _lens(n, seed, max_len=260):
    """n lengths: about one in ten empty, one in ten a single token, the rest
    2 .. max_len, in no particular order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        r = rng.random()
        out.append(0 if r < 0.1 else 1 if r < 0.2 else int(rng.integers(2, max_len + 1)))
    if sum(out) == 0:
        out[0] = 1
    return out


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("mask", ["causal", "full", ("window", 64)], ids=str)
@pytest.mark.parametrize("dtype,d,heads,n", [("bf16", 128, (8, 2), 150), ("bf16", 72, (4, 4), 70),
                                             ("f32", 64, (4, 1), 130)], ids=str)
def test_prefill_many_sequences(orc, dtype, d, heads, n, mask):
    hq, hkv = heads
    cu = _cu(_lens(n, seed=n + d))
    q, k, v = W.draw_qkv(cu, hq, hkv, d, dtype, 1.0, seed=3 * n + d)
    scale = 1.0 / math.sqrt(d)
    want = orc.attention(q, k, v, cu, mask, scale)
    got = G.run_hip(q, k, v, cu, mask, scale, dtype)
    assert G.max_err(got, want) <= G.TOL[dtype], (n, mask)


@pytest.mark.parametrize("mask", ["causal", ("window", 100)], ids=str)
def test_kv_many_sequences_with_lse(orc, mask):
    """100 sequences whose queries end longer key sequences (a chunk of up to
    a third of the keys, some sequences with no query), with the log-sum-exp."""
    rng = np.random.Generator(np.random.PCG64(77))
    lk = _lens(100, seed=78, max_len=400)
    lq = [min(x, int(rng.integers(0, x // 3 + 2))) for x in lk]
    cu_q, cu_k = _cu(lq), _cu(lk)
    conv = W.BF16
    q = W.round_to(rng.standard_normal((int(cu_q[-1]), 8, 128)), conv)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), 2, 128)), conv)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), 2, 128)), conv)
    scale = 1.0 / math.sqrt(128)
    want, want_lse = orc.attention(q, k, v, cu_q, mask, scale, return_lse=True, cu_seqlens_k=cu_k)
    got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, scale, "bf16")
    assert G.max_err(got, want) <= G.TOL["bf16"], "output"
    assert G.max_err(got_lse, want_lse) <= G.LSE_TOL["bf16"], "lse"


def test_decode_many_sequences(orc):
    """140 caches of 1 .. 900 tokens, one query each, 16/2 heads, d 128."""
    import torch

    import long_context_attention_prefill_amd as lcap

    rng = np.random.Generator(np.random.PCG64(140))
    lens = [int(x) for x in rng.integers(1, 901, 140)]
    cu_k = _cu(lens)
    conv = W.BF16
    q = W.round_to(rng.standard_normal((len(lens), 16, 128)), conv)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), 2, 128)), conv)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), 2, 128)), conv)
    scale = 1.0 / math.sqrt(128)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    out, lse = lcap.attn_decode(tq, tk, tv, [int(x) for x in cu_k], mask="causal", scale=scale,
                                lse=True)
    torch.cuda.synchronize()
    cu_q = np.arange(len(cu_k))
    want, want_lse = orc.attention(q, k, v, cu_q, "causal", scale, return_lse=True, cu_seqlens_k=cu_k)
    assert G.max_err(out.double().cpu().numpy(), want) <= G.TOL["bf16"], "output"
    assert G.max_err(lse.double().cpu().numpy(), want_lse) <= G.LSE_TOL["bf16"], "lse"
