"""attn_decode (one query per sequence over its key/value cache) against the
fp64 oracle, through the C ABI: the oracle's queries-against-longer-keys
form with one query per sequence.  Tolerances as for attn_prefill_kv."""
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


LENS = [1, 2, 31, 32, 33, 100, 1000, 5000]


def _case(lens, hq, hkv, d, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    conv = W.BF16 if dtype == "bf16" else W.F32
    q = W.round_to(rng.standard_normal((len(lens), hq, d)), conv)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), conv)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), conv)
    return q, k, v, cu_k


def _run(q, k, v, cu_k, mask, scale, dtype, workspace=None):
    import torch

    import long_context_attention_prefill_amd as lcap

    tq, tk, tv = (G.to_device(x, dtype) for x in (q, k, v))
    out, lse = lcap.attn_decode(tq, tk, tv, [int(x) for x in cu_k], mask=mask, scale=scale,
                                lse=True, workspace=workspace)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def _check(orc, q, k, v, cu_k, mask, scale, dtype, **kw):
    got, got_lse = _run(q, k, v, cu_k, mask, scale, dtype, **kw)
    cu_q = np.arange(len(cu_k))
    want, want_lse = orc.attention(q, k, v, cu_q, mask, scale, return_lse=True, cu_seqlens_k=cu_k)
    assert G.max_err(got, want) <= G.TOL[dtype], "output"
    assert G.max_err(got_lse, want_lse) <= G.LSE_TOL[dtype], "lse"


@pytest.mark.parametrize("mask", ["causal", "full", ("window", 1), ("window", 40), ("window", 256)],
                         ids=str)
@pytest.mark.parametrize("heads", [(16, 2), (8, 8), (16, 1), (40, 1), (64, 2)], ids=str)
@pytest.mark.parametrize("d", [64, 128])
def test_decode_parity(orc, d, heads, mask):
    hq, hkv = heads
    q, k, v, cu_k = _case(LENS, hq, hkv, d, "bf16", seed=hq * 7 + d)
    _check(orc, q, k, v, cu_k, mask, 1 / math.sqrt(d), "bf16")


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
def test_decode_unusual_scales(orc, scale):
    q, k, v, cu_k = _case([3, 70, 700], 8, 2, 128, "bf16", seed=5)
    _check(orc, q, k, v, cu_k, "causal", scale, "bf16")


def test_decode_direct_mode(orc):
    """Caches that fit one chunk are written without the merge."""
    import long_context_attention_prefill_amd as lcap

    lens = [1, 5, 17, 32, 32, 2]
    assert lcap.attn_decode_workspace_size(np.concatenate([[0], np.cumsum(lens)]), 16, 2, 128) == 0
    q, k, v, cu_k = _case(lens, 16, 2, 128, "bf16", seed=6)
    _check(orc, q, k, v, cu_k, "causal", 1 / math.sqrt(128), "bf16")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 72), ("f32", 72)])
def test_decode_through_prefill_path(orc, dtype, d):
    q, k, v, cu_k = _case([1, 40, 300], 4, 2, d, dtype, seed=7)
    _check(orc, q, k, v, cu_k, "causal", 1 / math.sqrt(d), dtype)


def test_decode_many_sequences(orc):
    """More than 64 sequences: several launches share one workspace."""
    rng = np.random.Generator(np.random.PCG64(8))
    lens = rng.integers(1, 600, 150).tolist()
    q, k, v, cu_k = _case(lens, 8, 1, 128, "bf16", seed=8)
    _check(orc, q, k, v, cu_k, "causal", 1 / math.sqrt(128), "bf16")


@pytest.mark.parametrize("lens,heads", [([131072], (8, 1)), ([32768], (256, 1))], ids=str)
def test_decode_long_cache(orc, lens, heads):
    """Hundreds of chunks per (sequence, head): the merge takes several passes
    of loads, with one (sequence, head) per workgroup or spread over several."""
    hq, hkv = heads
    q, k, v, cu_k = _case(lens, hq, hkv, 128, "bf16", seed=12)
    _check(orc, q, k, v, cu_k, "causal", 1 / math.sqrt(128), "bf16")


def test_decode_workspace_reuse(orc):
    """One workspace for two calls in a row, the second on a smaller cache."""
    import torch

    import long_context_attention_prefill_amd as lcap

    big = [4000, 3000]
    small = [50, 700]
    need = lcap.attn_decode_workspace_size(np.concatenate([[0], np.cumsum(big)]), 16, 2, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for lens, seed in ((big, 9), (small, 10)):
        q, k, v, cu_k = _case(lens, 16, 2, 128, "bf16", seed=seed)
        _check(orc, q, k, v, cu_k, "causal", 1 / math.sqrt(128), "bf16", workspace=ws)


def test_decode_matches_prefill_kv():
    """The same attention as attn_prefill_kv with one query per sequence."""
    import torch

    import long_context_attention_prefill_amd as lcap

    q, k, v, cu_k = _case(LENS, 16, 2, 128, "bf16", seed=11)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    cu = [int(x) for x in cu_k]
    a, la = lcap.attn_decode(tq, tk, tv, cu, lse=True)
    b, lb = lcap.attn_prefill_kv(tq, tk, tv, list(range(len(LENS) + 1)), cu, lse=True)
    torch.cuda.synchronize()
    assert G.max_err(a.double().cpu().numpy(), b.double().cpu().numpy()) <= G.TOL["bf16"]
    assert G.max_err(la.double().cpu().numpy(), lb.double().cpu().numpy()) <= 2 * G.LSE_TOL["bf16"]
