"""attn_prefill_kv (queries that end longer key sequences: chunked prefill,
decode) against the fp64 oracle, through the C ABI.

Tolerances: outputs as for attn_prefill (max abs 2e-2 bf16, 1e-4 fp32); the
log-sum-exp within 2^-8 (bf16) and 1e-4 (fp32), derived in gpu_util.  Mask
and offset handling is checked bit-exactly by the count and index probes.
"""
import math
import zlib

import numpy as np
import pytest

import gpu_util as G
import probes
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


KV_LAYOUTS = {
    "chunks": ([0, 100, 100, 229], [0, 300, 357, 500]),
    "decode": ([0, 1, 2, 3, 4], [0, 1, 65, 200, 457]),
    "square": ([0, 129, 300], [0, 129, 300]),
    "tail": ([0, 5], [0, 1000]),
}
MASKS = ["causal", "full", ("window", 1), ("window", 7), ("window", 64), ("window", 256)]


def _draw(cu_q, cu_k, hq, hkv, d, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    conv = (lambda x: W.round_to(x, W.BF16)) if dtype == "bf16" else (lambda x: W.round_to(x, W.F32))
    q = conv(rng.standard_normal((int(cu_q[-1]), hq, d)))
    k = conv(rng.standard_normal((int(cu_k[-1]), hkv, d)))
    v = conv(rng.standard_normal((int(cu_k[-1]), hkv, d)))
    return q, k, v


@pytest.mark.parametrize("layout", sorted(KV_LAYOUTS))
@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("d", [64, 72, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_small_parity(orc, dtype, d, mask, layout):
    cu_q, cu_k = KV_LAYOUTS[layout]
    hq, hkv = (4, 2) if d != 72 else (3, 1)
    seed = zlib.crc32(f"kv{dtype}{d}{mask}{layout}".encode()) % 10000
    q, k, v = _draw(cu_q, cu_k, hq, hkv, d, dtype, seed)
    scale = 1.0 / math.sqrt(d)
    want, want_lse = orc.attention(q, k, v, cu_q, mask, scale, return_lse=True, cu_seqlens_k=cu_k)
    got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, scale, dtype)
    assert G.max_err(got, want) <= G.TOL[dtype], "output"
    assert G.max_err(got_lse, want_lse) <= G.LSE_TOL[dtype], "lse"


def test_kv_square_equals_prefill():
    """With equal packings the kv entry point is attn_prefill, bit for bit."""
    import torch

    import long_context_attention_prefill_amd as lcap

    cu = [0, 300, 301, 777]
    q, k, v = _draw(cu, cu, 4, 2, 128, "bf16", 9)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    for mask in ("causal", "full", ("window", 33)):
        a = lcap.attn_prefill(tq, tk, tv, cu, mask=mask)
        b = lcap.attn_prefill_kv(tq, tk, tv, cu, cu, mask=mask)
        torch.cuda.synchronize()
        assert torch.equal(a, b), mask


def test_kv_lse_into_given_tensor():
    import torch

    import long_context_attention_prefill_amd as lcap

    cu_q, cu_k = [0, 3], [0, 50]
    q, k, v = _draw(cu_q, cu_k, 2, 1, 64, "f32", 4)
    tq, tk, tv = (G.to_device(x, "f32") for x in (q, k, v))
    lse = torch.full((3, 2), 7.0, device="cuda")
    out, l2 = lcap.attn_prefill_kv(tq, tk, tv, cu_q, cu_k, lse=lse)
    torch.cuda.synchronize()
    assert l2 is lse and not bool((lse == 7.0).any())


def _sample_rows(cu_q, hq, rng, per_seq=10):
    rows = []
    for b in range(len(cu_q) - 1):
        s, n = int(cu_q[b]), int(cu_q[b + 1] - cu_q[b])
        if n == 0:
            continue
        pick = {0, n // 2, n - 1} | set(rng.integers(0, n, per_seq).tolist())
        rows += [s + i for i in sorted(pick)]
    rows = np.array(rows)
    return np.repeat(rows, hq), np.tile(np.arange(hq), rows.size)


def test_kv_chunked_prefill_10k(orc):
    """The last 2048 queries of a 10240-token sequence (16/2 heads, d 128,
    bf16, causal) over all its keys: sampled rows and their LSE."""
    cu_q, cu_k = [0, 2048], [0, 10240]
    q, k, v = _draw(cu_q, cu_k, 16, 2, 128, "bf16", 10)
    got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, "causal", 1 / math.sqrt(128), "bf16")
    rows, heads = _sample_rows(cu_q, 16, np.random.Generator(np.random.PCG64(3)))
    want, want_lse = orc.attention_rows(q, k, v, cu_q, "causal", 1 / math.sqrt(128), rows, heads,
                                        return_lse=True, cu_seqlens_k=cu_k)
    assert G.max_err(got[rows, heads], want) <= G.TOL["bf16"]
    assert G.max_err(got_lse[rows, heads], want_lse) <= G.LSE_TOL["bf16"]


def test_kv_decode_batch(orc):
    """One new query per sequence over caches of 1 .. 8192 tokens."""
    lens = [1, 2, 17, 128, 129, 1000, 4096, 8192]
    cu_k = np.concatenate([[0], np.cumsum(lens)])
    cu_q = np.arange(len(lens) + 1)
    q, k, v = _draw(cu_q, cu_k, 16, 2, 128, "bf16", 11)
    for mask in ("causal", ("window", 256)):
        got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, 1 / math.sqrt(128), "bf16")
        want, want_lse = orc.attention(q, k, v, cu_q, mask, 1 / math.sqrt(128), return_lse=True,
                                       cu_seqlens_k=cu_k)
        assert G.max_err(got, want) <= G.TOL["bf16"], mask
        assert G.max_err(got_lse, want_lse) <= G.LSE_TOL["bf16"], mask


PROBE_KV = ([0, 1, 301, 301, 1600], [0, 700, 1000, 1290, 5000])


@pytest.mark.parametrize("mask", ["causal", "full", ("window", 1), ("window", 256)], ids=str)
@pytest.mark.parametrize("d", [64, 128])
def test_kv_probe_count(mask, d):
    cu_q, cu_k = (np.array(c) for c in PROBE_KV)
    q, k, v = W.probe_count_inputs(cu_q, 4, 2, d, cu_k=cu_k)
    got = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, 1 / math.sqrt(d), "bf16", lse=False)
    probes.check_count_output_kv(got, cu_q, cu_k, mask, d)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("mask", ["causal", "full", ("window", 64)], ids=str)
def test_kv_probe_index(mask, sign):
    cu_q, cu_k = (np.array(c) for c in PROBE_KV)
    q, k, v = W.probe_index_inputs(cu_q, 4, 2, 128, sign, cu_k=cu_k)
    got = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, 1 / math.sqrt(128), "bf16", lse=False)
    probes.check_index_output_kv(got, cu_q, cu_k, mask, 4, 2, sign)
