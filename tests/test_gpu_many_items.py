"""head_dim-128 launches of many items (>= 3072 workgroups): window and
full masks run 32-key tiles at three workgroups per CU, causal masks 64-key
tiles with work tickets.  Element-wise against the fp64 oracle where it
finishes in seconds (window and full masks over packed batches, every row),
and for causal at that size through the exact probes at every row (mask,
first and last visible key, KV head map) plus sampled oracle rows.  Ragged
lengths put partial tiles and empty sequences in the batch."""
import math

import numpy as np
import pytest

import gpu_util as G
import probes
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


def _items(cu, hq):
    lens = np.diff(np.asarray(cu))
    return int(sum((n + 127) // 128 for n in lens if n > 0)) * hq


# 63 + 55 + 40 + 36 + 1 + 2 = 197 query tiles x 16 heads = 3152 items
WINDOW_CU = np.cumsum([0, 8000, 7001, 0, 5000, 4575, 1, 130])
# 64 sequences (one launch) of 257..383 tokens: 3 tiles x 16 heads each
FULL_LENS = [257 + (37 * i) % 128 for i in range(64)]
FULL_CU = np.cumsum([0] + FULL_LENS)
# 97 query tiles (the last partial) x 32 heads = 3104 items
CAUSAL_CU = np.array([0, 12400])


@pytest.mark.parametrize("mask,cu,hq,hkv", [
    (("window", 64), WINDOW_CU, 16, 2),
    (("window", 200), WINDOW_CU, 16, 16),
    ("full", FULL_CU, 16, 2),
], ids=["window64-gqa8", "window200-mha", "full-short-seqs"])
def test_many_items_against_oracle(orc, mask, cu, hq, hkv):
    assert _items(cu, hq) >= 3072
    q, k, v = W.draw_qkv(cu, hq, hkv, D, W.BF16, 1.0, seed=81)
    got = G.run_hip(q, k, v, cu, mask, 1 / math.sqrt(D), "bf16")
    want = orc.attention(q, k, v, cu, mask, 1 / math.sqrt(D))
    assert G.max_err(got, want) <= G.TOL["bf16"]


def test_many_items_causal_sampled_rows(orc):
    cu, hq, hkv = CAUSAL_CU, 32, 2
    assert _items(cu, hq) >= 3072
    q, k, v = W.draw_qkv(cu, hq, hkv, D, W.BF16, 1.0, seed=82)
    got = G.run_hip(q, k, v, cu, "causal", 1 / math.sqrt(D), "bf16")
    pick = np.array([0, 1, 31, 32, 127, 128, 4095, 6000, 12287, 12288, 12399])
    rows = np.repeat(pick, 4)
    heads = np.tile(np.array([0, 7, 16, 31]), pick.size)
    want = orc.attention_rows(q, k, v, cu, "causal", 1 / math.sqrt(D), rows, heads)
    assert G.max_err(got[rows, heads], want) <= G.TOL["bf16"]


@pytest.mark.parametrize("mask,cu,hq,hkv", [
    ("causal", CAUSAL_CU, 32, 2),
    (("window", 64), WINDOW_CU, 16, 2),
], ids=["causal", "window64"])
def test_many_items_probe_count(mask, cu, hq, hkv):
    q, k, v = W.probe_count_inputs(cu, hq, hkv, D)
    got = G.run_hip(q, k, v, cu, mask, 1 / math.sqrt(D), "bf16")
    probes.check_count_output(got, cu, mask, D)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("mask,cu,hq,hkv", [
    ("causal", CAUSAL_CU, 32, 2),
    (("window", 64), WINDOW_CU, 16, 2),
], ids=["causal", "window64"])
def test_many_items_probe_index(mask, cu, hq, hkv, sign):
    q, k, v = W.probe_index_inputs(cu, hq, hkv, D, sign)
    got = G.run_hip(q, k, v, cu, mask, 1 / math.sqrt(D), "bf16")
    probes.check_index_output(got, cu, mask, hq, hkv, sign)


def test_many_items_kv_with_lse(orc):
    """Queries ending longer key sequences, with the log-sum-exp, at 3000+ items."""
    lens_q = [6000, 5000, 0, 8800, 1]
    lens_k = [6000, 5600, 300, 9000, 900]
    cu_q, cu_k = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    hq, hkv = 32, 4
    assert _items(cu_q, hq) >= 3072
    rng = np.random.Generator(np.random.PCG64(83))
    q = W.round_to(rng.standard_normal((int(cu_q[-1]), hq, D)), W.BF16)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, D)), W.BF16)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, D)), W.BF16)
    mask = ("window", 96)
    got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, 1 / math.sqrt(D), "bf16", lse=True)
    want, want_lse = orc.attention(q, k, v, cu_q, mask, 1 / math.sqrt(D), return_lse=True, cu_seqlens_k=cu_k)
    assert G.max_err(got, want) <= G.TOL["bf16"]
    assert G.max_err(got_lse, want_lse) <= G.LSE_TOL["bf16"]
