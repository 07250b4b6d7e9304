"""Key halves (bf16 launches of few items: 64-row workgroups whose two pairs
of waves sweep the two halves of the key tiles and merge their softmax
partitions in LDS) against the fp64 oracle, through the C ABI, next to the
same head dims and masks on launches that run whole 128-row tiles.

``takes_halves`` restates the planner's rule so every case asserts which
path it exercises.  Tolerances as in test_gpu_parity (max abs 2e-2 for bf16)
and test_gpu_kv (log-sum-exp); mask, offsets and the overflow re-sweep (the
index probe's scores grow 45 nats per key) are checked bit-exactly by the
probes.
"""
import math
import zlib

import numpy as np
import pytest

import gpu_util as G
import probes
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

FEW_ITEMS = 128  # 128-row items of a launch that leaves CUs idle
MAX_ITEMS = 384  # unequal items: up to 1.5 per CU


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


def takes_halves(cu_q, cu_k, hq, mask):
    """The planner's choice for one launch (<= 64 sequences) of bf16 work."""
    nq = np.diff(np.asarray(cu_q, dtype=np.int64))
    nk = np.diff(np.asarray(cu_k, dtype=np.int64))
    items, keys = 0, []
    for a, b in zip(nq, nk):
        off = b - a
        for q0 in range(0, int(a), 128):
            q1 = min(q0 + 128, a) - 1 + off
            lo, hi = 0, b
            if mask == "causal":
                hi = q1 + 1
            elif mask != "full":
                w = mask[1]
                lo = ((q0 + off) // w) * w
                hi = min((q1 // w) * w + w, b)
            items += hq
            keys.append(hi - lo)
    if items <= FEW_ITEMS:
        return True
    if items > MAX_ITEMS:
        return False
    return 2 * max(keys) * items >= 3 * sum(keys) * hq


def _draw(cu_q, cu_k, hq, hkv, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = W.round_to(rng.standard_normal((int(cu_q[-1]), hq, d)), W.BF16)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    return q, k, v


MASKS = ["causal", "full", ("window", 100), ("window", 256)]
# (cu, hq, hkv, halves expected): ragged batches of few items, and launches
# of many equal items (whole rows)
CASES = {
    "halves-ragged": ([0, 700, 701, 1900, 1964], 4, 2, True),
    "halves-one-tile": ([0, 97], 8, 8, True),
    "whole-rows": ([0, 3000, 3001, 4100], 16, 2, False),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("d", [64, 72, 128])
def test_halves_and_whole_rows(orc, d, mask, case):
    cu, hq, hkv, halves = CASES[case]
    assert takes_halves(cu, cu, hq, mask) == halves
    seed = zlib.crc32(f"halves{d}{mask}{case}".encode()) % 10000
    q, k, v = _draw(cu, cu, hq, hkv, d, seed)
    scale = 1.0 / math.sqrt(d)
    got = G.run_hip(q, k, v, cu, mask, scale, "bf16")
    want = orc.attention(q, k, v, cu, mask, scale)
    assert G.max_err(got, want) <= G.TOL["bf16"]


KV_CASES = {
    "prefix": ([0, 300], [0, 2000]),
    "chunks": ([0, 129, 130, 400], [0, 1500, 1600, 2300]),
}


@pytest.mark.parametrize("layout", sorted(KV_CASES))
@pytest.mark.parametrize("mask", ["causal", "full", ("window", 200)], ids=str)
@pytest.mark.parametrize("d", [72, 128])
def test_halves_kv_with_lse(orc, d, mask, layout):
    """Queries over a longer key sequence (bottom-right alignment), with the
    log-sum-exp, which the merge recombines from both halves."""
    cu_q, cu_k = KV_CASES[layout]
    hq, hkv = 8, 2
    assert takes_halves(cu_q, cu_k, hq, mask)
    seed = zlib.crc32(f"halveskv{d}{mask}{layout}".encode()) % 10000
    q, k, v = _draw(cu_q, cu_k, hq, hkv, d, seed)
    scale = 1.0 / math.sqrt(d)
    want, want_lse = orc.attention(q, k, v, cu_q, mask, scale, return_lse=True, cu_seqlens_k=cu_k)
    got, got_lse = G.run_hip_kv(q, k, v, cu_q, cu_k, mask, scale, "bf16")
    assert G.max_err(got, want) <= G.TOL["bf16"], "output"
    assert G.max_err(got_lse, want_lse) <= G.LSE_TOL["bf16"], "lse"


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("mask", ["causal", "full", ("window", 256)], ids=str)
@pytest.mark.parametrize("d", [64, 128])
def test_halves_probe_index(d, mask, sign):
    """Every row: exact first or last visible key and KV head; the probe's
    scores overflow the first tile's reference, so each half re-sweeps for
    its exact maxima before the merge."""
    cu, hq, hkv = np.array([0, 2048]), 8, 8
    assert takes_halves(cu, cu, hq, mask)
    q, k, v = W.probe_index_inputs(cu, hq, hkv, d, sign)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / math.sqrt(d), "bf16")
    probes.check_index_output(got, cu, mask, hq, hkv, sign)


@pytest.mark.parametrize("mask", ["causal", ("window", 64), ("window", 300)], ids=str)
def test_halves_probe_count(mask):
    """Every row: exact count of visible keys per class, over a ragged batch."""
    cu, hq, hkv, d = np.array([0, 1000, 1001, 2500]), 4, 2, 72
    assert takes_halves(cu, cu, hq, mask)
    q, k, v = W.probe_count_inputs(cu, hq, hkv, d)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / math.sqrt(d), "bf16")
    probes.check_count_output(got, cu, mask, d)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("mask", ["causal", "full", ("window", 256)], ids=str)
@pytest.mark.parametrize("d", [64, 72, 128])
def test_whole_rows_probe_index(d, mask, sign):
    """The same exact probes on a launch of many items (whole 128-row tiles,
    64-key steps at every head dim): first or last visible key and KV head at
    every row, with the probe's overflow and re-sweep in every workgroup."""
    cu, hq, hkv = np.array([0, 3000, 3001, 4100]), 16, 16
    assert not takes_halves(cu, cu, hq, mask)
    q, k, v = W.probe_index_inputs(cu, hq, hkv, d, sign)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / math.sqrt(d), "bf16")
    probes.check_index_output(got, cu, mask, hq, hkv, sign)


@pytest.mark.parametrize("mask", ["causal", "full", ("window", 300)], ids=str)
@pytest.mark.parametrize("d", [64, 72])
def test_whole_rows_probe_count(d, mask):
    """Every row of a launch of many items: exact count of visible keys."""
    cu, hq, hkv = np.array([0, 3000, 3001, 4100]), 16, 2
    assert not takes_halves(cu, cu, hq, mask)
    q, k, v = W.probe_count_inputs(cu, hq, hkv, d)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / math.sqrt(d), "bf16")
    probes.check_count_output(got, cu, mask, d)
