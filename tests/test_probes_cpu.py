"""The vectorised probe expectations against explicit visible sets, and the
oracle on the probe inputs at small sizes (CPU only)."""
import numpy as np
import pytest

import pins
import probes
from long_context_attention_prefill_amd import workloads as W

CUS = [[0, 1], [0, 37, 37, 290, 291, 600], [0, 129, 140]]
MASKS = ["causal", "full", ("window", 1), ("window", 7), ("window", 64), ("window", 1000)]


@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("cu", CUS, ids=str)
def test_interval_matches_sets(cu, mask):
    lo, hi = probes.visible_interval(cu, mask)
    for b in range(len(cu) - 1):
        s, n = cu[b], cu[b + 1] - cu[b]
        for i in range(n):
            vis = pins.visible_set(mask, i, n)
            assert set(range(lo[s + i] - s, hi[s + i] - s)) == vis


@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_oracle_passes_probe_checks(orc, mask):
    cu = np.array(CUS[1])
    q, k, v = W.probe_count_inputs(cu, 2, 1, 72)
    probes.check_count_output(orc.attention(q, k, v, cu, mask, 1 / 72 ** 0.5), cu, mask, 72)
    for sign in (1, -1):
        q, k, v = W.probe_index_inputs(cu, 4, 2, 64, sign)
        out = orc.attention(q, k, v, cu, mask, 0.125)
        probes.check_index_output(out, cu, mask, 4, 2, sign)


def test_probe_checks_catch_errors(orc):
    cu = np.array(CUS[1])
    q, k, v = W.probe_count_inputs(cu, 1, 1, 64)
    out = orc.attention(q, k, v, cu, "causal", 0.125)
    bad = out.copy()
    bad[300, 0, :] = orc.attention(q, k, v, cu, "full", 0.125)[300, 0, :]
    with pytest.raises(AssertionError):
        probes.check_count_output(bad, cu, "causal", 64)
    q, k, v = W.probe_index_inputs(cu, 2, 1, 64, 1)
    out = orc.attention(q, k, v, cu, ("window", 7), 0.125)
    with pytest.raises(AssertionError):
        probes.check_index_output(out, cu, ("window", 8), 2, 1, 1)


KV_CUS = [([0, 1, 2, 3], [0, 1, 40, 300]), ([0, 37, 37, 160], [0, 290, 291, 600]),
          ([0, 129, 140], [0, 129, 140])]


@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("cus", KV_CUS, ids=str)
def test_kv_interval_matches_sets(cus, mask):
    cu_q, cu_k = cus
    lo, hi = probes.visible_interval_kv(cu_q, cu_k, mask)
    for b in range(len(cu_q) - 1):
        sq, lq = cu_q[b], cu_q[b + 1] - cu_q[b]
        sk, lk = cu_k[b], cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            vis = pins.visible_set_kv(mask, i, lq, lk)
            assert set(range(lo[sq + i] - sk, hi[sq + i] - sk)) == vis


@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_oracle_passes_kv_probe_checks(orc, mask):
    cu_q, cu_k = (np.array(c) for c in KV_CUS[1])
    q, k, v = W.probe_count_inputs(cu_q, 2, 1, 72, cu_k=cu_k)
    out = orc.attention(q, k, v, cu_q, mask, 1 / 72 ** 0.5, cu_seqlens_k=cu_k)
    probes.check_count_output_kv(out, cu_q, cu_k, mask, 72)
    for sign in (1, -1):
        q, k, v = W.probe_index_inputs(cu_q, 4, 2, 64, sign, cu_k=cu_k)
        out = orc.attention(q, k, v, cu_q, mask, 0.125, cu_seqlens_k=cu_k)
        probes.check_index_output_kv(out, cu_q, cu_k, mask, 4, 2, sign)
