"""One sequence of 32767 tokens, three times the longest full-size workload:
the index probe's 15-bit key code reaches exactly this far (and the last
query tile is ragged).

Against the oracle on sampled rows (first, last, middle and random rows of
every head, max abs 2e-2 bf16), and bit-exact at every row by the index probe
(bf16) and the count probe (expected integers from the mask definitions).  A
bf16 count-probe output carries a relative rounding of up to 2^-9, which
resolves per-class counts below 256 only; a causal row here counts up to 256
keys per class, so that case runs the count probe on the fp32 kernel (exact
to 2^-24), the window case (at most 64 per class) on bf16.  The causal case
at 8/1 heads is 2048 items, so it runs with work tickets.
"""
import numpy as np
import pytest

import gpu_util as G
import probes
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

N = 32767
CASES = {
    "causal-8x1-d128": ([0, N], 8, 1, 128, "causal"),
    "window4096-4x2-d64": ([0, N], 4, 2, 64, ("window", 4096)),
}
COUNT_DTYPE = {"causal-8x1-d128": "f32", "window4096-4x2-d64": "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


def _rows(n, hq, rng):
    pick = {0, 1, 127, 128, n // 2, n - 129, n - 2, n - 1} | set(rng.integers(0, n, 24).tolist())
    rows = np.array(sorted(pick))
    return np.repeat(rows, hq), np.tile(np.arange(hq), rows.size)


@pytest.mark.parametrize("case", sorted(CASES))
def test_long_sequence_parity(orc, case):
    cu, hq, hkv, d, mask = CASES[case]
    cu = np.array(cu)
    q, k, v = W.draw_qkv(cu, hq, hkv, d, "bf16", 0.5, seed=len(case) * 11)
    scale = 1.0 / np.sqrt(d)
    print(f"[long] {case}", flush=True)
    got = G.run_hip(q, k, v, cu, mask, scale, "bf16")
    rows, heads = _rows(N, hq, np.random.Generator(np.random.PCG64(3)))
    want = orc.attention_rows(q, k, v, cu, mask, scale, rows, heads)
    assert G.max_err(got[rows, heads], want) <= G.TOL["bf16"], case


@pytest.mark.parametrize("case", sorted(CASES))
def test_long_sequence_probe_count(case):
    cu, hq, hkv, d, mask = CASES[case]
    cu = np.array(cu)
    q, k, v = W.probe_count_inputs(cu, hq, hkv, d)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / np.sqrt(d), COUNT_DTYPE[case])
    probes.check_count_output(got, cu, mask, d)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("case", sorted(CASES))
def test_long_sequence_probe_index(case, sign):
    cu, hq, hkv, d, mask = CASES[case]
    cu = np.array(cu)
    q, k, v = W.probe_index_inputs(cu, hq, hkv, d, sign)
    got = G.run_hip(q, k, v, cu, mask, 1.0 / np.sqrt(d), "bf16")
    probes.check_index_output(got, cu, mask, hq, hkv, sign)
