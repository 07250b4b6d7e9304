"""Projections on the GPU (include/proj.h) against the fp64 oracle.

Dequantization is compared bit for bit: both sides take the product in
float32 and round it once to bf16 (nearest even).  The GEMM's bound follows
from its arithmetic: inputs exact in bf16, products exact in fp32, sums in
fp32 (error <= K 2^-24 sum_k |x||w|, far below the next term) and the output
rounded once to bf16 (<= 2^-8 |y|: round to nearest keeps 8 significant
bits): |y - y_ref| <= 2^-8 |y_ref| + 2^-20 (|x| |w|^T) elementwise.  Through
dequantization the weights carry their own bf16 rounding (<= 2^-8 |w| each),
so against the exact fp64 weights the bound gains 2^-8 (|x| |w|^T).
"""
import numpy as np
import pytest

from oracle import proj
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


def _weights(n, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.integers(-128, 128, (n, k)).astype(np.int8)
    scale = rng.uniform(0.5, 2.0, n).astype(np.float32) / 127.0
    return q, scale


def _bf16(x):
    return W.round_to(x, W.BF16)


def _dequant_gpu(q, scale):
    import torch

    import long_context_attention_prefill_amd as lcap

    w = lcap.proj_dequantize_int8(torch.from_numpy(q).cuda(), torch.from_numpy(scale).cuda())
    torch.cuda.synchronize()
    return w.double().cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 16), (7, 48), (5, 37), (3, 1), (2560, 2048), (300, 1000)],
                         ids=str)
def test_dequantize_bit_exact(shape):
    q, scale = _weights(*shape, seed=shape[0] + shape[1])
    scale[0] = -scale[0]  # any finite scale
    got = _dequant_gpu(q, scale)
    want = proj.dequantize_bf16(q, scale)
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} weights differ"


def _linear_gpu(x, w):
    import torch

    import long_context_attention_prefill_amd as lcap

    y = lcap.proj_linear(torch.from_numpy(x).to(torch.bfloat16).cuda(),
                         torch.from_numpy(w).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    return y.double().cpu().numpy()


@pytest.mark.parametrize("tnk", [(1, 1, 1), (1, 1, 16), (3, 5, 7), (64, 96, 128), (257, 130, 300),
                                 (2048, 2560, 2048)], ids=str)
def test_linear_within_bound(tnk):
    t, n, k = tnk
    rng = np.random.Generator(np.random.PCG64(t * 7 + n + k))
    x = _bf16(rng.standard_normal((t, k)))
    w = _bf16(rng.standard_normal((n, k)) * 0.05)
    got = _linear_gpu(x, w)
    want = proj.linear(x, w)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -20 * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) - bound))


@pytest.mark.parametrize("tnk", [(10240, 2560, 2048), (10240, 2048, 2048)], ids=str)
def test_int8_projection_full_size(tnk):
    """Dequantize once, then project: the attention workload's QKV and output
    projections at full size, against exact fp64 weights."""
    import torch

    import long_context_attention_prefill_amd as lcap

    t, n, k = tnk
    q, scale = _weights(n, k, seed=n + k)
    rng = np.random.Generator(np.random.PCG64(t + n))
    x = _bf16(rng.standard_normal((t, k)))
    w_dev = lcap.proj_dequantize_int8(torch.from_numpy(q).cuda(), torch.from_numpy(scale).cuda())
    y = lcap.proj_linear(torch.from_numpy(x).to(torch.bfloat16).cuda(), w_dev)
    torch.cuda.synchronize()
    got = y.double().cpu().numpy()
    w_exact = proj.dequantize(q, scale)
    want = proj.linear(x, w_exact)
    mag = np.abs(x) @ np.abs(w_exact).T
    bound = 2.0 ** -8 * np.abs(want) + (2.0 ** -8 + 2.0 ** -20) * mag
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) - bound))


def test_errors_leave_outputs_untouched():
    import torch

    import long_context_attention_prefill_amd as lcap

    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3, 8), dtype=torch.bfloat16, device="cuda")
    lib = lcap.load_library()
    y = torch.full((4, 3), 7.0, dtype=torch.bfloat16, device="cuda")
    assert lib.proj_linear(x.data_ptr(), w.data_ptr(), y.data_ptr(), 4, 3, 0, None) == lcap.ATTN_EINVAL
    assert lib.proj_linear(x.data_ptr(), w.data_ptr(), x.data_ptr(), 4, 3, 8, None) == lcap.ATTN_EINVAL
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
