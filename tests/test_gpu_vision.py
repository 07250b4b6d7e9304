"""vision_attention_block (QKV GEMM with the bias in its epilogue, the HIP
attention kernels reading q, k, v in place from the QKV rows, output GEMM
with its bias) against the fp64 oracle, through the C ABI, on the same seeded
inputs.

Tolerance.  bf16: the block rounds q, k and v once each to bf16, the
attention rounds its probabilities and its output to bf16, and the result is
rounded once more (each within 2^-8 relative: round to nearest keeps 8
significant bits); the GEMMs and the softmax sum in fp32.  A numpy replay of
exactly those roundings on these input distributions (SigLIP2's shape, images
of 77-1024 patches, full and window masks) stays within 0.65 % of max |out|
(max abs error) and 0.53 % of rms(out) (rms error); the bars are 2^-5 of
max |out_ref| and 2^-6 of rms(out_ref), a factor 3 to 5 over that.  A dropped
bias moves outputs by about 20 % of rms(out), swapped q and k blocks or a
wrong head layout by far more.  fp32: every product is exact and every sum
of at most 1152 terms is within n 2^-24 relative in the worst case (7e-5),
typically within 1e-6; the bars are 1e-4 of max |out_ref| and 1e-5 of
rms(out_ref).
"""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

BARS = {"bf16": (2.0 ** -5, 2.0 ** -6), "f32": (1e-4, 1e-5)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


@pytest.fixture(scope="module")
def orc():
    import oracle

    return oracle.load()


def _run(inputs, lens, H, dtype, mask, scale=None, workspace=None):
    import torch

    import long_context_attention_prefill_amd as lcap

    dev = [G.to_device(a, dtype) for a in inputs]
    cu = [0] + np.cumsum(lens).tolist()
    out = lcap.vision_attention_block(*dev, cu, H, mask=mask, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


def _assert_close(got, want, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if want.size == 0:
        return
    max_rel, rms_rel = BARS[dtype]
    err = np.abs(got - want)
    mx = float(np.max(np.abs(want)))
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert float(err.max()) <= max_rel * mx, f"{what}: max err {err.max():.3e} vs max|ref| {mx:.3e}"
    assert float(np.sqrt(np.mean(err ** 2))) <= rms_rel * rms, \
        f"{what}: rms err {np.sqrt(np.mean(err ** 2)):.3e} vs rms(ref) {rms:.3e}"


def _check(orc, lens, hidden, H, d, dtype, mask, seed, scale=None):
    from oracle import vision

    inputs = W.make_vision_inputs(lens, hidden, H, d, dtype, seed)
    cu = [0] + np.cumsum(lens).tolist()
    got = _run(inputs, lens, H, dtype, mask, scale)
    want = vision.attention_block(orc, *inputs, cu, H, mask, scale)
    _assert_close(got, want, dtype, f"lens {lens} d {d} {dtype} {mask}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 72, 128])
@pytest.mark.parametrize("mask", ["full", ("window", 16), "causal"], ids=str)
def test_vision_small(orc, dtype, d, mask):
    _check(orc, [130, 64, 1, 77], 256, 2, d, dtype, mask, seed=d + len(str(mask)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lens", [[1], [63], [300]], ids=str)
def test_vision_lengths(orc, dtype, lens):
    _check(orc, lens, 128, 4, 72, dtype, "full", seed=sum(lens))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vision_siglip_shape_window(orc, dtype):
    """SigLIP2's width with window blocks of 64 patches over two images."""
    _check(orc, [768, 300], 1152, 16, 72, dtype, ("window", 64), seed=33)


@pytest.mark.parametrize("scale", [0.25, 0.02])
def test_vision_scales(orc, scale):
    """Twice the default scale (1/8 at d = 64) and a small one.  q and k are
    rounded to bf16 before their product, so the logit error grows with the
    logits: at 8 times the default (logits of std about 18 here) the rounding
    replay alone reaches 3.2 % of max |out|, past the bar, and the kernel
    matched that replay to every printed digit.  At twice the default the
    replay gives 1.0 % and 0.6 %."""
    _check(orc, [200], 128, 2, 64, "bf16", "full", seed=34, scale=scale)


def test_vision_workspace_reuse_and_determinism(orc):
    """One workspace for a large call, a smaller one, then the large one again
    (bit-identical to the first)."""
    import torch

    import long_context_attention_prefill_amd as lcap
    from oracle import vision

    need = lcap.vision_attention_block_workspace_size(900, 4, 72, 256, lcap.ATTN_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    first = None
    for lens, seed in (([900], 35), ([100, 20], 36), ([900], 35)):
        inputs = W.make_vision_inputs(lens, 256, 4, 72, "bf16", seed)
        got = _run(inputs, lens, 4, "bf16", "full", workspace=ws)
        want = vision.attention_block(orc, *inputs, [0] + np.cumsum(lens).tolist(), 4, "full")
        _assert_close(got, want, "bf16", f"lens {lens}")
        if lens == [900]:
            if first is None:
                first = got
            else:
                assert np.array_equal(got, first), "repeated call differs"


def test_vision_empty_batch():
    import torch

    import long_context_attention_prefill_amd as lcap

    inputs = W.make_vision_inputs([0], 128, 2, 64, "bf16", 37)
    dev = [G.to_device(a, "bf16") for a in inputs]
    out = lcap.vision_attention_block(*dev, [0, 0], 2)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 128)


@pytest.mark.parametrize("name", sorted(W.VISION_WORKLOADS))
def test_vision_workloads_full_size(orc, name):
    """The bench workloads at full size, every output."""
    spec = W.VISION_WORKLOADS[name]
    _check(orc, spec["lens"], spec["hidden"], spec["n_heads"], spec["d"], spec["dtype"], "full",
           seed=spec["seed"])
