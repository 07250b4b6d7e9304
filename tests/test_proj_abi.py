"""The projection C ABI without a GPU: exports and host-side argument checks."""
import os
import re

import pytest

import long_context_attention_prefill_amd as lcap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "proj.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lcap.library_path()):
        from long_context_attention_prefill_amd import build

        build.build()
    return lcap.load_library()


def test_exports_every_declared_function(lib):
    names = re.findall(r"^\s*\w+\s*\*?\s*(proj_\w+)\s*\(", open(HEADER).read(), re.M)
    assert set(names) == {"proj_dequantize_int8", "proj_linear"}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


Q, S, Wt, X, Y = (0x10000000 * i for i in range(1, 6))


@pytest.mark.parametrize("args", [
    (None, S, Wt, 4, 16), (Q, None, Wt, 4, 16), (Q, S, None, 4, 16),
    (Q + 8, S, Wt, 4, 16), (Q, S + 2, Wt, 4, 16), (Q, S, Wt + 8, 4, 16),
    (Q, S, Q, 4, 16), (Q, S, S - 16, 4, 16), (Q, S, Wt, -1, 16), (Q, S, Wt, 4, -1),
], ids=str)
def test_dequantize_rejects(lib, args):
    assert lib.proj_dequantize_int8(*args, None) == lcap.ATTN_EINVAL


def test_dequantize_empty_is_a_no_op(lib):
    assert lib.proj_dequantize_int8(None, None, None, 0, 16, None) == lcap.ATTN_OK
    assert lib.proj_dequantize_int8(None, None, None, 5, 0, None) == lcap.ATTN_OK


@pytest.mark.parametrize("args,code", [
    ((None, Wt, Y, 4, 3, 8), lcap.ATTN_EINVAL), ((X, None, Y, 4, 3, 8), lcap.ATTN_EINVAL),
    ((X, Wt, None, 4, 3, 8), lcap.ATTN_EINVAL), ((X + 2, Wt, Y, 4, 3, 8), lcap.ATTN_EINVAL),
    ((X, Wt, Y + 8, 4, 3, 8), lcap.ATTN_EINVAL), ((X, Wt, X, 4, 3, 8), lcap.ATTN_EINVAL),
    ((X, Wt, Wt + 16, 4, 3, 8), lcap.ATTN_EINVAL), ((X, Wt, Y, -1, 3, 8), lcap.ATTN_EINVAL),
    ((X, Wt, Y, 4, 3, 0), lcap.ATTN_EINVAL), ((X, Wt, Y, 1 << 31, 3, 8), lcap.ATTN_EUNSUPPORTED),
    ((None, None, None, 0, 3, 8), lcap.ATTN_OK), ((None, None, None, 4, 0, 8), lcap.ATTN_OK),
], ids=str)
def test_linear_checks(lib, args, code):
    assert lib.proj_linear(*args, None) == code
