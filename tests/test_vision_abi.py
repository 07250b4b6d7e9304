"""The vision block's C ABI without a GPU: exports, workspace sizes and the
host-side argument checks (every call here is rejected before device work)."""
import ctypes
import math
import os
import re

import pytest

import long_context_attention_prefill_amd as lcap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vision_block.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lcap.library_path()):
        from long_context_attention_prefill_amd import build

        build.build()
    return lcap.load_library()


def test_exports_every_declared_function(lib):
    names = re.findall(r"^\s*\w+\s*\*?\s*(vision_\w+)\s*\(", open(HEADER).read(), re.M)
    assert set(names) == {"vision_attention_block", "vision_attention_block_workspace_size"}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def _r256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("T,H,d,hidden,dtype,es", [
    (3840, 16, 72, 1152, lcap.ATTN_BF16, 2), (3840, 16, 72, 1152, lcap.ATTN_F32, 4),
    (5, 2, 64, 1024, lcap.ATTN_BF16, 2), (1, 1, 128, 8, lcap.ATTN_F32, 4),
])
def test_workspace_size(T, H, d, hidden, dtype, es):
    want = _r256(T * 3 * H * d * es) + _r256(T * H * d * es)
    assert lcap.vision_attention_block_workspace_size(T, H, d, hidden, dtype) == want
    assert lcap.vision_attention_block_workspace_size(0, H, d, hidden, dtype) == 0


@pytest.mark.parametrize("args,code", [
    ((-1, 16, 72, 1152, lcap.ATTN_BF16), lcap.ATTN_EINVAL),
    ((8, 0, 72, 1152, lcap.ATTN_BF16), lcap.ATTN_EINVAL),
    ((8, 16, 72, 1150, lcap.ATTN_BF16), lcap.ATTN_EINVAL),
    ((8, 16, 96, 1152, lcap.ATTN_BF16), lcap.ATTN_EUNSUPPORTED),
    ((8, 16, 72, 1152, 3), lcap.ATTN_EUNSUPPORTED),
    ((1 << 31, 16, 72, 1152, lcap.ATTN_BF16), lcap.ATTN_EUNSUPPORTED),
], ids=str)
def test_workspace_size_rejects(lib, args, code):
    out = ctypes.c_uint64(0)
    assert lib.vision_attention_block_workspace_size(*args, ctypes.byref(out)) == code


X, WQ, BQ, WO, BO, OUT, WS = (0x10000000 * i for i in range(1, 8))
T, H, D, HID = 8, 2, 64, 128
NEED = _r256(T * 3 * H * D * 2) + _r256(T * H * D * 2)
BASE = dict(x=X, wq=WQ, bq=BQ, wo=WO, bo=BO, out=OUT, cu=[0, 3, 8], h=H, d=D, hidden=HID,
            dtype=lcap.ATTN_BF16, mask=lcap.ATTN_FULL, window=0, scale=0.125, ws=WS, ws_bytes=NEED)


def _call(lib, **kw):
    a = dict(BASE, **kw)
    cu = (ctypes.c_int32 * len(a["cu"]))(*a["cu"])
    return lib.vision_attention_block(a["x"], a["wq"], a["bq"], a["wo"], a["bo"], a["out"], cu,
                                      len(a["cu"]) - 1, a["h"], a["d"], a["hidden"], a["dtype"],
                                      a["mask"], a["window"], a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), lcap.ATTN_EINVAL), (dict(wq=None), lcap.ATTN_EINVAL),
    (dict(bq=None), lcap.ATTN_EINVAL), (dict(wo=None), lcap.ATTN_EINVAL),
    (dict(bo=None), lcap.ATTN_EINVAL), (dict(out=None), lcap.ATTN_EINVAL),
    (dict(x=X + 8), lcap.ATTN_EINVAL), (dict(bo=BO + 4), lcap.ATTN_EINVAL),
    (dict(out=X), lcap.ATTN_EINVAL), (dict(out=WO + 64), lcap.ATTN_EINVAL),
    (dict(ws=None), lcap.ATTN_EINVAL), (dict(ws=WS + 8), lcap.ATTN_EINVAL),
    (dict(ws_bytes=NEED - 1), lcap.ATTN_EINVAL), (dict(ws=BQ - 256), lcap.ATTN_EINVAL),
    (dict(ws=OUT - 1024), lcap.ATTN_EINVAL),
    (dict(hidden=100), lcap.ATTN_EINVAL), (dict(h=0), lcap.ATTN_EINVAL),
    (dict(cu=[1, 8]), lcap.ATTN_EINVAL), (dict(cu=[0, 5, 3]), lcap.ATTN_EINVAL),
    (dict(mask=7), lcap.ATTN_EINVAL), (dict(mask=lcap.ATTN_WINDOW, window=0), lcap.ATTN_EINVAL),
    (dict(scale=math.nan), lcap.ATTN_EINVAL), (dict(scale=math.inf), lcap.ATTN_EINVAL),
    (dict(d=96), lcap.ATTN_EUNSUPPORTED), (dict(dtype=3), lcap.ATTN_EUNSUPPORTED),
], ids=str)
def test_block_rejects_before_any_device_work(lib, kw, code):
    assert _call(lib, **kw) == code


def test_block_without_tokens(lib):
    """No tokens: nothing to do, but the mask and scale are still checked."""
    none = dict(x=None, wq=None, bq=None, wo=None, bo=None, out=None, ws=None, ws_bytes=0)
    assert _call(lib, cu=[0, 0, 0], **none) == lcap.ATTN_OK
    assert _call(lib, cu=[0], **none) == lcap.ATTN_OK
    assert _call(lib, cu=[0, 0], mask=9, **none) == lcap.ATTN_EINVAL
    assert _call(lib, cu=[0, 0], scale=math.nan, **none) == lcap.ATTN_EINVAL
