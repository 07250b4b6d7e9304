"""The gated-delta-rule C ABI without a GPU: exports, workspace sizes and the
host-side argument checks (include/gdn_prefill.h)."""
import ctypes
import os
import re

import pytest

import long_context_attention_prefill_amd as lcap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_prefill.h")

ITEM_BYTES = 73984  # per 64-token chunk and head, as the header states


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lcap.library_path()):
        from long_context_attention_prefill_amd import build

        build.build()
    return lcap.load_library()


def test_exports_every_declared_function(lib):
    names = re.findall(r"^\s*\w+\s*\*?\s*(gdn_\w+)\s*\(", open(HEADER).read(), re.M)
    assert set(names) == {"gdn_prefill", "gdn_prefill_workspace_size", "gdn_prefill_check"}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def ws(lib, cu, h=16, dk=128, dv=128, dtype=1, n=None):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    out = ctypes.c_uint64(0)
    st = lib.gdn_prefill_workspace_size(arr, len(cu) - 1 if n is None else n, h, dk, dv, dtype,
                                        ctypes.byref(out))
    return st, out.value


def test_workspace_size(lib):
    assert ws(lib, [0, 10240]) == (0, 160 * 16 * ITEM_BYTES)
    assert ws(lib, [0, 1, 65, 65]) == (0, (1 + 1) * 16 * ITEM_BYTES)
    assert ws(lib, [0, 0]) == (0, 0)
    # 70 sequences of 64 tokens: launches of 64 and 6 sequences; sized for the larger
    cu = [64 * i for i in range(71)]
    assert ws(lib, cu, h=2) == (0, 64 * 2 * ITEM_BYTES)
    assert ws(lib, [0, 10], dk=64)[0] == lcap.ATTN_EUNSUPPORTED
    assert ws(lib, [0, 10], dtype=2)[0] == lcap.ATTN_EUNSUPPORTED
    assert ws(lib, [1, 10])[0] == lcap.ATTN_EINVAL
    assert ws(lib, [0, 10, 5])[0] == lcap.ATTN_EINVAL
    assert ws(lib, [0, 10], h=0)[0] == lcap.ATTN_EINVAL


# fake, aligned, disjoint device addresses: the checks never dereference them
Q, K, V, G, B, S0, O, S1, WS = (0x10000000 * i for i in range(1, 10))


def check(lib, q=Q, k=K, v=V, g=G, b=B, s0=S0, o=O, s1=S1, cu=(0, 100, 300), h=4, dk=128,
          dv=128, dtype=1, scale=0.1, w=WS, wbytes=None):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    if wbytes is None:
        wbytes = ws(lib, list(cu), h=h)[1]
    return lib.gdn_prefill_check(q, k, v, g, b, s0, o, s1, arr, len(cu) - 1, h, dk, dv, dtype,
                                 ctypes.c_float(scale), w, wbytes)


def test_check_accepts_valid(lib):
    assert check(lib) == lcap.ATTN_OK
    assert check(lib, s0=None, s1=None) == lcap.ATTN_OK
    assert check(lib, s1=S0) == lcap.ATTN_OK  # final state written over the initial one
    assert check(lib, q=None, k=None, v=None, g=None, b=None, o=None, cu=(0, 0), w=None) == 0


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k=None), dict(v=None), dict(g=None), dict(b=None), dict(o=None),
    dict(q=Q + 8), dict(o=O + 2), dict(g=G + 2), dict(s0=S0 + 4), dict(s1=S1 + 8),
    dict(o=Q), dict(o=V + 16), dict(s1=K), dict(o=S0), dict(s1=S0 + 16),
    dict(w=None), dict(w=WS + 8), dict(w=Q), dict(wbytes=16),
    dict(cu=(1, 100)), dict(cu=(0, 100, 50)), dict(h=0),
    dict(scale=float("nan")), dict(scale=float("inf")),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_check_rejects_invalid(lib, kw):
    assert check(lib, **kw) == lcap.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(dk=64), dict(dv=64), dict(dtype=2), dict(dtype=0)], ids=str)
def test_check_rejects_unsupported(lib, kw):
    assert check(lib, **kw) == lcap.ATTN_EUNSUPPORTED


def test_prefill_rejects_before_any_device_work(lib):
    cu = (ctypes.c_int32 * 2)(0, 100)
    st = lib.gdn_prefill(Q, K, V, G, B, None, O, None, cu, 1, 4, 128, 128, 1, ctypes.c_float(0.1),
                         None, 0, None)
    assert st == lcap.ATTN_EINVAL  # workspace missing
    z = (ctypes.c_int32 * 2)(0, 0)
    assert lib.gdn_prefill(None, None, None, None, None, None, None, None, z, 1, 4, 128, 128, 1,
                           ctypes.c_float(0.1), None, 0, None) == 0
