"""The C ABI without a GPU: the library loads, exports what the header
declares, and its host-side argument checks return the documented codes."""
import ctypes
import os
import re

import pytest

import long_context_attention_prefill_amd as lcap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_prefill.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lcap.library_path()):
        from long_context_attention_prefill_amd import build

        build.build()
    return lcap.load_library()


def header_text():
    return open(HEADER).read()


def test_exports_every_declared_function(lib):
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", header_text(), re.M)
    assert set(names) >= {"attn_prefill", "attn_prefill_check", "attn_strerror", "attn_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_binding_constants_match_header():
    defs = dict(re.findall(r"#define\s+(ATTN_\w+)\s+\(?(-?\d+)\)?", header_text()))
    for name, val in defs.items():
        assert getattr(lcap, name) == int(val), name


def test_version_and_strerror(lib):
    assert lcap.attn_version() >= 10000
    for st in (0, -1, -2, -3, 99):
        assert isinstance(lcap.attn_strerror(st), str) and lcap.attn_strerror(st)
    assert lcap.attn_strerror(-1) != lcap.attn_strerror(-2)


# fake, aligned, non-overlapping "device" addresses: the check never dereferences them
Q, K, V, O = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def check(lib, q=Q, k=K, v=V, o=O, cu=(0, 10, 30), hq=4, hkv=2, d=128, dtype=1, mask=0,
          window=0, scale=0.1, n_seqs=None):
    arr = (ctypes.c_int32 * max(len(cu), 1))(*cu) if cu is not None else None
    if n_seqs is None:
        n_seqs = len(cu) - 1 if cu is not None else 0
    return lib.attn_prefill_check(q, k, v, o, arr, n_seqs, hq, hkv, d, dtype, mask, window,
                                  ctypes.c_float(scale))


def test_check_accepts_valid(lib):
    assert check(lib) == lcap.ATTN_OK
    for d in (64, 72, 128):
        for dtype in (lcap.ATTN_BF16, lcap.ATTN_F32):
            for mask, w in ((0, 0), (1, 0), (2, 1), (2, 256)):
                assert check(lib, d=d, dtype=dtype, mask=mask, window=w) == lcap.ATTN_OK
    assert check(lib, scale=0.0) == lcap.ATTN_OK
    assert check(lib, scale=-1.0) == lcap.ATTN_OK
    # empty batches: no pointer is needed
    assert check(lib, q=0, k=0, v=0, o=0, cu=(0,)) == lcap.ATTN_OK
    assert check(lib, q=0, k=0, v=0, o=0, cu=(0, 0, 0)) == lcap.ATTN_OK
    assert check(lib, q=0, k=0, v=0, o=0, cu=None, n_seqs=0) == lcap.ATTN_OK


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0),
    dict(q=Q + 2), dict(o=O + 8), dict(k=K + 4),
    dict(cu=(1, 10, 30)), dict(cu=(0, 20, 10)), dict(cu=None, n_seqs=2), dict(n_seqs=-1),
    dict(hq=0), dict(hkv=0), dict(hq=4, hkv=3), dict(hq=-4),
    dict(mask=3), dict(mask=-1), dict(mask=2, window=0), dict(mask=2, window=-5),
    dict(scale=float("nan")), dict(scale=float("inf")),
    dict(o=Q), dict(o=Q + 16), dict(o=K - 16), dict(o=V + 32),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_check_rejects_invalid(lib, kw):
    assert check(lib, **kw) == lcap.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(d=0), dict(dtype=0),
                                dict(dtype=3)], ids=str)
def test_check_rejects_unsupported(lib, kw):
    assert check(lib, **kw) == lcap.ATTN_EUNSUPPORTED


def test_prefill_rejects_before_any_device_work(lib):
    """attn_prefill itself returns the check's code without touching a GPU."""
    cu = (ctypes.c_int32 * 2)(0, 8)
    st = lib.attn_prefill(Q, K, V, O, cu, 1, 4, 2, 128, 1, 2, 0, ctypes.c_float(0.1), None)
    assert st == lcap.ATTN_EINVAL
    st = lib.attn_prefill(Q, K, V, O, cu, 1, 4, 2, 80, 1, 0, 0, ctypes.c_float(0.1), None)
    assert st == lcap.ATTN_EUNSUPPORTED
    # T = 0 succeeds with no work
    z = (ctypes.c_int32 * 3)(0, 0, 0)
    assert lib.attn_prefill(0, 0, 0, 0, z, 2, 4, 2, 128, 1, 0, 0, ctypes.c_float(0.1), None) == 0


# ---------------------------------------------------------------- attn_prefill_kv

L = 0x50000000  # fake, aligned lse address


def check_kv(lib, q=Q, k=K, v=V, o=O, lse=L, cu_q=(0, 4, 5), cu_k=(0, 10, 30), hq=4, hkv=2,
             d=128, dtype=1, mask=0, window=0, scale=0.1, n_seqs=None):
    aq = (ctypes.c_int32 * len(cu_q))(*cu_q)
    ak = (ctypes.c_int32 * len(cu_k))(*cu_k)
    if n_seqs is None:
        n_seqs = len(cu_q) - 1
    return lib.attn_prefill_kv_check(q, k, v, o, lse, aq, ak, n_seqs, hq, hkv, d, dtype, mask,
                                     window, ctypes.c_float(scale))


def test_kv_check_accepts_valid(lib):
    assert check_kv(lib) == lcap.ATTN_OK
    assert check_kv(lib, lse=None) == lcap.ATTN_OK
    assert check_kv(lib, cu_q=(0, 10, 30), cu_k=(0, 10, 30)) == lcap.ATTN_OK  # square
    assert check_kv(lib, cu_q=(0, 1, 2), cu_k=(0, 100, 101)) == lcap.ATTN_OK  # decode
    for mask, w in ((0, 0), (1, 0), (2, 7)):
        assert check_kv(lib, mask=mask, window=w) == lcap.ATTN_OK
    # no queries at all: nothing to launch, no pointer needed
    assert check_kv(lib, q=0, o=0, lse=0, cu_q=(0, 0, 0)) == lcap.ATTN_OK


@pytest.mark.parametrize("kw", [
    dict(cu_q=(0, 11, 12)),                  # more queries than keys in sequence 0
    dict(cu_q=(0, 4, 25)),                   # more queries than keys in sequence 1
    dict(cu_k=(1, 10, 30)), dict(cu_q=(1, 4, 5)),
    dict(cu_k=(0, 10, 5)), dict(cu_q=(0, 4, 3)),
    dict(lse=L + 2), dict(lse=Q), dict(lse=O + 64), dict(lse=K + 4096),
    dict(o=K), dict(q=0), dict(k=K + 8),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_kv_check_rejects_invalid(lib, kw):
    assert check_kv(lib, **kw) == lcap.ATTN_EINVAL


def test_kv_rejects_before_any_device_work(lib):
    aq = (ctypes.c_int32 * 2)(0, 9)
    ak = (ctypes.c_int32 * 2)(0, 8)
    st = lib.attn_prefill_kv(Q, K, V, O, L, aq, ak, 1, 4, 2, 128, 1, 0, 0, ctypes.c_float(0.1), None)
    assert st == lcap.ATTN_EINVAL
    z = (ctypes.c_int32 * 2)(0, 0)
    assert lib.attn_prefill_kv(0, K, V, 0, 0, z, ak, 1, 4, 2, 128, 1, 0, 0, ctypes.c_float(0.1),
                               None) == 0


# ---------------------------------------------------------------- attn_decode

def ws_size(lib, cu_k=(0, 10, 3000), hq=16, hkv=2, d=128, dtype=1, mask=0, window=0, n_seqs=None):
    ak = (ctypes.c_int32 * len(cu_k))(*cu_k)
    out = ctypes.c_uint64(0)
    if n_seqs is None:
        n_seqs = len(cu_k) - 1
    st = lib.attn_decode_workspace_size(ak, n_seqs, hq, hkv, d, dtype, mask, window, ctypes.byref(out))
    return st, out.value


def test_decode_workspace_size(lib):
    st, n = ws_size(lib)
    assert st == lcap.ATTN_OK and n > 0
    # one chunk per sequence: written directly, no workspace
    assert ws_size(lib, cu_k=(0, 1, 33, 65)) == (lcap.ATTN_OK, 0)
    # fp32 and head_dim 72 run through the prefill path
    assert ws_size(lib, dtype=2) == (lcap.ATTN_OK, 0)
    assert ws_size(lib, d=72) == (lcap.ATTN_OK, 0)
    # the size grows with the cache
    assert ws_size(lib, cu_k=(0, 100000))[1] >= ws_size(lib, cu_k=(0, 1000))[1]
    for bad in (dict(cu_k=(0, 0, 10)), dict(cu_k=(1, 10)), dict(hq=3, hkv=2), dict(mask=2),
                dict(n_seqs=-1)):
        assert ws_size(lib, **bad)[0] == lcap.ATTN_EINVAL, bad
    assert ws_size(lib, d=96)[0] == lcap.ATTN_EUNSUPPORTED


def test_decode_rejects_before_any_device_work(lib):
    ak = (ctypes.c_int32 * 3)(0, 10, 3000)
    st, need = ws_size(lib)
    W_ = 0x60000000

    def call(ws, nbytes, q=Q, o=O, cu=ak):
        return lib.attn_decode(q, K, V, o, None, cu, 2, 16, 2, 128, 1, 0, 0, ctypes.c_float(0.1),
                               ws, nbytes, None)
    assert call(None, 0) == lcap.ATTN_EINVAL            # workspace needed
    assert call(W_, need - 16) == lcap.ATTN_EINVAL      # too small
    assert call(W_ + 8, need) == lcap.ATTN_EINVAL       # misaligned
    assert call(K, need) == lcap.ATTN_EINVAL            # overlaps k
    empty = (ctypes.c_int32 * 3)(0, 10, 10)
    assert call(W_, need, cu=empty) == lcap.ATTN_EINVAL  # a sequence without keys
    assert lib.attn_decode(0, 0, 0, 0, None, None, 0, 16, 2, 128, 1, 0, 0, ctypes.c_float(0.1),
                           None, 0, None) == 0


def test_decode_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """A decode whose workspace exceeds the static scratch is refused before any
    device work (host-only check; the fake pointers are never touched)."""
    cu = [0]
    for _ in range(64):
        cu.append(cu[-1] + 100000)
    need = lcap.attn_decode_workspace_size(cu, 64, 2, 128, lcap.ATTN_BF16, "causal")
    assert need > lcap.ATTN_DECODE_SCRATCH_BYTES
    arr = (ctypes.c_int32 * len(cu))(*cu)
    # the caches span 3.3 GB each: fake addresses far enough apart not to overlap
    kk, vv = 0x1000000000, 0x2000000000
    st = lib.attn_decode_noalloc(Q, kk, vv, O, None, arr, 64, 64, 2, 128, 1, 0, 0,
                                 ctypes.c_float(0.1), None)
    assert st == lcap.ATTN_EUNSUPPORTED
    # argument errors come first, as for attn_decode
    st = lib.attn_decode_noalloc(None, kk, vv, O, None, arr, 64, 64, 2, 128, 1, 0, 0,
                                 ctypes.c_float(0.1), None)
    assert st == lcap.ATTN_EINVAL
