"""fp64 CPU oracle for exact attention prefill -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with them.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, OpenMP over rows);
this module compiles it with gcc and marshals numpy arrays to it.  See the C
file's header for what is computed and which passage of the pages each part
follows (paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU": abstract,
result (iii); gist.science technical summary, Metodologia, attention rewrite).

Mask specifications accepted here: ``"causal"``, ``"full"`` or
``("window", W)`` with W > 0.

``cu_seqlens_k`` (optional, on ``attention`` and ``attention_rows``): the
keys/values have their own packing, sequence b holding Lk_b >= Lq_b tokens,
and its Lq_b queries are the last Lq_b positions of the sequence (query i at
position i + Lk_b - Lq_b).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "libattn_oracle.so")

_MASK_CODES = {"causal": 0, "full": 1, "window": 2}


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle (or a variant of its source) into a shared object."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    i32 = ctypes.c_int32
    lib.oracle_attention.argtypes = [dp, dp, dp, ip, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_double, dp, dp]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [dp, dp, dp, ip, i32, i32, i32, i32, i32, i32,
                                          ctypes.c_double, lp, ip, ctypes.c_int64, dp, dp]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_probs.argtypes = [dp, dp, dp, ip, i32, i32, i32, i32, i32, i32,
                                           ctypes.c_double, ctypes.c_int64, i32, dp]
    lib.oracle_attention_probs.restype = ctypes.c_int64
    lib.oracle_attention_kv.argtypes = [dp, dp, dp, ip, ip, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_double, dp, dp]
    lib.oracle_attention_kv.restype = ctypes.c_int
    lib.oracle_attention_kv_rows.argtypes = [dp, dp, dp, ip, ip, i32, i32, i32, i32, i32, i32,
                                             ctypes.c_double, lp, ip, ctypes.c_int64, dp, dp]
    lib.oracle_attention_kv_rows.restype = ctypes.c_int
    return lib


_LIB = None


def load(path: str | None = None) -> "Oracle":
    """An Oracle bound to ``path`` (default: the library $ATTN_ORACLE_LIBRARY names,
    else the committed source, built on demand)."""
    global _LIB
    if path is not None:
        return Oracle(_bind(path))
    if _LIB is None:
        override = os.environ.get("ATTN_ORACLE_LIBRARY")  # a prebuilt variant (e.g. sanitizer build)
        if override:
            _LIB = _bind(override)
        else:
            if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                build()
            _LIB = _bind(LIBRARY)
    return Oracle(_LIB)


def _mask(mask) -> tuple[int, int]:
    if isinstance(mask, str):
        if mask not in ("causal", "full"):
            raise ValueError(f"unknown mask {mask!r}")
        return _MASK_CODES[mask], 0
    kind, w = mask
    if kind != "window" or int(w) <= 0:
        raise ValueError(f"bad mask {mask!r}")
    return _MASK_CODES["window"], int(w)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    def __init__(self, lib: ctypes.CDLL):
        self._lib = lib

    @staticmethod
    def _prep(q, k, v, cu_seqlens, cu_seqlens_k=None):
        q, k, v = _f64(q), _f64(k), _f64(v)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        cu_k = cu if cu_seqlens_k is None else np.ascontiguousarray(
            np.asarray(cu_seqlens_k, dtype=np.int32))
        if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape:
            raise ValueError("q must be [Tq,Hq,d]; k and v [Tk,Hkv,d]")
        T, hq, d = q.shape
        if k.shape[2] != d:
            raise ValueError("q, k, v disagree on d")
        if cu.ndim != 1 or cu.size < 1 or int(cu[-1]) != T:
            raise ValueError("cu_seqlens must end at Tq")
        if cu_k.shape != cu.shape or int(cu_k[-1]) != k.shape[0]:
            raise ValueError("cu_seqlens_k must have n_seqs+1 entries and end at Tk")
        return q, k, v, cu, cu_k, T, hq, k.shape[1], d

    def attention(self, q, k, v, cu_seqlens, mask, scale, return_lse=False, cu_seqlens_k=None):
        """Every output row, fp64 [Tq, Hq, d] (and the log-sum-exp [Tq, Hq])."""
        q, k, v, cu, cu_k, T, hq, hkv, d = self._prep(q, k, v, cu_seqlens, cu_seqlens_k)
        code, w = _mask(mask)
        out = np.zeros((T, hq, d), dtype=np.float64)
        lse = np.zeros((T, hq), dtype=np.float64)
        rc = self._lib.oracle_attention_kv(
            _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
            _ptr(cu, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32), cu.size - 1, hq, hkv, d,
            code, w, float(scale), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return (out, lse) if return_lse else out

    def attention_rows(self, q, k, v, cu_seqlens, mask, scale, rows, heads, return_lse=False,
                       cu_seqlens_k=None):
        """Selected rows: out[r] is packed query token rows[r], query head heads[r]."""
        q, k, v, cu, cu_k, T, hq, hkv, d = self._prep(q, k, v, cu_seqlens, cu_seqlens_k)
        code, w = _mask(mask)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        heads = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        if rows.shape != heads.shape or rows.ndim != 1:
            raise ValueError("rows and heads must be 1-D and equal in length")
        out = np.zeros((rows.size, d), dtype=np.float64)
        lse = np.zeros(rows.size, dtype=np.float64)
        rc = self._lib.oracle_attention_kv_rows(
            _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
            _ptr(cu, ctypes.c_int32), _ptr(cu_k, ctypes.c_int32), cu.size - 1, hq, hkv, d,
            code, w, float(scale), _ptr(rows, ctypes.c_int64), _ptr(heads, ctypes.c_int32),
            rows.size, _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return (out, lse) if return_lse else out

    def probs(self, q, k, v, cu_seqlens, mask, scale, t, h):
        """Softmax weights of row (t, h) over its sequence's keys (0 where invisible)."""
        q, k, v, cu, _, T, hq, hkv, d = self._prep(q, k, v, cu_seqlens)
        code, w = _mask(mask)
        b = int(np.searchsorted(cu, t, side="right") - 1)
        while b + 1 < cu.size and cu[b + 1] <= t:
            b += 1
        n = int(cu[b + 1] - cu[b])
        p = np.zeros(n, dtype=np.float64)
        cnt = self._lib.oracle_attention_probs(
            _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
            _ptr(cu, ctypes.c_int32), cu.size - 1, hq, hkv, d, code, w, float(scale),
            int(t), int(h), _ptr(p, ctypes.c_double))
        if cnt < 0:
            raise ValueError("oracle rejected its arguments")
        return p
