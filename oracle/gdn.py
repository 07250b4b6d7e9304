"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path never imports, links or
calls it, and it shares no code with it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, the token-by-token
scan of the recurrence; OpenMP over (sequence, head) pairs); this module
compiles it with gcc and marshals numpy arrays.  See the C file's header for
the recurrence and where the pages name it (paper "A Modern Multimodal
Assistant on a 6 GB 2011 GPU": abstract, result (i); gist.science technical
summary, Metodologia, recurrent layers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "libgdn_oracle.so")


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle (or a variant of its source) into a shared object."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i32 = ctypes.c_int32
    lib.oracle_gated_delta_rule.argtypes = [dp, dp, dp, dp, dp, dp, ip, i32, i32, i32, i32,
                                            ctypes.c_double, dp, dp]
    lib.oracle_gated_delta_rule.restype = ctypes.c_int
    return lib


_LIB = None


def load(path: str | None = None) -> "GdnOracle":
    """A GdnOracle bound to ``path`` (default: the library $GDN_ORACLE_LIBRARY names,
    else the committed source, built on demand)."""
    global _LIB
    if path is not None:
        return GdnOracle(_bind(path))
    if _LIB is None:
        override = os.environ.get("GDN_ORACLE_LIBRARY")  # a prebuilt variant (e.g. sanitizer build)
        if override:
            _LIB = _bind(override)
        else:
            if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                build()
            _LIB = _bind(LIBRARY)
    return GdnOracle(_LIB)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class GdnOracle:
    def __init__(self, lib: ctypes.CDLL):
        self._lib = lib

    def gated_delta_rule(self, q, k, v, g, beta, cu_seqlens, scale, initial_state=None):
        """Outputs [T, H, dv] and final states [n_seqs, H, dv, dk], fp64.

        q, k: [T, H, dk]; v: [T, H, dv]; g (log of the per-token decay) and
        beta: [T, H]; initial_state: None (zeros) or [n_seqs, H, dv, dk].
        """
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        if q.ndim != 3 or k.shape != q.shape or v.ndim != 3 or v.shape[:2] != q.shape[:2]:
            raise ValueError("q, k must be [T, H, dk] and v [T, H, dv]")
        T, H, dk = q.shape
        dv = v.shape[2]
        if g.shape != (T, H) or beta.shape != (T, H):
            raise ValueError("g and beta must be [T, H]")
        if cu.ndim != 1 or cu.size < 1 or int(cu[-1]) != T:
            raise ValueError("cu_seqlens must end at T")
        n = cu.size - 1
        s0 = None
        if initial_state is not None:
            s0 = _f64(initial_state)
            if s0.shape != (n, H, dv, dk):
                raise ValueError("initial_state must be [n_seqs, H, dv, dk]")
        out = np.zeros((T, H, dv), dtype=np.float64)
        fin = np.zeros((n, H, dv, dk), dtype=np.float64)
        rc = self._lib.oracle_gated_delta_rule(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            None if s0 is None else _ptr(s0), _ptr(cu, ctypes.c_int32), n, H, dk, dv,
            float(scale), _ptr(out), _ptr(fin))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out, fin
