"""fp64 CPU oracle for the projections -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product path never uses it.

What it computes (paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU":
8-bit language weights dequantized once before the vendor GEMM -- abstract,
result (i); gist.science technical summary, Metodologia, GEMM efficiency).
The pages give no quantization format; the reading used here is symmetric
int8 with one float scale per output row, w[n][k] = scale[n] * q[n][k], and
the projection y = x w^T (y[t][n] = sum_k x[t][k] w[n][k]).
"""
from __future__ import annotations

import numpy as np


def dequantize(q, scale):
    """w[n][k] = scale[n] * q[n][k], fp64 (exact: an int8 times a float32)."""
    q = np.asarray(q)
    scale = np.asarray(scale, dtype=np.float64)
    if q.ndim != 2 or scale.shape != (q.shape[0],):
        raise ValueError("q must be [N, K] and scale [N]")
    return q.astype(np.float64) * scale[:, None]


def dequantize_bf16(q, scale):
    """The dequantized weights as the bf16 values the kernel stores: the
    product taken in float32 (as the kernel takes it) and rounded once to
    bf16, nearest even -- both sides make that rounding decision in the same
    precision.  Returned as float64."""
    q = np.asarray(q)
    s32 = np.asarray(scale, dtype=np.float32)
    prod = (q.astype(np.float32) * s32[:, None]).astype(np.float64)
    m, e = np.frexp(prod)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def linear(x, w):
    """y = x w^T in fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T, K] and w [N, K]")
    return x @ w.T
