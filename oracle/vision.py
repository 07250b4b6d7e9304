"""fp64 CPU oracle for the vision attention block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product path never uses it.

What it computes.  The paper "A Modern Multimodal Assistant on a 6 GB 2011
GPU" runs a SigLIP2 vision tower (FP32 weights) whose bidirectional
attention it rewrote with the language model's GEMM method, cutting image
encoding 6x (abstract, result (iii); gist.science technical summary,
Metodologia: FP32 vision weights, stage-by-stage port of the encoder
layers).  The pages give no layer formula; the reading used here is the
standard attention half of a transformer encoder layer:

    [q | k | v] = x W_qkv^T + b_qkv      (each block heads-contiguous: [T][H][d])
    a = softmax(scale q k^T) v             per head, per image, under the mask
    out = a W_o^T + b_o                    (a laid out [T][H d])

in fp64 throughout: the projections are numpy products, the attention is the
fp64 attention oracle of this package (oracle/attn_oracle.c), called with the
image packing and the mask.
"""
from __future__ import annotations

import numpy as np


def attention_block(orc, x, w_qkv, b_qkv, w_o, b_o, cu_seqlens, n_heads, mask="full", scale=None):
    """out [T, hidden] in fp64; ``orc`` is the attention oracle (``oracle.load()``)."""
    x = np.asarray(x, dtype=np.float64)
    w_qkv = np.asarray(w_qkv, dtype=np.float64)
    b_qkv = np.asarray(b_qkv, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    b_o = np.asarray(b_o, dtype=np.float64)
    T, hidden = x.shape
    H = int(n_heads)
    hd = w_qkv.shape[0] // 3
    d = hd // H
    if w_qkv.shape != (3 * H * d, hidden) or b_qkv.shape != (3 * H * d,) or \
            w_o.shape != (hidden, H * d) or b_o.shape != (hidden,):
        raise ValueError("weight shapes disagree with x and n_heads")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    # the QKV projection, then its three column blocks, each [T][H][d]
    qkv = x @ w_qkv.T + b_qkv
    q = qkv[:, 0 * hd:1 * hd].reshape(T, H, d)
    k = qkv[:, 1 * hd:2 * hd].reshape(T, H, d)
    v = qkv[:, 2 * hd:3 * hd].reshape(T, H, d)
    a = orc.attention(q, k, v, cu_seqlens, mask, scale)
    # heads side by side again, then the output projection
    return a.reshape(T, H * d) @ w_o.T + b_o
