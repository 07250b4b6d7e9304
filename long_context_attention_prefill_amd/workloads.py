"""Seeded synthetic inputs for attention prefill.

This module only draws and lays out inputs; it holds none of attention's
arithmetic, so the fp64 oracle and the HIP library can both be fed from it
without sharing any of the computation.  Arrays are numpy float64 holding
values already rounded to the target dtype (bf16 by round-to-nearest-even,
or fp32), laid out packed as q[T, Hq, d], k/v[T, Hkv, d] with cu_seqlens
int32[n_seqs + 1].

The workloads stand in for the paper's own (paper "A Modern Multimodal
Assistant on a 6 GB 2011 GPU", abstract result (iii): causal language-model
prefill at 2k and 10k tokens, a needle planted at 60 % depth of a 10k-token
document; gist.science technical summary, Metodologia: bidirectional vision
tower attention; abstract: window-attention merger).  No document, image or
weight of that paper is used: every value is drawn here from a seed.

Seed convention: numpy ``Generator(PCG64(seed))``; Q, then K, then V, each a
C-order ``standard_normal`` draw of its full shape times sigma.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (nearest, ties to even); returns float64."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == F32:
        return x.astype(np.float32).astype(np.float64)
    if dtype != BF16:
        raise ValueError(dtype)
    # bf16 keeps 8 significant bits: scale the fraction to [128, 256), round
    # half to even, scale back.  Magnitudes here are far from bf16's limits.
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


@dataclass
class Workload:
    name: str
    cu_seqlens: list
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    mask: object  # "causal" | "full" | ("window", W)
    sigma: float
    seed: int
    scale: float = None
    needle_pos: int | None = None  # local position of the planted key
    needle_coords: tuple = (31, 62)  # marker coordinate per KV head
    extra: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.scale is None:
            self.scale = 1.0 / math.sqrt(self.head_dim)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def seq_lens(self) -> list:
        cu = self.cu_seqlens
        return [int(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]


# The five workloads, in the order they are quoted (sizes of the pages'
# 2k/10k prefill and vision-tower cases; shapes of heads and dims fixed here).
WORKLOADS = {
    "1": Workload("causal fp32 N=256 1 head d=64", [0, 256], 1, 1, 64, F32,
                  "causal", 1.0, seed=1, scale=1.0 / 8.0),
    "2": Workload("causal bf16 N=2048 16/16 heads d=128", [0, 2048], 16, 16, 128, BF16,
                  "causal", 1.0, seed=2),
    "3": Workload("causal bf16 N=10240 16/2 heads d=128 needle@6144", [0, 10240], 16, 2,
                  128, BF16, "causal", 0.5, seed=3, needle_pos=6144),
    "4": Workload("full bf16 N=1024 16/16 heads d=72", [0, 1024], 16, 16, 72, BF16,
                  "full", 1.0, seed=4),
    "5a": Workload("packed causal bf16 2048+5120+8192+10240 16/2 heads d=128",
                   [0, 2048, 7168, 15360, 25600], 16, 2, 128, BF16, "causal", 1.0, seed=5),
    "5b": Workload("packed window-256 bf16 2048+5120+8192+10240 16/2 heads d=128",
                   [0, 2048, 7168, 15360, 25600], 16, 2, 128, BF16, ("window", 256), 1.0,
                   seed=5),
}


def draw_qkv(cu_seqlens, hq, hkv, d, dtype, sigma, seed):
    """Q, K, V ~ N(0, sigma^2) from ``seed``, rounded to ``dtype``."""
    T = int(cu_seqlens[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((T, hq, d)) * sigma
    k = rng.standard_normal((T, hkv, d)) * sigma
    v = rng.standard_normal((T, hkv, d)) * sigma
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def plant_needle(q, k, v, pos, coords):
    """Plant a retrievable key at local position ``pos`` of a one-sequence batch.

    For each KV head g: every query head of g gets the last row's query of the
    group's first head, the key at ``pos`` becomes 8 times that query (exact
    in bf16: a power-of-two multiple), and the value at ``pos`` becomes the
    one-hot vector at ``coords[g]``.  In place; returns the arrays.
    """
    T, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    last = T - 1
    for g in range(hkv):
        lead = q[last, G * g].copy()
        for h in range(G * g, G * (g + 1)):
            q[last, h] = lead
        k[pos, g] = 8.0 * lead
        v[pos, g] = 0.0
        v[pos, g, coords[g % len(coords)]] = 1.0
    return q, k, v


def make_inputs(w: Workload):
    """(q, k, v, cu_seqlens) for a workload, as float64 arrays of dtype values."""
    cu = np.asarray(w.cu_seqlens, dtype=np.int32)
    q, k, v = draw_qkv(cu, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, w.sigma, w.seed)
    if w.needle_pos is not None:
        plant_needle(q, k, v, w.needle_pos, w.needle_coords)
    return q, k, v, cu


def random_case(seed, max_seqs=4, max_len=300, dims=(64, 72, 128), ratios=(1, 2, 8),
                masks=("causal", "full", "window"), dtype=BF16, allow_empty=True):
    """A small random packed batch: lengths (some 0 or 1), head shape and mask."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_seqs = int(rng.integers(1, max_seqs + 1))
    lens = []
    for _ in range(n_seqs):
        r = rng.random()
        if allow_empty and r < 0.1:
            lens.append(0)
        elif r < 0.2:
            lens.append(1)
        else:
            lens.append(int(rng.integers(2, max_len + 1)))
    if sum(lens) == 0:
        lens[0] = 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = int(rng.choice(dims))
    G = int(rng.choice(ratios))
    hkv = int(rng.integers(1, 3))
    hq = G * hkv
    kind = str(rng.choice(masks))
    if kind == "window":
        mask = ("window", int(rng.choice([1, 7, 64, 100, 256, 4096])))
    else:
        mask = kind
    q, k, v = draw_qkv(cu, hq, hkv, d, dtype, 1.0, int(rng.integers(1 << 30)))
    scale = 1.0 / math.sqrt(d)
    return dict(q=q, k=k, v=v, cu=cu, hq=hq, hkv=hkv, d=d, mask=mask, scale=scale,
                dtype=dtype)


# ---------------------------------------------------------------------------
# Exact-probe inputs.  All values are small integers or powers of two, exact in
# bf16, chosen so that an exact integer property of the visible key set can be
# read back from the output.  They carry no attention arithmetic; the tests
# derive the expected integers from the mask definitions themselves.
# ---------------------------------------------------------------------------

CHUNK = 16  # keys per class in the count probe


def probe_count_inputs(cu, hq, hkv, d, cu_k=None):
    """Q = 0 (every visible key weighs the same); V[j, g, c] = 1 iff c is the
    class of packed key j, class = (j // 16) mod d.  cu_k: the keys' own
    packing when it differs from the queries' (cu)."""
    Tq = int(cu[-1])
    T = int((cu if cu_k is None else cu_k)[-1])
    q = np.zeros((Tq, hq, d))
    k = np.zeros((T, hkv, d))
    v = np.zeros((T, hkv, d))
    j = np.arange(T)
    v[j, :, (j // CHUNK) % d] = 1.0
    return q, k, v


def probe_index_inputs(cu, hq, hkv, d, sign, cu_k=None):
    """K[j] = (j >> 7, j & 127, 0, ...) from the packed index j; Q = sign *
    (2^17, 2^9, 0, ...).  The logit is then strictly monotone in j with gaps of
    at least 512 * scale, so the weight sits on the last (sign=+1) or first
    (sign=-1) visible key.  V[j, g, b] = bit b of j for b < 15, and
    V[j, g, 15 + g] = 1 marks the KV head.  cu_k: the keys' own packing."""
    Tq = int(cu[-1])
    T = int((cu if cu_k is None else cu_k)[-1])
    assert d >= 16 + hkv and T < (1 << 15)
    q = np.zeros((Tq, hq, d))
    k = np.zeros((T, hkv, d))
    v = np.zeros((T, hkv, d))
    j = np.arange(T)
    q[:, :, 0] = sign * float(1 << 17)
    q[:, :, 1] = sign * float(1 << 9)
    k[:, :, 0] = (j >> 7)[:, None]
    k[:, :, 1] = (j & 127)[:, None]
    for b in range(15):
        v[:, :, b] = ((j >> b) & 1)[:, None]
    for g in range(hkv):
        v[:, g, 15 + g] = 1.0
    return q, k, v


# ---------------------------------------------------------------------------
# Gated delta rule (the recurrent layers of the paper's hybrid backbone:
# abstract, result (i); gist.science summary, Metodologia).  The pages give
# the layer type and the 2k/10k-token prefill, not its head count or sizes;
# these shapes (16 heads of 128 key and value dims) are a plain choice for a
# 0.8B-parameter backbone.
# ---------------------------------------------------------------------------

def make_gdn_inputs(lens, n_heads, dk, dv, seed, decay=(0.85, 1.0)):
    """(q, k, v, g, beta) for a packed batch of sequences of ``lens`` tokens.

    q and k rows are unit-norm directions (the layer normalises them before
    the recurrence) rounded to bf16; v ~ N(0, 1) rounded to bf16; the decay
    alpha ~ U(decay) enters as g = log(alpha) and beta ~ U(0, 1), both
    rounded to fp32.  Draw order from ``Generator(PCG64(seed))``: q, k, v,
    alpha, beta, each C-order over its full shape.
    """
    T = int(np.sum(lens))
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((T, n_heads, dk))
    k = rng.standard_normal((T, n_heads, dk))
    v = rng.standard_normal((T, n_heads, dv))
    alpha = rng.uniform(decay[0], decay[1], (T, n_heads))
    beta = rng.uniform(0.0, 1.0, (T, n_heads))
    q = round_to(q / np.linalg.norm(q, axis=-1, keepdims=True), BF16)
    k = round_to(k / np.linalg.norm(k, axis=-1, keepdims=True), BF16)
    return (q, k, round_to(v, BF16), round_to(np.log(alpha), F32), round_to(beta, F32))


GDN_WORKLOADS = {
    # the 10k-token prefill of the paper's long-context case
    "gdn10k": dict(lens=[10240], n_heads=16, dk=128, dv=128, seed=21),
    # the packed 4-sequence batch of the attention workloads
    "gdn_packed": dict(lens=[2048, 5120, 8192, 10240], n_heads=16, dk=128, dv=128, seed=22),
}


# ---------------------------------------------------------------------------
# Vision tower attention block (the paper's SigLIP2 encoder layers: abstract,
# result (iii); gist.science summary, Metodologia: FP32 vision weights).  The
# pages give neither layer sizes nor image token counts; the shapes here are
# SigLIP2's so400m encoder (hidden 1152, 16 heads of 72) and images of 768
# patches (a 448 x 336 slice at 14-pixel patches), packed NaViT-style.
# ---------------------------------------------------------------------------

def make_vision_inputs(lens, hidden, n_heads, d, dtype, seed, qk_gain=1.5, bias_sigma=0.05):
    """(x, w_qkv, b_qkv, w_o, b_o) for a packed batch of images of ``lens`` patches.

    x ~ N(0, 1) (normalised activations); w_qkv ~ N(0, 1/hidden) with its q
    and k row blocks times ``qk_gain`` (sharper attention than chance);
    w_o ~ N(0, 1/(n_heads d)); both biases ~ N(0, bias_sigma^2).  Every array
    is rounded to ``dtype``.  Draw order from ``Generator(PCG64(seed))``: x,
    w_qkv, b_qkv, w_o, b_o, each C-order over its full shape.
    """
    T = int(np.sum(lens))
    hd = n_heads * d
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((T, hidden))
    w_qkv = rng.standard_normal((3 * hd, hidden)) / math.sqrt(hidden)
    w_qkv[:2 * hd] *= qk_gain
    b_qkv = rng.standard_normal(3 * hd) * bias_sigma
    w_o = rng.standard_normal((hidden, hd)) / math.sqrt(hd)
    b_o = rng.standard_normal(hidden) * bias_sigma
    return tuple(round_to(a, dtype) for a in (x, w_qkv, b_qkv, w_o, b_o))


VISION_WORKLOADS = {
    # a multi-slice image: five slices of 768 patches, packed
    "vision_slices_bf16": dict(lens=[768] * 5, hidden=1152, n_heads=16, d=72, dtype=BF16, seed=31),
    # the same in fp32, the precision the pages keep the vision weights in
    "vision_slices_f32": dict(lens=[768] * 5, hidden=1152, n_heads=16, d=72, dtype=F32, seed=32),
}
