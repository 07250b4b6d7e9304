"""Expected integers for the exact probes at any size.

The visible set of every row is an interval of keys; ``visible_interval``
derives it, vectorised, from the mask definitions (causal: keys up to the
row; full: the whole sequence; window: the row's block of W tokens aligned to
the sequence start).  test_probes_cpu.py checks it against the explicit sets
of pins.visible_set on small sizes.
"""
from __future__ import annotations

import numpy as np

from long_context_attention_prefill_amd import workloads as W


def visible_interval(cu, mask):
    """Packed [lo, hi) of visible keys for every packed query row."""
    cu = np.asarray(cu, dtype=np.int64)
    T = int(cu[-1])
    lo = np.zeros(T, dtype=np.int64)
    hi = np.zeros(T, dtype=np.int64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        i = np.arange(e - s)
        if mask == "causal":
            lo[s:e], hi[s:e] = s, s + i + 1
        elif mask == "full":
            lo[s:e], hi[s:e] = s, e
        else:
            w = int(mask[1])
            start = (i // w) * w
            lo[s:e] = s + start
            hi[s:e] = s + np.minimum(start + w, e - s)
    return lo, hi


def class_counts(cu, mask, d):
    """[T, d] int64: visible keys of each class (j // 16) % d, and [T] totals."""
    T = int(cu[-1])
    cls = (np.arange(T) // W.CHUNK) % d
    pref = np.zeros((T + 1, d), dtype=np.int64)
    np.add.at(pref, (np.arange(T) + 1, cls), 1)
    pref = np.cumsum(pref, axis=0)
    lo, hi = visible_interval(cu, mask)
    return pref[hi] - pref[lo], hi - lo


def check_count_output(out, cu, mask, d):
    """out: [T, H, d] float output of the count probe. Returns #rows checked."""
    want, nvis = class_counts(cu, mask, d)
    got = np.rint(np.asarray(out, dtype=np.float64) * nvis[:, None, None]).astype(np.int64)
    bad = np.argwhere(got != want[:, None, :])
    assert bad.size == 0, f"count probe mismatch at (t, h, class) {bad[:5].tolist()}"
    return out.shape[0]


def decode_indices(out):
    """[T, H] integers from the 15 bit-lanes of the index probe's output."""
    bits = np.rint(np.asarray(out[..., :15], dtype=np.float64)).astype(np.int64)
    assert np.all((bits == 0) | (bits == 1)), "index probe output is not 0/1"
    return np.sum(bits << np.arange(15), axis=-1)


def check_index_output(out, cu, mask, hq, hkv, sign):
    lo, hi = visible_interval(cu, mask)
    want = (hi - 1) if sign > 0 else lo
    got = decode_indices(out)
    bad = np.argwhere(got != want[:, None])
    assert bad.size == 0, f"index probe mismatch at (t, h) {bad[:5].tolist()}"
    marks = np.rint(np.asarray(out[..., 15:15 + hkv], dtype=np.float64)).astype(np.int64)
    want_marks = np.zeros((hq, hkv), dtype=np.int64)
    want_marks[np.arange(hq), np.arange(hq) // (hq // hkv)] = 1
    assert np.array_equal(marks, np.broadcast_to(want_marks, marks.shape)), "kv head marker"


# ---------------------------------------------------------------- queries ending longer key sequences

def visible_interval_kv(cu_q, cu_k, mask):
    """Packed key [lo, hi) for every packed query row when the Lq queries of a
    sequence are the last Lq of its Lk positions (query i at i + Lk - Lq)."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    Tq = int(cu_q[-1])
    lo = np.zeros(Tq, dtype=np.int64)
    hi = np.zeros(Tq, dtype=np.int64)
    for b in range(len(cu_q) - 1):
        sq, eq = int(cu_q[b]), int(cu_q[b + 1])
        sk, nk = int(cu_k[b]), int(cu_k[b + 1] - cu_k[b])
        pos = np.arange(eq - sq) + (nk - (eq - sq))
        if mask == "causal":
            lo[sq:eq], hi[sq:eq] = sk, sk + pos + 1
        elif mask == "full":
            lo[sq:eq], hi[sq:eq] = sk, sk + nk
        else:
            w = int(mask[1])
            start = (pos // w) * w
            lo[sq:eq] = sk + start
            hi[sq:eq] = sk + np.minimum(start + w, nk)
    return lo, hi


def check_count_output_kv(out, cu_q, cu_k, mask, d):
    Tk = int(cu_k[-1])
    cls = (np.arange(Tk) // W.CHUNK) % d
    pref = np.zeros((Tk + 1, d), dtype=np.int64)
    np.add.at(pref, (np.arange(Tk) + 1, cls), 1)
    pref = np.cumsum(pref, axis=0)
    lo, hi = visible_interval_kv(cu_q, cu_k, mask)
    want, nvis = pref[hi] - pref[lo], hi - lo
    got = np.rint(np.asarray(out, dtype=np.float64) * nvis[:, None, None]).astype(np.int64)
    bad = np.argwhere(got != want[:, None, :])
    assert bad.size == 0, f"count probe mismatch at (t, h, class) {bad[:5].tolist()}"


def check_index_output_kv(out, cu_q, cu_k, mask, hq, hkv, sign):
    lo, hi = visible_interval_kv(cu_q, cu_k, mask)
    want = (hi - 1) if sign > 0 else lo
    got = decode_indices(out)
    bad = np.argwhere(got != want[:, None])
    assert bad.size == 0, f"index probe mismatch at (t, h) {bad[:5].tolist()}"
    marks = np.rint(np.asarray(out[..., 15:15 + hkv], dtype=np.float64)).astype(np.int64)
    want_marks = np.zeros((hq, hkv), dtype=np.int64)
    want_marks[np.arange(hq), np.arange(hq) // (hq // hkv)] = 1
    assert np.array_equal(marks, np.broadcast_to(want_marks, marks.shape)), "kv head marker"
