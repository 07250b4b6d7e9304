"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the mathematics or an independent routine fixes:

* hand-derived exact cases (tests/golden/handworked.json),
* a library routine: torch's scaled_dot_product_attention on CPU in float64,
* closed forms (zero scale gives plain means, window 1 gives V, ...),
* invariants (key shift, joint key/value permutation, GQA = repeated MHA,
  packed batch = separate calls),
* exact integer probes (count of visible keys per class, index of the first
  and last visible key) whose expected integers come from the mask
  definitions written out here as explicit sets,
* the needle planted at 60 % depth of a 10k-token sequence, which the pages
  say exact attention retrieves (paper "A Modern Multimodal Assistant on a
  6 GB 2011 GPU", abstract, result (iii)).

The same list runs against deliberately broken copies of the oracle (see
test_oracle_mutants.py): every planted mistake must trip at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from long_context_attention_prefill_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# visible sets written out as explicit Python sets (an independent statement of
# the three masks; shares nothing with the oracle's range formula)
# ---------------------------------------------------------------------------

def visible_set(mask, i, n):
    if mask == "causal":
        return {j for j in range(n) if j <= i}
    if mask == "full":
        return set(range(n))
    _, w = mask
    return {j for j in range(n) if j // w == i // w}


def dense_mask(cu, mask):
    """Boolean [T, T] matrix, True where packed query t may see packed key u."""
    T = int(cu[-1])
    M = np.zeros((T, T), dtype=bool)
    for b in range(len(cu) - 1):
        s, n = int(cu[b]), int(cu[b + 1] - cu[b])
        for i in range(n):
            for j in visible_set(mask, i, n):
                M[s + i, s + j] = True
    return M


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite oracle output"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand(cu, hq, hkv, d, seed, sigma=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(cu[-1])
    return (rng.standard_normal((T, hq, d)) * sigma, rng.standard_normal((T, hkv, d)) * sigma,
            rng.standard_normal((T, hkv, d)) * sigma)


MASKS = ["causal", "full", ("window", 1), ("window", 3), ("window", 5), ("window", 64)]


# ---------------------------------------------------------------------------
# 1. hand-derived exact cases
# ---------------------------------------------------------------------------

def pin_handworked(orc):
    with open(os.path.join(HERE, "golden", "handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        mask = c["mask"] if isinstance(c["mask"], str) else tuple(c["mask"])
        scale = math.log(2.0) if c["scale"] == "ln2" else float(c["scale"])
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        out, lse = orc.attention(q, k, v, c["cu_seqlens"], mask, scale, return_lse=True)
        want = np.array([[[float(Fraction(x)) for x in row] for row in tok] for tok in c["out"]])
        want_lse = np.log(np.array([[float(Fraction(x)) for x in tok] for tok in c["lse_arg"]]))
        _close(out, want, 1e-14, c["name"])
        _close(lse, want_lse, 1e-14, c["name"] + " lse")


# ---------------------------------------------------------------------------
# 2. a library routine: torch SDPA, CPU, float64
# ---------------------------------------------------------------------------

def _torch_sdpa(q, k, v, cu, mask, scale):
    import torch
    import torch.nn.functional as F

    T, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    out = np.zeros_like(q)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        n = e - s
        if n == 0:
            continue
        tq = torch.from_numpy(q[s:e]).permute(1, 0, 2)  # [Hq, n, d]
        tk = torch.from_numpy(k[s:e]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        tv = torch.from_numpy(v[s:e]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        if mask == "causal":
            o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
        elif mask == "full":
            o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        else:
            w = mask[1]
            idx = torch.arange(n)
            allowed = (idx[:, None] // w) == (idx[None, :] // w)
            o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
        out[s:e] = o.permute(1, 0, 2).numpy()
    return out


def pin_torch_sdpa(orc):
    cases = [
        ([0, 37], 1, 1, 64, "causal"),
        ([0, 50, 50, 81, 82], 4, 2, 72, "causal"),
        ([0, 64, 100], 8, 1, 128, "full"),
        ([0, 19, 45], 2, 2, 16, ("window", 7)),
        ([0, 33, 129], 4, 1, 8, ("window", 32)),
        ([0, 5, 70], 3, 3, 4, ("window", 1)),
    ]
    for seed, (cu, hq, hkv, d, mask) in enumerate(cases):
        q, k, v = _rand(cu, hq, hkv, d, 100 + seed)
        scale = 1.0 / math.sqrt(d) * (1.0 + 0.3 * seed)
        got = orc.attention(q, k, v, cu, mask, scale)
        want = _torch_sdpa(q, k, v, np.array(cu), mask, scale)
        _close(got, want, 1e-12, f"sdpa {cu} {mask}")


# ---------------------------------------------------------------------------
# 3. closed forms
# ---------------------------------------------------------------------------

def pin_zero_scale_means(orc):
    """scale = 0: every visible key weighs the same, so each row is the plain
    mean of its visible values."""
    cu = [0, 9, 9, 30]
    q, k, v = _rand(cu, 2, 1, 5, 7)
    for mask in MASKS:
        got = orc.attention(q, k, v, cu, mask, 0.0)
        for b in range(len(cu) - 1):
            s, n = cu[b], cu[b + 1] - cu[b]
            for i in range(n):
                vis = sorted(visible_set(mask, i, n))
                mean = v[[s + j for j in vis], 0].mean(axis=0)
                for h in range(2):
                    _close(got[s + i, h], mean, 1e-14, f"zero scale {mask} row {i}")


def pin_window_one_is_v(orc):
    """Window 1: each row sees only itself."""
    cu = [0, 17, 40]
    q, k, v = _rand(cu, 4, 2, 6, 8)
    got = orc.attention(q, k, v, cu, ("window", 1), 0.37)
    _close(got, np.repeat(v, 2, axis=1), 1e-15, "window 1")


def pin_first_row_and_single_token(orc):
    """Causal row 0 of every sequence, and any length-1 sequence, returns v_0."""
    cu = [0, 1, 12, 13, 40]
    q, k, v = _rand(cu, 2, 2, 7, 9)
    for mask in ("causal", "full", ("window", 4)):
        got = orc.attention(q, k, v, cu, mask, 0.8)
        for b in range(len(cu) - 1):
            s, n = cu[b], cu[b + 1] - cu[b]
            if mask == "causal" or n == 1:
                _close(got[s], v[s], 1e-15, f"row0 {mask} seq {b}")


def pin_constant_values(orc):
    """Constant V gives that constant in every row."""
    cu = [0, 25, 61]
    q, k, _ = _rand(cu, 4, 1, 9, 10)
    c = np.linspace(-2.0, 3.0, 9)
    v = np.broadcast_to(c, (61, 1, 9)).copy()
    for mask in MASKS:
        got = orc.attention(q, k, v, cu, mask, 0.5)
        _close(got, np.broadcast_to(c, got.shape), 1e-13, f"const V {mask}")


def pin_wide_window_is_full(orc):
    cu = [0, 31, 63]
    q, k, v = _rand(cu, 2, 1, 8, 11)
    a = orc.attention(q, k, v, cu, ("window", 32), 0.4)
    b = orc.attention(q, k, v, cu, "full", 0.4)
    _close(a, b, 0.0, "window >= len vs full")


def pin_two_key_sigmoid(orc):
    """Causal row 1 sees two keys: weight of key 1 is sigmoid(s_1 - s_0)."""
    cu = [0, 2]
    q, k, v = _rand(cu, 1, 1, 4, 12)
    scale = 0.9
    got = orc.attention(q, k, v, cu, "causal", scale)
    s0 = scale * float(q[1, 0] @ k[0, 0])
    s1 = scale * float(q[1, 0] @ k[1, 0])
    w1 = 1.0 / (1.0 + math.exp(-(s1 - s0)))
    _close(got[1, 0], (1 - w1) * v[0, 0] + w1 * v[1, 0], 1e-15, "sigmoid")


# ---------------------------------------------------------------------------
# 4. invariants
# ---------------------------------------------------------------------------

def pin_probabilities_sum_to_one(orc):
    cu = [0, 13, 40]
    q, k, v = _rand(cu, 2, 1, 6, 13)
    for mask in MASKS:
        for t in (0, 5, 12, 13, 27, 39):
            for h in (0, 1):
                p = orc.probs(q, k, v, cu, mask, 0.7, t, h)
                b = 0 if t < 13 else 1
                i = t - cu[b]
                vis = visible_set(mask, i, cu[b + 1] - cu[b])
                assert abs(p.sum() - 1.0) < 1e-14, (mask, t, h, p.sum())
                assert all(p[j] > 0 for j in vis), (mask, t, "visible key with 0 weight")
                assert all(p[j] == 0 for j in range(len(p)) if j not in vis), (mask, t)


def pin_key_shift(orc):
    """Adding one vector to every key adds a per-row constant to the scores."""
    cu = [0, 20, 47]
    q, k, v = _rand(cu, 2, 2, 8, 14)
    shift = np.linspace(-1.0, 1.0, 8)
    for mask in MASKS:
        a = orc.attention(q, k, v, cu, mask, 0.6)
        b = orc.attention(q, k + shift, v, cu, mask, 0.6)
        _close(a, b, 1e-12, f"key shift {mask}")


def pin_joint_permutation(orc):
    """Full attention does not depend on the order of the (key, value) pairs."""
    cu = [0, 29]
    q, k, v = _rand(cu, 2, 1, 6, 15)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(29)
    a = orc.attention(q, k, v, cu, "full", 0.8)
    b = orc.attention(q, k[perm], v[perm], cu, "full", 0.8)
    _close(a, b, 1e-13, "joint permutation")


def pin_gqa_equals_repeated_mha(orc):
    cu = [0, 21, 50]
    q, k, v = _rand(cu, 8, 2, 5, 16)
    for mask in MASKS:
        a = orc.attention(q, k, v, cu, mask, 0.5)
        b = orc.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), cu, mask, 0.5)
        _close(a, b, 0.0, f"gqa {mask}")
        # and head h really reads kv head h // 4: swapping kv heads swaps groups
        c = orc.attention(q, k[:, ::-1], v[:, ::-1], cu, mask, 0.5)
        d = orc.attention(np.concatenate([q[:, 4:], q[:, :4]], axis=1), k, v, cu, mask, 0.5)
        _close(c, np.concatenate([d[:, 4:], d[:, :4]], axis=1), 0.0, f"gqa map {mask}")


def pin_packed_equals_separate(orc):
    cu = [0, 11, 11, 30, 31, 58]
    q, k, v = _rand(cu, 2, 1, 7, 17)
    for mask in MASKS:
        a = orc.attention(q, k, v, cu, mask, 0.45)
        for b in range(len(cu) - 1):
            s, e = cu[b], cu[b + 1]
            if e == s:
                continue
            one = orc.attention(q[s:e], k[s:e], v[s:e], [0, e - s], mask, 0.45)
            _close(a[s:e], one, 0.0, f"packed vs separate {mask} seq {b}")


def pin_rows_api_matches_full(orc):
    cu = [0, 40, 77]
    q, k, v = _rand(cu, 4, 2, 8, 18)
    full, lse = orc.attention(q, k, v, cu, "causal", 0.3, return_lse=True)
    rows = np.array([0, 39, 40, 41, 76, 5])
    heads = np.array([0, 3, 1, 2, 3, 0])
    part, plse = orc.attention_rows(q, k, v, cu, "causal", 0.3, rows, heads, return_lse=True)
    _close(part, full[rows, heads], 0.0, "rows api")
    _close(plse, lse[rows, heads], 0.0, "rows api lse")


def pin_lse_definition(orc):
    """LSE equals log(sum exp(scores)) over the visible keys, via scipy."""
    from scipy.special import logsumexp

    cu = [0, 15, 33]
    q, k, v = _rand(cu, 2, 1, 4, 19)
    for mask in MASKS:
        _, lse = orc.attention(q, k, v, cu, mask, 1.3, return_lse=True)
        for b in range(2):
            s, n = cu[b], cu[b + 1] - cu[b]
            for i in range(n):
                for h in range(2):
                    vis = sorted(visible_set(mask, i, n))
                    sc = [1.3 * float(q[s + i, h] @ k[s + j, 0]) for j in vis]
                    assert abs(lse[s + i, h] - logsumexp(sc)) < 1e-12, (mask, i, h)


def pin_dense_bruteforce(orc):
    """Explicit [T, T] score matrix over the whole packed batch with a mask
    built from the visible sets; scipy softmax row by row."""
    from scipy.special import softmax

    cu = [0, 6, 6, 19, 20, 34]
    q, k, v = _rand(cu, 4, 2, 5, 20)
    T = 34
    for mask in MASKS:
        M = dense_mask(cu, mask)
        got = orc.attention(q, k, v, cu, mask, 0.55)
        for h in range(4):
            g = h // 2
            S = 0.55 * q[:, h, :] @ k[:, g, :].T
            S = np.where(M, S, -np.inf)
            P = softmax(S, axis=1)
            _close(got[:, h, :], P @ v[:, g, :], 1e-13, f"dense {mask} head {h}")
        assert T == M.shape[0]


# ---------------------------------------------------------------------------
# 4b. queries against a longer key sequence (chunked prefill, decode): the
# Lq queries of a sequence are its last Lq positions, query i at i + Lk - Lq
# ---------------------------------------------------------------------------

def visible_set_kv(mask, i, lq, lk):
    """Visible keys of local query i when Lq queries end a sequence of Lk keys,
    as an explicit set (the position offset written out independently)."""
    pos = i + (lk - lq)
    if mask == "causal":
        return {j for j in range(lk) if j <= pos}
    if mask == "full":
        return set(range(lk))
    _, w = mask
    return {j for j in range(lk) if j // w == pos // w}


def _rand_kv(cu_q, cu_k, hq, hkv, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((int(cu_q[-1]), hq, d)), rng.standard_normal((int(cu_k[-1]), hkv, d)),
            rng.standard_normal((int(cu_k[-1]), hkv, d)))


KV_CASES = [
    ([0, 5, 5, 12], [0, 21, 30, 50], 4, 2, 8),    # chunks of 5 and 7 queries, an empty chunk
    ([0, 1, 2, 3], [0, 17, 18, 40], 2, 1, 16),    # decode: one query per sequence
    ([0, 9], [0, 9], 2, 2, 4),                    # the square case
]


def pin_kv_torch_sdpa(orc):
    """torch SDPA (CPU, float64) with an explicit boolean mask built from
    visible_set_kv, and scipy's logsumexp for the LSE."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    for seed, (cu_q, cu_k, hq, hkv, d) in enumerate(KV_CASES):
        q, k, v = _rand_kv(cu_q, cu_k, hq, hkv, d, 300 + seed)
        for mask in MASKS:
            scale = 0.7 / math.sqrt(d)
            got, lse = orc.attention(q, k, v, cu_q, mask, scale, return_lse=True, cu_seqlens_k=cu_k)
            for b in range(len(cu_q) - 1):
                sq, lq = cu_q[b], cu_q[b + 1] - cu_q[b]
                sk, lk = cu_k[b], cu_k[b + 1] - cu_k[b]
                if lq == 0:
                    continue
                allowed = torch.tensor([[j in visible_set_kv(mask, i, lq, lk) for j in range(lk)]
                                        for i in range(lq)])
                G = hq // hkv
                tq = torch.from_numpy(q[sq:sq + lq]).permute(1, 0, 2)
                tk = torch.from_numpy(k[sk:sk + lk]).permute(1, 0, 2).repeat_interleave(G, dim=0)
                tv = torch.from_numpy(v[sk:sk + lk]).permute(1, 0, 2).repeat_interleave(G, dim=0)
                o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
                _close(got[sq:sq + lq], o.permute(1, 0, 2).numpy(), 1e-12, f"kv sdpa {cu_q} {cu_k} {mask}")
                for i in range(lq):
                    vis = sorted(visible_set_kv(mask, i, lq, lk))
                    for h in range(hq):
                        sc = [scale * float(q[sq + i, h] @ k[sk + j, h // G]) for j in vis]
                        assert abs(lse[sq + i, h] - logsumexp(sc)) < 1e-12, (mask, b, i, h)


def pin_kv_suffix_of_square(orc):
    """Lq queries ending a sequence of Lk give exactly the last Lq rows of the
    square attention over the whole sequence."""
    cu_k = [0, 30, 30, 71]
    q_full, k, v = _rand(cu_k, 4, 2, 6, 31)
    lqs = [11, 0, 41]
    cu_q = [0, 11, 11, 52]
    rows = np.concatenate([np.arange(cu_k[b + 1] - lqs[b], cu_k[b + 1]) for b in range(3)])
    for mask in MASKS:
        square = orc.attention(q_full, k, v, cu_k, mask, 0.4)
        part = orc.attention(q_full[rows], k, v, cu_q, mask, 0.4, cu_seqlens_k=cu_k)
        _close(part, square[rows], 0.0, f"suffix {mask}")


def pin_kv_decode_single_query(orc):
    """One query per sequence under the causal mask sees every key of its
    sequence: numpy softmax over all of them."""
    cu_q, cu_k = [0, 1, 2], [0, 13, 40]
    q, k, v = _rand_kv(cu_q, cu_k, 4, 1, 8, 32)
    got = orc.attention(q, k, v, cu_q, "causal", 0.5, cu_seqlens_k=cu_k)
    for b in range(2):
        ks, vs = k[cu_k[b]:cu_k[b + 1], 0], v[cu_k[b]:cu_k[b + 1], 0]
        for h in range(4):
            sc = 0.5 * (ks @ q[b, h])
            w_ = np.exp(sc - sc.max())
            _close(got[b, h], (w_ / w_.sum()) @ vs, 1e-13, f"decode seq {b} head {h}")


def pin_lse_merges_split_keys(orc):
    """Two halves of a row's keys, each with its output and LSE, merge into the
    whole row: o = (o1 e^lse1 + o2 e^lse2) / (e^lse1 + e^lse2), lse = log(e^lse1 + e^lse2)."""
    n, a = 50, 21
    q, k, v = _rand([0, n], 2, 1, 8, 33)
    qr = q[n - 1:n]
    whole, lw = orc.attention(qr, k, v, [0, 1], "full", 0.9, return_lse=True, cu_seqlens_k=[0, n])
    o1, l1 = orc.attention(qr, k[:a], v[:a], [0, 1], "full", 0.9, return_lse=True, cu_seqlens_k=[0, a])
    o2, l2 = orc.attention(qr, k[a:], v[a:], [0, 1], "full", 0.9, return_lse=True, cu_seqlens_k=[0, n - a])
    mx = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - mx), np.exp(l2 - mx)
    merged = (o1 * w1[..., None] + o2 * w2[..., None]) / (w1 + w2)[..., None]
    _close(merged, whole, 1e-13, "lse merge")
    _close(mx + np.log(w1 + w2), lw, 1e-13, "lse merge lse")


# ---------------------------------------------------------------------------
# 5. exact integer probes (expected integers from the explicit visible sets)
# ---------------------------------------------------------------------------

PROBE_CU = [0, 37, 37, 290, 291, 600]


def expected_class_counts(cu, mask, d, t):
    b = int(np.searchsorted(cu, t, side="right") - 1)
    s, n = int(cu[b]), int(cu[b + 1] - cu[b])
    vis = visible_set(mask, t - s, n)
    cnt = np.zeros(d, dtype=np.int64)
    for j in vis:
        cnt[((s + j) // W.CHUNK) % d] += 1
    return cnt, len(vis)


def pin_probe_count(orc):
    cu = np.array(PROBE_CU)
    d = 64
    q, k, v = W.probe_count_inputs(cu, 2, 1, d)
    for mask in ("causal", "full", ("window", 7), ("window", 100)):
        out = orc.attention(q, k, v, cu, mask, 1.0 / 8.0)
        for t in range(int(cu[-1])):
            cnt, nvis = expected_class_counts(cu, mask, d, t)
            for h in range(2):
                got = np.rint(out[t, h] * nvis).astype(np.int64)
                assert np.array_equal(got, cnt), (mask, t, h)


def expected_first_last(cu, mask, t):
    b = int(np.searchsorted(cu, t, side="right") - 1)
    s, n = int(cu[b]), int(cu[b + 1] - cu[b])
    vis = visible_set(mask, t - s, n)
    return s + min(vis), s + max(vis)


def decode_index(row):
    bits = np.rint(row[:15]).astype(np.int64)
    assert np.all((bits == 0) | (bits == 1))
    return int(sum(int(b) << i for i, b in enumerate(bits)))


def pin_probe_index(orc):
    cu = np.array(PROBE_CU)
    d, hq, hkv = 32, 4, 2
    for sign in (+1, -1):
        q, k, v = W.probe_index_inputs(cu, hq, hkv, d, sign)
        for mask in ("causal", "full", ("window", 7), ("window", 64)):
            out = orc.attention(q, k, v, cu, mask, 1.0 / math.sqrt(d))
            assert np.all(np.isfinite(out)), mask
            for t in range(int(cu[-1])):
                first, last = expected_first_last(cu, mask, t)
                for h in range(hq):
                    assert decode_index(out[t, h]) == (last if sign > 0 else first), \
                        (sign, mask, t, h)
                    marks = np.rint(out[t, h, 15:15 + hkv]).astype(np.int64)
                    want = np.zeros(hkv, dtype=np.int64)
                    want[h // (hq // hkv)] = 1
                    assert np.array_equal(marks, want), (sign, mask, t, h, "kv head")


# ---------------------------------------------------------------------------
# 6. the needle at 60 % depth of the 10k-token causal workload
# ---------------------------------------------------------------------------

def check_needle(out_last, w):
    """out_last[h, :] = output of the last row for query head h."""
    G = w.n_q_heads // w.n_kv_heads
    for h in range(w.n_q_heads):
        c = w.needle_coords[(h // G) % len(w.needle_coords)]
        row = np.asarray(out_last[h], dtype=np.float64)
        assert int(np.argmax(row)) == c, (h, int(np.argmax(row)), c)
        assert row[c] >= 0.99, (h, row[c])


def pin_needle(orc):
    w = W.WORKLOADS["3"]
    q, k, v, cu = W.make_inputs(w)
    T = w.total_tokens
    rows = np.full(w.n_q_heads, T - 1)
    heads = np.arange(w.n_q_heads)
    out = orc.attention_rows(q, k, v, cu, w.mask, w.scale, rows, heads)
    check_needle(out, w)
    # and without the planted key the marker is not retrieved
    k2 = k.copy()
    k2[w.needle_pos] = W.round_to(
        np.random.Generator(np.random.PCG64(99)).standard_normal(k2[w.needle_pos].shape) * 0.5,
        W.BF16)
    out2 = orc.attention_rows(q, k2, v, cu, w.mask, w.scale, rows, heads)
    for h in range(w.n_q_heads):
        c = w.needle_coords[h // (w.n_q_heads // w.n_kv_heads)]
        assert out2[h, c] < 0.5, (h, out2[h, c])


ALL_PINS = [
    pin_handworked, pin_torch_sdpa, pin_zero_scale_means, pin_window_one_is_v,
    pin_first_row_and_single_token, pin_constant_values, pin_wide_window_is_full,
    pin_two_key_sigmoid, pin_probabilities_sum_to_one, pin_key_shift, pin_joint_permutation,
    pin_gqa_equals_repeated_mha, pin_packed_equals_separate, pin_rows_api_matches_full,
    pin_lse_definition, pin_dense_bruteforce, pin_kv_torch_sdpa, pin_kv_suffix_of_square,
    pin_kv_decode_single_query, pin_lse_merges_split_keys, pin_probe_count, pin_probe_index,
    pin_needle,
]
