"""Pins of the vision-block oracle (oracle/vision.py): a case worked by hand,
a pure-Python brute force over every index, and closed forms the block's
definition fixes (zero output weights, one-token windows, head relabelling).

Each pin takes the oracle module and the attention oracle it composes with."""
import math

import numpy as np

TOL = 1e-12


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
    if not err <= tol:
        raise AssertionError(f"{what}: max abs error {err:.3e} > {tol:.1e}")


def pin_hand_worked(vision, orc):
    """Two tokens, one head of dim 1, hidden 2, scale 1/2.  With x = I the
    projection rows are the per-token values: q = (2 ln 3, 0), k = (0, 1),
    v = (4, 8).  Token 0's logits are (0, ln 3): weights 1/4, 3/4 and
    a_0 = 1 + 6 = 7; token 1's logits are (0, 0): a_1 = 6.  Then
    out = a (1, -2) + (0, 1): (7, -13) and (6, -11)."""
    x = np.eye(2)
    w_qkv = np.array([[2 * math.log(3.0), 0.0], [0.0, 1.0], [4.0, 8.0]])
    b_qkv = np.zeros(3)
    w_o = np.array([[1.0], [-2.0]])
    b_o = np.array([0.0, 1.0])
    got = vision.attention_block(orc, x, w_qkv, b_qkv, w_o, b_o, [0, 2], 1, "full", 0.5)
    _close(got, [[7.0, -13.0], [6.0, -11.0]], TOL, "hand-worked block")


def _brute(x, w_qkv, b_qkv, w_o, b_o, cu, H, mask, scale):
    """Every sum written out as a loop, no array algebra."""
    T, hidden = len(x), len(x[0])
    hd = len(w_qkv) // 3
    d = hd // H
    proj = [[b_qkv[r] + sum(x[t][c] * w_qkv[r][c] for c in range(hidden)) for r in range(3 * hd)]
            for t in range(T)]
    a = [[0.0] * hd for _ in range(T)]
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        for t in range(s0, s1):
            i = t - s0
            for h in range(H):
                keys = []
                for j in range(s1 - s0):
                    if mask == "causal" and j > i:
                        continue
                    if isinstance(mask, tuple) and j // mask[1] != i // mask[1]:
                        continue
                    keys.append(j)
                logit = {j: scale * sum(proj[t][h * d + c] * proj[s0 + j][hd + h * d + c] for c in range(d))
                         for j in keys}
                top = max(logit.values())
                wsum = sum(math.exp(logit[j] - top) for j in keys)
                for c in range(d):
                    a[t][h * d + c] = sum(math.exp(logit[j] - top) * proj[s0 + j][2 * hd + h * d + c]
                                          for j in keys) / wsum
    return [[b_o[n] + sum(a[t][m] * w_o[n][m] for m in range(hd)) for n in range(len(w_o))] for t in range(T)]


def pin_bruteforce(vision, orc):
    """Two images (3 and 2 tokens), 2 heads of dim 2, hidden 3, under every
    mask kind, against the loops above."""
    rng = np.random.Generator(np.random.PCG64(7))
    T, H, d, hidden = 5, 2, 2, 3
    x = rng.standard_normal((T, hidden))
    w_qkv = rng.standard_normal((3 * H * d, hidden))
    b_qkv = rng.standard_normal(3 * H * d) * 0.3
    w_o = rng.standard_normal((hidden, H * d))
    b_o = rng.standard_normal(hidden) * 0.3
    cu = [0, 3, 5]
    for mask in ("full", "causal", ("window", 2)):
        want = _brute(x.tolist(), w_qkv.tolist(), b_qkv.tolist(), w_o.tolist(), b_o.tolist(), cu, H, mask, 0.7)
        got = vision.attention_block(orc, x, w_qkv, b_qkv, w_o, b_o, cu, H, mask, 0.7)
        _close(got, want, 1e-12, f"brute force, mask {mask}")


def pin_zero_output_weights(vision, orc):
    """W_o = 0 leaves the output bias alone in every row, whatever the rest."""
    rng = np.random.Generator(np.random.PCG64(8))
    x = rng.standard_normal((6, 4))
    w_qkv = rng.standard_normal((12, 4))
    b_o = rng.standard_normal(4)
    got = vision.attention_block(orc, x, w_qkv, np.ones(12), np.zeros((4, 4)), b_o, [0, 6], 2, "full")
    _close(got, np.tile(b_o, (6, 1)), 0.0, "zero W_o")


def pin_one_token_windows(vision, orc):
    """Windows of one token: each token sees only itself, its softmax weight
    is 1 and the attention output is its own value, so the block is the
    affine map out = (x W_v^T + b_v) W_o^T + b_o, however large q and k are."""
    rng = np.random.Generator(np.random.PCG64(9))
    T, H, d, hidden = 7, 2, 3, 5
    x = rng.standard_normal((T, hidden))
    w_qkv = rng.standard_normal((3 * H * d, hidden))
    w_qkv[:2 * H * d] *= 50.0
    b_qkv = rng.standard_normal(3 * H * d)
    w_o = rng.standard_normal((hidden, H * d))
    b_o = rng.standard_normal(hidden)
    v = x @ w_qkv[2 * H * d:].T + b_qkv[2 * H * d:]
    got = vision.attention_block(orc, x, w_qkv, b_qkv, w_o, b_o, [0, 4, 7], H, ("window", 1))
    _close(got, v @ w_o.T + b_o, 1e-12, "one-token windows")


def pin_head_relabelling(vision, orc):
    """Heads are independent: relabelling them in W_qkv (rows, each block),
    b_qkv and W_o (columns) leaves the output unchanged; relabelling them in
    W_o alone does not."""
    rng = np.random.Generator(np.random.PCG64(10))
    T, H, d, hidden = 6, 3, 2, 4
    x = rng.standard_normal((T, hidden))
    w_qkv = rng.standard_normal((3 * H * d, hidden))
    b_qkv = rng.standard_normal(3 * H * d)
    w_o = rng.standard_normal((hidden, H * d))
    b_o = rng.standard_normal(hidden)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    rows = np.concatenate([blk * H * d + cols for blk in range(3)])
    base = vision.attention_block(orc, x, w_qkv, b_qkv, w_o, b_o, [0, 6], H, "full")
    same = vision.attention_block(orc, x, w_qkv[rows], b_qkv[rows], w_o[:, cols], b_o, [0, 6], H, "full")
    _close(same, base, 1e-12, "consistent head relabelling")
    moved = vision.attention_block(orc, x, w_qkv, b_qkv, w_o[:, cols], b_o, [0, 6], H, "full")
    if float(np.max(np.abs(moved - base))) < 1e-3:
        raise AssertionError("relabelling W_o alone changed nothing")


ALL_PINS = [pin_hand_worked, pin_bruteforce, pin_zero_output_weights, pin_one_token_windows,
            pin_head_relabelling]
