"""Pins of the gated-delta-rule oracle: what the mathematics fixes, checked
against oracle/gdn_oracle.c (CPU only).

The oracle is the token-by-token scan of the recurrence (paper "A Modern
Multimodal Assistant on a 6 GB 2011 GPU", abstract result (i) and gist.science
summary, Metodologia: gated-delta-net layers; the recurrence of the gated
delta rule paper the pages link).  None of these pins re-types that scan:
each checks a consequence of the definition that a dropped term, a wrong sign,
a transposed state or an index slip would break.
"""
import numpy as np

TOL = 1e-10


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    if not err <= tol:
        raise AssertionError(f"{what}: max abs error {err:.3e} > {tol:.1e}")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(cu, H, dk, dv, seed, decay=(0.7, 1.0)):
    """fp64 inputs: unit-norm q and k (as the layer feeds them), normal v,
    alpha = exp(g) uniform in `decay`, beta uniform in (0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(cu[-1])
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    g = np.log(rng.uniform(decay[0], decay[1], (T, H)))
    beta = rng.uniform(0.0, 1.0, (T, H))
    return q, k, v, g, beta


def pin_gdn_single_token(gdn):
    """One token: o = S' q' + beta (v - S' k)(k . q'), S' = alpha S0, q' = scale q."""
    rng = np.random.Generator(np.random.PCG64(1))
    dk, dv, scale = 5, 3, 0.7
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    s0 = rng.standard_normal((dv, dk))
    g, beta = -0.3, 0.6
    out, fin = gdn.gated_delta_rule(q[None, None], k[None, None], v[None, None], [[g]], [[beta]],
                                    [0, 1], scale, initial_state=s0[None, None])
    sp = np.exp(g) * s0
    want_s = sp + beta * np.outer(v - sp @ k, k)
    _close(fin[0, 0], want_s, TOL, "state after one token")
    _close(out[0, 0], want_s @ (scale * q), TOL, "output of one token")
    # with a zero initial state the output is beta (k . q') v
    out, _ = gdn.gated_delta_rule(q[None, None], k[None, None], v[None, None], [[g]], [[beta]],
                                  [0, 1], scale)
    _close(out[0, 0], beta * np.dot(k, scale * q) * v, TOL, "one token from zero state")


def pin_gdn_overwrite(gdn):
    """alpha = beta = 1 with one unit key written again and again: the delta
    rule replaces what the key retrieves, so S_t k = v_t after every token."""
    rng = np.random.Generator(np.random.PCG64(2))
    T, dk, dv = 7, 6, 4
    k1 = _unit(rng.standard_normal(dk))
    k = np.tile(k1, (T, 1, 1))
    v = rng.standard_normal((T, 1, dv))
    out, fin = gdn.gated_delta_rule(k, k, v, np.zeros((T, 1)), np.ones((T, 1)), [0, T], 1.0)
    _close(out[:, 0], v[:, 0], TOL, "retrieval of the latest value")
    _close(fin[0, 0], np.outer(v[-1, 0], k1), TOL, "state holds only the last value")


def pin_gdn_orthonormal_keys_linear_attention(gdn):
    """alpha = beta = 1 and orthonormal keys: no write interferes with another,
    so o_t = sum_{j <= t} (k_j . q'_t) v_j (causal linear attention)."""
    rng = np.random.Generator(np.random.PCG64(3))
    T, dk, dv, scale = 6, 8, 5, 0.4
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:T][:, None, :]
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    out, _ = gdn.gated_delta_rule(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), [0, T], scale)
    for t in range(T):
        want = sum(np.dot(k[j, 0], scale * q[t, 0]) * v[j, 0] for j in range(t + 1))
        _close(out[t, 0], want, TOL, f"linear attention row {t}")


def pin_gdn_zero_beta_decay_only(gdn):
    """beta = 0: nothing is written; the state only decays, S_t = exp(sum g) S0."""
    cu = [0, 9]
    q, k, v, g, _ = rand_inputs(cu, 2, 6, 4, seed=4)
    s0 = np.random.Generator(np.random.PCG64(5)).standard_normal((1, 2, 4, 6))
    scale = 0.9
    out, fin = gdn.gated_delta_rule(q, k, v, g, np.zeros_like(g), cu, scale, initial_state=s0)
    cg = np.cumsum(g, axis=0)
    for t in range(9):
        for h in range(2):
            _close(out[t, h], np.exp(cg[t, h]) * s0[0, h] @ (scale * q[t, h]), TOL,
                   f"decayed read t={t} h={h}")
    _close(fin[0], np.exp(cg[-1])[:, None, None] * s0[0], TOL, "decayed final state")


def pin_gdn_forget_gate_resets(gdn):
    """alpha = 0 at token r erases everything before it: outputs from r on equal
    a fresh run over tokens r.. (the earlier tokens and S0 do not matter)."""
    cu = [0, 12]
    q, k, v, g, beta = rand_inputs(cu, 1, 5, 3, seed=6)
    r = 5
    g[r, 0] = -1e4  # exp underflows to exactly 0
    s0 = np.random.Generator(np.random.PCG64(7)).standard_normal((1, 1, 3, 5))
    out, fin = gdn.gated_delta_rule(q, k, v, g, beta, cu, 1.0, initial_state=s0)
    g2 = g[r:].copy()
    g2[0, 0] = 0.0
    out2, fin2 = gdn.gated_delta_rule(q[r:], k[r:], v[r:], g2, beta[r:], [0, 12 - r], 1.0)
    _close(out[r:], out2, TOL, "outputs after the reset")
    _close(fin, fin2, TOL, "final state after the reset")


def pin_gdn_state_passing(gdn):
    """A sequence split in two: run the first part, hand its final state to the
    second part as initial state -- outputs and final state are unchanged."""
    cu = [0, 23]
    q, k, v, g, beta = rand_inputs(cu, 3, 6, 5, seed=8)
    s0 = np.random.Generator(np.random.PCG64(9)).standard_normal((1, 3, 5, 6))
    out, fin = gdn.gated_delta_rule(q, k, v, g, beta, cu, 0.5, initial_state=s0)
    for cut in (1, 9, 22):
        o1, f1 = gdn.gated_delta_rule(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], [0, cut],
                                      0.5, initial_state=s0)
        o2, f2 = gdn.gated_delta_rule(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:],
                                      [0, 23 - cut], 0.5, initial_state=f1)
        _close(np.concatenate([o1, o2]), out, TOL, f"outputs split at {cut}")
        _close(f2, fin, TOL, f"final state split at {cut}")


def pin_gdn_packed_equals_separate(gdn):
    """A packed batch (empty and one-token sequences included) equals separate
    calls; each sequence starts from its own initial state."""
    lens = [4, 0, 1, 9, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = rand_inputs(cu, 2, 4, 3, seed=10)
    s0 = np.random.Generator(np.random.PCG64(11)).standard_normal((len(lens), 2, 3, 4))
    out, fin = gdn.gated_delta_rule(q, k, v, g, beta, cu, 1.3, initial_state=s0)
    for b in range(len(lens)):
        a, e = cu[b], cu[b + 1]
        o, f = gdn.gated_delta_rule(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], [0, e - a], 1.3,
                                    initial_state=s0[b:b + 1])
        _close(out[a:e], o, TOL, f"sequence {b} outputs")
        _close(fin[b], f[0], TOL, f"sequence {b} final state")


def pin_gdn_linear_in_values_and_state(gdn):
    """For fixed q, k, g, beta the map (V, S0) -> (O, S_final) is linear."""
    cu = [0, 10]
    q, k, v1, g, beta = rand_inputs(cu, 2, 5, 4, seed=12)
    rng = np.random.Generator(np.random.PCG64(13))
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = rng.standard_normal((2, 1, 2, 4, 5))
    a, b = 0.75, -1.5
    o1, f1 = gdn.gated_delta_rule(q, k, v1, g, beta, cu, 1.0, initial_state=s1)
    o2, f2 = gdn.gated_delta_rule(q, k, v2, g, beta, cu, 1.0, initial_state=s2)
    o3, f3 = gdn.gated_delta_rule(q, k, a * v1 + b * v2, g, beta, cu, 1.0,
                                  initial_state=a * s1 + b * s2)
    _close(o3, a * o1 + b * o2, TOL, "outputs")
    _close(f3, a * f1 + b * f2, TOL, "final state")


def pin_gdn_dense_transitions(gdn):
    """Brute force on a tiny case: the state as products of explicit d x d
    transition matrices, S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) +
    beta_t v_t k_t^T, and every output S_t q'_t; keys not unit-norm, dk != dv."""
    rng = np.random.Generator(np.random.PCG64(14))
    T, H, dk, dv, scale = 6, 2, 4, 3, 0.8
    q = rng.standard_normal((T, H, dk))
    k = 0.7 * rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = np.log(rng.uniform(0.5, 1.0, (T, H)))
    beta = rng.uniform(0.0, 1.0, (T, H))
    s0 = rng.standard_normal((1, H, dv, dk))
    out, fin = gdn.gated_delta_rule(q, k, v, g, beta, [0, T], scale, initial_state=s0)
    for h in range(H):
        S = s0[0, h]
        for t in range(T):
            trans = np.exp(g[t, h]) * (np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h]))
            S = S @ trans + beta[t, h] * np.outer(v[t, h], k[t, h])
            _close(out[t, h], S @ (scale * q[t, h]), TOL, f"dense output t={t} h={h}")
        _close(fin[0, h], S, TOL, f"dense final state h={h}")


def chunked_wy(q, k, v, g, beta, cu, scale, chunk, initial_state=None):
    """The chunked form of the same recurrence (intra-/inter-chunk, WY
    representation), fp64, derived independently of the scan:
    within a chunk with cumulative log-gates gam_i and Gam_i = exp(gam_i),
      A_ij = beta_i exp(gam_i - gam_j) k_i . k_j  (i > j),  T = (I + A)^-1,
      W = T diag(beta Gam) K,  U = T diag(beta) V,  U' = U - W S^T,
      O = diag(Gam) Q' S^T + (Q' K^T o M) U',  M_ij = exp(gam_i - gam_j) (i >= j),
      S <- Gam_last S + U'^T diag(exp(gam_last - gam)) K."""
    T, H, dk = q.shape
    dv = v.shape[2]
    n = len(cu) - 1
    out = np.zeros((T, H, dv))
    fin = np.zeros((n, H, dv, dk))
    for b in range(n):
        for h in range(H):
            S = np.zeros((dv, dk)) if initial_state is None else initial_state[b, h].copy()
            for a in range(cu[b], cu[b + 1], chunk):
                e = min(a + chunk, cu[b + 1])
                K, V, Q = k[a:e, h], v[a:e, h], scale * q[a:e, h]
                bt = beta[a:e, h]
                gam = np.cumsum(g[a:e, h])
                G = np.exp(gam)
                L = np.tril(np.exp(gam[:, None] - gam[None, :]))
                A = np.tril(bt[:, None] * L * (K @ K.T), -1)
                Tm = np.linalg.solve(np.eye(e - a) + A, np.eye(e - a))
                W = Tm @ ((bt * G)[:, None] * K)
                U = Tm @ (bt[:, None] * V)
                Up = U - W @ S.T
                out[a:e, h] = G[:, None] * (Q @ S.T) + ((Q @ K.T) * L) @ Up
                S = G[-1] * S + Up.T @ (np.exp(gam[-1] - gam)[:, None] * K)
            fin[b, h] = S
    return out, fin


def pin_gdn_chunked_form(gdn):
    """The chunked intra-/inter-chunk form (the rewrite the pages describe)
    equals the scan for chunk lengths 1, 3, 16 and 64 on a ragged batch."""
    lens = [37, 5, 64, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = rand_inputs(cu, 2, 8, 6, seed=15)
    s0 = np.random.Generator(np.random.PCG64(16)).standard_normal((len(lens), 2, 6, 8))
    out, fin = gdn.gated_delta_rule(q, k, v, g, beta, cu, 0.35, initial_state=s0)
    for c in (1, 3, 16, 64):
        o, f = chunked_wy(q, k, v, g, beta, cu, 0.35, c, initial_state=s0)
        _close(o, out, 1e-9, f"chunked outputs, chunk {c}")
        _close(f, fin, 1e-9, f"chunked final state, chunk {c}")


ALL_PINS = [
    pin_gdn_single_token,
    pin_gdn_overwrite,
    pin_gdn_orthonormal_keys_linear_attention,
    pin_gdn_zero_beta_decay_only,
    pin_gdn_forget_gate_resets,
    pin_gdn_state_passing,
    pin_gdn_packed_equals_separate,
    pin_gdn_linear_in_values_and_state,
    pin_gdn_dense_transitions,
    pin_gdn_chunked_form,
]
