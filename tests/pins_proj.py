"""Pins of the projection oracle (oracle/proj.py): values derived by hand,
a brute-force loop, and what the per-row scale and y = x w^T fix."""
import numpy as np

TOL = 1e-12


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
    if not err <= tol:
        raise AssertionError(f"{what}: max abs error {err:.3e} > {tol:.1e}")


def pin_dequantize_by_hand(proj):
    q = np.array([[1, -2, 0], [127, -128, 3]], dtype=np.int8)
    scale = np.array([0.5, 3.0], dtype=np.float32)
    _close(proj.dequantize(q, scale), [[0.5, -1.0, 0.0], [381.0, -384.0, 9.0]], 0.0, "dequantize")


def pin_dequantize_bf16_rounding(proj):
    """bf16 keeps 8 significant bits (nearest, ties to even):
    1 + 2^-8 is a tie between 1 and 1 + 2^-7 and goes to 1 (even);
    3 (1 + 2^-8) = 3.01171875 lies past the midpoint 3.0078125 of 3 and
    3.015625 and goes up; 127 (1 + 2^-7) = 127.9921875 rounds to 128 (spacing
    0.5 below 128); 128.5 is a tie between 128 and 129 and goes to 128."""
    q = np.array([[1, 3], [127, 0], [1, -1]], dtype=np.int8)
    scale = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -7, 128.5], dtype=np.float32)
    want = [[1.0, 3.015625], [128.0, 0.0], [128.0, -128.0]]
    _close(proj.dequantize_bf16(q, scale), want, 0.0, "bf16 rounding")


def pin_linear_bruteforce(proj):
    rng = np.random.Generator(np.random.PCG64(1))
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    want = np.zeros((3, 4))
    for t in range(3):
        for n in range(4):
            for k in range(5):
                want[t, n] += x[t, k] * w[n, k]
    _close(proj.linear(x, w), want, TOL, "y = x w^T")


def pin_linear_identity_and_permutation(proj):
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.standard_normal((6, 4))
    _close(proj.linear(x, np.eye(4)), x, 0.0, "identity weights")
    perm = np.array([2, 0, 3, 1])
    _close(proj.linear(x, np.eye(4)[perm]), x[:, perm], 0.0, "permutation weights")


def pin_scale_is_per_output_row(proj):
    """All-ones int8 weights: y[t][n] = scale[n] * sum_k x[t][k] (N != K)."""
    rng = np.random.Generator(np.random.PCG64(3))
    x = rng.standard_normal((5, 7))
    scale = np.array([0.25, -2.0, 3.5], dtype=np.float32)
    y = proj.linear(x, proj.dequantize(np.ones((3, 7), dtype=np.int8), scale))
    _close(y, x.sum(axis=1)[:, None] * scale.astype(np.float64)[None, :], TOL, "per-row scale")


ALL_PINS = [pin_dequantize_by_hand, pin_dequantize_bf16_rounding, pin_linear_bruteforce,
            pin_linear_identity_and_permutation, pin_scale_is_per_output_row]
