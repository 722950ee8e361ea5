"""Pins for the oracle's f64 products.

y[r] = sum_c w(r,c) x[c] with W[out,in] row-major ("nurllama 0.18.1 API",
kernels.nu section, layout contract). Pinned by exact rational brute force
on one- and two-block matrices (non-square, so a transposed operand fails),
by invariants (pooled rows bit-identical to serial, scaling by 2^k, row
permutation) and by the matmul/matvec agreement.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth


def _exact(w_row: np.ndarray, x: np.ndarray) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(w_row, x)),
               Fraction(0))


@pytest.mark.parametrize("fmt,rows,cols", [
    (8, 1, 32), (8, 2, 64), (8, 3, 40), (12, 1, 256), (12, 2, 512), (12, 3, 300),
    (6, 2, 64), (6, 3, 40), (13, 2, 512), (13, 3, 300), (14, 2, 512), (14, 3, 300),
])
def test_brute_force_rational(oracle, fmt, rows, cols):
    rng = np.random.default_rng(fmt * 100 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    w = oracle.dequant(fmt, W, rows, cols)
    y, S = oracle.matvec(fmt, W, rows, cols, x)
    for r in range(rows):
        exact = _exact(w[r], x)
        sabs = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(w[r], x))
        # sequential f64 summation of exact products: |err| <= (n-1) u S
        bound = Fraction(cols - 1) * Fraction(2.0 ** -53) * sabs
        assert abs(Fraction(float(y[r])) - exact) <= bound
        assert abs(Fraction(float(S[r])) - sabs) <= bound
    # a transposed or mis-strided operand would not produce these rows
    assert y.shape == (rows,)


def test_hand_computed_dot(oracle):
    # Q8_0, d = 0.5, q = 1..32, x = 1 everywhere except x[0] = -2:
    # y = 0.5 * (sum_{q=1..32} q - 3 * 1) = 0.5 * (528 - 3) = 262.5
    b = np.zeros(34, np.uint8)
    b[0], b[1] = 0x00, 0x38
    b[2:] = np.arange(1, 33, dtype=np.uint8)
    x = np.ones(32, np.float32)
    x[0] = -2.0
    y, S = oracle.matvec(8, b, 1, 32, x)
    assert y[0] == 262.5
    assert S[0] == 0.5 * (528 - 1 + 2)


def test_threads_bit_identical_and_matmul_rows(oracle):
    rng = np.random.default_rng(3)
    rows, cols, M = 37, 768, 3
    W = synth.weights(12, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    Y1, S1 = oracle.matmul(12, W, rows, cols, X, nthreads=1)
    Y4, S4 = oracle.matmul(12, W, rows, cols, X, nthreads=4)
    assert np.array_equal(Y1, Y4) and np.array_equal(S1, S4)
    for m in range(M):
        y, s = oracle.matvec(12, W, rows, cols, X[m])
        assert np.array_equal(y, Y1[m]) and np.array_equal(s, S1[m])


def test_scaling_and_permutation_invariants(oracle):
    rng = np.random.default_rng(4)
    rows, cols = 20, 96
    W = synth.weights(8, rows, cols, rng)
    x = synth.activations(cols, rng)
    y, S = oracle.matvec(8, W, rows, cols, x)
    y8, S8 = oracle.matvec(8, W, rows, cols, x * np.float32(8.0))
    assert np.array_equal(y8, 8.0 * y) and np.array_equal(S8, 8.0 * S)
    perm = rng.permutation(rows)
    Wp = W.reshape(rows, -1)[perm].reshape(-1)
    yp, _ = oracle.matvec(8, Wp, rows, cols, x)
    assert np.array_equal(yp, y[perm])
    assert np.all(S >= np.abs(y))


def test_select_rows(oracle):
    rng = np.random.default_rng(6)
    rows, cols = 9, 512
    W = synth.weights(12, rows, cols, rng)
    x = synth.activations(cols, rng)
    y, _ = oracle.matvec(12, W, rows, cols, x)
    idx = [8, 0, 4]
    ys, _ = oracle.matvec(12, oracle.select_rows(12, W, cols, idx), 3, cols, x)
    assert np.array_equal(ys, y[idx])
