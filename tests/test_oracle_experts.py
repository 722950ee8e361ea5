"""Pins for the oracle's expert-batched matvec: expert selection, the
input-row mapping a / xk, and invalid ids, on hand-built Q8_0 experts whose
outputs are known exactly."""
import numpy as np

import synth


def _blk(d16, q):
    b = np.zeros(34, np.uint8)
    b[0], b[1] = d16 & 0xFF, d16 >> 8
    b[2:] = np.array(q, np.int8).view(np.uint8)
    return b


def test_expert_selection_and_input_rows(oracle):
    # 3 experts, 2 rows, 32 columns; expert e's row r has d = 1 and every
    # code = 10 * e + r + 1, so w . x = (10 e + r + 1) * sum(x)
    rows, cols, n_expert = 2, 32, 3
    W = np.concatenate([_blk(0x3C00, 10 * e + r + 1) for e in range(n_expert) for r in range(rows)])
    X = np.stack([np.full(cols, 1.0 / 32, np.float32), np.full(cols, 2.0 / 32, np.float32)])
    xk = 2
    expid = [2, 0, 1, 2]          # positions 0, 0, 1, 1
    Y, S = oracle.experts_matvec(8, W, n_expert, rows, cols, X, xk, expid)
    want = [[21, 22], [1, 2], [2 * 11, 2 * 12], [2 * 21, 2 * 22]]
    assert Y.tolist() == want and S.tolist() == want


def test_invalid_ids_give_nan_rows(oracle):
    rows, cols, n_expert = 2, 32, 2
    W = np.concatenate([_blk(0x3C00, 1) for _ in range(n_expert * rows)])
    X = np.ones((4, cols), np.float32)
    Y, _ = oracle.experts_matvec(8, W, n_expert, rows, cols, X, 1, [1, -1, 2, 0])
    assert np.isnan(Y[1]).all() and np.isnan(Y[2]).all()
    assert Y[0].tolist() == [32.0, 32.0] and Y[3].tolist() == [32.0, 32.0]


def test_equals_per_assignment_matvec(oracle):
    rng = synth.rng_for(40, 0)
    rows, cols, n_expert, xk = 9, 512, 5, 3
    W = synth.weights(12, n_expert * rows, cols, rng)
    X = synth.activations((4, cols), rng)
    expid = rng.integers(0, n_expert, 12)
    Y, S = oracle.experts_matvec(12, W, n_expert, rows, cols, X, xk, expid)
    rb = oracle.row_bytes(12, cols)
    for a, e in enumerate(expid):
        y, s = oracle.matvec(12, W[e * rows * rb:(e + 1) * rows * rb], rows, cols, X[a // xk])
        assert np.array_equal(Y[a], y) and np.array_equal(S[a], s)
