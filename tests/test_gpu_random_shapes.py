"""Seeded random shapes on the GPU against the f64 oracle: every format,
rows and columns drawn across block boundaries and ragged tails, and the
entry points that take them (gq_matvec, gq_matvec_acc, gq_matvec_batch,
gq_matmul, gq_dequant). Products must lie within 2e-4 * sum |w x| of the
oracle, dequant must equal it bit for bit, the batched rows must equal the
lone matvec bit for bit, and no kernel may write past its output."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

FORMATS = (8, 12, 6, 13, 14, 1008)
N_CASES = 160


def _case(i):
    rng = np.random.default_rng([2026, i])
    fmt = FORMATS[i % len(FORMATS)]
    qk = 256 if fmt in (12, 13, 14) else 32
    # columns: a whole number of blocks, a ragged tail, or a single block
    nb = int(rng.integers(1, 40 if qk == 256 else 300))
    cols = nb * qk - int(rng.integers(0, qk)) if rng.random() < 0.5 else nb * qk
    rows = int(rng.choice([1, 2, 3, 5, 63, 64, 65, 127, 300, 1000, 2049]))
    M = int(rng.choice([1, 2, 3, 5, 15, 16, 17, 40]))
    return fmt, rows, max(1, cols), M, rng


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(gq, oracle, i):
    fmt, rows, cols, M, rng = _case(i)
    base = 8 if fmt == 1008 else fmt
    print(f"[random {i}] fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    W = synth.weights(base, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    Wd, Xd = to_dev(W), to_dev(X)
    if fmt == 1008:
        Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
    ref, S = oracle.matmul(base, W, rows, cols, X, nthreads=oracle_threads())

    # matvec of the first activation row, then accumulate the second onto it
    y = sentinel_buffer(rows)
    gq.gq_matvec(fmt, Wd, rows, cols, Xd[0], y=y[:rows])
    assert_pad_untouched(y, rows)
    y0 = to_host(y)[:rows].copy()
    assert_within_tolerance(y0, ref[0], S[0], "matvec")
    if M >= 2:
        gq.gq_matvec_acc(fmt, Wd, rows, cols, Xd[1], y[:rows])
        acc = to_host(y)[:rows]
        assert np.array_equal(acc.view(np.uint32),
                              (y0 + to_host(gq.gq_matvec(fmt, Wd, rows, cols, Xd[1]))).view(np.uint32))

    # all rows: the batched matvec (bit-identical rows) and gq_matmul (tolerance)
    Yb = sentinel_buffer(M * rows)
    gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd, Y=Yb[:M * rows])
    assert_pad_untouched(Yb, M * rows)
    yb = to_host(Yb)[:M * rows].reshape(M, rows)
    assert np.array_equal(yb[0].view(np.uint32), y0.view(np.uint32))
    Ym = sentinel_buffer(M * rows)
    gq.gq_matmul(fmt, Wd, rows, cols, Xd, Y=Ym[:M * rows])
    assert_pad_untouched(Ym, M * rows)
    assert_within_tolerance(to_host(Ym)[:M * rows].reshape(M, rows), ref, S, "matmul")

    # dequant, bit-exact
    out = sentinel_buffer(rows * cols)
    gq.gq_dequant(fmt, Wd, rows, cols, out=out[:rows * cols])
    assert_pad_untouched(out, rows * cols)
    got = to_host(out)[:rows * cols].reshape(rows, cols)
    assert np.array_equal(got.view(np.uint32), oracle.dequant(base, W, rows, cols).view(np.uint32))
