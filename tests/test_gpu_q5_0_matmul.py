"""Q5_0 prefill products on the fp16 matrix cores (rows of an even number of
blocks, from a 4-byte aligned W) against the f64 oracle: each tile with a
partial last 256-column step (odd blocks start 2 bytes into a dword), blocks
past a row's end whose bytes (the next row's) hold an infinite scale,
activations over a wide dynamic range, the stated bound for an outlier on a
zero-scale block, and the rows that keep the fp32 matrix cores (an odd
number of blocks, or W not 4-byte aligned). The exact-integer check of the
operands is in test_gpu_q6_matmul.py."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

Q50 = 6
BB = 22  # bytes of a Q5_0 block: d, qh (4 bytes), 16 nibble bytes


def _run(gq, Wd, rows, cols, X):
    M = X.shape[0]
    Y = sentinel_buffer(M * rows)
    gq.gq_matmul(Q50, Wd, rows, cols, to_dev(X), Y=Y[:M * rows])
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[:M * rows].reshape(M, rows)


def _sample(rows, step):
    idx = np.unique(np.concatenate([np.arange(0, rows, step), [1, 15, 16, 127, 128, rows - 1]]))
    return idx[idx < rows]


@pytest.mark.parametrize("rows,M", [
    (14336, 64),    # 128 x 32 tiles
    (14336, 16),    # 64 x 16 split in two along k
    (4096, 32),     # one wave per 32 weight rows
    (300, 20),      # one wave per 16 weight rows
    (4864, 512),    # the Qwen2.5-0.5B FFN shape below, 128 x 32 tiles
])
def test_q5_0_each_tile_partial_last_step(gq, oracle, rows, M):
    """Rows of 3968 columns (124 blocks: the last 256-column step holds 4 of
    its 8 blocks), or the 896-wide Qwen2.5-0.5B rows (28 blocks), on each
    tile; the oracle on a sample of rows."""
    cols = 896 if rows == 4864 else 3968
    rng = synth.rng_for(640, rows + M)
    W = synth.weights(Q50, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[q5_0 matmul] tiles rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, to_dev(W), rows, cols, X)
    idx = _sample(rows, 97)
    Ws = oracle.select_rows(Q50, W, cols, idx)
    ref, S = oracle.matmul(Q50, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"q5_0 rows={rows} M={M}")


@pytest.mark.parametrize("rows,M", [(64, 20), (14336, 64)])
def test_q5_0_blocks_past_the_row_end(gq, oracle, rows, M):
    """Block 0 of every odd row has an infinite scale; an even row's last
    step reads those bytes as its missing blocks, which must not reach it."""
    cols = 3968
    rng = synth.rng_for(641, rows)
    W = synth.weights(Q50, rows, cols, rng).copy()
    rb = gq.gq_row_bytes(Q50, cols)
    W.reshape(rows, rb)[1::2, 0:2] = np.frombuffer(np.float16(np.inf).tobytes(), np.uint8)
    X = synth.activations((M, cols), rng)
    print(f"[q5_0 matmul] past the row end rows={rows} M={M}", flush=True)
    Y = _run(gq, to_dev(W), rows, cols, X)
    idx = _sample(rows, 97)
    idx = idx[idx % 2 == 0]
    Ws = oracle.select_rows(Q50, W, cols, idx)
    ref, S = oracle.matmul(Q50, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, "q5_0 past the row end")


def test_q5_0_wide_dynamic_range(gq, oracle):
    """Activations whose magnitudes span 2^-113 .. 2^100 across rows and
    256-column steps, each within 2^13 of the largest in its row's step, meet
    the plain bound."""
    rows, cols, M = 80, 1024, 40
    rng = synth.rng_for(642, 0)
    W = synth.weights(Q50, rows, cols, rng)
    scale = np.exp2(rng.integers(-100, 101, size=(M, cols // 256))).astype(np.float64)
    mag = np.exp2(rng.uniform(-13.0, 0.0, size=(M, cols)))
    sign = np.where(rng.random((M, cols)) < 0.5, -1.0, 1.0)
    X = (sign * mag * np.repeat(scale, 256, axis=1)).astype(np.float32)
    X[rng.random((M, cols)) < 0.05] = 0.0
    print("[q5_0 matmul] wide dynamic range", flush=True)
    Y = _run(gq, to_dev(W), rows, cols, X)
    ref, S = oracle.matmul(Q50, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, "q5_0 wide dynamic range")


def test_q5_0_outlier_on_zero_scale(gq, oracle):
    """Block 0 of every row has d = 0 and one activation row holds 2^40 there:
    that row stays within 2^-33 * 2^40 * sum_{c < 256} |w(r, c)|; the other
    rows, and that row's second step, meet the plain bound."""
    rows, cols, M, hot = 64, 512, 20, 7
    rng = synth.rng_for(643, 0)
    W = synth.weights(Q50, rows, cols, rng).copy()
    W.reshape(rows, 16 * BB)[:, 0:2] = 0          # d of block 0
    X = synth.activations((M, cols), rng)
    X[hot, 0] = np.float32(2.0 ** 40)
    print("[q5_0 matmul] outlier", flush=True)
    Wd = to_dev(W)
    Y = _run(gq, Wd, rows, cols, X)
    ref, S = oracle.matmul(Q50, W, rows, cols, X, nthreads=oracle_threads())
    others = np.arange(M) != hot
    assert_within_tolerance(Y[others], ref[others], S[others], "rows without the outlier")
    w0 = np.abs(oracle.dequant(Q50, W, rows, cols)[:, :256].astype(np.float64)).sum(axis=1)
    err = np.abs(Y[hot].astype(np.float64) - ref[hot])
    assert (err <= 2e-4 * S[hot] + 2.0 ** -33 * 2.0 ** 40 * w0).all()
    X1 = X.copy()
    X1[:, :256] = 0.0
    Y1 = _run(gq, Wd, rows, cols, X1)
    ref1, S1 = oracle.matmul(Q50, W, rows, cols, X1, nthreads=oracle_threads())
    assert_within_tolerance(Y1, ref1, S1, "outlier's other step")


@pytest.mark.parametrize("cols,offset", [(1056, 0), (1024, 2)])
def test_q5_0_rows_off_the_dword_grid(gq, oracle, cols, offset):
    """Rows of an odd number of blocks, and W starting 2 bytes into a dword:
    the fp32 matrix cores take these; every output meets the oracle's bound."""
    import torch
    rows, M = 300, 48
    rng = synth.rng_for(644, cols + offset)
    W = synth.weights(Q50, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    buf = torch.zeros(W.size + 64, dtype=torch.uint8, device="cuda")
    buf[offset:offset + W.size].copy_(to_dev(W))
    print(f"[q5_0 matmul] off the dword grid cols={cols} W offset={offset}", flush=True)
    Y = _run(gq, buf[offset:offset + W.size], rows, cols, X)
    ref, S = oracle.matmul(Q50, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"q5_0 off the dword grid cols={cols} offset={offset}")
