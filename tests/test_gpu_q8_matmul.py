"""Q8_0 prefill products on the fp16 matrix cores -- packed rows that are a
whole number of dwords long, and the split per-row layout -- against the f64
oracle: each tile with a partial last 256-column step, blocks past a row's
end whose bytes (the next row's) hold an infinite scale, activations over a
wide dynamic range, the stated bound for an outlier on zero codes, and the
packed rows that keep the fp32 matrix cores (an odd number of blocks, or W
not 4-byte aligned)."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

Q8, SPLIT = 8, 1008


def _weights(gq, fmt, W, rows, cols):
    Wd = to_dev(W)
    return Wd if fmt == Q8 else gq.gq_q8_0_split_repack(Wd, rows, cols)


def _run(gq, fmt, Wd, rows, cols, X):
    M = X.shape[0]
    Y = sentinel_buffer(M * rows)
    gq.gq_matmul(fmt, Wd, rows, cols, to_dev(X), Y=Y[:M * rows])
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[:M * rows].reshape(M, rows)


def _sample(rows, step):
    idx = np.unique(np.concatenate([np.arange(0, rows, step), [1, 15, 16, 127, 128, rows - 1]]))
    return idx[idx < rows]


@pytest.mark.parametrize("fmt", [Q8, SPLIT])
@pytest.mark.parametrize("rows,M", [
    (14336, 512),   # split: 128 x 64 tiles; packed: 128 x 32
    (14336, 64),    # split: 128 x 32 split in two along k; packed: 128 x 32
    (14336, 16),    # 64 x 16 split in four (split) or two (packed)
    (4096, 32),     # one wave per 32 weight rows
    (300, 20),      # one wave per 16 weight rows
])
def test_q8_each_tile_partial_last_step(gq, oracle, fmt, rows, M):
    """Rows of 3968 columns (124 blocks: the last 256-column step holds 4 of
    its 8 blocks) on each tile; the oracle on a sample of rows."""
    cols = 3968
    rng = synth.rng_for(620, fmt * 100000 + rows + M)
    W = synth.weights(Q8, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[q8 matmul] tiles fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, fmt, _weights(gq, fmt, W, rows, cols), rows, cols, X)
    assert np.isfinite(Y).all()
    idx = _sample(rows, 97)
    Ws = oracle.select_rows(Q8, W, cols, idx)
    ref, S = oracle.matmul(Q8, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"q8 fmt={fmt} rows={rows} M={M}")


@pytest.mark.parametrize("fmt", [Q8, SPLIT])
@pytest.mark.parametrize("rows,M", [(64, 20), (14336, 64)])
def test_q8_blocks_past_the_row_end(gq, oracle, fmt, rows, M):
    """Block 0 of every odd row has an infinite scale. In the packed layout
    the blocks that would follow an even row's last one are the next row's
    first blocks, so the last step reads that scale; it must not reach the
    even row (whose outputs meet the oracle's bound)."""
    cols = 3968
    rng = synth.rng_for(621, fmt * 100000 + rows)
    W = synth.weights(Q8, rows, cols, rng).copy()
    rb = gq.gq_row_bytes(Q8, cols)
    Wr = W.reshape(rows, rb)
    Wr[1::2, 0:2] = np.frombuffer(np.float16(np.inf).tobytes(), np.uint8)
    X = synth.activations((M, cols), rng)
    print(f"[q8 matmul] past the row end fmt={fmt} rows={rows} M={M}", flush=True)
    Y = _run(gq, fmt, _weights(gq, fmt, W, rows, cols), rows, cols, X)
    idx = _sample(rows, 97)
    idx = idx[idx % 2 == 0]
    Ws = oracle.select_rows(Q8, W, cols, idx)
    ref, S = oracle.matmul(Q8, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"q8 past the row end fmt={fmt}")


@pytest.mark.parametrize("fmt", [Q8, SPLIT])
def test_q8_wide_dynamic_range(gq, oracle, fmt):
    """Activations whose magnitudes span 2^-113 .. 2^100 across rows and
    256-column steps, each within 2^13 of the largest in its row's step, meet
    the plain bound."""
    rows, cols, M = 80, 1024, 40
    rng = synth.rng_for(622, fmt)
    W = synth.weights(Q8, rows, cols, rng)
    scale = np.exp2(rng.integers(-100, 101, size=(M, cols // 256))).astype(np.float64)
    mag = np.exp2(rng.uniform(-13.0, 0.0, size=(M, cols)))
    sign = np.where(rng.random((M, cols)) < 0.5, -1.0, 1.0)
    X = (sign * mag * np.repeat(scale, 256, axis=1)).astype(np.float32)
    X[rng.random((M, cols)) < 0.05] = 0.0
    print(f"[q8 matmul] wide dynamic range fmt={fmt}", flush=True)
    Y = _run(gq, fmt, _weights(gq, fmt, W, rows, cols), rows, cols, X)
    ref, S = oracle.matmul(Q8, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"q8 wide dynamic range fmt={fmt}")


@pytest.mark.parametrize("fmt", [Q8, SPLIT])
def test_q8_outlier_on_zero_codes(gq, oracle, fmt):
    """Block 0 of every row has all codes zero and one activation row holds
    2^40 there: that row's other activations of the step fall below 2^-14 of
    its largest and are carried to an absolute 2^-34 * 2^40 only. That row
    stays within the stated extra term 2^-33 * 2^40 * sum_{c < 256} |w(r, c)|;
    the other rows, and that row's second step, meet the plain bound."""
    rows, cols, M, hot = 64, 512, 20, 7
    rng = synth.rng_for(623, fmt)
    W = synth.weights(Q8, rows, cols, rng).copy()
    rb = gq.gq_row_bytes(Q8, cols)
    W.reshape(rows, rb)[:, 2:34] = 0          # codes of block 0
    X = synth.activations((M, cols), rng)
    X[hot, 0] = np.float32(2.0 ** 40)
    print(f"[q8 matmul] outlier fmt={fmt}", flush=True)
    Wd = _weights(gq, fmt, W, rows, cols)
    Y = _run(gq, fmt, Wd, rows, cols, X)
    ref, S = oracle.matmul(Q8, W, rows, cols, X, nthreads=oracle_threads())
    others = np.arange(M) != hot
    assert_within_tolerance(Y[others], ref[others], S[others], "rows without the outlier")
    w0 = np.abs(oracle.dequant(Q8, W, rows, cols)[:, :256].astype(np.float64)).sum(axis=1)
    extra = 2.0 ** -33 * 2.0 ** 40 * w0
    err = np.abs(Y[hot].astype(np.float64) - ref[hot])
    assert (err <= 2e-4 * S[hot] + extra).all()
    X1 = X.copy()
    X1[:, :256] = 0.0
    Y1 = _run(gq, fmt, Wd, rows, cols, X1)
    ref1, S1 = oracle.matmul(Q8, W, rows, cols, X1, nthreads=oracle_threads())
    assert_within_tolerance(Y1, ref1, S1, "outlier's other step")


@pytest.mark.parametrize("cols,offset", [(4000, 0), (1024, 2)])
def test_q8_packed_rows_off_the_dword_grid(gq, oracle, cols, offset):
    """Packed rows of an odd number of blocks (2 bytes past a dword boundary
    every other row), and W starting 2 bytes into a dword: the fp32 matrix
    cores take these; every output meets the oracle's bound."""
    import torch
    rows, M = 300, 48
    rng = synth.rng_for(624, cols + offset)
    W = synth.weights(Q8, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    buf = torch.zeros(W.size + 64, dtype=torch.uint8, device="cuda")
    buf[offset:offset + W.size].copy_(to_dev(W))
    print(f"[q8 matmul] off the dword grid cols={cols} W offset={offset}", flush=True)
    Y = _run(gq, Q8, buf[offset:offset + W.size], rows, cols, X)
    ref, S = oracle.matmul(Q8, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"q8 off the dword grid cols={cols} offset={offset}")


def test_q8_packed_and_split_agree(gq, oracle):
    """The two layouts of one matrix on a grid that both give to the per-wave
    kernel (only the loads differ): the same bits, within the oracle's bound,
    and the same bits again on a repeated call."""
    rows, cols, M = 300, 1024, 24
    rng = synth.rng_for(625, 0)
    W = synth.weights(Q8, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print("[q8 matmul] packed vs split", flush=True)
    Yp = _run(gq, Q8, _weights(gq, Q8, W, rows, cols), rows, cols, X)
    Sd = _weights(gq, SPLIT, W, rows, cols)
    Ys = _run(gq, SPLIT, Sd, rows, cols, X)
    ref, S = oracle.matmul(Q8, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Yp, ref, S, "packed")
    assert np.array_equal(Yp.view(np.uint32), Ys.view(np.uint32))
    assert np.array_equal(Ys.view(np.uint32), _run(gq, SPLIT, Sd, rows, cols, X).view(np.uint32))
