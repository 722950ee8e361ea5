"""Q6_K prefill products on the fp16 matrix cores (rows that are a whole
number of dwords long, from a 4-byte aligned W) against the f64 oracle: each
tile with a partial last super-block (odd steps start 2 bytes into a dword),
exact integer products at the extreme scales and codes, activations over a
wide dynamic range, the stated bound for an outlier on a zero sub-block
scale, and the rows that keep the fp32 matrix cores (an odd number of
super-blocks, or W not 4-byte aligned). Split and packed Q8_0 and Q5_0
get the same exact-integer check."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

Q6, Q8, SPLIT, Q50 = 14, 8, 1008, 6
SB = 210  # bytes of a Q6_K super-block: ql[128], qh[64], scales[16], d


def _run(gq, fmt, Wd, rows, cols, X):
    M = X.shape[0]
    Y = sentinel_buffer(M * rows)
    gq.gq_matmul(fmt, Wd, rows, cols, to_dev(X), Y=Y[:M * rows])
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[:M * rows].reshape(M, rows)


def _sample(rows, step):
    idx = np.unique(np.concatenate([np.arange(0, rows, step), [1, 15, 16, 127, 128, rows - 1]]))
    return idx[idx < rows]


@pytest.mark.parametrize("rows,M", [
    (14336, 512),   # 128 x 64 tiles
    (14336, 64),    # 128 x 32
    (14336, 16),    # 64 x 16 split in four along k
    (4096, 32),     # one wave per 32 weight rows
    (300, 20),      # one wave per 16 weight rows
])
def test_q6_each_tile_partial_last_super_block(gq, oracle, rows, M):
    """Rows of 4000 columns (16 super-blocks, the last one 160 columns) on
    each tile; the oracle on a sample of rows."""
    cols = 4000
    rng = synth.rng_for(630, rows + M)
    W = synth.weights(Q6, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[q6 matmul] tiles rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, Q6, to_dev(W), rows, cols, X)
    idx = _sample(rows, 97)
    Ws = oracle.select_rows(Q6, W, cols, idx)
    ref, S = oracle.matmul(Q6, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"q6 rows={rows} M={M}")


def _q6_unit_d_weights(rng, rows, cols):
    """Q6_K rows with d = 1, random codes and int8 scales that include
    -128, -127, -1, 0, 1 and 127 in every row."""
    nsb = cols // 256
    W = rng.integers(0, 256, size=(rows, nsb, SB), dtype=np.uint8)
    sc = rng.integers(-128, 128, size=(rows, nsb, 16)).astype(np.int8)
    sc[:, 0, :6] = np.array([-128, -127, -1, 0, 1, 127], np.int8)
    W[:, :, 192:208] = sc.view(np.uint8)
    W[:, :, 208:210] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    return W.reshape(-1)


def _q5_0_unit_d_weights(rng, rows, cols):
    """Q5_0 rows with d = 1 and random qh and nibbles (codes 0 .. 31)."""
    nb = cols // 32
    W = rng.integers(0, 256, size=(rows, nb, 22), dtype=np.uint8)
    W[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    W[:, 0, 2:6] = 0xFF            # block 0 of every row: all fifth bits set
    W[:, 0, 6:22] = 0xFF           # ... and every nibble 15: codes 31
    return W.reshape(-1)


def _q8_unit_d_weights(rng, rows, cols):
    nb = cols // 32
    W = rng.integers(0, 256, size=(rows, nb, 34), dtype=np.uint8)
    W[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    W[:, 0, 2:6] = np.array([-128, 127, -127, 0], np.int8).view(np.uint8)
    return W.reshape(-1)


@pytest.mark.parametrize("fmt", [Q6, Q8, SPLIT, Q50])
@pytest.mark.parametrize("rows,M", [(64, 32), (4096, 512)])
def test_fp16_route_exact_integer_products(gq, oracle, fmt, rows, M):
    """d = 1, codes and scales over their whole ranges (Q6_K: int8 scales
    down to -128, so sc (q - 32) spans -4096 .. 4096; Q8_0: codes -128 ..
    127; Q5_0: codes 0 .. 31) and activations in {-1, 0, 1}: every product
    and partial sum is an integer below 2^24, so Y must equal the exact sum
    bit for bit -- which holds only if the weight operands are exact."""
    cols = 512
    rng = synth.rng_for(631, fmt * 100000 + rows)
    base = {Q6: Q6, Q8: Q8, SPLIT: Q8, Q50: Q50}[fmt]
    make = {Q6: _q6_unit_d_weights, Q8: _q8_unit_d_weights, SPLIT: _q8_unit_d_weights,
            Q50: _q5_0_unit_d_weights}[fmt]
    W = make(rng, rows, cols)
    X = rng.integers(-1, 2, size=(M, cols)).astype(np.float32)
    Wd = to_dev(W)
    if fmt == SPLIT:
        Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
    print(f"[fp16 route] exact integers fmt={fmt} rows={rows} M={M}", flush=True)
    Y = _run(gq, fmt, Wd, rows, cols, X)
    Wf = oracle.dequant(base, W, rows, cols).astype(np.float64)
    assert np.array_equal(Wf, np.round(Wf)) and np.abs(Wf).max() <= 4096
    want = X.astype(np.float64) @ Wf.T
    assert np.abs(want).max() < 2 ** 24
    assert np.array_equal(Y.astype(np.float64), want)


def test_q6_wide_dynamic_range(gq, oracle):
    """Activations whose magnitudes span 2^-113 .. 2^100 across rows and
    super-blocks, each within 2^13 of the largest in its row's super-block,
    meet the plain bound."""
    rows, cols, M = 80, 1024, 40
    rng = synth.rng_for(632, 0)
    W = synth.weights(Q6, rows, cols, rng)
    scale = np.exp2(rng.integers(-100, 101, size=(M, cols // 256))).astype(np.float64)
    mag = np.exp2(rng.uniform(-13.0, 0.0, size=(M, cols)))
    sign = np.where(rng.random((M, cols)) < 0.5, -1.0, 1.0)
    X = (sign * mag * np.repeat(scale, 256, axis=1)).astype(np.float32)
    X[rng.random((M, cols)) < 0.05] = 0.0
    print("[q6 matmul] wide dynamic range", flush=True)
    Y = _run(gq, Q6, to_dev(W), rows, cols, X)
    ref, S = oracle.matmul(Q6, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, "q6 wide dynamic range")


def test_q6_outlier_on_zero_scale(gq, oracle):
    """Sub-block 0 of every row has scale 0 and one activation row holds 2^40
    there: that row's other activations of the super-block fall below 2^-14
    of its largest and are carried to an absolute 2^-34 * 2^40 only. That row
    stays within 2^-33 * 2^40 * sum_{c < 256} |w(r, c)|; the other rows, and
    that row's second super-block, meet the plain bound."""
    rows, cols, M, hot = 64, 512, 20, 7
    rng = synth.rng_for(633, 0)
    W = synth.weights(Q6, rows, cols, rng).copy()
    W.reshape(rows, 2 * SB)[:, 192] = 0          # scale of sub-block 0
    X = synth.activations((M, cols), rng)
    X[hot, 0] = np.float32(2.0 ** 40)
    print("[q6 matmul] outlier", flush=True)
    Wd = to_dev(W)
    Y = _run(gq, Q6, Wd, rows, cols, X)
    ref, S = oracle.matmul(Q6, W, rows, cols, X, nthreads=oracle_threads())
    others = np.arange(M) != hot
    assert_within_tolerance(Y[others], ref[others], S[others], "rows without the outlier")
    w0 = np.abs(oracle.dequant(Q6, W, rows, cols)[:, :256].astype(np.float64)).sum(axis=1)
    err = np.abs(Y[hot].astype(np.float64) - ref[hot])
    assert (err <= 2e-4 * S[hot] + 2.0 ** -33 * 2.0 ** 40 * w0).all()
    X1 = X.copy()
    X1[:, :256] = 0.0
    Y1 = _run(gq, Q6, Wd, rows, cols, X1)
    ref1, S1 = oracle.matmul(Q6, W, rows, cols, X1, nthreads=oracle_threads())
    assert_within_tolerance(Y1, ref1, S1, "outlier's other super-block")


@pytest.mark.parametrize("cols,offset", [(768, 0), (1024, 2)])
def test_q6_rows_off_the_dword_grid(gq, oracle, cols, offset):
    """Rows of an odd number of super-blocks (every other row starts 2 bytes
    into a dword), and W starting 2 bytes into a dword: the fp32 matrix cores
    take these; every output meets the oracle's bound."""
    import torch
    rows, M = 300, 48
    rng = synth.rng_for(634, cols + offset)
    W = synth.weights(Q6, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    buf = torch.zeros(W.size + 64, dtype=torch.uint8, device="cuda")
    buf[offset:offset + W.size].copy_(to_dev(W))
    print(f"[q6 matmul] off the dword grid cols={cols} W offset={offset}", flush=True)
    Y = _run(gq, Q6, buf[offset:offset + W.size], rows, cols, X)
    ref, S = oracle.matmul(Q6, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"q6 off the dword grid cols={cols} offset={offset}")
