"""gq_matmul on the GPU against the f64 oracle: the M sweep across the
small-M / matrix-core threshold, the Llama-3-8B prefill shapes at
M = 16, 64, 512, and edge cases."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _run(gq, fmt, W, rows, cols, X):
    M = X.shape[0]
    Y = sentinel_buffer(M * rows)
    Xd = to_dev(X) if isinstance(X, np.ndarray) else X
    gq.gq_matmul(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols, Xd, Y=Y)
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[: M * rows].reshape(M, rows)


def _check(gq, oracle, fmt, W, rows, cols, X, what):
    print(f"[matmul] {what} fmt={fmt} rows={rows} cols={cols} M={X.shape[0]}", flush=True)
    Y = _run(gq, fmt, W, rows, cols, X)
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    return assert_within_tolerance(Y, ref, S, what)


@pytest.mark.parametrize("M", list(range(1, 18)) + [31, 63, 64, 65, 512])
@pytest.mark.parametrize("fmt,rows,cols", [(12, 300, 896), (8, 200, 576), (12, 130, 4096)])
def test_m_sweep(gq, oracle, fmt, rows, cols, M):
    rng = synth.rng_for(500, rows)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), synth.rng_for(501, M))
    _check(gq, oracle, fmt, W, rows, cols, X, "m-sweep")


@pytest.mark.parametrize("which", ["gate", "down"])
@pytest.mark.parametrize("M", [16, 64, 512])
def test_llama3_8b_prefill(gq, oracle, which, M):
    """Llama-3-8B prefill shapes at full size: every output (all rows, all M)
    against the oracle."""
    W, X, rows, cols = synth.prefill_inputs(which, M)
    print(f"[matmul] llama3-8b prefill {which} M={M} (full check)", flush=True)
    Y = _run(gq, 12, W, rows, cols, X)
    ref, S = oracle.matmul(12, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"prefill {which} M={M}")


@pytest.mark.parametrize("fmt,rows,cols,M", [
    (12, 1, 256, 16), (12, 65, 300, 17), (8, 63, 70, 20), (8, 5, 33, 3), (12, 4, 1, 16),
    (12, 64, 1024, 64), (8, 17, 40000, 2), (12, 3, 33024, 5),
])
def test_edge_shapes(gq, oracle, fmt, rows, cols, M):
    rng = synth.rng_for(600, rows * 1000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    _check(gq, oracle, fmt, W, rows, cols, X, "edge")


def test_rows_agree_with_matvec_and_empty(gq, oracle):
    import torch
    rows, cols, M = 100, 512, 20
    W = synth.weights(12, rows, cols, synth.rng_for(700, 1))
    X = synth.activations((M, cols), synth.rng_for(700, 2))
    Wd = to_dev(W)
    Y = _run(gq, 12, Wd, rows, cols, X)
    ref, S = oracle.matmul(12, W, rows, cols, X)
    assert_within_tolerance(Y, ref, S, "matmul")
    # determinism
    assert np.array_equal(_run(gq, 12, Wd, rows, cols, X).view(np.uint32), Y.view(np.uint32))
    # M == 0 and rows == 0 are empty products
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    gq.gq_matmul(12, Wd, rows, cols, torch.empty((0, cols), device="cuda"), Y=e)
    gq.gq_matmul(12, Wd, 0, cols, to_dev(X), Y=e)


@pytest.mark.parametrize("fmt,rows,cols,M", [
    (12, 4096, 4096, 4), (12, 896, 896, 15), (8, 4096, 4096, 7), (14, 2048, 768, 3),
    (13, 300, 4096, 2), (6, 4864, 896, 9),
])
def test_few_rows_round_like_matvec(gq, fmt, rows, cols, M):
    """Few activation rows over a small product are the batched matvec: every
    row of Y equals gq_matvec of its activation row bit for bit."""
    rng = synth.rng_for(610, fmt * 100000 + rows + M)
    W = to_dev(synth.weights(fmt, rows, cols, rng))
    X = to_dev(synth.activations((M, cols), rng))
    print(f"[matmul] few rows fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = to_host(gq.gq_matmul(fmt, W, rows, cols, X))
    for m in range(M):
        y = to_host(gq.gq_matvec(fmt, W, rows, cols, X[m]))
        assert np.array_equal(y.view(np.uint32), Y[m].view(np.uint32)), m


@pytest.mark.parametrize("fmt,rows,cols,M", [
    (12, 14336, 4096, 5),     # Q4_K past the batched-matvec bound: fp16 matrix cores
    (8, 151936, 896, 2),      # Q8_0 lm_head, two rows: the fp32 few-row kernel
    (14, 4096, 14336, 5),     # Q6_K: fp16 matrix cores
    (13, 14336, 4096, 3),     # Q5_K past the batched-matvec bound: fp16 matrix cores
])
def test_few_rows_large_products(gq, oracle, fmt, rows, cols, M):
    """A few activation rows over products larger than 2^28 weight-rows run
    on the other kernels; the oracle checks a sample of output rows."""
    rng = synth.rng_for(611, fmt * 100000 + M)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[matmul] large few-row product fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, fmt, W, rows, cols, X)
    idx = np.unique(np.concatenate([np.arange(0, rows, 131), [1, 31, 32, 63, 64, rows - 1]]))
    Ws = oracle.select_rows(fmt, W, cols, idx)
    ref, S = oracle.matmul(fmt, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"large few-row fmt={fmt} M={M}")


@pytest.mark.parametrize("fmt", [12, 13])
@pytest.mark.parametrize("rows,M", [
    (14336, 512),   # 256 x 64 tiles
    (14336, 160),   # 256 x 64 tiles, the last m-tile half full
    (4096, 512),    # 256 x 32 tiles
    (14336, 64),    # 128 x 32 tiles, k split in two
    (14336, 16),    # 64 x 16 tiles, k split in four
    (300, 20),      # one wave per tile
])
def test_fp16_route_ragged_row_on_each_tile(gq, oracle, fmt, rows, M):
    """Q4_K and Q5_K rows of 4000 columns (the last super-block a partial
    one) on each fp16 matrix-core tile: the product equals, bit for bit, the
    one over 4096 columns whose last 96 activations are zero (the storage and
    the scaling of every super-block are the same), and the oracle on a
    sample of rows."""
    cols, full = 4000, 4096
    rng = synth.rng_for(613, fmt * 100000 + rows + M)
    W = synth.weights(fmt, rows, full, rng)
    X = synth.activations((M, cols), rng)
    Xp = np.zeros((M, full), np.float32)
    Xp[:, :cols] = X
    print(f"[matmul] fp16-route ragged fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Wd = to_dev(W)
    Y = _run(gq, fmt, Wd, rows, cols, X)
    Yp = _run(gq, fmt, Wd, rows, full, Xp)
    assert np.array_equal(Y.view(np.uint32), Yp.view(np.uint32))
    idx = np.unique(np.concatenate([np.arange(0, rows, 97), [1, 15, 16, 255, 256, rows - 1]]))
    idx = idx[idx < rows]
    Ws = oracle.select_rows(fmt, W, cols, idx)
    ref, S = oracle.matmul(fmt, Ws, idx.size, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"fp16-route ragged fmt={fmt} M={M}")


@pytest.mark.parametrize("fmt,rows", [(12, 16), (12, 300), (14, 16)])
def test_many_activation_rows(gq, oracle, fmt, rows):
    """4.3 million activation rows of 8 columns: the matrix-core grids have
    more than 65535 m-tiles in their second dimension (64-row tiles: 67188).
    Every output is finite, nothing is written past Y, and sampled rows on
    both sides of the 65536th m-tile meet the oracle's bound."""
    cols, M = 8, 4_300_000
    rng = synth.rng_for(614, fmt * 1000 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[matmul] many activation rows fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, fmt, W, rows, cols, X)
    assert np.isfinite(Y).all()
    idx = np.array([0, 1, 65535 * 64 - 1, 65535 * 64, 65536 * 64 + 5, M - 1])
    ref, S = oracle.matmul(fmt, W, rows, cols, X[idx])
    assert_within_tolerance(Y[idx], ref, S, f"many activation rows fmt={fmt}")


@pytest.mark.parametrize("fmt", [12, 13])
@pytest.mark.parametrize("rows,cols,M", [
    (2464, 232, 100),   # 64 x 16 tiles, k split in four: one super-block
    (2926, 292, 100),   # two super-blocks
    (2373, 664, 100),   # three super-blocks
    (14336, 256, 64),   # 128 x 32 tiles, k split in two: one super-block
])
def test_fp16_route_fewer_super_blocks_than_k_groups(gq, oracle, fmt, rows, cols, M):
    """Q4_K and Q5_K products on the tiles that split the super-blocks over
    wave groups, with fewer super-blocks than groups: the idle groups must
    not disturb the result (every output against the oracle)."""
    rng = synth.rng_for(615, fmt * 100000 + rows + cols)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    _check(gq, oracle, fmt, W, rows, cols, X, "fewer super-blocks than k groups")


@pytest.mark.parametrize("fmt", [12, 13])
def test_fp16_route_wide_dynamic_range(gq, oracle, fmt):
    """Q4_K and Q5_K on the fp16 matrix cores: activations whose magnitudes
    span 2^-113 .. 2^100 across rows and super-blocks, each within 2^13 of
    the largest in its row's super-block, meet the plain bound (every
    super-block is scaled by its own power of two before the fp16 split)."""
    rows, cols, M = 80, 1024, 40
    rng = synth.rng_for(611, fmt)
    W = synth.weights(fmt, rows, cols, rng)
    nsb = cols // 256
    scale = np.exp2(rng.integers(-100, 101, size=(M, nsb))).astype(np.float64)
    mag = np.exp2(rng.uniform(-13.0, 0.0, size=(M, cols)))
    sign = np.where(rng.random((M, cols)) < 0.5, -1.0, 1.0)
    X = (sign * mag * np.repeat(scale, 256, axis=1)).astype(np.float32)
    X[rng.random((M, cols)) < 0.05] = 0.0
    _check(gq, oracle, fmt, W, rows, cols, X, "wide dynamic range")


@pytest.mark.parametrize("fmt", [12, 13])
def test_fp16_route_outlier_on_zero_weight(gq, oracle, fmt):
    """The documented limit of the fp16 split: in super-block 0 every weight
    of sub-block 0 is zero (sc_0 = m_0 = 0 in every row) and one activation
    row holds 2^40 there, so that row's other activations of the super-block
    fall below 2^-14 of its largest and are carried only to an absolute
    2^-34 * 2^40. That row stays within the stated extra term; every other row,
    and that row's other super-blocks, meet the plain bound. Q4_K and Q5_K
    share the header and scale bytes, so the same bytes are cleared."""
    rows, cols, M, hot = 64, 512, 20, 7
    rng = synth.rng_for(612, fmt)
    W = synth.weights(fmt, rows, cols, rng).copy()
    sbb = {12: 144, 13: 176}[fmt]           # bytes of one super-block
    qmax = {12: 15, 13: 31}[fmt]            # largest code
    blk0 = W.reshape(rows, 2 * sbb)[:, :sbb]  # super-block 0 of every row
    blk0[:, 4] &= 0xC0                      # sc_0 = 0 (top bits belong to sc_4)
    blk0[:, 8] &= 0xC0                      # m_0 = 0 (top bits belong to m_4)
    X = synth.activations((M, cols), rng)
    X[hot, 0] = np.float32(2.0 ** 40)
    print(f"[matmul] outlier rows={rows} cols={cols} M={M}", flush=True)
    Y = _run(gq, fmt, W, rows, cols, X)
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    others = np.arange(M) != hot
    assert_within_tolerance(Y[others], ref[others], S[others], "rows without the outlier")
    # the stated extra term for the hot row: 2^-33 max_b sum_c (|d sc q| + |dmin m|),
    # bounded with sc <= 63, q <= qmax, m <= 63 from each row's d and dmin
    hdr = blk0[:, :4].copy().view(np.float16).astype(np.float64).reshape(rows, 2)
    per_col = np.abs(hdr[:, 0]) * 63 * qmax + np.abs(hdr[:, 1]) * 63
    extra = 2.0 ** -33 * 2.0 ** 40 * 256 * per_col
    err = np.abs(Y[hot].astype(np.float64) - ref[hot])
    assert (err <= 2e-4 * S[hot] + extra).all()
    # the same row without the outlier's super-block: super-block 1 alone
    X1 = X.copy()
    X1[:, :256] = 0.0
    Y1 = _run(gq, fmt, W, rows, cols, X1)
    ref1, S1 = oracle.matmul(fmt, W, rows, cols, X1, nthreads=oracle_threads())
    assert_within_tolerance(Y1, ref1, S1, "outlier's other super-block")
