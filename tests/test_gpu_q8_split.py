"""The split per-row Q8_0 layout on the GPU: gq_q8_0_split_repack equals the
oracle's repack byte for byte (padding included), and every entry point on
the repacked weights matches the oracle: dequant bit for bit, matvec,
accumulate, matmul and expert-batched calls within the product tolerance;
the matvec on the repacked tensor also equals the oracle's matvec of the
original blocks (the same weights)."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

SPLIT = 1008

SHAPES = [(1, 32), (63, 64), (65, 96), (3, 70), (5, 33), (64, 1024), (7, 1053), (130, 4096),
          (17, 40000), (1000, 160), (151936, 896),
          # more row lengths: 28 to 1792 chunks, one ragged
          (5, 448), (9, 1792), (300, 3584), (64, 14336), (33, 890), (3, 28672)]


def _repack(gq, oracle, W, rows, cols):
    Wd = to_dev(W)
    got = to_host(gq.gq_q8_0_split_repack(Wd, rows, cols))
    want = oracle.q8_0_split_repack(W, rows, cols)
    assert np.array_equal(got, want), (rows, cols)
    return got


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_repack_matvec_dequant(gq, oracle, rows, cols):
    rng = synth.rng_for(970, rows * 100000 + cols)
    W = synth.weights(8, rows, cols, rng)
    x = synth.activations(cols, rng)
    print(f"[split] rows={rows} cols={cols}", flush=True)
    S = _repack(gq, oracle, W, rows, cols)
    Sd, xd = to_dev(S), to_dev(x)
    y = sentinel_buffer(rows)
    gq.gq_matvec(SPLIT, Sd, rows, cols, xd, y=y)
    assert_pad_untouched(y, rows)
    ref, Sref = oracle.matvec(8, W, rows, cols, x, nthreads=oracle_threads())
    assert_within_tolerance(to_host(y)[:rows], ref, Sref, "split matvec")
    if rows * cols <= 64 * 1024 * 1024:
        out = sentinel_buffer(rows * cols)
        gq.gq_dequant(SPLIT, Sd, rows, cols, out=out)
        assert_pad_untouched(out, rows * cols)
        got = to_host(out)[: rows * cols].reshape(rows, cols)
        assert np.array_equal(got.view(np.uint32), oracle.dequant(8, W, rows, cols).view(np.uint32))


def test_repack_from_a_row_range_at_two_byte_offset(gq, oracle):
    rows, cols = 40, 160                       # 5 blocks per row
    W = synth.weights(8, rows + 1, cols, synth.rng_for(971, 0))
    Wd = to_dev(W)
    for off in (34, 68):
        sub = W[off:off + rows * oracle.row_bytes(8, cols)]
        got = to_host(gq.gq_q8_0_split_repack(Wd[off:], rows, cols))
        assert np.array_equal(got, oracle.q8_0_split_repack(sub, rows, cols))


@pytest.mark.parametrize("M", [2, 7, 16, 33, 64])
def test_split_matmul(gq, oracle, M):
    rows, cols = 300, 1024
    rng = synth.rng_for(972, M)
    W = synth.weights(8, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    Sd = gq.gq_q8_0_split_repack(to_dev(W), rows, cols)
    Y = sentinel_buffer(M * rows)
    gq.gq_matmul(SPLIT, Sd, rows, cols, to_dev(X), Y=Y)
    assert_pad_untouched(Y, M * rows)
    ref, S = oracle.matmul(8, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(to_host(Y)[: M * rows].reshape(M, rows), ref, S, f"split matmul M={M}")


def test_split_acc_and_experts(gq, oracle):
    import torch
    rows, cols, n_expert = 200, 896, 3
    rng = synth.rng_for(973, 0)
    W = synth.weights(8, n_expert * rows, cols, rng)
    Sd = gq.gq_q8_0_split_repack(to_dev(W), n_expert * rows, cols)
    x = synth.activations(cols, rng)
    xd = to_dev(x)
    # accumulate onto y0: y0 + the plain split matvec, bit for bit
    y0 = synth.activations(rows, rng)
    y = to_dev(y0.copy())
    gq.gq_matvec_acc(SPLIT, Sd, rows, cols, xd, y)
    plain = to_host(gq.gq_matvec(SPLIT, Sd, rows, cols, xd))
    assert np.array_equal(to_host(y).view(np.uint32), (y0 + plain).view(np.uint32))
    # expert-batched over the three experts of the repacked tensor
    ids = np.array([2, 0, 1, 1], np.int32)
    X = synth.activations((2, cols), rng)
    Y = to_host(gq.gq_matvec_experts(SPLIT, Sd, n_expert, rows, cols, to_dev(X), 2, to_dev(ids)))
    ref, S = oracle.experts_matvec(8, W, n_expert, rows, cols, X, 2, ids)
    assert_within_tolerance(Y, ref, S, "split experts")


def test_split_swiglu_equals_host_activation_of_matvec(gq):
    rows, cols = 300, 896
    rng = synth.rng_for(974, 0)
    W = synth.weights(8, 2 * rows, cols, rng)
    Sd = gq.gq_q8_0_split_repack(to_dev(W), 2 * rows, cols)
    xd = to_dev(synth.activations(cols, rng))
    y = to_host(gq.gq_matvec_swiglu(SPLIT, Sd, rows, cols, xd))
    gu = to_host(gq.gq_matvec(SPLIT, Sd, 2 * rows, cols, xd))
    g, u = gu[:rows], gu[rows:]
    with np.errstate(over="ignore"):
        host = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
    assert np.all(np.abs(y - host) <= 8 * 2.0 ** -24 * np.abs(host) + 1e-37)
