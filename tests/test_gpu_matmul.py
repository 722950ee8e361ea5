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
    (14, 4096, 14336, 5),     # Q6_K: fp32 matrix cores
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
