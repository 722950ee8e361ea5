"""gq_matvec_batch on the GPU: every output row equals the lone gq_matvec of
its activation row bit for bit (a batched call never changes results), the
outputs are within the product tolerance of the f64 oracle, and shapes
cover every format, ragged rows and tails, rows wider than one row group,
and batch sizes from 2 up to a prompt chunk."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

# (fmt, rows, cols, batch)
CASES = [
    (12, 4096, 4096, 2),      # Llama-3-8B q projection, two tokens
    (12, 14336, 4096, 3),     # gate
    (12, 4096, 14336, 4),     # down: rows of 224 units (group width 256)
    (12, 896, 896, 5),        # Qwen2.5-0.5B, ragged super-blocks
    (12, 37, 300, 7),         # ragged rows and columns, odd batch
    (8, 1536, 576, 3),        # SmolLM-135M Q8_0 (block pairs)
    (8, 300, 1000, 2),        # Q8_0 single blocks (odd block count)
    (8, 9, 40000, 2),         # rows wider than 256 units: segmented kernel
    (6, 896, 4864, 3),        # Q5_0
    (13, 4096, 4096, 2),      # Q5_K
    (14, 2048, 768, 4),       # Q6_K, three super-blocks per row
    (1008, 1000, 896, 3),     # Q8_0 split layout
    (12, 64, 1024, 64),       # a prompt chunk of 64 positions
]


def _weights(fmt, rows, cols, rng):
    if fmt == 1008:   # the split layout is made on the device from Q8_0 blocks
        return synth.weights(8, rows, cols, rng)
    return synth.weights(fmt, rows, cols, rng)


@pytest.mark.parametrize("fmt,rows,cols,batch", CASES)
def test_batch_rows_equal_matvec(gq, oracle, fmt, rows, cols, batch):
    rng = synth.rng_for(970, fmt * 10 ** 6 + rows * 10 + batch)
    W = _weights(fmt, rows, cols, rng)
    X = synth.activations((batch, cols), rng)
    print(f"[batch] fmt={fmt} rows={rows} cols={cols} batch={batch}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    if fmt == 1008:
        Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
    Yb = sentinel_buffer(batch * rows)
    gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd, Y=Yb[:batch * rows])
    assert_pad_untouched(Yb, batch * rows)
    got = to_host(Yb)[:batch * rows].reshape(batch, rows)
    ref, S = oracle.matmul(8 if fmt == 1008 else fmt, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(got, ref, S, "batch")
    for b in range(batch):
        y = gq.gq_matvec(fmt, Wd, rows, cols, Xd[b])
        assert np.array_equal(to_host(y).view(np.uint32), got[b].view(np.uint32)), b


def test_batch_repeatable_and_empty(gq):
    import torch
    fmt, rows, cols, batch = 12, 14336, 4096, 4
    rng = synth.rng_for(971, 0)
    Wd = to_dev(synth.weights(fmt, rows, cols, rng))
    Xd = to_dev(synth.activations((batch, cols), rng))
    first = to_host(gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd))
    for _ in range(3):
        again = to_host(gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd))
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    # no activation rows: nothing is launched or written
    Y0 = torch.full((1, rows), 7.0, device="cuda")
    gq.gq_matvec_batch(fmt, Wd, rows, cols, torch.empty(0, device="cuda"), Y=Y0)
    assert (to_host(Y0) == 7.0).all()


@pytest.mark.parametrize("fmt,rows,cols", [(12, 8, 256), (8, 300, 64)])
def test_batch_past_65535_rows(gq, oracle, fmt, rows, cols):
    """70000 activation rows: the batch is the grid's second dimension, past
    65535. Sampled rows on both sides of that boundary equal gq_matvec bit
    for bit and meet the oracle's bound; nothing is written past Y."""
    batch = 70000
    rng = synth.rng_for(972, fmt * 1000 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((batch, cols), rng)
    print(f"[batch] past 65535 fmt={fmt} rows={rows} cols={cols} batch={batch}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Yb = sentinel_buffer(batch * rows)
    gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd, Y=Yb[:batch * rows])
    assert_pad_untouched(Yb, batch * rows)
    got = to_host(Yb)[:batch * rows].reshape(batch, rows)
    assert np.isfinite(got).all()
    idx = [0, 1, 65534, 65535, 65536, batch - 1]
    ref, S = oracle.matmul(fmt, W, rows, cols, X[idx])
    assert_within_tolerance(got[idx], ref, S, "batch past 65535")
    for b in idx:
        y = gq.gq_matvec(fmt, Wd, rows, cols, Xd[b])
        assert np.array_equal(to_host(y).view(np.uint32), got[b].view(np.uint32)), b
