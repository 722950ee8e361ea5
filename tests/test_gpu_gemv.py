"""gq_matvec on the GPU against the f64 oracle: every output within
2e-4 * sum_c |w*x| on all workload shapes and edge shapes, plus exact
invariants (one-hot columns equal the dequant bit for bit, 2^k scaling, row
permutation, run-to-run determinism) and output canaries."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _run(gq, fmt, W, rows, cols, x):
    y = sentinel_buffer(rows)
    gq.gq_matvec(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols,
                 to_dev(x) if isinstance(x, np.ndarray) else x, y=y)
    assert_pad_untouched(y, rows)
    return to_host(y)[:rows]


def _check(gq, oracle, fmt, W, rows, cols, x, what):
    print(f"[matvec] {what} fmt={fmt} rows={rows} cols={cols}", flush=True)
    y = _run(gq, fmt, W, rows, cols, x)
    ref, S = oracle.matvec(fmt, W, rows, cols, x, nthreads=oracle_threads())
    return assert_within_tolerance(y, ref, S, what)


def test_smollm_ffn_up_q8_0(gq, oracle):
    fmt, rows, cols = synth.SMOLLM_FFN_UP
    W, x = synth.matrix_and_x(fmt, rows, cols, 0, 0)
    _check(gq, oracle, fmt, W, rows, cols, x, "smollm-135m ffn_up")


@pytest.mark.parametrize("i", range(4))
def test_qwen05b_decode_q4_k(gq, oracle, i):
    fmt, rows, cols = synth.QWEN05_DECODE[i]
    W, x = synth.matrix_and_x(fmt, rows, cols, 1, i)
    _check(gq, oracle, fmt, W, rows, cols, x, f"qwen2.5-0.5b {rows}x{cols}")


def test_qwen05b_lm_head_q8_0(gq, oracle):
    fmt, rows, cols = synth.QWEN05_LM_HEAD
    W, x = synth.matrix_and_x(fmt, rows, cols, 2, 0)
    _check(gq, oracle, fmt, W, rows, cols, x, "qwen2.5-0.5b lm_head")


@pytest.mark.parametrize("layer", [0, 31])
@pytest.mark.parametrize("proj", range(7))
def test_llama3_8b_decode_q4_k(gq, oracle, layer, proj):
    name, rows, cols, _, _ = synth.llama3_8b_matrix(layer, proj)
    W, x = synth.llama3_8b_weight_and_x(layer, proj)
    _check(gq, oracle, 12, W, rows, cols, x, f"llama3-8b layer{layer} {name}")


@pytest.mark.parametrize("fmt,rows,cols", [
    (8, 1, 32), (8, 63, 64), (8, 65, 96), (8, 64, 1024), (8, 3, 70), (8, 5, 33),
    (8, 7, 1053), (8, 33, 4096), (8, 17, 40000),
    (12, 1, 256), (12, 64, 1024), (12, 65, 896), (12, 63, 300), (12, 2, 14336),
    (12, 3, 4864), (12, 9, 250), (12, 4, 1), (12, 130, 2048), (12, 5, 33024),
    (12, 1000, 512),
])
def test_edge_shapes(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(200, rows * 100000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    _check(gq, oracle, fmt, W, rows, cols, x, "edge")


@pytest.mark.parametrize("rows,cols", [
    (8193, 64), (8200, 250), (9001, 576), (8197, 1004), (8200, 2048), (8197, 4096), (9000, 96),
])
def test_q8_0_tall_matrices(gq, oracle, rows, cols):
    """Tall Q8_0 matrices: an even number of blocks per row runs on block
    pairs (row group widths 4..64 lanes), an odd one (96 columns) on single
    blocks. Ragged rows and columns."""
    rng = synth.rng_for(210, rows * 100000 + cols)
    W = synth.weights(8, rows, cols, rng)
    x = synth.activations(cols, rng)
    _check(gq, oracle, 8, W, rows, cols, x, "tall q8_0")


def test_q8_0_row_range_at_two_byte_offset(gq, oracle):
    rows, cols = 50, 160                       # 5 blocks per row: odd
    W = synth.weights(8, rows + 1, cols, synth.rng_for(9, 9))
    x = synth.activations(cols, synth.rng_for(9, 10))
    Wd = to_dev(W)
    for off in (34, 68, oracle.row_bytes(8, cols)):
        y = _run(gq, 8, Wd[off:], rows, cols, x)
        rb = oracle.row_bytes(8, cols)
        ref, S = oracle.matvec(8, W[off:off + rows * rb], rows, cols, x)
        assert_within_tolerance(y, ref, S, f"offset {off}")


@pytest.mark.parametrize("fmt,rows,cols", [(8, 64, 1024), (8, 10, 70), (12, 64, 1024),
                                           (12, 16, 896), (12, 8, 4864)])
def test_one_hot_columns_equal_dequant(gq, oracle, fmt, rows, cols):
    """x = e_c reproduces column c of the dequantised matrix exactly."""
    rng = synth.rng_for(300, cols)
    W = synth.weights(fmt, rows, cols, rng)
    w = oracle.dequant(fmt, W, rows, cols)
    Wd = to_dev(W)
    qk = 32 if fmt == 8 else 256
    cand = {0, 1, 15, 16, 31, 32, 33, 63, 64, 127, 128, 191, 255, 256, 257, cols - 1, cols // 2}
    cand |= {qk * k + o for k in range(3) for o in (0, qk - 1)}
    for c in sorted(v for v in cand if 0 <= v < cols):
        x = np.zeros(cols, np.float32)
        x[c] = 1.0
        y = _run(gq, fmt, Wd, rows, cols, x)
        assert np.array_equal(y, w[:, c]), f"column {c}"


@pytest.mark.parametrize("fmt,rows,cols", [(8, 300, 896), (12, 300, 4096), (12, 70, 896)])
def test_exact_invariants(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(400, cols)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    Wd, xd = to_dev(W), to_dev(x)
    y = _run(gq, fmt, Wd, rows, cols, xd)
    # run to run: bit-identical
    assert np.array_equal(_run(gq, fmt, Wd, rows, cols, xd).view(np.uint32), y.view(np.uint32))
    # scaling x by a power of two scales y exactly
    for k in (-3, 5):
        y2 = _run(gq, fmt, Wd, rows, cols, to_dev(x * np.float32(2.0 ** k)))
        assert np.array_equal(y2, y * np.float32(2.0 ** k))
    # permuting W's rows permutes y bit for bit
    perm = rng.permutation(rows)
    rb = oracle.row_bytes(fmt, cols)
    Wp = W.reshape(rows, rb)[perm].reshape(-1)
    yp = _run(gq, fmt, to_dev(Wp), rows, cols, xd)
    assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))


def test_side_stream_and_empty(gq):
    import torch
    rows, cols = 256, 512
    W = synth.weights(12, rows, cols, synth.rng_for(5, 5))
    x = synth.activations(cols, synth.rng_for(5, 6))
    Wd, xd = to_dev(W), to_dev(x)
    y0 = _run(gq, 12, Wd, rows, cols, xd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = gq.gq_matvec(12, Wd, rows, cols, xd)
    s.synchronize()
    assert np.array_equal(to_host(y1).view(np.uint32), y0.view(np.uint32))
    # rows == 0 is an empty product
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    gq.gq_matvec(12, Wd, 0, cols, xd, y=e)
