"""The int8-activation path on the GPU: gq_quantize_q8_1 byte for byte
against the oracle's quantiser, and gq_matvec_q8_1 within 2e-4 * sum |w x^|
of the oracle's W x^ (x^ the dequantised Q8_1 row) on the decode shapes,
ragged rows and the LDS limit."""
import numpy as np
import pytest

import synth
from helpers import assert_pad_untouched, assert_within_tolerance, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu


def _quantize_gpu(gq, X):
    import torch
    n, cols = X.shape
    nbytes = n * gq.gq_row_bytes(gq.GQ_FMT_Q8_1, cols)
    out = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    gq.gq_quantize_q8_1(to_dev(X), n, cols, out=out[:nbytes])
    host = to_host(out)
    assert (host[nbytes:] == 0xA5).all(), "wrote past the output"
    return host[:nbytes]


@pytest.mark.parametrize("n,cols,seed", [(1, 4096, 0), (1, 14336, 1), (3, 896, 2), (2, 300, 3),
                                         (5, 33, 4), (1, 32, 5), (64, 576, 6)])
def test_quantize_bit_exact(gq, oracle, n, cols, seed):
    rng = np.random.default_rng(1000 + seed)
    scale = np.exp2(rng.integers(-30, 30, size=(n, 1)))
    X = (rng.standard_normal((n, cols)) * scale).astype(np.float32)
    X[rng.random((n, cols)) < 0.03] = 0.0
    print(f"[q8_1] quantize n={n} cols={cols}", flush=True)
    got = _quantize_gpu(gq, X)
    want = oracle.quantize_q8_1(X)
    assert np.array_equal(got, want)


def test_quantize_ties_tiny_and_zero_blocks(gq, oracle):
    # block 0: a scale of exactly 1 with half-integer values (ties go away
    # from zero); block 1: values near the fp32 normal limit (subnormal fp16
    # scale); block 2: all zero; block 3: one value only; block 4: largest
    # magnitude 1e-38, so 1 / d overflows (codes clamped to +-127, zeros 0)
    x = np.zeros(160, np.float32)
    x[0:31] = (np.arange(-15, 16) + 0.5).astype(np.float32)
    x[31] = 127.0
    x[32:64] = np.float32(3e-37) * np.arange(1, 33, dtype=np.float32)
    x[100] = -5.0
    x[128], x[129], x[140] = 1e-38, -1e-38, 2e-39
    X = x.reshape(1, -1)
    assert np.array_equal(_quantize_gpu(gq, X), oracle.quantize_q8_1(X))


def _run_matvec(gq, fmt, W, rows, cols, xq):
    import torch
    y = torch.full((rows + 64,), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_matvec_q8_1(fmt, to_dev(W), rows, cols, to_dev(xq), y=y[:rows])
    assert_pad_untouched(y, rows)
    return to_host(y)[:rows]


def _check(gq, oracle, fmt, W, rows, cols, x, what):
    print(f"[q8_1] matvec {what} fmt={fmt} rows={rows} cols={cols}", flush=True)
    xq = oracle.quantize_q8_1(x)
    y = _run_matvec(gq, fmt, W, rows, cols, xq)
    ref, S = oracle.matvec_q8_1(fmt, W, rows, cols, xq, nthreads=oracle_threads())
    return assert_within_tolerance(y, ref, S, what)


@pytest.mark.parametrize("layer", [0, 31])
@pytest.mark.parametrize("proj", range(7))
def test_llama3_8b_decode(gq, oracle, layer, proj):
    name, rows, cols, _, _ = synth.llama3_8b_matrix(layer, proj)
    W, x = synth.llama3_8b_weight_and_x(layer, proj)
    _check(gq, oracle, 12, W, rows, cols, x, f"llama3-8b layer{layer} {name}")


def test_smollm_and_qwen_shapes(gq, oracle):
    fmt, rows, cols = synth.SMOLLM_FFN_UP
    W, x = synth.matrix_and_x(fmt, rows, cols, 0, 0)
    _check(gq, oracle, fmt, W, rows, cols, x, "smollm-135m ffn_up")
    for i in range(4):
        fmt, rows, cols = synth.QWEN05_DECODE[i]
        W, x = synth.matrix_and_x(fmt, rows, cols, 1, i)
        _check(gq, oracle, fmt, W, rows, cols, x, f"qwen2.5-0.5b {rows}x{cols}")
    fmt, rows, cols = synth.QWEN05_LM_HEAD
    W, x = synth.matrix_and_x(fmt, rows, cols, 2, 0)
    _check(gq, oracle, fmt, W, rows, cols, x, "qwen2.5-0.5b lm_head")


@pytest.mark.parametrize("fmt,rows,cols", [
    (8, 1, 32), (8, 3, 70), (8, 5, 33), (8, 64, 1024), (8, 7, 1053), (8, 9, 40000),
    (12, 1, 256), (12, 2, 300), (12, 3, 896), (12, 65, 4096), (12, 6, 14336), (12, 5, 1000),
])
def test_edge_shapes(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(777, fmt * 100000 + rows * 1000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations((cols,), rng)
    _check(gq, oracle, fmt, W, rows, cols, x, "edge")


@pytest.mark.parametrize("fmt", [8, 12])
def test_lds_limit(gq, oracle, fmt):
    # 131072 columns: the largest row the kernel stages (160 KB of LDS)
    rows, cols = 3, 131072
    rng = synth.rng_for(778, fmt)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations((cols,), rng)
    _check(gq, oracle, fmt, W, rows, cols, x, "lds limit")


def test_deterministic_and_matches_fp32_path_within_quantisation(gq, oracle):
    name, rows, cols, _, _ = synth.llama3_8b_matrix(0, 4)
    W, x = synth.llama3_8b_weight_and_x(0, 4)
    xq = oracle.quantize_q8_1(x)
    y1 = _run_matvec(gq, 12, W, rows, cols, xq)
    y2 = _run_matvec(gq, 12, W, rows, cols, xq)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # against the fp32-activation product: the quantisation error bound
    # sum_c |w| (d_b / 2 + 127 |d_b - fp16(d_b)|) plus the arithmetic tolerances
    ref32, S32 = oracle.matvec(12, W, rows, cols, x, nthreads=oracle_threads())
    wabs = np.abs(oracle.dequant(12, W, rows, cols)).astype(np.float64)
    amax = np.abs(x.reshape(-1, 32)).max(axis=1).astype(np.float32)
    d32 = (amax / np.float32(127.0)).astype(np.float64)
    d16 = d32.astype(np.float16).astype(np.float64)
    per = np.repeat(d32 / 2 + 127 * np.abs(d32 - d16) + 4e-7 * amax, 32)[:cols]
    bound = wabs @ per + 4e-4 * S32
    assert (np.abs(y1.astype(np.float64) - ref32) <= bound).all()
