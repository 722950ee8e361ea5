"""Q5_0, Q5_K and Q6_K on the GPU against the oracle: gq_dequant bit for bit,
gq_matvec and gq_matmul within 2e-4 * sum_c |w*x| per output, on the shapes
of the model files that mix these formats with Q4_K (full size, the
Llama-3-8B Q6_K lm_head included) and on edge shapes that cover every
row-group width, the segmented wide-row kernel, ragged tails, 2-byte aligned
rows and row-range views; plus exact invariants (one-hot columns equal the
dequant, 2^k scaling, row permutation, run-to-run determinism)."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

Q5_0, Q5_K, Q6_K = 6, 13, 14
QK = {Q5_0: 32, Q5_K: 256, Q6_K: 256}


def _matvec(gq, fmt, W, rows, cols, x):
    y = sentinel_buffer(rows)
    gq.gq_matvec(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols,
                 to_dev(x) if isinstance(x, np.ndarray) else x, y=y)
    assert_pad_untouched(y, rows)
    return to_host(y)[:rows]


def _matmul(gq, fmt, W, rows, cols, X):
    M = X.shape[0]
    Y = sentinel_buffer(M * rows)
    gq.gq_matmul(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols, to_dev(X), Y=Y)
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[: M * rows].reshape(M, rows)


def _dequant_check(gq, oracle, fmt, W, rows, cols, what):
    print(f"[formats] dequant {what} fmt={fmt} rows={rows} cols={cols}", flush=True)
    ref = oracle.dequant(fmt, W, rows, cols)
    out = sentinel_buffer(rows * cols)
    gq.gq_dequant(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols, out=out)
    got = to_host(out)[: rows * cols].reshape(rows, cols)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), what
    assert_pad_untouched(out, rows * cols)


def _matvec_check(gq, oracle, fmt, W, rows, cols, x, what):
    print(f"[formats] matvec {what} fmt={fmt} rows={rows} cols={cols}", flush=True)
    y = _matvec(gq, fmt, W, rows, cols, x)
    ref, S = oracle.matvec(fmt, W, rows, cols, x, nthreads=oracle_threads())
    return assert_within_tolerance(y, ref, S, what)


# ------------------------------------------------------ model-file shapes

@pytest.mark.parametrize("i", range(len(synth.MIXED_FORMATS)))
def test_model_shapes_matvec(gq, oracle, i):
    name, fmt, rows, cols, W, x = synth.mixed_format_weight_and_x(i)
    _matvec_check(gq, oracle, fmt, W, rows, cols, x, name)


@pytest.mark.parametrize("i", [1, 2, 5, 7])
def test_model_shapes_dequant(gq, oracle, i):
    name, fmt, rows, cols, W, _ = synth.mixed_format_weight_and_x(i)
    _dequant_check(gq, oracle, fmt, W, rows, cols, name)


def test_lm_head_q6_k_dequant_sampled(gq, oracle):
    """The 431 MB Q6_K lm_head expanded in one call; sampled rows compared
    bit for bit (all of them through the row-range view of the oracle)."""
    name, fmt, rows, cols, W, _ = synth.mixed_format_weight_and_x(0)
    print(f"[formats] dequant {name} (sampled rows)", flush=True)
    import torch
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    gq.gq_dequant(fmt, to_dev(W), rows, cols, out=out)
    idx = np.unique(np.concatenate([np.arange(0, rows, 1013), [1, 2, 3, rows - 2, rows - 1]]))
    ref = oracle.dequant(fmt, oracle.select_rows(fmt, W, cols, idx), idx.size, cols)
    got = out[torch.from_numpy(idx).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------ edge shapes

EDGE = [
    # Q5_0: one block, row-group widths 4..256, ragged, 2-byte aligned rows
    # (odd block counts), the segmented kernel (more than 256 blocks per row)
    (Q5_0, 1, 32), (Q5_0, 63, 64), (Q5_0, 65, 96), (Q5_0, 3, 70), (Q5_0, 5, 33),
    (Q5_0, 64, 1024), (Q5_0, 7, 1053), (Q5_0, 130, 4096), (Q5_0, 9, 8224), (Q5_0, 1000, 160),
    # Q5_K / Q6_K: one super-block, ragged, widths 4..256, segmented (> 64
    # super-blocks per row), Q6_K rows alternating 4- and 2-byte alignment
    (Q5_K, 1, 256), (Q5_K, 65, 300), (Q5_K, 64, 1024), (Q5_K, 3, 4864), (Q5_K, 9, 250),
    (Q5_K, 4, 1), (Q5_K, 130, 2048), (Q5_K, 5, 16640), (Q5_K, 1000, 512),
    (Q6_K, 1, 256), (Q6_K, 65, 256), (Q6_K, 63, 300), (Q6_K, 64, 1024), (Q6_K, 7, 4864),
    (Q6_K, 9, 250), (Q6_K, 4, 1), (Q6_K, 131, 2304), (Q6_K, 5, 16640), (Q6_K, 1000, 512),
    (Q6_K, 33, 14336),
]


@pytest.mark.parametrize("fmt,rows,cols", EDGE)
def test_edge_matvec(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(900, fmt * 10 ** 8 + rows * 100000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    _matvec_check(gq, oracle, fmt, W, rows, cols, x, "edge")


@pytest.mark.parametrize("fmt,rows,cols", EDGE)
def test_edge_dequant(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(901, fmt * 10 ** 8 + rows * 100000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    _dequant_check(gq, oracle, fmt, W, rows, cols, "edge")


@pytest.mark.parametrize("M", [2, 3, 7, 15, 16, 17, 31])
@pytest.mark.parametrize("fmt,rows,cols", [(Q5_0, 200, 896), (Q5_K, 130, 1024), (Q6_K, 130, 4096),
                                           (Q6_K, 33, 300), (Q5_0, 17, 8224)])
def test_matmul_m_sweep(gq, oracle, fmt, rows, cols, M):
    rng = synth.rng_for(902, fmt * 1000 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), synth.rng_for(903, M))
    print(f"[formats] matmul fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = _matmul(gq, fmt, W, rows, cols, X)
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"matmul fmt={fmt} M={M}")


def test_matmul_full_size_q6_k_down(gq, oracle):
    """Llama-3-8B Q6_K ffn_down shape with 8 activation rows; sampled rows."""
    name, fmt, rows, cols, W, _ = synth.mixed_format_weight_and_x(1)
    X = synth.activations((8, cols), synth.rng_for(904, 8))
    print(f"[formats] matmul {name} M=8", flush=True)
    Y = _matmul(gq, fmt, W, rows, cols, X)
    idx = np.unique(np.concatenate([np.arange(0, rows, 37), [1, 63, 64, rows - 1]]))
    ref, S = oracle.matmul(fmt, oracle.select_rows(fmt, W, cols, idx), idx.size, cols, X,
                           nthreads=oracle_threads())
    assert_within_tolerance(Y[:, idx], ref, S, f"{name} M=8")


# ------------------------------------------------- alignment and views

@pytest.mark.parametrize("fmt,cols", [(Q5_0, 160), (Q6_K, 256), (Q5_0, 896)])
def test_row_range_at_two_byte_offset(gq, oracle, fmt, cols):
    """A row range of a tensor starting one block in (2 mod 4 bytes) or one
    row in: matvec within tolerance, dequant bit for bit."""
    rows = 40
    rb = oracle.row_bytes(fmt, cols)
    blk = {Q5_0: 22, Q6_K: 210}[fmt]
    W = synth.weights(fmt, rows + 1, cols, synth.rng_for(905, fmt))
    x = synth.activations(cols, synth.rng_for(906, fmt))
    Wd = to_dev(W)
    import torch
    for off in (blk, 3 * blk, rb):
        n = (W.size - off) // rb
        sub = W[off:off + n * rb]
        print(f"[formats] view fmt={fmt} offset={off} rows={n}", flush=True)
        y = _matvec(gq, fmt, Wd[off:], n, cols, x)
        ref, S = oracle.matvec(fmt, sub, n, cols, x)
        assert_within_tolerance(y, ref, S, f"offset {off}")
        out = torch.empty((n, cols), dtype=torch.float32, device="cuda")
        gq.gq_dequant(fmt, Wd[off:], n, cols, out=out)
        assert np.array_equal(to_host(out).view(np.uint32), oracle.dequant(fmt, sub, n, cols).view(np.uint32))


def test_q5_k_rejects_two_byte_alignment(gq):
    W = to_dev(synth.weights(Q5_K, 3, 256, synth.rng_for(907, 0)))
    x = to_dev(synth.activations(256, synth.rng_for(907, 1)))
    with pytest.raises(gq.GQError) as e:
        gq.gq_matvec(Q5_K, W[2:], 2, 256, x)
    assert e.value.status == gq.GQ_ERR_ALIGN


# ---------------------------------------------------------- exactness

@pytest.mark.parametrize("fmt,rows,cols", [(Q5_0, 64, 1024), (Q5_0, 10, 70), (Q5_K, 64, 1024),
                                           (Q5_K, 16, 896), (Q6_K, 64, 1024), (Q6_K, 8, 4864),
                                           (Q6_K, 16, 300)])
def test_one_hot_columns_equal_dequant(gq, oracle, fmt, rows, cols):
    """x = e_c reproduces column c of the dequantised matrix exactly."""
    rng = synth.rng_for(908, fmt * 1000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    w = oracle.dequant(fmt, W, rows, cols)
    Wd = to_dev(W)
    qk = QK[fmt]
    cand = {0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128, 129, 160, 191, 192,
            224, 255, 256, 257, cols - 1, cols // 2}
    cand |= {qk * k + o for k in range(3) for o in (0, qk - 1)}
    for c in sorted(v for v in cand if 0 <= v < cols):
        x = np.zeros(cols, np.float32)
        x[c] = 1.0
        y = _matvec(gq, fmt, Wd, rows, cols, x)
        assert np.array_equal(y, w[:, c]), f"fmt {fmt} column {c}"


@pytest.mark.parametrize("fmt,rows,cols", [(Q5_0, 300, 896), (Q5_K, 300, 4096), (Q6_K, 300, 4096)])
def test_exact_invariants(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(909, fmt)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    Wd, xd = to_dev(W), to_dev(x)
    y = _matvec(gq, fmt, Wd, rows, cols, xd)
    assert np.array_equal(_matvec(gq, fmt, Wd, rows, cols, xd).view(np.uint32), y.view(np.uint32))
    for k in (-3, 5):
        y2 = _matvec(gq, fmt, Wd, rows, cols, to_dev(x * np.float32(2.0 ** k)))
        assert np.array_equal(y2, y * np.float32(2.0 ** k))
    perm = rng.permutation(rows)
    rb = oracle.row_bytes(fmt, cols)
    yp = _matvec(gq, fmt, to_dev(W.reshape(rows, rb)[perm].reshape(-1)), rows, cols, xd)
    assert np.array_equal(yp.view(np.uint32), y[perm].view(np.uint32))
    # a matmul row equals the matvec bit for bit when M == 1
    Y1 = _matmul(gq, fmt, Wd, rows, cols, x.reshape(1, cols))
    assert np.array_equal(Y1[0].view(np.uint32), y.view(np.uint32))


def test_special_scales(gq, oracle):
    """Subnormal, negative, zero and extreme fp16 scales; int8 scale -128."""
    rng = np.random.default_rng(910)
    specials = [0x0001, 0x03FF, 0x8001, 0x0400, 0x7BFF, 0xFBFF, 0x0000, 0x8000, 0xBC00]
    # Q5_0
    b5 = []
    for d16 in specials:
        b = rng.integers(0, 256, 22, dtype=np.uint8)
        b[0], b[1] = d16 & 0xFF, d16 >> 8
        b5.append(b)
    W = np.concatenate(b5 * 8)          # 8 blocks per row
    rows = len(b5)
    _dequant_check(gq, oracle, Q5_0, W, rows, 256, "q5_0 special scales")
    x = synth.activations(256, rng)
    _matvec_check(gq, oracle, Q5_0, W, rows, 256, x, "q5_0 special scales")
    # Q5_K
    bk = []
    for d16, dm16 in [(0x0001, 0x0001), (0x8001, 0x03FF), (0x7BFF, 0x0001), (0x0001, 0x7BFF),
                      (0x0000, 0x0000), (0x8000, 0x8000), (0xBC00, 0xC000)]:
        b = rng.integers(0, 256, 176, dtype=np.uint8)
        b[0], b[1], b[2], b[3] = d16 & 0xFF, d16 >> 8, dm16 & 0xFF, dm16 >> 8
        bk.append(b)
    W = np.concatenate(bk)
    _dequant_check(gq, oracle, Q5_K, W, len(bk), 256, "q5_k special scales")
    # Q6_K, with every scale -128 or 127 in some blocks
    b6 = []
    for d16 in specials:
        for fill in (None, 0x80, 0x7F):
            b = rng.integers(0, 256, 210, dtype=np.uint8)
            if fill is not None:
                b[192:208] = fill
            b[208], b[209] = d16 & 0xFF, d16 >> 8
            b6.append(b)
    W = np.concatenate(b6)
    _dequant_check(gq, oracle, Q6_K, W, len(b6), 256, "q6_k special scales")
    finite = [b for b in b6 if int(b[208]) | (int(b[209]) << 8) not in (0x7BFF, 0xFBFF)]
    Wf = np.concatenate(finite)
    x = synth.activations(256, rng)
    _matvec_check(gq, oracle, Q6_K, Wf, len(finite), 256, x, "q6_k special scales")


@pytest.mark.parametrize("M", [16, 64, 512])
@pytest.mark.parametrize("i", [1, 3, 7])
def test_prefill_full_size(gq, oracle, i, M):
    """The 8B-shaped Q6_K down, Q5_K gate and Q5_0 (Qwen 4864x896) matrices
    with M activation rows; every output against the oracle."""
    name, fmt, rows, cols, W, _ = synth.mixed_format_weight_and_x(i)
    X = synth.activations((M, cols), synth.rng_for(911, M))
    print(f"[formats] prefill {name} M={M} (full check)", flush=True)
    Y = _matmul(gq, fmt, W, rows, cols, X)
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, f"{name} M={M}")


@pytest.mark.parametrize("fmt,rows,cols,M", [(8, 4096, 4096, 64), (8, 65, 1004, 33), (8, 65, 1006, 33),
                                             (6, 130, 8224, 17), (6, 130, 8192, 17), (14, 63, 300, 48),
                                             (14, 63, 302, 48),
                                             (13, 200, 1024, 100)])
def test_matrix_core_edges(gq, oracle, fmt, rows, cols, M):
    """Ragged rows, columns and activation rows on the matrix cores: the fp16
    kernels for the rows they take, the fp32 ones for the others (an odd
    number of blocks, or a length not a multiple of 4, which takes the
    scalar activation loads)."""
    rng = synth.rng_for(912, fmt * 1000 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    print(f"[formats] matrix-core fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Y = _matmul(gq, fmt, W, rows, cols, X)
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    assert_within_tolerance(Y, ref, S, "matrix-core edge")
