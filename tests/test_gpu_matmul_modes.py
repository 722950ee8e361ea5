"""gq_matmul_acc and gq_matmul_swiglu on the GPU, one case per route (the
matvec at M = 1, per-row matvecs in the few-row range, the Q4_K / Q5_K fp16
matrix cores with each of their tiles, Q8_0 on the fp16 matrix cores, the
fp32 matrix cores for the other formats and for rows those kernels do not
take): the accumulating form
equals Y0 + gq_matmul bit for bit and the oracle within tolerance; the SwiGLU
form meets the derived bound against the f64 oracle and equals the host's
fp32 SwiGLU of the two halves' gq_matmul to a few ulps."""
import numpy as np
import pytest

import synth
from helpers import assert_pad_untouched, oracle_threads, sentinel_buffer, to_dev, to_host

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24

# (fmt, rows, cols, M): matvec, per-row matvecs, the Q4_K tiles (per-wave,
# 64x16 split in four, 128x32 split in two, 256x32, 256x64), Q5_K on the
# per-wave and 128x32 tiles, Q8_0 on the fp16 matrix cores (M = 4, below the
# stored form's threshold; the per-wave and 128x32 tiles), Q6_K and Q5_0 on
# them (the per-wave and 128x32 tiles), Q4_K rows of 898 columns, Q8_0 rows
# of 29 blocks, Q6_K rows of 3 super-blocks and Q5_0 rows of 33 blocks on the
# fp32 matrix cores
CASES = [
    (12, 300, 896, 1), (12, 300, 896, 5),
    (12, 4096, 14336, 16), (12, 14336, 4096, 16), (12, 14336, 4096, 64), (12, 4096, 4096, 300),
    (12, 14336, 1024, 512), (13, 300, 1024, 20), (13, 14336, 4096, 64),
    (12, 130, 898, 20), (8, 200, 576, 4), (8, 300, 1024, 40), (8, 4096, 4096, 160),
    (8, 300, 900, 40), (14, 256, 768, 33), (14, 300, 1024, 40), (14, 4096, 4096, 160),
    (6, 300, 896, 40), (6, 4864, 896, 160), (6, 300, 1056, 40),
]


def _inputs(fmt, wrows, cols, M, seed):
    rng = synth.rng_for(971, seed)
    W = synth.weights(fmt, wrows, cols, rng)
    X = synth.activations((M, cols), rng)
    return W, X


def _call(gq, name, fmt, Wd, rows, cols, Xd, M, Y0=None):
    Y = sentinel_buffer(M * rows)
    if Y0 is not None:
        Y[:M * rows].copy_(to_dev(Y0.reshape(-1)))
    getattr(gq, name)(fmt, Wd, rows, cols, Xd, Y=Y[:M * rows])
    assert_pad_untouched(Y, M * rows)
    return to_host(Y)[:M * rows].reshape(M, rows)


@pytest.mark.parametrize("fmt,rows,cols,M", CASES)
def test_matmul_acc(gq, oracle, fmt, rows, cols, M):
    W, X = _inputs(fmt, rows, cols, M, fmt * 10 ** 6 + rows * 10 + M)
    Y0 = synth.activations((M, rows), synth.rng_for(972, M)).astype(np.float32)
    print(f"[modes] acc fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = _call(gq, "gq_matmul_acc", fmt, Wd, rows, cols, Xd, M, Y0)
    # bit for bit: the plain product added in fp32
    P = _call(gq, "gq_matmul", fmt, Wd, rows, cols, Xd, M)
    assert np.array_equal(Y.view(np.uint32), (Y0 + P).view(np.uint32))
    ref, S = oracle.matmul(fmt, W, rows, cols, X, nthreads=oracle_threads())
    want = Y0.astype(np.float64) + ref
    assert (np.abs(Y.astype(np.float64) - want) <= 2e-4 * S + U32 * np.abs(want) + 1e-30).all()


@pytest.mark.parametrize("fmt,rows,cols,M", CASES)
def test_matmul_swiglu(gq, oracle, fmt, rows, cols, M):
    W, X = _inputs(fmt, 2 * rows, cols, M, fmt * 10 ** 6 + rows * 10 + M + 1)
    print(f"[modes] swiglu fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = _call(gq, "gq_matmul_swiglu", fmt, Wd, rows, cols, Xd, M)
    rb = gq.gq_row_bytes(fmt, cols)
    GU, S = oracle.matmul(fmt, W, 2 * rows, cols, X, nthreads=oracle_threads())
    g_ref, u_ref, Sg, Su = GU[:, :rows], GU[:, rows:], S[:, :rows], S[:, rows:]
    y_ref = oracle.silu(g_ref) * u_ref
    eg, eu = 2e-4 * Sg, 2e-4 * Su
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + (np.abs(oracle.silu(g_ref)) + 1.1 * eg) * eu
    bound += 8 * U32 * np.abs(y_ref) + 1e-30
    assert not np.isnan(Y).any()
    assert (np.abs(Y.astype(np.float64) - y_ref) <= bound).all()
    # the two halves through gq_matmul, the activation on the host in fp32
    G = _call(gq, "gq_matmul", fmt, Wd[: rows * rb], rows, cols, Xd, M)
    U = _call(gq, "gq_matmul", fmt, Wd[rows * rb:], rows, cols, Xd, M)
    g = G.astype(np.float32)
    with np.errstate(over="ignore"):
        y_host = (g / (np.float32(1) + np.exp(-g)) * U.astype(np.float32)).astype(np.float32)
    assert np.all(np.abs(Y - y_host) <= 8 * U32 * np.abs(y_host) + 1e-37)
    if M == 1 or (M < 16 and M * rows * cols <= 1 << 28):
        # the matvec range: every row is gq_matvec_swiglu of its activation row
        for m in range(M):
            y = sentinel_buffer(rows)
            gq.gq_matvec_swiglu(fmt, Wd, rows, cols, Xd[m], y=y[:rows])
            assert np.array_equal(to_host(y)[:rows].view(np.uint32), Y[m].view(np.uint32))
