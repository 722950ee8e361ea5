"""Seeded random shapes on the GPU against the f64 oracle: every format,
rows and columns drawn across block boundaries and ragged tails, and the
entry points that take them (gq_matvec, gq_matvec_acc, gq_matvec_batch,
gq_matmul, gq_dequant; and on a second set of shapes with M >= 16,
gq_matmul_acc, gq_matmul_swiglu, the int8-activation pair and the grouped
expert product). Products must lie within 2e-4 * sum |w x| of the oracle
(the SwiGLU form within the bound derived from it), dequant and the Q8_1
quantiser must equal it bit for bit, the batched rows must equal the lone
matvec bit for bit, and no kernel may write past its output."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

FORMATS = (8, 12, 6, 13, 14, 1008)
N_CASES = 160


def _case(i):
    rng = np.random.default_rng([2026, i])
    fmt = FORMATS[i % len(FORMATS)]
    qk = 256 if fmt in (12, 13, 14) else 32
    # columns: a whole number of blocks, a ragged tail, or a single block
    nb = int(rng.integers(1, 40 if qk == 256 else 300))
    cols = nb * qk - int(rng.integers(0, qk)) if rng.random() < 0.5 else nb * qk
    rows = int(rng.choice([1, 2, 3, 5, 63, 64, 65, 127, 300, 1000, 2049]))
    M = int(rng.choice([1, 2, 3, 5, 15, 16, 17, 40]))
    return fmt, rows, max(1, cols), M, rng


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(gq, oracle, i):
    fmt, rows, cols, M, rng = _case(i)
    base = 8 if fmt == 1008 else fmt
    print(f"[random {i}] fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)
    W = synth.weights(base, rows, cols, rng)
    X = synth.activations((M, cols), rng)
    Wd, Xd = to_dev(W), to_dev(X)
    if fmt == 1008:
        Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
    ref, S = oracle.matmul(base, W, rows, cols, X, nthreads=oracle_threads())

    # matvec of the first activation row, then accumulate the second onto it
    y = sentinel_buffer(rows)
    gq.gq_matvec(fmt, Wd, rows, cols, Xd[0], y=y[:rows])
    assert_pad_untouched(y, rows)
    y0 = to_host(y)[:rows].copy()
    assert_within_tolerance(y0, ref[0], S[0], "matvec")
    if M >= 2:
        gq.gq_matvec_acc(fmt, Wd, rows, cols, Xd[1], y[:rows])
        acc = to_host(y)[:rows]
        assert np.array_equal(acc.view(np.uint32),
                              (y0 + to_host(gq.gq_matvec(fmt, Wd, rows, cols, Xd[1]))).view(np.uint32))

    # all rows: the batched matvec (bit-identical rows) and gq_matmul (tolerance)
    Yb = sentinel_buffer(M * rows)
    gq.gq_matvec_batch(fmt, Wd, rows, cols, Xd, Y=Yb[:M * rows])
    assert_pad_untouched(Yb, M * rows)
    yb = to_host(Yb)[:M * rows].reshape(M, rows)
    assert np.array_equal(yb[0].view(np.uint32), y0.view(np.uint32))
    Ym = sentinel_buffer(M * rows)
    gq.gq_matmul(fmt, Wd, rows, cols, Xd, Y=Ym[:M * rows])
    assert_pad_untouched(Ym, M * rows)
    assert_within_tolerance(to_host(Ym)[:M * rows].reshape(M, rows), ref, S, "matmul")

    # dequant, bit-exact
    out = sentinel_buffer(rows * cols)
    gq.gq_dequant(fmt, Wd, rows, cols, out=out[:rows * cols])
    assert_pad_untouched(out, rows * cols)
    got = to_host(out)[:rows * cols].reshape(rows, cols)
    assert np.array_equal(got.view(np.uint32), oracle.dequant(base, W, rows, cols).view(np.uint32))


N_CASES_2 = 90
U32 = 2.0 ** -24


def _case2(i):
    rng = np.random.default_rng([2027, i])
    fmt = FORMATS[i % len(FORMATS)]
    qk = 256 if fmt in (12, 13, 14) else 32
    nb = int(rng.integers(1, 24 if qk == 256 else 160))
    cols = nb * qk - int(rng.integers(0, qk)) if rng.random() < 0.5 else nb * qk
    rows = int(rng.choice([1, 3, 17, 64, 65, 300, 777]))
    M = int(rng.choice([16, 17, 33, 64]))
    return fmt, rows, max(1, cols), M, rng


@pytest.mark.parametrize("i", range(N_CASES_2))
def test_random_shape_modes_int8_grouped(gq, oracle, i):
    """The prefill product's accumulate and SwiGLU forms at M >= 16 (the
    matrix-core routes), the int8-activation pair (Q8_0, Q4_K) and the
    grouped expert product on seeded random shapes."""
    fmt, rows, cols, M, rng = _case2(i)
    base = 8 if fmt == 1008 else fmt
    print(f"[random2 {i}] fmt={fmt} rows={rows} cols={cols} M={M}", flush=True)

    # gate|up tensor: 2 * rows weight rows
    W = synth.weights(base, 2 * rows, cols, rng)
    X = synth.activations((M, cols), rng)
    Wd, Xd = to_dev(W), to_dev(X)
    if fmt == 1008:
        Wd = gq.gq_q8_0_split_repack(Wd, 2 * rows, cols)
    rb = gq.gq_row_bytes(fmt, cols)
    GU, S = oracle.matmul(base, W, 2 * rows, cols, X, nthreads=oracle_threads())

    # accumulate: Y0 + gq_matmul of the gate half, bit for bit
    Y0 = synth.activations((M, rows), rng).astype(np.float32)
    Ya = sentinel_buffer(M * rows)
    Ya[:M * rows].copy_(to_dev(Y0.reshape(-1)))
    gq.gq_matmul_acc(fmt, Wd[:rows * rb], rows, cols, Xd, Y=Ya[:M * rows])
    assert_pad_untouched(Ya, M * rows)
    P = to_host(gq.gq_matmul(fmt, Wd[:rows * rb], rows, cols, Xd))
    assert np.array_equal(to_host(Ya)[:M * rows].reshape(M, rows).view(np.uint32),
                          (Y0 + P).view(np.uint32))
    assert_within_tolerance(P, GU[:, :rows], S[:, :rows], "matmul (gate half)")

    # SwiGLU: the derived bound against the f64 oracle
    Ys = sentinel_buffer(M * rows)
    gq.gq_matmul_swiglu(fmt, Wd, rows, cols, Xd, Y=Ys[:M * rows])
    assert_pad_untouched(Ys, M * rows)
    ys = to_host(Ys)[:M * rows].reshape(M, rows).astype(np.float64)
    g, u = GU[:, :rows], GU[:, rows:]
    eg, eu = 2e-4 * S[:, :rows], 2e-4 * S[:, rows:]
    y_ref = oracle.silu(g) * u
    bound = 1.1 * eg * (np.abs(u) + eu) + (np.abs(oracle.silu(g)) + 1.1 * eg) * eu
    bound += 8 * U32 * np.abs(y_ref) + 1e-30
    assert (np.abs(ys - y_ref) <= bound).all()

    # int8 activations (Q8_0 and Q4_K weights): quantiser byte-exact, matvec
    # within 2e-4 * sum |w x^| of W x^
    if fmt in (8, 12):
        import torch
        nbytes = gq.gq_row_bytes(gq.GQ_FMT_Q8_1, cols)
        xq = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
        gq.gq_quantize_q8_1(Xd[0], 1, cols, out=xq[:nbytes])
        hq = to_host(xq)
        assert (hq[nbytes:] == 0xA5).all()
        want_q = oracle.quantize_q8_1(X[0])
        assert np.array_equal(hq[:nbytes], want_q)
        y = sentinel_buffer(rows)
        gq.gq_matvec_q8_1(fmt, Wd[:rows * rb], rows, cols, xq[:nbytes], y=y[:rows])
        assert_pad_untouched(y, rows)
        ref8, S8 = oracle.matvec_q8_1(fmt, W[:rows * rb], rows, cols, want_q,
                                      nthreads=oracle_threads())   # fmt is 8 or 12: rb is its own
        assert_within_tolerance(to_host(y)[:rows], ref8, S8, "int8 matvec")

    # grouped expert product: the two halves as two experts, random counts
    counts = [int(c) for c in rng.integers(0, M + 1, 2)]
    total = sum(counts)
    if total:
        Yg = sentinel_buffer(total * rows)
        gq.gq_matmul_experts(fmt, Wd, 2, rows, cols, Xd[:total] if total <= M else
                             to_dev(np.concatenate([X, X])[:total]), counts, Y=Yg[:total * rows])
        assert_pad_untouched(Yg, total * rows)
        got = to_host(Yg)[:total * rows].reshape(total, rows)
        Xg = np.concatenate([X, X])[:total]
        o = 0
        for e, m in enumerate(counts):
            if m:
                rbb = gq.gq_row_bytes(base, cols)   # the host copy is in the base layout
                We = W[e * rows * rbb:(e + 1) * rows * rbb]
                ref_e, S_e = oracle.matmul(base, We, rows, cols, Xg[o:o + m], nthreads=oracle_threads())
                assert_within_tolerance(got[o:o + m], ref_e, S_e, f"grouped expert {e}")
            o += m
