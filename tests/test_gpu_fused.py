"""The fused decode variants on the GPU: the gate|up matvec with the SwiGLU
activation applied before the store, the accumulating matvec, and fused
q|k|v / gate|up tensors passed whole to gq_matvec (their parts are row
ranges). Each is checked against the f64 oracle and against the plain
gq_matvec on the same rows."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # unit roundoff of fp32


def _swiglu(gq, fmt, W, rows, cols, x):
    y = sentinel_buffer(rows)
    gq.gq_matvec_swiglu(fmt, to_dev(W) if isinstance(W, np.ndarray) else W, rows, cols,
                        to_dev(x) if isinstance(x, np.ndarray) else x, y=y)
    assert_pad_untouched(y, rows)
    return to_host(y)[:rows]


def _matvec(gq, fmt, W, rows, cols, x):
    y = sentinel_buffer(rows)
    gq.gq_matvec(fmt, W, rows, cols, x, y=y)
    assert_pad_untouched(y, rows)
    return to_host(y)[:rows]


def _silu_mul_f32(g, u):
    g = g.astype(np.float32)
    with np.errstate(over="ignore"):
        return (g / (np.float32(1) + np.exp(-g)) * u.astype(np.float32)).astype(np.float32)


SWIGLU_SHAPES = [
    (12, 14336, 4096),   # Llama-3-8B gate|up, 2 x 14336 rows
    (12, 4864, 896),     # Qwen2.5-0.5B gate|up, ragged Q4_K rows
    (8, 1536, 576),      # SmolLM-135M gate|up, Q8_0 block pairs
    (8, 300, 96),        # single Q8_0 blocks (odd block count)
    (14, 1024, 4096), (13, 1024, 4096), (6, 700, 896),
    (12, 1, 256), (12, 3, 300), (12, 65, 14336),  # 14336 columns: 4-wave row groups
    (12, 5, 33024), (8, 9, 40000),                # wider than 256 units: segmented rows
]


@pytest.mark.parametrize("fmt,rows,cols", SWIGLU_SHAPES)
def test_swiglu_against_oracle_and_matvec(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(950, fmt * 10 ** 6 + rows)
    W = synth.weights(fmt, 2 * rows, cols, rng)
    x = synth.activations(cols, rng)
    print(f"[fused] swiglu fmt={fmt} rows={rows} cols={cols}", flush=True)
    Wd, xd = to_dev(W), to_dev(x)
    y = _swiglu(gq, fmt, Wd, rows, cols, xd)
    # 1. against the f64 oracle: g and u are each within 2e-4 * S of theirs,
    # |silu'| <= 1.1, and the fp32 activation adds a few roundings.
    y_ref, g_ref, u_ref, Sg, Su = oracle.swiglu_matvec(fmt, W, rows, cols, x,
                                                      nthreads=oracle_threads())
    eg, eu = 2e-4 * Sg, 2e-4 * Su
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + (np.abs(oracle.silu(g_ref)) + 1.1 * eg) * eu
    bound += 8 * U32 * np.abs(y_ref) + 1e-30
    err = np.abs(y.astype(np.float64) - y_ref)
    assert not np.isnan(y).any()
    bad = err > bound
    assert not bad.any(), (np.flatnonzero(bad)[:5], y[bad][:5], y_ref[bad][:5])
    # 2. against the plain matvec of the two halves, with the activation
    # evaluated on the host in fp32: the sums are the same bits, so only the
    # exp (two implementations, each within ~1 ulp), divide and multiply
    # roundings can differ -- up to about 5 ulp of y where 1 + e^-g ~ e^-g.
    gu = _matvec(gq, fmt, Wd, 2 * rows, cols, xd)
    y_host = _silu_mul_f32(gu[:rows], gu[rows:])
    assert np.all(np.abs(y - y_host) <= 8 * U32 * np.abs(y_host) + 1e-37), \
        np.max(np.abs(y - y_host) / np.maximum(np.abs(y_host), 1e-30))


def test_swiglu_extreme_gates(gq, oracle):
    """Gate sums far in the tails: silu(-large) = -0 * u, silu(+large) = g."""
    rows, cols = 4, 32
    x = np.ones(cols, np.float32)

    def blk(d16, q):
        b = np.zeros(34, np.uint8)
        b[0], b[1] = d16 & 0xFF, d16 >> 8
        b[2:] = np.array(q, np.int8).view(np.uint8)
        return b

    # gate sums: 32*127*d for d = 32 (-> 130048), -32 (-> -130048), 0, tiny
    gate = [blk(0x5000, 127), blk(0xD000, 127), blk(0x0000, 5), blk(0x0001, 1)]
    up = [blk(0x3C00, 3)] * 4          # u = 96
    W = np.concatenate(gate + up)
    y = _swiglu(gq, 8, W, rows, cols, x)
    y_ref, g_ref, u_ref, _, _ = oracle.swiglu_matvec(8, W, rows, cols, x)
    assert y[0] == np.float32(130048.0 * 96) and y[1] == 0.0 and y[2] == 0.0
    assert abs(y[3] - y_ref[3]) <= 4 * U32 * abs(y_ref[3])


@pytest.mark.parametrize("fmt,rows,cols", [(12, 4096, 4096), (12, 4096, 14336), (8, 1536, 576),
                                           (8, 301, 96), (14, 4096, 4096), (12, 3, 300)])
def test_acc_adds_the_matvec(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(951, fmt * 10 ** 6 + rows)
    W = synth.weights(fmt, rows, cols, rng)
    x = synth.activations(cols, rng)
    y0 = synth.activations(rows, rng) * np.float32(3.0)
    print(f"[fused] acc fmt={fmt} rows={rows} cols={cols}", flush=True)
    Wd, xd = to_dev(W), to_dev(x)
    y = sentinel_buffer(rows)
    y[:rows].copy_(to_dev(y0))
    gq.gq_matvec_acc(fmt, Wd, rows, cols, xd, y)
    assert_pad_untouched(y, rows)
    got = to_host(y)[:rows]
    # one fp32 addition onto the plain matvec's result, bit for bit
    plain = _matvec(gq, fmt, Wd, rows, cols, xd)
    assert np.array_equal(got.view(np.uint32), (y0 + plain).view(np.uint32))
    ref, S = oracle.matvec(fmt, W, rows, cols, x, nthreads=oracle_threads())
    err = np.abs(got.astype(np.float64) - (y0.astype(np.float64) + ref))
    assert np.all(err <= 2e-4 * S + U32 * np.abs(y0.astype(np.float64) + ref) + 1e-30)


def test_fused_qkv_tensor_equals_separate_calls(gq):
    """A q|k|v tensor (Llama-3-8B layer 0 shapes) passed whole: the rows of
    each part come out bit for bit as from the part's own call."""
    parts = [synth.llama3_8b_weight_and_x(0, p)[0] for p in range(3)]   # q, k, v
    rows = [4096, 1024, 1024]
    cols = 4096
    x = synth.activations(cols, synth.rng_for(952, 0))
    xd = to_dev(x)
    whole = _matvec(gq, 12, to_dev(np.concatenate(parts)), sum(rows), cols, xd)
    off = 0
    for W, r in zip(parts, rows):
        y = _matvec(gq, 12, to_dev(W), r, cols, xd)
        assert np.array_equal(y.view(np.uint32), whole[off:off + r].view(np.uint32))
        off += r


def test_swiglu_row_range_of_a_larger_tensor(gq, oracle):
    """The gate|up pair addressed inside a bigger buffer (a row-range view):
    the kernel reads only its 2 * rows rows."""
    rows, cols = 96, 1024
    rng = synth.rng_for(953, 0)
    W = synth.weights(12, 2 * rows + 7, cols, rng)
    x = synth.activations(cols, rng)
    rb = oracle.row_bytes(12, cols)
    Wd = to_dev(W)
    sub = W[3 * rb:(3 + 2 * rows) * rb]
    y = _swiglu(gq, 12, Wd[3 * rb:], rows, cols, to_dev(x))
    y_ref, g_ref, u_ref, Sg, Su = oracle.swiglu_matvec(12, sub, rows, cols, x)
    eg, eu = 2e-4 * Sg, 2e-4 * Su
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + (np.abs(oracle.silu(g_ref)) + 1.1 * eg) * eu
    assert np.all(np.abs(y - y_ref) <= bound + 8 * U32 * np.abs(y_ref) + 1e-30)
