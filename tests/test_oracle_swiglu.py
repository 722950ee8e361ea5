"""Pins for the oracle's SwiGLU pieces: silu against closed forms and
identities, and the gate|up row order of the fused tensor against a
hand-built matrix whose gate and up sums are known exactly."""
import math

import numpy as np

import synth


def test_silu_closed_forms(oracle):
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert abs(oracle.silu(ln3) - 0.75 * ln3) <= 2e-16
    assert abs(oracle.silu(-ln3) + 0.25 * ln3) <= 2e-16
    assert oracle.silu(0.0) == 0.0
    # sigmoid(ln 9) = 9/10
    assert abs(oracle.silu(math.log(9.0)) - 0.9 * math.log(9.0)) <= 4e-16
    assert oracle.silu(800.0) == 800.0
    big_neg = oracle.silu(-800.0)
    assert big_neg == 0.0 and math.copysign(1.0, big_neg) == -1.0


def test_silu_identities():
    import oracle
    v = np.random.default_rng(30).normal(0, 6, 10000)
    # silu(v) - silu(-v) = v * (sigmoid(v) + sigmoid(-v)) = v
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-12 * np.abs(v).max())
    # silu(v) / v = sigmoid(v) is increasing and in (0, 1)
    order = np.argsort(v)
    sig = oracle.silu(v[order]) / v[order]
    assert np.all(np.diff(sig) >= -1e-15) and np.all((sig > 0) & (sig < 1))


def test_silu_derivative_bound():
    """|silu'| <= 1.1 everywhere (the maximum is about 1.0998 near v = 2.4);
    the GPU tolerance for the fused gate|up epilogue relies on it."""
    import oracle
    v = np.linspace(-40, 40, 800001)
    h = 1e-6
    d = (oracle.silu(v + h) - oracle.silu(v - h)) / (2 * h)
    assert d.max() < 1.0999 and d.min() > -0.1
    assert abs(d.max() - 1.0998) < 2e-4


def test_swiglu_gate_rows_come_first(oracle):
    """Q8_0, 2 output rows, one block: gate rows have q = 1 everywhere (d =
    0.5 / 1.0), up rows q = 2 (d = 1.0 / 0.25); x = 1/32 everywhere, so
    g = (0.5, 1.0), u = (2.0, 0.5) exactly."""
    rows, cols = 2, 32
    x = np.full(cols, 1.0 / 32, np.float32)

    def blk(d16, q):
        b = np.zeros(34, np.uint8)
        b[0], b[1] = d16 & 0xFF, d16 >> 8
        b[2:] = q
        return b

    W = np.concatenate([blk(0x3800, 1), blk(0x3C00, 1), blk(0x3C00, 2), blk(0x3400, 2)])
    y, g, u, Sg, Su = oracle.swiglu_matvec(8, W, rows, cols, x)
    assert list(g) == [0.5, 1.0] and list(u) == [2.0, 0.5]
    want = [0.5 / (1 + math.exp(-0.5)) * 2.0, 1.0 / (1 + math.exp(-1.0)) * 0.5]
    assert np.allclose(y, want, rtol=1e-15, atol=0)
    assert list(Sg) == [0.5, 1.0] and list(Su) == [2.0, 0.5]


def test_swiglu_matches_two_matvecs(oracle):
    rng = synth.rng_for(31, 0)
    rows, cols = 7, 512
    W = synth.weights(12, 2 * rows, cols, rng)
    x = synth.activations(cols, rng)
    y, g, u, Sg, Su = oracle.swiglu_matvec(12, W, rows, cols, x)
    rb = oracle.row_bytes(12, cols)
    g2, sg2 = oracle.matvec(12, W[: rows * rb], rows, cols, x)
    u2, su2 = oracle.matvec(12, W[rows * rb:], rows, cols, x)
    assert np.array_equal(g, g2) and np.array_equal(u, u2)
    assert np.array_equal(Sg, sg2) and np.array_equal(Su, su2)
    assert np.array_equal(y, oracle.silu(g2) * u2)
