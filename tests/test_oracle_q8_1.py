"""Pins for the oracle's Q8_1 activation quantiser (the int8-activation path
of the Loom porting skill, "What the starter generates": llama.cpp's Q8_1
numerics; the reading is spelled out in oracle/gq_oracle.c). Hand-worked
blocks, the closed form of ties-away rounding on a grid where the scale is
exactly 1, invariants (max code 127, power-of-two scaling, sign symmetry,
ragged tails), the error bound of the dequantised values, and a product that
is an exact integer."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def blocks(q, n, cols):
    """(d16, s16, codes) of every block of n rows."""
    nb = (cols + 31) // 32
    b = q.reshape(n, nb, 36)
    d16 = b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)
    s16 = b[:, :, 2].astype(np.uint16) | (b[:, :, 3].astype(np.uint16) << 8)
    return d16, s16, b[:, :, 4:].view(np.int8)


def test_row_bytes():
    assert oracle.row_bytes(oracle.TYPE_Q8_1, 32) == 36
    assert oracle.row_bytes(oracle.TYPE_Q8_1, 33) == 72
    assert oracle.row_bytes(oracle.TYPE_Q8_1, 4096) == 128 * 36


def test_hand_worked_block():
    # amax 127 -> d = 1, id = 1: codes are x rounded half away from zero
    x = np.zeros(32, np.float32)
    x[:8] = [127.0, -63.5, 2.5, -2.5, 0.5, -0.5, 0.49999997, -126.5]
    q = oracle.quantize_q8_1(x)
    assert q.size == 36
    d16, s16, c = blocks(q, 1, 32)
    assert d16[0, 0] == 0x3C00                        # 1.0
    assert list(c[0, 0, :8]) == [127, -64, 3, -3, 1, -1, 0, -127]
    assert (c[0, 0, 8:] == 0).all()
    # s = fp16(d * sum q) = fp16(-64)
    assert s16[0, 0] == 0xD400


def test_zero_block_and_ragged_tail():
    x = np.zeros(40, np.float32)
    x[32:40] = 3.0
    q = oracle.quantize_q8_1(x)
    assert q.size == 72
    assert (q[:36] == 0).all()                       # amax = 0: d = s = 0, codes 0
    d16, s16, c = blocks(q, 1, 40)
    # the 8 real values of block 1 map to 127, the 24 columns past cols to 0
    assert (c[0, 1, :8] == 127).all() and (c[0, 1, 8:] == 0).all()
    assert np.float16(3.0 / 127.0).view(np.uint16) == d16[0, 1]
    # values past cols in the caller's buffer do not matter
    y = np.concatenate([x, np.full(24, 1e9, np.float32)])
    assert np.array_equal(oracle.quantize_q8_1(y[:40]), q)


def test_ties_away_closed_form():
    # block max 127 gives d = 127/127 = 1 exactly, so x * id = x: every half
    # integer k/2 rounds to sign(k) * ceil(|k|/2)
    k = np.arange(-254, 255)
    vals = (k / 2.0).astype(np.float32)
    rows = []
    for i in range(0, vals.size, 31):
        chunk = np.zeros(32, np.float32)
        part = vals[i:i + 31]
        chunk[:part.size] = part
        chunk[31] = 127.0
        rows.append(chunk)
    X = np.stack(rows)
    q = oracle.quantize_q8_1(X)
    d16, _, c = blocks(q, X.shape[0], 32)
    assert (d16 == 0x3C00).all()
    got = c[:, :, :31].reshape(-1)[: vals.size].astype(np.int64)
    want = np.sign(k) * ((np.abs(k) + 1) // 2)
    assert np.array_equal(got, want)


def test_invariants_random():
    rng = np.random.default_rng(7)
    n, cols = 40, 300
    X = (rng.standard_normal((n, cols)) * np.exp2(rng.integers(-20, 20, size=(n, 1)))).astype(np.float32)
    q = oracle.quantize_q8_1(X)
    d16, s16, c = blocks(q, n, cols)
    nb = d16.shape[1]
    Xp = np.zeros((n, nb * 32), np.float32)
    Xp[:, :cols] = X
    Xb = Xp.reshape(n, nb, 32)
    amax = np.abs(Xb).max(axis=2)
    # the largest magnitude of every block maps to +-127, nothing exceeds it
    assert (np.abs(c.astype(np.int64)).max(axis=2)[amax > 0] == 127).all()
    # the code of the largest element carries its sign
    arg = np.abs(Xb).argmax(axis=2)
    top = np.take_along_axis(c, arg[:, :, None], axis=2)[:, :, 0]
    assert (np.sign(top) == np.sign(np.take_along_axis(Xb, arg[:, :, None], axis=2)[:, :, 0])).all()
    # sign symmetry and exact power-of-two scaling
    assert np.array_equal(blocks(oracle.quantize_q8_1(-X), n, cols)[2], -c)
    q2 = oracle.quantize_q8_1(X * np.float32(2.0 ** 5))
    d2, _, c2 = blocks(q2, n, cols)
    assert np.array_equal(c2, c)
    ok = (d16 > 0x0400) & (d2 < 0x7800)              # both scales normal fp16
    assert np.array_equal(d2[ok], d16[ok] + (5 << 10))
    # s = fp16(d * sum q)
    d32 = amax / np.float32(127.0)
    sums = c.astype(np.int64).sum(axis=2).astype(np.float32)
    assert np.array_equal(s16, (sums * d32).astype(np.float32).astype(np.float16).view(np.uint16))


def test_dequant_error_bound():
    rng = np.random.default_rng(8)
    n, cols = 16, 512
    X = (rng.standard_normal((n, cols)) * 3.0).astype(np.float32)
    q = oracle.quantize_q8_1(X)
    xh = oracle.dequant_q8_1(q, n, cols)
    d16, _, c = blocks(q, n, cols)
    # x^ is fp16 d times q, decoded independently here with numpy's fp16
    dv = d16.view(np.float16).astype(np.float64)
    want = (dv[:, :, None] * c.astype(np.float64)).reshape(n, -1)[:, :cols]
    assert np.array_equal(xh.astype(np.float64), want)
    # |x - x^| <= d/2 + 127 |d - fp16(d)| (rounding to the grid of d, then
    # the grid's scale stored in fp16), with a few ulps for the f32 steps
    amax = np.abs(X.reshape(n, -1, 32)).max(axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float64)
    bound = d32 / 2 + 127 * np.abs(d32 - dv) + 4e-7 * amax
    err = np.abs(X.astype(np.float64) - xh.astype(np.float64)).reshape(n, -1, 32)
    assert (err <= bound[:, :, None]).all()


def test_product_is_integer_with_unit_scales():
    # Q8_0 weights with d = 1 and activations with block max 127 (d = 1):
    # every product term is an integer, so W x^ is an exact integer sum
    rng = np.random.default_rng(9)
    rows, cols = 5, 64
    codes = rng.integers(-128, 128, size=(rows, cols)).astype(np.int8)
    W = np.zeros((rows, cols // 32, 34), np.uint8)
    W[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    W[:, :, 2:] = codes.reshape(rows, cols // 32, 32).view(np.uint8)
    xi = rng.integers(-127, 128, size=cols).astype(np.float32)
    xi[0] = 127.0
    xi[32] = -127.0
    q = oracle.quantize_q8_1(xi)
    y, S = oracle.matvec_q8_1(8, W.reshape(-1), rows, cols, q)
    want = codes.astype(np.int64) @ xi.astype(np.int64)
    assert np.array_equal(y, want.astype(np.float64))
    assert np.array_equal(S, (np.abs(codes.astype(np.int64)) @ np.abs(xi.astype(np.int64))).astype(np.float64))


def test_scale_whose_reciprocal_overflows():
    # largest magnitude 1e-38: d = amax / 127 is below 2^-128, so 1 / d is
    # +inf and x * (1 / d) is +-inf (x != 0) or NaN (x = 0). The reading
    # clamps: codes +-127 by sign, 0 for zeros; fp16(d) and fp16(d sum q)
    # are 0, so every x^ is 0.
    x = np.zeros(32, np.float32)
    x[0], x[1], x[5] = 1e-38, -1e-38, 3e-39
    d32 = np.float32(1e-38) / np.float32(127.0)
    assert d32 < np.float32(2.0 ** -128)
    with np.errstate(divide="ignore", over="ignore"):
        assert np.isinf(np.float32(1.0) / d32)
    q = oracle.quantize_q8_1(x)
    d16, s16, c = blocks(q, 1, 32)
    want = np.zeros(32, np.int64)
    want[0], want[1], want[5] = 127, -127, 127
    assert np.array_equal(c[0, 0].astype(np.int64), want)
    assert d16[0, 0] == 0 and s16[0, 0] == 0
    assert (oracle.dequant_q8_1(q, 1, 32) == 0).all()
    # the largest block whose reciprocal still is finite keeps its codes
    y = np.zeros(32, np.float32)
    y[0] = np.float32(2.0 ** -128) * np.float32(127.0) * np.float32(1.0 + 2.0 ** -20)
    y[1] = -y[0] / np.float32(2.0)
    with np.errstate(divide="ignore", over="ignore"):
        assert np.isfinite(np.float32(1.0) / (y[0] / np.float32(127.0)))
    cq = blocks(oracle.quantize_q8_1(y), 1, 32)[2][0, 0].astype(np.int64)
    assert cq[0] == 127 and cq[1] == -64 and (cq[2:] == 0).all()


def test_weights_of_type_q8_1_are_rejected():
    with pytest.raises(Exception):
        oracle.dequant(oracle.TYPE_Q8_1, np.zeros(36, np.uint8), 1, 32)
