"""Pins for the oracle's Q8_0 dequant.

Q8_0 weight = d * q with d an fp16 and q an int8: the product of an 11-bit and
an 8-bit significand is exact in binary32, so the closed form
float32(float64(d) * q) is the exact answer. It is checked for every finite
fp16 d against all 256 codes (including -128, which the format allows).
The block byte layout (d first, little endian, then 32 int8) is the public
GGUF one; the pages only name the format ("nurllama 0.18.1 API", model.nu).
"""
import numpy as np


def _block_bytes(d16: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Test-side packing: d16 [n] uint16, q [n, 32] int8 -> [n*34] uint8."""
    n = d16.shape[0]
    b = np.empty((n, 34), np.uint8)
    b[:, 0] = d16 & 0xFF
    b[:, 1] = d16 >> 8
    b[:, 2:] = q.astype(np.int8).view(np.uint8)
    return b.reshape(-1)


def test_q8_0_closed_form_exhaustive(oracle):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(bits.view(np.float16))
    d16 = bits[finite]                                    # 63,488 values
    q_all = np.arange(-128, 128, dtype=np.int16).reshape(8, 32)
    d_rep = np.repeat(d16, 8)
    q = np.tile(q_all, (d16.size, 1))
    W = _block_bytes(d_rep, q)
    rows = d16.size
    got = oracle.dequant(8, W, rows, 256)                 # 8 blocks per row
    ref = (d16.view(np.float16).astype(np.float64)[:, None]
           * np.arange(-128, 128, dtype=np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_q8_0_hand_block(oracle):
    # d = 0.5 (0x3800), q = [-128, -127, ..., 0 ..] known values
    q = np.array([-128, -127, -1, 0, 1, 2, 127] + list(range(-12, 13)), np.int16)
    assert q.size == 32
    W = _block_bytes(np.array([0x3800], np.uint16), q.reshape(1, 32))
    got = oracle.dequant(8, W, 1, 32)[0]
    assert list(got[:7]) == [-64.0, -63.5, -0.5, 0.0, 0.5, 1.0, 63.5]
    assert np.array_equal(got, q.astype(np.float32) * 0.5)


def test_q8_0_negative_and_subnormal_scale(oracle):
    q = np.arange(-16, 16, dtype=np.int16).reshape(1, 32)
    for d16, dval in [(0xB800, -0.5), (0x0001, 2.0 ** -24), (0x8003, -3 * 2.0 ** -24)]:
        W = _block_bytes(np.array([d16], np.uint16), q)
        got = oracle.dequant(8, W, 1, 32)[0]
        ref = (np.float64(dval) * q[0].astype(np.float64)).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # q = 0 with d < 0 gives -0.0
    W = _block_bytes(np.array([0xB800], np.uint16), np.zeros((1, 32), np.int16))
    assert np.all(np.signbit(oracle.dequant(8, W, 1, 32)))


def test_q8_0_ragged_and_row_stride(oracle):
    rng = np.random.default_rng(5)
    rows, cols = 3, 70                                    # 3 blocks per row, last partial
    nb = 3
    d16 = np.full(rows * nb, 0x3C00, np.uint16)           # d = 1
    q = rng.integers(-128, 128, size=(rows * nb, 32)).astype(np.int16)
    W = _block_bytes(d16, q)
    assert oracle.row_bytes(8, cols) == nb * 34
    got = oracle.dequant(8, W, rows, cols)
    ref = q.reshape(rows, nb * 32)[:, :cols].astype(np.float32)
    assert np.array_equal(got, ref)
