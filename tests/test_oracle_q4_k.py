"""Pins for the oracle's Q4_K decode.

Q4_K is named on the pages ("nurllama" README, "What it runs"; the
nx_f32_llm_v4 source notes it is about 4.5 bits per weight) but its byte
layout is not printed there; the public GGUF layout is used:

  bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 twelve scale bytes, 16-143 codes.
  Scale bytes, as 96 bits: for j < 4, byte j holds sc_j in bits 0-5 and the
  top two bits of sc_{j+4} in bits 6-7; byte 4+j holds m_j and the top two
  bits of m_{j+4}; byte 8+j holds the low four bits of sc_{j+4} (bits 0-3)
  and of m_{j+4} (bits 4-7).
  Weight i = 64g + 32h + l lives in sub-block j = 2g + h; its 4-bit code is
  nibble h (0 = low) of code byte 32g + l.
  w = (d * sc_j) * code - dmin * m_j.

The test side packs fields into bytes from that description; the oracle
decodes them. The arithmetic is pinned by the closed form
float32(float64(d)*sc*code - float64(dmin)*m) over all 64 x 64 x 16
(sc, m, code) combinations, and the layout by hand-built blocks with known
values and a packing bijection.
"""
import numpy as np
import pytest


def pack_scales(sc, m) -> np.ndarray:
    """Test-side packer: eight 6-bit sc and m codes -> 12 bytes."""
    sc = np.asarray(sc, np.int64)
    m = np.asarray(m, np.int64)
    s = np.zeros(12, np.int64)
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[4 + j] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[8 + j] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return s.astype(np.uint8)


def pack_codes(codes) -> np.ndarray:
    """256 four-bit codes (weight order) -> 128 code bytes."""
    codes = np.asarray(codes, np.int64).reshape(256)
    qs = np.zeros(128, np.int64)
    for g in range(4):
        for l in range(32):
            qs[32 * g + l] = codes[64 * g + l] | (codes[64 * g + 32 + l] << 4)
    return qs.astype(np.uint8)


def make_block(d16: int, dmin16: int, sc, m, codes) -> np.ndarray:
    b = np.zeros(144, np.uint8)
    b[0], b[1] = d16 & 0xFF, d16 >> 8
    b[2], b[3] = dmin16 & 0xFF, dmin16 >> 8
    b[4:16] = pack_scales(sc, m)
    b[16:] = pack_codes(codes)
    return b


def f16(v: float) -> int:
    return int(np.array(v, np.float16).view(np.uint16))


def test_scale_packing_bijection_random(oracle):
    rng = np.random.default_rng(7)
    for _ in range(20000):
        s = rng.integers(0, 256, 12, dtype=np.uint8)
        sc, m = oracle.q4_k_unpack_scales(s)
        assert sc.max() < 64 and m.max() < 64
        assert np.array_equal(pack_scales(sc, m), s)


def test_scale_packing_every_code_every_position(oracle):
    rng = np.random.default_rng(8)
    for pos in range(16):
        for v in range(64):
            sc = rng.integers(0, 64, 8)
            m = rng.integers(0, 64, 8)
            (sc if pos < 8 else m)[pos % 8] = v
            got_sc, got_m = oracle.q4_k_unpack_scales(pack_scales(sc, m))
            assert np.array_equal(got_sc, sc) and np.array_equal(got_m, m)


def test_hand_built_block_large_codes(oracle):
    # d = 1, dmin = 0.5, sc_j = 56 + j, m_j = 40 + 3j (all >= 16, so the
    # high two bits of every 6-bit code are exercised), code_i = i mod 16.
    sc = [56 + j for j in range(8)]
    m = [40 + 3 * j for j in range(8)]
    codes = [i % 16 for i in range(256)]
    blk = make_block(0x3C00, 0x3800, sc, m, codes)
    got = oracle.dequant(12, blk, 1, 256)[0]
    want = [(56 + i // 32) * (i % 16) - 0.5 * (40 + 3 * (i // 32)) for i in range(256)]
    assert list(got) == want


def test_hand_built_block_distinguishes_nibbles(oracle):
    # codes differ between the low (h=0) and high (h=1) nibble halves and
    # between groups g: code_i = (i // 16) mod 16. d = 0.25, dmin = -1.
    sc = [j + 1 for j in range(8)]
    m = [2 * j for j in range(8)]
    codes = [(i // 16) % 16 for i in range(256)]
    blk = make_block(f16(0.25), f16(-1.0), sc, m, codes)
    got = oracle.dequant(12, blk, 1, 256)[0]
    want = [0.25 * (i // 32 + 1) * ((i // 16) % 16) + 2 * (i // 32) for i in range(256)]
    assert list(got) == want
    # spot values written out by hand
    assert got[0] == 0.0            # j=0, code 0
    assert got[16] == 0.25          # j=0, code 1
    assert got[32] == 0.5 * 2 + 2   # j=1: sc=2, code 2, m=2 -> 0.25*2*2 + 2
    assert got[255] == 0.25 * 8 * 15 + 14


def test_closed_form_exhaustive_grid(oracle):
    """All (sc, m, code) in 64 x 64 x 16 for several (d, dmin)."""
    pairs = np.array([(s, mm) for s in range(64) for mm in range(64)])  # 4096
    nsb = pairs.shape[0] // 8                                            # 512
    codes = np.array([l % 16 for l in range(32)] * 8)                    # per block
    dd = [(1.0, 0.5), (-1.5, 1.0), (0.0, 0.5), (2.0 ** -24, 65504.0),
          (65504.0, 2.0 ** -24), (2.0 ** -14, -2.5), (0.000123, 0.00091),
          (-7.25, -0.0009765625)]
    blocks = []
    for d, dmin in dd:
        for b in range(nsb):
            p = pairs[8 * b:8 * b + 8]
            blocks.append(make_block(f16(d), f16(dmin), p[:, 0], p[:, 1], codes))
    W = np.concatenate(blocks)
    got = oracle.dequant(12, W, len(blocks), 256)
    k = 0
    for d, dmin in dd:
        d64 = np.float64(np.float16(d))
        dm64 = np.float64(np.float16(dmin))
        for b in range(nsb):
            p = pairs[8 * b:8 * b + 8]
            j = np.arange(256) // 32
            want = (d64 * p[j, 0] * codes - dm64 * p[j, 1]).astype(np.float32)
            assert np.array_equal(got[k].view(np.uint32), want.view(np.uint32)), (d, dmin, b)
            k += 1


def test_ragged_tail_is_ignored(oracle):
    rng = np.random.default_rng(11)
    rows, cols = 3, 896                  # 4 super-blocks per row, last half used
    rb = oracle.row_bytes(12, cols)
    assert rb == 4 * 144
    W = rng.integers(0, 256, rows * rb, dtype=np.uint8)
    W.reshape(rows, 4, 144)[:, :, 1] = 0x30   # keep d, dmin finite and moderate
    W.reshape(rows, 4, 144)[:, :, 3] = 0x30
    ref = oracle.dequant(12, W, rows, cols)
    W2 = W.copy().reshape(rows, 4, 144)
    last = W2[:, 3]
    # fields that belong only to sub-blocks 4..7 of the last super-block
    last[:, 12:16] = rng.integers(0, 256, (rows, 4), dtype=np.uint8)
    last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, (rows, 8), dtype=np.uint8) << 6)
    last[:, 16 + 64:] = rng.integers(0, 256, (rows, 64), dtype=np.uint8)
    got = oracle.dequant(12, W2.reshape(-1), rows, cols)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("cols", [256, 300, 512 + 40])
def test_row_bytes_and_partial_rows(oracle, cols):
    nb = -(-cols // 256)
    assert oracle.row_bytes(12, cols) == 144 * nb
    rng = np.random.default_rng(cols)
    W = rng.integers(0, 256, 2 * 144 * nb, dtype=np.uint8)
    W.reshape(2, nb, 144)[:, :, 1] = 0x2C
    W.reshape(2, nb, 144)[:, :, 3] = 0x2C
    full = oracle.dequant(12, W, 2, 256 * nb)
    part = oracle.dequant(12, W, 2, cols)
    assert np.array_equal(full[:, :cols], part)
