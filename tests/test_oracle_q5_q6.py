"""Pins for the oracle's Q5_0, Q5_K and Q6_K decode.

The pages name these formats next to Q4_K ("nurllama" README, "What it runs";
"nurllama 0.18.1 API", kernels.nu section, its per-format kernel list) but
print none of their byte layouts. The public GGUF layouts are used, restated
here as the test side packs them:

  Q5_0 (22 B / 32 weights): bytes 0-1 d (fp16); bytes 2-5 a little-endian
    32-bit word whose bit i is bit 4 of code i; bytes 6-21: byte b holds the
    low four bits of code b (bits 0-3) and of code 16 + b (bits 4-7).
    w_i = d * (code_i - 16).
  Q5_K (176 B / 256 weights): bytes 0-15 as in Q4_K (d, dmin, the twelve
    6-bit scale / min bytes); bytes 16-47 qh; bytes 48-175 the low nibbles,
    placed as Q4_K places its codes. Weight i = 64g + 32h + l (sub-block
    j = 2g + h) takes bit j of qh[l] as bit 4 of its code.
    w_i = (d * sc_j) * code_i - dmin * m_j.
  Q6_K (210 B / 256 weights): bytes 0-127 ql, 128-191 qh, 192-207 sixteen
    int8 scales, 208-209 d (fp16). Weight i = 128n + 32k + l takes its low
    four bits from nibble k >> 1 of ql[64n + 32(k & 1) + l], its high two bits
    from bits 2k, 2k+1 of qh[32n + l], and scale i // 16.
    w_i = (d * scale_{i//16}) * (code_i - 32).

The packers below scatter codes into bytes from that description (the
oracle gathers them); the arithmetic is pinned by closed forms over every
code and scale value, evaluated here in float64 and rounded once to float32.
All three products are exact in float32 (Q6_K: an 11-bit fp16 significand
times |scale * (code - 32)| <= 4096 stays below 2^24), so the closed form is
the value itself, bit for bit.
"""
import numpy as np
import pytest

from test_oracle_q4_k import pack_scales

Q5_0, Q5_K, Q6_K = 6, 13, 14


def f16(v: float) -> int:
    return int(np.array(v, np.float16).view(np.uint16))


def put16(b: np.ndarray, at: int, bits: int) -> None:
    b[at], b[at + 1] = bits & 0xFF, bits >> 8


# ------------------------------------------------------------------ packers

def make_q5_0(d16: int, codes) -> np.ndarray:
    codes = [int(c) for c in codes]
    assert len(codes) == 32 and all(0 <= c < 32 for c in codes)
    b = np.zeros(22, np.uint8)
    put16(b, 0, d16)
    qh = 0
    for i, c in enumerate(codes):
        qh |= (c >> 4) << i
    for k in range(4):
        b[2 + k] = (qh >> (8 * k)) & 0xFF
    for i in range(16):
        b[6 + i] = (codes[i] & 15) | ((codes[16 + i] & 15) << 4)
    return b


def make_q5_k(d16: int, dmin16: int, sc, m, codes) -> np.ndarray:
    codes = [int(c) for c in codes]
    assert len(codes) == 256 and all(0 <= c < 32 for c in codes)
    b = np.zeros(176, np.uint8)
    put16(b, 0, d16)
    put16(b, 2, dmin16)
    b[4:16] = pack_scales(sc, m)
    for i, c in enumerate(codes):
        g, h, l = i // 64, (i // 32) % 2, i % 32
        b[16 + l] |= (c >> 4) << (2 * g + h)
        b[48 + 32 * g + l] |= (c & 15) << (4 * h)
    return b


def make_q6_k(d16: int, scales, codes) -> np.ndarray:
    codes = [int(c) for c in codes]
    assert len(codes) == 256 and all(0 <= c < 64 for c in codes)
    scales = [int(s) for s in scales]
    assert len(scales) == 16 and all(-128 <= s < 128 for s in scales)
    b = np.zeros(210, np.uint8)
    for i, c in enumerate(codes):
        n, k, l = i // 128, (i // 32) % 4, i % 32
        b[64 * n + 32 * (k & 1) + l] |= (c & 15) << (4 * (k >> 1))
        b[128 + 32 * n + l] |= (c >> 4) << (2 * k)
    b[192:208] = np.array(scales, np.int8).view(np.uint8)
    put16(b, 208, d16)
    return b


def bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


# -------------------------------------------------------------------- Q5_0

def test_q5_0_closed_form_every_code(oracle):
    ds = [1.0, -0.5, 0.0, -0.0, 2.0 ** -24, 65504.0, 2.0 ** -14, 0.000123, -7.25, 3.0]
    codes = list(range(32))
    W = np.concatenate([make_q5_0(f16(d), codes) for d in ds])
    got = oracle.dequant(Q5_0, W, len(ds), 32)
    for r, d in enumerate(ds):
        want = np.float64(np.float16(d)) * (np.arange(32) - 16.0)
        assert np.array_equal(bits(got[r]), bits(want)), d


def test_q5_0_hand_block(oracle):
    # d = 0.5; code_i = 31 - i, so bit 4 is set exactly for i < 16 and the
    # low nibbles of the two halves differ: w_i = 0.5 * (15 - i).
    blk = make_q5_0(0x3800, [31 - i for i in range(32)])
    assert blk[2:6].tolist() == [0xFF, 0xFF, 0x00, 0x00]
    assert blk[6] == 0xFF and blk[21] == 0x00   # codes 31, 15 | codes 16, 0
    got = oracle.dequant(Q5_0, blk, 1, 32)[0]
    assert list(got) == [0.5 * (15 - i) for i in range(32)]
    assert got[0] == 7.5 and got[16] == -0.5 and got[31] == -8.0


def test_q5_0_high_bit_only(oracle):
    # low nibbles all zero, bit 4 set on odd weights: w = d * (16*odd - 16)
    blk = np.zeros(22, np.uint8)
    put16(blk, 0, 0x3C00)
    blk[2:6] = [0xAA, 0xAA, 0xAA, 0xAA]
    got = oracle.dequant(Q5_0, blk, 1, 32)[0]
    assert list(got) == [0.0 if i % 2 else -16.0 for i in range(32)]


def test_q5_0_ragged_tail_and_stride(oracle):
    rng = np.random.default_rng(21)
    rows, cols = 3, 40                   # 2 blocks per row, 8 columns used
    assert oracle.row_bytes(Q5_0, cols) == 44
    W = rng.integers(0, 256, rows * 44, dtype=np.uint8).reshape(rows, 2, 22)
    W[:, :, 1] = 0x2C                    # finite, moderate scales
    ref = oracle.dequant(Q5_0, W.reshape(-1), rows, cols)
    W2 = W.copy()
    last = W2[:, 1]
    # bits and nibbles of weights 8..31 of the last block
    last[:, 3:6] = rng.integers(0, 256, (rows, 3), dtype=np.uint8)
    last[:, 6 + 8:22] = rng.integers(0, 256, (rows, 8), dtype=np.uint8)
    last[:, 6:6 + 8] = (last[:, 6:6 + 8] & 0x0F) | (rng.integers(0, 16, (rows, 8), dtype=np.uint8) << 4)
    got = oracle.dequant(Q5_0, W2.reshape(-1), rows, cols)
    assert np.array_equal(bits(ref), bits(got))
    # each row starts at r * row_bytes: row 1 decoded alone equals row 1
    alone = oracle.dequant(Q5_0, W.reshape(rows, -1)[1], 1, cols)
    assert np.array_equal(bits(alone[0]), bits(ref[1]))


# -------------------------------------------------------------------- Q5_K

def test_q5_k_closed_form_grid(oracle):
    """Every (sc, m) pair with every 5-bit code, for several (d, dmin)."""
    pairs = np.array([(s, mm) for s in range(64) for mm in range(64)])  # 4096
    nsb = pairs.shape[0] // 8
    codes = [i % 32 for i in range(256)]           # each sub-block: 0..31
    dd = [(1.0, 0.5), (-1.5, 1.0), (2.0 ** -24, 65504.0), (0.000123, 0.00091),
          (-7.25, -0.0009765625)]
    blocks = []
    for d, dmin in dd:
        for b in range(nsb):
            p = pairs[8 * b:8 * b + 8]
            blocks.append(make_q5_k(f16(d), f16(dmin), p[:, 0], p[:, 1], codes))
    got = oracle.dequant(Q5_K, np.concatenate(blocks), len(blocks), 256)
    j = np.arange(256) // 32
    c = np.array(codes, np.float64)
    k = 0
    for d, dmin in dd:
        d64, dm64 = np.float64(np.float16(d)), np.float64(np.float16(dmin))
        for b in range(nsb):
            p = pairs[8 * b:8 * b + 8]
            want = d64 * p[j, 0] * c - dm64 * p[j, 1]
            assert np.array_equal(bits(got[k]), bits(want)), (d, dmin, b)
            k += 1


def test_q5_k_hand_block(oracle):
    # d = 1, dmin = 0.25, sc_j = j + 1, m_j = 4j; code_i = (i + i // 32) % 32
    # so that each sub-block's bit-4 pattern is shifted differently.
    sc = [j + 1 for j in range(8)]
    m = [4 * j for j in range(8)]
    codes = [(i + i // 32) % 32 for i in range(256)]
    blk = make_q5_k(0x3C00, f16(0.25), sc, m, codes)
    got = oracle.dequant(Q5_K, blk, 1, 256)[0]
    want = [(i // 32 + 1) * codes[i] - 0.25 * 4 * (i // 32) for i in range(256)]
    assert list(got) == want
    assert got[31] == 31.0                # j=0: code 31, sc 1, m 0
    assert got[32] == 2 * 1 - 1.0         # j=1: code 1, sc 2, m 4
    assert got[255] == 8 * ((255 + 7) % 32) - 7.0


def test_q5_k_qh_bits_select_sub_block(oracle):
    # all nibbles zero, qh[l] = 1 << (l % 8): only weight l of sub-block
    # j = l % 8 gets code 16. w = 16 * d * sc_j there and -dmin * m_j else.
    blk = np.zeros(176, np.uint8)
    put16(blk, 0, 0x3C00)
    put16(blk, 2, 0x3C00)
    blk[4:16] = pack_scales([1] * 8, [1] * 8)
    for l in range(32):
        blk[16 + l] = 1 << (l % 8)
    got = oracle.dequant(Q5_K, blk, 1, 256)[0]
    want = [15.0 if (i % 32) % 8 == i // 32 else -1.0 for i in range(256)]
    assert list(got) == want


def test_q5_k_ragged_tail(oracle):
    rng = np.random.default_rng(22)
    rows, cols = 3, 896                   # 4 super-blocks, half of the last used
    assert oracle.row_bytes(Q5_K, cols) == 4 * 176
    W = rng.integers(0, 256, rows * 4 * 176, dtype=np.uint8).reshape(rows, 4, 176)
    W[:, :, 1] = 0x30
    W[:, :, 3] = 0x30
    ref = oracle.dequant(Q5_K, W.reshape(-1), rows, cols)
    W2 = W.copy()
    last = W2[:, 3]
    # scale codes of sub-blocks 4..7, qh bits 4..7, nibbles of groups 2, 3
    last[:, 12:16] = rng.integers(0, 256, (rows, 4), dtype=np.uint8)
    last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, (rows, 8), dtype=np.uint8) << 6)
    last[:, 16:48] = (last[:, 16:48] & 0x0F) | (rng.integers(0, 16, (rows, 32), dtype=np.uint8) << 4)
    last[:, 48 + 64:] = rng.integers(0, 256, (rows, 64), dtype=np.uint8)
    got = oracle.dequant(Q5_K, W2.reshape(-1), rows, cols)
    assert np.array_equal(bits(ref), bits(got))


# -------------------------------------------------------------------- Q6_K

def test_q6_k_closed_form_every_scale_and_code(oracle):
    """All 256 int8 scales x all 64 codes, for several d."""
    codes = [i % 64 for i in range(256)]           # each 16-run: 16 codes
    ds = [1.0, -0.5, 2.0 ** -24, 65504.0 / 4096, 0.0000143, -3.75, 2.0 ** -14]
    blocks, want = [], []
    c = np.array(codes, np.float64) - 32.0
    for d in ds:
        d64 = np.float64(np.float16(d))
        # 16 scales per block; 64 codes span 4 scale groups, so cycle codes
        # through offsets to meet every (scale, code) pair
        for sb in range(16):                       # 16 blocks x 16 scales = 256
            scales = [((sb * 16 + t) % 256) - 128 for t in range(16)]
            for shift in range(4):
                cs = [(x + 16 * shift) % 64 for x in codes]
                blocks.append(make_q6_k(f16(d), scales, cs))
                cc = np.array(cs, np.float64) - 32.0
                want.append(d64 * np.array(scales, np.float64)[np.arange(256) // 16] * cc)
    got = oracle.dequant(Q6_K, np.concatenate(blocks), len(blocks), 256)
    assert np.array_equal(bits(got), bits(np.array(want)))
    assert c.min() == -32 and c.max() == 31


def test_q6_k_hand_block(oracle):
    # d = 0.5; scale_s = s - 8 (negative, zero and positive); code_i = i % 64
    scales = [s - 8 for s in range(16)]
    codes = [i % 64 for i in range(256)]
    blk = make_q6_k(0x3800, scales, codes)
    got = oracle.dequant(Q6_K, blk, 1, 256)[0]
    want = [0.5 * (i // 16 - 8) * (i % 64 - 32) for i in range(256)]
    assert list(got) == want
    assert got[0] == 0.5 * -8 * -32        # 128
    assert got[63] == 0.5 * -5 * 31
    assert got[128] == 0.0                 # scale 0
    assert got[255] == 0.5 * 7 * 31


def test_q6_k_positions_of_fields(oracle):
    # one code at a time set to 63 (others 32 -> 0): exactly that weight is
    # non-zero, with all scales 1 and d = 1
    base = [32] * 256
    for i in [0, 17, 31, 32, 63, 64, 100, 127, 128, 161, 200, 223, 224, 255]:
        cs = list(base)
        cs[i] = 63
        blk = make_q6_k(0x3C00, [1] * 16, cs)
        got = oracle.dequant(Q6_K, blk, 1, 256)[0]
        want = np.zeros(256, np.float32)
        want[i] = 31.0
        assert np.array_equal(got, want), i
    # the first byte of qh carries bits 4-5 of weights 0, 32, 64, 96
    blk = make_q6_k(0x3C00, [1] * 16, [0] * 256)
    blk[128] = 0b11100100                  # k=0: 0, k=1: 1, k=2: 2, k=3: 3
    got = oracle.dequant(Q6_K, blk, 1, 256)[0]
    assert [got[0], got[32], got[64], got[96]] == [-32.0, -16.0, 0.0, 16.0]
    assert got[1] == -32.0 and got[128] == -32.0


def test_q6_k_ragged_tail(oracle):
    rng = np.random.default_rng(23)
    rows, cols = 3, 640                    # 3 super-blocks, first half of last
    assert oracle.row_bytes(Q6_K, cols) == 3 * 210
    W = rng.integers(0, 256, rows * 3 * 210, dtype=np.uint8).reshape(rows, 3, 210)
    W[:, :, 209] = 0x20
    ref = oracle.dequant(Q6_K, W.reshape(-1), rows, cols)
    W2 = W.copy()
    last = W2[:, 2]
    # fields of weights 128..255 of the last super-block: ql[64:128],
    # qh[32:64], scales 8..15
    last[:, 64:128] = rng.integers(0, 256, (rows, 64), dtype=np.uint8)
    last[:, 160:192] = rng.integers(0, 256, (rows, 32), dtype=np.uint8)
    last[:, 200:208] = rng.integers(0, 256, (rows, 8), dtype=np.uint8)
    got = oracle.dequant(Q6_K, W2.reshape(-1), rows, cols)
    assert np.array_equal(bits(ref), bits(got))


@pytest.mark.parametrize("fmt,qk,nbytes", [(Q5_0, 32, 22), (Q5_K, 256, 176), (Q6_K, 256, 210)])
def test_row_bytes(oracle, fmt, qk, nbytes):
    for cols in (1, qk - 1, qk, qk + 1, 896, 4096, 14336):
        assert oracle.row_bytes(fmt, cols) == -(-cols // qk) * nbytes
