"""Pins for the split per-row Q8_0 layout (the q8_0 repack of "nurllama
0.18.1 API", kernels.nu section; the layout is the reading taken: per row the
nb fp16 scales, zero padding to a multiple of 16 bytes, then the nb * 32
codes in block order)."""
import numpy as np
import pytest

import synth

SPLIT = 1008


def test_repack_layout_by_hand(oracle):
    # 2 rows x 3 blocks; block (r, b) has d bits 0x3C00 + 16 r + b and codes
    # q_i = 10 b + i - 50 (so every byte differs between blocks)
    rows, nb = 2, 3
    cols = 32 * nb
    W = []
    for r in range(rows):
        for b in range(nb):
            blk = np.zeros(34, np.uint8)
            d16 = 0x3C00 + 16 * r + b
            blk[0], blk[1] = d16 & 0xFF, d16 >> 8
            blk[2:] = (np.arange(32) + 10 * b - 50).astype(np.int8).view(np.uint8)
            W.append(blk)
    W = np.concatenate(W)
    got = oracle.q8_0_split_repack(W, rows, cols).reshape(rows, -1)
    assert got.shape[1] == 16 + 96 == oracle.row_bytes(SPLIT, cols)
    for r in range(rows):
        want = np.zeros(112, np.uint8)
        for b in range(nb):
            d16 = 0x3C00 + 16 * r + b
            want[2 * b], want[2 * b + 1] = d16 & 0xFF, d16 >> 8
            want[16 + 32 * b:16 + 32 * b + 32] = (np.arange(32) + 10 * b - 50).astype(np.int8).view(np.uint8)
        assert np.array_equal(got[r], want), r


@pytest.mark.parametrize("rows,cols", [(5, 576), (3, 896), (4, 33), (7, 4096), (2, 32 * 8), (2, 32 * 9)])
def test_split_decodes_to_the_same_weights(oracle, rows, cols):
    rng = synth.rng_for(50, cols)
    W = synth.weights(8, rows, cols, rng)
    S = oracle.q8_0_split_repack(W, rows, cols)
    nb = -(-cols // 32)
    assert oracle.row_bytes(SPLIT, cols) == -(-2 * nb // 16) * 16 + 32 * nb
    a = oracle.dequant(8, W, rows, cols)
    b = oracle.dequant(SPLIT, S, rows, cols)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    x = synth.activations(cols, rng)
    y1, s1 = oracle.matvec(8, W, rows, cols, x)
    y2, s2 = oracle.matvec(SPLIT, S, rows, cols, x)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    # the padding is zero
    pad = S.reshape(rows, -1)[:, 2 * nb:-(-2 * nb // 16) * 16]
    assert (pad == 0).all()
