"""gq_dequant on the GPU is bit-identical to the oracle's fp32 dequant
(memcmp, including the sign of zero), on every workload matrix and on edge
shapes. Called through the C ABI via the Python binding."""
import numpy as np
import pytest

import synth
from helpers import assert_pad_untouched, sentinel_buffer, to_dev, to_host

pytestmark = pytest.mark.gpu


def _check(gq, oracle, fmt, W, rows, cols, what):
    print(f"[dequant] {what} fmt={fmt} rows={rows} cols={cols}", flush=True)
    ref = oracle.dequant(fmt, W, rows, cols)
    out = sentinel_buffer(rows * cols)
    gq.gq_dequant(fmt, to_dev(W), rows, cols, out=out)
    got = to_host(out)[: rows * cols].reshape(rows, cols)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), what
    assert_pad_untouched(out, rows * cols)


def test_smollm_ffn_up_q8_0(gq, oracle):
    fmt, rows, cols = synth.SMOLLM_FFN_UP
    W, _ = synth.matrix_and_x(fmt, rows, cols, 0, 0)
    _check(gq, oracle, fmt, W, rows, cols, "smollm-135m ffn_up")


@pytest.mark.parametrize("i", range(4))
def test_qwen05b_decode_q4_k(gq, oracle, i):
    fmt, rows, cols = synth.QWEN05_DECODE[i]
    W, _ = synth.matrix_and_x(fmt, rows, cols, 1, i)
    _check(gq, oracle, fmt, W, rows, cols, f"qwen2.5-0.5b {rows}x{cols}")


def test_qwen05b_lm_head_q8_0(gq, oracle):
    fmt, rows, cols = synth.QWEN05_LM_HEAD
    W, _ = synth.matrix_and_x(fmt, rows, cols, 2, 0)
    _check(gq, oracle, fmt, W, rows, cols, "qwen2.5-0.5b lm_head")


@pytest.mark.parametrize("proj", range(7))
def test_llama3_8b_layer0_q4_k(gq, oracle, proj):
    name, rows, cols, seed, mid = synth.llama3_8b_matrix(0, proj)
    W, _ = synth.llama3_8b_weight_and_x(0, proj)
    _check(gq, oracle, 12, W, rows, cols, f"llama3-8b layer0 {name}")


@pytest.mark.parametrize("fmt,rows,cols", [
    (8, 1, 32), (8, 63, 64), (8, 65, 96), (8, 64, 1024), (8, 3, 70), (8, 5, 33),
    (8, 7, 1053), (12, 1, 256), (12, 64, 1024), (12, 65, 896), (12, 63, 300),
    (12, 2, 14336), (12, 3, 4864), (12, 9, 250), (12, 4, 1),
])
def test_edge_shapes(gq, oracle, fmt, rows, cols):
    rng = synth.rng_for(100, rows * 100000 + cols)
    W = synth.weights(fmt, rows, cols, rng)
    _check(gq, oracle, fmt, W, rows, cols, "edge")


def test_q8_0_row_range_at_two_byte_offset(gq, oracle):
    # a row range of a Q8_0 tensor that starts one block in: 2-byte aligned
    rows, cols = 40, 96
    W = synth.weights(8, rows + 1, cols, synth.rng_for(7, 7))
    rb = oracle.row_bytes(8, cols)
    import torch
    Wd = to_dev(W)
    for off in (34, rb):      # one block in (2 mod 4), one row in
        sub = Wd[off:]
        n = (W.size - off) // rb
        ref = oracle.dequant(8, W[off:off + n * rb], n, cols)
        out = torch.empty((n, cols), dtype=torch.float32, device="cuda")
        gq.gq_dequant(8, sub, n, cols, out=out)
        assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32))


def test_special_scales(gq, oracle):
    """Subnormal, negative and zero fp16 scales; q = -128; code extremes."""
    blocks = []
    for d16 in (0x0001, 0x03FF, 0x8001, 0x0400, 0x7BFF, 0xFBFF, 0x0000, 0x8000, 0x3C00):
        q = np.arange(-128, 128, dtype=np.int16).reshape(8, 32)
        for k in range(8):
            b = np.zeros(34, np.uint8)
            b[0], b[1] = d16 & 0xFF, d16 >> 8
            b[2:] = q[k].astype(np.int8).view(np.uint8)
            blocks.append(b)
    W8 = np.concatenate(blocks)
    _check(gq, oracle, 8, W8, len(blocks) // 8, 256, "q8_0 special scales")
    rng = np.random.default_rng(3)
    sb = []
    for d16, dm16 in [(0x0001, 0x0001), (0x8001, 0x03FF), (0x7BFF, 0x0001), (0x0001, 0x7BFF),
                      (0x0000, 0x0000), (0x8000, 0x8000), (0xBC00, 0xC000)]:
        b = rng.integers(0, 256, 144, dtype=np.uint8)
        b[0], b[1], b[2], b[3] = d16 & 0xFF, d16 >> 8, dm16 & 0xFF, dm16 >> 8
        sb.append(b)
    W4 = np.concatenate(sb)
    _check(gq, oracle, 12, W4, len(sb), 256, "q4_k special scales")
