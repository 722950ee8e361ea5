"""The block sizes reproduce the figures the pages print (tests/golden)."""
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")


def _figures():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("="))
                out[k] = float(v)
    return out


def test_q4_k_bits_per_weight(oracle):
    f = _figures()
    assert oracle.row_bytes(12, 256) * 8 / 256 == f["q4_k_bits_per_weight"]


def test_q4_decode_arithmetic_intensity(oracle):
    f = _figures()
    ai = 2.0 / (oracle.row_bytes(12, 4096) / 4096)   # 2 flop per weight
    assert abs(ai - f["q4_decode_ai_flop_per_byte"]) < 0.01


def test_lm_head_macs(oracle):
    f = _figures()
    macs = f["lm_head_hidden"] * f["lm_head_vocab"]
    assert round(macs / 1e6) == f["lm_head_macs_millions"]
    # the Q8_0 lm_head stream: 34 B per 32 values, about 1 byte per value
    b = oracle.row_bytes(8, 896) * 151936
    assert b == 144_643_072
    assert round(b / macs) == f["q8_0_bytes_per_value_approx"]
