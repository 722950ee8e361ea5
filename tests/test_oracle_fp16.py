"""Pins for the oracle's hand-written binary16 decode and encode.

The decode is compared against numpy's float16 -> float32 conversion over
all 65,536 bit patterns (an exhaustive library compare); the encoder against
numpy's float -> float16 rounding (round to nearest, ties to even).
"""
import numpy as np


def test_f16_decode_all_patterns(oracle):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    # non-NaN: identical bits, including the sign of zero and subnormals
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # NaN keeps its sign (payload is left unspecified)
    assert np.array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))


def test_f16_decode_special_values(oracle):
    cases = {
        0x0000: 0.0, 0x8000: -0.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
        0x0400: 2.0 ** -14, 0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0,
        0x3555: 0.333251953125, 0x7C00: np.inf, 0xFC00: -np.inf,
    }
    got = oracle.f16_to_f32(np.array(list(cases), np.uint16))
    for g, (h, v) in zip(got, cases.items()):
        assert g == v and np.signbit(g) == np.signbit(v), hex(h)


def test_f16_encode_matches_numpy(oracle):
    rng = np.random.default_rng(123)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),   # subnormal range
        (rng.standard_normal(5000) * 3e4).astype(np.float32),     # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e9, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5], np.float32),
    ])
    # the exact midpoints between neighbouring fp16 values test ties-to-even
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((allf[:-1] + allf[1:]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids[::7], -mids[::11]])
    with np.errstate(over="ignore"):   # values past 65520 round to inf on purpose
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_rne(v) for v in vals], np.uint16)
    assert np.array_equal(got, ref)
