"""The seeded generators: deterministic, right sizes, fields in range."""
import numpy as np

import synth


def test_sizes_and_determinism():
    for fmt, rows, cols in [(8, 5, 576), (12, 3, 896), (12, 2, 4864), (6, 4, 896),
                            (13, 3, 896), (14, 3, 4096)]:
        a = synth.weights(fmt, rows, cols, synth.rng_for(0, 1))
        b = synth.weights(fmt, rows, cols, synth.rng_for(0, 1))
        c = synth.weights(fmt, rows, cols, synth.rng_for(0, 2))
        assert a.dtype == np.uint8 and a.size == rows * synth.packed_row_bytes(fmt, cols)
        assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_q8_0_fields():
    W = synth.weights(8, 64, 576, synth.rng_for(0, 0)).reshape(-1, 34)
    d = W[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    q = W[:, 2:].view(np.int8)
    assert q.min() >= -127 and q.max() <= 127
    # max|N(0, 0.02)| over 32 draws / 127 lies around 0.02 * 2.4 / 127
    assert np.all(d > 0) and 2e-4 < np.median(d) < 6e-4


def test_q4_k_fields():
    W = synth.weights(12, 256, 512, synth.rng_for(1, 0)).reshape(-1, 144)
    d = W[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = W[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.5 * 1.2e-4 * 0.999 and d.max() <= 1.5 * 1.2e-4 * 1.001
    assert dmin.min() >= 0.5 * 9.2e-4 * 0.999 and dmin.max() <= 1.5 * 9.2e-4 * 1.001
    # the 140 code bytes are uniform
    assert abs(W[:, 4:].mean() - 127.5) < 1.0


def test_q5_0_fields():
    W = synth.weights(6, 64, 896, synth.rng_for(0, 0)).reshape(-1, 22)
    d = W[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    assert np.all(d > 0) and 2e-3 < np.median(d) < 5e-3   # ~0.02 * 2.4 / 16
    assert abs(W[:, 2:].mean() - 127.5) < 1.5


def test_q5_k_fields():
    W = synth.weights(13, 256, 512, synth.rng_for(1, 0)).reshape(-1, 176)
    d = W[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = W[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.5 * 5.9e-5 * 0.999 and d.max() <= 1.5 * 5.9e-5 * 1.001
    assert dmin.min() >= 0.5 * 9.2e-4 * 0.999 and dmin.max() <= 1.5 * 9.2e-4 * 1.001
    assert abs(W[:, 4:].mean() - 127.5) < 1.0


def test_q6_k_fields():
    W = synth.weights(14, 256, 512, synth.rng_for(1, 0)).reshape(-1, 210)
    d = W[:, 208:210].copy().view(np.float16).astype(np.float64).ravel()
    # d lies in fp16's subnormal range (spacing 2^-24), as real Q6_K scales do
    ulp = 2.0 ** -24
    assert d.min() >= 0.5 * 1.4e-5 - ulp and d.max() <= 1.5 * 1.4e-5 + ulp
    assert np.all(d < 2.0 ** -14)
    sc = W[:, 192:208].view(np.int8)
    assert sc.min() == -128 and sc.max() == 127
    assert abs(W[:, :208].mean() - 127.5) < 1.0


def test_prefill_weights_are_decode_layer0():
    W, X, rows, cols = synth.prefill_inputs("down", 16)
    Wd, _ = synth.llama3_8b_weight_and_x(0, 6)
    assert (rows, cols) == (4096, 14336) and X.shape == (16, 14336)
    assert np.array_equal(W, Wd)
