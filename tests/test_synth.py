"""The seeded generators: deterministic, right sizes, fields in range."""
import numpy as np

import synth


def test_sizes_and_determinism():
    for fmt, rows, cols in [(8, 5, 576), (12, 3, 896), (12, 2, 4864)]:
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


def test_prefill_weights_are_decode_layer0():
    W, X, rows, cols = synth.prefill_inputs("down", 16)
    Wd, _ = synth.llama3_8b_weight_and_x(0, 6)
    assert (rows, cols) == (4096, 14336) and X.shape == (16, 14336)
    assert np.array_equal(W, Wd)
