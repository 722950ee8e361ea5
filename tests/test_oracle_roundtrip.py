"""Round trip: test-only quantiser -> oracle dequant stays within the error
bound the quantiser guarantees (Q8_0 as in the converter of "nurllama 0.18.1
API", convert.nu section, which encodes Q8_0; Q4_K with a plain covering
quantiser of our own, since the pages print none)."""
import numpy as np
import pytest


def _inputs(kind, shape, rng):
    if kind == "normal":
        return (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(-1.0, 3.0, shape).astype(np.float32)
    if kind == "positive":
        return rng.uniform(0.1, 0.2, shape).astype(np.float32)
    return np.zeros(shape, np.float32)


@pytest.mark.parametrize("kind", ["normal", "uniform", "positive", "zero"])
@pytest.mark.parametrize("cols", [32 * 9, 70])
def test_q8_0_roundtrip(oracle, kind, cols):
    rng = np.random.default_rng(1)
    w = _inputs(kind, (5, cols), rng)
    W = oracle.quantize(8, w)
    back = oracle.dequant(8, W, 5, cols)
    nb = -(-cols // 32)
    d = oracle.f16_to_f32(W.reshape(5, nb, 34)[:, :, :2].copy().view(np.uint16)).reshape(5, nb)
    for b in range(nb):
        blk = slice(32 * b, min(cols, 32 * b + 32))
        a = np.abs(w[:, blk]).max(axis=1).astype(np.float64)
        db = d[:, b].astype(np.float64)
        bound = 0.5 * db + 127 * np.abs(a / 127 - db)
        err = np.abs(back[:, blk].astype(np.float64) - w[:, blk]).max(axis=1)
        assert np.all(err <= bound * (1 + 1e-12) + 1e-30)
    if kind == "zero":
        assert np.all(back == 0)


@pytest.mark.parametrize("kind", ["normal", "uniform", "positive", "zero"])
@pytest.mark.parametrize("cols", [256 * 2, 300])
def test_q4_k_roundtrip(oracle, kind, cols):
    rng = np.random.default_rng(2)
    w = _inputs(kind, (4, cols), rng)
    W = oracle.quantize(12, w)
    back = oracle.dequant(12, W, 4, cols)
    nb = -(-cols // 256)
    blk = W.reshape(4, nb, 144)
    d = oracle.f16_to_f32(blk[:, :, 0:2].copy().view(np.uint16)).reshape(4, nb)
    for r in range(4):
        for b in range(nb):
            sc, _ = oracle.q4_k_unpack_scales(blk[r, b, 4:16])
            for j in range(8):
                c0, c1 = 256 * b + 32 * j, min(cols, 256 * b + 32 * j + 32)
                if c0 >= cols:
                    continue
                step = float(d[r, b]) * float(sc[j])
                ww = w[r, c0:c1].astype(np.float64)
                err = np.abs(back[r, c0:c1].astype(np.float64) - ww)
                bound = 0.5 * step + 2.0 ** -23 * (np.abs(ww) + 15 * step)
                assert np.all(err <= bound), (kind, r, b, j)
    if kind == "zero":
        assert np.all(back == 0)
