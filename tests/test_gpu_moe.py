"""MoE bucketing, gather and scatter on the GPU against the oracle, bit for
bit (index work and copies exactly; the scatter in the same fp32 order), and
the whole prefill chain -- bucket, gather, grouped product, scatter --
against the f64 expert matvecs within the stated bound."""
import numpy as np
import pytest

import synth
from helpers import oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu


def _ids(rng, n, n_expert, invalid=0.0):
    """Expert ids skewed towards the low experts (as a router's picks are),
    with a share of ids outside [0, n_expert)."""
    p = 1.0 / np.arange(1, n_expert + 1)
    ids = rng.choice(n_expert, size=n, p=p / p.sum()).astype(np.int32)
    bad = rng.random(n) < invalid
    ids[bad] = rng.choice(np.array([-1, -7, n_expert, n_expert + 5, 2 ** 31 - 1], np.int64),
                          size=int(bad.sum())).astype(np.int32)
    return ids


@pytest.mark.parametrize("n,n_expert,invalid", [
    (1, 1, 0.0), (8, 4, 0.0), (1000, 8, 0.05), (1024, 8, 0.0), (1025, 8, 0.0),
    (32768, 128, 0.01), (5000, 1024, 0.02), (3000, 3, 0.5), (64, 16, 1.0),
    (1 << 20, 64, 0.01),   # 1024 tiles of the one-workgroup walk
])
def test_bucket_matches_oracle(gq, oracle, n, n_expert, invalid):
    import torch
    rng = synth.rng_for(910, n * 7 + n_expert)
    ids = _ids(rng, n, n_expert, invalid)
    if (n, n_expert) == (8, 4):
        ids = np.array([2, 0, 2, 1, 0, 0, 3, 2], np.int32)
    print(f"[moe] bucket n={n} n_expert={n_expert} invalid={invalid}", flush=True)
    order = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    counts, order, pos = gq.gq_moe_bucket(to_dev(ids), n_expert, order=order)
    c, o, p = to_host(counts), to_host(order), to_host(pos)
    wc, wo, wp = oracle.moe_bucket(ids, n_expert)
    assert np.array_equal(c, wc)
    assert np.array_equal(p, wp)
    placed = int(wc.sum())
    assert np.array_equal(o[:placed], wo[:placed])
    assert (o[placed:] == -7).all()       # the unused tail is left alone
    # the same placement again
    counts2, order2, pos2 = gq.gq_moe_bucket(to_dev(ids), n_expert)
    assert np.array_equal(to_host(pos2), p) and np.array_equal(to_host(counts2), c)


def test_bucket_no_assignments_writes_zero_counts(gq):
    import torch
    counts = torch.full((5,), 99, dtype=torch.int64, device="cuda")
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    gq.gq_moe_bucket(empty, 5, counts=counts)
    assert to_host(counts).tolist() == [0] * 5


@pytest.mark.parametrize("n_tok,k,cols,n_expert", [
    (300, 2, 4096, 8),    # 16-byte copies
    (77, 8, 33, 16),      # 4-byte copies, ragged row
    (1, 1, 1, 1),
])
def test_gather_matches_oracle(gq, oracle, n_tok, k, cols, n_expert):
    import torch
    rng = synth.rng_for(911, n_tok * k + cols)
    ids = _ids(rng, n_tok * k, n_expert, 0.05 if n_tok > 1 else 0.0)
    X = synth.activations((n_tok, cols), rng)
    _, _, pos = gq.gq_moe_bucket(to_dev(ids), n_expert)
    Xb = torch.full((n_tok * k, cols), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[moe] gather n_tok={n_tok} k={k} cols={cols}", flush=True)
    gq.gq_moe_gather(to_dev(X), k, pos, Xb=Xb)
    want = oracle.moe_gather(X, k, to_host(pos), cols)
    got = to_host(Xb)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(want)].view(np.uint32), want[~np.isnan(want)].view(np.uint32))


@pytest.mark.parametrize("n_tok,k,rows,n_expert", [
    (300, 2, 4096, 8), (77, 8, 33, 16), (1000, 1, 5, 3), (5, 4, 1, 2),
])
def test_scatter_matches_oracle(gq, oracle, n_tok, k, rows, n_expert):
    rng = synth.rng_for(912, n_tok * k + rows)
    ids = _ids(rng, n_tok * k, n_expert, 0.05)
    _, _, pos = gq.gq_moe_bucket(to_dev(ids), n_expert)
    Yb = synth.activations((n_tok * k, rows), rng)
    w = rng.random(n_tok * k).astype(np.float32)
    out0 = synth.activations((n_tok, rows), rng)
    out = to_dev(out0.copy())
    print(f"[moe] scatter n_tok={n_tok} k={k} rows={rows}", flush=True)
    gq.gq_moe_scatter(to_dev(Yb), pos, to_dev(w), k, out)
    want = oracle.moe_scatter(out0, Yb, to_host(pos), w, k)
    assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt", [12, 8])
def test_prefill_chain_against_expert_matvecs(gq, oracle, fmt):
    """Bucket -> gather -> gq_matmul_experts (counts copied to the host) ->
    scatter, against out0 + sum_j w * (W_e x_t) from the oracle's f64 expert
    matvecs: each expert row within 2e-4 * S of exact, and the fp32 combine
    (k products, k + 1 sums) within 2k + 2 roundings of its terms' size."""
    import torch
    n_tok, k, n_expert, rows, cols = 96, 2, 8, 320, 512
    rng = synth.rng_for(913, fmt)
    W = np.concatenate([synth.weights(fmt, rows, cols, rng) for _ in range(n_expert)])
    X = synth.activations((n_tok, cols), rng)
    ids = _ids(rng, n_tok * k, n_expert)
    w = rng.random(n_tok * k).astype(np.float32)
    out0 = synth.activations((n_tok, rows), rng)
    print(f"[moe] prefill chain fmt={fmt}", flush=True)
    Wd = to_dev(W)
    counts, order, pos = gq.gq_moe_bucket(to_dev(ids), n_expert)
    Xb = gq.gq_moe_gather(to_dev(X), k, pos)
    m = to_host(counts).tolist()
    Yb = gq.gq_matmul_experts(fmt, Wd, n_expert, rows, cols, Xb, m)
    out = to_dev(out0.copy())
    gq.gq_moe_scatter(Yb, pos, to_dev(w), k, out)
    torch.cuda.synchronize()
    got = to_host(out).astype(np.float64)
    Ye, Se = oracle.experts_matvec(fmt, W, n_expert, rows, cols, X, k, ids, nthreads=oracle_threads())
    ref = out0.astype(np.float64).copy()
    bound = np.zeros_like(ref)
    mag = np.abs(out0).astype(np.float64)
    for a in range(n_tok * k):
        ref[a // k] += float(w[a]) * Ye[a]
        bound[a // k] += float(w[a]) * 2e-4 * Se[a]
        mag[a // k] += float(w[a]) * np.abs(Ye[a])
    bound += (2 * k + 2) * 2.0 ** -24 * mag
    assert (np.abs(got - ref) <= bound).all()
