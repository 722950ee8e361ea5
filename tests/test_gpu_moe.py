"""MoE bucketing, gather and scatter on the GPU against the oracle, bit for
bit (index work and copies exactly; the scatter in the same fp32 order), and
the whole prefill chain -- bucket, gather, grouped product, scatter --
against the f64 expert matvecs within the stated bound."""
import numpy as np
import pytest

import synth
from helpers import assert_within_tolerance, oracle_threads, to_dev, to_host

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


@pytest.mark.parametrize("fmt", [12, 13, 8, 1008, 14, 6])
def test_grouped_product_with_device_counts(gq, oracle, fmt):
    """gq_matmul_experts_dev against the oracle per expert (counts skewed,
    one expert empty), Y rows past the counts left alone, and the same bits
    on a second call."""
    import torch
    n_expert, rows, cols = 6, 320, 512
    counts = [150, 0, 70, 33, 1, 90]
    total = sum(counts) + 17   # rows past the counts stay untouched
    rng = synth.rng_for(914, fmt)
    base = 8 if fmt == 1008 else fmt
    W = np.concatenate([synth.weights(base, rows, cols, rng) for _ in range(n_expert)])
    X = synth.activations((total, cols), rng)
    Wd = to_dev(W)
    if fmt == 1008:
        Wd = gq.gq_q8_0_split_repack(Wd, n_expert * rows, cols)
    cd = to_dev(np.array(counts, np.int64))
    Y = torch.full((total, rows), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[moe] grouped product, device counts fmt={fmt}", flush=True)
    gq.gq_matmul_experts_dev(fmt, Wd, n_expert, rows, cols, to_dev(X), cd, Y=Y)
    got = to_host(Y).copy()
    eb = rows * gq.gq_row_bytes(base, cols)
    m0 = 0
    for e, m in enumerate(counts):
        if m:
            ref, S = oracle.matmul(base, W[e * eb:(e + 1) * eb], rows, cols, X[m0:m0 + m],
                                   nthreads=oracle_threads())
            assert_within_tolerance(got[m0:m0 + m], ref, S, f"expert {e} fmt={fmt}")
        m0 += m
    assert np.isnan(got[m0:]).all()
    gq.gq_matmul_experts_dev(fmt, Wd, n_expert, rows, cols, to_dev(X), cd, Y=Y)
    assert np.array_equal(to_host(Y).view(np.uint32), got.view(np.uint32))


def test_grouped_product_device_counts_clamped(gq, oracle):
    """Counts that add up past the rows given (and a negative one): the
    groups are cut at the total, every row computed is its expert's product."""
    import torch
    n_expert, rows, cols, total = 4, 64, 256, 100
    counts = [60, -5, 70, 40]        # 60 rows, none, the last 40 rows, nothing left
    rng = synth.rng_for(915, 0)
    W = np.concatenate([synth.weights(12, rows, cols, rng) for _ in range(n_expert)])
    X = synth.activations((total, cols), rng)
    Y = torch.full((total, rows), float("nan"), dtype=torch.float32, device="cuda")
    print("[moe] grouped product, clamped device counts", flush=True)
    gq.gq_matmul_experts_dev(12, to_dev(W), n_expert, rows, cols, to_dev(X),
                             to_dev(np.array(counts, np.int64)), Y=Y)
    got = to_host(Y)
    eb = rows * gq.gq_row_bytes(12, cols)
    for e, lo, hi in ((0, 0, 60), (2, 60, 100)):
        ref, S = oracle.matmul(12, W[e * eb:(e + 1) * eb], rows, cols, X[lo:hi])
        assert_within_tolerance(got[lo:hi], ref, S, f"clamped expert {e}")


def test_moe_prefill_chain_in_one_graph(gq, oracle):
    """Bucket, gather, the grouped product with device counts and the
    scatter captured in one HIP graph and replayed with new ids and data:
    every replay within the chain's bound against the f64 expert matvecs."""
    import torch
    n_tok, k, n_expert, rows, cols = 64, 2, 8, 256, 512
    n = n_tok * k
    rng = synth.rng_for(916, 0)
    W = np.concatenate([synth.weights(12, rows, cols, rng) for _ in range(n_expert)])
    Wd = to_dev(W)
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    X = torch.zeros((n_tok, cols), dtype=torch.float32, device="cuda")
    w = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.zeros((n_tok, rows), dtype=torch.float32, device="cuda")
    counts = torch.empty(n_expert, dtype=torch.int64, device="cuda")
    order = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int32, device="cuda")
    Xb = torch.empty((n, cols), dtype=torch.float32, device="cuda")
    Yb = torch.empty((n, rows), dtype=torch.float32, device="cuda")

    def step():
        gq.gq_moe_bucket(ids, n_expert, counts, order, pos)
        gq.gq_moe_gather(X, k, pos, Xb)
        gq.gq_matmul_experts_dev(12, Wd, n_expert, rows, cols, Xb, counts, Y=Yb)
        gq.gq_moe_scatter(Yb, pos, w, k, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        r2 = synth.rng_for(917, rep)
        hid = _ids(r2, n, n_expert)
        hX = synth.activations((n_tok, cols), r2)
        hw = r2.random(n).astype(np.float32)
        ho = synth.activations((n_tok, rows), r2)
        for t, h in ((ids, hid), (X, hX), (w, hw), (out, ho)):
            t.copy_(torch.from_numpy(h))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[moe] graph replay {rep}", flush=True)
        got = to_host(out).astype(np.float64)
        Ye, Se = oracle.experts_matvec(12, W, n_expert, rows, cols, hX, k, hid, nthreads=oracle_threads())
        ref = ho.astype(np.float64).copy()
        bound = np.zeros_like(ref)
        mag = np.abs(ho).astype(np.float64)
        for a in range(n):
            ref[a // k] += float(hw[a]) * Ye[a]
            bound[a // k] += float(hw[a]) * 2e-4 * Se[a]
            mag[a // k] += float(hw[a]) * np.abs(Ye[a])
        bound += (2 * k + 2) * 2.0 ** -24 * mag
        assert (np.abs(got - ref) <= bound).all()
