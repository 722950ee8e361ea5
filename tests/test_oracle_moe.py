"""Pins for the oracle's MoE bucketing, gather and scatter: a hand-worked
bucketing, agreement with a stable sort by expert id (another algorithm),
invalid ids, the gather read back through the order rather than the
positions, and scatters whose products and sums are exact integers."""
import numpy as np

import synth


def test_hand_worked_bucketing(oracle):
    # 4 positions x 2 slots, 4 experts. Ids per assignment a = 0..7:
    #   2 0 | 2 1 | 0 0 | 3 2
    # counts: e0 = {1, 4, 5}, e1 = {3}, e2 = {0, 2, 7}, e3 = {6} -> 3 1 3 1;
    # buckets start at 0, 3, 4, 7; inside a bucket the assignments keep
    # their order: bucket 0 = 1 4 5, bucket 1 = 3, bucket 2 = 0 2 7, bucket 3 = 6
    counts, order, pos = oracle.moe_bucket([2, 0, 2, 1, 0, 0, 3, 2], 4)
    assert counts.tolist() == [3, 1, 3, 1]
    assert order.tolist() == [1, 4, 5, 3, 0, 2, 7, 6]
    assert pos.tolist() == [4, 0, 5, 3, 1, 2, 7, 6]


def test_invalid_ids_are_dropped(oracle):
    counts, order, pos = oracle.moe_bucket([1, -1, 0, 5, 1, 2], 3)
    assert counts.tolist() == [1, 2, 1]
    assert pos.tolist() == [1, -1, 0, -1, 2, 3]
    assert order.tolist() == [2, 0, 4, 5, -1, -1]


def test_agrees_with_a_stable_sort(oracle):
    for seed, (n, n_expert) in enumerate([(1, 1), (37, 3), (1000, 8), (4096, 128), (777, 1024)]):
        rng = synth.rng_for(900, seed)
        ids = rng.integers(-2, n_expert + 2, size=n).astype(np.int32)
        counts, order, pos = oracle.moe_bucket(ids, n_expert)
        valid = (ids >= 0) & (ids < n_expert)
        assert counts.tolist() == np.bincount(ids[valid], minlength=n_expert).tolist()
        # the placed assignments, ordered by id with ties in index order
        idx = np.flatnonzero(valid)
        want = idx[np.argsort(ids[valid], kind="stable")]
        placed = int(valid.sum())
        assert np.array_equal(order[:placed], want)
        assert (order[placed:] == -1).all()
        assert np.array_equal(pos[want], np.arange(placed))
        assert (pos[~valid] == -1).all()


def test_gather_through_the_order(oracle):
    rng = synth.rng_for(901, 0)
    n_tok, k, n_expert, cols = 50, 3, 7, 12
    ids = rng.integers(0, n_expert, size=n_tok * k).astype(np.int32)
    ids[5] = -1
    X = (np.arange(n_tok * cols, dtype=np.float32).reshape(n_tok, cols) + 0.5)
    counts, order, pos = oracle.moe_bucket(ids, n_expert)
    Xb = oracle.moe_gather(X, k, pos, cols)
    placed = int(counts.sum())
    for p in range(placed):
        assert np.array_equal(Xb[p], X[order[p] // k])
    assert np.isnan(Xb[placed:]).all()


def test_scatter_exact_integers(oracle):
    # integer weights and rows: every product and partial sum is an exact
    # integer in fp32, so the result is the exact sum
    rng = synth.rng_for(902, 0)
    n_tok, k, rows, n_expert = 20, 4, 9, 5
    ids = rng.integers(0, n_expert, size=n_tok * k).astype(np.int32)
    ids[[3, 17]] = 99  # dropped slots add nothing
    counts, order, pos = oracle.moe_bucket(ids, n_expert)
    n = n_tok * k
    Yb = rng.integers(-50, 51, size=(n, rows)).astype(np.float32)
    w = rng.integers(-3, 4, size=n).astype(np.float32)
    out0 = rng.integers(-1000, 1001, size=(n_tok, rows)).astype(np.float32)
    got = oracle.moe_scatter(out0, Yb, pos, w, k)
    want = out0.astype(np.float64).copy()
    for a in range(n):
        if pos[a] >= 0:
            want[a // k] += float(w[a]) * Yb[pos[a]].astype(np.float64)
    assert np.array_equal(got.astype(np.float64), want)


def test_scatter_one_slot_is_one_rounding(oracle):
    # k = 1, w = 1: out + Yb[pos] with a single fp32 rounding
    rng = synth.rng_for(903, 0)
    n, rows = 16, 33
    pos = rng.permutation(n).astype(np.int32)
    Yb = rng.standard_normal((n, rows)).astype(np.float32)
    out0 = rng.standard_normal((n, rows)).astype(np.float32)
    got = oracle.moe_scatter(out0, Yb, pos, np.ones(n, np.float32), 1)
    want = (out0.astype(np.float64) + Yb[pos].astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, want)
