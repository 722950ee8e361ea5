"""gq_matvec_experts on the GPU: every assignment equals the plain gq_matvec
of its expert and activation row bit for bit, the outputs are within the
product tolerance of the f64 oracle, invalid expert ids give NaN rows
without disturbing the others, and shapes cover mixture-of-experts decode
(top-k of many small experts) and prefill-sized assignment batches."""
import numpy as np
import pytest

import synth
from helpers import (assert_pad_untouched, assert_within_tolerance, oracle_threads,
                     sentinel_buffer, to_dev, to_host)

pytestmark = pytest.mark.gpu

# (fmt, n_expert, rows, cols, positions, xk)
CASES = [
    (12, 16, 768, 2048, 1, 8),     # 128-expert-style gate/up expert, top-8 decode
    (12, 16, 2048, 768, 1, 8),     # its down projection (three 256-column super-blocks)
    (8, 8, 768, 2048, 2, 4),       # Q8_0 experts (block pairs)
    (14, 8, 2048, 768, 1, 8),      # Q6_K down experts
    (13, 8, 768, 2048, 3, 2),      # Q5_K
    (6, 4, 300, 896, 2, 2),        # Q5_0, 896-wide
    (12, 8, 14336, 4096, 1, 2),    # Mixtral-style experts, top-2
    (12, 6, 64, 1024, 48, 8),      # a prefill batch: 384 assignments
    (12, 3, 5, 300, 5, 1),         # ragged rows, one expert per position
    (8, 5, 9, 40000, 1, 3),        # rows wider than 256 units: segmented kernel
]


@pytest.mark.parametrize("fmt,n_expert,rows,cols,positions,xk", CASES)
def test_experts(gq, oracle, fmt, n_expert, rows, cols, positions, xk):
    import torch
    rng = synth.rng_for(960, fmt * 10 ** 6 + n_expert * 1000 + rows)
    W = synth.weights(fmt, n_expert * rows, cols, rng)
    X = synth.activations((positions, cols), rng)
    n_assign = positions * xk
    expid = rng.integers(0, n_expert, n_assign).astype(np.int32)
    print(f"[experts] fmt={fmt} n_expert={n_expert} rows={rows} cols={cols} "
          f"n_assign={n_assign}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = torch.full((n_assign + 1, rows), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_matvec_experts(fmt, Wd, n_expert, rows, cols, Xd, xk, to_dev(expid), Y=Y)
    got = to_host(Y)
    assert np.isnan(got[n_assign]).all(), "wrote past the last assignment"
    got = got[:n_assign]
    ref, S = oracle.experts_matvec(fmt, W, n_expert, rows, cols, X, xk, expid,
                                   nthreads=oracle_threads())
    assert_within_tolerance(got, ref, S, "experts")
    # each assignment is the plain matvec of its expert, bit for bit
    rb = gq.gq_row_bytes(fmt, cols)
    for a in sorted(set([0, n_assign - 1] + list(range(0, n_assign, max(1, n_assign // 6))))):
        e = int(expid[a])
        y = gq.gq_matvec(fmt, Wd[e * rows * rb:(e + 1) * rows * rb], rows, cols, Xd[a // xk])
        assert np.array_equal(to_host(y).view(np.uint32), got[a].view(np.uint32)), a


def test_experts_past_65535_assignments(gq, oracle):
    """70000 assignments (35000 positions, top 2 of 4 experts): the
    assignments are the grid's second dimension, past 65535. Every output
    meets the oracle's bound and assignments on both sides of the boundary
    equal gq_matvec of their expert bit for bit."""
    import torch
    fmt, n_expert, rows, cols, xk, n_assign = 12, 4, 8, 256, 2, 70000
    rng = synth.rng_for(963, 0)
    W = synth.weights(fmt, n_expert * rows, cols, rng)
    X = synth.activations((n_assign // xk, cols), rng)
    expid = rng.integers(0, n_expert, n_assign).astype(np.int32)
    print(f"[experts] past 65535: n_assign={n_assign} rows={rows} cols={cols}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = torch.full((n_assign + 1, rows), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_matvec_experts(fmt, Wd, n_expert, rows, cols, Xd, xk, to_dev(expid), Y=Y)
    got = to_host(Y)
    assert np.isnan(got[n_assign]).all(), "wrote past the last assignment"
    got = got[:n_assign]
    ref, S = oracle.experts_matvec(fmt, W, n_expert, rows, cols, X, xk, expid,
                                   nthreads=oracle_threads())
    assert_within_tolerance(got, ref, S, "experts past 65535")
    rb = gq.gq_row_bytes(fmt, cols)
    for a in (0, 65534, 65535, 65536, n_assign - 1):
        e = int(expid[a])
        y = gq.gq_matvec(fmt, Wd[e * rows * rb:(e + 1) * rows * rb], rows, cols, Xd[a // xk])
        assert np.array_equal(to_host(y).view(np.uint32), got[a].view(np.uint32)), a


def test_invalid_ids_and_empty(gq, oracle):
    import torch
    fmt, n_expert, rows, cols = 12, 4, 300, 1024
    rng = synth.rng_for(961, 0)
    W = synth.weights(fmt, n_expert * rows, cols, rng)
    X = synth.activations((3, cols), rng)
    expid = np.array([3, -1, 0, 4, 2, 1 << 30], np.int32)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = gq.gq_matvec_experts(fmt, Wd, n_expert, rows, cols, Xd, 2, to_dev(expid))
    got = to_host(Y)
    for a in (1, 3, 5):
        assert np.isnan(got[a]).all(), a
    ref, S = oracle.experts_matvec(fmt, W, n_expert, rows, cols, X, 2, expid)
    for a in (0, 2, 4):
        assert_within_tolerance(got[a], ref[a], S[a], f"assignment {a}")
    # no assignments: nothing is launched or written
    Y0 = torch.full((1, rows), 7.0, device="cuda")
    gq.gq_matvec_experts(fmt, Wd, n_expert, rows, cols, Xd, 2,
                         torch.empty(0, dtype=torch.int32, device="cuda"), Y=Y0)
    assert (to_host(Y0) == 7.0).all()


# (fmt, rows, cols, rows per expert): groups that take the matvec (1), the
# batched matvec (3, 5), and the matrix cores (17 and up), with empty experts
GROUPED = [
    (12, 512, 2048, [0, 1, 3, 17, 40, 70, 5, 120]),
    (14, 256, 768, [33, 0, 2, 64]),          # Q6_K, 3 super-blocks a row: fp32 matrix cores
    (14, 256, 1024, [33, 0, 2, 64]),         # Q6_K, rows of 840 bytes: grouped on the fp16 ones
    (8, 300, 900, [9, 16, 0, 1]),            # Q8_0, rows of 29 blocks: few-row kernel / fp32 matrix cores
    (12, 64, 300, [0, 0, 7]),                # ragged rows, one expert with all the rows
    (13, 256, 1024, [20, 0, 2, 64]),         # Q5_K: grouped on the fp16 matrix cores
    (8, 256, 1024, [20, 0, 3, 64]),          # Q8_0 (rows of 1088 bytes): grouped as well
    (6, 256, 896, [20, 0, 3, 64]),           # Q5_0, 28 blocks a row: grouped as well
]


@pytest.mark.parametrize("fmt,rows,cols,counts", GROUPED)
def test_grouped_prefill(gq, oracle, fmt, rows, cols, counts):
    """Each expert's block of gq_matmul_experts is within tolerance of the
    oracle. Q4_K and Q5_K with cols % 4 == 0, and Q8_0, Q5_0 and Q6_K whose
    rows are also a whole number of dwords, run as one grouped launch: a second call gives
    the same bits. The others run gq_matmul per expert: each block equals
    gq_matmul of that expert's matrix and rows bit for bit."""
    n_expert, total = len(counts), sum(counts)
    rng = synth.rng_for(962, fmt * 1000 + rows)
    W = synth.weights(fmt, n_expert * rows, cols, rng)
    X = synth.activations((total, cols), rng)
    print(f"[grouped] fmt={fmt} rows={rows} cols={cols} counts={counts}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = sentinel_buffer(total * rows)
    gq.gq_matmul_experts(fmt, Wd, n_expert, rows, cols, Xd, counts, Y=Y[:total * rows])
    assert_pad_untouched(Y, total * rows)
    got = to_host(Y)[:total * rows].reshape(total, rows)
    rb = gq.gq_row_bytes(fmt, cols)
    grouped = cols % 4 == 0 and (fmt in (12, 13) or (fmt in (6, 8, 14) and rb % 4 == 0))
    o = 0
    for e, m in enumerate(counts):
        if m == 0:
            continue
        We = W[e * rows * rb:(e + 1) * rows * rb]
        ref, S = oracle.matmul(fmt, We, rows, cols, X[o:o + m], nthreads=oracle_threads())
        assert_within_tolerance(got[o:o + m], ref, S, f"expert {e}")
        if not grouped:
            one = to_host(gq.gq_matmul(fmt, Wd[e * rows * rb:(e + 1) * rows * rb], rows, cols, Xd[o:o + m]))
            assert np.array_equal(one.view(np.uint32), got[o:o + m].view(np.uint32)), e
        o += m
    if grouped:
        Y2 = sentinel_buffer(total * rows)
        gq.gq_matmul_experts(fmt, Wd, n_expert, rows, cols, Xd, counts, Y=Y2[:total * rows])
        again = to_host(Y2)[:total * rows].reshape(total, rows)
        assert np.array_equal(again.view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("fmt", [12, 8, 14])
def test_grouped_prefill_past_64_experts(gq, oracle, fmt):
    """130 experts (some with no rows): the grouped product runs as three
    launches of at most 64 experts; every expert's block is within tolerance
    of the oracle and a second call gives the same bits."""
    n_expert, rows, cols = 130, 48, 1024
    rng = synth.rng_for(964, fmt)
    counts = [int(c) for c in rng.integers(0, 6, n_expert)]
    counts[0], counts[63], counts[64], counts[129] = 0, 3, 5, 2
    total = sum(counts)
    W = synth.weights(fmt, n_expert * rows, cols, rng)
    X = synth.activations((total, cols), rng)
    print(f"[grouped] {n_expert} experts fmt={fmt} rows={rows} cols={cols} total={total}", flush=True)
    Wd, Xd = to_dev(W), to_dev(X)
    Y = sentinel_buffer(total * rows)
    gq.gq_matmul_experts(fmt, Wd, n_expert, rows, cols, Xd, counts, Y=Y[:total * rows])
    assert_pad_untouched(Y, total * rows)
    got = to_host(Y)[:total * rows].reshape(total, rows)
    rb = gq.gq_row_bytes(fmt, cols)
    o = 0
    for e, m in enumerate(counts):
        if m:
            ref, S = oracle.matmul(fmt, W[e * rows * rb:(e + 1) * rows * rb], rows, cols, X[o:o + m])
            assert_within_tolerance(got[o:o + m], ref, S, f"expert {e}")
        o += m
    Y2 = sentinel_buffer(total * rows)
    gq.gq_matmul_experts(fmt, Wd, n_expert, rows, cols, Xd, counts, Y=Y2[:total * rows])
    assert np.array_equal(to_host(Y2)[:total * rows].view(np.uint32), got.reshape(-1).view(np.uint32))
