"""gq_matvec inside a captured HIP graph (the form the decode-step
benchmark times): the graph is replayed several times with new activations
written eagerly between replays, and every replay must equal an eager call
on the same inputs bit for bit (and the f64 oracle within tolerance)."""
import numpy as np
import pytest

import synth
from helpers import assert_within_tolerance, oracle_threads, to_dev, to_host

pytestmark = pytest.mark.gpu

# (fmt, rows, cols): a Q4_K matrix with wide rows, a Q4_K one with short
# ragged rows, the Q8_0 block-pair path and the single-block Q8_0 path
SHAPES = [(12, 1024, 4096), (12, 300, 896), (8, 2000, 896), (8, 500, 96)]


def test_graph_replays_match_eager(gq, oracle):
    import torch

    mats, xs, ys = [], [], []
    for k, (fmt, rows, cols) in enumerate(SHAPES):
        rng = synth.rng_for(800, k)
        mats.append(to_dev(synth.weights(fmt, rows, cols, rng)))
        xs.append(torch.empty(cols, dtype=torch.float32, device="cuda"))
        ys.append(torch.empty(rows, dtype=torch.float32, device="cuda"))

    def step():
        for (fmt, rows, cols), W, x, y in zip(SHAPES, mats, xs, ys):
            gq.gq_matvec(fmt, W, rows, cols, x, y=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for x in xs:
            x.zero_()
        step()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for rep in range(3):
        host_x = [synth.activations(cols, synth.rng_for(801 + rep, k))
                  for k, (_, _, cols) in enumerate(SHAPES)]
        for x, hx in zip(xs, host_x):
            x.copy_(torch.from_numpy(hx))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(y).copy() for y in ys]
        step()  # the same calls, eagerly
        eager = [to_host(y) for y in ys]
        print(f"[graph] replay {rep}", flush=True)
        for k, (fmt, rows, cols) in enumerate(SHAPES):
            assert np.array_equal(got[k].view(np.uint32), eager[k].view(np.uint32)), (rep, k)
            Wh = to_host(mats[k])
            ref, S = oracle.matvec(fmt, Wh, rows, cols, host_x[k], nthreads=oracle_threads())
            assert_within_tolerance(got[k], ref, S, f"graph replay {rep} fmt={fmt} {rows}x{cols}")


def test_graph_replays_of_fused_variants(gq, oracle):
    """gq_matvec_acc, gq_matvec_swiglu and gq_matvec_experts captured in one
    graph: each replay (after eager resets of the accumulated output and new
    activations) equals the same calls made eagerly, bit for bit."""
    import torch

    rng = synth.rng_for(810, 0)
    rows, cols = 600, 1024
    Wacc = to_dev(synth.weights(12, rows, cols, rng))
    Wgu = to_dev(synth.weights(14, 2 * rows, cols, rng))
    n_expert, erows, xk, n_assign = 6, 300, 2, 8
    Wex = to_dev(synth.weights(13, n_expert * erows, cols, rng))
    ids = to_dev(rng.integers(0, n_expert, n_assign).astype(np.int32))
    x = torch.empty(cols, dtype=torch.float32, device="cuda")
    X = torch.empty((n_assign // xk, cols), dtype=torch.float32, device="cuda")
    y0 = torch.empty(rows, dtype=torch.float32, device="cuda")
    yacc = torch.empty(rows, dtype=torch.float32, device="cuda")
    ysw = torch.empty(rows, dtype=torch.float32, device="cuda")
    Yex = torch.empty((n_assign, erows), dtype=torch.float32, device="cuda")

    def step():
        gq.gq_matvec_acc(12, Wacc, rows, cols, x, yacc)
        gq.gq_matvec_swiglu(14, Wgu, rows, cols, x, y=ysw)
        gq.gq_matvec_experts(13, Wex, n_expert, erows, cols, X, xk, ids, Y=Yex)

    def fill(rep):
        r = synth.rng_for(811 + rep, 0)
        x.copy_(torch.from_numpy(synth.activations(cols, r)))
        X.copy_(torch.from_numpy(synth.activations((n_assign // xk, cols), r)))
        y0.copy_(torch.from_numpy(synth.activations(rows, r)))
        yacc.copy_(y0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fill(0)
        step()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for rep in range(3):
        fill(rep + 1)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(t).copy() for t in (yacc, ysw, Yex)]
        yacc.copy_(y0)
        step()
        eager = [to_host(t) for t in (yacc, ysw, Yex)]
        print(f"[graph] fused variants replay {rep}", flush=True)
        for g, e in zip(got, eager):
            assert np.array_equal(g.view(np.uint32), e.view(np.uint32)), rep
        # the accumulated output is fl(y0 + p) with |p - W x| <= 2e-4 S: within
        # 2e-4 S plus the one rounding of the fp32 addition (2^-24 |y0 + W x|,
        # and the same of the tolerance itself)
        ref, S = oracle.matvec(12, to_host(Wacc), rows, cols, to_host(x))
        want = to_host(y0).astype(np.float64) + ref
        err = np.abs(got[0].astype(np.float64) - want)
        assert (err <= 2e-4 * S * (1 + 2.0 ** -23) + 2.0 ** -24 * np.abs(want) + 1e-38).all(), \
            f"graph acc replay {rep}"


# (fmt, rows, cols, M): the Q4_K matrix-core tiles (64x16 split in four,
# 128x32 split in two, 256x64), the fp32 matrix cores, the int8 path
# Q4_K on three fp16 tiles, Q6_K / Q8_0 / Q5_K on the fp16 kernels, Q6_K
# rows of 3 super-blocks on the fp32 matrix cores
MATMULS = [(12, 14336, 4096, 16), (12, 14336, 4096, 64), (12, 4096, 4096, 512), (14, 1024, 4096, 40),
           (8, 4096, 4096, 64), (13, 1024, 4096, 32), (14, 1024, 768, 40)]


def test_graph_replays_of_products(gq, oracle):
    """gq_matmul (every tile family), gq_matmul_acc, gq_matmul_swiglu and the
    int8-activation pair captured in one graph: no entry point allocates, so
    all of them capture; each replay (after new activations and a reset of
    the accumulated output, written eagerly) equals the same calls made
    eagerly, bit for bit."""
    import torch

    Ws, Xs, Ys = [], [], []
    for k, (fmt, rows, cols, M) in enumerate(MATMULS):
        rng = synth.rng_for(820, k)
        Ws.append(to_dev(synth.weights(fmt, rows, cols, rng)))
        Xs.append(torch.empty((M, cols), dtype=torch.float32, device="cuda"))
        Ys.append(torch.empty((M, rows), dtype=torch.float32, device="cuda"))
    rows, cols, M = 2048, 4096, 64
    rng = synth.rng_for(821, 0)
    Wgu = to_dev(synth.weights(12, 2 * rows, cols, rng))
    Xm = torch.empty((M, cols), dtype=torch.float32, device="cuda")
    Y0 = torch.empty((M, rows), dtype=torch.float32, device="cuda")
    Yacc = torch.empty((M, rows), dtype=torch.float32, device="cuda")
    Ysw = torch.empty((M, rows), dtype=torch.float32, device="cuda")
    xq = torch.empty(gq.gq_row_bytes(gq.GQ_FMT_Q8_1, cols), dtype=torch.uint8, device="cuda")
    y8 = torch.empty(rows, dtype=torch.float32, device="cuda")

    def step():
        for (fmt, r, c, m), W, X, Y in zip(MATMULS, Ws, Xs, Ys):
            gq.gq_matmul(fmt, W, r, c, X, Y=Y)
        gq.gq_matmul_acc(12, Wgu, rows, cols, Xm, Yacc)
        gq.gq_matmul_swiglu(12, Wgu, rows, cols, Xm, Y=Ysw)
        gq.gq_quantize_q8_1(Xm[0], 1, cols, out=xq)
        gq.gq_matvec_q8_1(12, Wgu, rows, cols, xq, y=y8)

    def fill(rep):
        r = synth.rng_for(822 + rep, 0)
        for (fmt, rr, c, m), X in zip(MATMULS, Xs):
            X.copy_(torch.from_numpy(synth.activations((m, c), r)))
        Xm.copy_(torch.from_numpy(synth.activations((M, cols), r)))
        Y0.copy_(torch.from_numpy(synth.activations((M, rows), r)))
        Yacc.copy_(Y0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fill(0)
        step()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    outs = Ys + [Yacc, Ysw, xq, y8]
    for rep in range(3):
        fill(rep + 1)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [to_host(t).copy() for t in outs]
        Yacc.copy_(Y0)
        step()
        eager = [to_host(t) for t in outs]
        print(f"[graph] products replay {rep}", flush=True)
        for i, (g, e) in enumerate(zip(got, eager)):
            assert np.array_equal(g.view(np.uint8), e.view(np.uint8)), (rep, i)
    # the last replay's first product against the oracle
    fmt, r, c, m = MATMULS[0]
    ref, S = oracle.matmul(fmt, to_host(Ws[0]), r, c, to_host(Xs[0]), nthreads=oracle_threads())
    assert_within_tolerance(got[0], ref, S, "graph product")


def test_graph_moe_steps(gq, oracle):
    """The MoE bucketing, gather and scatter captured in one graph, replayed
    with new expert ids, activations, expert rows and outputs written eagerly
    between replays: every replay bit-equal to the oracle."""
    import torch
    n_tok, k, n_expert, cols, rows = 200, 2, 8, 96, 64
    n = n_tok * k
    ids = torch.zeros(n, dtype=torch.int32, device="cuda")
    X = torch.zeros((n_tok, cols), dtype=torch.float32, device="cuda")
    Yb = torch.zeros((n, rows), dtype=torch.float32, device="cuda")
    w = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.zeros((n_tok, rows), dtype=torch.float32, device="cuda")
    counts = torch.empty(n_expert, dtype=torch.int64, device="cuda")
    order = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int32, device="cuda")
    Xb = torch.empty((n, cols), dtype=torch.float32, device="cuda")

    def step():
        gq.gq_moe_bucket(ids, n_expert, counts, order, pos)
        gq.gq_moe_gather(X, k, pos, Xb)
        gq.gq_moe_scatter(Yb, pos, w, k, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for rep in range(3):
        rng = synth.rng_for(805, rep)
        hid = rng.integers(0, n_expert, size=n).astype(np.int32)
        hX = synth.activations((n_tok, cols), rng)
        hY = synth.activations((n, rows), rng)
        hw = rng.random(n).astype(np.float32)
        ho = synth.activations((n_tok, rows), rng)
        for t, h in ((ids, hid), (X, hX), (Yb, hY), (w, hw), (out, ho)):
            t.copy_(torch.from_numpy(h))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] moe replay {rep}", flush=True)
        wc, wo, wp = oracle.moe_bucket(hid, n_expert)
        assert np.array_equal(to_host(counts), wc) and np.array_equal(to_host(pos), wp)
        assert np.array_equal(to_host(order), wo)
        assert np.array_equal(to_host(Xb).view(np.uint32), oracle.moe_gather(hX, k, wp, cols).view(np.uint32))
        want = oracle.moe_scatter(ho, hY, wp, hw, k)
        assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32))
