"""Randomized sweep of gq_matmul (store and accumulate), gq_matvec, the
split Q8_0 repack and the MoE prefill chain on the GPU, for a time budget: every case draws a format,
rows (1..2999), columns (up to 70 blocks or super-blocks, ragged or whole)
and activation rows M (1..200) from a seeded generator, checks a sample of
output rows against the f64 oracle at 2e-4 * sum |w x| and that nothing is
written past the outputs. Prints each case before running it and exits 1 on
any failure. Not collected by pytest (the seeded parity tests are); run it on
a machine with a GPU:

    python tests/fuzz.py [--seconds 240] [--seed 11]
"""
import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

FORMATS = (8, 12, 6, 13, 14, 1008)
M_CHOICES = (1, 2, 3, 7, 15, 16, 17, 31, 64, 65, 100, 200)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--seconds", type=float, default=240.0)
    ap.add_argument("--seed", type=int, default=11)
    args = ap.parse_args()

    import torch

    import gguf_block_quant_gq_amd as gq
    import oracle
    import synth
    from helpers import oracle_threads, sentinel_buffer, to_dev, to_host

    torch.cuda.set_device(0)
    failures = 0

    def within(got, ref, S, what, info):
        nonlocal failures
        ok = np.abs(got.astype(np.float64) - ref) <= 2e-4 * S + 1e-30
        if not ok.all():
            failures += 1
            i = tuple(np.argwhere(~ok)[0])
            print(f"  FAIL {what} {info} at {i}: got {got[i]} ref {ref[i]} S {S[i]}", flush=True)

    def pad_ok(buf, n, what, info):
        nonlocal failures
        if not np.isnan(to_host(buf)[n:]).all():
            failures += 1
            print(f"  FAIL {what} {info}: wrote past the output", flush=True)

    def moe_case(n, rng):
        """The MoE prefill chain on random ids: bucketing, gather and scatter
        bit-equal to the oracle, the grouped product with device counts on a
        sample of rows against the oracle's expert products."""
        fmt = int(rng.choice([12, 13, 8, 1008, 14, 6]))
        base = 8 if fmt == 1008 else fmt
        step = {12: 4, 13: 4, 1008: 4, 8: 64, 6: 64, 14: 512}[fmt]
        cols = int(rng.integers(1, 12)) * step if fmt == 14 else int(rng.integers(1, 1500 // step + 2)) * step
        rows = int(rng.integers(1, 600))
        n_expert, k, n_tok = int(rng.integers(1, 41)), int(rng.integers(1, 5)), int(rng.integers(1, 301))
        info = f"case {n} moe fmt={fmt} rows={rows} cols={cols} experts={n_expert} k={k} positions={n_tok}"
        print(info, flush=True)
        ids = rng.integers(-1, n_expert + 1, size=n_tok * k).astype(np.int32)
        W = synth.weights(base, n_expert * rows, cols, rng)
        X = synth.activations((n_tok, cols), rng)
        Wd = to_dev(W)
        if fmt == 1008:
            Wd = gq.gq_q8_0_split_repack(Wd, n_expert * rows, cols)
        counts, order, pos = gq.gq_moe_bucket(to_dev(ids), n_expert)
        wc, wo, wp = oracle.moe_bucket(ids, n_expert)
        nonlocal failures
        if not (np.array_equal(to_host(counts), wc) and np.array_equal(to_host(pos), wp)):
            failures += 1
            print(f"  FAIL bucket {info}", flush=True)
            return
        placed = int(wc.sum())
        Xb = gq.gq_moe_gather(to_dev(X), k, pos)
        Yb = gq.gq_matmul_experts_dev(fmt, Wd, n_expert, rows, cols, Xb, counts) if placed else None
        if placed:
            eb = rows * oracle.row_bytes(base, cols)
            Yh = to_host(Yb)
            for p in np.unique(rng.integers(0, placed, 6)):
                a = int(wo[p])
                e = int(ids[a])
                idx = np.unique(rng.integers(0, rows, 8))
                ref, S = oracle.matmul(base, oracle.select_rows(base, W[e * eb:(e + 1) * eb], cols, idx),
                                       idx.size, cols, X[a // k][None, :])
                within(Yh[p][idx][None, :], ref, S, "grouped product, device counts", info)
        w = rng.random(n_tok * k).astype(np.float32)
        out0 = synth.activations((n_tok, rows), rng)
        out = to_dev(out0.copy())
        # Yb has n_assign rows; the scatter reads the placed ones through pos
        Ybf = Yb if placed else to_dev(np.zeros((n_tok * k, rows), np.float32))
        gq.gq_moe_scatter(Ybf, pos, to_dev(w), k, out)
        want = oracle.moe_scatter(out0, to_host(Ybf), wp, w, k)
        if not np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32)):
            failures += 1
            print(f"  FAIL scatter {info}", flush=True)

    t0, n = time.time(), 0
    while time.time() - t0 < args.seconds:
        rng = np.random.default_rng([args.seed, n])
        if rng.random() < 0.15:
            moe_case(n, rng)
            n += 1
            continue
        fmt = FORMATS[int(rng.integers(0, len(FORMATS)))]
        base = 8 if fmt == 1008 else fmt
        qk = 256 if base in (12, 13, 14) else 32
        cols = int(rng.integers(1, 70 * qk))
        if rng.random() < 0.5:
            # the fp16 matrix-core route needs cols % 4 == 0 (and, for Q8_0,
            # Q5_0 and Q6_K, rows of an even number of blocks or super-blocks)
            cols = (cols + 3) // 4 * 4
        rows = int(rng.integers(1, 3000))
        M = int(rng.choice(M_CHOICES))
        acc = M > 1 and rng.random() < 0.5
        info = f"case {n} fmt={fmt} rows={rows} cols={cols} M={M}{' acc' if acc else ''}"
        print(info, flush=True)
        W = synth.weights(base, rows, cols, rng)
        X = synth.activations((M, cols), rng)
        Wd, Xd = to_dev(W), to_dev(X)
        if fmt == 1008:
            Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
        idx = np.unique(np.concatenate([rng.integers(0, rows, 12), [0, rows - 1]]))
        ref, S = oracle.matmul(base, oracle.select_rows(base, W, cols, idx), idx.size, cols, X,
                               nthreads=oracle_threads())
        Y = sentinel_buffer(M * rows)
        if acc:
            Y[:M * rows].zero_()
            gq.gq_matmul_acc(fmt, Wd, rows, cols, Xd, Y[:M * rows])
        else:
            gq.gq_matmul(fmt, Wd, rows, cols, Xd, Y=Y[:M * rows])
        pad_ok(Y, M * rows, "matmul", info)
        within(to_host(Y)[:M * rows].reshape(M, rows)[:, idx], ref, S, "matmul", info)
        y = sentinel_buffer(rows)
        gq.gq_matvec(fmt, Wd, rows, cols, Xd[M - 1], y=y[:rows])
        pad_ok(y, rows, "matvec", info)
        within(to_host(y)[:rows][idx], ref[M - 1], S[M - 1], "matvec", info)
        n += 1
    print(f"fuzz done: {n} cases, {failures} failures, {time.time() - t0:.0f} s, seed {args.seed}",
          flush=True)
    return 1 if failures else 0


if __name__ == "__main__":
    sys.exit(main())
