"""CPU oracle for GGUF Q8_0 / Q4_K / Q5_0 / Q5_K / Q6_K dequant, matvec and
small matmul.

TEST INFRASTRUCTURE ONLY. This package defines the values the GPU library
must reproduce. Only the test-suite, the smoke check and the CPU-baseline leg
of ``bench.py`` may import it; the product path never does. It shares no
code with ``gguf_block_quant_gq_amd``.

The arithmetic lives in ``gq_oracle.c`` (plain C, ``-O2 -ffp-contract=off``):
hand-decoded fp16, block unpack, fp32 dequant ``(d*sc)*q - dmin*m`` (Q4_K,
Q5_K), ``(d*scale)*(q - 32)`` (Q6_K), ``d*(q - 16)`` (Q5_0) or ``d*q``
(Q8_0), and f64-accumulated sums. The page and section each step
follows are cited in that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gq_oracle.c")
# GQ_SANITIZE=1 (set by tests/sanitize.py) selects a build with the clang
# address and undefined-behaviour sanitizers, loaded into a process that has
# their runtime preloaded.
_SANITIZE = os.environ.get("GQ_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libgq_oracle_san.so" if _SANITIZE else "libgq_oracle.so")

TYPE_Q8_0 = 8
TYPE_Q4_K = 12
TYPE_Q5_0 = 6
TYPE_Q5_K = 13
TYPE_Q6_K = 14
TYPE_Q8_0_SPLIT = 1008
TYPE_Q8_1 = 9  # activation blocks only

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC,
           "-lm", "-lpthread"]
    if _SANITIZE:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-ffp-contract=off",
               "-fno-fast-math", "-fsanitize=address", "-fsanitize=undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-shared-libsan",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC,
               "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gqo_row_bytes.argtypes = [i32, i64]
    lib.gqo_row_bytes.restype = i64
    lib.gqo_f16_to_f32_n.argtypes = [vp, i64, vp]
    lib.gqo_f16_to_f32_n.restype = None
    lib.gqo_f32_to_f16_rne.argtypes = [ctypes.c_float]
    lib.gqo_f32_to_f16_rne.restype = ctypes.c_uint16
    lib.gqo_q4_k_unpack_scales.argtypes = [vp, vp, vp]
    lib.gqo_q4_k_unpack_scales.restype = None
    lib.gqo_dequant.argtypes = [i32, vp, i64, i64, vp]
    lib.gqo_dequant.restype = i32
    lib.gqo_matvec.argtypes = [i32, vp, i64, i64, vp, vp, vp, i32]
    lib.gqo_matvec.restype = i32
    lib.gqo_matmul.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp, i32]
    lib.gqo_matmul.restype = i32
    lib.gqo_q8_0_split_repack.argtypes = [vp, i64, i64, vp]
    lib.gqo_q8_0_split_repack.restype = i32
    lib.gqo_quantize_q8_0.argtypes = [vp, i64, i64, vp]
    lib.gqo_quantize_q8_0.restype = i32
    lib.gqo_quantize_q4_k.argtypes = [vp, i64, i64, vp]
    lib.gqo_quantize_q4_k.restype = i32
    lib.gqo_quantize_q8_1.argtypes = [vp, i64, i64, vp]
    lib.gqo_quantize_q8_1.restype = i32
    lib.gqo_dequant_q8_1.argtypes = [vp, i64, i64, vp]
    lib.gqo_dequant_q8_1.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(status: int, what: str) -> None:
    if status != 0:
        raise ValueError(f"oracle {what} failed with status {status}")


def _as_bytes(W) -> np.ndarray:
    W = np.ascontiguousarray(W)
    if W.dtype != np.uint8:
        W = W.view(np.uint8)
    return W.reshape(-1)


def row_bytes(fmt: int, cols: int) -> int:
    return int(_load().gqo_row_bytes(fmt, cols))


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).reshape(-1)
    out = np.empty(h.shape, np.float32)
    _load().gqo_f16_to_f32_n(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_f16_rne(f: float) -> int:
    return int(_load().gqo_f32_to_f16_rne(float(f)))


def q4_k_unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    s = np.ascontiguousarray(s12, dtype=np.uint8).reshape(12)
    sc = np.empty(8, np.uint8)
    m = np.empty(8, np.uint8)
    _load().gqo_q4_k_unpack_scales(_ptr(s), _ptr(sc), _ptr(m))
    return sc, m


def dequant(fmt: int, W, rows: int, cols: int) -> np.ndarray:
    Wb = _as_bytes(W)
    if Wb.size < rows * row_bytes(fmt, cols):
        raise ValueError("W holds fewer bytes than rows * row_bytes")
    out = np.empty((rows, cols), np.float32)
    _check(_load().gqo_dequant(fmt, _ptr(Wb), rows, cols, _ptr(out)), "dequant")
    return out


def matmul(fmt: int, W, rows: int, cols: int, X, nthreads: int = 1):
    """Y[m, r] = sum_c w(r,c) X[m,c] in f64, and S[m, r] = sum_c |w X|."""
    Wb = _as_bytes(W)
    if Wb.size < rows * row_bytes(fmt, cols):
        raise ValueError("W holds fewer bytes than rows * row_bytes")
    X = np.ascontiguousarray(X, dtype=np.float32)
    X2 = X.reshape(-1, cols)
    M = X2.shape[0]
    Y = np.empty((M, rows), np.float64)
    S = np.empty((M, rows), np.float64)
    _check(_load().gqo_matmul(fmt, _ptr(Wb), rows, cols, _ptr(X2), M,
                              _ptr(Y), _ptr(S), int(nthreads)), "matmul")
    return Y, S


def matvec(fmt: int, W, rows: int, cols: int, x, nthreads: int = 1):
    """y[r] = sum_c w(r,c) x[c] in f64, and S[r] = sum_c |w x|."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(cols)
    Y, S = matmul(fmt, W, rows, cols, x.reshape(1, cols), nthreads)
    return Y[0], S[0]


def select_rows(fmt: int, W, cols: int, row_idx) -> np.ndarray:
    """The packed bytes of the given rows, as a new contiguous matrix."""
    Wb = _as_bytes(W)
    rb = row_bytes(fmt, cols)
    idx = np.asarray(row_idx, dtype=np.int64)
    return Wb.reshape(-1, rb)[idx].reshape(-1) if Wb.size % rb == 0 else \
        np.concatenate([Wb[i * rb:(i + 1) * rb] for i in idx])


def quantize(fmt: int, w) -> np.ndarray:
    """Test-only reference quantiser: fp32 [rows, cols] -> packed bytes."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim == 1:
        w = w.reshape(1, -1)
    rows, cols = w.shape
    out = np.zeros(rows * row_bytes(fmt, cols), np.uint8)
    fn = _load().gqo_quantize_q8_0 if fmt == TYPE_Q8_0 else _load().gqo_quantize_q4_k
    if fmt not in (TYPE_Q8_0, TYPE_Q4_K):
        raise ValueError(f"unknown type {fmt}")
    _check(fn(_ptr(w), rows, cols, _ptr(out)), "quantize")
    return out


def silu(v):
    """silu(v) = v / (1 + e^-v) = v * sigmoid(v), in f64: the activation of the
    SwiGLU feed-forward ("nurllama 0.18.1 API", model.nu section: the llama
    shape's SwiGLU FFN; kernels.nu section: g <- silu(g) * u in place). For
    very negative v, e^-v overflows to inf and the result is -0."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_matvec(fmt: int, W, rows: int, cols: int, x, nthreads: int = 1):
    """The fused gate|up projection: W holds 2*rows rows, gate rows first and
    up rows after them (one tensor whose parts are row ranges: "nurllama"
    README, "What it runs", phi3's ffn_up). Returns (y, g, u, S_g, S_u) with
    g, u the f64 matvecs of the two halves, y = silu(g) * u in f64 and S the
    sums of |w*x| of each half."""
    Y, S = matvec(fmt, W, 2 * rows, cols, x, nthreads)
    g, u = Y[:rows], Y[rows:]
    return silu(g) * u, g, u, S[:rows], S[rows:]


def experts_matvec(fmt: int, W, n_expert: int, rows: int, cols: int, X, xk: int, expid,
                   nthreads: int = 1):
    """The expert-batched matvec of a mixture-of-experts layer ("nurllama
    0.18.1 API", kernels.nu section: one batched matvec over all expert
    assignments, output row a using expert expid[a] and input row a / xk of
    x). W holds the n_expert matrices back to back. Returns (Y, S), both
    [n_assign, rows] f64; an id outside [0, n_expert) gives a NaN row."""
    Wb = _as_bytes(W)
    eb = rows * row_bytes(fmt, cols)
    if Wb.size < n_expert * eb:
        raise ValueError("W holds fewer bytes than n_expert * rows * row_bytes")
    X = np.ascontiguousarray(X, dtype=np.float32).reshape(-1, cols)
    ids = np.asarray(expid, dtype=np.int64).reshape(-1)
    Y = np.full((ids.size, rows), np.nan)
    S = np.full((ids.size, rows), np.nan)
    for a, e in enumerate(ids):
        if 0 <= e < n_expert:
            Y[a], S[a] = matvec(fmt, Wb[e * eb:(e + 1) * eb], rows, cols, X[a // xk], nthreads)
    return Y, S


def moe_bucket(expid, n_expert: int):
    """The assignments bucketed by expert (the Loom porting skill, "What the
    starter generates": the MoE generator buckets the rows by expert before
    the grouped GEMMs; the order inside a bucket is not printed, the reading
    taken is the assignments' own order). Returns (counts, order, pos):
    counts[e] = how many ids equal e; pos[a] = the first slot of bucket e
    (the counts of the experts before e) plus how many earlier assignments
    have the same id; order[pos[a]] = a. An id outside [0, n_expert) is
    dropped: pos -1, counted nowhere, and order's unused tail stays -1."""
    ids = np.asarray(expid, dtype=np.int64).reshape(-1)
    counts = np.zeros(n_expert, dtype=np.int64)
    for e in ids:
        if 0 <= e < n_expert:
            counts[e] += 1
    start = np.zeros(n_expert, dtype=np.int64)
    running = 0
    for e in range(n_expert):
        start[e] = running
        running += counts[e]
    pos = np.full(ids.size, -1, dtype=np.int32)
    order = np.full(ids.size, -1, dtype=np.int32)
    nxt = start.copy()
    for a, e in enumerate(ids):
        if 0 <= e < n_expert:
            pos[a] = nxt[e]
            order[nxt[e]] = a
            nxt[e] += 1
    return counts, order, pos


def moe_gather(X, k: int, pos, cols: int) -> np.ndarray:
    """Each placed assignment's activation row in its bucket slot:
    Xb[pos[a]] = X[a // k] (a = position * k + slot). Slots no assignment
    fills are NaN here (the GPU leaves them as they were)."""
    X = np.ascontiguousarray(X, dtype=np.float32).reshape(-1, cols)
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    n = pos.size
    Xb = np.full((n, cols), np.nan, dtype=np.float32)
    for a in range(n):
        if 0 <= pos[a] < n:
            Xb[pos[a]] = X[a // k]
    return Xb


def moe_scatter(out, Yb, pos, w, k: int) -> np.ndarray:
    """The scatter that ends an MoE layer ("nurllama 0.18.1 API", kernels.nu
    section: for each position, the weighted sum over its k selected experts'
    rows is added onto the output). Here the experts' rows sit in bucket
    order, so slot j of position t reads row pos[t k + j]. In fp32 as the
    pages' buffers are, summed in slot order starting from 0, every product
    and sum rounded on its own, then added onto out; a dropped slot (pos
    outside [0, n)) adds nothing. Returns the new out."""
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    n = pos.size
    Yb = np.ascontiguousarray(Yb, dtype=np.float32).reshape(n, -1)
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    res = np.array(out, dtype=np.float32).reshape(n // k, -1).copy()
    for t in range(n // k):
        acc = np.zeros(res.shape[1], dtype=np.float32)
        for j in range(k):
            a = t * k + j
            if 0 <= pos[a] < n:
                prod = np.multiply(w[a], Yb[pos[a]], dtype=np.float32)
                acc = np.add(acc, prod, dtype=np.float32)
        res[t] = np.add(res[t], acc, dtype=np.float32)
    return res


def q8_0_split_repack(W, rows: int, cols: int) -> np.ndarray:
    """Q8_0 rows repacked into the split per-row layout (scales first, padded
    to 16 bytes, then the codes): the oracle's reading of the q8_0 repack of
    "nurllama 0.18.1 API", kernels.nu section."""
    Wb = _as_bytes(W)
    if Wb.size < rows * row_bytes(TYPE_Q8_0, cols):
        raise ValueError("W holds fewer bytes than rows * row_bytes")
    out = np.empty(rows * row_bytes(TYPE_Q8_0_SPLIT, cols), np.uint8)
    _check(_load().gqo_q8_0_split_repack(_ptr(Wb), rows, cols, _ptr(out)), "q8_0_split_repack")
    return out



def quantize_q8_1(X, cols: int | None = None) -> np.ndarray:
    """Activations [n, cols] (or one row) -> Q8_1 blocks, n rows of
    row_bytes(TYPE_Q8_1, cols) bytes: the int8-activation path's input
    (the Loom porting skill, "What the starter generates": llama.cpp's Q8_1
    numerics; the reading is spelled out in gq_oracle.c)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 1:
        X = X.reshape(1, -1)
    n, c = X.shape
    out = np.empty(n * row_bytes(TYPE_Q8_1, c), np.uint8)
    _check(_load().gqo_quantize_q8_1(_ptr(X), n, c, _ptr(out)), "quantize_q8_1")
    return out


def dequant_q8_1(xq, n: int, cols: int) -> np.ndarray:
    """The values x^ = fp16 d * q that the int8 path multiplies, [n, cols]."""
    xb = _as_bytes(xq)
    if xb.size < n * row_bytes(TYPE_Q8_1, cols):
        raise ValueError("xq holds fewer bytes than n * row_bytes")
    out = np.empty((n, cols), np.float32)
    _check(_load().gqo_dequant_q8_1(_ptr(xb), n, cols, _ptr(out)), "dequant_q8_1")
    return out


def matvec_q8_1(fmt: int, W, rows: int, cols: int, xq, nthreads: int = 1):
    """y = W x^ with x^ the dequantised Q8_1 activation row (f64, with
    S = sum |w x^|): the definition the int8-activation matvec is held to."""
    xh = dequant_q8_1(xq, 1, cols)[0]
    return matvec(fmt, W, rows, cols, xh, nthreads=nthreads)
