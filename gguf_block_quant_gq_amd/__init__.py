"""Python binding of libgq, the MI355X (gfx950) block-quantised GEMV/GEMM library.

The functions mirror the C ABI in ``include/gq.h`` one for one and only
marshal arguments: torch tensors are used for device memory and streams, and
every step of the computation runs in the HIP kernels of ``libgq.so``. There
is no CPU fallback: if the library is not built, loading raises.

    gq_dequant(fmt, W, rows, cols, out=None)           -> out [rows, cols] fp32
    gq_matvec(fmt, W, rows, cols, x, y=None)           -> y [rows] fp32
    gq_matvec_acc(fmt, W, rows, cols, x, y)            -> y += W x
    gq_matvec_swiglu(fmt, W, rows, cols, x, y=None)    -> y = silu(W_gate x) * (W_up x)
    gq_q8_0_split_repack(W, rows, cols, out=None)      -> W in the split Q8_0 layout
    gq_matvec_experts(fmt, W, n_expert, rows, cols, X, xk, expid, Y=None)
                                                       -> Y[a] = W[expid[a]] X[a // xk]
    gq_matmul(fmt, W, rows, cols, X, Y=None)           -> Y [M, rows] fp32
    gq_matmul_acc(fmt, W, rows, cols, X, Y)            -> Y += W X
    gq_matmul_swiglu(fmt, W, rows, cols, X, Y=None)    -> Y = silu(W_gate X) * (W_up X)
    gq_quantize_q8_1(X, n, cols, out=None)             -> Q8_1 activation blocks
    gq_matvec_q8_1(fmt, W, rows, cols, xq, y=None)     -> y = W x^ (int8 activations)
    gq_moe_bucket(expid, n_expert)                     -> (counts, order, pos) by expert
    gq_moe_gather(X, k, pos, Xb=None)                  -> Xb[pos[a]] = X[a // k]
    gq_moe_scatter(Yb, pos, w, k, out)                 -> out[t] += sum_j w Yb[pos[t k + j]]
    gq_matmul_experts_dev(fmt, W, n_expert, rows, cols, X, counts, Y=None)
                                                       -> gq_matmul_experts, counts on the device

W is a uint8 CUDA tensor holding rows * gq_row_bytes(fmt, cols) bytes of
GGUF blocks; fmt is FMT_Q8_0 (8), FMT_Q4_K (12), FMT_Q5_0 (6), FMT_Q5_K (13)
or FMT_Q6_K (14).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GQ_LIBRARY names another build of the same library (the sanitizer build
# that tests/sanitize.py loads); by default the in-tree one.
LIB_PATH = os.environ.get("GQ_LIBRARY") or os.path.join(HERE, "libgq.so")

FMT_Q8_0 = 8
FMT_Q4_K = 12
FMT_Q5_0 = 6
FMT_Q5_K = 13
FMT_Q6_K = 14
FMT_Q8_0_SPLIT = 1008  # Q8_0 repacked by gq_q8_0_split_repack (scales apart from codes)
GQ_FMT_Q8_1 = 9        # activation blocks of the int8 path (gq_quantize_q8_1), never weights

GQ_OK = 0
GQ_ERR_NULL = 1
GQ_ERR_FMT = 2
GQ_ERR_SHAPE = 3
GQ_ERR_ALIGN = 4
GQ_ERR_DEVICE = 5
GQ_ERR_OVERLAP = 6

EXPORTS = ("gq_row_bytes", "gq_status_str", "gq_dequant", "gq_matvec", "gq_matvec_acc",
           "gq_matvec_swiglu", "gq_matvec_experts", "gq_matvec_batch", "gq_q8_0_split_repack",
           "gq_matmul", "gq_matmul_experts", "gq_quantize_q8_1", "gq_matvec_q8_1",
           "gq_matmul_acc", "gq_matmul_swiglu", "gq_moe_bucket", "gq_moe_gather", "gq_moe_scatter",
           "gq_matmul_experts_dev")

_lib = None


class GQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


def load_library():
    """Load libgq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "python gguf_block_quant_gq_amd/_build.py")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gq_row_bytes.argtypes = [i32, i64]
    lib.gq_row_bytes.restype = i64
    lib.gq_status_str.argtypes = [i32]
    lib.gq_status_str.restype = ctypes.c_char_p
    lib.gq_dequant.argtypes = [i32, vp, i64, i64, vp]
    lib.gq_dequant.restype = i32
    for name in ("gq_matvec", "gq_matvec_acc", "gq_matvec_swiglu"):
        getattr(lib, name).argtypes = [i32, vp, i64, i64, vp, vp, vp]
        getattr(lib, name).restype = i32
    lib.gq_q8_0_split_repack.argtypes = [vp, i64, i64, vp, vp]
    lib.gq_q8_0_split_repack.restype = i32
    lib.gq_matvec_experts.argtypes = [i32, vp, i64, i64, i64, vp, i64, vp, i64, vp, vp]
    lib.gq_matvec_experts.restype = i32
    lib.gq_matmul_experts.argtypes = [i32, vp, i64, i64, i64, vp, ctypes.POINTER(i64), vp, vp]
    lib.gq_matmul_experts.restype = i32
    for name in ("gq_matmul", "gq_matvec_batch", "gq_matmul_acc", "gq_matmul_swiglu"):
        getattr(lib, name).argtypes = [i32, vp, i64, i64, vp, i64, vp, vp]
        getattr(lib, name).restype = i32
    lib.gq_quantize_q8_1.argtypes = [vp, i64, i64, vp, vp]
    lib.gq_quantize_q8_1.restype = i32
    lib.gq_matvec_q8_1.argtypes = [i32, vp, i64, i64, vp, vp, vp]
    lib.gq_matvec_q8_1.restype = i32
    lib.gq_moe_bucket.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.gq_moe_bucket.restype = i32
    lib.gq_moe_gather.argtypes = [vp, i64, i64, vp, i64, vp, vp]
    lib.gq_moe_gather.restype = i32
    lib.gq_moe_scatter.argtypes = [vp, i64, vp, vp, i64, i64, vp, vp]
    lib.gq_moe_scatter.restype = i32
    lib.gq_matmul_experts_dev.argtypes = [i32, vp, i64, i64, i64, vp, vp, i64, vp, vp]
    lib.gq_matmul_experts_dev.restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().gq_status_str(int(status)).decode()


def gq_row_bytes(fmt: int, cols: int) -> int:
    return int(load_library().gq_row_bytes(int(fmt), int(cols)))


# ------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    return int(t.data_ptr())


def _check_dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device (and its stream)
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_w(fmt, W, rows, cols):
    _check_dev(W, "W")
    need = rows * gq_row_bytes(fmt, cols) if gq_row_bytes(fmt, cols) >= 0 else 0
    if W.numel() * W.element_size() < need:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, needs {need}")


def _stream_handle(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def gq_dequant(fmt: int, W, rows: int, cols: int, out=None):
    """Bit-exact fp32 expansion of W (blocks until done, null stream)."""
    torch = _torch()
    _check_w(fmt, W, rows, cols)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=W.device)
    _check_dev(out, "out", torch.float32)
    if out.numel() < rows * cols:
        raise ValueError("out is too small")
    st = load_library().gq_dequant(int(fmt), _ptr(W), int(rows), int(cols), _ptr(out))
    if st != GQ_OK:
        raise GQError(st, "gq_dequant")
    return out


def _matvec(name: str, fmt: int, W, rows: int, cols: int, x, y, stream, wrows: int):
    torch = _torch()
    _check_w(fmt, W, wrows, cols)
    _check_dev(x, "x", torch.float32)
    if x.numel() < cols:
        raise ValueError("x is too small")
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=W.device)
    _check_dev(y, "y", torch.float32)
    if y.numel() < rows:
        raise ValueError("y is too small")
    st = getattr(load_library(), name)(int(fmt), _ptr(W), int(rows), int(cols), _ptr(x), _ptr(y),
                                       _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, name)
    return y


def gq_matvec(fmt: int, W, rows: int, cols: int, x, y=None, stream=None):
    """y = W x on `stream` (default: torch's current stream), asynchronous."""
    return _matvec("gq_matvec", fmt, W, rows, cols, x, y, stream, rows)


def gq_quantize_q8_1(X, n: int, cols: int, out=None, stream=None):
    """n rows of cols fp32 activations -> Q8_1 blocks (uint8, n *
    gq_row_bytes(GQ_FMT_Q8_1, cols) bytes), asynchronous."""
    torch = _torch()
    _check_dev(X, "X", torch.float32)
    if X.numel() < n * cols:
        raise ValueError("X is too small")
    need = n * gq_row_bytes(GQ_FMT_Q8_1, cols)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=X.device)
    _check_dev(out, "out", torch.uint8)
    if out.numel() < need:
        raise ValueError("out is too small")
    st = load_library().gq_quantize_q8_1(_ptr(X), int(n), int(cols), _ptr(out), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_quantize_q8_1")
    return out


def gq_matvec_q8_1(fmt: int, W, rows: int, cols: int, xq, y=None, stream=None):
    """y = W x^ with xq one quantised activation row (gq_quantize_q8_1),
    integer dot products, asynchronous."""
    torch = _torch()
    _check_w(fmt, W, rows, cols)
    _check_dev(xq, "xq", torch.uint8)
    if xq.numel() < gq_row_bytes(GQ_FMT_Q8_1, cols):
        raise ValueError("xq is too small")
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=W.device)
    _check_dev(y, "y", torch.float32)
    if y.numel() < rows:
        raise ValueError("y is too small")
    st = load_library().gq_matvec_q8_1(int(fmt), _ptr(W), int(rows), int(cols), _ptr(xq), _ptr(y),
                                       _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_matvec_q8_1")
    return y


def gq_matvec_acc(fmt: int, W, rows: int, cols: int, x, y, stream=None):
    """y += W x (y holds the addend), asynchronous."""
    if y is None:
        raise ValueError("gq_matvec_acc needs y")
    return _matvec("gq_matvec_acc", fmt, W, rows, cols, x, y, stream, rows)


def gq_matvec_swiglu(fmt: int, W, rows: int, cols: int, x, y=None, stream=None):
    """y[r] = silu(g_r) * u_r for the gate|up tensor W (2 * rows weight rows:
    gate rows first, then up rows), asynchronous."""
    return _matvec("gq_matvec_swiglu", fmt, W, rows, cols, x, y, stream, 2 * rows)


def gq_matvec_experts(fmt: int, W, n_expert: int, rows: int, cols: int, X, xk: int, expid,
                      Y=None, stream=None):
    """Y[a] = W[expid[a]] @ X[a // xk] for every assignment a (expid: int32
    CUDA tensor of n_assign ids), asynchronous."""
    torch = _torch()
    _check_w(fmt, W, n_expert * rows, cols)
    _check_dev(X, "X", torch.float32)
    _check_dev(expid, "expid", torch.int32)
    n_assign = expid.numel()
    if X.numel() < -(-n_assign // max(1, xk)) * cols:
        raise ValueError("X is too small")
    if Y is None:
        Y = torch.empty((n_assign, rows), dtype=torch.float32, device=W.device)
    _check_dev(Y, "Y", torch.float32)
    if Y.numel() < n_assign * rows:
        raise ValueError("Y is too small")
    st = load_library().gq_matvec_experts(int(fmt), _ptr(W), int(n_expert), int(rows), int(cols),
                                          _ptr(X), int(xk), _ptr(expid), int(n_assign), _ptr(Y),
                                          _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_matvec_experts")
    return Y


def gq_q8_0_split_repack(W, rows: int, cols: int, out=None, stream=None):
    """Q8_0 rows -> the split per-row layout (uint8 tensor of
    rows * gq_row_bytes(FMT_Q8_0_SPLIT, cols) bytes), asynchronous."""
    torch = _torch()
    _check_w(FMT_Q8_0, W, rows, cols)
    need = rows * gq_row_bytes(FMT_Q8_0_SPLIT, cols)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=W.device)
    _check_dev(out, "out", torch.uint8)
    if out.numel() < need:
        raise ValueError("out is too small")
    st = load_library().gq_q8_0_split_repack(_ptr(W), int(rows), int(cols), _ptr(out),
                                             _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_q8_0_split_repack")
    return out


def _rows_product(name: str, fmt: int, W, rows: int, cols: int, X, Y, stream, wrows=None):
    torch = _torch()
    _check_w(fmt, W, rows if wrows is None else wrows, cols)
    _check_dev(X, "X", torch.float32)
    if X.numel() % cols != 0:
        raise ValueError("X must hold M * cols floats")
    M = X.numel() // cols
    if Y is None:
        Y = torch.empty((M, rows), dtype=torch.float32, device=W.device)
    _check_dev(Y, "Y", torch.float32)
    if Y.numel() < M * rows:
        raise ValueError("Y is too small")
    st = getattr(load_library(), name)(int(fmt), _ptr(W), int(rows), int(cols), _ptr(X), int(M),
                                       _ptr(Y), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, name)
    return Y


def gq_matmul(fmt: int, W, rows: int, cols: int, X, Y=None, stream=None):
    """Y[M, rows] = X[M, cols] W^T on `stream`, asynchronous."""
    return _rows_product("gq_matmul", fmt, W, rows, cols, X, Y, stream)


def gq_matmul_acc(fmt: int, W, rows: int, cols: int, X, Y, stream=None):
    """Y[M, rows] += X[M, cols] W^T (Y holds the addend), asynchronous."""
    if Y is None:
        raise ValueError("gq_matmul_acc needs Y")
    return _rows_product("gq_matmul_acc", fmt, W, rows, cols, X, Y, stream)


def gq_matmul_swiglu(fmt: int, W, rows: int, cols: int, X, Y=None, stream=None):
    """Y[m, r] = silu(g) * u for the gate|up tensor W (2 * rows weight rows:
    gate rows first, then up rows), asynchronous."""
    return _rows_product("gq_matmul_swiglu", fmt, W, rows, cols, X, Y, stream, wrows=2 * rows)


def gq_matvec_batch(fmt: int, W, rows: int, cols: int, X, Y=None, stream=None):
    """Y[b] = W @ X[b] for every row b of X, each row bit-identical to
    gq_matvec of that row, asynchronous."""
    return _rows_product("gq_matvec_batch", fmt, W, rows, cols, X, Y, stream)


def gq_matmul_experts(fmt: int, W, n_expert: int, rows: int, cols: int, X, m_per_expert,
                      Y=None, stream=None):
    """Y = the per-expert products of activation rows bucketed by expert:
    X [sum(m_per_expert), cols] holds expert 0's rows first, then expert 1's,
    ...; m_per_expert is a host sequence of n_expert counts. Asynchronous."""
    torch = _torch()
    counts = [int(m) for m in m_per_expert]
    if len(counts) != n_expert:
        raise ValueError("m_per_expert must hold n_expert counts")
    total = sum(counts)
    _check_w(fmt, W, n_expert * rows, cols)
    _check_dev(X, "X", torch.float32)
    if X.numel() < total * cols:
        raise ValueError("X is too small")
    if Y is None:
        Y = torch.empty((total, rows), dtype=torch.float32, device=W.device)
    _check_dev(Y, "Y", torch.float32)
    if Y.numel() < total * rows:
        raise ValueError("Y is too small")
    arr = (ctypes.c_int64 * max(1, n_expert))(*counts)
    st = load_library().gq_matmul_experts(int(fmt), _ptr(W), int(n_expert), int(rows), int(cols),
                                          _ptr(X), arr, _ptr(Y), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_matmul_experts")
    return Y


def gq_moe_bucket(expid, n_expert: int, counts=None, order=None, pos=None, stream=None):
    """Stable bucketing of the assignments by expert id (expid: int32 GPU
    tensor of n_assign ids): returns (counts int64 [n_expert], order int32
    [n_assign], pos int32 [n_assign]); order is written for the placed
    assignments only. Asynchronous."""
    torch = _torch()
    _check_dev(expid, "expid", torch.int32)
    n_assign = expid.numel()
    dev = expid.device
    if counts is None:
        counts = torch.empty(max(0, int(n_expert)), dtype=torch.int64, device=dev)
    if order is None:
        order = torch.full((n_assign,), -1, dtype=torch.int32, device=dev)
    if pos is None:
        pos = torch.empty(n_assign, dtype=torch.int32, device=dev)
    _check_dev(counts, "counts", torch.int64)
    _check_dev(order, "order", torch.int32)
    _check_dev(pos, "pos", torch.int32)
    if counts.numel() < n_expert or order.numel() < n_assign or pos.numel() < n_assign:
        raise ValueError("an output is too small")
    st = load_library().gq_moe_bucket(_ptr(expid), int(n_assign), int(n_expert), _ptr(counts),
                                      _ptr(order), _ptr(pos), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_moe_bucket")
    return counts, order, pos


def gq_moe_gather(X, k: int, pos, Xb=None, stream=None):
    """Xb[pos[a]] = X[a // k] for the placed assignments (X: fp32 [ceil(n_assign
    / k), cols] GPU tensor, pos from gq_moe_bucket). Asynchronous."""
    torch = _torch()
    _check_dev(X, "X", torch.float32)
    _check_dev(pos, "pos", torch.int32)
    n_assign = pos.numel()
    cols = X.shape[-1] if X.dim() > 1 else X.numel()
    if X.numel() < -(-n_assign // max(1, k)) * cols:
        raise ValueError("X is too small")
    if Xb is None:
        Xb = torch.empty((n_assign, cols), dtype=torch.float32, device=X.device)
    _check_dev(Xb, "Xb", torch.float32)
    if Xb.numel() < n_assign * cols:
        raise ValueError("Xb is too small")
    st = load_library().gq_moe_gather(_ptr(X), int(cols), int(k), _ptr(pos), int(n_assign), _ptr(Xb),
                                      _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_moe_gather")
    return Xb


def gq_moe_scatter(Yb, pos, w, k: int, out, stream=None):
    """out[t] += sum_j w[t k + j] * Yb[pos[t k + j]] over the placed slots, in
    slot order, each product and sum rounded in fp32 (Yb: [n_assign, rows],
    w: fp32 [n_assign], out: [n_assign / k, rows]). Asynchronous."""
    torch = _torch()
    _check_dev(Yb, "Yb", torch.float32)
    _check_dev(pos, "pos", torch.int32)
    _check_dev(w, "w", torch.float32)
    _check_dev(out, "out", torch.float32)
    n_assign = pos.numel()
    rows = Yb.shape[-1] if Yb.dim() > 1 else Yb.numel()
    if w.numel() < n_assign or Yb.numel() < n_assign * rows:
        raise ValueError("w or Yb is too small")
    if k > 0 and out.numel() < (n_assign // k) * rows:
        raise ValueError("out is too small")
    st = load_library().gq_moe_scatter(_ptr(Yb), int(rows), _ptr(pos), _ptr(w), int(n_assign), int(k),
                                       _ptr(out), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_moe_scatter")
    return out


def gq_matmul_experts_dev(fmt: int, W, n_expert: int, rows: int, cols: int, X, counts, Y=None,
                          stream=None):
    """gq_matmul_experts with the per-expert row counts in an int64 GPU
    tensor (gq_moe_bucket's counts): X [total, cols] bucketed by expert, Y
    [total, rows]; no host synchronisation. Asynchronous."""
    torch = _torch()
    _check_w(fmt, W, n_expert * rows, cols)
    _check_dev(X, "X", torch.float32)
    _check_dev(counts, "counts", torch.int64)
    if counts.numel() < n_expert:
        raise ValueError("counts must hold n_expert values")
    total = X.numel() // cols
    if Y is None:
        Y = torch.empty((total, rows), dtype=torch.float32, device=W.device)
    _check_dev(Y, "Y", torch.float32)
    if Y.numel() < total * rows:
        raise ValueError("Y is too small")
    st = load_library().gq_matmul_experts_dev(int(fmt), _ptr(W), int(n_expert), int(rows), int(cols), _ptr(X),
                                              _ptr(counts), int(total), _ptr(Y), _stream_handle(stream))
    if st != GQ_OK:
        raise GQError(st, "gq_matmul_experts_dev")
    return Y
