"""The C-ABI library loads, exports what include/gq.h declares, and rejects
bad arguments on the host before any HIP call (so these run without a GPU).
No compute call is made here."""
import ctypes
import os
import re

import pytest

import gguf_block_quant_gq_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            with open(os.path.join(ROOT, "include", h)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(gq_\w+)\s*\(", text, re.M)
    return sorted(set(names))


class _NoLaunch:
    """The library with every status-returning entry point wrapped: a call
    that returns GQ_ERR_DEVICE has passed every host check, so on a machine
    with a GPU it would have launched a kernel on the fake pointers these
    tests use. Every call here must be rejected before that point."""

    _PLAIN = {"gq_row_bytes", "gq_status_str"}

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        f = getattr(self._real, name)
        if name in self._PLAIN or not name.startswith("gq_"):
            return f

        def call(*args):
            st = f(*args)
            assert st != gq.GQ_ERR_DEVICE, f"{name}{args} passed every host check"
            return st
        return call


@pytest.fixture(scope="module")
def lib():
    return _NoLaunch(gq.load_library())


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"gq_dequant", "gq_matvec", "gq_matmul", "gq_row_bytes", "gq_status_str"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(gq.EXPORTS) == set(names)


def test_row_bytes(lib):
    assert gq.gq_row_bytes(8, 32) == 34
    assert gq.gq_row_bytes(8, 896) == 28 * 34
    assert gq.gq_row_bytes(8, 33) == 68
    assert gq.gq_row_bytes(12, 256) == 144
    assert gq.gq_row_bytes(12, 896) == 4 * 144
    assert gq.gq_row_bytes(12, 14336) == 56 * 144
    assert gq.gq_row_bytes(6, 896) == 28 * 22
    assert gq.gq_row_bytes(13, 896) == 4 * 176
    assert gq.gq_row_bytes(14, 4096) == 16 * 210
    assert gq.gq_row_bytes(7, 256) < 0
    assert gq.gq_row_bytes(8, -1) < 0


def test_row_bytes_matches_oracle(oracle):
    for fmt in (6, 8, 12, 13, 14):
        for cols in (1, 31, 32, 33, 255, 256, 257, 896, 4096, 4864, 14336):
            assert gq.gq_row_bytes(fmt, cols) == oracle.row_bytes(fmt, cols)


def test_status_strings(lib):
    for s in range(7):
        assert gq.status_str(s).startswith("GQ_")
    assert "unknown" in gq.status_str(99)


W_OK = 0x10000        # fake, never dereferenced: validation fails first
X_OK = 0x20000
Y_OK = 0x30000


def _mv(lib, fmt=12, W=W_OK, rows=4, cols=256, x=X_OK, y=Y_OK):
    return lib.gq_matvec(fmt, W, rows, cols, x, y, None)


def _mva(lib, fmt=12, W=W_OK, rows=4, cols=256, x=X_OK, y=Y_OK):
    return lib.gq_matvec_acc(fmt, W, rows, cols, x, y, None)


def _mvs(lib, fmt=12, W=W_OK, rows=4, cols=256, x=X_OK, y=Y_OK):
    return lib.gq_matvec_swiglu(fmt, W, rows, cols, x, y, None)


def _mm(lib, fmt=12, W=W_OK, rows=4, cols=256, X=X_OK, M=2, Y=Y_OK):
    return lib.gq_matmul(fmt, W, rows, cols, X, M, Y, None)


def _mb(lib, fmt=12, W=W_OK, rows=4, cols=256, X=X_OK, M=2, Y=Y_OK):
    return lib.gq_matvec_batch(fmt, W, rows, cols, X, M, Y, None)


def _dq(lib, fmt=12, W=W_OK, rows=4, cols=256, out=Y_OK):
    return lib.gq_dequant(fmt, W, rows, cols, out)


@pytest.mark.parametrize("call", [_mv, _mva, _mvs, _mm, _mb, _dq])
def test_validation_before_any_device_call(lib, call):
    for bad in (0, 7, 10, 11, 15, -1):   # Q5_1, Q2_K, Q3_K, IQ... have no kernels
        assert call(lib, fmt=bad) == gq.GQ_ERR_FMT
    assert call(lib, rows=-1) == gq.GQ_ERR_SHAPE
    assert call(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert call(lib, cols=-5) == gq.GQ_ERR_SHAPE
    assert call(lib, rows=1 << 40) == gq.GQ_ERR_SHAPE
    assert call(lib, W=None) == gq.GQ_ERR_NULL
    assert call(lib, W=W_OK + 2) == gq.GQ_ERR_ALIGN        # Q4_K needs 4-byte W
    assert call(lib, fmt=8, W=W_OK + 1) == gq.GQ_ERR_ALIGN  # Q8_0 needs 2-byte W
    assert call(lib, fmt=6, W=W_OK + 1) == gq.GQ_ERR_ALIGN  # Q5_0 likewise
    assert call(lib, fmt=14, W=W_OK + 1) == gq.GQ_ERR_ALIGN  # Q6_K likewise
    assert call(lib, fmt=13, W=W_OK + 2) == gq.GQ_ERR_ALIGN  # Q5_K needs 4-byte W
    # empty products succeed without touching anything
    assert call(lib, rows=0, W=None) == gq.GQ_OK


def test_validation_size_bound(lib):
    # rows, cols and M are at most 2^30: one more is rejected before any
    # pointer is looked at; at the bound the NULL check comes next
    big = 1 << 30
    assert _mv(lib, rows=big + 1) == gq.GQ_ERR_SHAPE
    assert _mv(lib, rows=big, W=None) == gq.GQ_ERR_NULL
    assert _mv(lib, fmt=8, cols=big + 1) == gq.GQ_ERR_SHAPE
    assert _mv(lib, fmt=8, cols=big, W=None) == gq.GQ_ERR_NULL
    assert _mm(lib, M=big + 1) == gq.GQ_ERR_SHAPE
    assert _mm(lib, M=big, X=None) == gq.GQ_ERR_NULL
    assert _mvs(lib, rows=big // 2 + 1) == gq.GQ_ERR_SHAPE      # 2 * rows weight rows
    assert _dq(lib, rows=big + 1) == gq.GQ_ERR_SHAPE


def test_validation_vectors(lib):
    assert _mv(lib, x=None) == gq.GQ_ERR_NULL
    assert _mv(lib, y=None) == gq.GQ_ERR_NULL
    assert _mv(lib, x=X_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mv(lib, y=Y_OK + 1) == gq.GQ_ERR_ALIGN
    assert _mv(lib, y=W_OK) == gq.GQ_ERR_OVERLAP
    assert _mv(lib, y=X_OK + 4) == gq.GQ_ERR_OVERLAP
    assert _mm(lib, M=-1) == gq.GQ_ERR_SHAPE
    assert _mm(lib, M=0, X=None) == gq.GQ_OK
    assert _mm(lib, X=None) == gq.GQ_ERR_NULL
    assert _mm(lib, Y=None) == gq.GQ_ERR_NULL
    assert _mm(lib, Y=X_OK) == gq.GQ_ERR_OVERLAP
    assert _dq(lib, out=None) == gq.GQ_ERR_NULL
    assert _dq(lib, out=W_OK) == gq.GQ_ERR_OVERLAP
    assert _dq(lib, out=Y_OK + 2) == gq.GQ_ERR_ALIGN
    # a Q8_0 row range may start on any 34-byte block, i.e. a 2-byte boundary
    # (the alignment check passes, the overlap check after it fires)
    assert _mv(lib, fmt=8, W=W_OK + 34, y=W_OK + 40) == gq.GQ_ERR_OVERLAP
    # the gate|up epilogue reads 2 * rows weight rows: an output placed just
    # past rows * row_bytes still overlaps W; 2^30 rows overflow the row index
    assert _mvs(lib, rows=4, y=W_OK + 4 * 144) == gq.GQ_ERR_OVERLAP
    assert _mv(lib, rows=4, y=W_OK + 4 * 144 - 4) == gq.GQ_ERR_OVERLAP
    assert _mvs(lib, rows=1 << 30) == gq.GQ_ERR_SHAPE
    assert _mva(lib, y=None) == gq.GQ_ERR_NULL
    assert _mva(lib, y=W_OK + 8) == gq.GQ_ERR_OVERLAP
    # likewise Q5_0 (22-byte blocks) and Q6_K (210-byte super-blocks)
    assert _mv(lib, fmt=6, W=W_OK + 22, y=W_OK + 24) == gq.GQ_ERR_OVERLAP
    assert _mv(lib, fmt=14, W=W_OK + 210, y=W_OK + 212) == gq.GQ_ERR_OVERLAP


def test_validation_batch(lib):
    assert _mb(lib, M=-1) == gq.GQ_ERR_SHAPE
    assert _mb(lib, M=2 ** 30 + 1) == gq.GQ_ERR_SHAPE    # past the 2^30 size bound
    assert _mb(lib, M=2 ** 30, Y=None) == gq.GQ_ERR_NULL
    assert _mb(lib, M=65536, Y=None) == gq.GQ_ERR_NULL
    assert _mb(lib, M=0, X=None, Y=None) == gq.GQ_OK
    assert _mb(lib, X=None) == gq.GQ_ERR_NULL
    assert _mb(lib, Y=None) == gq.GQ_ERR_NULL
    assert _mb(lib, X=X_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mb(lib, Y=Y_OK + 1) == gq.GQ_ERR_ALIGN
    # Y is [M, rows]: the second output row overlapping X's second row
    assert _mb(lib, Y=X_OK + 256 * 4 + 4) == gq.GQ_ERR_OVERLAP
    assert _mb(lib, Y=W_OK + 4 * 144 - 4) == gq.GQ_ERR_OVERLAP


def test_validation_q4k_matrix_core_bounds(lib):
    """The Q4_K fp16 matrix-core kernel addresses its tiles with 31-bit buffer
    offsets (64 activation rows, 256 weight rows): wider rows are rejected on
    the host, before any device call (so this runs without a GPU)."""
    big = 1 << 23                       # 64 * 4 * cols == 2^31
    far = 1 << 40                       # X, Y far apart: no overlap with W
    # M = 16 with these widths is past the batched matvec's work bound
    assert _mm(lib, rows=16, cols=big, M=16, X=far, Y=2 * far) == gq.GQ_ERR_SHAPE
    assert _mm(lib, rows=16, cols=big + 256, M=64, X=far, Y=2 * far) == gq.GQ_ERR_SHAPE
    assert _mge(lib, counts=(16, 0, 20), rows=16, cols=big, X=far, Y=2 * far) == gq.GQ_ERR_SHAPE
    # (calls that pass validation are not made here: with a GPU present they
    # would launch on these fake pointers)


def _mge(lib, counts=(2, 0, 3), fmt=12, W=W_OK, rows=4, cols=256, X=X_OK, Y=Y_OK, n_expert=None):
    import ctypes
    arr = (ctypes.c_int64 * max(1, len(counts)))(*counts) if counts is not None else None
    n = n_expert if n_expert is not None else len(counts)
    return lib.gq_matmul_experts(fmt, W, n, rows, cols, X, arr, Y, None)


def test_validation_grouped_experts(lib):
    for bad in (0, 7, 15):
        assert _mge(lib, fmt=bad) == gq.GQ_ERR_FMT
    assert _mge(lib, n_expert=-1) == gq.GQ_ERR_SHAPE
    assert _mge(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert _mge(lib, counts=(2, -1, 3)) == gq.GQ_ERR_SHAPE        # every count checked first
    assert _mge(lib, counts=(1 << 62, 1 << 62)) == gq.GQ_ERR_SHAPE
    # every count an int, but more than 2^30 activation rows in all
    assert _mge(lib, counts=(1 << 29, (1 << 29) + 1)) == gq.GQ_ERR_SHAPE
    assert _mge(lib, counts=None, n_expert=3) == gq.GQ_ERR_NULL
    assert _mge(lib, counts=(), W=None, X=None, Y=None) == gq.GQ_OK   # no experts
    assert _mge(lib, counts=(0, 0), W=None, X=None, Y=None) == gq.GQ_OK  # no rows
    assert _mge(lib, rows=0, W=None) == gq.GQ_OK
    assert _mge(lib, X=None) == gq.GQ_ERR_NULL
    assert _mge(lib, Y=None) == gq.GQ_ERR_NULL
    assert _mge(lib, W=W_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mge(lib, X=X_OK + 2) == gq.GQ_ERR_ALIGN
    # Y is [5, rows]: overlapping X's last row, or the last expert's weights
    assert _mge(lib, Y=X_OK + 4 * 256 * 4) == gq.GQ_ERR_OVERLAP
    assert _mge(lib, Y=W_OK + 3 * 4 * 144 - 4) == gq.GQ_ERR_OVERLAP


def _mx(lib, fmt=12, W=W_OK, n_expert=4, rows=4, cols=256, X=X_OK, xk=2, expid=0x40000,
        n_assign=8, Y=Y_OK):
    return lib.gq_matvec_experts(fmt, W, n_expert, rows, cols, X, xk, expid, n_assign, Y, None)


def test_validation_experts(lib):
    for bad in (0, 7, 15):
        assert _mx(lib, fmt=bad) == gq.GQ_ERR_FMT
    assert _mx(lib, n_expert=0) == gq.GQ_ERR_SHAPE
    assert _mx(lib, xk=0) == gq.GQ_ERR_SHAPE
    assert _mx(lib, n_assign=-1) == gq.GQ_ERR_SHAPE
    assert _mx(lib, n_assign=2 ** 30 + 1) == gq.GQ_ERR_SHAPE
    assert _mx(lib, n_assign=65536, Y=None) == gq.GQ_ERR_NULL
    # X rows times cols overflowing 64 bits
    assert _mx(lib, n_assign=2 ** 30, xk=1, cols=2 ** 30 + 1, rows=1) == gq.GQ_ERR_SHAPE
    assert _mx(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert _mx(lib, n_assign=0, W=None, expid=None) == gq.GQ_OK
    assert _mx(lib, rows=0, W=None) == gq.GQ_OK
    assert _mx(lib, expid=None) == gq.GQ_ERR_NULL
    assert _mx(lib, X=None) == gq.GQ_ERR_NULL
    assert _mx(lib, W=W_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mx(lib, expid=0x40002) == gq.GQ_ERR_ALIGN
    # Y overlapping the expert ids, or the last expert's weights
    assert _mx(lib, expid=Y_OK + 16) == gq.GQ_ERR_OVERLAP
    assert _mx(lib, Y=W_OK + 4 * 4 * 144 - 4) == gq.GQ_ERR_OVERLAP


def _bk(lib, expid=0x40000, n_assign=8, n_expert=4, counts=0x50000, order=0x60000, pos=0x70000):
    return lib.gq_moe_bucket(expid, n_assign, n_expert, counts, order, pos, None)


def _ga(lib, X=X_OK, cols=64, k=2, pos=0x70000, n_assign=8, Xb=0x80000):
    return lib.gq_moe_gather(X, cols, k, pos, n_assign, Xb, None)


def _sc(lib, Yb=0x80000, rows=64, pos=0x70000, w=0x60000, n_assign=8, k=2, out=Y_OK):
    return lib.gq_moe_scatter(Yb, rows, pos, w, n_assign, k, out, None)


def test_validation_moe_bucket_gather_scatter(lib):
    assert _bk(lib, n_expert=0) == gq.GQ_ERR_SHAPE
    assert _bk(lib, n_expert=1025) == gq.GQ_ERR_SHAPE
    assert _bk(lib, n_assign=-1) == gq.GQ_ERR_SHAPE
    assert _bk(lib, n_assign=2 ** 30 + 1) == gq.GQ_ERR_SHAPE
    assert _bk(lib, counts=None) == gq.GQ_ERR_NULL
    assert _bk(lib, expid=None) == gq.GQ_ERR_NULL
    assert _bk(lib, order=None) == gq.GQ_ERR_NULL
    assert _bk(lib, pos=None) == gq.GQ_ERR_NULL
    assert _bk(lib, counts=0x50004) == gq.GQ_ERR_ALIGN
    assert _bk(lib, pos=0x70002) == gq.GQ_ERR_ALIGN
    assert _bk(lib, order=0x70000 + 16) == gq.GQ_ERR_OVERLAP
    assert _bk(lib, counts=0x40000 + 8) == gq.GQ_ERR_OVERLAP

    assert _ga(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert _ga(lib, k=0) == gq.GQ_ERR_SHAPE
    assert _ga(lib, n_assign=-1) == gq.GQ_ERR_SHAPE
    assert _ga(lib, cols=2 ** 30 + 1) == gq.GQ_ERR_SHAPE
    assert _ga(lib, n_assign=0, X=None, pos=None, Xb=None) == gq.GQ_OK
    assert _ga(lib, X=None) == gq.GQ_ERR_NULL
    assert _ga(lib, Xb=None) == gq.GQ_ERR_NULL
    assert _ga(lib, X=X_OK + 2) == gq.GQ_ERR_ALIGN
    assert _ga(lib, Xb=X_OK + 64) == gq.GQ_ERR_OVERLAP      # Xb over X
    assert _ga(lib, Xb=0x70000 - 64) == gq.GQ_ERR_OVERLAP   # Xb over pos

    assert _sc(lib, rows=-1) == gq.GQ_ERR_SHAPE
    assert _sc(lib, k=0) == gq.GQ_ERR_SHAPE
    assert _sc(lib, n_assign=7) == gq.GQ_ERR_SHAPE           # not a multiple of k
    assert _sc(lib, rows=2 ** 30 + 1) == gq.GQ_ERR_SHAPE
    assert _sc(lib, rows=0, Yb=None) == gq.GQ_OK
    assert _sc(lib, n_assign=0, Yb=None, pos=None, w=None, out=None) == gq.GQ_OK
    assert _sc(lib, w=None) == gq.GQ_ERR_NULL
    assert _sc(lib, out=None) == gq.GQ_ERR_NULL
    assert _sc(lib, w=0x60002) == gq.GQ_ERR_ALIGN
    assert _sc(lib, out=0x80000 + 4) == gq.GQ_ERR_OVERLAP    # out over Yb
    assert _sc(lib, out=0x60000 - 16) == gq.GQ_ERR_OVERLAP   # out over w


def _gd(lib, fmt=12, W=W_OK, n_expert=4, rows=4, cols=256, X=X_OK, m=0x90000, total=8, Y=Y_OK):
    return lib.gq_matmul_experts_dev(fmt, W, n_expert, rows, cols, X, m, total, Y, None)


def test_validation_grouped_device_counts(lib):
    assert _gd(lib, fmt=7) == gq.GQ_ERR_FMT
    assert _gd(lib, n_expert=0) == gq.GQ_ERR_SHAPE
    assert _gd(lib, n_expert=1025) == gq.GQ_ERR_SHAPE
    assert _gd(lib, total=-1) == gq.GQ_ERR_SHAPE
    assert _gd(lib, total=2 ** 30 + 1) == gq.GQ_ERR_SHAPE
    assert _gd(lib, cols=258) == gq.GQ_ERR_SHAPE            # not a multiple of 4
    assert _gd(lib, fmt=8, cols=96) == gq.GQ_ERR_SHAPE      # Q8_0 rows of 3 blocks: not whole dwords
    assert _gd(lib, fmt=14, cols=768) == gq.GQ_ERR_SHAPE    # Q6_K rows of 3 super-blocks
    assert _gd(lib, total=0, W=None, X=None, m=None, Y=None) == gq.GQ_OK
    assert _gd(lib, rows=0, W=None) == gq.GQ_OK
    assert _gd(lib, m=None) == gq.GQ_ERR_NULL
    assert _gd(lib, W=None) == gq.GQ_ERR_NULL
    assert _gd(lib, m=0x90004) == gq.GQ_ERR_ALIGN
    assert _gd(lib, fmt=8, cols=128, W=W_OK + 2) == gq.GQ_ERR_ALIGN   # dword rows need a 4-byte W
    assert _gd(lib, Y=X_OK + 64) == gq.GQ_ERR_OVERLAP
    assert _gd(lib, m=Y_OK + 8) == gq.GQ_ERR_OVERLAP


def test_split_layout_row_bytes_and_repack_validation(lib, oracle):
    for cols in (1, 31, 32, 33, 896, 4096, 14336):
        assert gq.gq_row_bytes(1008, cols) == oracle.row_bytes(1008, cols)
    rp = lib.gq_q8_0_split_repack
    # a 2-byte aligned W passes the alignment check (the overlap check after
    # it fires; no call here passes every check, so none would launch)
    assert rp(W_OK + 2, 4, 896, W_OK + 12, None) == gq.GQ_ERR_OVERLAP
    assert rp(W_OK + 1, 4, 896, Y_OK, None) == gq.GQ_ERR_ALIGN       # W: 2-byte aligned
    assert rp(W_OK, 4, 896, Y_OK + 2, None) == gq.GQ_ERR_ALIGN       # out: 4-byte aligned
    assert rp(None, 4, 896, Y_OK, None) == gq.GQ_ERR_NULL
    assert rp(W_OK, -1, 896, Y_OK, None) == gq.GQ_ERR_SHAPE
    assert rp(W_OK, 0, 896, None, None) == gq.GQ_OK
    assert rp(W_OK, 4, 896, W_OK + 8, None) == gq.GQ_ERR_OVERLAP
    # the split layout needs 4-byte aligned W in every entry point
    assert _mv(lib, fmt=1008, W=W_OK + 2) == gq.GQ_ERR_ALIGN


def _q81(lib, x=X_OK, n=2, cols=256, xq=Y_OK):
    return lib.gq_quantize_q8_1(x, n, cols, xq, None)


def _mvq(lib, fmt=12, W=W_OK, rows=4, cols=256, xq=X_OK, y=Y_OK):
    return lib.gq_matvec_q8_1(fmt, W, rows, cols, xq, y, None)


def test_validation_int8_activation_path(lib):
    assert lib.gq_row_bytes(gq.GQ_FMT_Q8_1, 33) == 72
    # Q8_1 is an activation format: no weight entry point takes it
    assert _mv(lib, fmt=gq.GQ_FMT_Q8_1) == gq.GQ_ERR_FMT
    assert _mm(lib, fmt=gq.GQ_FMT_Q8_1) == gq.GQ_ERR_FMT
    assert _dq(lib, fmt=gq.GQ_FMT_Q8_1) == gq.GQ_ERR_FMT
    assert _mvq(lib, fmt=gq.GQ_FMT_Q8_1) == gq.GQ_ERR_FMT
    for fmt in (6, 13, 14, 1008, 0):   # formats without an integer-dot kernel
        assert _mvq(lib, fmt=fmt) == gq.GQ_ERR_FMT
    assert _mvq(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert _mvq(lib, rows=-1) == gq.GQ_ERR_SHAPE
    assert _mvq(lib, cols=131072 + 256) == gq.GQ_ERR_SHAPE    # the row is staged in LDS
    assert _mvq(lib, rows=0, W=None, xq=None, y=None) == gq.GQ_OK
    assert _mvq(lib, W=None) == gq.GQ_ERR_NULL
    assert _mvq(lib, xq=None) == gq.GQ_ERR_NULL
    assert _mvq(lib, y=None) == gq.GQ_ERR_NULL
    assert _mvq(lib, W=W_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mvq(lib, xq=X_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mvq(lib, y=Y_OK + 2) == gq.GQ_ERR_ALIGN
    assert _mvq(lib, y=X_OK + 4) == gq.GQ_ERR_OVERLAP        # y over the quantised row
    assert _mvq(lib, y=W_OK + 100) == gq.GQ_ERR_OVERLAP      # y over W
    assert _q81(lib, n=-1) == gq.GQ_ERR_SHAPE
    assert _q81(lib, cols=0) == gq.GQ_ERR_SHAPE
    assert _q81(lib, n=0, x=None, xq=None) == gq.GQ_OK
    assert _q81(lib, x=None) == gq.GQ_ERR_NULL
    assert _q81(lib, xq=None) == gq.GQ_ERR_NULL
    assert _q81(lib, x=X_OK + 2) == gq.GQ_ERR_ALIGN
    assert _q81(lib, xq=Y_OK + 1) == gq.GQ_ERR_ALIGN
    assert _q81(lib, xq=X_OK + 1024) == gq.GQ_ERR_OVERLAP    # output over the second row of x


def test_validation_matmul_modes(lib):
    for name in ("gq_matmul_acc", "gq_matmul_swiglu"):
        fn = getattr(lib, name)
        call = lambda fmt=12, W=W_OK, rows=4, cols=256, X=X_OK, M=2, Y=Y_OK: fn(fmt, W, rows, cols, X, M, Y, None)
        assert call(fmt=7) == gq.GQ_ERR_FMT
        assert call(fmt=gq.GQ_FMT_Q8_1) == gq.GQ_ERR_FMT
        assert call(rows=-1) == gq.GQ_ERR_SHAPE
        assert call(cols=0) == gq.GQ_ERR_SHAPE
        assert call(M=-1) == gq.GQ_ERR_SHAPE
        assert call(rows=0, W=None, X=None, Y=None) == gq.GQ_OK
        assert call(M=0, W=None, X=None, Y=None) == gq.GQ_OK
        assert call(W=None) == gq.GQ_ERR_NULL
        assert call(W=W_OK + 2) == gq.GQ_ERR_ALIGN
        assert call(Y=X_OK + 256 * 4) == gq.GQ_ERR_OVERLAP
    # the SwiGLU form reads 2 * rows weight rows: Y over the up half overlaps
    assert lib.gq_matmul_swiglu(12, W_OK, 4, 256, X_OK, 2, W_OK + 6 * 144, None) == gq.GQ_ERR_OVERLAP
    # the Q4_K matrix-core bound holds per half
    far = 1 << 40
    assert lib.gq_matmul_swiglu(12, W_OK, 16, 1 << 23, far, 16, 2 * far, None) == gq.GQ_ERR_SHAPE


def test_c_client_compiles_as_c11():
    """The header and the C client compile as strict C11 with gcc (the client
    itself runs on the GPU in test_gpu_c_client.py)."""
    import subprocess
    src = os.path.join(ROOT, "tests", "c_client.c")
    r = subprocess.run(["gcc", "-std=c11", "-fsyntax-only", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        f"-I{os.path.join(ROOT, 'include')}", src],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
