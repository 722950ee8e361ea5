// gq_api.hip -- the extern "C" entry points of libgq (declared in gq.h):
// argument validation on the host, kernel choice, launch.
//
// The dispatch mirrors the quantised matvec dispatch of "nurllama 0.18.1
// API" (kernels.nu section): the ggml tensor type picks the kernel, and a
// type without a kernel is reported to the caller (GQ_ERR_FMT) so that it
// can fall back. Every check runs before the first HIP call.
#include <atomic>
#include <climits>
#include <cstdint>

#include "../../include/gq.h"
#include "gq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device (cached per device).
int current_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev >= kMaxDevices) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    return n;
  }
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Rows, columns, activation rows, batch rows and assignments are at most
// 2^30: the kernels index them with 32-bit ints, and every index they form
// (an index plus a grid stride, a row plus a tile, a unit count times 32)
// then stays below 2^31.
constexpr int64_t kMaxDim = int64_t(1) << 30;

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Shape and format checks shared by every entry point. On success *rb is
// the row stride in bytes and *wbytes the size of W.
int check_shape(int fmt, int64_t rows, int64_t cols, int64_t M, int64_t* rb, int64_t* wbytes) {
  if (gq_row_bytes(fmt, 1) < 0 || fmt == GQ_FMT_Q8_1) return GQ_ERR_FMT;  // Q8_1: activations only
  if (rows < 0 || cols <= 0 || M < 0) return GQ_ERR_SHAPE;
  if (rows > kMaxDim || cols > kMaxDim || M > kMaxDim) return GQ_ERR_SHAPE;
  *rb = gq_row_bytes(fmt, cols);
  if (*rb <= 0) return GQ_ERR_SHAPE;
  if (rows > 0 && *rb > INT64_MAX / rows) return GQ_ERR_SHAPE;
  *wbytes = rows * *rb;
  return GQ_OK;
}

// Formats whose block size is not a multiple of 4 bytes (Q8_0 34, Q5_0 22,
// Q6_K 210) take 2-byte aligned W, so that a row range starting at any
// block boundary is accepted; Q4_K and Q5_K blocks (144, 176 B) and the
// split Q8_0 layout (rows of whole 16-byte chunks) take 4.
int check_align(int fmt, const void* W) {
  const bool two = fmt == GQ_FMT_Q8_0 || fmt == GQ_FMT_Q5_0 || fmt == GQ_FMT_Q6_K;
  const uintptr_t need = two ? 2 : 4;
  return ((uintptr_t)W % need) ? GQ_ERR_ALIGN : GQ_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? GQ_OK : GQ_ERR_DEVICE; }

// Activation rows from which the Q8_0 / Q5_0 / Q5_K / Q6_K products run on
// the matrix cores (gemm_f32.hip; Q8_0 rows the fp16 kernels take go there)
// instead of the fp32 few-row kernel (measured: K-quants are faster there
// from M = 2 on; Q8_0 at M = 4 is still faster on the few-row kernel, 21 vs
// 31 us for 4096 x 4096 on the fp32 matrix cores, 27 vs 37 us for the
// 14336 x 4096 gate on the fp16 ones, and 2.8x slower at M = 16).
#ifndef GQ_F32_MIN_M_KQUANT
#define GQ_F32_MIN_M_KQUANT 2
#endif
#ifndef GQ_F32_MIN_M_BLOCK32
#define GQ_F32_MIN_M_BLOCK32 8
#endif
// Products of a few activation rows (M < 16) with M * rows * cols at most
// this many weight-rows run as the batched matvec.
#ifndef GQ_BATCH_MAX_WORK
#define GQ_BATCH_MAX_WORK (int64_t(1) << 28)
#endif
constexpr int64_t kBatchMaxWork = GQ_BATCH_MAX_WORK;

int64_t f32_matrix_core_min_m(int fmt) {
  if (fmt == GQ_FMT_Q8_0_SPLIT) return 2;  // the few-row kernel has no split-layout unit
  return (fmt == GQ_FMT_Q5_K || fmt == GQ_FMT_Q6_K) ? GQ_F32_MIN_M_KQUANT : GQ_F32_MIN_M_BLOCK32;
}

}  // namespace

extern "C" int64_t gq_row_bytes(int fmt, int64_t cols) {
  if (cols < 0 || cols > INT64_MAX - 256) return -1;
  switch (fmt) {
    case GQ_FMT_Q8_0: return ((cols + 31) / 32) * 34;
    case GQ_FMT_Q5_0: return ((cols + 31) / 32) * 22;
    case GQ_FMT_Q4_K: return ((cols + 255) / 256) * 144;
    case GQ_FMT_Q5_K: return ((cols + 255) / 256) * 176;
    case GQ_FMT_Q6_K: return ((cols + 255) / 256) * 210;
    case GQ_FMT_Q8_0_SPLIT: {
      const int64_t nb = (cols + 31) / 32;
      return ((2 * nb + 15) / 16) * 16 + 32 * nb;
    }
    case GQ_FMT_Q8_1: return ((cols + 31) / 32) * 36;
    default: return -1;
  }
}

extern "C" const char* gq_status_str(int status) {
  switch (status) {
    case GQ_OK: return "GQ_OK";
    case GQ_ERR_NULL: return "GQ_ERR_NULL: a required pointer is NULL";
    case GQ_ERR_FMT: return "GQ_ERR_FMT: unsupported block format";
    case GQ_ERR_SHAPE: return "GQ_ERR_SHAPE: bad or overflowing rows/cols/M";
    case GQ_ERR_ALIGN: return "GQ_ERR_ALIGN: misaligned pointer";
    case GQ_ERR_DEVICE: return "GQ_ERR_DEVICE: HIP runtime error";
    case GQ_ERR_OVERLAP: return "GQ_ERR_OVERLAP: output overlaps an input";
    default: return "unknown gq status";
  }
}

extern "C" int gq_dequant(int fmt, const void* W, int64_t rows, int64_t cols, float* out) {
  int64_t rb = 0, wbytes = 0;
  int st = check_shape(fmt, rows, cols, 0, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if (rows > INT64_MAX / 4 / cols) return GQ_ERR_SHAPE;
  if (rows == 0) return GQ_OK;
  if (!W || !out) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)out % 4) return GQ_ERR_ALIGN;
  if (overlaps(out, rows * cols * 4, W, wbytes)) return GQ_ERR_OVERLAP;

  (void)hipGetLastError();  // start from a clean error state
  gq::DequantArgs a{(const uint8_t*)W, out, rb, rows, (int)cols, 0};
  hipError_t e = gq::launch_dequant(fmt, a, 0);
  if (e != hipSuccess) return GQ_ERR_DEVICE;
  return finish(hipStreamSynchronize(0));
}

namespace {

// Shared by the three matvec entry points: validation, then one launch. The
// gate|up epilogue reads 2 * rows weight rows and writes rows outputs.
int matvec_common(int fmt, const void* W, int64_t rows, int64_t cols, const float* x, float* y,
                  void* stream, int epi) {
  const int64_t wmul = epi == gq::kEpiSwiglu ? 2 : 1;
  if (rows > kMaxDim / wmul) return GQ_ERR_SHAPE;
  int64_t rb = 0, wbytes = 0;
  int st = check_shape(fmt, rows * wmul, cols, 1, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if (rows == 0) return GQ_OK;
  if (!W || !x || !y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)x % 4 || (uintptr_t)y % 4) return GQ_ERR_ALIGN;
  if (overlaps(y, rows * 4, W, wbytes) || overlaps(y, rows * 4, x, cols * 4)) return GQ_ERR_OVERLAP;

  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  gq::GemvArgs a{(const uint8_t*)W, x, y, rb, (int)rows, (int)cols, 0};
  return finish(gq::launch_gemv(fmt, a, cus, (hipStream_t)stream, epi));
}

}  // namespace

extern "C" int gq_matvec(int fmt, const void* W, int64_t rows, int64_t cols, const float* x,
                         float* y, void* stream) {
  return matvec_common(fmt, W, rows, cols, x, y, stream, gq::kEpiStore);
}

extern "C" int gq_matvec_acc(int fmt, const void* W, int64_t rows, int64_t cols, const float* x,
                             float* y, void* stream) {
  return matvec_common(fmt, W, rows, cols, x, y, stream, gq::kEpiAcc);
}

extern "C" int gq_matvec_swiglu(int fmt, const void* W, int64_t rows, int64_t cols,
                                const float* x, float* y, void* stream) {
  return matvec_common(fmt, W, rows, cols, x, y, stream, gq::kEpiSwiglu);
}

extern "C" int gq_matvec_experts(int fmt, const void* W, int64_t n_expert, int64_t rows,
                                 int64_t cols, const float* X, int64_t xk, const int32_t* expid,
                                 int64_t n_assign, float* Y, void* stream) {
  int64_t rb = 0, ebytes = 0;
  int st = check_shape(fmt, rows, cols, 1, &rb, &ebytes);
  if (st != GQ_OK) return st;
  // the assignments are the grid's second dimension (an int index)
  if (n_expert < 1 || n_expert > INT_MAX || xk < 1 || xk > INT_MAX || n_assign < 0 ||
      n_assign > kMaxDim)
    return GQ_ERR_SHAPE;
  if (rows == 0 || n_assign == 0) return GQ_OK;
  if (ebytes > INT64_MAX / n_expert) return GQ_ERR_SHAPE;
  const int64_t wbytes = ebytes * n_expert;
  const int64_t xrows = (n_assign + xk - 1) / xk;
  if (rows > INT64_MAX / 4 / n_assign || cols > INT64_MAX / 4 / xrows) return GQ_ERR_SHAPE;
  const int64_t xbytes = xrows * cols * 4, ybytes = n_assign * rows * 4;
  if (!W || !X || !expid || !Y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)X % 4 || (uintptr_t)Y % 4 || (uintptr_t)expid % 4) return GQ_ERR_ALIGN;
  if (overlaps(Y, ybytes, W, wbytes) || overlaps(Y, ybytes, X, xbytes) ||
      overlaps(Y, ybytes, expid, n_assign * 4))
    return GQ_ERR_OVERLAP;

  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  gq::GemvArgs a{(const uint8_t*)W, X, Y, rb, (int)rows, (int)cols, 0};
  const gq::ExpertArgs ex{expid, ebytes, (int)n_expert, (int)xk, (int)n_assign};
  return finish(gq::launch_gemv(fmt, a, cus, (hipStream_t)stream, gq::kEpiStore, &ex));
}

namespace {

// Shared by gq_matvec_batch and the few-row routing of gq_matmul (arguments
// already checked): one launch of the matvec kernels over `batch` activation
// rows, each row a grid slice of its own.
int batch_launch(int fmt, const void* W, int64_t rb, int64_t rows, int64_t cols, const float* X,
                 int64_t batch, float* Y, void* stream, int cus) {
  gq::GemvArgs a{(const uint8_t*)W, X, Y, rb, (int)rows, (int)cols, 0};
  const gq::ExpertArgs ex{nullptr, 0, 1, 1, (int)batch};
  return finish(gq::launch_gemv(fmt, a, cus, (hipStream_t)stream, gq::kEpiStore, &ex));
}

}  // namespace

extern "C" int gq_matvec_batch(int fmt, const void* W, int64_t rows, int64_t cols,
                               const float* X, int64_t batch, float* Y, void* stream) {
  int64_t rb = 0, wbytes = 0;
  int st = check_shape(fmt, rows, cols, batch, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if (rows == 0 || batch == 0) return GQ_OK;
  if (rows > INT64_MAX / 4 / batch || cols > INT64_MAX / 4 / batch) return GQ_ERR_SHAPE;
  if (!W || !X || !Y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)X % 4 || (uintptr_t)Y % 4) return GQ_ERR_ALIGN;
  if (overlaps(Y, batch * rows * 4, W, wbytes) || overlaps(Y, batch * rows * 4, X, batch * cols * 4))
    return GQ_ERR_OVERLAP;
  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return batch_launch(fmt, W, rb, rows, cols, X, batch, Y, stream, cus);
}

extern "C" int gq_q8_0_split_repack(const void* W, int64_t rows, int64_t cols, void* out,
                                    void* stream) {
  int64_t rb = 0, wbytes = 0, orb = 0, obytes = 0;
  int st = check_shape(GQ_FMT_Q8_0, rows, cols, 1, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if ((st = check_shape(GQ_FMT_Q8_0_SPLIT, rows, cols, 1, &orb, &obytes)) != GQ_OK) return st;
  if (rows == 0) return GQ_OK;
  if (!W || !out) return GQ_ERR_NULL;
  if ((st = check_align(GQ_FMT_Q8_0, W)) != GQ_OK) return st;
  if ((st = check_align(GQ_FMT_Q8_0_SPLIT, out)) != GQ_OK) return st;
  if (overlaps(out, obytes, W, wbytes)) return GQ_ERR_OVERLAP;
  (void)hipGetLastError();
  return finish(gq::launch_q8_0_split_repack((const uint8_t*)W, rows, (int)cols, rb, (uint8_t*)out,
                                             orb, (hipStream_t)stream));
}

namespace {

// The three output modes of the prefill product.
enum MatmulMode { kModeStore = 0, kModeAcc = 1, kModeSwiglu = 2 };

// The layouts the fp16 matrix-core kernels take: Q4_K, Q5_K and split Q8_0
// rows that are whole groups of four floats, and Q8_0, Q5_0 and Q6_K ones
// whose rows are also a whole number of dwords from a dword-aligned W (their
// loads are dword loads).
bool f16_layout(int fmt, int64_t cols, int64_t rb, const void* W) {
  if (cols % 4 != 0) return false;
  if (fmt == GQ_FMT_Q4_K || fmt == GQ_FMT_Q5_K || fmt == GQ_FMT_Q8_0_SPLIT) return true;
  const bool dword_rows = rb % 4 == 0 && (uintptr_t)W % 4 == 0;
  return (fmt == GQ_FMT_Q8_0 || fmt == GQ_FMT_Q5_0 || fmt == GQ_FMT_Q6_K) && dword_rows;
}

bool batched_matvec(int64_t M, int64_t rows, int64_t cols) {
  return M > 1 && M < 16 && rows * cols <= kBatchMaxWork / M;
}

// Whether a product of M activation rows past the batched-matvec bound runs
// on the fp16 matrix cores: every layout above, except that packed Q8_0 and
// Q5_0 with fewer rows than the matrix cores' threshold keep the few-row
// kernel for the stored form.
bool f16_route(int fmt, int64_t cols, int64_t rb, const void* W, int64_t M, int epi) {
  if (!f16_layout(fmt, cols, rb, W)) return false;
  const bool few_row_kernel = fmt == GQ_FMT_Q8_0 || fmt == GQ_FMT_Q5_0;
  return !few_row_kernel || M >= f32_matrix_core_min_m(fmt) || epi != gq::kMmStore;
}

// Whether the kernel that gq_matmul picks for this shape can address it
// (its tiles use 31-bit buffer offsets); checked before any HIP call.
bool matmul_addressable(int fmt, const void* W, int64_t rows, int64_t cols, int64_t M, int64_t rb,
                        int mode) {
  const int epi = mode == kModeStore ? gq::kMmStore : gq::kMmAcc;
  if (M > 1 && !batched_matvec(M, rows, cols) && f16_route(fmt, cols, rb, W, M, epi))
    return gq::gemm_f16_fits(rows, cols, rb);
  return true;
}

// One matrix-core product of the route for (fmt, cols, M) with a GEMM epilogue.
int matrix_product(int fmt, const uint8_t* W, int64_t rb, int64_t rows, int64_t cols, const float* X,
                   int64_t M, float* Y, hipStream_t s, int cus, int epi) {
  gq::GemmArgs a{W, X, Y, rb, (int)rows, (int)cols, (int)M, 0};
  if (f16_route(fmt, cols, rb, W, M, epi)) {
    const int64_t off = 0;
    return finish(gq::launch_gemm_f16(fmt, a, &M, &off, 1, 0, cus, s, epi));
  }
  // the few-row fp32 kernel stores only: the other modes take the fp32 matrix cores
  if (fmt == GQ_FMT_Q4_K || M >= f32_matrix_core_min_m(fmt) || epi != gq::kMmStore)
    return finish(gq::launch_gemm_f32(fmt, a, cus, s, epi));
  return finish(gq::launch_gemm_small(fmt, a, cus, s));
}

// gq_matmul (and its accumulate / SwiGLU forms) after the checks: the kernel
// route for M activation rows. One activation row is the matvec (same
// rounding, its kernel and epilogue). A few rows over a small enough product
// run as matvecs, so each row again rounds exactly as the matvec does (its
// cost grows with M * rows * cols: every row repeats the decode; measured
// faster than the matrix cores up to about 2^28 weight-rows for every
// format): one batched launch for the stored form, one launch per row for
// the others. Larger products of the layouts in f16_route run on the fp16
// matrix cores (exact operands), the others on the fp32 matrix cores from a
// per-format M, else on the fp32 few-row kernel. The SwiGLU form on the
// matrix cores is two launches: Y = W_up X, then Y = silu(W_gate X) * Y.
int matmul_route(int fmt, const void* W, int64_t rb, int64_t rows, int64_t cols, const float* X,
                 int64_t M, float* Y, void* stream, int cus, int mode = kModeStore) {
  const hipStream_t s = (hipStream_t)stream;
  const int gemv_epi = mode == kModeAcc ? gq::kEpiAcc : mode == kModeSwiglu ? gq::kEpiSwiglu : gq::kEpiStore;
  if (M == 1) {
    gq::GemvArgs v{(const uint8_t*)W, X, Y, rb, (int)rows, (int)cols, 0};
    return finish(gq::launch_gemv(fmt, v, cus, s, gemv_epi));
  }
  if (batched_matvec(M, rows, cols)) {
    if (mode == kModeStore) return batch_launch(fmt, W, rb, rows, cols, X, M, Y, stream, cus);
    for (int64_t m = 0; m < M; ++m) {
      gq::GemvArgs v{(const uint8_t*)W, X + m * cols, Y + m * rows, rb, (int)rows, (int)cols, 0};
      const int st = finish(gq::launch_gemv(fmt, v, cus, s, gemv_epi));
      if (st != GQ_OK) return st;
    }
    return GQ_OK;
  }
  const uint8_t* w = (const uint8_t*)W;
  if (mode == kModeSwiglu) {
    const int st = matrix_product(fmt, w + rows * rb, rb, rows, cols, X, M, Y, s, cus, gq::kMmStore);
    if (st != GQ_OK) return st;
    return matrix_product(fmt, w, rb, rows, cols, X, M, Y, s, cus, gq::kMmSiluMul);
  }
  return matrix_product(fmt, w, rb, rows, cols, X, M, Y, s, cus,
                        mode == kModeAcc ? gq::kMmAcc : gq::kMmStore);
}

// The checks and launch shared by gq_matmul, gq_matmul_acc and
// gq_matmul_swiglu (W holds 2 * rows weight rows for the SwiGLU form).
int matmul_entry(int fmt, const void* W, int64_t rows, int64_t cols, const float* X, int64_t M, float* Y,
                 void* stream, int mode) {
  int64_t rb = 0, wbytes = 0;
  const int64_t wrows = mode == kModeSwiglu ? 2 * rows : rows;
  if (rows > kMaxDim) return GQ_ERR_SHAPE;
  int st = check_shape(fmt, wrows, cols, M, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if (M > 0 && (rows > INT64_MAX / 4 / M || cols > INT64_MAX / 4 / M)) return GQ_ERR_SHAPE;
  if (rows == 0 || M == 0) return GQ_OK;
  if (!W || !X || !Y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)X % 4 || (uintptr_t)Y % 4) return GQ_ERR_ALIGN;
  if (overlaps(Y, M * rows * 4, W, wbytes) || overlaps(Y, M * rows * 4, X, M * cols * 4))
    return GQ_ERR_OVERLAP;
  if (!matmul_addressable(fmt, W, rows, cols, M, rb, mode)) return GQ_ERR_SHAPE;

  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return matmul_route(fmt, W, rb, rows, cols, X, M, Y, stream, cus, mode);
}

}  // namespace

extern "C" int gq_matmul(int fmt, const void* W, int64_t rows, int64_t cols, const float* X,
                         int64_t M, float* Y, void* stream) {
  return matmul_entry(fmt, W, rows, cols, X, M, Y, stream, kModeStore);
}

extern "C" int gq_matmul_acc(int fmt, const void* W, int64_t rows, int64_t cols, const float* X,
                             int64_t M, float* Y, void* stream) {
  return matmul_entry(fmt, W, rows, cols, X, M, Y, stream, kModeAcc);
}

extern "C" int gq_matmul_swiglu(int fmt, const void* W, int64_t rows, int64_t cols, const float* X,
                                int64_t M, float* Y, void* stream) {
  return matmul_entry(fmt, W, rows, cols, X, M, Y, stream, kModeSwiglu);
}

extern "C" int gq_matmul_experts(int fmt, const void* W, int64_t n_expert, int64_t rows,
                                 int64_t cols, const float* X, const int64_t* m_per_expert,
                                 float* Y, void* stream) {
  int64_t rb = 0, ebytes = 0;
  int st = check_shape(fmt, rows, cols, 1, &rb, &ebytes);
  if (st != GQ_OK) return st;
  if (n_expert < 0 || n_expert > INT_MAX) return GQ_ERR_SHAPE;
  if (n_expert == 0 || rows == 0) return GQ_OK;
  if (!m_per_expert) return GQ_ERR_NULL;
  // total activation rows, with every count checked before any launch
  int64_t total = 0;
  for (int64_t e = 0; e < n_expert; ++e) {
    const int64_t m = m_per_expert[e];
    if (m < 0 || m > INT_MAX || total > INT64_MAX - m) return GQ_ERR_SHAPE;
    total += m;
  }
  if (total == 0) return GQ_OK;
  // activation rows are int indices in the kernels (bounded as gq_matmul's M)
  if (total > kMaxDim) return GQ_ERR_SHAPE;
  if (ebytes > INT64_MAX / n_expert) return GQ_ERR_SHAPE;
  if (rows > INT64_MAX / 4 / total || cols > INT64_MAX / 4 / total) return GQ_ERR_SHAPE;
  const int64_t wbytes = ebytes * n_expert, xbytes = total * cols * 4, ybytes = total * rows * 4;
  if (!W || !X || !Y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)X % 4 || (uintptr_t)Y % 4) return GQ_ERR_ALIGN;
  if (overlaps(Y, ybytes, W, wbytes) || overlaps(Y, ybytes, X, xbytes)) return GQ_ERR_OVERLAP;
  if (f16_layout(fmt, cols, rb, W) && !gq::gemm_f16_fits(rows, cols, rb)) return GQ_ERR_SHAPE;

  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  if (f16_layout(fmt, cols, rb, W)) {
    // one grouped launch per 64 experts: group e multiplies expert e by its
    // m_per_expert[e] rows of X (starting after the earlier experts' rows)
    gq::GemmArgs a{(const uint8_t*)W, X, Y, rb, (int)rows, (int)cols, 0, 0};
    constexpr int64_t kChunk = 64;
    int64_t off[kChunk];
    int64_t m0 = 0;
    for (int64_t e0 = 0; e0 < n_expert; e0 += kChunk) {
      const int ne = (int)(n_expert - e0 < kChunk ? n_expert - e0 : kChunk);
      for (int g = 0; g < ne; ++g) {
        off[g] = m0;
        m0 += m_per_expert[e0 + g];
      }
      a.W = (const uint8_t*)W + e0 * ebytes;
      st = finish(gq::launch_gemm_f16(fmt, a, m_per_expert + e0, off, ne, ebytes, cus, (hipStream_t)stream));
      if (st != GQ_OK) return st;
    }
    return GQ_OK;
  }
  // one gq_matmul per expert with rows, in expert order on the caller's stream
  int64_t m0 = 0;
  for (int64_t e = 0; e < n_expert; ++e) {
    const int64_t m = m_per_expert[e];
    if (m == 0) continue;
    st = matmul_route(fmt, (const uint8_t*)W + e * ebytes, rb, rows, cols, X + m0 * cols, m,
                      Y + m0 * rows, stream, cus);
    if (st != GQ_OK) return st;
    m0 += m;
  }
  return GQ_OK;
}

extern "C" int gq_quantize_q8_1(const float* x, int64_t n, int64_t cols, void* xq, void* stream) {
  if (n < 0 || cols <= 0 || n > kMaxDim || cols > kMaxDim) return GQ_ERR_SHAPE;
  const int64_t rb = gq_row_bytes(GQ_FMT_Q8_1, cols);
  if (n > 0 && (rb > INT64_MAX / n || cols > INT64_MAX / 4 / n || n * ((cols + 31) / 32) > INT64_MAX / 8))
    return GQ_ERR_SHAPE;
  if (n == 0) return GQ_OK;
  if (!x || !xq) return GQ_ERR_NULL;
  if ((uintptr_t)x % 4 || (uintptr_t)xq % 4) return GQ_ERR_ALIGN;
  if (overlaps(xq, n * rb, x, n * cols * 4)) return GQ_ERR_OVERLAP;
  (void)hipGetLastError();
  return finish(gq::launch_quantize_q8_1(x, n, (int)cols, (uint8_t*)xq, (hipStream_t)stream));
}

extern "C" int gq_matvec_q8_1(int fmt, const void* W, int64_t rows, int64_t cols, const void* xq, float* y,
                              void* stream) {
  int64_t rb = 0, wbytes = 0;
  int st = check_shape(fmt, rows, cols, 1, &rb, &wbytes);
  if (st != GQ_OK) return st;
  if (fmt != GQ_FMT_Q8_0 && fmt != GQ_FMT_Q4_K) return GQ_ERR_FMT;
  if (cols > 131072) return GQ_ERR_SHAPE;  // the quantised row is staged in LDS
  if (rows == 0) return GQ_OK;
  if (!W || !xq || !y) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((uintptr_t)xq % 4 || (uintptr_t)y % 4) return GQ_ERR_ALIGN;
  if (overlaps(y, rows * 4, W, wbytes) || overlaps(y, rows * 4, xq, gq_row_bytes(GQ_FMT_Q8_1, cols)))
    return GQ_ERR_OVERLAP;
  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return finish(gq::launch_gemv_q8a(fmt, (const uint8_t*)W, rb, (int)rows, (int)cols, (const uint8_t*)xq, y, cus,
                                    (hipStream_t)stream));
}

extern "C" int gq_moe_bucket(const int32_t* expid, int64_t n_assign, int64_t n_expert, int64_t* counts,
                             int32_t* order, int32_t* pos, void* stream) {
  if (n_expert < 1 || n_expert > gq::kMaxBucketExperts || n_assign < 0 || n_assign > kMaxDim)
    return GQ_ERR_SHAPE;
  if (!counts || (n_assign > 0 && (!expid || !order || !pos))) return GQ_ERR_NULL;
  if ((uintptr_t)counts % 8 || (uintptr_t)expid % 4 || (uintptr_t)order % 4 || (uintptr_t)pos % 4)
    return GQ_ERR_ALIGN;
  const int64_t ib = n_assign * 4, cb = n_expert * 8;
  if (overlaps(counts, cb, expid, ib) || overlaps(counts, cb, order, ib) || overlaps(counts, cb, pos, ib) ||
      overlaps(order, ib, expid, ib) || overlaps(pos, ib, expid, ib) || overlaps(order, ib, pos, ib))
    return GQ_ERR_OVERLAP;
  if (current_cus() <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return finish(gq::launch_moe_bucket(expid, (int)n_assign, (int)n_expert, counts, order, pos,
                                      (hipStream_t)stream));
}

extern "C" int gq_moe_gather(const float* X, int64_t cols, int64_t k, const int32_t* pos, int64_t n_assign,
                             float* Xb, void* stream) {
  if (cols < 1 || cols > kMaxDim || k < 1 || k > kMaxDim || n_assign < 0 || n_assign > kMaxDim)
    return GQ_ERR_SHAPE;
  if (n_assign == 0) return GQ_OK;
  const int64_t xrows = (n_assign + k - 1) / k;
  if (cols > INT64_MAX / 4 / n_assign) return GQ_ERR_SHAPE;
  if (!X || !pos || !Xb) return GQ_ERR_NULL;
  if ((uintptr_t)X % 4 || (uintptr_t)pos % 4 || (uintptr_t)Xb % 4) return GQ_ERR_ALIGN;
  const int64_t xbb = n_assign * cols * 4;
  if (overlaps(Xb, xbb, X, xrows * cols * 4) || overlaps(Xb, xbb, pos, n_assign * 4)) return GQ_ERR_OVERLAP;
  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return finish(gq::launch_moe_gather(X, (int)cols, (int)k, pos, (int)n_assign, Xb, cus, (hipStream_t)stream));
}

extern "C" int gq_moe_scatter(const float* Yb, int64_t rows, const int32_t* pos, const float* w,
                              int64_t n_assign, int64_t k, float* out, void* stream) {
  if (rows < 0 || rows > kMaxDim || k < 1 || k > kMaxDim || n_assign < 0 || n_assign > kMaxDim ||
      n_assign % k != 0)
    return GQ_ERR_SHAPE;
  if (rows == 0 || n_assign == 0) return GQ_OK;
  if (rows > INT64_MAX / 4 / n_assign) return GQ_ERR_SHAPE;
  if (!Yb || !pos || !w || !out) return GQ_ERR_NULL;
  if ((uintptr_t)Yb % 4 || (uintptr_t)pos % 4 || (uintptr_t)w % 4 || (uintptr_t)out % 4) return GQ_ERR_ALIGN;
  const int64_t n_tok = n_assign / k, ob = n_tok * rows * 4;
  if (overlaps(out, ob, Yb, n_assign * rows * 4) || overlaps(out, ob, pos, n_assign * 4) ||
      overlaps(out, ob, w, n_assign * 4))
    return GQ_ERR_OVERLAP;
  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  return finish(gq::launch_moe_scatter(Yb, (int)rows, pos, w, (int)n_tok, (int)k, out, cus,
                                       (hipStream_t)stream));
}

extern "C" int gq_matmul_experts_dev(int fmt, const void* W, int64_t n_expert, int64_t rows, int64_t cols,
                                     const float* X, const int64_t* m_dev, int64_t total, float* Y,
                                     void* stream) {
  int64_t rb = 0, ebytes = 0;
  int st = check_shape(fmt, rows, cols, 1, &rb, &ebytes);
  if (st != GQ_OK) return st;
  if (n_expert < 1 || n_expert > gq::kMaxBucketExperts || total < 0 || total > kMaxDim) return GQ_ERR_SHAPE;
  // the fp16 matrix-core layouts only (rows of whole dwords where the format needs it)
  const bool dword_format = fmt == GQ_FMT_Q8_0 || fmt == GQ_FMT_Q5_0 || fmt == GQ_FMT_Q6_K;
  if (cols % 4 != 0 || (dword_format && rb % 4 != 0)) return GQ_ERR_SHAPE;
  if (rows == 0 || total == 0) return GQ_OK;
  if (ebytes > INT64_MAX / n_expert) return GQ_ERR_SHAPE;
  if (rows > INT64_MAX / 4 / total || cols > INT64_MAX / 4 / total) return GQ_ERR_SHAPE;
  if (!gq::gemm_f16_fits(rows, cols, rb)) return GQ_ERR_SHAPE;
  const int64_t wbytes = ebytes * n_expert, xbytes = total * cols * 4, ybytes = total * rows * 4;
  if (!W || !X || !Y || !m_dev) return GQ_ERR_NULL;
  if ((st = check_align(fmt, W)) != GQ_OK) return st;
  if ((dword_format && (uintptr_t)W % 4) || (uintptr_t)X % 4 || (uintptr_t)Y % 4 || (uintptr_t)m_dev % 8)
    return GQ_ERR_ALIGN;
  if (overlaps(Y, ybytes, W, wbytes) || overlaps(Y, ybytes, X, xbytes) || overlaps(Y, ybytes, m_dev, n_expert * 8))
    return GQ_ERR_OVERLAP;
  const int cus = current_cus();
  if (cus <= 0) return GQ_ERR_DEVICE;
  (void)hipGetLastError();
  gq::GemmArgs a{(const uint8_t*)W, X, Y, rb, (int)rows, (int)cols, 0, 0};
  return finish(gq::launch_gemm_f16_dev(fmt, a, m_dev, (int)n_expert, (int)total, ebytes, cus,
                                        (hipStream_t)stream));
}
