// gemm_f32.hip -- Y = X W^T on the fp32 matrix cores for Q8_0 (packed or
// split per row), Q5_0, Q5_K and Q6_K weights (the prompt-chunk product, "nurllama 0.18.1 API",
// model.nu section; the Loom inventory's prefill GEMMs per format).
//
// These formats scale every 16 or 32 weights, and scale * code needs up to
// 18 significant bits (Q8_0 d*q), so no exact fp16 operand exists (the Q4_K
// path in gemm_mfma.hip relies on sc*code <= 945). Here each k-chunk of the
// weight tile is dequantised exactly to fp32 in LDS (gq_quads.h, the same
// values gq_dequant writes) and multiplied with fp32 activations by
// v_mfma_f32_16x16x4f32, accumulating in fp32.
//
// A workgroup (4 waves) owns 64 weight rows x 16*WM activation rows and a
// range of k-chunks (split over blockIdx.z when the tiles alone cannot fill
// the GPU; the split partial products are added in split order afterwards).
// Per chunk of 128 k: every thread decodes 8 quads of weights into the W
// tile and stores its share of the X tile (both requested into registers
// during the previous chunk); then wave w multiplies weight rows
// 16w..16w+15 by all activation rows. Within each group of 16 k, lane
// (i, q) = (lane & 15, lane >> 4) supplies k = 4q + s at MFMA step s for both
// operands (the same permutation of k on both sides leaves the sum
// unchanged), so each operand is one 16-byte LDS read per 16 k.
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_quads.h"

namespace gq {

namespace {

constexpr int kKC = 128;        // k per chunk
constexpr int kLD = kKC + 4;    // LDS row stride in floats (keeps 16-byte rows, spreads banks)
constexpr int kRowsWG = 64;     // weight rows per workgroup

struct F32Args {
  const uint8_t* W;
  const float* X;
  float* out;            // Y, or the split partials
  int64_t row_bytes;
  int64_t split_stride;  // floats between the partials of two splits
  int rows, cols, M;
  int nchunk;            // k-chunks in a row
  int per_split;         // k-chunks per split
  int xvec;              // X rows are 16-byte aligned and cols % 4 == 0
};

template <class Q, int WM>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(F32Args a) {
  __shared__ __attribute__((aligned(16))) float Wl[kRowsWG * kLD];
  __shared__ __attribute__((aligned(16))) float Xl[16 * WM * kLD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.x * kRowsWG;
  const int m0 = blockIdx.y * 16 * WM;
  const int z = blockIdx.z;
  const int c_begin = z * a.per_split;
  const int c_end = min(a.nchunk, c_begin + a.per_split);

  f32x4 acc[WM];
#pragma unroll
  for (int t = 0; t < WM; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The next chunk's raw weight bytes and activations are requested into
  // registers before the current chunk is multiplied, so their latency hides
  // behind the matrix-core work; they are decoded into LDS after it.
  typename Q::Raw wr[8];
  f32x4 xr[2 * WM];
  auto fetch = [&](int c) {
    const int k0 = c * kKC;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // 64 rows x 128 k = 2048 quads, 32 threads per row
      const int qd = tid + 256 * j;
      const int row = r0 + (qd >> 5), k = k0 + 4 * (qd & 31);
      if (row < a.rows && k < a.cols) Q::load(wr[j], a.W + (int64_t)row * a.row_bytes, k, a.cols);
    }
#pragma unroll
    for (int j = 0; j < 2 * WM; ++j) {  // 16*WM rows x 128 k, zero past M and cols
      const int qd = tid + 256 * j;
      const int m = m0 + (qd >> 5), k = k0 + 4 * (qd & 31);
      f32x4 xv = {0.f, 0.f, 0.f, 0.f};
      if (m < a.M) {
        const float* xp = a.X + (int64_t)m * a.cols + k;
        if (a.xvec) {
          if (k < a.cols) xv = load_f32x4(xp);
        } else {
          xv.x = k < a.cols ? xp[0] : 0.f;
          xv.y = k + 1 < a.cols ? xp[1] : 0.f;
          xv.z = k + 2 < a.cols ? xp[2] : 0.f;
          xv.w = k + 3 < a.cols ? xp[3] : 0.f;
        }
      }
      xr[j] = xv;
    }
  };
  auto commit = [&](int c) {
    const int k0 = c * kKC;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int qd = tid + 256 * j;
      const int rl = qd >> 5, kk = 4 * (qd & 31);
      const int row = r0 + rl, k = k0 + kk;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (row < a.rows && k < a.cols) {
        Q::decode(wr[j], k, v);
#pragma unroll
        for (int e = 1; e < 4; ++e)
          if (k + e >= a.cols) v[e] = 0.f;  // past the row's last column
      }
      *(f32x4*)&Wl[rl * kLD + kk] = f32x4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int j = 0; j < 2 * WM; ++j) {
      const int qd = tid + 256 * j;
      *(f32x4*)&Xl[(qd >> 5) * kLD + 4 * (qd & 31)] = xr[j];
    }
  };

  if (c_begin < c_end) fetch(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    commit(c);
    __syncthreads();
    if (c + 1 < c_end) fetch(c + 1);
#pragma unroll 4
    for (int k16 = 0; k16 < kKC; k16 += 16) {
      const f32x4 wf = *(const f32x4*)&Wl[(16 * wave + i) * kLD + k16 + 4 * q];
      f32x4 xf[WM];
#pragma unroll
      for (int t = 0; t < WM; ++t) xf[t] = *(const f32x4*)&Xl[(16 * t + i) * kLD + k16 + 4 * q];
#pragma unroll
      for (int t = 0; t < WM; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[t].x, wf.x, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[t].y, wf.y, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[t].z, wf.z, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[t].w, wf.w, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // D lane layout: column (weight row) i, activation rows 4q..4q+3
  const int r = r0 + 16 * wave + i;
  if (r >= a.rows) return;
  float* out = a.out + (int64_t)z * a.split_stride;
#pragma unroll
  for (int t = 0; t < WM; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * t + 4 * q + e;
      if (m < a.M) out[(int64_t)m * a.rows + r] = acc[t][e];
    }
  }
}

template <class Q, int WM>
hipError_t launch(const F32Args& a, int gx, int gy, int ks, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f32_kernel<Q, WM>), dim3(gx, gy, ks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class Q>
hipError_t launch_wm(const F32Args& a, int WM, int gx, int gy, int ks, hipStream_t s) {
  if (WM == 4) return launch<Q, 4>(a, gx, gy, ks, s);
  if (WM == 2) return launch<Q, 2>(a, gx, gy, ks, s);
  return launch<Q, 1>(a, gx, gy, ks, s);
}

}  // namespace

hipError_t launch_gemm_f32(int fmt, GemmArgs a, int cus, hipStream_t s) {
  if (fmt != kFmtQ8_0 && fmt != kFmtQ5_0 && fmt != kFmtQ5_K && fmt != kFmtQ6_K && fmt != kFmtQ8_0Split)
    return hipErrorInvalidValue;
  const int mtiles = (a.M + 15) / 16;
  const int WM = mtiles >= 4 ? 4 : mtiles >= 2 ? 2 : 1;
  const int gx = (a.rows + kRowsWG - 1) / kRowsWG;
  const int gy = (mtiles + WM - 1) / WM;
  const int nchunk = (a.cols + kKC - 1) / kKC;
  // split the k-chunks until two workgroups per CU are busy (>= 2 chunks each)
  int ks = 1;
  while ((int64_t)gx * gy * ks < 2LL * cus && nchunk / (2 * ks) >= 2) ks *= 2;
  const int per_split = (nchunk + ks - 1) / ks;
  ks = (nchunk + per_split - 1) / per_split;

  void* ws = nullptr;
  const int64_t n = (int64_t)a.M * a.rows;
  if (ks > 1) {
    const hipError_t e = ws_alloc((size_t)ks * n * sizeof(float), s, &ws);
    if (e != hipSuccess) return e;
  }
  const int xvec = (a.cols % 4 == 0) && (((uintptr_t)a.X & 15) == 0);
  const F32Args fa{a.W, a.X, ks > 1 ? (float*)ws : a.Y, a.row_bytes, n,
                   a.rows, a.cols, a.M, nchunk, per_split, xvec};
  hipError_t e;
  switch (fmt) {
    case kFmtQ8_0: e = launch_wm<Q8Quad>(fa, WM, gx, gy, ks, s); break;
    case kFmtQ5_0: e = launch_wm<Q5_0Quad>(fa, WM, gx, gy, ks, s); break;
    case kFmtQ5_K: e = launch_wm<Q5KQuad>(fa, WM, gx, gy, ks, s); break;
    case kFmtQ8_0Split: e = launch_wm<Q8SplitQuad>(fa, WM, gx, gy, ks, s); break;
    default: e = launch_wm<Q6KQuad>(fa, WM, gx, gy, ks, s); break;
  }
  if (ks > 1) {
    if (e == hipSuccess) e = launch_split_sum((const float*)ws, a.Y, n, ks, s);
    const hipError_t ef = ws_free(ws, s);
    if (e == hipSuccess) e = ef;
  }
  return e;
}

}  // namespace gq
