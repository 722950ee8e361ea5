// gemm_f32.hip -- Y = X W^T on the fp32 matrix cores for Q8_0 (packed or
// split per row), Q5_0, Q5_K and Q6_K weights (the prompt-chunk product, "nurllama 0.18.1 API",
// model.nu section; the Loom inventory's prefill GEMMs per format).
//
// These formats scale every 16 or 32 weights, and scale * code needs up to
// 18 significant bits (Q8_0 d*q), so no exact fp16 operand exists (the Q4_K
// path in gemm_f16.hip relies on sc*code <= 945). Here each k-chunk of the
// weight tile is dequantised exactly to fp32 in LDS (gq_quads.h, the same
// values gq_dequant writes) and multiplied with fp32 activations by
// v_mfma_f32_16x16x4f32, accumulating in fp32.
//
// A workgroup of KS groups of RW waves owns 16 RW weight rows x 16 WM
// activation rows; group g takes the k-chunks g, g + KS, ... and the groups'
// products are added in group order at the end (deterministic; no memory
// beyond the arguments). Per chunk of 128 k: every thread of a group decodes
// 8 quads of weights into the group's W tile and stores its share of the X
// tile (both requested into registers during the previous chunk); then wave
// w of the group multiplies weight rows 16w..16w+15 by all activation rows.
// Within each group of 16 k, lane (i, q) = (lane & 15, lane >> 4) supplies
// k = 4q + s at MFMA step s for both operands (the same permutation of k on
// both sides leaves the sum unchanged), so each operand is one 16-byte LDS
// read per 16 k.
//
// Q4_K runs here only for rows whose length is not a multiple of 4 (the
// fp16 matrix-core kernel reads activations four at a time).
#include "gemv_common.h"
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_quads.h"

namespace gq {

namespace {


struct F32Args {
  const uint8_t* W;
  const float* X;
  float* Y;
  int64_t row_bytes;
  int rows, cols, M;
  int nchunk;  // k-chunks in a row (of the kernel's chunk size)
  int xvec;    // X rows are 16-byte aligned and cols % 4 == 0
};

template <class Q, int WM, int RW, int KS, int PF, int KC, int EPI>
__global__ __launch_bounds__(64 * RW * KS) void gemm_f32_kernel(F32Args a) {
  static_assert(PF == 1 || PF == 2, "prefetch depth");
  static_assert(KC == 64 || KC == 128, "chunk");
  constexpr int kLD = KC + 4;               // LDS row stride in floats (16-byte rows, banks spread)
  constexpr int kQR = KC / 4;               // quads per tile row
  constexpr int kGT = 64 * RW;              // threads per group
  constexpr int kWQ = 16 * RW * kQR / kGT;  // W quads per thread and chunk
  constexpr int kXQ = 16 * WM * kQR / kGT;  // X quads per thread and chunk
  constexpr int kTile = (16 * RW + 16 * WM) * kLD;
  static_assert(kXQ >= 1 && (16 * WM * kQR) % kGT == 0, "X share");
  __shared__ __attribute__((aligned(16))) float lds[KS * kTile];

  const int tid = threadIdx.x % kGT;
  const int grp = threadIdx.x / kGT;
  const int wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.x * 16 * RW;
  const int m0 = blockIdx.y * 16 * WM;
  float* Wl = lds + grp * kTile;
  float* Xl = Wl + 16 * RW * kLD;
  // this group's chunks grp, grp + KS, ... (n of them); every group takes
  // the workgroup's step count so that the barriers match
  const int n = a.nchunk > grp ? (a.nchunk - grp + KS - 1) / KS : 0;
  const int steps = (a.nchunk + KS - 1) / KS;

  f32x4 acc[WM];
#pragma unroll
  for (int t = 0; t < WM; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The next chunk's raw weight bytes and activations are requested into
  // registers before the current chunk is multiplied, so their latency hides
  // behind the matrix-core work; they are decoded into LDS after it.
  typename Q::Raw wr_[2][kWQ];
  f32x4 xr_[2][kXQ];
  auto fetch = [&](int c, int st) {
    typename Q::Raw (&wr)[kWQ] = wr_[st];
    f32x4 (&xr)[kXQ] = xr_[st];
    const int k0 = c * KC;
#pragma unroll
    for (int j = 0; j < kWQ; ++j) {  // 16 RW rows x KC k
      const int qd = tid + kGT * j;
      const int row = r0 + qd / kQR, k = k0 + 4 * (qd % kQR);
      if (row < a.rows && k < a.cols) Q::load(wr[j], a.W + (int64_t)row * a.row_bytes, k, a.cols);
    }
#pragma unroll
    for (int j = 0; j < kXQ; ++j) {  // 16*WM rows x KC k, zero past M and cols
      const int qd = tid + kGT * j;
      const int m = m0 + qd / kQR, k = k0 + 4 * (qd % kQR);
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
  auto commit = [&](int c, int st) {
    const typename Q::Raw (&wr)[kWQ] = wr_[st];
    const f32x4 (&xr)[kXQ] = xr_[st];
    const int k0 = c * KC;
#pragma unroll
    for (int j = 0; j < kWQ; ++j) {
      const int qd = tid + kGT * j;
      const int rl = qd / kQR, kk = 4 * (qd % kQR);
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
    for (int j = 0; j < kXQ; ++j) {
      const int qd = tid + kGT * j;
      *(f32x4*)&Xl[(qd / kQR) * kLD + 4 * (qd % kQR)] = xr[j];
    }
  };

  auto multiply = [&]() {
#pragma unroll 4
    for (int k16 = 0; k16 < KC; k16 += 16) {
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
  };
  // step s: decode chunk s (its requests were made PF steps earlier) into
  // the tiles, then request chunk s + PF into the freed registers, then
  // multiply
  auto step = [&](int s, int st) {
    if (s < n) commit(grp + KS * s, st);
    __syncthreads();
    if (s + PF < n) fetch(grp + KS * (s + PF), st);
    if (s < n) multiply();
    __syncthreads();
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < n) fetch(grp + KS * p, p);
  for (int s = 0; s < steps; s += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (s + p < steps) step(s + p, p);
  }

  // groups 1.. park their sums in LDS (the tiles are free now); group 0 adds
  // them in group order
  if constexpr (KS > 1) {
    f32x4* red = (f32x4*)lds;  // [KS - 1][RW][WM][64]
    if (grp > 0) {
#pragma unroll
      for (int t = 0; t < WM; ++t) red[(((grp - 1) * RW + wave) * WM + t) * 64 + lane] = acc[t];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int t = 0; t < WM; ++t) {
        const f32x4 o = red[(((g - 1) * RW + wave) * WM + t) * 64 + lane];
        acc[t] = f32x4{acc[t].x + o.x, acc[t].y + o.y, acc[t].z + o.z, acc[t].w + o.w};
      }
  }

  // D lane layout: column (weight row) i, activation rows 4q..4q+3
  const int r = r0 + 16 * wave + i;
  if (r >= a.rows) return;
#pragma unroll
  for (int t = 0; t < WM; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + 16 * t + 4 * q + e;
      if (m < a.M) {
        float* p = a.Y + (int64_t)m * a.rows + r;
        if constexpr (EPI == kMmAcc) *p += acc[t][e];
        else if constexpr (EPI == kMmSiluMul) *p = silu_mul(acc[t][e], *p);
        else *p = acc[t][e];
      }
    }
  }
}

template <class Q, int WM, int RW, int KS, int PF, int KC, int EPI>
hipError_t launch(F32Args a, int gy, hipStream_t s) {
  const int gx = (a.rows + 16 * RW - 1) / (16 * RW);
  a.nchunk = (a.cols + KC - 1) / KC;
  hipLaunchKernelGGL((gemm_f32_kernel<Q, WM, RW, KS, PF, KC, EPI>), dim3(gx, gy), dim3(64 * RW * KS), 0, s, a);
  return hipGetLastError();
}

// Tiles, measured on MI355X (Q6_K 4096 x 14336, Q5_K 14336 x 4096, Q8_0
// 4096 x 14336): 64 weight rows per workgroup (four waves sharing the
// tiles) when that grid gives two workgroups per CU, or about one per CU
// with two or four m-tiles; otherwise 16 rows per workgroup with its waves
// splitting k (each decoding its own 16-row tile): eight waves for one
// m-tile (Q6_K M = 16: 58 us against 127 with four), six or eight with 64-k
// chunks (so that their tiles fit the LDS) for four or two (Q6_K M = 64:
// 158 us against 232 with four).
template <class Q, int EPI>
hipError_t launch_wm(const F32Args& a, int cus, hipStream_t s) {
  const int mtiles = (a.M + 15) / 16;
  const int WM = mtiles >= 4 ? 4 : mtiles >= 2 ? 2 : 1;
  const int gy = (mtiles + WM - 1) / WM;
  const int64_t grid = (int64_t)((a.rows + 63) / 64) * gy;
  if (grid >= 2LL * cus || (WM > 1 && grid >= (int64_t)cus * 7 / 8)) {
    if (WM == 4) return launch<Q, 4, 4, 1, 1, 128, EPI>(a, gy, s);
    if (WM == 2) return launch<Q, 2, 4, 1, 1, 128, EPI>(a, gy, s);
    return launch<Q, 1, 4, 1, 1, 128, EPI>(a, gy, s);
  }
  if (WM == 4) return launch<Q, 4, 1, 6, 1, 64, EPI>(a, gy, s);
  if (WM == 2) return launch<Q, 2, 1, 8, 1, 64, EPI>(a, gy, s);
  return launch<Q, 1, 1, 8, 1, 128, EPI>(a, mtiles, s);
}

}  // namespace

namespace {

template <int EPI>
hipError_t launch_gemm_f32_epi(int fmt, const F32Args& fa, int cus, hipStream_t s) {
  switch (fmt) {
    case kFmtQ8_0: return launch_wm<Q8Quad, EPI>(fa, cus, s);
    case kFmtQ5_0: return launch_wm<Q5_0Quad, EPI>(fa, cus, s);
    case kFmtQ4_K: return launch_wm<Q4KQuad, EPI>(fa, cus, s);
    case kFmtQ5_K: return launch_wm<Q5KQuad, EPI>(fa, cus, s);
    case kFmtQ6_K: return launch_wm<Q6KQuad, EPI>(fa, cus, s);
    case kFmtQ8_0Split: return launch_wm<Q8SplitQuad, EPI>(fa, cus, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_f32(int fmt, GemmArgs a, int cus, hipStream_t s, int epi) {
  const int xvec = (a.cols % 4 == 0) && (((uintptr_t)a.X & 15) == 0);
  const F32Args fa{a.W, a.X, a.Y, a.row_bytes, a.rows, a.cols, a.M, 0, xvec};
  switch (epi) {
    case kMmStore: return launch_gemm_f32_epi<kMmStore>(fmt, fa, cus, s);
    case kMmAcc: return launch_gemm_f32_epi<kMmAcc>(fmt, fa, cus, s);
    case kMmSiluMul: return launch_gemm_f32_epi<kMmSiluMul>(fmt, fa, cus, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gq
