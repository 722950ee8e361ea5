// gemm_small.hip -- Y = X W^T for a few activation rows and Q8_0 or Q5_0
// weights.
//
// The prompt-chunk form of the product ("nurllama 0.18.1 API", model.nu
// section: the matmuls run over several positions at once so each weight is
// read once per chunk). Same row-group decomposition as gemv.hip, but each
// lane decodes its W units once per row batch into registers (codes as fp32
// plus the unit's scale factors) and then sweeps the M activation rows,
// reading each row's x values for its units from global memory (they stay in
// L2: M * cols * 4 bytes). Accumulators are kept per (row, m) and folded
// across the group at the end, in a fixed order.
//
// W is streamed from HBM once per tile of kMaxM activation rows. It serves
// 2 <= M < 8 only: from there on (and for the K-quants from M = 2) the
// matrix-core kernels were measured faster, since this kernel re-reads every
// activation row from L2 for each batch of weight rows.
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_units.h"

namespace gq {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxM = 15;

template <class F, int G, int U, int RB>
__global__ __launch_bounds__(kThreads) void gemm_small_kernel(GemmArgs a) {
  static_assert(G >= 4 && G <= kThreads && (G & (G - 1)) == 0, "G");
  constexpr int kGroups = kThreads / G;
  constexpr int kWavesPerGroup = G > 64 ? G / 64 : 1;
  constexpr int kSeg = G * U;

  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;
  const typename F::Lane ln = F::lane(gl);

  __shared__ float red[kThreads / 64][RB][kMaxM];

  const int nseg = (a.units + kSeg - 1) / kSeg;
  const int rows_per_iter = kGroups * RB;
  for (int r0 = blockIdx.x * rows_per_iter; r0 < a.rows; r0 += gridDim.x * rows_per_iter) {
    const int rbase = r0 + grp * RB;
    for (int m0 = 0; m0 < a.M; m0 += kMaxM) {
      const int mt = (a.M - m0) < kMaxM ? (a.M - m0) : kMaxM;
      float acc[RB][kMaxM];
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int m = 0; m < kMaxM; ++m) acc[i][m] = 0.f;

      for (int seg = 0; seg < nseg; ++seg) {
        const int ubase = seg * kSeg;
        typename F::Dec dec[RB][U];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int row = rbase + i;
          const uint8_t* rp = a.W + (int64_t)row * a.row_bytes;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int unit = ubase + u * G + gl;
            typename F::Raw raw;
            if (row < a.rows && F::valid(unit, a.units, a.cols)) F::load(raw, rp, unit);
            else F::zero(raw);
            F::decode(dec[i][u], raw, ln);
          }
        }
#pragma unroll
        for (int m = 0; m < kMaxM; ++m) {
          if (m < mt) {
            const float* xm = a.X + (int64_t)(m0 + m) * a.cols;
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const int unit = ubase + u * G + gl;
              typename F::X xr;
              if (F::valid(unit, a.units, a.cols)) F::load_x(xr, xm, unit, a.cols);
              else F::zero_x(xr);
              F::finish_x(xr);
#pragma unroll
              for (int i = 0; i < RB; ++i) acc[i][m] += F::dot_dec(dec[i][u], xr);
            }
          }
        }
      }

#pragma unroll
      for (int m = 0; m < kMaxM; ++m) {
        if (m < mt) {
          if constexpr (G <= 64) {
#pragma unroll
            for (int i = 0; i < RB; ++i) {
              const float v = group_sum_last<G>(acc[i][m]);
              const int row = rbase + i;
              if (gl == G - 1 && row < a.rows) a.Y[(int64_t)(m0 + m) * a.rows + row] = v;
            }
          } else {
#pragma unroll
            for (int i = 0; i < RB; ++i) {
              const float v = group_sum_last<64>(acc[i][m]);
              if ((tid & 63) == 63) red[tid >> 6][i][m] = v;
            }
          }
        }
      }
      if constexpr (G > 64) {
        __syncthreads();
        if (gl < RB) {
          const int row = rbase + gl;
          const int w0 = grp * kWavesPerGroup;
          for (int m = 0; m < mt; ++m) {
            float v = red[w0][gl][m];
#pragma unroll
            for (int w = 1; w < kWavesPerGroup; ++w) v += red[w0 + w][gl][m];
            if (row < a.rows) a.Y[(int64_t)(m0 + m) * a.rows + row] = v;
          }
        }
        __syncthreads();
      }
    }
  }
}

template <class F, int G, int U, int RB>
hipError_t launch_one(const GemmArgs& a, int max_blocks, hipStream_t s) {
  constexpr int kGroups = kThreads / G;
  int64_t tiles = ((int64_t)a.rows + kGroups * RB - 1) / (kGroups * RB);
  int blocks = (int)(tiles < max_blocks ? tiles : max_blocks);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((gemm_small_kernel<F, G, U, RB>), dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <class F, int RB>
hipError_t dispatch(const GemmArgs& a, int max_blocks, hipStream_t s) {
  const int n = a.units;
  if (n <= 8) return launch_one<F, 8, 1, RB>(a, max_blocks, s);
  if (n <= 16) return launch_one<F, 16, 1, RB>(a, max_blocks, s);
  if (n <= 32) return launch_one<F, 32, 1, RB>(a, max_blocks, s);
  if (n <= 64) return launch_one<F, 64, 1, RB>(a, max_blocks, s);
  if (n <= 128) return launch_one<F, 128, 1, RB>(a, max_blocks, s);
  return launch_one<F, 256, 1, RB>(a, max_blocks, s);
}

}  // namespace

hipError_t launch_gemm_small(int fmt, GemmArgs a, int cus, hipStream_t s) {
  // Q8_0 and Q5_0 with a few activation rows (below the fp32 matrix-core
  // threshold); the K-quants always run on the matrix cores.
  switch (fmt) {
    case kFmtQ8_0:
      a.units = (a.cols + 31) / 32;
      return dispatch<Q8Unit, 2>(a, cus * 4, s);
    case kFmtQ5_0:
      a.units = (a.cols + 31) / 32;
      return dispatch<Q5_0Unit, 2>(a, cus * 4, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace gq
