// gemv.hip -- y = W x for GGUF Q8_0 / Q4_K weights on gfx950.
//
// The decode-step matrix-vector product is bound by the bytes of W
// (nx_f32_llm_v4 source, model binder: decode is memory-bandwidth bound, so
// bytes moved is the runtime). The kernels stream each packed block once,
// straight from HBM, and decode it in registers.
//
// Work decomposition ("row groups"): the 256 threads of a workgroup form
// 256/G groups of G lanes (G a power of two, 8..256). A group owns one row at
// a time; its lanes split the row into units -- a Q8_0 block (32 weights,
// 34 B) or a 16-byte Q4_K code chunk (32 weights) -- lane l owning units
// l, l + G, ..., l + (U-1)G. Because a lane always owns the same units, the
// x values of those units are loaded once into registers and reused for every
// row the group visits; nothing else is staged. Consecutive lanes own
// consecutive units, so each load instruction of a wave reads one contiguous
// span of the row. Each group keeps RB rows in flight, then folds its lanes'
// partial sums with a fixed butterfly (and, for G > 64, through LDS), so the
// result is deterministic. Rows wider than G*U units are walked in segments,
// reloading x per segment.
//
// Prior art: the one-warp-per-row matvec of the "nurllama" README ("What it
// runs": the warp walks the row's blocks, lanes split each block, a shuffle
// reduction folds the partials), re-shaped for 64-wide wavefronts.
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_units.h"

namespace gq {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ the kernel
template <class F, int G, int U, int RB>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  static_assert(G >= 8 && G <= kThreads && (G & (G - 1)) == 0, "G");
  constexpr int kGroups = kThreads / G;
  constexpr int kWavesPerGroup = G > 64 ? G / 64 : 1;
  constexpr int kSeg = G * U;  // units per segment

  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;
  const typename F::Lane ln = F::lane(gl);

  __shared__ float red[kThreads / 64][RB];

  typename F::X xr[U];
  const int nseg = (a.units + kSeg - 1) / kSeg;
  if (nseg == 1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int unit = u * G + gl;
      if (F::valid(unit, a.units, a.cols)) F::load_x(xr[u], a.x, unit, a.cols);
      else F::zero_x(xr[u]);
    }
  }

  const int rows_per_iter = kGroups * RB;
  for (int r0 = blockIdx.x * rows_per_iter; r0 < a.rows; r0 += gridDim.x * rows_per_iter) {
    const int rbase = r0 + grp * RB;
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = 0.f;

    for (int seg = 0; seg < nseg; ++seg) {
      const int ubase = seg * kSeg;
      if (nseg > 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int unit = ubase + u * G + gl;
          if (F::valid(unit, a.units, a.cols)) F::load_x(xr[u], a.x, unit, a.cols);
          else F::zero_x(xr[u]);
        }
      }
      typename F::Raw raw[RB][U];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = rbase + i;
        const uint8_t* rp = a.W + (int64_t)row * a.row_bytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int unit = ubase + u * G + gl;
          if (row < a.rows && F::valid(unit, a.units, a.cols)) F::load(raw[i][u], rp, unit);
          else F::zero(raw[i][u]);
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc[i] += F::dot(raw[i][u], xr[u], ln);
      }
    }

    if constexpr (G <= 64) {
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i] = group_sum<G>(acc[i]);
      if (gl < RB) {
        float v = acc[0];
#pragma unroll
        for (int i = 1; i < RB; ++i)
          if (gl == i) v = acc[i];
        const int row = rbase + gl;
        if (row < a.rows) a.y[row] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i] = group_sum<64>(acc[i]);
      const int wave = tid >> 6;
      if ((tid & 63) == 0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) red[wave][i] = acc[i];
      }
      __syncthreads();
      if (gl < RB) {
        const int w0 = grp * kWavesPerGroup;
        float v = red[w0][gl];
#pragma unroll
        for (int w = 1; w < kWavesPerGroup; ++w) v += red[w0 + w][gl];
        const int row = rbase + gl;
        if (row < a.rows) a.y[row] = v;
      }
      __syncthreads();
    }
  }
}

template <class F, int G, int U, int RB>
hipError_t launch_one(const GemvArgs& a, int max_blocks, hipStream_t s) {
  constexpr int kGroups = kThreads / G;
  int64_t tiles = ((int64_t)a.rows + kGroups * RB - 1) / (kGroups * RB);
  int blocks = (int)(tiles < max_blocks ? tiles : max_blocks);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((gemv_kernel<F, G, U, RB>), dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// Pick (G, U): the smallest G*U that covers the row's units (at most 4 units
// per lane), preferring fewer idle lanes; wide rows use G = 256, U = 4 and
// segments.
template <class F>
hipError_t dispatch(const GemvArgs& a, int max_blocks, hipStream_t s) {
  const int n = a.units;
  if (n <= 8) return launch_one<F, 8, 1, 4>(a, max_blocks, s);
  if (n <= 16) return launch_one<F, 16, 1, 4>(a, max_blocks, s);
  if (n <= 32) return launch_one<F, 32, 1, 4>(a, max_blocks, s);
  if (n <= 64) return launch_one<F, 64, 1, 4>(a, max_blocks, s);
  if (n <= 128) return launch_one<F, 64, 2, 4>(a, max_blocks, s);
  if (n <= 192) return launch_one<F, 64, 3, 2>(a, max_blocks, s);
  if (n <= 256) return launch_one<F, 64, 4, 2>(a, max_blocks, s);
  if (n <= 512) return launch_one<F, 256, 2, 4>(a, max_blocks, s);
  return launch_one<F, 256, 4, 2>(a, max_blocks, s);
}

}  // namespace

hipError_t launch_gemv(int fmt, const GemvArgs& a, int max_blocks, hipStream_t s) {
  if (fmt == kFmtQ8_0) return dispatch<Q8Unit>(a, max_blocks, s);
  return dispatch<Q4KUnit>(a, max_blocks, s);
}

}  // namespace gq
