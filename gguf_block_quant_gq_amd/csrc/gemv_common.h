// gemv_common.h -- pieces shared by the matvec kernel families (gemv.hip,
// gemv_q4k.hip): the expert-batched argument block and its binding to a
// workgroup, and the row epilogues (overwrite, accumulate, SwiGLU).
#pragma once

#include <type_traits>

#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

// Kernel arguments: the plain form, or the expert-batched form with the
// expert table appended (a separate instantiation, so the plain matvec's
// prologue and argument block carry none of its indirection).
struct GemvExpertArgs {
  GemvArgs g;
  ExpertArgs e;
};

template <bool EXPERTS>
using KernelArgs = typename std::conditional<EXPERTS, GemvExpertArgs, GemvArgs>::type;

__device__ __forceinline__ GemvArgs base_args(const GemvArgs& a) { return a; }
__device__ __forceinline__ GemvArgs base_args(const GemvExpertArgs& a) { return a.g; }

// Expert-batched calls: point a (the workgroup's copy of the arguments) at
// the expert, activation row and output row of assignment blockIdx.y. An
// expert id outside [0, n_expert) reads no weights: the assignment's output
// row is filled with NaN instead. Without an id table (the batched matvec)
// every assignment uses W itself. Returns false when there is nothing more
// to do (uniform per workgroup).
__device__ __forceinline__ bool bind_assignment(GemvArgs& a, const ExpertArgs& ex) {
  const int as = blockIdx.y;
  const int e = ex.expid ? ex.expid[as] : 0;
  a.x += (int64_t)(as / ex.xk) * a.cols;
  a.y += (int64_t)as * a.rows;
  if (e < 0 || e >= ex.n_expert) {
    for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < a.rows; r += gridDim.x * blockDim.x)
      a.y[r] = __builtin_nanf("");
    return false;
  }
  a.W += (int64_t)e * ex.expert_bytes;
  return true;
}

// silu(g) * u = g / (1 + e^-g) * u, in fp32 (e^-g overflows to inf for very
// negative g, giving -0 * u).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.f + expf(-g)) * u;
}

// Output rows per item: the gate|up epilogue turns two weight rows (r and
// rows + r) into one output row.
template <int EPI>
constexpr int weight_rows_per_out() {
  return EPI == kEpiSwiglu ? 2 : 1;
}

// One finished output row: overwrite, accumulate, or the SwiGLU of its gate
// and up sums (g, u).
template <int EPI>
__device__ __forceinline__ void store_row(float* y, int row, float g, float u) {
  if constexpr (EPI == kEpiSwiglu) y[row] = silu_mul(g, u);
  else if constexpr (EPI == kEpiAcc) y[row] += g;
  else y[row] = g;
}

}  // namespace gq
