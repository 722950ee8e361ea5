// moe.hip -- the index and copy steps around the grouped prefill product of
// a mixture-of-experts layer: bucketing of the (position, expert)
// assignments by expert, the gather of each assignment's activation row into
// its bucket, and the weighted scatter of the experts' output rows back to
// the positions.
//
// The Loom porting skill ("What the starter generates", the MoE generator)
// buckets the rows by expert ahead of the grouped GEMMs; the batched kernel
// set of "nurllama 0.18.1 API" (kernels.nu section) carries the assignment
// table as an expert id and a weight per (position, selected expert) pair and
// ends the layer with a scatter that adds, for every position, the weighted
// sum of its experts' rows onto the output.
//
// Bucketing is a stable counting sort: assignment a (= position * k + slot)
// with expert e goes to bucket e, after every earlier assignment of that
// expert. One workgroup walks the assignments in tiles of 1024 (one per
// thread): inside a wave, lanes with the same expert are ranked by ballot;
// per-wave counts in LDS give each wave's offset; a running count per expert
// carries over from tile to tile. No atomics, so the placement is the same on
// every run.
#include <algorithm>

#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / 64;

__global__ __launch_bounds__(kBucketThreads) void moe_bucket_kernel(const int32_t* __restrict__ expid,
                                                                    int n_assign, int n_expert,
                                                                    int64_t* __restrict__ counts,
                                                                    int32_t* __restrict__ order,
                                                                    int32_t* __restrict__ pos) {
  __shared__ int wcnt[kBucketWaves][kMaxBucketExperts];  // this tile's count per wave and expert
  __shared__ int run[kMaxBucketExperts];                 // assignments of each expert in earlier tiles
  __shared__ int scan[kBucketThreads];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t below = lane == 0 ? 0ull : ~0ull >> (64 - lane);  // the lanes under this one

  for (int e = tid; e < n_expert; e += kBucketThreads) {
    run[e] = 0;
#pragma unroll
    for (int v = 0; v < kBucketWaves; ++v) wcnt[v][e] = 0;
  }
  __syncthreads();

  // pass 1: each valid assignment's rank among the earlier ones of its expert
  for (int t0 = 0; t0 < n_assign; t0 += kBucketThreads) {
    const int a = t0 + tid;
    const int e = a < n_assign ? expid[a] : -1;
    const bool valid = e >= 0 && e < n_expert;
    int rank = 0;
    uint64_t left = __ballot(valid);
    while (left) {  // one round per distinct expert in the wave
      const int leader = __ffsll((unsigned long long)left) - 1;
      const int key = __shfl(e, leader);
      const uint64_t m = __ballot(valid && e == key);
      if (valid && e == key) rank = __popcll(m & below);
      if (lane == leader) wcnt[w][key] = __popcll(m);
      left &= ~m;
    }
    __syncthreads();
    if (valid) {
      int r = run[e] + rank;
      for (int v = 0; v < w; ++v) r += wcnt[v][e];
      pos[a] = r;
    }
    __syncthreads();
    // carry the tile's counts (in wave order) and clear them for the next tile
    for (int e2 = tid; e2 < n_expert; e2 += kBucketThreads) {
      int s = run[e2];
#pragma unroll
      for (int v = 0; v < kBucketWaves; ++v) {
        s += wcnt[v][e2];
        wcnt[v][e2] = 0;
      }
      run[e2] = s;
    }
    __syncthreads();
  }

  // counts, and the first bucket position of each expert (exclusive prefix
  // sum over the experts, n_expert <= the workgroup's threads)
  const int own = tid < n_expert ? run[tid] : 0;
  scan[tid] = own;
  for (int off = 1; off < kBucketThreads; off <<= 1) {
    __syncthreads();
    const int t = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += t;
  }
  if (tid < n_expert) counts[tid] = own;
  __syncthreads();
  if (tid < n_expert) run[tid] = scan[tid] - own;
  __syncthreads();

  // pass 2: positions (each thread re-reads the ranks it wrote) and the order
  for (int t0 = 0; t0 < n_assign; t0 += kBucketThreads) {
    const int a = t0 + tid;
    if (a < n_assign) {
      const int e = expid[a];
      if (e >= 0 && e < n_expert) {
        const int p = run[e] + pos[a];
        pos[a] = p;
        order[p] = a;
      } else {
        pos[a] = -1;
      }
    }
  }
}

// Xb[pos[a]] = X[a / k] for every assignment with a position in [0, n_assign)
__global__ __launch_bounds__(256) void moe_gather_kernel(const float* __restrict__ X, int cols, int k,
                                                         const int32_t* __restrict__ pos, int n_assign,
                                                         float* __restrict__ Xb, bool vec4) {
  for (int a = blockIdx.x; a < n_assign; a += gridDim.x) {
    const int p = pos[a];
    if (p < 0 || p >= n_assign) continue;
    const float* src = X + (int64_t)(a / k) * cols;
    float* dst = Xb + (int64_t)p * cols;
    if (vec4) {
      for (int c = threadIdx.x; c < cols / 4; c += blockDim.x)
        reinterpret_cast<float4*>(dst)[c] = reinterpret_cast<const float4*>(src)[c];
    } else {
      for (int c = threadIdx.x; c < cols; c += blockDim.x) dst[c] = src[c];
    }
  }
}

// out[t] += sum_j w[t k + j] * Yb[pos[t k + j]], in slot order, every
// product and sum rounded on its own (no fused multiply-add); four columns
// per thread when the rows allow 16-byte accesses
template <bool kVec4>
__global__ __launch_bounds__(256) void moe_scatter_kernel(const float* __restrict__ Yb, int rows,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ wts, int n_tok, int k,
                                                          int n_assign, float* __restrict__ out) {
#pragma clang fp contract(off)  // a product and the sum it enters round separately
  constexpr int V = kVec4 ? 4 : 1;
  typedef float vec __attribute__((ext_vector_type(V)));
  const int nv = rows / V;
  for (int t = blockIdx.x; t < n_tok; t += gridDim.x) {
    vec* o = reinterpret_cast<vec*>(out + (int64_t)t * rows);
    for (int r = threadIdx.x; r < nv; r += blockDim.x) {
      vec s = {};
      for (int j = 0; j < k; ++j) {
        const int a = t * k + j;
        const int p = pos[a];
        if (p >= 0 && p < n_assign) {
          const vec y = reinterpret_cast<const vec*>(Yb + (int64_t)p * rows)[r];
          s = s + wts[a] * y;
        }
      }
      o[r] = o[r] + s;
    }
  }
}

}  // namespace

hipError_t launch_moe_bucket(const int32_t* expid, int n_assign, int n_expert, int64_t* counts,
                             int32_t* order, int32_t* pos, hipStream_t s) {
  hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(kBucketThreads), 0, s, expid, n_assign, n_expert,
                     counts, order, pos);
  return hipGetLastError();
}

hipError_t launch_moe_gather(const float* X, int cols, int k, const int32_t* pos, int n_assign, float* Xb,
                             int cus, hipStream_t s) {
  const bool vec4 = cols % 4 == 0 && (uintptr_t)X % 16 == 0 && (uintptr_t)Xb % 16 == 0;
  const int blocks = (int)std::min<int64_t>(n_assign, (int64_t)cus * 8);
  hipLaunchKernelGGL(moe_gather_kernel, dim3(blocks), dim3(256), 0, s, X, cols, k, pos, n_assign, Xb, vec4);
  return hipGetLastError();
}

hipError_t launch_moe_scatter(const float* Yb, int rows, const int32_t* pos, const float* wts, int n_tok,
                              int k, float* out, int cus, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>(n_tok, (int64_t)cus * 8);
  const bool vec4 = rows % 4 == 0 && (uintptr_t)Yb % 16 == 0 && (uintptr_t)out % 16 == 0;
  if (vec4)
    hipLaunchKernelGGL(moe_scatter_kernel<true>, dim3(blocks), dim3(256), 0, s, Yb, rows, pos, wts, n_tok, k,
                       n_tok * k, out);
  else
    hipLaunchKernelGGL(moe_scatter_kernel<false>, dim3(blocks), dim3(256), 0, s, Yb, rows, pos, wts, n_tok, k,
                       n_tok * k, out);
  return hipGetLastError();
}

}  // namespace gq
