// gq_internal.h -- host-side launch interface between the C ABI (gq_api.hip)
// and the kernel files. Not installed; the public interface is include/gq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kFmtQ8_0 = 8;
constexpr int kFmtQ4_K = 12;
constexpr int kFmtQ5_0 = 6;
constexpr int kFmtQ5_K = 13;
constexpr int kFmtQ6_K = 14;
constexpr int kFmtQ8_0Split = 1008;  // Q8_0 repacked: scales first, then codes

struct GemvArgs {
  const uint8_t* W;
  const float* x;
  float* y;
  int64_t row_bytes;
  int rows;   // output rows (the gate|up epilogue reads 2 * rows weight rows)
  int cols;
  int units;  // units per row (set by the launcher)
};

// The expert-batched form (gq_matvec_experts): assignment a = blockIdx.y
// multiplies expert expid[a] (at W + expid[a] * expert_bytes) by activation
// row a / xk of x and writes row a of y (rows floats each). With expid null
// (gq_matvec_batch) every assignment multiplies W itself. Kept out of
// GemvArgs so that the plain matvec's kernel arguments stay small.
struct ExpertArgs {
  const int32_t* expid;
  int64_t expert_bytes;
  int n_expert;
  int xk;
  int n_assign;
};

// What the matvec does with each finished row sum.
enum GemvEpilogue : int {
  kEpiStore = 0,   // y[r] = sum
  kEpiAcc = 1,     // y[r] += sum
  kEpiSwiglu = 2,  // y[r] = silu(sum of row r) * (sum of row rows + r)
};

// What the prefill products do with each finished output (one write per
// output element, so the read-modify-write forms are exact and race-free).
enum GemmEpilogue : int {
  kMmStore = 0,    // Y = sum
  kMmAcc = 1,      // Y += sum
  kMmSiluMul = 2,  // Y = silu(sum) * Y (Y holds the up projection: the SwiGLU's second half)
};

struct DequantArgs {
  const uint8_t* W;
  float* out;
  int64_t row_bytes;
  int64_t rows;
  int cols;
  int units;  // per row: blocks (Q8_0, Q5_0) or super-blocks (K-quants); set by the launcher
};

struct GemmArgs {
  const uint8_t* W;
  const float* X;
  float* Y;
  int64_t row_bytes;
  int rows;
  int cols;
  int M;
  int units;
};

// Q8_0 rows -> the split per-row layout (gq_q8_0_split_repack).
hipError_t launch_q8_0_split_repack(const uint8_t* W, int64_t rows, int cols, int64_t row_bytes,
                                    uint8_t* out, int64_t out_row_bytes, hipStream_t s);

// All launchers enqueue on `s` and return the launch status.
// `units` is filled in by the launcher; `cus` is the device's CU count.
hipError_t launch_dequant(int fmt, DequantArgs a, hipStream_t s);
hipError_t launch_gemv(int fmt, GemvArgs a, int cus, hipStream_t s, int epi = kEpiStore,
                       const ExpertArgs* ex = nullptr);
// The Q4_K matvec for rows of 33..256 units (gemv_q4k.hip): whether a call
// fits it, and its launch (same epilogues and batched form as launch_gemv).
bool gemv_q4k_supports(const GemvArgs& a, int cus, const ExpertArgs* ex);
hipError_t launch_gemv_q4k(GemvArgs a, int cus, hipStream_t s, int epi, const ExpertArgs* ex);
hipError_t launch_gemm_small(int fmt, GemmArgs a, int cus, hipStream_t s);
// The product on the fp16 matrix cores (gemm_f16.hip; fmt is kFmtQ4_K,
// kFmtQ5_K, kFmtQ8_0Split, or kFmtQ8_0 / kFmtQ5_0 / kFmtQ6_K with rows a
// multiple of 4 bytes long and W 4-byte aligned), one launch for n_groups
// products that share a shape: group g multiplies the weight tensor at
// W + g * group_w_bytes by the group_m[g] activation rows starting at row
// group_off[g] of X, into the same rows of Y (a single product: one group).
// It takes cols % 4 == 0 (activations are read four at a time);
// gemm_f16_fits: whether its 31-bit buffer offsets cover the shape.
bool gemm_f16_fits(int64_t rows, int64_t cols, int64_t row_bytes);
hipError_t launch_gemm_f16(int fmt, const GemmArgs& a, const int64_t* group_m, const int64_t* group_off,
                           int n_groups, int64_t group_w_bytes, int cus, hipStream_t s, int epi = kMmStore);
// The grouped product with the per-group row counts on the device (n_expert
// int64 counts at dev_m, total rows of X and Y); the fp16 layouts only.
hipError_t launch_gemm_f16_dev(int fmt, const GemmArgs& a, const int64_t* dev_m, int n_expert, int total,
                               int64_t group_w_bytes, int cus, hipStream_t s);
// The int8-activation path (gemv_q8a.hip): Q8_1 quantisation of n rows of
// activations, and y = W x^ for Q8_0 / Q4_K weights with integer dots.
hipError_t launch_quantize_q8_1(const float* x, int64_t n, int cols, uint8_t* out, hipStream_t s);
hipError_t launch_gemv_q8a(int fmt, const uint8_t* W, int64_t row_bytes, int rows, int cols,
                           const uint8_t* xq, float* y, int cus, hipStream_t s);

// The fp32 matrix-core product (gemm_f32.hip): Q8_0, Q8_0 split, Q5_0, Q5_K,
// Q6_K, and Q4_K rows whose length is not a multiple of 4.
hipError_t launch_gemm_f32(int fmt, GemmArgs a, int cus, hipStream_t s, int epi = kMmStore);

// MoE bucketing, gather and scatter (moe.hip); arguments checked by the
// caller. The bucketing runs in one workgroup with an LDS count per expert.
constexpr int kMaxBucketExperts = 1024;
hipError_t launch_moe_bucket(const int32_t* expid, int n_assign, int n_expert, int64_t* counts,
                             int32_t* order, int32_t* pos, hipStream_t s);
hipError_t launch_moe_gather(const float* X, int cols, int k, const int32_t* pos, int n_assign, float* Xb,
                             int cus, hipStream_t s);
hipError_t launch_moe_scatter(const float* Yb, int rows, const int32_t* pos, const float* wts, int n_tok,
                              int k, float* out, int cus, hipStream_t s);

}  // namespace gq
