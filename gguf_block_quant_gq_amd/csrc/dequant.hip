// dequant.hip -- bit-exact expansion of GGUF Q8_0 / Q4_K rows to fp32.
//
// The device counterpart of the host dequant fallback ("nurllama 0.18.1 API",
// model.nu section: a type without a device matvec falls back to host
// dequantisation; the "nurllama" README, "How it is checked", has the device
// kernels agree with that host oracle). Every product here is exact in fp32:
// Q8_0 d*q (11-bit x 8-bit significands) and Q4_K (d*sc)*code, dmin*m
// (at most 21 significant bits), so w = A*code - B rounds exactly once,
// whatever the compiler contracts. fp16 scales are converted with the
// hardware conversion, which keeps fp16 subnormals.
//
// One thread per unit (a Q8_0 block or a 16-byte Q4_K code chunk); the
// kernel is bound by the fp32 writes (4 B out per <= 1.07 B in).
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d, bool vec) {
  if (vec) {
    f32x4 v = {a, b, c, d};
    *(f32x4*)p = v;
  } else {
    p[0] = a; p[1] = b; p[2] = c; p[3] = d;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q8_0_kernel(DequantArgs a) {
  const int64_t total = a.rows * (int64_t)a.units;
  for (int64_t u = blockIdx.x * (int64_t)kThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kThreads) {
    const int64_t row = u / a.units;
    const int j = (int)(u - row * a.units);
    Q8Raw raw;
    q8_load(a.W + row * a.row_bytes + (int64_t)j * kQ8Bytes, raw);
    uint32_t q[8];
    q8_codes(raw, q);
    const float d = half_bits_to_float(raw.d16);
    const int c0 = j * kQ8Weights;
    float* o = a.out + row * a.cols + c0;
    if (c0 + kQ8Weights <= a.cols) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        store4(o + 4 * k, d * i8_at(q[k], 0), d * i8_at(q[k], 1), d * i8_at(q[k], 2),
               d * i8_at(q[k], 3), VEC);
    } else {
#pragma unroll
      for (int i = 0; i < kQ8Weights; ++i)
        if (c0 + i < a.cols) o[i] = d * i8_at(q[i >> 2], i & 3);
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q4_k_kernel(DequantArgs a) {
  const int64_t total = a.rows * (int64_t)a.units;
  for (int64_t u = blockIdx.x * (int64_t)kThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kThreads) {
    const int64_t row = u / a.units;
    const int k = (int)(u - row * a.units);
    const int sb = k >> 3, c = k & 7, g = c >> 1, t = c & 1;
    const int c0 = sb * kQ4KWeights + 64 * g + 16 * t;
    if (c0 >= a.cols) continue;
    const uint8_t* blk = a.W + row * a.row_bytes + (int64_t)sb * kQ4KBytes;
    const u32x4 h = load_u32x4(blk);
    const u32x4 v = load_u32x4(blk + 16 + 16 * c);
    uint32_t sc[2], m[2];
    q4k_scales(q4k_scale_sel(g), h.y, h.z, h.w, sc, m);
    const float d = half_bits_to_float(h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(h.x >> 16);
    const float A0 = d * (float)sc[0], A1 = d * (float)sc[1];      // exact
    const float B0 = dmin * (float)m[0], B1 = dmin * (float)m[1];  // exact
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      lo[i] = A0 * (float)(byte & 15u) - B0;
      hi[i] = A1 * (float)(byte >> 4) - B1;
    }
    float* o = a.out + row * a.cols + c0;
    if (c0 + 48 <= a.cols) {
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        store4(o + i, lo[i], lo[i + 1], lo[i + 2], lo[i + 3], VEC);
        store4(o + 32 + i, hi[i], hi[i + 1], hi[i + 2], hi[i + 3], VEC);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < a.cols) o[i] = lo[i];
        if (c0 + 32 + i < a.cols) o[32 + i] = hi[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_dequant(int fmt, DequantArgs a, hipStream_t s) {
  a.units = fmt == kFmtQ8_0 ? (a.cols + 31) / 32 : 8 * ((a.cols + 255) / 256);
  const int64_t total = a.rows * (int64_t)a.units;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  const bool vec = (a.cols % 4 == 0) && (((uintptr_t)a.out & 15) == 0);
  dim3 grid((unsigned)blocks), block(kThreads);
  if (fmt == kFmtQ8_0) {
    if (vec) hipLaunchKernelGGL(dequant_q8_0_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(dequant_q8_0_kernel<false>, grid, block, 0, s, a);
  } else {
    if (vec) hipLaunchKernelGGL(dequant_q4_k_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(dequant_q4_k_kernel<false>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gq
