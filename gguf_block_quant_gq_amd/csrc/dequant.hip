// dequant.hip -- bit-exact expansion of GGUF Q8_0 / Q4_K / Q5_0 / Q5_K / Q6_K
// rows to fp32.
//
// The device counterpart of the host dequant fallback ("nurllama 0.18.1 API",
// model.nu section: a type without a device matvec falls back to host
// dequantisation; the "nurllama" README, "How it is checked", has the device
// kernels agree with that host oracle). Every product here is exact in fp32:
// Q8_0 d*q (11-bit x 8-bit significands), Q5_0 d*(code-16), Q4_K / Q5_K
// (d*sc)*code and dmin*m (at most 22 significant bits), so w = A*code - B
// rounds exactly once, whatever the compiler contracts, and Q6_K
// (d*scale)*(code-32) (an 11-bit significand times an integer below 2^12).
// fp16 scales are converted with the hardware conversion, which keeps fp16
// subnormals.
//
// One wave per 256 consecutive outputs of a row (a K-quant super-block, or
// eight Q8_0 / Q5_0 blocks): lane l produces outputs 4l..4l+3, so every wave
// store writes one contiguous kilobyte, with non-temporal stores (the kernel is
// bound by the fp32 writes, 4 B out per <= 1.07 B in), and the wave's loads
// stay inside one span of the row of at most 272 bytes.
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_quads.h"

namespace gq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Store the lane's 4 outputs at o (column c0 of a row of `cols`).
template <bool VEC>
__device__ __forceinline__ void store_quad(float* o, int c0, int cols, float a, float b, float c, float d) {
  if (VEC && c0 + 4 <= cols) {
    const f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, (f32x4*)o);  // streamed out, never re-read here
  } else {
    if (c0 < cols) o[0] = a;
    if (c0 + 1 < cols) o[1] = b;
    if (c0 + 2 < cols) o[2] = c;
    if (c0 + 3 < cols) o[3] = d;
  }
}

// Wave item = (row, 8-block group). Lane l: block 8 gi + (l >> 3), codes
// 4 (l & 7) .. +3 of it, i.e. bytes 2 + 4 (l & 7) .. +3 of the block.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q8_0_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int groups = (a.units + 7) / 8;
  const int64_t items = a.rows * (int64_t)groups;
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / groups;
    const int gi = (int)(it - row * groups);
    const int blk = 8 * gi + (lane >> 3);
    const int c0 = blk * kQ8Weights + 4 * (lane & 7);
    if (c0 >= a.cols) continue;
    const uint8_t* p = a.W + row * a.row_bytes + (int64_t)blk * kQ8Bytes;
    const float d = half_bits_to_float(load_u16(p));
    const uint8_t* cp = p + 2 + 4 * (lane & 7);  // 2-byte aligned
    const uint32_t q = load_u16(cp) | (load_u16(cp + 2) << 16);
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, d * i8_at(q, 0), d * i8_at(q, 1), d * i8_at(q, 2), d * i8_at(q, 3));
  }
}

// Wave item = (row, super-block). Lane l: sub-block j = l >> 3, outputs
// 32 j + 4 (l & 7) .. +3, whose codes are the low (j even) or high (j odd)
// nibbles of code bytes 32 (j >> 1) + 4 (l & 7) .. +3: one dword.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q4_k_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int nsb = a.units;
  const int64_t items = a.rows * (int64_t)nsb;
  const int j = lane >> 3, g = j >> 1, h = j & 1;
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / nsb;
    const int sb = (int)(it - row * nsb);
    const int c0 = sb * kQ4KWeights + 4 * lane;
    if (c0 >= a.cols) continue;
    const uint8_t* blk = a.W + row * a.row_bytes + (int64_t)sb * kQ4KBytes;
    const u32x4 hd = load_u32x4(blk);
    const uint32_t w = load_u32(blk + 16 + 32 * g + 4 * (lane & 7));
    uint32_t sc[2], m[2];
    q4k_scales(q4k_scale_sel(g), hd.y, hd.z, hd.w, sc, m);
    const float d = half_bits_to_float(hd.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hd.x >> 16);
    const float A = d * (float)sc[h];     // exact
    const float B = dmin * (float)m[h];   // exact
    const uint32_t n = (h ? w >> 4 : w) & 0x0F0F0F0Fu;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = A * (float)((n >> (8 * e)) & 0xFFu) - B;
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, v[0], v[1], v[2], v[3]);
  }
}

// Wave item = (row, 8-block group), as for Q8_0. Lane l: block 8 gi + (l >> 3),
// weights 4 (l & 7) .. +3 of it (decode in Q5_0Quad, 2-byte loads only).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q5_0_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int groups = (a.units + 7) / 8;
  const int64_t items = a.rows * (int64_t)groups;
  const int i0 = 4 * (lane & 7);
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / groups;
    const int gi = (int)(it - row * groups);
    const int blk = 8 * gi + (lane >> 3);
    const int c0 = blk * kQ5_0Weights + i0;
    if (c0 >= a.cols) continue;
    float v[4];
    Q5_0Quad::get(a.W + row * a.row_bytes, c0, v);
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, v[0], v[1], v[2], v[3]);
  }
}

// Wave item = (row, super-block); lane l produces outputs 4l .. 4l+3
// (sub-block l >> 3; decode in Q5KQuad).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q5_k_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int nsb = a.units;
  const int64_t items = a.rows * (int64_t)nsb;
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / nsb;
    const int sb = (int)(it - row * nsb);
    const int c0 = sb * kQ5KWeights + 4 * lane;
    if (c0 >= a.cols) continue;
    float v[4];
    Q5KQuad::get(a.W + row * a.row_bytes, c0, v);
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, v[0], v[1], v[2], v[3]);
  }
}

// Wave item = (row, super-block); lane l produces outputs 4l .. 4l+3 (half
// l >> 5, run (l >> 3) & 3; decode in Q6KQuad).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q6_k_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int nsb = a.units;
  const int64_t items = a.rows * (int64_t)nsb;
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / nsb;
    const int sb = (int)(it - row * nsb);
    const int c0 = sb * kQ6KWeights + 4 * lane;
    if (c0 >= a.cols) continue;
    float v[4];
    Q6KQuad::get(a.W + row * a.row_bytes, c0, v);
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, v[0], v[1], v[2], v[3]);
  }
}

// Split Q8_0 rows: wave item = (row, 8-block group) as for Q8_0; lane l's four
// codes are one aligned dword of the code region.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_q8_0_split_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int groups = (a.units + 7) / 8;
  const int64_t items = a.rows * (int64_t)groups;
  for (int64_t it = blockIdx.x * (int64_t)kWaves + (threadIdx.x >> 6); it < items;
       it += (int64_t)gridDim.x * kWaves) {
    const int64_t row = it / groups;
    const int gi = (int)(it - row * groups);
    const int c0 = 256 * gi + 4 * lane;
    if (c0 >= a.cols) continue;
    float v[4];
    Q8SplitQuad::get(a.W + row * a.row_bytes, c0, a.cols, v);
    float* o = a.out + row * a.cols + c0;
    store_quad<VEC>(o, c0, a.cols, v[0], v[1], v[2], v[3]);
  }
}

// One thread per (row, block): the block's scale to bytes 2b of the output
// row, its codes to the code region, and (block 0) zeros over the padding.
__global__ __launch_bounds__(kThreads) void q8_0_split_repack_kernel(const uint8_t* W, int64_t rows,
                                                                     int nb, int64_t rb, uint8_t* out,
                                                                     int64_t orb) {
  const int sb = split_scale_bytes(nb);
  const int64_t total = rows * (int64_t)nb;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t row = t / nb;
    const int b = (int)(t - row * nb);
    Q8Raw raw;
    q8_load(W + row * rb + (int64_t)b * kQ8Bytes, raw);
    uint32_t q[8];
    q8_codes(raw, q);
    uint8_t* o = out + row * orb;
    *(uint16_t*)(o + 2 * b) = (uint16_t)raw.d16;
    u32x4* c = (u32x4*)(o + sb + 32 * b);
    c[0] = u32x4{q[0], q[1], q[2], q[3]};
    c[1] = u32x4{q[4], q[5], q[6], q[7]};
    if (b == 0)
      for (int p = 2 * nb; p < sb; p += 2) *(uint16_t*)(o + p) = 0;
  }
}

}  // namespace

hipError_t launch_q8_0_split_repack(const uint8_t* W, int64_t rows, int cols, int64_t row_bytes,
                                    uint8_t* out, int64_t out_row_bytes, hipStream_t s) {
  const int nb = (cols + 31) / 32;
  int64_t blocks = (rows * (int64_t)nb + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(q8_0_split_repack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, W, rows, nb,
                     row_bytes, out, out_row_bytes);
  return hipGetLastError();
}

hipError_t launch_dequant(int fmt, DequantArgs a, hipStream_t s) {
  // units per row: blocks (Q8_0, Q5_0; a wave takes 8) or super-blocks
  const bool small_blocks = fmt == kFmtQ8_0 || fmt == kFmtQ5_0 || fmt == kFmtQ8_0Split;
  a.units = small_blocks ? (a.cols + 31) / 32 : (a.cols + 255) / 256;
  const int64_t items = a.rows * (int64_t)(small_blocks ? (a.units + 7) / 8 : a.units);
  int64_t blocks = (items + kWaves - 1) / kWaves;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const bool vec = (a.cols % 4 == 0) && (((uintptr_t)a.out & 15) == 0);
  dim3 grid((unsigned)blocks), block(kThreads);
#define GQ_DQ_LAUNCH(kern)                                                  \
  do {                                                                      \
    if (vec) hipLaunchKernelGGL(kern<true>, grid, block, 0, s, a);          \
    else hipLaunchKernelGGL(kern<false>, grid, block, 0, s, a);             \
  } while (0)
  switch (fmt) {
    case kFmtQ8_0: GQ_DQ_LAUNCH(dequant_q8_0_kernel); break;
    case kFmtQ4_K: GQ_DQ_LAUNCH(dequant_q4_k_kernel); break;
    case kFmtQ5_0: GQ_DQ_LAUNCH(dequant_q5_0_kernel); break;
    case kFmtQ5_K: GQ_DQ_LAUNCH(dequant_q5_k_kernel); break;
    case kFmtQ6_K: GQ_DQ_LAUNCH(dequant_q6_k_kernel); break;
    case kFmtQ8_0Split: GQ_DQ_LAUNCH(dequant_q8_0_split_kernel); break;
    default: return hipErrorInvalidValue;
  }
#undef GQ_DQ_LAUNCH
  return hipGetLastError();
}

}  // namespace gq
