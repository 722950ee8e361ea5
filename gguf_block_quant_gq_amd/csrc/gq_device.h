// gq_device.h -- device-side building blocks shared by the libgq kernels:
// block geometry, raw block loads and in-register unpacking for GGUF Q8_0 and
// Q4_K, and wavefront reductions. gfx950 (CDNA4, wave64) only.
//
// Block formats (named in "nurllama 0.18.1 API", model.nu section, and in the
// "nurllama" README, "What it runs"; byte layouts are GGUF's public ones):
//   Q8_0: 34 B = fp16 d | 32 x int8 q            w = d * q
//   Q4_K: 144 B = fp16 d | fp16 dmin | 12 B scales | 128 B 4-bit codes
//         w = (d * sc_j) * code - dmin * m_j, sub-block j = 2g + h for weight
//         64g + 32h + l, code = nibble h of code byte 32g + l.
//   Q5_0: 22 B = fp16 d | 32-bit qh | 16 B nibbles   w = d * (code - 16);
//         weight i < 16: low nibble of byte i, i >= 16: high nibble of byte
//         i - 16; bit 4 of the code = bit i of qh.
//   Q5_K: 176 B = the 16-byte Q4_K header | 32 B qh | 128 B nibbles placed as
//         Q4_K's codes; bit 4 of weight 64g + 32h + l's code = bit 2g + h of
//         qh[l]. w = (d * sc_j) * code - dmin * m_j.
//   Q6_K: 210 B = 128 B ql | 64 B qh | 16 int8 scales | fp16 d; weight
//         128n + 32k + l: low bits = nibble k >> 1 of ql[64n + 32(k & 1) + l],
//         top two bits = bits 2k, 2k + 1 of qh[32n + l], scale i / 16;
//         w = (d * scale) * (code - 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {

constexpr int kQ8Weights = 32;
constexpr int kQ8Bytes = 34;
constexpr int kQ4KWeights = 256;
constexpr int kQ4KBytes = 144;
constexpr int kQ4KChunksPerBlock = 8;  // 16-byte code chunks per super-block
constexpr int kQ5_0Weights = 32;
constexpr int kQ5_0Bytes = 22;
constexpr int kQ5KWeights = 256;
constexpr int kQ5KBytes = 176;
constexpr int kQ6KWeights = 256;
constexpr int kQ6KBytes = 210;

// Q8_0 split per-row layout: the nb fp16 scales, zero padding to a multiple
// of 16 bytes, then the nb * 32 codes in block order.
__host__ __device__ constexpr int split_scale_bytes(int nb) { return ((2 * nb + 15) / 16) * 16; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 4-bit code c placed in a byte and read as an OCP fp8 e4m3 value is
// exactly c * 2^-9: codes 0..7 are subnormals m * 2^-9 and codes 8..15 are
// (1 + m/8) * 2^-6 = (8 + m) * 2^-9. v_cvt_pk_f32_fp8 therefore turns two
// code bytes into two exact fp32 values with one instruction.
constexpr float kFp8CodeScale = 512.0f;  // 2^9, multiplied back into the scale

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  _Float16 h;
  uint16_t b = (uint16_t)bits;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// 16-byte load from an address that is only known to be 4-byte aligned.
__device__ __forceinline__ u32x4 load_u32x4(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

__device__ __forceinline__ f32x4 load_f32x4(const float* p) {
  f32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

__device__ __forceinline__ uint32_t load_u32(const uint8_t* p) {
  uint32_t v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 4);
  return v;
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
  uint16_t v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 2), 2);
  return v;
}

// ----------------------------------------------------------------- Q8_0 --
// A Q8_0 block starts on any 2-byte boundary. Its 32 code bytes start at
// a + 2. They are read as 9 dwords from B = (a + 2) & ~3 and realigned with
// v_alignbyte; every dword read contains at least one byte of the block, so
// no read leaves the block's own 4-byte-aligned span (when the codes are
// already aligned the ninth dword is not needed and re-reads the eighth).
struct Q8Raw {
  uint32_t d16;
  uint32_t w[9];
  uint32_t shift;  // 0 or 2
};

__device__ __forceinline__ void q8_load(const uint8_t* blk, Q8Raw& r) {
  r.d16 = load_u16(blk);
  r.shift = (uint32_t)(((uintptr_t)blk + 2) & 3);
  const uint8_t* p = blk + 2 - r.shift;  // 4-aligned; pointer arithmetic keeps global loads
  u32x4 v0 = load_u32x4(p);
  u32x4 v1 = load_u32x4(p + 16);
  r.w[0] = v0.x; r.w[1] = v0.y; r.w[2] = v0.z; r.w[3] = v0.w;
  r.w[4] = v1.x; r.w[5] = v1.y; r.w[6] = v1.z; r.w[7] = v1.w;
  r.w[8] = load_u32(p + (r.shift ? 32 : 28));
}

__device__ __forceinline__ void q8_zero(Q8Raw& r) {
  r.d16 = 0;
#pragma unroll
  for (int k = 0; k < 9; ++k) r.w[k] = 0;
  r.shift = 0;
}

// The 32 code bytes as 8 aligned dwords.
__device__ __forceinline__ void q8_codes(const Q8Raw& r, uint32_t q[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = __builtin_amdgcn_alignbyte(r.w[k + 1], r.w[k], r.shift);
}

__device__ __forceinline__ float i8_at(uint32_t w, int byte) {
  return (float)(int8_t)(w >> (8 * byte));
}

// sum_i q_i * x_i over one block (fp32, exact products, fixed order).
__device__ __forceinline__ float q8_block_dot(const uint32_t q[8], const float x[32]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s0 = __builtin_fmaf(i8_at(q[k], b), x[4 * k + b], s0);
      s1 = __builtin_fmaf(i8_at(q[k + 1], b), x[4 * k + 4 + b], s1);
    }
  }
  return s0 + s1;
}

// The same sum with the codes already converted to fp32.
__device__ __forceinline__ float q8_block_dot_f(const float q[32], const float x[32]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      s0 = __builtin_fmaf(q[4 * k + b], x[4 * k + b], s0);
      s1 = __builtin_fmaf(q[4 * k + 4 + b], x[4 * k + 4 + b], s1);
    }
  }
  return s0 + s1;
}

// ----------------------------------------------------------------- Q4_K --
// Scale codes of sub-blocks j = 2g and 2g + 1 from the header dwords
// h1 = s[0..3], h2 = s[4..7], h3 = s[8..11] (12-byte field, 6-bit codes):
//   j < 4 : sc_j = s[j] & 63,                      m_j = s[j+4] & 63
//   j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
//           m_j  = (s[j+4] >> 4) | (s[j]   >> 6) << 4
struct Q4KScaleSel {
  // per-lane constants for the lane's fixed pair of sub-blocks
  bool high;      // g >= 2
  uint32_t o_lo;  // bit offset of the low field of sc for sub-block 2g
  uint32_t o_hi;  // bit offset of the 2-bit high field (g >= 2)
};

__device__ __forceinline__ Q4KScaleSel q4k_scale_sel(int g) {
  Q4KScaleSel s;
  s.high = g >= 2;
  int j = 2 * g;
  s.o_lo = s.high ? 8u * (uint32_t)(j - 4) : 8u * (uint32_t)j;
  s.o_hi = s.high ? 8u * (uint32_t)(j - 4) + 6u : 0u;
  return s;
}

__device__ __forceinline__ void q4k_scales(const Q4KScaleSel& s, uint32_t h1, uint32_t h2,
                                           uint32_t h3, uint32_t sc[2], uint32_t m[2]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t o = s.o_lo + 8u * e;
    if (!s.high) {
      sc[e] = __builtin_amdgcn_ubfe(h1, o, 6);
      m[e] = __builtin_amdgcn_ubfe(h2, o, 6);
    } else {
      uint32_t oh = s.o_hi + 8u * e;
      sc[e] = __builtin_amdgcn_ubfe(h3, o, 4) | (__builtin_amdgcn_ubfe(h1, oh, 2) << 4);
      m[e] = __builtin_amdgcn_ubfe(h3, o + 4, 4) | (__builtin_amdgcn_ubfe(h2, oh, 2) << 4);
    }
  }
}

// Lane constants for the scale fields of sub-blocks 2g and 2g + 1 (see
// q4_scales).
struct Q4Sel {
  uint32_t sel;  // v_perm_b32 selector: bytes a, a + 1 of each source
  uint32_t sh;   // 0 (g < 2) or 2 (g >= 2)
  uint32_t mt;   // mask of the P bits kept
  uint32_t mq;   // mask of the Q bits kept
};

__device__ __forceinline__ Q4Sel q4_sel(int g) {
  const uint32_t a = 2u * (uint32_t)(g & 1);
  Q4Sel s;
  s.sel = a | ((a + 1) << 8) | ((a + 4) << 16) | ((a + 5) << 24);
  s.sh = g < 2 ? 0u : 2u;
  s.mt = g < 2 ? 0x3F3F3F3Fu : 0x30303030u;
  s.mq = g < 2 ? 0u : 0x0F0F0F0Fu;
  return s;
}

// The codes sc_2g, sc_2g+1, m_2g, m_2g+1 as the four bytes of one dword.
// With h1, h2, h3 = scale bytes 0..3, 4..7, 8..11 and a = 2(g & 1):
//   g < 2 : sc_j = s[j] & 63, m_j = s[j + 4] & 63 (j = a, a + 1), i.e.
//           bytes a, a + 1 of h1 and of h2, masked to six bits;
//   g >= 2: low four bits from bytes a, a + 1 of h3 (sc: low nibble, m: high
//           nibble), top two bits from bits 6-7 of the same bytes of h1 (sc)
//           and h2 (m).
// P = [h1.a, h1.a+1, h2.a, h2.a+1] and Q = [h3.a, h3.a+1, (h3>>4).a, (h3>>4).a+1]
// give both cases as (Q & mq) | ((P >> sh) & mt).
__device__ __forceinline__ uint32_t q4_scales(const u32x4& h, const Q4Sel& s) {
  const uint32_t p = __builtin_amdgcn_perm(h.z, h.y, s.sel);
  const uint32_t q = __builtin_amdgcn_perm(h.w >> 4, h.w, s.sel);
  const uint32_t t = (p >> s.sh) & s.mt;
  return (q & s.mq) | t;
}

// The 32 codes of one 16-byte chunk as fp32 values code * 2^-9:
// lo[l] = low nibble of byte l (sub-block 2g), hi[l] = high nibble (2g + 1).
__device__ __forceinline__ void q4k_chunk_codes(u32x4 v, float lo[16], float hi[16]) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t l4 = w[k] & 0x0F0F0F0Fu;
    uint32_t h4 = (w[k] >> 4) & 0x0F0F0F0Fu;
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(l4, false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(l4, true);
    f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(h4, false);
    f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(h4, true);
    lo[4 * k + 0] = a.x; lo[4 * k + 1] = a.y; lo[4 * k + 2] = b.x; lo[4 * k + 3] = b.y;
    hi[4 * k + 0] = c.x; hi[4 * k + 1] = c.y; hi[4 * k + 2] = d.x; hi[4 * k + 3] = d.y;
  }
}

// ------------------------------------------------------------ reductions --
// Sum over aligned groups of G lanes (G a power of two <= 64) with DPP only
// (no LDS traffic). Within a 16-lane DPP row the butterfly quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror leaves the row
// total in every lane of the row; row_bcast:15 then adds row 0's total into
// row 1 and row 2's into row 3, and row_bcast:31 adds lane 31 into rows 2-3.
// The group total ends up in the group's LAST lane (lane G-1 of the group);
// the association order is fixed, so results are deterministic.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

template <int G>
__device__ __forceinline__ float group_sum_last(float v) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G");
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (G >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if constexpr (G >= 32) v += dpp_f32<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  if constexpr (G >= 64) v += dpp_f32<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// ------------------------------------------- direct global-to-LDS loads --
// The streaming kernels move data straight from a buffer into LDS and wait
// for it with explicit vector-memory counts: that counter retires in order,
// so a wave waits for a given load with vmcnt(N), N = the number of vector
// memory operations it issued after that load.

// One 16-byte-per-lane direct load from a buffer into LDS: lane l's bytes
// land at lds + 16 l (lds is wave-uniform). The LDS address-space cast only
// exists for the GPU; the host pass of a kernel template never runs it.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, void* lds, int voff, int soff) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#else
  (void)rs, (void)lds, (void)voff, (void)soff;
#endif
}

// s_waitcnt with only the vector-memory counter limited to n.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A workgroup barrier that orders the compiler's memory accesses but adds
// no wait of its own (the waits before it are explicit).
__device__ __forceinline__ void bare_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

// Keeps the compiler from moving memory operations across this point: the
// explicit wait counts rely on the vector-memory issue order of the source.
__device__ __forceinline__ void issue_fence() { __asm__ volatile("" ::: "memory"); }

}  // namespace gq
