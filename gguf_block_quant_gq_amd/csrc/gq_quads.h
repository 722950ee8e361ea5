// gq_quads.h -- four consecutive dequantised weights of one row, exactly:
// the per-lane step of gq_dequant and of the fp32 matrix-core GEMM's weight
// tiles. Block layouts as in gq_device.h; every product here is exact in fp32
// (Q8_0 d*q; Q5_0 d*(code-16); Q5_K (d*sc)*code and dmin*m, so A*code - B
// rounds once whatever the compiler contracts; Q6_K (d*scale)*(code-32)), so
// the values equal the oracle's bit for bit.
//
// i0 is a multiple of 4 and lies inside the row's blocks; the four weights
// are i0..i0+3 (columns past the row's last one are decoded like any other:
// the caller drops or zeroes them).
#pragma once

#include "gq_device.h"

namespace gq {

// Each decoder is split into load (the raw bytes, into registers) and decode
// (the arithmetic), so that a caller can request the next tile's bytes before
// working on the current one; get() does both.

// Q8_0: block i0 / 32, codes (i0 % 32) .. +3 at block bytes 2 + (i0 % 32).
struct Q8Quad {
  struct Raw {
    uint32_t d16, q;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0) {
    const uint8_t* p = row + (int64_t)(i0 >> 5) * kQ8Bytes;
    r.d16 = load_u16(p);
    const uint8_t* cp = p + 2 + (i0 & 31);  // 2-byte aligned
    r.q = load_u16(cp) | (load_u16(cp + 2) << 16);
  }
  __device__ static void decode(const Raw& r, int, float v[4]) {
    const float d = half_bits_to_float(r.d16);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = d * i8_at(r.q, e);
  }
  __device__ static void get(const uint8_t* row, int i0, float v[4]) {
    Raw r;
    load(r, row, i0);
    decode(r, i0, v);
  }
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int) { load(r, row, i0); }
};

// Q5_0: block i0 / 32, t = i0 % 32: nibble bytes (t % 16) .. +3 (low nibbles
// for t < 16, high ones above), bits t .. t+3 of qh. 2-byte loads only.
struct Q5_0Quad {
  struct Raw {
    uint32_t d16, qh16, q;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0) {
    const uint8_t* p = row + (int64_t)(i0 >> 5) * kQ5_0Bytes;
    const int t = i0 & 31;
    r.d16 = load_u16(p);
    r.qh16 = load_u16(p + 2 + 2 * (t >> 4));
    const uint8_t* qp = p + 6 + (t & 15);
    r.q = load_u16(qp) | (load_u16(qp + 2) << 16);
  }
  __device__ static void decode(const Raw& r, int i0, float v[4]) {
    const int t = i0 & 31;
    const float d = half_bits_to_float(r.d16);
    const uint32_t hb = (r.qh16 >> (t & 15)) & 0xFu;
    const uint32_t nib = (t >= 16 ? r.q >> 4 : r.q) & 0x0F0F0F0Fu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int code = (int)(((nib >> (8 * e)) & 0xFu) | (((hb >> e) & 1u) << 4));
      v[e] = d * (float)(code - 16);
    }
  }
  __device__ static void get(const uint8_t* row, int i0, float v[4]) {
    Raw r;
    load(r, row, i0);
    decode(r, i0, v);
  }
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int) { load(r, row, i0); }
};

// Q4_K: super-block i0 / 256, i = i0 % 256 in sub-block j = i / 32 (g = j / 2,
// h = j % 2) at position l0 = i % 32: one code dword (low nibbles for h = 0,
// high ones for h = 1) and the header.
struct Q4KQuad {
  struct Raw {
    u32x4 hd;
    uint32_t w;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0) {
    const uint8_t* blk = row + (int64_t)(i0 >> 8) * kQ4KBytes;
    const int i = i0 & 255, g = i >> 6, l0 = i & 31;
    r.hd = load_u32x4(blk);
    r.w = load_u32(blk + 16 + 32 * g + l0);
  }
  __device__ static void decode(const Raw& r, int i0, float v[4]) {
    const int i = i0 & 255, j = i >> 5, g = j >> 1, h = j & 1;
    uint32_t sc[2], m[2];
    q4k_scales(q4k_scale_sel(g), r.hd.y, r.hd.z, r.hd.w, sc, m);
    const float A = half_bits_to_float(r.hd.x & 0xFFFFu) * (float)sc[h];  // exact
    const float B = half_bits_to_float(r.hd.x >> 16) * (float)m[h];       // exact
    const uint32_t code = (h ? r.w >> 4 : r.w) & 0x0F0F0F0Fu;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = A * (float)((code >> (8 * e)) & 0xFFu) - B;
  }
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int) { load(r, row, i0); }
};

// Q5_K: super-block i0 / 256, i = i0 % 256 in sub-block j = i / 32 (g = j / 2,
// h = j % 2) at position l0 = i % 32: one code dword, one qh dword, the header.
struct Q5KQuad {
  struct Raw {
    u32x4 hd;
    uint32_t qh, w;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0) {
    const uint8_t* blk = row + (int64_t)(i0 >> 8) * kQ5KBytes;
    const int i = i0 & 255, g = i >> 6, l0 = i & 31;
    r.hd = load_u32x4(blk);
    r.qh = load_u32(blk + 16 + l0);
    r.w = load_u32(blk + 48 + 32 * g + l0);
  }
  __device__ static void decode(const Raw& r, int i0, float v[4]) {
    const int i = i0 & 255, j = i >> 5, g = j >> 1, h = j & 1;
    uint32_t sc[2], m[2];
    q4k_scales(q4k_scale_sel(g), r.hd.y, r.hd.z, r.hd.w, sc, m);
    const float A = half_bits_to_float(r.hd.x & 0xFFFFu) * (float)sc[h];  // exact
    const float B = half_bits_to_float(r.hd.x >> 16) * (float)m[h];       // exact
    const uint32_t code = ((h ? r.w >> 4 : r.w) & 0x0F0F0F0Fu) | (((r.qh >> j) & 0x01010101u) << 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = A * (float)((code >> (8 * e)) & 0xFFu) - B;
  }
  __device__ static void get(const uint8_t* row, int i0, float v[4]) {
    Raw r;
    load(r, row, i0);
    decode(r, i0, v);
  }
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int) { load(r, row, i0); }
};

// Q6_K: super-block i0 / 256, i = i0 % 256 = 128 n + 32 k + l0: nibble k / 2
// of ql bytes 64 n + 32 (k % 2) + l0 .., bits 2k, 2k+1 of qh bytes
// 32 n + l0 .., scale i / 16. Super-blocks are 2-byte aligned.
struct Q6KQuad {
  struct Raw {
    uint32_t ql, qh, s2, d16;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0) {
    const uint8_t* blk = row + (int64_t)(i0 >> 8) * kQ6KBytes;
    const int i = i0 & 255, n = i >> 7, k = (i >> 5) & 3, l0 = i & 31, si = i >> 4;
    const uint8_t* lp = blk + 64 * n + 32 * (k & 1) + l0;
    const uint8_t* hp = blk + 128 + 32 * n + l0;
    r.ql = load_u16(lp) | (load_u16(lp + 2) << 16);
    r.qh = load_u16(hp) | (load_u16(hp + 2) << 16);
    r.s2 = load_u16(blk + 192 + (si & ~1));
    r.d16 = load_u16(blk + 208);
  }
  __device__ static void decode(const Raw& r, int i0, float v[4]) {
    const int i = i0 & 255, k = (i >> 5) & 3, si = i >> 4;
    const float scale = (float)(int8_t)(r.s2 >> (8 * (si & 1)));
    const float A = half_bits_to_float(r.d16) * scale;  // exact
    const uint32_t code = ((k >> 1 ? r.ql >> 4 : r.ql) & 0x0F0F0F0Fu) | (((r.qh >> (2 * k)) & 0x03030303u) << 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = A * (float)((int)((code >> (8 * e)) & 0xFFu) - 32);
  }
  __device__ static void get(const uint8_t* row, int i0, float v[4]) {
    Raw r;
    load(r, row, i0);
    decode(r, i0, v);
  }
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int) { load(r, row, i0); }
};

// Q8_0 split per-row layout: code i0 .. i0+3 at the code region + i0 (4-byte
// aligned), the scale of block i0 / 32 at bytes 2 (i0 / 32).
struct Q8SplitQuad {
  struct Raw {
    uint32_t d16, q;
  };
  __device__ static void load(Raw& r, const uint8_t* row, int i0, int cols) {
    r.d16 = load_u16(row + 2 * (i0 >> 5));
    r.q = load_u32(row + split_scale_bytes((cols + 31) / 32) + i0);
  }
  __device__ static void decode(const Raw& r, int, float v[4]) {
    const float d = half_bits_to_float(r.d16);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = d * i8_at(r.q, e);
  }
  __device__ static void get(const uint8_t* row, int i0, int cols, float v[4]) {
    Raw r;
    load(r, row, i0, cols);
    decode(r, i0, v);
  }
};

}  // namespace gq
