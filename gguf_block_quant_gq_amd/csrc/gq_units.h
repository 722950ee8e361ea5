// gq_units.h -- the unit of work of the row-group kernels (gemv.hip,
// gemm_small.hip): a Q8_0 block or a 16-byte Q4_K code chunk, 32 weights
// either way. For each format: the x values a lane keeps for its unit, the
// raw bytes of the unit in one row, their in-register decode, and the unit's
// contribution sum_i w_i * x_i.
#pragma once

#include "gq_device.h"

namespace gq {

// ------------------------------------------------------------- Q8_0 unit
struct Q8Unit {
  using Base = Q8Unit;
  static constexpr int kWeights = kQ8Weights;
  static constexpr int kPerUnitCols = 32;  // x columns per unit
  struct X {
    float v[32];
  };
  struct Raw {
    Q8Raw r;
  };
  struct Lane {};  // no per-lane constants

  __device__ static Lane lane(int) { return Lane{}; }

  __device__ static int units_per_row(int cols) { return (cols + 31) / 32; }

  __device__ static bool valid(int unit, int units, int cols) {
    return unit < units;  // every block holds at least one column
  }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    int c0 = unit * kQ8Weights;
    if (c0 + 32 <= cols) {
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        f32x4 t = load_f32x4(xv + c0 + i);
        x.v[i] = t.x; x.v[i + 1] = t.y; x.v[i + 2] = t.z; x.v[i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x.v[i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
    }
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x.v[i] = 0.f;
  }

  __device__ static void finish_x(X&) {}

  // x arrives as 16-byte chunks (4 floats): 8 per unit, in column order.
  static constexpr int kChunks = 8;
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      x.v[4 * k] = c[k].x; x.v[4 * k + 1] = c[k].y; x.v[4 * k + 2] = c[k].z; x.v[4 * k + 3] = c[k].w;
    }
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    q8_load(row + (int64_t)unit * kQ8Bytes, raw.r);
  }

  __device__ static void zero(Raw& raw) { q8_zero(raw.r); }

  __device__ static float dot(const Raw& raw, const X& x, const Lane&) {
    uint32_t q[8];
    q8_codes(raw.r, q);
    float s = q8_block_dot(q, x.v);
    return half_bits_to_float(raw.r.d16) * s;
  }

  // Decoded form, reused across several activation vectors: the unit's
  // dequantised weights w = d * q (exact in fp32).
  struct Dec {
    float w[32];
  };

  __device__ static void decode(Dec& dec, const Raw& raw, const Lane&) {
    uint32_t q[8];
    q8_codes(raw.r, q);
    const float d = half_bits_to_float(raw.r.d16);
#pragma unroll
    for (int i = 0; i < 32; ++i) dec.w[i] = d * i8_at(q[i >> 2], i & 3);
  }

  __device__ static float dot_dec(const Dec& dec, const X& x) {
    return q8_block_dot_f(dec.w, x.v);
  }
};

// -------------------------------------------------------- Q8_0 pair unit
// Two consecutive Q8_0 blocks (68 bytes = 17 dwords), used when every row
// starts on a 4-byte boundary (even block count, 4-byte aligned W): the lane
// loads them with four 16-byte loads and one 4-byte load, both scales
// included (first block: d in bytes 0-1, codes in 2..33; second block: d in
// bytes 34-35, codes in 36..67, dword aligned). Columns 64 u .. 64 u + 63.
struct Q8PairUnit {
  using Base = Q8PairUnit;
  static constexpr int kPerUnitCols = 64;
  struct X {
    float v[64];
  };
  struct Raw {
    uint32_t w[17];
  };
  struct Lane {};

  __device__ static Lane lane(int) { return Lane{}; }

  __device__ static bool valid(int unit, int units, int) { return unit < units; }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    const int c0 = unit * 64;
    if (c0 + 64 <= cols) {
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const f32x4 t = load_f32x4(xv + c0 + i);
        x.v[i] = t.x; x.v[i + 1] = t.y; x.v[i + 2] = t.z; x.v[i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x.v[i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
    }
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x.v[i] = 0.f;
  }

  __device__ static void finish_x(X&) {}

  static constexpr int kChunks = 16;
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      x.v[4 * k] = c[k].x; x.v[4 * k + 1] = c[k].y; x.v[4 * k + 2] = c[k].z; x.v[4 * k + 3] = c[k].w;
    }
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    const uint8_t* p = row + (int64_t)unit * (2 * kQ8Bytes);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 v = load_u32x4(p + 16 * k);
      raw.w[4 * k] = v.x; raw.w[4 * k + 1] = v.y; raw.w[4 * k + 2] = v.z; raw.w[4 * k + 3] = v.w;
    }
    raw.w[16] = load_u32(p + 64);
  }

  __device__ static void zero(Raw& raw) {
#pragma unroll
    for (int k = 0; k < 17; ++k) raw.w[k] = 0u;
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane&) {
    uint32_t q0[8], q1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      q0[k] = __builtin_amdgcn_alignbyte(raw.w[k + 1], raw.w[k], 2);
      q1[k] = raw.w[9 + k];
    }
    const float s0 = q8_block_dot(q0, x.v);
    const float s1 = q8_block_dot(q1, x.v + 32);
    const float d0 = half_bits_to_float(raw.w[0] & 0xFFFFu);
    const float d1 = half_bits_to_float(raw.w[8] >> 16);
    return __builtin_fmaf(d1, s1, d0 * s0);
  }
};

// ------------------------------------------------------------- Q4_K unit
// Unit = the 32 code bytes of group g (0..3) of super-block sb: byte l holds
// the code of weight 64g + l in its low nibble (sub-block 2g) and of weight
// 64g + 32 + l in its high nibble (sub-block 2g + 1). Columns
// sb*256 + 64g + [0, 64). With the min term factored out the unit
// contributes
//   d*sc_2g*sum(lo*x_a) + d*sc_2g+1*sum(hi*x_b) - dmin*(m_2g*X_a + m_2g+1*X_b)
// where x_a, x_b are the unit's two 32-column x slices and X_a, X_b their
// sums (kept per lane, next to the x values).
struct Q4KUnit {
  using Base = Q4KUnit;
  static constexpr int kPerBlock = 4;  // units per super-block
  static constexpr int kPerUnitCols = 64;  // x columns per unit
  struct X {
    float a[32], b[32];
    float sa, sb;
  };
  struct Raw {
    u32x4 q0, q1, h;
  };
  // Per-lane constants: the lane's group g is fixed (G is a multiple of 4),
  // so the bit positions of its two scale and min codes are too.
  struct Lane {
    int g;
    bool high;          // g >= 2: sub-blocks 4..7
    uint32_t o_sc[2];   // bit offset of the low 4 bits of sc_j
    uint32_t o_m[2];    // bit offset of the low 4 bits of m_j
    uint32_t o_top[2];  // bit offset of the top 2 bits of sc_j (in s[0..3]) / m_j (in s[4..7])
  };

  __device__ static Lane lane(int gl) {
    Lane l;
    l.g = gl & 3;
    l.high = l.g >= 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t j = 2u * l.g + e;
      const uint32_t i = j & 3u;
      l.o_sc[e] = 8u * i;
      l.o_m[e] = l.high ? 8u * i + 4u : 8u * i;
      l.o_top[e] = l.high ? 8u * i + 6u : 8u * i + 4u;
    }
    return l;
  }

  __device__ static int units_per_row(int cols) { return 4 * ((cols + 255) / 256); }

  __device__ static int col0(int unit) { return (unit >> 2) * kQ4KWeights + 64 * (unit & 3); }

  __device__ static bool valid(int unit, int units, int cols) {
    return unit < units && col0(unit) < cols;
  }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    const int c0 = col0(unit);
    if (c0 + 64 <= cols) {
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        f32x4 p = load_f32x4(xv + c0 + i);
        f32x4 q = load_f32x4(xv + c0 + 32 + i);
        x.a[i] = p.x; x.a[i + 1] = p.y; x.a[i + 2] = p.z; x.a[i + 3] = p.w;
        x.b[i] = q.x; x.b[i + 1] = q.y; x.b[i + 2] = q.z; x.b[i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        x.a[i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
        x.b[i] = (c0 + 32 + i < cols) ? xv[c0 + 32 + i] : 0.f;
      }
    }
  }

  // x arrives as 16-byte chunks (4 floats): 16 per unit, in column order
  // (chunks 0-7 are x_a, 8-15 are x_b).
  static constexpr int kChunks = 16;
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x.a[4 * k] = c[k].x; x.a[4 * k + 1] = c[k].y; x.a[4 * k + 2] = c[k].z; x.a[4 * k + 3] = c[k].w;
      x.b[4 * k] = c[8 + k].x; x.b[4 * k + 1] = c[8 + k].y;
      x.b[4 * k + 2] = c[8 + k].z; x.b[4 * k + 3] = c[8 + k].w;
    }
  }

  // The sums of the unit's two x slices (the min term's factor); separate
  // from load_x so that the loads can be in flight while W is requested.
  __device__ static void finish_x(X& x) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      s0 += x.a[i];
      s1 += x.b[i];
    }
    x.sa = s0;
    x.sb = s1;
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x.a[i] = x.b[i] = 0.f;
    x.sa = x.sb = 0.f;
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    const uint8_t* blk = row + (int64_t)(unit >> 2) * kQ4KBytes;
    const int g = unit & 3;
    raw.h = load_u32x4(blk);
    raw.q0 = load_u32x4(blk + 16 + 32 * g);
    raw.q1 = load_u32x4(blk + 32 + 32 * g);
  }

  __device__ static void zero(Raw& raw) {
    raw.q0 = raw.q1 = raw.h = u32x4{0, 0, 0, 0};
  }

  // sc_j = low 4 bits | top 2 bits << 4, both read with lane-constant
  // offsets; only the register holding the low bits depends on the lane.
  __device__ static void scales(const Raw& raw, const Lane& ln, float sc[2], float m[2]) {
    const uint32_t h1 = raw.h.y, h2 = raw.h.z, h3 = raw.h.w;
    const uint32_t src_sc = ln.high ? h3 : h1;
    const uint32_t src_m = ln.high ? h3 : h2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t s = __builtin_amdgcn_ubfe(src_sc, ln.o_sc[e], 4) |
                         (__builtin_amdgcn_ubfe(h1, ln.o_top[e], 2) << 4);
      const uint32_t mm = __builtin_amdgcn_ubfe(src_m, ln.o_m[e], 4) |
                          (__builtin_amdgcn_ubfe(h2, ln.o_top[e], 2) << 4);
      sc[e] = (float)s;
      m[e] = (float)mm;
    }
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane& ln) {
    // four independent accumulation chains (two per sub-block)
    float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
    const uint32_t w[8] = {raw.q0.x, raw.q0.y, raw.q0.z, raw.q0.w,
                           raw.q1.x, raw.q1.y, raw.q1.z, raw.q1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t l4 = w[k] & 0x0F0F0F0Fu;
      const uint32_t h4 = (w[k] >> 4) & 0x0F0F0F0Fu;
      const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(l4, false);
      const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(l4, true);
      const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(h4, false);
      const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(h4, true);
      s0 = __builtin_fmaf(a.x, x.a[4 * k + 0], s0);
      s1 = __builtin_fmaf(c.x, x.b[4 * k + 0], s1);
      t0 = __builtin_fmaf(a.y, x.a[4 * k + 1], t0);
      t1 = __builtin_fmaf(c.y, x.b[4 * k + 1], t1);
      s0 = __builtin_fmaf(b.x, x.a[4 * k + 2], s0);
      s1 = __builtin_fmaf(d.x, x.b[4 * k + 2], s1);
      t0 = __builtin_fmaf(b.y, x.a[4 * k + 3], t0);
      t1 = __builtin_fmaf(d.y, x.b[4 * k + 3], t1);
    }
    s0 += t0;
    s1 += t1;
    float sc[2], m[2];
    scales(raw, ln, sc, m);
    const float d = half_bits_to_float(raw.h.x & 0xFFFFu) * kFp8CodeScale;
    const float dmin = half_bits_to_float(raw.h.x >> 16);
    const float qs = __builtin_fmaf(sc[1], s1, sc[0] * s0);
    const float ms = __builtin_fmaf(m[1], x.sb, m[0] * x.sa);
    return __builtin_fmaf(d, qs, -dmin * ms);
  }
};

}  // namespace gq
