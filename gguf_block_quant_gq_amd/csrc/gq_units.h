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
  static constexpr int kWeights = kQ8Weights;
  struct X {
    float v[32];
  };
  struct Raw {
    Q8Raw r;
  };
  struct Lane {};  // no per-lane constants

  __device__ static Lane lane(int) { return Lane{}; }

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

  // Decoded form, reused across several activation vectors.
  struct Dec {
    float q[32];
    float d;
  };

  __device__ static void decode(Dec& dec, const Raw& raw, const Lane&) {
    uint32_t q[8];
    q8_codes(raw.r, q);
#pragma unroll
    for (int i = 0; i < 32; ++i) dec.q[i] = i8_at(q[i >> 2], i & 3);
    dec.d = half_bits_to_float(raw.r.d16);
  }

  __device__ static float dot_dec(const Dec& dec, const X& x) {
    return dec.d * q8_block_dot_f(dec.q, x.v);
  }
};

// ------------------------------------------------------------- Q4_K unit
// Unit = 16-byte code chunk c (0..7) of super-block sb: g = c/2, t = c%2.
// Its low nibbles are columns sb*256 + 64g + 16t + [0,16) (sub-block 2g),
// its high nibbles the same + 32 (sub-block 2g+1). With the min term
// factored out, a chunk contributes
//   d*sc_2g*sum(lo*x) + d*sc_2g+1*sum(hi*x) - dmin*(m_2g*X_lo + m_2g+1*X_hi)
// where X_lo, X_hi are the sums of the chunk's x values (kept per lane).
struct Q4KUnit {
  static constexpr int kWeights = 32;
  struct X {
    float lo[16], hi[16];
    float slo, shi;
  };
  struct Raw {
    u32x4 q, h;
  };
  struct Lane {
    Q4KScaleSel sel;
    int c;
  };

  // The chunk position c = unit % 8 equals lane % 8 because G is a multiple
  // of 8, so it is a per-lane constant.
  __device__ static Lane lane(int gl) {
    Lane l;
    l.c = gl & 7;
    l.sel = q4k_scale_sel(l.c >> 1);
    return l;
  }

  __device__ static int col0(int unit) {
    int sb = unit >> 3, c = unit & 7;
    return sb * kQ4KWeights + 64 * (c >> 1) + 16 * (c & 1);
  }

  __device__ static bool valid(int unit, int units, int cols) {
    return unit < units && col0(unit) < cols;
  }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    int c0 = col0(unit);
    if (c0 + 48 <= cols) {
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        f32x4 a = load_f32x4(xv + c0 + i);
        f32x4 b = load_f32x4(xv + c0 + 32 + i);
        x.lo[i] = a.x; x.lo[i + 1] = a.y; x.lo[i + 2] = a.z; x.lo[i + 3] = a.w;
        x.hi[i] = b.x; x.hi[i + 1] = b.y; x.hi[i + 2] = b.z; x.hi[i + 3] = b.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x.lo[i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
        x.hi[i] = (c0 + 32 + i < cols) ? xv[c0 + 32 + i] : 0.f;
      }
    }
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a += x.lo[i];
      b += x.hi[i];
    }
    x.slo = a;
    x.shi = b;
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x.lo[i] = x.hi[i] = 0.f;
    x.slo = x.shi = 0.f;
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    int sb = unit >> 3, c = unit & 7;
    const uint8_t* blk = row + (int64_t)sb * kQ4KBytes;
    raw.h = load_u32x4(blk);
    raw.q = load_u32x4(blk + 16 + 16 * c);
  }

  __device__ static void zero(Raw& raw) {
    raw.q = u32x4{0, 0, 0, 0};
    raw.h = u32x4{0, 0, 0, 0};
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane& ln) {
    float lo[16], hi[16];
    q4k_chunk_codes(raw.q, lo, hi);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0 = __builtin_fmaf(lo[i], x.lo[i], s0);
      s1 = __builtin_fmaf(hi[i], x.hi[i], s1);
    }
    uint32_t sc[2], m[2];
    q4k_scales(ln.sel, raw.h.y, raw.h.z, raw.h.w, sc, m);
    float d = half_bits_to_float(raw.h.x & 0xFFFFu) * kFp8CodeScale;
    float dmin = half_bits_to_float(raw.h.x >> 16);
    float qs = __builtin_fmaf((float)sc[1], s1, (float)sc[0] * s0);
    float ms = __builtin_fmaf((float)m[1], x.shi, (float)m[0] * x.slo);
    return __builtin_fmaf(d, qs, -dmin * ms);
  }

  // Decoded form, reused across several activation vectors: the codes as
  // code * 2^-9 and the four per-chunk factors.
  struct Dec {
    float lo[16], hi[16];
    float a0, a1, b0, b1;  // d*sc*2^9 and dmin*m for sub-blocks 2g, 2g+1
  };

  __device__ static void decode(Dec& dec, const Raw& raw, const Lane& ln) {
    q4k_chunk_codes(raw.q, dec.lo, dec.hi);
    uint32_t sc[2], m[2];
    q4k_scales(ln.sel, raw.h.y, raw.h.z, raw.h.w, sc, m);
    float d = half_bits_to_float(raw.h.x & 0xFFFFu) * kFp8CodeScale;
    float dmin = half_bits_to_float(raw.h.x >> 16);
    dec.a0 = d * (float)sc[0];
    dec.a1 = d * (float)sc[1];
    dec.b0 = dmin * (float)m[0];
    dec.b1 = dmin * (float)m[1];
  }

  __device__ static float dot_dec(const Dec& dec, const X& x) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0 = __builtin_fmaf(dec.lo[i], x.lo[i], s0);
      s1 = __builtin_fmaf(dec.hi[i], x.hi[i], s1);
    }
    float qs = __builtin_fmaf(dec.a1, s1, dec.a0 * s0);
    float ms = __builtin_fmaf(dec.b1, x.shi, dec.b0 * x.slo);
    return qs - ms;
  }
};

}  // namespace gq
