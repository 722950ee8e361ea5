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

  __device__ static bool valid(int unit, int units, int /*cols*/) {
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
  __device__ static int x_chunk(int gl, int k) { return kChunks * gl + k; }
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
  __device__ static int x_chunk(int gl, int k) { return kChunks * gl + k; }
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
  // so the selectors and masks that gather its two scale and min codes are
  // too (q4_scales).
  struct Lane {
    int g;
    Q4Sel sel;
  };

  __device__ static Lane lane(int gl) {
    Lane l;
    l.g = gl & 3;
    l.sel = q4_sel(l.g);
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
  __device__ static int x_chunk(int gl, int k) { return kChunks * gl + k; }
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

  // sc_2g, sc_2g+1, m_2g, m_2g+1 gathered into one dword (q4_scales), one
  // v_cvt_f32_ubyte each.
  __device__ static void scales(const Raw& raw, const Lane& ln, float sc[2], float m[2]) {
    const uint32_t scm = q4_scales(raw.h, ln.sel);
    sc[0] = (float)(scm & 0xFFu);
    sc[1] = (float)((scm >> 8) & 0xFFu);
    m[0] = (float)((scm >> 16) & 0xFFu);
    m[1] = (float)(scm >> 24);
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

// ------------------------------------------------- 5- and 6-bit helpers
// Byte t of w as an fp32 value (one v_cvt_f32_ubyte per weight).
__device__ __forceinline__ float ubyte_at(uint32_t w, int t) {
  return (float)((w >> (8 * t)) & 0xFFu);
}

// Four consecutive bits n (0..15) spread to bit 4 of bytes 0..3. The 24-bit
// product n * (1 + 2^7 + 2^14 + 2^21) puts bit t of n at bit t + 7u for
// every u, all 16 positions distinct (so nothing carries); bit t lands on
// bit 8t exactly when u = t.
__device__ __forceinline__ uint32_t spread4_bit4(uint32_t n) {
  return (__umul24(n, 0x204081u) & 0x01010101u) << 4;
}

// Rotate right (v_alignbit with both halves the same register).
__device__ __forceinline__ uint32_t rotr(uint32_t v, uint32_t r) {
  return __builtin_amdgcn_alignbit(v, v, r);
}

// ------------------------------------------------------------- Q5_0 unit
// Unit = one 22-byte block (32 weights, columns 32u .. 32u + 31). Blocks are
// only 2-byte aligned, so the lane loads the six dwords from the 4-byte
// boundary at or below the block start (their first bytes always lie inside
// the block or the dword holding its first two bytes) and shifts them in
// registers. code_i = nibble | (bit i of qh) << 4; w_i = d * (code_i - 16),
// so the unit contributes d * (sum code_i x_i - 16 * sum x_i).
struct Q5_0Unit {
  using Base = Q5_0Unit;
  static constexpr int kPerUnitCols = 32;
  struct X {
    float v[32];
    float s;  // sum of the 32 x values
  };
  struct Raw {
    uint32_t w[6];
    uint32_t shift;  // 0 or 2: bytes between the 4-byte boundary and the block
  };
  struct Lane {};

  __device__ static Lane lane(int) { return Lane{}; }

  __device__ static bool valid(int unit, int units, int) { return unit < units; }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    const int c0 = unit * 32;
    if (c0 + 32 <= cols) {
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 t = load_f32x4(xv + c0 + i);
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
    x.s = 0.f;
  }

  __device__ static void finish_x(X& x) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      s0 += x.v[i];
      s1 += x.v[i + 1];
    }
    x.s = s0 + s1;
  }

  static constexpr int kChunks = 8;
  __device__ static int x_chunk(int gl, int k) { return kChunks * gl + k; }
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      x.v[4 * k] = c[k].x; x.v[4 * k + 1] = c[k].y; x.v[4 * k + 2] = c[k].z; x.v[4 * k + 3] = c[k].w;
    }
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    const uint8_t* blk = row + (int64_t)unit * kQ5_0Bytes;
    raw.shift = (uint32_t)((uintptr_t)blk & 3u);
    const uint8_t* p = blk - raw.shift;  // pointer arithmetic keeps global loads
    const u32x4 v = load_u32x4(p);
    raw.w[0] = v.x; raw.w[1] = v.y; raw.w[2] = v.z; raw.w[3] = v.w;
    raw.w[4] = load_u32(p + 16);
    raw.w[5] = load_u32(p + 20);
  }

  __device__ static void zero(Raw& raw) {
#pragma unroll
    for (int k = 0; k < 6; ++k) raw.w[k] = 0u;
    raw.shift = 0u;
  }

  // The block's fields: fp16 d bits, qh, and the 16 nibble bytes as 4 dwords.
  __device__ static void fields(const Raw& r, uint32_t& d16, uint32_t& qh, uint32_t q[4]) {
    uint32_t b[6];
#pragma unroll
    for (int k = 0; k < 5; ++k) b[k] = __builtin_amdgcn_alignbyte(r.w[k + 1], r.w[k], r.shift);
    b[5] = __builtin_amdgcn_alignbyte(0u, r.w[5], r.shift);
    d16 = b[0] & 0xFFFFu;
    qh = __builtin_amdgcn_alignbyte(b[1], b[0], 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_alignbyte(b[k + 2], b[k + 1], 2);
  }

  // codes of weights 4k..4k+3 (ca) and 16+4k..16+4k+3 (cb) as bytes 0..31
  __device__ static void codes(uint32_t qh, const uint32_t q[4], int k, uint32_t& ca, uint32_t& cb) {
    ca = (q[k] & 0x0F0F0F0Fu) | spread4_bit4(__builtin_amdgcn_ubfe(qh, 4 * k, 4));
    cb = ((q[k] >> 4) & 0x0F0F0F0Fu) | spread4_bit4(__builtin_amdgcn_ubfe(qh, 16 + 4 * k, 4));
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane&) {
    uint32_t d16, qh, q[4];
    fields(raw, d16, qh, q);
    float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t ca, cb;
      codes(qh, q, k, ca, cb);
#pragma unroll
      for (int t = 0; t < 4; t += 2) {
        s0 = __builtin_fmaf(ubyte_at(ca, t), x.v[4 * k + t], s0);
        t0 = __builtin_fmaf(ubyte_at(ca, t + 1), x.v[4 * k + t + 1], t0);
        s1 = __builtin_fmaf(ubyte_at(cb, t), x.v[16 + 4 * k + t], s1);
        t1 = __builtin_fmaf(ubyte_at(cb, t + 1), x.v[16 + 4 * k + t + 1], t1);
      }
    }
    const float sum = (s0 + t0) + (s1 + t1);
    return half_bits_to_float(d16) * __builtin_fmaf(-16.f, x.s, sum);
  }

  // Decoded form for several activation rows: w_i = d * (code_i - 16), exact.
  struct Dec {
    float w[32];
  };

  __device__ static void decode(Dec& dec, const Raw& raw, const Lane&) {
    uint32_t d16, qh, q[4];
    fields(raw, d16, qh, q);
    const float d = half_bits_to_float(d16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t ca, cb;
      codes(qh, q, k, ca, cb);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dec.w[4 * k + t] = d * (ubyte_at(ca, t) - 16.f);
        dec.w[16 + 4 * k + t] = d * (ubyte_at(cb, t) - 16.f);
      }
    }
  }

  __device__ static float dot_dec(const Dec& dec, const X& x) { return q8_block_dot_f(dec.w, x.v); }
};

// ------------------------------------------------------------- Q5_K unit
// Same unit, x handling and scale fields as Q4_K (the 32 nibble bytes of
// group g, columns 64u .. 64u + 63); bit 4 of each code comes from the 32 qh
// bytes: bit 2g of qh[l] for weight 64g + l (sub-block 2g), bit 2g + 1 for
// weight 64g + 32 + l. A rotation moves that bit of every byte to bit 4,
// and the 5-bit codes are converted one byte at a time.
struct Q5KUnit : Q4KUnit {
  using Base = Q5KUnit;
  struct Raw {
    u32x4 h, qh0, qh1, q0, q1;
  };
  struct Lane : Q4KUnit::Lane {
    uint32_t rot_a, rot_b;  // rotate-right amounts taking bit 2g / 2g+1 to bit 4
  };

  __device__ static Lane lane(int gl) {
    Lane l;
    static_cast<Q4KUnit::Lane&>(l) = Q4KUnit::lane(gl);
    l.rot_a = (2u * l.g + 28u) & 31u;
    l.rot_b = (2u * l.g + 29u) & 31u;
    return l;
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    const uint8_t* blk = row + (int64_t)(unit >> 2) * kQ5KBytes;
    const int g = unit & 3;
    raw.h = load_u32x4(blk);
    raw.qh0 = load_u32x4(blk + 16);
    raw.qh1 = load_u32x4(blk + 32);
    raw.q0 = load_u32x4(blk + 48 + 32 * g);
    raw.q1 = load_u32x4(blk + 64 + 32 * g);
  }

  __device__ static void zero(Raw& raw) {
    raw.h = raw.qh0 = raw.qh1 = raw.q0 = raw.q1 = u32x4{0, 0, 0, 0};
  }

  // 5-bit codes of weights 64g + 4k.. (ca, sub-block 2g) and 64g + 32 + 4k..
  // (cb, sub-block 2g + 1) as bytes.
  __device__ static void codes(const Raw& raw, const Lane& ln, int k, uint32_t& ca, uint32_t& cb) {
    const uint32_t w[8] = {raw.q0.x, raw.q0.y, raw.q0.z, raw.q0.w,
                           raw.q1.x, raw.q1.y, raw.q1.z, raw.q1.w};
    const uint32_t hq[8] = {raw.qh0.x, raw.qh0.y, raw.qh0.z, raw.qh0.w,
                            raw.qh1.x, raw.qh1.y, raw.qh1.z, raw.qh1.w};
    ca = (rotr(hq[k], ln.rot_a) & 0x10101010u) | (w[k] & 0x0F0F0F0Fu);
    cb = (rotr(hq[k], ln.rot_b) & 0x10101010u) | ((w[k] >> 4) & 0x0F0F0F0Fu);
  }

  __device__ static void scale_codes(const Raw& raw, const Lane& ln, float sc[2], float m[2]) {
    Q4KUnit::Raw hr;
    hr.h = raw.h;
    Q4KUnit::scales(hr, ln, sc, m);
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane& ln) {
    float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t ca, cb;
      codes(raw, ln, k, ca, cb);
      s0 = __builtin_fmaf(ubyte_at(ca, 0), x.a[4 * k + 0], s0);
      s1 = __builtin_fmaf(ubyte_at(cb, 0), x.b[4 * k + 0], s1);
      t0 = __builtin_fmaf(ubyte_at(ca, 1), x.a[4 * k + 1], t0);
      t1 = __builtin_fmaf(ubyte_at(cb, 1), x.b[4 * k + 1], t1);
      s0 = __builtin_fmaf(ubyte_at(ca, 2), x.a[4 * k + 2], s0);
      s1 = __builtin_fmaf(ubyte_at(cb, 2), x.b[4 * k + 2], s1);
      t0 = __builtin_fmaf(ubyte_at(ca, 3), x.a[4 * k + 3], t0);
      t1 = __builtin_fmaf(ubyte_at(cb, 3), x.b[4 * k + 3], t1);
    }
    s0 += t0;
    s1 += t1;
    float sc[2], m[2];
    scale_codes(raw, ln, sc, m);
    const float d = half_bits_to_float(raw.h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(raw.h.x >> 16);
    const float qs = __builtin_fmaf(sc[1], s1, sc[0] * s0);
    const float ms = __builtin_fmaf(m[1], x.sb, m[0] * x.sa);
    return __builtin_fmaf(d, qs, -dmin * ms);
  }
};

// ------------------------------------------------------------- Q6_K unit
// Unit u: super-block u >> 2, part p = u & 3 = 2n + e (n = half, e = 0/1).
// Its 64 weights are two 32-runs that share their code bytes: run a =
// weights 128n + 32e + l (low nibbles of ql[64n + 32e + l], top bits 2e and
// 2e + 1 of qh[32n + l], scales 8n + 2e + l/16) and run b = weights
// 128n + 32e + 64 + l (high nibbles of the same bytes, top bits 2e + 4 and
// 2e + 5, scales 8n + 2e + 4 + l/16). The x slices are therefore the column
// ranges [128n + 32e, +32) and [128n + 32e + 64, +32) of the super-block;
// the four parts together cover it once.
// Super-blocks are only 2-byte aligned (210 B), so each field is loaded from
// the 4-byte boundary at or below it and shifted in registers. With
// w = (d * scale) * (code - 32), a scale group of 16 weights contributes
// d * scale * (sum code * x - 32 * sum x); the four x sums are kept with x.
struct Q6KUnit {
  using Base = Q6KUnit;
  static constexpr int kPerUnitCols = 64;
  struct X {
    float a[32], b[32];
    float s[4];  // sums of a[0..15], a[16..31], b[0..15], b[16..31]
  };
  struct Raw {
    uint32_t l[9], h[9], s[3];
    uint32_t d16;
    uint32_t shift;  // 0 or 2
  };
  struct Lane {
    uint32_t n, e;
    uint32_t rot_a;   // rotate right: bits 2e, 2e+1 of each qh byte -> 4, 5
    uint32_t rot_b;   // bits 2e+4, 2e+5 -> 4, 5
    uint32_t sc_off;  // bit offset of the run's first scale in its dword (16e)
  };

  __device__ static Lane lane(int gl) {
    Lane l;
    const uint32_t p = (uint32_t)gl & 3u;
    l.n = p >> 1;
    l.e = p & 1u;
    l.rot_a = (2u * l.e + 28u) & 31u;
    l.rot_b = 2u * l.e;
    l.sc_off = 16u * l.e;
    return l;
  }

  __device__ static int col_a(int unit) {
    const int p = unit & 3;
    return (unit >> 2) * kQ6KWeights + 128 * (p >> 1) + 32 * (p & 1);
  }

  __device__ static bool valid(int unit, int units, int cols) {
    return unit < units && col_a(unit) < cols;
  }

  __device__ static void load_run(float* v, const float* xv, int c0, int cols) {
    if (c0 + 32 <= cols) {
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 t = load_f32x4(xv + c0 + i);
        v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
    }
  }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
    const int c0 = col_a(unit);
    load_run(x.a, xv, c0, cols);
    load_run(x.b, xv, c0 + 64, cols);
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x.a[i] = x.b[i] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) x.s[i] = 0.f;
  }

  __device__ static void finish_x(X& x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float sa = 0.f, sb = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sa += x.a[16 * h + i];
        sb += x.b[16 * h + i];
      }
      x.s[h] = sa;
      x.s[2 + h] = sb;
    }
  }

  // The unit's 16 x chunks: 8 of run a, then 8 of run b; in the staged x
  // of a group (4 units per super-block, 64 chunks) they sit at
  // 64 (gl >> 2) + 32n + 8e + [0, 8) and 16 chunks further on.
  static constexpr int kChunks = 16;
  __device__ static int x_chunk(int gl, int k) {
    const int p = gl & 3;
    return 64 * (gl >> 2) + 32 * (p >> 1) + 8 * (p & 1) + k + (k >= 8 ? 8 : 0);
  }
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x.a[4 * k] = c[k].x; x.a[4 * k + 1] = c[k].y; x.a[4 * k + 2] = c[k].z; x.a[4 * k + 3] = c[k].w;
      x.b[4 * k] = c[8 + k].x; x.b[4 * k + 1] = c[8 + k].y;
      x.b[4 * k + 2] = c[8 + k].z; x.b[4 * k + 3] = c[8 + k].w;
    }
  }

  __device__ static void load9(uint32_t (&w)[9], const uint8_t* p) {
    const u32x4 v0 = load_u32x4(p);
    const u32x4 v1 = load_u32x4(p + 16);
    w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
    w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    w[8] = load_u32(p + 32);
  }

  __device__ static void load(Raw& raw, const uint8_t* row, int unit) {
    const uint8_t* blk = row + (int64_t)(unit >> 2) * kQ6KBytes;
    const int p = unit & 3, n = p >> 1, e = p & 1;
    raw.shift = (uint32_t)((uintptr_t)blk & 3u);
    const uint8_t* base = blk - raw.shift;  // pointer arithmetic keeps global loads
    load9(raw.l, base + 64 * n + 32 * e);
    load9(raw.h, base + 128 + 32 * n);
    const uint8_t* sp = base + 192 + 8 * n;
    raw.s[0] = load_u32(sp);
    raw.s[1] = load_u32(sp + 4);
    raw.s[2] = load_u32(sp + 8);
    raw.d16 = load_u16(blk + 208);
  }

  __device__ static void zero(Raw& raw) {
#pragma unroll
    for (int k = 0; k < 9; ++k) raw.l[k] = raw.h[k] = 0u;
    raw.s[0] = raw.s[1] = raw.s[2] = 0u;
    raw.d16 = 0u;
    raw.shift = 0u;
  }

  // 6-bit codes of run a (ca) and run b (cb), weights 4k..4k+3, as bytes.
  __device__ static void codes(const Raw& raw, const Lane& ln, int k, uint32_t& ca, uint32_t& cb) {
    const uint32_t L = __builtin_amdgcn_alignbyte(raw.l[k + 1], raw.l[k], raw.shift);
    const uint32_t H = __builtin_amdgcn_alignbyte(raw.h[k + 1], raw.h[k], raw.shift);
    ca = (rotr(H, ln.rot_a) & 0x30303030u) | (L & 0x0F0F0F0Fu);
    cb = (rotr(H, ln.rot_b) & 0x30303030u) | ((L >> 4) & 0x0F0F0F0Fu);
  }

  // The four int8 scales of the unit: a0, a1, b0, b1.
  __device__ static void scales(const Raw& raw, const Lane& ln, float sc[4]) {
    const uint32_t s0 = __builtin_amdgcn_alignbyte(raw.s[1], raw.s[0], raw.shift);
    const uint32_t s1 = __builtin_amdgcn_alignbyte(raw.s[2], raw.s[1], raw.shift);
    // signed bytes through int8_t: a signed bit-field builtin here was
    // converted to float as unsigned by the compiler
    sc[0] = (float)(int8_t)(s0 >> ln.sc_off);
    sc[1] = (float)(int8_t)(s0 >> (ln.sc_off + 8));
    sc[2] = (float)(int8_t)(s1 >> ln.sc_off);
    sc[3] = (float)(int8_t)(s1 >> (ln.sc_off + 8));
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane& ln) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};  // a0, a1, b0, b1
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t ca, cb;
      codes(raw, ln, k, ca, cb);
      const int h = k >> 2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[h] = __builtin_fmaf(ubyte_at(ca, t), x.a[4 * k + t], acc[h]);
        acc[2 + h] = __builtin_fmaf(ubyte_at(cb, t), x.b[4 * k + t], acc[2 + h]);
      }
    }
    float sc[4];
    scales(raw, ln, sc);
    float r = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) r = __builtin_fmaf(sc[q], __builtin_fmaf(-32.f, x.s[q], acc[q]), r);
    return half_bits_to_float(raw.d16) * r;
  }
};

// ------------------------------------------------ Q8_0 split-layout unit
// Rows repacked so that the fp16 scales come first (split_scale_bytes(nb))
// and the codes follow in block order. Lane gl of a G-lane row group owns the
// 16-code chunks c_j = 4G * segment + gl + j G (j < 4): every 16-byte load of
// a wave reads one contiguous run of the row's codes. Chunk c holds columns
// 16c .. 16c + 15 and uses the scale of block c / 2. The scale region's size
// depends on the row length, so the kernels pass the column count to lane().
template <int G>
struct Q8SplitUnit {
  using Base = Q8SplitUnit<G>;
  static constexpr bool kWantsCols = true;
  static constexpr bool kQ8Like = true;
  static constexpr int kPerUnitCols = 64;
  struct X {
    float v[64];  // chunk j's 16 values at v[16 j ..]
  };
  struct Raw {
    u32x4 c[4];
    uint32_t d16[4];
  };
  struct Lane {
    int scale_bytes;  // offset of the codes in a row
    int nchunk;       // 16-code chunks per row
  };

  __device__ static Lane lane(int, int cols) {
    const int nb = (cols + 31) / 32;
    return Lane{split_scale_bytes(nb), 2 * nb};
  }

  __device__ static int chunk0(int unit) { return (unit / G) * 4 * G + unit % G; }

  __device__ static bool valid(int unit, int units, int cols) {
    return unit < units && 16 * chunk0(unit) < cols;
  }

  __device__ static void load_x(X& x, const float* xv, int unit, int cols) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = 16 * (chunk0(unit) + j * G);
      if (c0 + 16 <= cols) {
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const f32x4 t = load_f32x4(xv + c0 + i);
          x.v[16 * j + i] = t.x; x.v[16 * j + i + 1] = t.y; x.v[16 * j + i + 2] = t.z; x.v[16 * j + i + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x.v[16 * j + i] = (c0 + i < cols) ? xv[c0 + i] : 0.f;
      }
    }
  }

  __device__ static void zero_x(X& x) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x.v[i] = 0.f;
  }

  __device__ static void finish_x(X&) {}

  static constexpr int kChunks = 16;
  __device__ static int x_chunk(int gl, int k) { return 4 * (gl + (k >> 2) * G) + (k & 3); }
  __device__ static void set_x(X& x, const f32x4 (&c)[kChunks]) {
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      x.v[4 * k] = c[k].x; x.v[4 * k + 1] = c[k].y; x.v[4 * k + 2] = c[k].z; x.v[4 * k + 3] = c[k].w;
    }
  }

  // Chunks past the row's end read its last chunk (their x is zero).
  __device__ static void load(Raw& raw, const uint8_t* row, int unit, const Lane& ln) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int c = chunk0(unit) + j * G;
      c = c < ln.nchunk ? c : ln.nchunk - 1;
      raw.c[j] = load_u32x4(row + ln.scale_bytes + 16 * c);
      raw.d16[j] = load_u16(row + 2 * (c >> 1));
    }
  }

  __device__ static void zero(Raw& raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      raw.c[j] = u32x4{0, 0, 0, 0};
      raw.d16[j] = 0u;
    }
  }

  __device__ static float dot(const Raw& raw, const X& x, const Lane&) {
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {raw.c[j].x, raw.c[j].y, raw.c[j].z, raw.c[j].w};
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          s0 = __builtin_fmaf(i8_at(w[k], b), x.v[16 * j + 4 * k + b], s0);
          s1 = __builtin_fmaf(i8_at(w[k + 1], b), x.v[16 * j + 4 * k + 4 + b], s1);
        }
      }
      r = __builtin_fmaf(half_bits_to_float(raw.d16[j]), s0 + s1, r);
    }
    return r;
  }
};

}  // namespace gq
