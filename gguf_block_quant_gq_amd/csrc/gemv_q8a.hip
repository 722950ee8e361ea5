// gemv_q8a.hip -- the int8-activation decode path: activations quantised
// per 32 values into Q8_1 blocks, then y = W x^ with integer dot products.
//
// The Loom porting skill ("What the starter generates", the gen_llm.py row)
// runs its decode-shaped linears with int8 activations in llama.cpp's Q8_1
// numerics and 4-way integer dot products, keeping an fp32-activation switch.
// The page names the numerics without printing them; the public Q8_1 block
// is the reading taken (per 32 values: d = amax / 127, codes rounded half
// away from zero from x * (1 / d), then fp16 d, fp16 d * sum q and 32 int8
// codes, 36 bytes). The product is W x^ with x^ = fp16(d) * q.
//
// quantize_q8_1_kernel: eight lanes per block (four values each); the block
// max and the code sum go through a 3-step DPP butterfly.
//
// gemv_q8a_reg_kernel (rows of up to 256 units: Q4_K up to 16384 columns,
// Q8_0 up to 8192): groups of G lanes (the row's units rounded up to a power
// of two, 16..64) own a row each, two rows in flight; lane l owns units
// l, l + G, ... (a Q8_0 block, or a quarter of a Q4_K super-block: 64
// weights) and keeps their activation codes, scales and code sums in
// registers for every row it visits. Measured on MI355X against the fp32
// matvec (us, 4 workgroups per CU): Llama q 4096x4096 3.98 / 4.20, gate
// 14336x4096 8.19 / 8.14, down 4096x14336 10.71 / 9.99, Q8_0 lm_head
// 151936x896 28.4 / 25.9.
//
// gemv_q8a_kernel (wider rows): every workgroup stages the whole quantised
// activation row in LDS (codes, the fp32 scale and the exact code sum of
// every 32-value block); each wave then walks rows, its lanes taking the
// row's units in turn, two rows in flight.
//
// Per unit the weight codes meet the activation codes in
// v_dot4_i32_i8 (Q4_K nibbles are 0..15, exact as int8), giving exact int32
// sums per 32 weights; the scales are applied in fp32:
//   Q8_0: (d_w * d_x) * sum q_w q_x
//   Q4_K: d * ((sc_a sum_a) d_xa + (sc_b sum_b) d_xb)
//         - dmin * ((m_a Q_a) d_xa + (m_b Q_b) d_xb)
// with Q the activation code sums of the two sub-blocks (sc, m <= 63 and the
// sums <= 60960 keep every integer product below 2^24). The lanes' partial
// sums are folded with the DPP butterfly (fixed order).
#include "gemv_common.h"
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kQ81Bytes = 36;
constexpr int kQ81Values = 32;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_bits(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Max of non-negative floats and sum of ints over aligned groups of 8 lanes
// (every lane of the group gets the result).
__device__ __forceinline__ float group8_max(float v) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  b = max(b, dpp_bits<0xB1>(b));   // quad_perm [1,0,3,2]
  b = max(b, dpp_bits<0x4E>(b));   // quad_perm [2,3,0,1]
  b = max(b, dpp_bits<0x141>(b));  // row_half_mirror
  return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ int group8_sum(int v) {
  v += (int)dpp_bits<0xB1>((uint32_t)v);
  v += (int)dpp_bits<0x4E>((uint32_t)v);
  v += (int)dpp_bits<0x141>((uint32_t)v);
  return v;
}

__device__ __forceinline__ uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// n rows of cols activations -> n rows of nb Q8_1 blocks (row stride nb * 36).
__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float* x, uint8_t* out, int64_t n,
                                                            int cols, int nb) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 3;
  if (blk >= n * nb) return;  // whole 8-lane groups leave together
  const int sub = (int)(t & 7);
  const int64_t r = blk / nb;
  const int b = (int)(blk - r * nb);
  const int c0 = b * kQ81Values + 4 * sub;
  const float* xr = x + r * cols;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = c0 + e < cols ? xr[c0 + e] : 0.f;
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = group8_max(amax);
  const float d = amax / 127.0f;
  const float id = d != 0.f ? 1.0f / d : 0.f;
  int q[4], s = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // clamped to +-127, NaN to 0: only a block whose 1 / d overflows (max
    // |x| under about 3.7e-37) reaches these cases (its products are +-inf,
    // or NaN for x = 0); every other product rounds to at most 127
    const float p = v[e] * id;
    q[e] = p != p ? 0 : (int)roundf(fminf(fmaxf(p, -127.f), 127.f));
    s += q[e];
  }
  s = group8_sum(s);
  uint8_t* ob = out + blk * kQ81Bytes;
  const uint32_t codes = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
                         ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
  *(uint32_t*)(ob + 4 + 4 * sub) = codes;
  if (sub == 0) *(uint32_t*)ob = f16_bits(d) | (f16_bits((float)s * d) << 16);
}

struct Q8aArgs {
  const uint8_t* W;
  const uint8_t* xq;
  float* y;
  int64_t row_bytes;
  int rows, cols;
  int nb;     // Q8_1 blocks of the activation row
  int nbx;    // blocks staged in LDS (Q4_K: whole super-blocks, zero-filled)
  int units;  // units per weight row
};

// The LDS image of the activation row: codes (nbx * 32 bytes), then the fp32
// scale of every block, then its exact code sum.
struct XView {
  const uint32_t* codes;
  const float* d;
  const int* qs;
};

__device__ __forceinline__ XView stage_x(const Q8aArgs& a, uint8_t* lds) {
  uint32_t* codes = (uint32_t*)lds;
  float* d = (float*)(lds + a.nbx * kQ81Values);
  int* qs = (int*)(d + a.nbx);
  // one dword per thread: word 0 of a block is d|s, words 1..8 its codes
  for (int i = threadIdx.x; i < a.nbx * 9; i += 256) {
    const int b = i / 9, w = i - 9 * b;
    const uint32_t v = b < a.nb ? *(const uint32_t*)(a.xq + (int64_t)b * kQ81Bytes + 4 * w) : 0u;
    if (w == 0) d[b] = half_bits_to_float(v & 0xFFFFu);
    else codes[8 * b + w - 1] = v;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.nbx; b += 256) {
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4((int)codes[8 * b + k], 0x01010101, s, false);
    qs[b] = s;
  }
  __syncthreads();
  return XView{codes, d, qs};
}

__device__ __forceinline__ u32x4 lds_u32x4(const uint32_t* p) { return *(const u32x4*)p; }

// ---------------------------------------------------------------- Q8_0 --
struct Q8aQ8 {
  struct Raw {
    Q8Raw r;
  };
  struct Lane {};
  __device__ static Lane lane(int) { return Lane{}; }
  // A lane's activation data for one unit (its Q8_1 block), in registers.
  struct XU {
    uint32_t c[8];
    float d;
  };
  __device__ static void load_xu(XU& x, const uint8_t* xq, int u, int nb) {
    const bool valid = u < nb;
    const uint8_t* b = xq + (int64_t)(valid ? u : 0) * kQ81Bytes;
    const u32x4 c0 = valid ? load_u32x4(b + 4) : u32x4{0, 0, 0, 0};
    const u32x4 c1 = valid ? load_u32x4(b + 20) : u32x4{0, 0, 0, 0};
    x.c[0] = c0.x; x.c[1] = c0.y; x.c[2] = c0.z; x.c[3] = c0.w;
    x.c[4] = c1.x; x.c[5] = c1.y; x.c[6] = c1.z; x.c[7] = c1.w;
    x.d = valid ? half_bits_to_float(load_u16(b)) : 0.f;
  }
  __device__ static float dot_xu(const Raw& raw, const XU& x, const Lane&) {
    uint32_t q[8];
    q8_codes(raw.r, q);
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4((int)q[k], (int)x.c[k], s, false);
    return (half_bits_to_float(raw.r.d16) * x.d) * (float)s;
  }
  __device__ static void load(Raw& raw, const uint8_t* row, int u) { q8_load(row + (int64_t)u * kQ8Bytes, raw.r); }
  __device__ static float dot(const Raw& raw, const XView& x, int u, const Lane&) {
    uint32_t q[8];
    q8_codes(raw.r, q);
    const u32x4 x0 = lds_u32x4(x.codes + 8 * u), x1 = lds_u32x4(x.codes + 8 * u + 4);
    const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4((int)q[k], (int)xv[k], s, false);
    return (half_bits_to_float(raw.r.d16) * x.d[u]) * (float)s;
  }
};

// ---------------------------------------------------------------- Q4_K --
// Unit u: super-block u / 4, code group g = u % 4 (sub-blocks 2g, 2g + 1).
struct Q8aQ4K {
  struct Raw {
    u32x4 h, q0, q1;
  };
  struct Lane {
    Q4Sel sel;
  };
  // lanes step through the units by a multiple of 4, so a lane's group is lane % 4
  __device__ static Lane lane(int l) { return Lane{q4_sel(l & 3)}; }
  // A lane's activation data for one unit: the Q8_1 blocks of sub-blocks
  // 2u and 2u + 1 (codes, scales, exact code sums), in registers.
  struct XU {
    uint32_t a[8], b[8];
    float da, db;
    int qa, qb;
  };
  // Blocks at or past nb (the row's tail beyond cols, or a lane without a
  // unit) are not read: their codes and scales are zero.
  __device__ static void load_xu(XU& x, const uint8_t* xq, int u, int nb) {
    const bool va = 2 * u < nb, vb = 2 * u + 1 < nb;
    const uint8_t* ba = xq + (int64_t)(va ? 2 * u : 0) * kQ81Bytes;
    const uint8_t* bb = xq + (int64_t)(vb ? 2 * u + 1 : 0) * kQ81Bytes;
    const u32x4 z = {0, 0, 0, 0};
    const u32x4 a0 = va ? load_u32x4(ba + 4) : z, a1 = va ? load_u32x4(ba + 20) : z;
    const u32x4 b0 = vb ? load_u32x4(bb + 4) : z, b1 = vb ? load_u32x4(bb + 20) : z;
    x.a[0] = a0.x; x.a[1] = a0.y; x.a[2] = a0.z; x.a[3] = a0.w;
    x.a[4] = a1.x; x.a[5] = a1.y; x.a[6] = a1.z; x.a[7] = a1.w;
    x.b[0] = b0.x; x.b[1] = b0.y; x.b[2] = b0.z; x.b[3] = b0.w;
    x.b[4] = b1.x; x.b[5] = b1.y; x.b[6] = b1.z; x.b[7] = b1.w;
    x.da = va ? half_bits_to_float(load_u16(ba)) : 0.f;
    x.db = vb ? half_bits_to_float(load_u16(bb)) : 0.f;
    int qa = 0, qb = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      qa = __builtin_amdgcn_sdot4((int)x.a[k], 0x01010101, qa, false);
      qb = __builtin_amdgcn_sdot4((int)x.b[k], 0x01010101, qb, false);
    }
    x.qa = qa;
    x.qb = qb;
  }
  __device__ static float dot_xu(const Raw& raw, const XU& x, const Lane& ln) {
    const uint32_t w[8] = {raw.q0.x, raw.q0.y, raw.q0.z, raw.q0.w, raw.q1.x, raw.q1.y, raw.q1.z, raw.q1.w};
    int sa = 0, sb = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sa = __builtin_amdgcn_sdot4((int)(w[k] & 0x0F0F0F0Fu), (int)x.a[k], sa, false);
      sb = __builtin_amdgcn_sdot4((int)((w[k] >> 4) & 0x0F0F0F0Fu), (int)x.b[k], sb, false);
    }
    return combine(raw, ln, sa, sb, x.da, x.db, x.qa, x.qb);
  }
  __device__ static float combine(const Raw& raw, const Lane& ln, int sa, int sb, float dxa, float dxb, int qa,
                                  int qb) {
    const uint32_t scm = q4_scales(raw.h, ln.sel);  // sc_a, sc_b, m_a, m_b bytes
    const int sc_a = (int)(scm & 0xFFu), sc_b = (int)((scm >> 8) & 0xFFu);
    const int m_a = (int)((scm >> 16) & 0xFFu), m_b = (int)(scm >> 24);
    const float t = (float)(sc_a * sa) * dxa + (float)(sc_b * sb) * dxb;
    const float m = (float)(m_a * qa) * dxa + (float)(m_b * qb) * dxb;
    const float d = half_bits_to_float(raw.h.x & 0xFFFFu), dmin = half_bits_to_float(raw.h.x >> 16);
    return d * t - dmin * m;
  }
  __device__ static void load(Raw& raw, const uint8_t* row, int u) {
    const uint8_t* blk = row + (int64_t)(u >> 2) * kQ4KBytes;
    const int g = u & 3;
    raw.h = load_u32x4(blk);
    raw.q0 = load_u32x4(blk + 16 + 32 * g);
    raw.q1 = load_u32x4(blk + 32 + 32 * g);
  }
  __device__ static float dot(const Raw& raw, const XView& x, int u, const Lane& ln) {
    const int ja = 2 * u;  // sub-block index of the first half: 8 (u / 4) + 2 (u % 4)
    const uint32_t w[8] = {raw.q0.x, raw.q0.y, raw.q0.z, raw.q0.w, raw.q1.x, raw.q1.y, raw.q1.z, raw.q1.w};
    const u32x4 a0 = lds_u32x4(x.codes + 8 * ja), a1 = lds_u32x4(x.codes + 8 * ja + 4);
    const u32x4 b0 = lds_u32x4(x.codes + 8 * ja + 8), b1 = lds_u32x4(x.codes + 8 * ja + 12);
    const uint32_t xa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t xb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    int sa = 0, sb = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sa = __builtin_amdgcn_sdot4((int)(w[k] & 0x0F0F0F0Fu), (int)xa[k], sa, false);
      sb = __builtin_amdgcn_sdot4((int)((w[k] >> 4) & 0x0F0F0F0Fu), (int)xb[k], sb, false);
    }
    return combine(raw, ln, sa, sb, x.d[ja], x.d[ja + 1], x.qs[ja], x.qs[ja + 1]);
  }
};

// Waves walk rows in pairs (p = global wave + k * total waves: rows 2p, 2p + 1),
// the second row of a pair past the end re-reads the first and drops it.
template <class F>
__global__ __launch_bounds__(256) void gemv_q8a_kernel(Q8aArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const XView x = stage_x(a, lds);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nw = gridDim.x * 4;
  const typename F::Lane ln = F::lane(lane);
  const int pairs = (a.rows + 1) / 2;
  for (int p = gw; p < pairs; p += nw) {
    const int r0 = 2 * p, r1 = min(2 * p + 1, a.rows - 1);
    const uint8_t* w0 = a.W + (int64_t)r0 * a.row_bytes;
    const uint8_t* w1 = a.W + (int64_t)r1 * a.row_bytes;
    float s0 = 0.f, s1 = 0.f;
    for (int u = lane; u < a.units; u += 64) {
      typename F::Raw ra, rb;
      F::load(ra, w0, u);
      F::load(rb, w1, u);
      s0 += F::dot(ra, x, u, ln);
      s1 += F::dot(rb, x, u, ln);
    }
    s0 = group_sum_last<64>(s0);
    s1 = group_sum_last<64>(s1);
    if (lane == 63) {
      a.y[r0] = s0;
      if (2 * p + 1 < a.rows) a.y[r1] = s1;
    }
  }
}

// Register form, for rows of at most 4 G units: groups of G lanes own a row
// each (RB rows in flight); lane gl owns units gl, gl + G, ... (UL of them)
// and keeps their activation data in registers for every row it visits.
// Lanes whose unit lies past the row read the row's last unit with zero
// activations (no predicated loads).
template <class F, int G, int UL, int RB>
__global__ __launch_bounds__(256) void gemv_q8a_reg_kernel(Q8aArgs a) {
  static_assert(G >= 4 && G <= 64 && (G & (G - 1)) == 0, "G");
  constexpr int kGroups = 256 / G;
  const int gl = threadIdx.x % G;
  const int grp = blockIdx.x * kGroups + threadIdx.x / G;
  const int ngrp = gridDim.x * kGroups;
  const typename F::Lane ln = F::lane(gl);
  typename F::XU xu[UL];
  int uld[UL];  // the unit each lane loads (clamped to a real one)
#pragma unroll
  for (int k = 0; k < UL; ++k) {
    const int u = gl + k * G;
    F::load_xu(xu[k], a.xq, u < a.units ? u : a.units, a.nb);  // past the units: no blocks
    uld[k] = u < a.units ? u : a.units - 1;
  }
  for (int r0 = grp * RB; r0 < a.rows; r0 += ngrp * RB) {
    typename F::Raw raw[RB][UL];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int row = min(r0 + i, a.rows - 1);
      const uint8_t* wr = a.W + (int64_t)row * a.row_bytes;
#pragma unroll
      for (int k = 0; k < UL; ++k) F::load(raw[i][k], wr, uld[k]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < UL; ++k) s += F::dot_xu(raw[i][k], xu[k], ln);
      s = group_sum_last<G>(s);
      if (gl == G - 1 && r0 + i < a.rows) a.y[r0 + i] = s;
    }
  }
}

}  // namespace

hipError_t launch_quantize_q8_1(const float* x, int64_t n, int cols, uint8_t* out, hipStream_t s) {
  const int nb = (cols + kQ81Values - 1) / kQ81Values;
  const int64_t threads = n * nb * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, out, n, cols, nb);
  return hipGetLastError();
}

#ifndef GQ_Q8A_WG_PER_CU
#define GQ_Q8A_WG_PER_CU 2  // each workgroup stages the whole activation row
#endif

// The largest staged row: 131072 columns = 4096 blocks of 32 codes + 8 bytes
// (the host rejects wider rows), which is all 160 KB of a CU's LDS.
constexpr int kQ8aMaxLds = 4096 * (kQ81Values + 8);

template <class F>
hipError_t launch_q8a(const Q8aArgs& a, int grid, int lds, hipStream_t s) {
  if (lds > kQ8aMaxLds) return hipErrorInvalidValue;
  // LDS past the default 64 KB per workgroup must be requested; every call
  // requests the same maximum, so calls from several host threads cannot
  // lower the limit under one another's launch
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)gemv_q8a_kernel<F>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kQ8aMaxLds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gemv_q8a_kernel<F>, dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

#ifndef GQ_Q8A_REG_WG_PER_CU
#define GQ_Q8A_REG_WG_PER_CU 4
#endif
#ifndef GQ_Q8A_RB
#define GQ_Q8A_RB 2
#endif

template <class F, int G, int UL>
hipError_t launch_reg(const Q8aArgs& a, int cus, hipStream_t s) {
  constexpr int RB = GQ_Q8A_RB;
  const int64_t groups = (a.rows + RB - 1) / RB;
  const int grid = (int)min((groups + 256 / G - 1) / (256 / G), (int64_t)cus * GQ_Q8A_REG_WG_PER_CU);
  hipLaunchKernelGGL((gemv_q8a_reg_kernel<F, G, UL, RB>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Lanes per row: the units rounded up to a power of two (at least 16), up
// to 64; then up to 4 units per lane.
template <class F>
hipError_t launch_reg_any(const Q8aArgs& a, int cus, hipStream_t s) {
  if (a.units <= 16) return launch_reg<F, 16, 1>(a, cus, s);
  if (a.units <= 32) return launch_reg<F, 32, 1>(a, cus, s);
  if (a.units <= 64) return launch_reg<F, 64, 1>(a, cus, s);
  if (a.units <= 128) return launch_reg<F, 64, 2>(a, cus, s);
  if (a.units <= 192) return launch_reg<F, 64, 3>(a, cus, s);
  return launch_reg<F, 64, 4>(a, cus, s);
}

hipError_t launch_gemv_q8a(int fmt, const uint8_t* W, int64_t row_bytes, int rows, int cols,
                           const uint8_t* xq, float* y, int cus, hipStream_t s) {
  Q8aArgs a{W, xq, y, row_bytes, rows, cols, (cols + 31) / 32, 0, 0};
  if (fmt == kFmtQ4_K && 4 * ((cols + 255) / 256) <= 256) {
    a.units = 4 * ((cols + 255) / 256);
    return launch_reg_any<Q8aQ4K>(a, cus, s);
  }
  if (fmt == kFmtQ8_0 && a.nb <= 256) {
    a.units = a.nb;
    return launch_reg_any<Q8aQ8>(a, cus, s);
  }
  const int pairs = (rows + 1) / 2;
  const int grid = (int)min((int64_t)(pairs + 3) / 4, (int64_t)cus * GQ_Q8A_WG_PER_CU);
  if (fmt == kFmtQ4_K) {
    a.nbx = 8 * ((cols + 255) / 256);
    a.units = 4 * ((cols + 255) / 256);
    return launch_q8a<Q8aQ4K>(a, grid, a.nbx * (kQ81Values + 8), s);
  }
  if (fmt == kFmtQ8_0) {
    a.nbx = a.nb;
    a.units = a.nb;
    return launch_q8a<Q8aQ8>(a, grid, a.nbx * (kQ81Values + 8), s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gq
