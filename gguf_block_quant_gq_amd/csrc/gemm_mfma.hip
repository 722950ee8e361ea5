// gemm_mfma.hip -- Y = X W^T for Q4_K weights and M >= 16 activation rows,
// on the gfx950 matrix cores (v_mfma_f32_16x16x32_f16).
//
// The prompt-chunk product ("nurllama 0.18.1 API", model.nu section: the
// matmuls run over a chunk of positions at once, each weight read once per
// chunk) is a real dense contraction once M >= 16.
//
// Exactness. A Q4_K super-block contributes, per output,
//   d * sum_j sc_j * sum_{c in j} code_c * x_c  -  dmin * sum_j m_j * X_j
// with X_j the sum of x over sub-block j. The matrix-core operands are chosen
// so that every product is exact:
//   * A = sc_j * code_c, an integer <= 945, is exact in fp16;
//   * the 256 x values of one row and super-block are scaled by a power of
//     two (so the largest has magnitude in [2^9, 2^10)) and split into fp16
//     hi + lo parts, x' = hi + lo to about 2^-22 relative; both parts are
//     multiplied, so sum code*sc*x' is accumulated in fp32 from exact
//     products;
//   * the min term is one more matrix-core product per super-block with
//     A2 = m_j (exact) and B2 = the fp16 hi/lo parts of the scaled X_j.
// d, dmin and the power of two are applied per super-block in fp32. The
// result therefore meets the same accuracy bound as the fp32 paths for any
// finite input (no overflow or underflow of the fp16 parts).
//
// Work decomposition: a workgroup of WAVES waves owns 16*WAVES rows and
// 16*MT activation rows; wave w owns rows 16w..16w+15 and all MT m-tiles.
// Per super-block the workgroup stages its x block into LDS once (scaled,
// split, sub-block sums), each wave loads the packed bytes of its 16 rows
// (lane (i, q) reads bytes 8q..8q+7 of each 32-byte code group of row i,
// exactly the k range its A operand needs), builds A in registers and runs
// 2*8*MT + 2*MT MFMAs.
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kXStride = 256 + 8;  // halves per staged x row (padding breaks bank conflicts)

// Within each group of 8 k, the A operand holds the codes of bytes in the
// order 0,2,1,3,4,6,5,7 (that is how the nibble pairs are extracted); the
// staged x uses the same order. The permutation is its own inverse.
__device__ __forceinline__ int kslot(int k) {
  const int e = k & 7;
  const int p = (e == 1 || e == 5) ? e + 1 : (e == 2 || e == 6) ? e - 1 : e;
  return (k & ~7) | p;
}

// Four packed fp16 pairs (1024 + code) from the low (H = 0) or high (H = 1)
// nibbles of 8 code bytes, then sc * code exactly:
// fma((1024 + c), sc, -1024 sc) = c * sc is representable, so the single
// rounding of the fma is exact.
template <int H>
__device__ __forceinline__ h8 build_a(uint32_t w0, uint32_t w1, h2 sc, h2 nsc) {
  constexpr uint32_t M = 0x000F000Fu, MAGIC = 0x64006400u;
  uint32_t p[4];
  p[0] = ((w0 >> (4 * H)) & M) | MAGIC;
  p[1] = ((w0 >> (8 + 4 * H)) & M) | MAGIC;
  p[2] = ((w1 >> (4 * H)) & M) | MAGIC;
  p[3] = ((w1 >> (8 + 4 * H)) & M) | MAGIC;
  h8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 v = __builtin_bit_cast(h2, p[i]);
    const h2 o = __builtin_elementwise_fma(v, sc, nsc);
    r[2 * i] = o[0];
    r[2 * i + 1] = o[1];
  }
  return r;
}

__device__ __forceinline__ float dpp_max8(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  return v;
}

template <int WAVES, int MT>
struct Smem {
  _Float16 xh[16 * MT][kXStride];
  _Float16 xl[16 * MT][kXStride];
  _Float16 sh[16 * MT][8];  // scaled sub-block sums, hi
  _Float16 sl[16 * MT][8];  // and lo
  int sexp[16 * MT];        // power-of-two exponent of the row's x block
  float2 dd[WAVES][16];     // (d, dmin) of each wave's 16 rows
};

// Stage x[m0 .. m0+BM) x [256 sb, 256 sb + 256) into LDS. Thread t handles
// (m, j) = (t / 8, t % 8): 32 consecutive columns of one row.
template <int WAVES, int MT>
__device__ __forceinline__ void stage_x(Smem<WAVES, MT>& sm, const GemmArgs& a, int m0, int sb) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kItems = 16 * MT * 8;
  for (int t = threadIdx.x; t < (kItems + kThreads - 1) / kThreads * kThreads; t += kThreads) {
    const bool live = t < kItems;
    const int m = t >> 3, j = t & 7;
    const int gm = m0 + m;
    const int c0 = 256 * sb + 32 * j;
    float v[32];
    if (live && gm < a.M && c0 + 32 <= a.cols) {
      const float* src = a.X + (int64_t)gm * a.cols + c0;
#pragma unroll
      for (int i = 0; i < 32; i += 4) {
        const f32x4 t4 = load_f32x4(src + i);
        v[i] = t4.x; v[i + 1] = t4.y; v[i + 2] = t4.z; v[i + 3] = t4.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        v[i] = (live && gm < a.M && c0 + i < a.cols) ? a.X[(int64_t)gm * a.cols + c0 + i] : 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = dpp_max8(mx);  // the 8 lanes of one row hold its 256 columns
    // largest |x'| in [2^9, 2^10): exponent e = 9 - ilogb(max)
    int e = 0;
    if (mx > 0.f) {
      const int be = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF);
      e = 136 - (be == 0 ? 1 : be);
      e = e > 126 ? 126 : (e < -126 ? -126 : e);
    }
    if (!live) continue;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      h8 hh, ll;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float xs = __builtin_ldexpf(v[i + u], e);
        const _Float16 h = (_Float16)xs;
        hh[u] = h;
        ll[u] = (_Float16)(xs - (float)h);
        s += xs;
      }
      // write in the permuted k order used by the A operand
      h8 ph, pl;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ph[kslot(u)] = hh[u];
        pl[kslot(u)] = ll[u];
      }
      *(h8*)&sm.xh[m][32 * j + i] = ph;
      *(h8*)&sm.xl[m][32 * j + i] = pl;
    }
    const _Float16 shh = (_Float16)s;
    sm.sh[m][j] = shh;
    sm.sl[m][j] = (_Float16)(s - (float)shh);
    if (j == 0) sm.sexp[m] = e;
  }
}

template <int WAVES, int MT>
__global__ __launch_bounds__(64 * WAVES) void gemm_q4k_mfma_kernel(GemmArgs a) {
  __shared__ Smem<WAVES, MT> sm;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;   // A row / B column / D column within the tile
  const int q = lane >> 4;   // k sub-range 8q..8q+7
  const int row0 = blockIdx.x * (16 * WAVES) + 16 * wave;
  const int m0 = blockIdx.y * (16 * MT);
  const int nsb = (a.cols + 255) / 256;

  const int my_row = row0 + i < a.rows ? row0 + i : a.rows - 1;  // clamped for loads
  const uint8_t* wrow = a.W + (int64_t)my_row * a.row_bytes;

  f4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int sb = 0; sb < nsb; ++sb) {
    // ---- this wave's packed bytes: 4 x 8 code bytes and the 16-byte header
    const uint8_t* blk = wrow + (int64_t)sb * kQ4KBytes;
    uint32_t cw[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 v;
      __builtin_memcpy(&v, __builtin_assume_aligned(blk + 16 + 32 * g + 8 * q, 4), 8);
      cw[2 * g] = v.x;
      cw[2 * g + 1] = v.y;
    }
    const u32x4 hd = load_u32x4(blk);

    stage_x<WAVES, MT>(sm, a, m0, sb);

    // ---- header: d, dmin, the 8 scale and min codes of row i
    const float d = half_bits_to_float(hd.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hd.x >> 16);
    if (q == 0) sm.dd[wave][i] = make_float2(d, dmin);
    uint32_t sc[8], mc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = (hd.y >> (8 * j)) & 63u;
      mc[j] = (hd.z >> (8 * j)) & 63u;
      sc[j + 4] = ((hd.w >> (8 * j)) & 15u) | (((hd.y >> (8 * j + 6)) & 3u) << 4);
      mc[j + 4] = ((hd.w >> (8 * j + 4)) & 15u) | (((hd.z >> (8 * j + 6)) & 3u) << 4);
    }
    __syncthreads();

    // ---- main term: 8 sub-blocks x (hi, lo)
    f4 p1[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) p1[t] = zero4;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const _Float16 scf = (_Float16)(float)sc[s];
      const h2 sc2 = {scf, scf};
      const _Float16 nscf = (_Float16)(-1024.0f * (float)sc[s]);
      const h2 nsc2 = {nscf, nscf};
      const uint32_t w0 = cw[2 * (s >> 1)], w1 = cw[2 * (s >> 1) + 1];
      const h8 A = (s & 1) ? build_a<1>(w0, w1, sc2, nsc2) : build_a<0>(w0, w1, sc2, nsc2);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const h8 bh = *(const h8*)&sm.xh[16 * t + i][32 * s + 8 * q];
        const h8 bl = *(const h8*)&sm.xl[16 * t + i][32 * s + 8 * q];
        p1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh, p1[t], 0, 0, 0);
        p1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl, p1[t], 0, 0, 0);
      }
    }

    // ---- min term: A2 = m_j at k = j (lanes q == 0), B2 = X_j parts
    h8 A2;
#pragma unroll
    for (int j = 0; j < 8; ++j) A2[j] = q == 0 ? (_Float16)(float)mc[j] : (_Float16)0.f;
    f4 p2[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      h8 bh = *(const h8*)&sm.sh[16 * t + i][0];
      h8 bl = *(const h8*)&sm.sl[16 * t + i][0];
      if (q != 0) {
        bh = h8{0, 0, 0, 0, 0, 0, 0, 0};
        bl = bh;
      }
      p2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, bh, zero4, 0, 0, 0);
      p2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, bl, p2[t], 0, 0, 0);
    }

    // ---- epilogue: acc += (d * P1 - dmin * P2) * 2^-e for the lane's rows
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int e = sm.sexp[16 * t + i];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2 dm = sm.dd[wave][4 * q + r];
        const float v = __builtin_fmaf(dm.x, p1[t][r], -dm.y * p2[t][r]);
        acc[t][r] += __builtin_ldexpf(v, -e);
      }
    }
    __syncthreads();  // the next super-block overwrites the staged x
  }

  // D lane layout: column (m) = i, rows 4q..4q+3
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int gm = m0 + 16 * t + i;
    if (gm >= a.M) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * q + r;
      if (row < a.rows) a.Y[(int64_t)gm * a.rows + row] = acc[t][r];
    }
  }
}

template <int WAVES, int MT>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.rows + 16 * WAVES - 1) / (16 * WAVES), (a.M + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((gemm_q4k_mfma_kernel<WAVES, MT>), grid, dim3(64 * WAVES), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(int fmt, GemmArgs a, int cus, hipStream_t s) {
  (void)cus;
  a.units = 0;
  if (fmt != kFmtQ4_K) return hipErrorInvalidValue;
  if (a.M <= 16) return launch<4, 1>(a, s);
  if (a.M <= 32) return launch<4, 2>(a, s);
  return launch<4, 4>(a, s);
}

}  // namespace gq
