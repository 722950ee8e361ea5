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
//   * the weight operand is sc_j * code_c, an integer <= 945, exact in fp16;
//   * the 256 x values of one activation row and super-block are scaled by a
//     power of two (so the largest has magnitude in [2^9, 2^10)) and split
//     into fp16 hi + lo parts, x' = hi + lo to about 2^-22 relative; both
//     parts are multiplied, so sum code*sc*x' is accumulated in fp32 from
//     exact products;
//   * the min term is one more matrix-core product per super-block with the
//     weight operand m_j (exact) and the fp16 hi and lo parts of the scaled
//     X_j side by side along k.
// d, dmin and the power of two are applied per super-block in fp32. The
// result meets the same accuracy bound as the fp32 paths for any finite
// input (no overflow or underflow of the fp16 parts).
//
// Two kernels run per call, on the caller's stream:
//   1. xprep converts X once into the operand layout above (one block of
//      kBlk bytes per 16-row m-tile and super-block: 8 hi and 8 lo sub-block
//      fragments, the min-term fragment and the 16 scales 2^-e), in
//      stream-ordered scratch, one workgroup per block;
//   2. the main kernel: a workgroup of 4 waves owns 64*WR weight rows and
//      16*WM activation rows (wave w: rows 16*WR*w .. +16*WR, all WM
//      m-tiles) and a range of super-blocks. The prepared fragments stream
//      through a 3-slot LDS ring in chunks of one sub-block (all WM m-tiles)
//      loaded two chunks ahead; each wave reads its Q4_K bytes straight from
//      global memory (lane (i, q) reads bytes 8q..8q+7 of each 32-byte code
//      group of its row i: exactly the k range its operand needs), a whole
//      super-block ahead, and builds the weight operand in registers.
// When the row and activation tiles alone cannot fill the GPU, the
// super-blocks are split over blockIdx.z and a third kernel adds the
// partial products in a fixed order (deterministic).
#include "gq_device.h"
#include "gq_internal.h"

#ifndef GQ_MM_BIG_M
#define GQ_MM_BIG_M 64  // above this many activation rows: 4 row tiles per wave
#endif
#ifndef GQ_MM_BIG_WR
// weight row tiles per wave for the large tile: 2 measured faster than 4 on
// MI355X (Q4_K 14336 x 4096 at M = 128 / 256 / 512: 59 / 89 / 165 us
// against 69 / 111 / 183 us), as the smaller tile gives twice the workgroups
#define GQ_MM_BIG_WR 2
#endif
#ifndef GQ_MM_BIG_WM
#define GQ_MM_BIG_WM 4  // activation m-tiles per wave for the large tile
#endif
#ifndef GQ_MM_WG_PER_CU
// split-K target: workgroups per CU. One measured faster than two for every
// tile (Q4_K gate / down, interleaved A/B: M = 16 34.9 / 32.1 -> 31.1 /
// 30.0 us, M = 64 46.6 / 41.9 -> 39.2 / 36.9 us)
#define GQ_MM_WG_PER_CU 1
#endif
#ifndef GQ_MM_TILE1_WR
// weight row tiles per wave for one m-tile (M <= 16): 1 measured faster than
// 2 on MI355X (Q4_K gate / down at M = 16: 32.5 / 28.7 us against 34.5 /
// 32.2 us, interleaved A/B); at M = 32 and 64 two stay ahead
#define GQ_MM_TILE1_WR 1
#endif

namespace gq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Prepared-activation block of one (m-tile, super-block).
constexpr int kFrag = 1024;             // one operand fragment: 64 lanes x 8 halves
constexpr int kHiOff = 0;               // 8 sub-block fragments, hi parts
constexpr int kLoOff = 8 * kFrag;       // 8 sub-block fragments, lo parts
constexpr int kMinOff = 16 * kFrag;     // min-term fragment
constexpr int kScaleOff = 17 * kFrag;   // 16 floats: 2^-e of each m row
constexpr int kBlk = 17 * kFrag + 64;
constexpr int kMinChunk = kFrag + 64;   // min fragment + scales, contiguous

// Within each group of 8 k, the weight operand holds the codes of bytes in
// the order 0,2,1,3,4,6,5,7 (that is how the nibble pairs are extracted);
// the prepared x uses the same order. The permutation is its own inverse.
__host__ __device__ constexpr int kslot(int k) {
  return (k & ~7) | ((k & 1) ? ((k & 2) ? (k & 7) : (k & 7) + 1)
                             : ((k & 2) ? (k & 7) - 1 : (k & 7)));
}
static_assert(kslot(0) == 0 && kslot(1) == 2 && kslot(2) == 1 && kslot(3) == 3 &&
              kslot(4) == 4 && kslot(5) == 6 && kslot(6) == 5 && kslot(7) == 7 &&
              kslot(9) == 10, "kslot");

// ------------------------------------------------------------------ xprep
struct PrepArgs {
  const float* X;
  uint8_t* xp;
  int M, cols, nsb, mtiles;
};

// One workgroup per (m-tile t, super-block sb); wave w converts sub-blocks
// 2w and 2w+1, lane (i, q) the 8 columns 8q..8q+7 of activation row 16t+i
// that it holds in the operand, so every fragment store is one coalesced
// 1 KB wave store. The per-row exponent comes from the max over all 256
// columns (lanes and waves), the sub-block sums from a lane butterfly.
__device__ __forceinline__ float xor_lanes(float v, int mask) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
      (int)((threadIdx.x & 63) ^ mask) << 2, __builtin_bit_cast(int, v)));
}

__global__ __launch_bounds__(256) void xprep_kernel(PrepArgs a) {
  __shared__ float red[4][16];       // per wave, per row: max |x|
  __shared__ float sums[16][8];      // per row, per sub-block: scaled sum
  __shared__ int sexp[16];
  const int t = blockIdx.x / a.nsb, sb = blockIdx.x % a.nsb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int m = 16 * t + i;
  float v[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c0 = 256 * sb + 32 * (2 * w + h) + 8 * q;
    if (m < a.M && c0 + 8 <= a.cols) {
      const float* src = a.X + (int64_t)m * a.cols + c0;
      const f32x4 u0 = load_f32x4(src), u1 = load_f32x4(src + 4);
      v[h][0] = u0.x; v[h][1] = u0.y; v[h][2] = u0.z; v[h][3] = u0.w;
      v[h][4] = u1.x; v[h][5] = u1.y; v[h][6] = u1.z; v[h][7] = u1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[h][k] = (m < a.M && c0 + k < a.cols) ? a.X[(int64_t)m * a.cols + c0 + k] : 0.f;
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(v[h][k]));
  mx = fmaxf(mx, xor_lanes(mx, 16));
  mx = fmaxf(mx, xor_lanes(mx, 32));
  if (q == 0) red[w][i] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i]));
  // largest |x'| in [2^9, 2^10): exponent e = 9 - ilogb(max)
  int e = 0;
  if (mx > 0.f) {
    const int be = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF);
    e = 136 - (be == 0 ? 1 : be);
    e = e > 126 ? 126 : (e < -126 ? -126 : e);
  }
  uint8_t* blk = a.xp + ((int64_t)t * a.nsb + sb) * kBlk;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int s = 2 * w + h;
    h8 ph, pl;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float x = __builtin_ldexpf(v[h][kslot(u)], e);
      const _Float16 hv = (_Float16)x;
      ph[u] = hv;
      pl[u] = (_Float16)(x - (float)hv);
      sum += x;
    }
    *(h8*)(blk + kHiOff + s * kFrag + lane * 16) = ph;
    *(h8*)(blk + kLoOff + s * kFrag + lane * 16) = pl;
    sum += xor_lanes(sum, 16);
    sum += xor_lanes(sum, 32);
    if (q == 0) sums[i][s] = sum;
  }
  if (w == 0 && q == 0) sexp[i] = e;
  __syncthreads();
  // min-term fragment: lanes q = 0 hold the hi parts of the 8 sub-block
  // sums, lanes q = 1 the lo parts (both in kslot order), lanes 2 and 3 zero
  if (w == 0) {
    h8 f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float sm = sums[i][kslot(u)];
      const _Float16 hv = (_Float16)sm;
      f[u] = q == 0 ? hv : q == 1 ? (_Float16)(sm - (float)hv) : (_Float16)0.f;
    }
    *(h8*)(blk + kMinOff + lane * 16) = f;
  } else if (w == 1 && lane < 16) {
    *(float*)(blk + kScaleOff + 4 * lane) = __builtin_ldexpf(1.f, -sexp[lane]);
  }
}

// ------------------------------------------------------------ main kernel
struct MmArgs {
  const uint8_t* W;
  const uint8_t* xp;
  float* out;
  int64_t row_bytes;
  int64_t split_stride;  // floats between the outputs of two super-block splits
  int rows, nsb, M, mtiles, ks;
};

// Four packed fp16 pairs (1024 + code) from the low (H = 0) or high (H = 1)
// nibbles of 8 code bytes, then sc * code exactly:
// fma((1024 + c), sc, -1024 sc) = c * sc is representable, so the single
// rounding of the fma is exact. The nibbles are masked into bytes once and
// v_perm_b32 places each byte under the 0x64 exponent byte of 1024.
template <int H>
__device__ __forceinline__ h8 build_w(uint32_t w0, uint32_t w1, h2 sc, h2 nsc) {
  constexpr uint32_t kMagic = 0x64646464u;
  const uint32_t n0 = (H ? w0 >> 4 : w0) & 0x0F0F0F0Fu;
  const uint32_t n1 = (H ? w1 >> 4 : w1) & 0x0F0F0F0Fu;
  uint32_t p[4];
  // selector bytes 0..3 pick from the second source, 4..7 from the first
  p[0] = __builtin_amdgcn_perm(kMagic, n0, 0x04020400u);  // bytes 0, 2
  p[1] = __builtin_amdgcn_perm(kMagic, n0, 0x04030401u);  // bytes 1, 3
  p[2] = __builtin_amdgcn_perm(kMagic, n1, 0x04020400u);
  p[3] = __builtin_amdgcn_perm(kMagic, n1, 0x04030401u);
  h8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const h2 o = __builtin_elementwise_fma(__builtin_bit_cast(h2, p[k]), sc, nsc);
    r[2 * k] = o[0];
    r[2 * k + 1] = o[1];
  }
  return r;
}

// Two 6-bit fields as an exact fp16 pair: (1024 + v) - 1024.
__device__ __forceinline__ h2 pair_f16(uint32_t two_fields) {
  const h2 v = __builtin_bit_cast(h2, two_fields | 0x64006400u);
  const h2 k = {(_Float16)1024.f, (_Float16)1024.f};
  return v - k;
}

// The decoded header of one row's super-block.
struct RowHead {
  float d, dmin;
  h2 sc[4];   // pairs (sc0, sc2), (sc1, sc3), (sc4, sc6), (sc5, sc7)
  h2 nsc[4];  // -1024 * sc
  h8 mfr;     // min-term operand: m_j in kslot order on lanes q < 2, else 0
};

__device__ __forceinline__ RowHead decode_head(u32x4 hd, int q) {
  RowHead h;
  h.d = half_bits_to_float(hd.x & 0xFFFFu);
  h.dmin = half_bits_to_float(hd.x >> 16);
  constexpr uint32_t L6 = 0x003F003Fu, L4 = 0x000F000Fu, H2 = 0x00300030u;
  h.sc[0] = pair_f16(hd.y & L6);
  h.sc[1] = pair_f16((hd.y >> 8) & L6);
  h.sc[2] = pair_f16((hd.w & L4) | ((hd.y >> 2) & H2));
  h.sc[3] = pair_f16(((hd.w >> 8) & L4) | ((hd.y >> 10) & H2));
  const h2 mm0 = pair_f16(hd.z & L6);
  const h2 mm1 = pair_f16((hd.z >> 8) & L6);
  const h2 mm2 = pair_f16(((hd.w >> 4) & L4) | ((hd.z >> 2) & H2));
  const h2 mm3 = pair_f16(((hd.w >> 12) & L4) | ((hd.z >> 10) & H2));
  const h2 k1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) h.nsc[k] = h.sc[k] * k1024;
  const _Float16 z = (_Float16)0.f;
  const bool on = q < 2;
  h.mfr = h8{on ? mm0[0] : z, on ? mm0[1] : z, on ? mm1[0] : z, on ? mm1[1] : z,
             on ? mm2[0] : z, on ? mm2[1] : z, on ? mm3[0] : z, on ? mm3[1] : z};
  return h;
}

// Vector-memory operations a wave has issued after requesting the chunk
// that step s (0..8) of a super-block reads, by the issue order of a step:
// [s == 0: WR header loads] [U chunk loads, for 8 steps ahead] compute
// [s odd: WR code-group loads]. The chunk was requested at step s-8; after
// it came that step's code loads (if odd), then 7 whole steps: 7 U chunk
// loads, the code loads of the odd ones, and a header load if one of them
// is a step 0. Over the 8 steps before s every position but s occurs.
__host__ __device__ constexpr int after_chunk(int s, int U, int WR) {
  return 7 * U + WR * (4 - (s & 1)) + ((s != 0 && s != 8) ? WR : 0);
}
// (s is a constant once the step loop is unrolled; the switch folds away)
template <int U, int WR>
__device__ __forceinline__ void wait_for_chunk(int s) {
  switch (s) {
    case 0: wait_vmcnt<after_chunk(0, U, WR)>(); break;
    case 1: wait_vmcnt<after_chunk(1, U, WR)>(); break;
    case 2: wait_vmcnt<after_chunk(2, U, WR)>(); break;
    case 3: wait_vmcnt<after_chunk(3, U, WR)>(); break;
    case 4: wait_vmcnt<after_chunk(4, U, WR)>(); break;
    case 5: wait_vmcnt<after_chunk(5, U, WR)>(); break;
    case 6: wait_vmcnt<after_chunk(6, U, WR)>(); break;
    case 7: wait_vmcnt<after_chunk(7, U, WR)>(); break;
    default: wait_vmcnt<after_chunk(8, U, WR)>(); break;
  }
}
static_assert(after_chunk(0, 2, 4) == 30 && after_chunk(1, 2, 4) == 30 && after_chunk(2, 2, 4) == 34 &&
              after_chunk(8, 2, 4) == 30, "after_chunk");


// The prepared x of one super-block arrives in 9 chunks: parts 0..7 the hi
// and lo fragments of sub-block `part` for the WM m-tiles, part 8 their
// min-term fragments and scales. Each chunk is moved by direct
// global-to-LDS loads (one wave instruction = one 1 KB fragment, lane l's
// 16 bytes landing at byte 16 l) into its own LDS array, so the compiler
// can tell the chunks apart. Chunk c is requested 8 steps before step c
// reads it; every wave issues the same U loads per chunk (padding with
// loads into a scratch array), so the number of vector-memory operations
// issued after a chunk's loads is a compile-time constant per step and the
// wait before the step's barrier covers exactly that chunk.
template <int WR, int WM>
__global__ __launch_bounds__(256) void gemm_q4k_mfma_kernel(MmArgs a) {
  constexpr int kSlotBytes = WM * 2 * kFrag;
  constexpr int kUnits = 2 * WM;              // 1 KB loads per chunk
  constexpr int kU = (kUnits + 3) / 4;        // per wave
  __shared__ __attribute__((aligned(16))) uint8_t sl0[kSlotBytes], sl1[kSlotBytes], sl2[kSlotBytes],
      sl3[kSlotBytes], sl4[kSlotBytes], sl5[kSlotBytes], sl6[kSlotBytes], sl7[kSlotBytes],
      sl8[kSlotBytes], spare[kFrag];
  uint8_t* const slots[9] = {sl0, sl1, sl2, sl3, sl4, sl5, sl6, sl7, sl8};

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, q = lane >> 4;
  const int row_w = blockIdx.x * (64 * WR) + 16 * WR * wave;
  const int mt0 = blockIdx.y * WM;
  const int z = blockIdx.z;
  const int sb0 = (int)((int64_t)a.nsb * z / a.ks);
  const int sb1 = (int)((int64_t)a.nsb * (z + 1) / a.ks);

  // Buffer loads from per-workgroup bases: the per-lane part of each address
  // is a 32-bit offset fixed for the whole kernel, the super-block part a
  // scalar offset. m-tiles past the last one are clamped for loads.
  const int mt_last = (a.mtiles - mt0 < WM ? a.mtiles - mt0 : WM) - 1;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.xp + (int64_t)mt0 * a.nsb * kBlk), (short)0,
      (int)((int64_t)(mt_last + 1) * a.nsb * kBlk), 0x00020000);
  // this wave's load units: unit u = wave + 4 j (u >= kUnits: padding)
  int xvoff[kU], mvoff[kU], mdst[kU];
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    const int u = wave + 4 * j < kUnits ? wave + 4 * j : 0;
    const int t = (u >> 1) < mt_last ? (u >> 1) : mt_last;
    xvoff[j] = t * a.nsb * kBlk + ((u & 1) ? kLoOff : kHiOff) + lane * 16;
    // part 8: units 0..WM-1 the min fragments, WM..2WM-1 the scales
    const int mt = u < WM ? u : u - WM;
    mvoff[j] = (mt < mt_last ? mt : mt_last) * a.nsb * kBlk + (u < WM ? kMinOff : kScaleOff) + lane * 16;
    mdst[j] = mt * kMinChunk + (u < WM ? 0 : kFrag);
  }
  auto request_chunk = [&](int sb, int part) {
    sb = sb < sb1 ? sb : sb1 - 1;  // past the end: reload the last (never read)
    uint8_t* dst = slots[part];
    issue_fence();
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      const bool live = wave + 4 * j < kUnits;
      if (part < 8) {
        load_lds16(xrs, live ? dst + (wave + 4 * j) * kFrag : spare, xvoff[j], sb * kBlk + part * kFrag);
      } else {
        const bool scale = live && wave + 4 * j >= WM;
        if (!scale || lane < 4)  // the 64-byte scale block is 4 lanes
          load_lds16(xrs, live ? dst + mdst[j] : spare, mvoff[j], sb * kBlk);
      }
    }
    issue_fence();
  };

  // The workgroup's weight rows from a per-workgroup base; each lane's row
  // is clamped to the last row for loads (stores are checked).
  const int row_g = blockIdx.x * (64 * WR);
  const int rows_g = a.rows - row_g < 64 * WR ? a.rows - row_g : 64 * WR;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + (int64_t)row_g * a.row_bytes), (short)0,
      (int)((int64_t)rows_g * a.row_bytes), 0x00020000);
  int wvoff[WR];
#pragma unroll
  for (int rt = 0; rt < WR; ++rt) {
    const int r = row_w + 16 * rt + i - row_g;
    wvoff[rt] = (r < rows_g ? r : rows_g - 1) * (int)a.row_bytes;
  }
  u32x4 hd[WR];
  uint32_t cw[WR][8];
  auto load_head = [&](int sb) {
    issue_fence();
#pragma unroll
    for (int rt = 0; rt < WR; ++rt)
      hd[rt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wvoff[rt], sb * kQ4KBytes, 0));
    issue_fence();
  };
  auto load_group = [&](int sb, int g) {
    issue_fence();
#pragma unroll
    for (int rt = 0; rt < WR; ++rt) {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                              wrs, wvoff[rt] + 16 + 32 * g + 8 * q, sb * kQ4KBytes, 0));
      cw[rt][2 * g] = v.x;
      cw[rt][2 * g + 1] = v.y;
    }
    issue_fence();
  };

  f4 acc[WR][WM], p1[WR][WM];
  const f4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rt = 0; rt < WR; ++rt)
#pragma unroll
    for (int t = 0; t < WM; ++t) acc[rt][t] = zero4;

  // Prologue, issued in the order of the steady state's last 8 steps (so
  // the wait counts below hold for the first super-block too): the first
  // super-block's header, then its chunks 0..7 with its code groups after
  // the odd ones.
  load_head(sb0);
#pragma unroll
  for (int p = 1; p <= 8; ++p) {
    request_chunk(sb0, p - 1);
    if (p & 1) load_group(sb0, p >> 1);
  }

  for (int sb = sb0; sb < sb1; ++sb) {
    const int sbn = sb + 1 < sb1 ? sb + 1 : sb1 - 1;
    RowHead h[WR];
#pragma unroll
    for (int rt = 0; rt < WR; ++rt) h[rt] = decode_head(hd[rt], q);

#pragma unroll
    for (int s = 0; s < 9; ++s) {
      // Wait for chunk (sb, s), requested 8 steps ago, then publish it.
      wait_for_chunk<kU, WR>(s);
      bare_barrier();
      if (s == 0) load_head(sbn);
      request_chunk(sb + (s + 8) / 9, (s + 8) % 9);
      const uint8_t* slot = slots[s];
      if (s < 8) {
        h8 xh[WM], xl[WM];
#pragma unroll
        for (int t = 0; t < WM; ++t) {
          xh[t] = *(const h8*)(slot + (2 * t) * kFrag + lane * 16);
          xl[t] = *(const h8*)(slot + (2 * t + 1) * kFrag + lane * 16);
        }
        const int pi = s < 4 ? (s & 1) : 2 + (s & 1);
        const int half = (s >> 1) & 1;
#pragma unroll
        for (int rt = 0; rt < WR; ++rt) {
          const _Float16 sv = h[rt].sc[pi][half], nv = h[rt].nsc[pi][half];
          const h2 sc2 = {sv, sv}, nsc2 = {nv, nv};
          const uint32_t w0 = cw[rt][2 * (s >> 1)], w1 = cw[rt][2 * (s >> 1) + 1];
          const h8 wf = (s & 1) ? build_w<1>(w0, w1, sc2, nsc2) : build_w<0>(w0, w1, sc2, nsc2);
#pragma unroll
          for (int t = 0; t < WM; ++t) {
            p1[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[t], wf, s == 0 ? zero4 : p1[rt][t], 0, 0, 0);
            p1[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[t], wf, p1[rt][t], 0, 0, 0);
          }
        }
        // this code group is done: fetch the next super-block's
        if (s & 1) load_group(sbn, s >> 1);
      } else {
#pragma unroll
        for (int t = 0; t < WM; ++t) {
          const h8 xm = *(const h8*)(slot + t * kMinChunk + lane * 16);
          const f4 scl = *(const f4*)(slot + t * kMinChunk + kFrag + q * 16);
#pragma unroll
          for (int rt = 0; rt < WR; ++rt) {
            const f4 p2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xm, h[rt].mfr, zero4, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = __builtin_fmaf(h[rt].d, p1[rt][t][e], -h[rt].dmin * p2[e]);
              acc[rt][t][e] = __builtin_fmaf(v, scl[e], acc[rt][t][e]);
            }
          }
        }
      }
    }
  }

  // D lane layout: column (weight row) = i, activation rows 4q..4q+3
  float* out = a.out + (int64_t)z * a.split_stride;
#pragma unroll
  for (int rt = 0; rt < WR; ++rt) {
    const int r = row_w + 16 * rt + i;
    if (r >= a.rows) continue;
#pragma unroll
    for (int t = 0; t < WM; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * (mt0 + t) + 4 * q + e;
        if (m < a.M) out[(int64_t)m * a.rows + r] = acc[rt][t][e];
      }
    }
  }
}

// Y = sum over the ks super-block splits, in split order.

template <int WR, int WM>
hipError_t launch_main(const MmArgs& m, int gx, int gy, hipStream_t s) {
  hipLaunchKernelGGL((gemm_q4k_mfma_kernel<WR, WM>), dim3(gx, gy, m.ks), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace

__global__ __launch_bounds__(256) void split_sum_kernel(const float* part, float* y, int64_t n, int ks) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  float v = part[idx];
  for (int z = 1; z < ks; ++z) v += part[(int64_t)z * n + idx];
  y[idx] = v;
}

hipError_t launch_split_sum(const float* part, float* y, int64_t n, int ks, hipStream_t s) {
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, y, n, ks);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(int fmt, GemmArgs a, int cus, hipStream_t s) {
  a.units = 0;
  if (fmt != kFmtQ4_K) return hipErrorInvalidValue;
  const int nsb = (a.cols + 255) / 256;
  const int mtiles = (a.M + 15) / 16;

  // tile shape by activation rows: WM m-tiles of 16, 64*WR weight rows
  int WR = GQ_MM_TILE1_WR, WM = 1;
  if (a.M > 16) WR = 2, WM = 2;
  if (a.M > 32) WM = 4;
  if (a.M > GQ_MM_BIG_M) {
    WR = GQ_MM_BIG_WR;
    WM = GQ_MM_BIG_WM;
  }
  const int gx = (a.rows + 64 * WR - 1) / (64 * WR);
  const int gy = (mtiles + WM - 1) / WM;
  // split the super-blocks until the grid covers the GPU (>= 2 super-blocks
  // each)
  const bool big = a.M > GQ_MM_BIG_M;
  const int64_t target = (int64_t)cus * GQ_MM_WG_PER_CU;
  int ks = 1;
  while ((int64_t)gx * gy * ks < target && nsb / (2 * ks) >= 2) ks *= 2;

  const size_t xp_bytes = (size_t)mtiles * nsb * kBlk;
  const size_t part_off = (xp_bytes + 255) & ~(size_t)255;
  const size_t part_bytes = ks > 1 ? (size_t)ks * a.M * a.rows * sizeof(float) : 0;
  void* ws = nullptr;
  hipError_t e = ws_alloc(part_off + part_bytes, s, &ws);
  if (e != hipSuccess) return e;

  PrepArgs pa{a.X, (uint8_t*)ws, a.M, a.cols, nsb, mtiles};
  hipLaunchKernelGGL(xprep_kernel, dim3((unsigned)((int64_t)mtiles * nsb)), dim3(256), 0, s, pa);
  e = hipGetLastError();

  MmArgs m{a.W, (const uint8_t*)ws, ks > 1 ? (float*)((uint8_t*)ws + part_off) : a.Y,
           a.row_bytes, (int64_t)a.M * a.rows, a.rows, nsb, a.M, mtiles, ks};
  if (e == hipSuccess) {
    if (big) e = launch_main<GQ_MM_BIG_WR, GQ_MM_BIG_WM>(m, gx, gy, s);
    else if (WM == 4) e = launch_main<2, 4>(m, gx, gy, s);
    else if (WM == 2) e = launch_main<2, 2>(m, gx, gy, s);
    else e = launch_main<GQ_MM_TILE1_WR, 1>(m, gx, gy, s);
  }
  if (e == hipSuccess && ks > 1) {
    const int64_t n = (int64_t)a.M * a.rows;
    e = launch_split_sum((const float*)m.out, a.Y, n, ks, s);
  }
  const hipError_t ef = ws_free(ws, s);
  return e != hipSuccess ? e : ef;
}

}  // namespace gq
