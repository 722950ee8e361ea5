// gemm_f16.hip -- Y = X W^T for Q4_K (and Q5_K, Q6_K, Q8_0, Q5_0) weights
// and two or more activation rows, on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_f16). One launch; the kernel uses no memory beyond
// its arguments. The other layouts are described with their traits below;
// this header describes Q4_K.
//
// The prompt-chunk product ("nurllama 0.18.1 API", model.nu section: the
// matmuls run over a chunk of positions at once, each weight read once per
// chunk) is a real dense contraction once M >= 16.
//
// Exact operands. A Q4_K super-block contributes, per output,
//   d * sum_j sc_j * sum_{c in j} code_c * x_c  -  dmin * sum_j m_j * X_j
// with X_j the sum of x over sub-block j:
//   * the weight operand is sc_j * code_c, an integer <= 63 * 15, exact in fp16;
//   * the 256 x of one activation row and super-block are scaled by 2^e so
//     that the largest magnitude lies in [2^9, 2^10), and split into fp16
//     parts hi = fp16(x 2^e) and lo = fp16(x 2^e - hi) (v_fma_mix: one
//     rounding each), so x 2^e = hi + lo to about 2^-22 relative; both parts
//     are multiplied, so the products are exact and the sums are fp32;
//   * the min term is one more product per super-block: each lane's partial
//     sums of x over its 8 columns of every sub-block (hi and lo parts, side
//     by side along k) against m_j repeated for every lane;
//   * d, dmin and 2^-e are applied per super-block in fp32.
// The fp16 parts keep this accuracy for every activation whose magnitude is
// at least 2^-14 of the largest one in its row and super-block (and for any
// row whose largest magnitude lies in [2^-117, 2^126)); smaller ones reach
// the fp16 subnormal range and are represented only to an absolute 2^-34 of
// that largest magnitude.
//
// Two kernels. The shared-activation kernel (gemm_f16_xs_kernel, below)
// converts each activation tile once per workgroup into LDS for every wave;
// it serves the grids that fill the GPU. The per-wave kernel serves the
// smaller ones: a workgroup of four waves owns 16 WR weight rows and 16
// activation rows; its waves take the super-blocks in turn (wave w: w, w + 4,
// ...) and each builds its own operands in registers:
//   * the weight rows' bytes arrive by buffer loads -- lane (i, q) reads the
//     header and bytes 8q..8q+7 of each 32-byte code group of its row i, which
//     is exactly the k range its operand needs -- and become sc * code with
//     one v_perm_b32 (code under the exponent of 1024) and one packed fp16
//     fma per code pair;
//   * lane (i, q) reads columns 8q..8q+7 of every sub-block of activation row
//     i, takes the row's largest magnitude with two lane exchanges, and
//     splits its values into the hi and lo operands.
// The four waves' products are added in LDS in wave order (deterministic).
#include "gemv_common.h"
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));


__device__ __forceinline__ h8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(h8, v);
}

// Codes of 8 consecutive bytes (w0 = bytes 0-3, w1 = bytes 4-7), low (H = 0)
// or high (H = 1) nibbles, as the fp16 values sc * code in byte order:
// v_perm_b32 puts each code byte under the exponent byte 0x64 of 1024, and
// fma((1024 + c), sc, -1024 sc) = c * sc is exact (one rounding of an exactly
// representable value).
template <int H>
__device__ __forceinline__ h8 weight_operand(uint32_t w0, uint32_t w1, h2 sc, h2 nsc) {
  constexpr uint32_t kMagic = 0x64646464u;
  const uint32_t n0 = (H ? w0 >> 4 : w0) & 0x0F0F0F0Fu;
  const uint32_t n1 = (H ? w1 >> 4 : w1) & 0x0F0F0F0Fu;
  // selector bytes 0..3 take bytes of the second source, 4..7 of the first
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(kMagic, n0, 0x04010400u);  // codes 0, 1
  p[1] = __builtin_amdgcn_perm(kMagic, n0, 0x04030402u);  // codes 2, 3
  p[2] = __builtin_amdgcn_perm(kMagic, n1, 0x04010400u);  // codes 4, 5
  p[3] = __builtin_amdgcn_perm(kMagic, n1, 0x04030402u);  // codes 6, 7
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, p[k]), sc, nsc));
  return as_h8(r[0], r[1], r[2], r[3]);
}

// The super-block layouts these kernels take. Q4_K and Q5_K share the
// header (fp16 d and dmin, then the twelve 6-bit scale/min bytes) and the
// nibble layout; Q5_K puts 32 bytes of fifth bits between them (bit 2g + h
// of byte l is bit 4 of weight 64g + 32h + l). Its codes reach 31 and
// sc * code 63 * 31 = 1953, still an exact fp16 integer, and the packed fma
// that forms sc * code from the biased code (up to 63 * 1055) rounds only
// its result, so the operand stays exact.
struct MmQ4K {
  static constexpr int kKind = 0, kBytes = 144, kCodes = 16;
  static constexpr bool kQh = false;
};
struct MmQ5K {
  static constexpr int kKind = 0, kBytes = 176, kCodes = 48;
  static constexpr bool kQh = true;
};
// Q8_0: one fp16 d and 32 int8 codes per block, eight blocks per 256-column
// step (kBytes: the step's bytes in a row). Each 32-wide k-slice of an
// operand is one block, so the weight operand is the codes themselves (exact
// in fp16) and d scales the slice's product in fp32. Packed (kKind 1): the
// 34-byte blocks as stored; the rows must be a multiple of 4 bytes long and W
// 4-byte aligned, so that every dword load below is aligned (an even block's
// codes start 2 bytes into a dword and are shifted out with v_alignbyte).
// Split (kKind 2): the per-row layout with the scales ahead of the codes.
struct MmQ8P {
  static constexpr int kKind = 1, kBytes = 272;
  static constexpr bool kQh = false;
};
struct MmQ8S {
  static constexpr int kKind = 2, kBytes = 256;
  static constexpr bool kQh = false;
};
// Q6_K (kKind 3): 210-byte super-blocks -- 128 bytes of low nibbles, 64 bytes
// of 2-bit high parts, 16 int8 sub-block scales, fp16 d -- with
// w = d * sc_s * (q - 32) over 16-weight sub-blocks s. sc * (q - 32) reaches
// 13 significant bits, so each k-slice takes two exact operands:
// 16 sh (q - 32) and sl (q - 32) with sc = 16 sh + sl, 0 <= sl < 16 (at most
// 4096 with its low 4 bits zero, and 480), four products per slice into two
// fp32 sums added per step; d is applied per super-block. A super-block starts 2 bytes into a
// dword on odd steps (210 = 2 mod 4): the rows must be a multiple of 4 bytes
// long and W 4-byte aligned, and every piece is loaded from the dword
// boundary before it and shifted into place.
struct MmQ6K {
  static constexpr int kKind = 3, kBytes = 210;
  static constexpr bool kQh = false;
};
// Q5_0 (kKind 4): 22-byte blocks -- fp16 d, a 32-bit word qh whose bit k is
// bit 4 of weight k, 16 bytes of nibbles (weight k < 16: low nibble of byte
// k, else high nibble of byte k - 16) -- with w = d * (q - 16). Handled as
// Q8_0: one block per k-slice, the operand q - 16 exact in fp16, d per
// block. Eight blocks make 176 bytes, so with rows of an even number of
// blocks and W 4-byte aligned even blocks are dword aligned and odd ones
// start 2 bytes into a dword.
struct MmQ50 {
  static constexpr int kKind = 4, kBytes = 176;
  static constexpr bool kQh = false;
};

// Eight int8 codes (the bytes of w0, then w1) as fp16 values: a byte with its
// sign bit flipped is 128 + code, v_perm_b32 places it under the exponent of
// 1024, and (1152 + code) - 1152 = code is exact.
__device__ __forceinline__ h8 q8_operand(uint32_t w0, uint32_t w1) {
  constexpr uint32_t kMagic = 0x64646464u;
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(kMagic, u0, 0x04010400u);  // codes 0, 1
  p[1] = __builtin_amdgcn_perm(kMagic, u0, 0x04030402u);  // codes 2, 3
  p[2] = __builtin_amdgcn_perm(kMagic, u1, 0x04010400u);  // codes 4, 5
  p[3] = __builtin_amdgcn_perm(kMagic, u1, 0x04030402u);  // codes 6, 7
  const h2 k = {(_Float16)-1152.f, (_Float16)-1152.f};
  uint32_t r[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p[c]) + k);
  return as_h8(r[0], r[1], r[2], r[3]);
}

// Q5_K: the Q4_K operand of sub-block J with the fifth bits merged in: qh0 /
// qh1 are the fifth-bit bytes of the same 8 code bytes (w0 / w1), and bit J
// of each is moved to bit 4 of its code byte.
template <int J>
__device__ __forceinline__ h8 weight_operand5(uint32_t w0, uint32_t w1, uint32_t qh0, uint32_t qh1,
                                              h2 sc, h2 nsc) {
  constexpr uint32_t kMagic = 0x64646464u;
  constexpr int H = J & 1;
  const uint32_t b0 = J <= 4 ? qh0 << (4 - J) : qh0 >> (J - 4);
  const uint32_t b1 = J <= 4 ? qh1 << (4 - J) : qh1 >> (J - 4);
  const uint32_t n0 = ((H ? w0 >> 4 : w0) & 0x0F0F0F0Fu) | (b0 & 0x10101010u);
  const uint32_t n1 = ((H ? w1 >> 4 : w1) & 0x0F0F0F0Fu) | (b1 & 0x10101010u);
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(kMagic, n0, 0x04010400u);  // codes 0, 1
  p[1] = __builtin_amdgcn_perm(kMagic, n0, 0x04030402u);  // codes 2, 3
  p[2] = __builtin_amdgcn_perm(kMagic, n1, 0x04010400u);  // codes 4, 5
  p[3] = __builtin_amdgcn_perm(kMagic, n1, 0x04030402u);  // codes 6, 7
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, p[k]), sc, nsc));
  return as_h8(r[0], r[1], r[2], r[3]);
}

// The weight operand of sub-block J for either layout.
template <class Fm, int J>
__device__ __forceinline__ h8 weight_op(u32x2 cw, u32x2 qh, h2 sc, h2 nsc) {
  if constexpr (Fm::kQh) return weight_operand5<J>(cw.x, cw.y, qh.x, qh.y, sc, nsc);
  else return weight_operand<J & 1>(cw.x, cw.y, sc, nsc);
}

// weight_op for a sub-block index that is a constant once the loop over the
// eight sub-blocks is unrolled.
template <class Fm>
__device__ __forceinline__ h8 weight_op_j(int j, u32x2 cw, u32x2 qh, h2 sc, h2 nsc) {
  switch (j) {
    case 0: return weight_op<Fm, 0>(cw, qh, sc, nsc);
    case 1: return weight_op<Fm, 1>(cw, qh, sc, nsc);
    case 2: return weight_op<Fm, 2>(cw, qh, sc, nsc);
    case 3: return weight_op<Fm, 3>(cw, qh, sc, nsc);
    case 4: return weight_op<Fm, 4>(cw, qh, sc, nsc);
    case 5: return weight_op<Fm, 5>(cw, qh, sc, nsc);
    case 6: return weight_op<Fm, 6>(cw, qh, sc, nsc);
    default: return weight_op<Fm, 7>(cw, qh, sc, nsc);
  }
}

// Two six-bit fields (bits 0-5 and 16-21) as an exact fp16 pair.
__device__ __forceinline__ h2 pair_f16(uint32_t two_fields) {
  const h2 v = __builtin_bit_cast(h2, two_fields | 0x64006400u);
  const h2 k = {(_Float16)1024.f, (_Float16)1024.f};
  return v - k;
}

// The header of one row's super-block, decoded for the operands: the eight
// scale codes as fp16 (sc) and times -1024 (nsc), the min-term operand
// (m_0..m_7), d and dmin.
struct RowHead {
  float d, dmin;
  h8 sc, nsc, mop;
};

__device__ __forceinline__ RowHead decode_head(u32x4 hd) {
  RowHead h;
  h.d = half_bits_to_float(hd.x & 0xFFFFu);
  h.dmin = half_bits_to_float(hd.x >> 16);
  // pairs (field j, field j + 2) from the 12 scale bytes s[0..11]:
  // j < 4: sc = s[j] & 63, m = s[j + 4] & 63; j >= 4: low 4 bits from s[j + 4],
  // top 2 bits from bits 6-7 of s[j - 4] (sc) or s[j] (m)
  constexpr uint32_t L6 = 0x003F003Fu, L4 = 0x000F000Fu, H2 = 0x00300030u;
  const h2 s02 = pair_f16(hd.y & L6), s13 = pair_f16((hd.y >> 8) & L6);
  const h2 s46 = pair_f16((hd.w & L4) | ((hd.y >> 2) & H2));
  const h2 s57 = pair_f16(((hd.w >> 8) & L4) | ((hd.y >> 10) & H2));
  const h2 m02 = pair_f16(hd.z & L6), m13 = pair_f16((hd.z >> 8) & L6);
  const h2 m46 = pair_f16(((hd.w >> 4) & L4) | ((hd.z >> 2) & H2));
  const h2 m57 = pair_f16(((hd.w >> 12) & L4) | ((hd.z >> 10) & H2));
  h.sc = h8{s02[0], s13[0], s02[1], s13[1], s46[0], s57[0], s46[1], s57[1]};
  const _Float16 k = (_Float16)-1024.f;
  h.nsc = h.sc * h8{k, k, k, k, k, k, k, k};
  h.mop = h8{m02[0], m13[0], m02[1], m13[1], m46[0], m57[0], m46[1], m57[1]};
  return h;
}

// fp16 parts of a * s and b * s: hi = fp16(v), lo = fp16(v - hi), each one
// rounding of the exact value (v_fma_mix), packed (a in the low half).
__device__ __forceinline__ void split2(float a, float b, float s, uint32_t& hi, uint32_t& lo) {
  __asm__("v_fma_mixlo_f16 %0, %2, %4, 0\n\t"
          "v_fma_mixhi_f16 %0, %3, %4, 0\n\t"
          "v_fma_mixlo_f16 %1, %2, %4, -%0 op_sel_hi:[0,0,1]\n\t"
          "v_fma_mixhi_f16 %1, %3, %4, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
          : "=&v"(hi), "=&v"(lo)
          : "v"(a), "v"(b), "v"(s));
}

__device__ __forceinline__ float lane_xor(float v, int mask) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
      (int)(((threadIdx.x & 63) ^ mask) << 2), __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float lane_read(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ u32x4 buf_b128(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}

__device__ __forceinline__ u32x2 buf_b64(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
}

// One product (or one group of a grouped product): W rows, X rows, Y rows.
struct MmTile {
  int64_t w_off;   // byte offset of the group's weight tensor from W
  int m_begin;     // first activation row of the group (in X and Y)
  int m_count;     // activation rows in the group
  int mtile0;      // first blockIdx.y of the group
};

constexpr int kMaxGroups = 64;

// The epilogue of one output element (see GemmEpilogue).
template <int EPI>
__device__ __forceinline__ void mm_out(float* p, float v) {
  if constexpr (EPI == kMmAcc) *p += v;
  else if constexpr (EPI == kMmSiluMul) *p = silu_mul(v, *p);
  else *p = v;
}

struct MmArgs {
  const uint8_t* W;
  const float* X;
  float* Y;
  int64_t row_bytes;
  int rows, cols, nsb;
  int nb;        // Q8_0: blocks of 32 per row
  int code_off;  // split Q8_0: bytes of a row's scale region
  int n_groups;
  MmTile g[kMaxGroups];
  // groups whose row counts live on the device (gq_matmul_experts_dev):
  // n_groups counts at dev_m, expert e's weights at W + e * dev_w_bytes, and
  // dev_total activation rows in X and Y; null for the table g above
  const int64_t* dev_m;
  int64_t dev_w_bytes;
  int dev_total;
};

// This workgroup's group: the table entry whose m-tiles hold blockIdx.y, or,
// with device counts, the group found by walking the counts (each clamped to
// the rows left of dev_total, so that no group reaches past X or Y). False
// when blockIdx.y lies past the last m-tile (the grid is sized for the most
// m-tiles the total can need).
__device__ __forceinline__ bool find_group(const MmArgs& a, int tm, MmTile& grp) {
  const int y = (int)blockIdx.y;
  if (a.dev_m == nullptr) {
    int gidx = 0;
    for (int g = 1; g < a.n_groups; ++g)
      if (y >= a.g[g].mtile0) gidx = g;
    grp = a.g[gidx];
    return true;
  }
  int tiles = 0, rows = 0;
  for (int e = 0; e < a.n_groups; ++e) {
    const int64_t c = a.dev_m[e];
    const int m = c < 0 ? 0 : (int)min(c, (int64_t)(a.dev_total - rows));
    const int t = (m + tm - 1) / tm;
    if (y < tiles + t) {
      grp = MmTile{a.dev_w_bytes * e, rows, m, tiles};
      return true;
    }
    tiles += t;
    rows += m;
  }
  return false;
}

// The weight bytes lane (i, q) needs for one 256-column step of R row tiles
// (row i of each): K-quants -- the super-block header and the lane's 8 code
// bytes of each 32-byte group (and Q5_K's fifth-bit bytes of the same
// positions).
template <class Fm, int R, int K = Fm::kKind>
struct WStage {
  u32x4 hd[R];
  u32x2 cw[R][4];
  u32x2 qh[R];
};
// Packed Q8_0: block 2h's 12 bytes from 2 bytes before the lane's codes,
// block 2h + 1's 8 code bytes, and the dwords holding the d of blocks 2q and
// 2q + 1 (low half, high half): lane (i, q) fetches two of its row's eight
// scales, and q8_scales hands them round the row's four lanes.
template <class Fm, int R>
struct WStage<Fm, R, 1> {
  u32x3 ce[R][4];
  u32x2 co[R][4];
  uint32_t dq[R][2];
};
// Split Q8_0: the lane's 8 code bytes of each block and the step's 8 scales.
template <class Fm, int R>
struct WStage<Fm, R, 2> {
  u32x2 cs[R][8];
  u32x4 dd[R];
};
// Q5_0: the lane's 8 nibble bytes of each block (bytes 8 (q % 2)..: 12 from
// 2 bytes early for the even blocks), and the dwords holding d and qh of
// blocks 2q and 2q + 1 (at 44q, 44q + 4, 44q + 20, 44q + 24), which the
// row's four lanes share through ds_bpermute.
template <class Fm, int R>
struct WStage<Fm, R, 4> {
  u32x3 qe[R][4];
  u32x2 qo[R][4];
  u32x2 dh[R][2];
};
// Q6_K: the lane's 8 bytes of each 32-byte group of low nibbles (group
// p = 2n + h at 32p + 8q) and of high parts (group n at 128 + 32n + 8q), the
// 16 scale bytes and the dword holding d, each from 2 bytes early on odd
// steps.
template <class Fm, int R>
struct WStage<Fm, R, 3> {
  u32x3 ql[R][4];
  u32x3 qh[R][2];
  u32x4 sc[R];
  uint32_t sd[R];
};

__device__ __forceinline__ u32x3 buf_b96(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, voff, soff, 0));
}

__device__ __forceinline__ uint32_t buf_b32(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
}

// Requests for the weight bytes of step sb: wv[t] is the byte offset of the
// lane's row in tile t, code_off where a split row's codes start. The
// per-lane parts of the offsets are checked by the buffer's range; the
// scalar part (the step) must be a real position.
template <class Fm, int R>
__device__ __forceinline__ void fetch_w(WStage<Fm, R>& st, __amdgpu_buffer_rsrc_t wrs, const int (&wv)[R], int q,
                                        int sb, int code_off) {
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if constexpr (Fm::kKind == 0) {
      st.hd[t] = buf_b128(wrs, wv[t], sb * Fm::kBytes);
#pragma unroll
      for (int g = 0; g < 4; ++g) st.cw[t][g] = buf_b64(wrs, wv[t] + Fm::kCodes + 32 * g + 8 * q, sb * Fm::kBytes);
      if constexpr (Fm::kQh) st.qh[t] = buf_b64(wrs, wv[t] + 16 + 8 * q, sb * Fm::kBytes);
    } else if constexpr (Fm::kKind == 1) {
      // block 2h at 68h (codes at 68h + 2 + 8q), block 2h + 1 at 68h + 34. A
      // row holds an even number of blocks, so its last block is an odd one,
      // whose 8-byte loads end inside it.
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        st.ce[t][h] = buf_b96(wrs, wv[t] + 68 * h + 8 * q, sb * Fm::kBytes);
        st.co[t][h] = buf_b64(wrs, wv[t] + 68 * h + 36 + 8 * q, sb * Fm::kBytes);
      }
      st.dq[t][0] = buf_b32(wrs, wv[t] + 68 * q, sb * Fm::kBytes);
      st.dq[t][1] = buf_b32(wrs, wv[t] + 68 * q + 32, sb * Fm::kBytes);
    } else if constexpr (Fm::kKind == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) st.cs[t][j] = buf_b64(wrs, wv[t] + code_off + 32 * j + 8 * q, sb * Fm::kBytes);
      st.dd[t] = buf_b128(wrs, wv[t], sb * 16);
    } else if constexpr (Fm::kKind == 3) {
      // the dword boundary at or before the step. On even steps the dword of
      // d also holds the next step's first 2 bytes; a row holds an even number
      // of super-blocks, so its last step is odd and that dword never crosses
      // the end of the buffer (whose range check would zero all of it).
      const int soff = sb * Fm::kBytes - 2 * (sb & 1);
#pragma unroll
      for (int p = 0; p < 4; ++p) st.ql[t][p] = buf_b96(wrs, wv[t] + 32 * p + 8 * q, soff);
#pragma unroll
      for (int n = 0; n < 2; ++n) st.qh[t][n] = buf_b96(wrs, wv[t] + 128 + 32 * n + 8 * q, soff);
      st.sc[t] = buf_b128(wrs, wv[t] + 192, soff);
      st.sd[t] = buf_b32(wrs, wv[t] + 208, soff);
    } else {
      // block 2h at 44h (nibbles from 44h + 6), 2h + 1 at 44h + 22 (from
      // 44h + 28); the row's last block is an odd one, whose loads end in it
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        st.qe[t][h] = buf_b96(wrs, wv[t] + 44 * h + 4 + 8 * (q & 1), sb * Fm::kBytes);
        st.qo[t][h] = buf_b64(wrs, wv[t] + 44 * h + 28 + 8 * (q & 1), sb * Fm::kBytes);
      }
      st.dh[t][0] = buf_b64(wrs, wv[t] + 44 * q, sb * Fm::kBytes);
      st.dh[t][1] = buf_b64(wrs, wv[t] + 44 * q + 20, sb * Fm::kBytes);
    }
  }
}

// Vector-memory requests of one fetch_w per row tile.
template <class Fm>
constexpr int fetch_w_ops() {
  return Fm::kKind == 0 ? (Fm::kQh ? 6 : 5) : Fm::kKind == 1 ? 10 : Fm::kKind == 2 ? 9 : Fm::kKind == 3 ? 8 : 10;
}

// Q8_0: the lane's 8 code bytes of block j of row tile t, and the block's d
// (zero for a block past the row's last, whose bytes belong to the next row).
template <class Fm, int R>
__device__ __forceinline__ u32x2 q8_codes(const WStage<Fm, R>& st, int t, int j) {
  if constexpr (Fm::kKind == 1) {
    if (j & 1) return st.co[t][j >> 1];
    const u32x3 r = st.ce[t][j >> 1];
    return u32x2{__builtin_amdgcn_alignbyte(r.y, r.x, 2), __builtin_amdgcn_alignbyte(r.z, r.y, 2)};
  } else {
    return st.cs[t][j];
  }
}

// The eight scales of row tile t as four dwords, d of blocks 2h and 2h + 1
// in dword h (low, high half). Packed: lane (i, h) holds that pair, so every
// lane reads it from there (ds_bpermute; i = lane % 16).
template <class Fm, int R>
__device__ __forceinline__ u32x4 q8_scales(const WStage<Fm, R>& st, int t, int i) {
  if constexpr (Fm::kKind == 1) {
    const int pair = (int)__builtin_amdgcn_perm(st.dq[t][1], st.dq[t][0], 0x07060100u);
    u32x4 d;
#pragma unroll
    for (int h = 0; h < 4; ++h) d[h] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * h + i) << 2, pair);
    return d;
  } else {
    return st.dd[t];
  }
}

// d of block j from q8_scales (zero for a block past the row's last).
__device__ __forceinline__ float q8_scale(u32x4 d4, int j, bool real) {
  const uint32_t w = d4[j >> 1];
  const float d = half_bits_to_float((j & 1) ? w >> 16 : w & 0xFFFFu);
  return real ? d : 0.f;
}

// Q5_0: the operand of block j (codes q - 16 of the lane's 8 weights) and
// its d (zero for a block past the row's last). Lane (i, h) holds the d and
// qh dwords of blocks 2h and 2h + 1 of row i.
template <class Fm, int R>
__device__ __forceinline__ h8 q5_operand(const WStage<Fm, R>& st, int t, int j, int i, int q, bool real, float& d) {
  const int src = (16 * (j >> 1) + i) << 2;
  uint32_t d16, qh;
  u32x2 L;
  if (j & 1) {
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)st.dh[t][1].x);
    qh = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)st.dh[t][1].y);
    d16 = b0 >> 16;
    L = st.qo[t][j >> 1];
  } else {
    const uint32_t a0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)st.dh[t][0].x);
    const uint32_t a1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)st.dh[t][0].y);
    d16 = a0 & 0xFFFFu;
    qh = __builtin_amdgcn_alignbyte(a1, a0, 2);
    const u32x3 e = st.qe[t][j >> 1];
    L = u32x2{__builtin_amdgcn_alignbyte(e.y, e.x, 2), __builtin_amdgcn_alignbyte(e.z, e.y, 2)};
  }
  d = real ? half_bits_to_float(d16) : 0.f;
  // weights 8q..8q+7: nibbles of bytes 8 (q % 2).. (high ones for q >= 2),
  // fifth bits = byte q of qh, each bit moved to bit 4 of its code byte
  // ((b * 0x204081) & 0x01010101 puts bit e of a 4-bit b in byte e)
  const uint32_t nsh = 4u * (uint32_t)(q >> 1);
  const uint32_t hb = (qh >> (8 * q)) & 0xFFu;
  const uint32_t c0 = ((L.x >> nsh) & 0x0F0F0F0Fu) | ((((hb & 0xFu) * 0x204081u) & 0x01010101u) << 4);
  const uint32_t c1 = ((L.y >> nsh) & 0x0F0F0F0Fu) | ((((hb >> 4) * 0x204081u) & 0x01010101u) << 4);
  constexpr uint32_t kMagic = 0x64646464u;
  const h2 bias = {(_Float16)-1040.f, (_Float16)-1040.f};
  uint32_t r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t pk = __builtin_amdgcn_perm(kMagic, k < 2 ? c0 : c1, (k & 1) ? 0x04030402u : 0x04010400u);
    r[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, pk) + bias);  // q - 16, exact
  }
  return as_h8(r[0], r[1], r[2], r[3]);
}

// Block formats (Q8_0, Q5_0): what a step of row tile t needs for every
// block (the Q8_0 scales), then each block's operand and d.
template <class Fm, int R>
__device__ __forceinline__ u32x4 blk_head(const WStage<Fm, R>& st, int t, int i) {
  if constexpr (Fm::kKind == 4) return u32x4{0u, 0u, 0u, 0u};
  else return q8_scales(st, t, i);
}

template <class Fm, int R>
__device__ __forceinline__ h8 blk_operand(const WStage<Fm, R>& st, u32x4 head, int t, int j, int i, int q,
                                          bool real, float& d) {
  if constexpr (Fm::kKind == 4) {
    return q5_operand(st, t, j, i, q, real, d);
  } else {
    const u32x2 c = q8_codes(st, t, j);
    d = q8_scale(head, j, real);
    return q8_operand(c.x, c.y);
  }
}

// Q6_K, one step of row tile t for lane (i, q): the scales of its 8 slices
// (slice j uses sub-block 2j + q / 2) as signed bytes, and d.
struct Q6Head {
  uint32_t s03, s47;
  float d;
};

template <class Fm, int R>
__device__ __forceinline__ Q6Head q6_head(const WStage<Fm, R>& st, int t, int sh, uint32_t sel) {
  const u32x4 c = st.sc[t];
  const uint32_t b0 = __builtin_amdgcn_alignbyte(c.y, c.x, sh), b1 = __builtin_amdgcn_alignbyte(c.z, c.y, sh);
  const uint32_t b2 = __builtin_amdgcn_alignbyte(c.w, c.z, sh), b3 = __builtin_amdgcn_alignbyte(st.sd[t], c.w, sh);
  Q6Head h;
  h.s03 = __builtin_amdgcn_perm(b1, b0, sel);
  h.s47 = __builtin_amdgcn_perm(b3, b2, sel);
  h.d = half_bits_to_float((st.sd[t] >> (8 * sh)) & 0xFFFFu);
  return h;
}

// The two weight operands of slice j (columns 32j..32j+31 of the step; the
// lane's 8 of them): 16 sh (q - 32) and sl (q - 32).
template <class Fm, int R>
__device__ __forceinline__ void q6_operands(const WStage<Fm, R>& st, int t, int j, int sh, const Q6Head& h,
                                            h8& ahi, h8& alo) {
  const int n = j >> 2, k4 = j & 3;
  const u32x3 lr = st.ql[t][2 * n + (k4 & 1)], hr = st.qh[t][n];
  uint32_t code[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t L = __builtin_amdgcn_alignbyte(w ? lr.z : lr.y, w ? lr.y : lr.x, sh);
    const uint32_t H = __builtin_amdgcn_alignbyte(w ? hr.z : hr.y, w ? hr.y : hr.x, sh);
    const uint32_t lo = ((k4 >> 1) ? L >> 4 : L) & 0x0F0F0F0Fu;
    const uint32_t hi = k4 == 0 ? H << 4 : k4 == 1 ? H << 2 : k4 == 2 ? H : H >> 2;
    code[w] = lo | (hi & 0x30303030u);
  }
  constexpr uint32_t kMagic = 0x64646464u;
  const int sc = (int)(int8_t)(((j < 4 ? h.s03 : h.s47) >> (8 * (j & 3))) & 0xFFu);
  const int sl = sc & 15;
  const _Float16 fh = (_Float16)(sc - sl), fl = (_Float16)sl;
  const h2 khi = {fh, fh}, klo = {fl, fl}, bias = {(_Float16)-1056.f, (_Float16)-1056.f};
  uint32_t rh[4], rl[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t pk = __builtin_amdgcn_perm(kMagic, code[k >> 1], (k & 1) ? 0x04030402u : 0x04010400u);
    const h2 c32 = __builtin_bit_cast(h2, pk) + bias;  // q - 32, exact
    rh[k] = __builtin_bit_cast(uint32_t, c32 * khi);
    rl[k] = __builtin_bit_cast(uint32_t, c32 * klo);
  }
  ahi = as_h8(rh[0], rh[1], rh[2], rh[3]);
  alo = as_h8(rl[0], rl[1], rl[2], rl[3]);
}

// An activation tile (16 rows x the 256 columns of one super-block) in LDS:
// row r at r * kXRow bytes. The 16-byte pad makes the lane reads of the
// operand layout (16 rows at the same column) hit 16 different bank groups.
constexpr int kXRow = 1024 + 16;
constexpr int kXTile = 16 * kXRow;

// KW waves per workgroup take the super-blocks in turn; each keeps the next
// super-block's bytes in flight (two stages) while it multiplies the current
// one. The activation tile is moved by direct global-to-LDS loads, one row
// (1 KB, contiguous) per wave instruction: reading the operand layout
// straight from memory would make every instruction touch 16 rows whose
// stride (cols * 4 bytes, a multiple of 4 KB for 4096 or 14336 columns)
// maps them all to one L2 channel.
template <class Fm, int WR, int KW, int EPI>
__global__ __launch_bounds__(KW * 64) void gemm_f16_kernel(MmArgs a) {
  __shared__ f32x4 red[KW][WR][64];
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[KW][2][kXTile];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  // Q6_K: the selector of the lane's scale bytes 2j + q / 2 (q6_head)
  const uint32_t sel6 = (uint32_t)(q >> 1) * 0x01010101u + 0x06040200u;

  // the group of this m-tile (groups are few; a linear scan on scalars)
  MmTile grp;
  if (!find_group(a, 16, grp)) return;
  const int m0 = grp.m_begin + ((int)blockIdx.y - grp.mtile0) * 16;  // first activation row
  const int m_end = grp.m_begin + grp.m_count;
  const int r0 = blockIdx.x * 16 * WR;

  // buffers over this workgroup's weight rows and activation rows (loads past
  // them return zero); per-lane offsets are fixed, super-block offsets scalar
  const int wrows = min(16 * WR, a.rows - r0);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + grp.w_off + (int64_t)r0 * a.row_bytes), (short)0, (int)(wrows * a.row_bytes), 0x00020000);
  const int xrows = min(16, m_end - m0);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + (int64_t)m0 * a.cols), (short)0, (int)(xrows * a.cols * 4), 0x00020000);
  int wv[WR];
#pragma unroll
  for (int t = 0; t < WR; ++t) wv[t] = min(16 * t + i, wrows - 1) * (int)a.row_bytes;
  const bool ragged = (a.cols & 255) != 0;

  // this wave's super-blocks: wave, wave + KW, ... (n of them); requests past
  // the last one re-read it (their results are never used)
  const int n = a.nsb > wave ? (a.nsb - wave + KW - 1) / KW : 0;
  auto fetch = [&](WStage<Fm, WR>& st, int slot, int k) {
    const int sb = wave + KW * (k < n ? k : n - 1);
    // every offset in the per-lane part (the buffer's range check covers it);
    // a ragged row's tail is clamped to the next row's start (cleared later)
    const int col = min(256 * sb + 4 * lane, a.cols) * 4;
    issue_fence();
#pragma unroll
    for (int r = 0; r < 16; ++r) load_lds16(xrs, &xbuf[wave][slot][r * kXRow], r * a.cols * 4 + col, 0);
    fetch_w<Fm, WR>(st, wrs, wv, q, sb, a.code_off);
    issue_fence();
  };
  // vector-memory operations of one fetch (they retire in order)
  constexpr int kFetchOps = 16 + fetch_w_ops<Fm>() * WR;

  f32x4 acc[WR];
#pragma unroll
  for (int t = 0; t < WR; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WStage<Fm, WR>& st, int slot, int k) {
    const int sb = wave + KW * k;
    // this stage's loads (one fetch was issued after them)
    wait_vmcnt<kFetchOps>();
    // lane (i, q): columns 8q..8q+7 of each sub-block of activation row i
    f32x4 xr[16];
    const uint8_t* xt = &xbuf[wave][slot][i * kXRow + 32 * q];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xr[2 * j] = *(const f32x4*)(xt + 128 * j);
      xr[2 * j + 1] = *(const f32x4*)(xt + 128 * j + 16);
    }
    if (ragged && sb == a.nsb - 1) {
      // columns past cols read the next row (or zero): clear them
      const int cbase = 256 * sb + 8 * q;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (cbase + 32 * j + e >= a.cols) xr[2 * j + e / 4][e % 4] = 0.f;
    }
    // the row's largest magnitude over the super-block (lanes i, i+16, i+32, i+48)
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xr[c].x), fabsf(xr[c].y)), fmaxf(fabsf(xr[c].z), fabsf(xr[c].w))));
    mx = fmaxf(mx, lane_xor(mx, 16));
    mx = fmaxf(mx, lane_xor(mx, 32));
    // 2^e with the largest magnitude in [2^9, 2^10): e = 136 - biased exponent
    int e = 0;
    if (mx > 0.f) {
      const int be = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF);
      e = 136 - be;
      e = e > 126 ? 126 : (e < -126 ? -126 : e);
    }
    const float s = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
    const float sinv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
    // 2^-e of the four activation rows whose outputs this lane holds (4q..4q+3)
    float sv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sv[c] = lane_read(sinv, 4 * q + c);

    // the activation operands of sub-block (or block) j
    auto x_operands = [&](int j, h8& xh, h8& xl) {
      const f32x4 a0 = xr[2 * j], a1 = xr[2 * j + 1];
      uint32_t hi[4], lo[4];
      split2(a0.x, a0.y, s, hi[0], lo[0]);
      split2(a0.z, a0.w, s, hi[1], lo[1]);
      split2(a1.x, a1.y, s, hi[2], lo[2]);
      split2(a1.z, a1.w, s, hi[3], lo[3]);
      xh = as_h8(hi[0], hi[1], hi[2], hi[3]);
      xl = as_h8(lo[0], lo[1], lo[2], lo[3]);
    };
    if constexpr (Fm::kKind == 0) {
      RowHead h[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) h[t] = decode_head(st.hd[t]);
      f32x4 p1[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) p1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      float ps[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh, xl;
        x_operands(j, xh, xl);
        const f32x4 a0 = xr[2 * j], a1 = xr[2 * j + 1];
        ps[j] = ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w));
#pragma unroll
        for (int t = 0; t < WR; ++t) {
          const u32x2 c = st.cw[t][j >> 1];
          const h2 sc = {h[t].sc[j], h[t].sc[j]}, nsc = {h[t].nsc[j], h[t].nsc[j]};
          const h8 wop = weight_op_j<Fm>(j, c, st.qh[t], sc, nsc);
          p1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, wop, p1[t], 0, 0, 0);
          p1[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, wop, p1[t], 0, 0, 0);
        }
      }
      uint32_t mh[4], ml[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) split2(ps[2 * c], ps[2 * c + 1], s, mh[c], ml[c]);
      const h8 mhi = as_h8(mh[0], mh[1], mh[2], mh[3]);
      const h8 mlo = as_h8(ml[0], ml[1], ml[2], ml[3]);
#pragma unroll
      for (int t = 0; t < WR; ++t) {
        f32x4 p2 = {0.f, 0.f, 0.f, 0.f};
        p2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(mhi, h[t].mop, p2, 0, 0, 0);
        p2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(mlo, h[t].mop, p2, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float v = __builtin_fmaf(h[t].d, p1[t][c], -(h[t].dmin * p2[c]));
          acc[t][c] = __builtin_fmaf(v, sv[c], acc[t][c]);
        }
      }
    } else if constexpr (Fm::kKind == 3) {
      // Q6_K: two exact weight operands per slice into two sums, d per step
      const int sh = 2 * (sb & 1);
      Q6Head hd[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) hd[t] = q6_head(st, t, sh, sel6);
      f32x4 ph[WR], pl[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) ph[t] = pl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh, xl;
        x_operands(j, xh, xl);
#pragma unroll
        for (int t = 0; t < WR; ++t) {
          h8 ahi, alo;
          q6_operands(st, t, j, sh, hd[t], ahi, alo);
          ph[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, ahi, ph[t], 0, 0, 0);
          pl[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, alo, pl[t], 0, 0, 0);
          ph[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, ahi, ph[t], 0, 0, 0);
          pl[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, alo, pl[t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < WR; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[t][c] = __builtin_fmaf(hd[t].d * (ph[t][c] + pl[t][c]), sv[c], acc[t][c]);
    } else {
      // Q8_0, Q5_0: block j's product scaled by its d, per block
      const int real = a.nb - 8 * sb;  // blocks of this step inside the row
      u32x4 d4[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) d4[t] = blk_head(st, t, i);
      f32x4 pd[WR];
#pragma unroll
      for (int t = 0; t < WR; ++t) pd[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh, xl;
        x_operands(j, xh, xl);
#pragma unroll
        for (int t = 0; t < WR; ++t) {
          float d;
          const h8 wop = blk_operand(st, d4[t], t, j, i, q, j < real, d);
          f32x4 p = {0.f, 0.f, 0.f, 0.f};
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh, wop, p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl, wop, p, 0, 0, 0);
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) pd[t][c4] = __builtin_fmaf(d, p[c4], pd[t][c4]);
        }
      }
#pragma unroll
      for (int t = 0; t < WR; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[t][c] = __builtin_fmaf(pd[t][c], sv[c], acc[t][c]);
    }
  };

  WStage<Fm, WR> sa, sbuf;
  if (n > 0) {
    fetch(sa, 0, 0);
    for (int k = 0; k < n; k += 2) {
      fetch(sbuf, 1, k + 1);
      compute(sa, 0, k);
      fetch(sa, 0, k + 2);
      if (k + 1 < n) compute(sbuf, 1, k + 1);
    }
    wait_vmcnt<0>();  // the last (unused) requests land before the LDS is left
  }

  // add the waves' products in wave order and store: lane (i, q) of row
  // tile t holds Y[m0 + 4q + c][r0 + 16t + i]
#pragma unroll
  for (int t = 0; t < WR; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  for (int t = wave; t < WR; t += KW) {
    f32x4 v = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      const f32x4 o = red[w][t][lane];
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
    }
    const int r = r0 + 16 * t + i;
    if (r < a.rows) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int m = m0 + 4 * q + c;
        if (m < m_end) mm_out<EPI>(a.Y + (int64_t)m * a.rows + r, v[c]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Shared-activation kernel: a workgroup of RS x KS waves owns 16 RS R weight
// rows (wave group row w: rows 16 R w .. 16 R w + 16 R - 1) and 16 C
// activation rows; wave group k (RS waves) takes the 256-column steps k,
// k + KS, ... Each step's activation tile is converted once, by the group's
// waves together, into the fp16 operand fragments in LDS, and every wave
// multiplies it against its own weight rows; so the conversion is paid once
// per 16 RS R weight rows instead of once per 16 WR. KS > 1 groups add their
// sums in LDS in group order at the end.
//
// Pipeline, per step k: the raw activation rows and the weight bytes of step
// k + D are requested (register rings; D steps in flight), step k is
// multiplied (LDS buffer k % 2), step k + 1 is converted into the other LDS
// buffer, and one barrier ends the step.

// One operand fragment (64 lanes x 16 bytes): lane L's 16 bytes sit at
// (L / 16) * 272 + (L % 16) * 16. The 16-byte gap after each group of 16
// lanes spreads the conversion's writes (one activation row at a time) over
// all bank groups; the operand reads stay conflict-free.
constexpr int kFragGroup = 272;
constexpr int kFragBytes = 4 * kFragGroup;
constexpr int kMinFrag = 16;  // fragments 0-7: hi parts of sub-blocks 0-7, 8-15: lo parts,
                              // 16, 17: the min-term hi and lo parts
// one 16-row m-tile of one 256-column step: K-quants 18 fragments, Q8_0 16
// (no min term)
template <class Fm>
constexpr int tile_bytes() {
  return (Fm::kKind == 0 ? 18 : 16) * kFragBytes;
}

// fp16 parts of a * s: hi = fp16(a s), lo = fp16(a s - hi), in the low halves.
__device__ __forceinline__ void split1(float a, float s, uint32_t& hi, uint32_t& lo) {
  __asm__("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
          "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]"
          : "=&v"(hi), "=&v"(lo)
          : "v"(a), "v"(s));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ f32x4 buf_f32x4(__amdgpu_buffer_rsrc_t rs, int voff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
}

template <class Fm, int R, int C, int D, int KS, int RS, int EPI>
__global__ __launch_bounds__(64 * RS * KS) void gemm_f16_xs_kernel(MmArgs a) {
  static_assert(RS == 4 || (RS == 8 && C % 2 == 0), "row groups");
  constexpr int CW = C * 4 / RS;          // m-tiles each wave converts
  constexpr int SW = D + 1;               // weight ring slots
  constexpr int SX = D == 1 ? 1 : D + 1;  // activation ring slots (divides SW)
  // hi and lo products in separate accumulators when there are too few
  // independent MFMA chains to cover the dependent-issue latency
  constexpr bool kSplitAcc = R * C < 4;
  constexpr int kTileBytes = tile_bytes<Fm>();
  constexpr int kStage = C * kTileBytes;
  __shared__ __attribute__((aligned(16))) uint8_t xs[KS][2][kStage];
  __shared__ __attribute__((aligned(16))) float xsv[KS][2][16 * C];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave % RS;  // weight-row group
  const int wk = wave / RS;  // super-block group: super-blocks wk, wk + KS, ...
  const int i = lane & 15, q = lane >> 4;
  const uint32_t sel6 = (uint32_t)(q >> 1) * 0x01010101u + 0x06040200u;  // Q6_K: q6_head

  MmTile grp;
  if (!find_group(a, 16 * C, grp)) return;
  const int m0 = grp.m_begin + ((int)blockIdx.y - grp.mtile0) * 16 * C;
  const int m_end = grp.m_begin + grp.m_count;
  const int r0 = blockIdx.x * 16 * RS * R;

  // weight rows of the workgroup (each lane's row clamped to a real one) and
  // activation rows of the tile (rows past the group read as zero)
  const int wrows = min(16 * RS * R, a.rows - r0);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + grp.w_off + (int64_t)r0 * a.row_bytes), (short)0, (int)(wrows * a.row_bytes), 0x00020000);
  const int xrows = min(16 * C, m_end - m0);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + (int64_t)m0 * a.cols), (short)0, (int)(xrows * a.cols * 4), 0x00020000);
  int wv[R];
#pragma unroll
  for (int t = 0; t < R; ++t) wv[t] = min(16 * (wr * R + t) + i, wrows - 1) * (int)a.row_bytes;
  const int n = a.nsb;
  const int nk = n > wk ? (n - wk + KS - 1) / KS : 0;  // this group's super-blocks
  const int nsteps = (n + KS - 1) / KS;                // the workgroup's steps (every group)

  // conversion: wave wr of a group converts rows w, w + 4, w + 8, w + 12
  // (w = wr % 4) of m-tiles wr / 4, wr / 4 + RS / 4, ..., one per 16-lane
  // row of the wave (r = lane / 16); in request v (0..3) lane l = lane % 16
  // holds columns 64 v + 4 l .. + 3, which are half of operand lane
  // (row, (l % 8) / 2) of sub-block 2 v + l / 8
  const int cr = lane >> 4, cl = lane & 15;
  const int ci = (wr & 3) + 4 * cr;  // the lane's row within each m-tile
  const int cb = wr >> 2;            // the first m-tile it converts
  const int cv_off = (cl >> 3) * kFragBytes + ((cl >> 1) & 3) * kFragGroup + ci * 16 + (cl & 1) * 8;
  const int cm_off = kMinFrag * kFragBytes + ((cl >> 1) & 3) * kFragGroup + ci * 16 + 2 * (cl >> 3);
  int xv[CW];  // byte offset of the lane's activation row of each m-tile it converts
#pragma unroll
  for (int c = 0; c < CW; ++c) xv[c] = (16 * (cb + c * RS / 4) + ci) * a.cols * 4;
  // operand reads: lane (i, q)
  const int rd_off = q * kFragGroup + i * 16;

  f32x4 xr[SX][CW][4];
  WStage<Fm, R> ws[SW];

  // the group's k-th super-block (k past the last re-reads the last; a group
  // with no super-block -- fewer super-blocks than groups -- re-reads
  // super-block 0, so that the scalar part of every weight load's offset,
  // which the buffer's range check does not cover, is a real position)
  auto sb_of = [&](int k) { return nk > 0 ? wk + KS * (k < nk ? k : nk - 1) : 0; };

  // requests for super-block sb (the column offset is clamped so that a
  // ragged row's tail stays inside the buffer)
  auto fetch = [&](int sb, int xslot, int wslot) {
    int col[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) col[v] = min(256 * sb + 64 * v + 4 * cl, a.cols) * 4;
    issue_fence();
#pragma unroll
    for (int c = 0; c < CW; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) xr[xslot][c][v] = buf_f32x4(xrs, xv[c] + col[v]);
    fetch_w<Fm, R>(ws[wslot], wrs, wv, q, sb, a.code_off);
    issue_fence();
  };

  // super-block sb's activation rows -> the group's LDS buffer buf
  auto convert = [&](int sb, int xslot, int buf) {
    uint8_t* base = &xs[wk][buf][0];
    if ((a.cols & 255) != 0 && sb == n - 1) {  // ragged last super-block: clear columns past the row
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (256 * sb + 64 * v + 4 * cl >= a.cols)
#pragma unroll
          for (int c = 0; c < CW; ++c) xr[xslot][c][v] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int ct = cb + c * RS / 4;  // the m-tile
      // the row's largest magnitude: 16 values per lane, then its 16 lanes
      float m = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const f32x4 x = xr[xslot][c][v];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
      }
      uint32_t mb = __builtin_bit_cast(uint32_t, m);
      mb = max(mb, dpp_u32<0xB1>(mb));   // quad_perm [1,0,3,2]
      mb = max(mb, dpp_u32<0x4E>(mb));   // quad_perm [2,3,0,1]
      mb = max(mb, dpp_u32<0x141>(mb));  // row_half_mirror
      mb = max(mb, dpp_u32<0x140>(mb));  // row_mirror
      // 2^e with the row's largest magnitude in [2^9, 2^10)
      int e = mb != 0 ? 136 - (int)(mb >> 23) : 0;
      e = e > 126 ? 126 : (e < -126 ? -126 : e);
      const float s = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
      uint8_t* tile = base + ct * kTileBytes;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const f32x4 x = xr[xslot][c][v];
        uint32_t h0, l0, h1, l1;
        split2(x.x, x.y, s, h0, l0);
        split2(x.z, x.w, s, h1, l1);
        *(u32x2*)(tile + 2 * v * kFragBytes + cv_off) = u32x2{h0, h1};
        *(u32x2*)(tile + (8 + 2 * v) * kFragBytes + cv_off) = u32x2{l0, l1};
        if constexpr (Fm::kKind == 0) {
          // this lane pair's 8 columns summed, for the min term
          const float s4 = (x.x + x.y) + (x.z + x.w);
          const float s8 = s4 + __builtin_bit_cast(float, dpp_u32<0xB1>(__builtin_bit_cast(uint32_t, s4)));
          if ((cl & 1) == 0) {
            uint32_t mh, ml;
            split1(s8, s, mh, ml);
            *(uint16_t*)(tile + cm_off + 4 * v) = (uint16_t)mh;
            *(uint16_t*)(tile + cm_off + 4 * v + kFragBytes) = (uint16_t)ml;
          }
        }
      }
      if (cl == 0) xsv[wk][buf][16 * ct + ci] = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
    }
  };

  f32x4 acc[R][C];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Q8_0, Q5_0: one block per k-slice, each slice's product scaled by its d
  auto compute_q8 = [&](int wslot, int buf, int sb) {
    if constexpr (Fm::kKind == 1 || Fm::kKind == 2 || Fm::kKind == 4) {
      const uint8_t* base = &xs[wk][buf][0];
      const int real = a.nb - 8 * sb;  // blocks of this step inside the row
      u32x4 d4[R];
#pragma unroll
      for (int t = 0; t < R; ++t) d4[t] = blk_head(ws[wslot], t, i);
      f32x4 pd[R][C];
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) pd[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh[C], xl[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xh[c] = *(const h8*)(base + c * kTileBytes + j * kFragBytes + rd_off);
          xl[c] = *(const h8*)(base + c * kTileBytes + (8 + j) * kFragBytes + rd_off);
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
          float d;
          const h8 wop = blk_operand(ws[wslot], d4[t], t, j, i, q, j < real, d);
#pragma unroll
          for (int c = 0; c < C; ++c) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[c], wop, p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[c], wop, p, 0, 0, 0);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) pd[t][c][cc] = __builtin_fmaf(d, p[cc], pd[t][c][cc]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f32x4 sv = *(const f32x4*)&xsv[wk][buf][16 * c + 4 * q];
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) acc[t][c][cc] = __builtin_fmaf(pd[t][c][cc], sv[cc], acc[t][c][cc]);
      }
    }
  };

  // Q6_K: two exact weight operands per slice into two sums, d per step
  auto compute_q6 = [&](int wslot, int buf, int sb) {
    if constexpr (Fm::kKind == 3) {
      const uint8_t* base = &xs[wk][buf][0];
      const int sh = 2 * (sb & 1);
      Q6Head hd[R];
#pragma unroll
      for (int t = 0; t < R; ++t) hd[t] = q6_head(ws[wslot], t, sh, sel6);
      f32x4 ph[R][C], pl[R][C];
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) ph[t][c] = pl[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh[C], xl[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xh[c] = *(const h8*)(base + c * kTileBytes + j * kFragBytes + rd_off);
          xl[c] = *(const h8*)(base + c * kTileBytes + (8 + j) * kFragBytes + rd_off);
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
          h8 ahi, alo;
          q6_operands(ws[wslot], t, j, sh, hd[t], ahi, alo);
#pragma unroll
          for (int c = 0; c < C; ++c) {
            ph[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[c], ahi, ph[t][c], 0, 0, 0);
            pl[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[c], alo, pl[t][c], 0, 0, 0);
            ph[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[c], ahi, ph[t][c], 0, 0, 0);
            pl[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[c], alo, pl[t][c], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f32x4 sv = *(const f32x4*)&xsv[wk][buf][16 * c + 4 * q];
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
            acc[t][c][cc] = __builtin_fmaf(hd[t].d * (ph[t][c][cc] + pl[t][c][cc]), sv[cc], acc[t][c][cc]);
      }
    }
  };

  auto compute = [&](int wslot, int buf) {
    if constexpr (Fm::kKind == 0) {
      const uint8_t* base = &xs[wk][buf][0];
      RowHead h[R];
#pragma unroll
      for (int t = 0; t < R; ++t) h[t] = decode_head(ws[wslot].hd[t]);
      f32x4 ph[R][C], pl[R][C];
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) ph[t][c] = pl[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h8 xh[C], xl[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xh[c] = *(const h8*)(base + c * kTileBytes + j * kFragBytes + rd_off);
          xl[c] = *(const h8*)(base + c * kTileBytes + (8 + j) * kFragBytes + rd_off);
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
          const u32x2 cw = ws[wslot].cw[t][j >> 1];
          const h2 sc = {h[t].sc[j], h[t].sc[j]}, nsc = {h[t].nsc[j], h[t].nsc[j]};
          const h8 wop = weight_op_j<Fm>(j, cw, ws[wslot].qh[t], sc, nsc);
#pragma unroll
          for (int c = 0; c < C; ++c) {
            ph[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[c], wop, ph[t][c], 0, 0, 0);
            if constexpr (kSplitAcc)
              pl[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[c], wop, pl[t][c], 0, 0, 0);
            else
              ph[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[c], wop, ph[t][c], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const h8 mh = *(const h8*)(base + c * kTileBytes + kMinFrag * kFragBytes + rd_off);
        const h8 ml = *(const h8*)(base + c * kTileBytes + (kMinFrag + 1) * kFragBytes + rd_off);
        const f32x4 sv = *(const f32x4*)&xsv[wk][buf][16 * c + 4 * q];
#pragma unroll
        for (int t = 0; t < R; ++t) {
          f32x4 p2 = {0.f, 0.f, 0.f, 0.f};
          p2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(mh, h[t].mop, p2, 0, 0, 0);
          p2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ml, h[t].mop, p2, 0, 0, 0);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const float p1 = kSplitAcc ? ph[t][c][cc] + pl[t][c][cc] : ph[t][c][cc];
            const float v = __builtin_fmaf(h[t].d, p1, -(h[t].dmin * p2[cc]));
            acc[t][c][cc] = __builtin_fmaf(v, sv[cc], acc[t][c][cc]);
          }
        }
      }
    }
  };

  // LDS writes done, then the workgroup barrier (no wait on the requests)
  auto step_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    bare_barrier();
  };

  // every group takes the same number of steps (a group with fewer
  // super-blocks idles through its last one), so the barriers match
#pragma unroll
  for (int d = 0; d < D; ++d) fetch(sb_of(d), d % SX, d % SW);
  if (nk > 0) convert(sb_of(0), 0, 0);
  step_barrier();
  for (int k0 = 0; k0 < nsteps; k0 += SW) {
#pragma unroll
    for (int u = 0; u < SW; ++u) {
      const int k = k0 + u;
      if (k < nsteps) {
        fetch(sb_of(k + D), (u + D) % SX, (u + D) % SW);
        if (k < nk) {
          if constexpr (Fm::kKind == 0) compute(u, k & 1);
          else if constexpr (Fm::kKind == 3) compute_q6(u, k & 1, sb_of(k));
          else compute_q8(u, k & 1, sb_of(k));
        }
        if (k + 1 < nk) convert(sb_of(k + 1), (u + 1) % SX, (k + 1) & 1);
        step_barrier();
      }
    }
  }

  // groups 1.. park their sums in LDS; group 0 adds them in group order
  if constexpr (KS > 1) {
    f32x4* red = (f32x4*)&xs[0][0][0];  // [KS - 1][RS][R][C][64]
    if (wk > 0) {
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) red[((((wk - 1) * RS + wr) * R + t) * C + c) * 64 + lane] = acc[t][c];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    bare_barrier();
    if (wk > 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int t = 0; t < R; ++t)
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const f32x4 o = red[((((g - 1) * RS + wr) * R + t) * C + c) * 64 + lane];
          acc[t][c] = f32x4{acc[t][c].x + o.x, acc[t][c].y + o.y, acc[t][c].z + o.z, acc[t][c].w + o.w};
        }
  }

#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int r = r0 + 16 * (wr * R + t) + i;
    if (r < a.rows) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int m = m0 + 16 * c + 4 * q + cc;
          if (m < m_end) mm_out<EPI>(a.Y + (int64_t)m * a.rows + r, acc[t][c][cc]);
        }
    }
  }
}

#ifndef GQ_MM_KW
#define GQ_MM_KW 4  // waves per workgroup (splitting the super-blocks)
#endif

template <class Fm, int WR, int EPI>
hipError_t launch(const MmArgs& a, int gx, int gy, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f16_kernel<Fm, WR, GQ_MM_KW, EPI>), dim3(gx, gy), dim3(GQ_MM_KW * 64), 0, s, a);
  return hipGetLastError();
}

template <class Fm, int R, int C, int D, int KS, int RS, int EPI>
hipError_t launch_xs(const MmArgs& a, int gy, hipStream_t s) {
  const int gx = (a.rows + 16 * RS * R - 1) / (16 * RS * R);
  hipLaunchKernelGGL((gemm_f16_xs_kernel<Fm, R, C, D, KS, RS, EPI>), dim3(gx, gy), dim3(64 * RS * KS), 0, s, a);
  return hipGetLastError();
}

// m-tiles of tm activation rows over the groups (the grid's y).
int64_t count_mtiles(const int64_t* group_m, int n_groups, int tm) {
  int64_t gy = 0;
  for (int g = 0; g < n_groups; ++g) gy += (group_m[g] + tm - 1) / tm;
  return gy;
}

// The group table for m-tiles of tm activation rows; returns the number of
// m-tiles (the grid's y), or -1 when the groups exceed the table.
int build_groups(MmArgs& m, const int64_t* group_m, const int64_t* group_off, int n_groups,
                 int64_t group_w_bytes, int tm) {
  int gy = 0, ng = 0;
  for (int g = 0; g < n_groups; ++g) {
    if (group_m[g] == 0) continue;
    if (ng == kMaxGroups) return -1;
    m.g[ng] = MmTile{group_w_bytes * g, (int)group_off[g], (int)group_m[g], gy};
    gy += (int)((group_m[g] + tm - 1) / tm);
    ++ng;
  }
  m.n_groups = ng;
  return gy;
}

}  // namespace

bool gemm_f16_fits(int64_t rows, int64_t cols, int64_t row_bytes) {
  // 31-bit buffer offsets: 256 weight rows and 64 activation rows of a tile
  return 256 * row_bytes < ((int64_t)1 << 31) && 64 * cols * 4 < ((int64_t)1 << 31) && rows <= INT32_MAX;
}

// Tile choice, measured on MI355X (Q4_K 14336 x 4096 gate / 4096 x 14336
// down). K-quants: the shared-activation tile with the least time, counted
// as rounds of one workgroup per CU times a relative workgroup time --
// 256 x 64 (100; gate M = 512: 189 us), 256 x 32 (70; down M = 512: 211 us),
// 128 x 32 split in two along k (44; gate M = 64: 39 us), 64 x 16 split in
// four (21; gate M = 16: 20 us, down M = 64: 54 us); the last only for grids
// of 3/4 of the CUs, or a quarter for rows of at most 4 steps -- else the
// per-wave kernel with as many weight-row tiles per workgroup as still fill
// the GPU (down M = 16: 31 us). Counting rounds matters between the sizes:
// at M = 160 the gate takes one round of 256 x 64 (94 us) rather than two of
// 256 x 32 (124 us). The other layouts take the largest tile their registers
// allow whose grid fills about every CU (below).
namespace {

template <class Fm, int EPI>
hipError_t launch_gemm_f16_epi(MmArgs& m, const GemmArgs& a, const int64_t* group_m, const int64_t* group_off,
                               int n_groups, int64_t group_w_bytes, int cus, hipStream_t s) {
  const int64_t fill = (int64_t)cus * 7 / 8;
  // the 64 x 16 shared tile from 3/4 of the CUs, and for rows of at most 4
  // steps from a quarter of them: measured faster than the per-wave kernel
  // there (8B down at M = 48: 55 against 68 us; 4864 x 896 at M = 32: 8.8
  // against 16 us), and slower below
  const bool xs16 = [&] {
    const int64_t g = ((a.rows + 63) / 64) * count_mtiles(group_m, n_groups, 16);
    return g >= (int64_t)cus * 3 / 4 || (m.nsb <= 4 && g >= cus / 4);
  }();
  auto grid = [&](int tr, int tm) { return ((a.rows + tr - 1) / tr) * count_mtiles(group_m, n_groups, tm); };
  // the grid's y: the m-tiles of the host table, or with device counts the
  // most the total can need (each non-empty group wastes under one m-tile)
  auto grid_y = [&](int tm) {
    if (m.dev_m) return (int)((m.dev_total + tm - 1) / tm + m.n_groups);
    return build_groups(m, group_m, group_off, n_groups, group_w_bytes, tm);
  };
  auto run_xs = [&](auto launch, int tm) {
    const int gy = grid_y(tm);
    if (gy < 0) return hipErrorInvalidValue;
    if (gy == 0) return hipSuccess;
    return launch(m, gy, s);
  };
  // per layout, the tiles whose registers fit without spilling
  if constexpr (Fm::kKind == 0) {
    // the tile with the least time: rounds of one workgroup per CU times the
    // tile's workgroup time (relative, measured on the Llama gate and down)
    auto cost = [&](int tr, int tm, int64_t w) { return (grid(tr, tm) + cus - 1) / cus * w; };
    const int64_t c0 = cost(256, 64, 100), c1 = cost(256, 32, 70), c2 = cost(128, 32, 44), c3 = cost(64, 16, 21);
    const int64_t best = min(min(c0, c1), min(c2, c3));
    if (c3 == best) {
      if (xs16) return run_xs(launch_xs<Fm, 1, 1, 1, 4, 4, EPI>, 16);
    } else if (c2 == best) {
      return run_xs(launch_xs<Fm, 1, 2, 1, 2, 8, EPI>, 32);
    } else if (c1 == best) {
      return run_xs(launch_xs<Fm, 2, 2, 2, 1, 8, EPI>, 32);
    } else {
      return run_xs(launch_xs<Fm, 2, 4, 1, 1, 8, EPI>, 64);
    }
  } else if constexpr (Fm::kKind == 2) {
    // Q8_0 steps carry twice the weight bytes per lane: 16-row tiles per wave
    if (grid(128, 64) >= fill) return run_xs(launch_xs<Fm, 1, 4, 1, 1, 8, EPI>, 64);
    if (grid(128, 32) >= fill) return run_xs(launch_xs<Fm, 1, 2, 1, 2, 8, EPI>, 32);
    if (xs16) return run_xs(launch_xs<Fm, 1, 1, 1, 4, 4, EPI>, 16);
  } else if constexpr (Fm::kKind == 3) {
    if (grid(128, 64) >= fill) return run_xs(launch_xs<Fm, 1, 4, 1, 1, 8, EPI>, 64);
    if (grid(128, 32) >= fill) return run_xs(launch_xs<Fm, 1, 2, 1, 1, 8, EPI>, 32);
    if (xs16) return run_xs(launch_xs<Fm, 1, 1, 1, 4, 4, EPI>, 16);
  } else {
    // packed Q8_0 and Q5_0 also hold 12 bytes per even block: 8-wave tiles only
    if (grid(128, 32) >= fill) return run_xs(launch_xs<Fm, 1, 2, 1, 1, 8, EPI>, 32);
    if (xs16) return run_xs(launch_xs<Fm, 1, 1, 1, 2, 4, EPI>, 16);
  }
  const int gy = grid_y(16);
  if (gy < 0) return hipErrorInvalidValue;
  if (gy == 0) return hipSuccess;
  if (grid(32, 16) >= fill) return launch<Fm, 2, EPI>(m, (a.rows + 31) / 32, gy, s);
  return launch<Fm, 1, EPI>(m, (a.rows + 15) / 16, gy, s);
}

template <class Fm>
hipError_t launch_gemm_fmt(MmArgs& m, const GemmArgs& a, const int64_t* group_m, const int64_t* group_off,
                           int n_groups, int64_t group_w_bytes, int cus, hipStream_t s, int epi) {
  switch (epi) {
    case kMmStore:
      return launch_gemm_f16_epi<Fm, kMmStore>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s);
    case kMmAcc:
      return launch_gemm_f16_epi<Fm, kMmAcc>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s);
    case kMmSiluMul:
      return launch_gemm_f16_epi<Fm, kMmSiluMul>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_f16(int fmt, const GemmArgs& a, const int64_t* group_m, const int64_t* group_off,
                           int n_groups, int64_t group_w_bytes, int cus, hipStream_t s, int epi) {
  MmArgs m{};
  m.W = a.W;
  m.X = a.X;
  m.Y = a.Y;
  m.row_bytes = a.row_bytes;
  m.rows = a.rows;
  m.cols = a.cols;
  m.nsb = (a.cols + 255) / 256;
  m.nb = (a.cols + 31) / 32;
  m.code_off = split_scale_bytes(m.nb);
  switch (fmt) {
    case kFmtQ4_K: return launch_gemm_fmt<MmQ4K>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    case kFmtQ5_K: return launch_gemm_fmt<MmQ5K>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    case kFmtQ8_0: return launch_gemm_fmt<MmQ8P>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    case kFmtQ8_0Split:
      return launch_gemm_fmt<MmQ8S>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    case kFmtQ6_K: return launch_gemm_fmt<MmQ6K>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    case kFmtQ5_0: return launch_gemm_fmt<MmQ50>(m, a, group_m, group_off, n_groups, group_w_bytes, cus, s, epi);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_f16_dev(int fmt, const GemmArgs& a, const int64_t* dev_m, int n_expert, int total,
                               int64_t group_w_bytes, int cus, hipStream_t s) {
  MmArgs m{};
  m.W = a.W;
  m.X = a.X;
  m.Y = a.Y;
  m.row_bytes = a.row_bytes;
  m.rows = a.rows;
  m.cols = a.cols;
  m.nsb = (a.cols + 255) / 256;
  m.nb = (a.cols + 31) / 32;
  m.code_off = split_scale_bytes(m.nb);
  m.n_groups = n_expert;
  m.dev_m = dev_m;
  m.dev_w_bytes = group_w_bytes;
  m.dev_total = total;
  // the tile is chosen as for one group of all the rows
  const int64_t tm = total, off = 0;
  switch (fmt) {
    case kFmtQ4_K: return launch_gemm_fmt<MmQ4K>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    case kFmtQ5_K: return launch_gemm_fmt<MmQ5K>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    case kFmtQ8_0: return launch_gemm_fmt<MmQ8P>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    case kFmtQ8_0Split: return launch_gemm_fmt<MmQ8S>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    case kFmtQ6_K: return launch_gemm_fmt<MmQ6K>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    case kFmtQ5_0: return launch_gemm_fmt<MmQ50>(m, a, &tm, &off, 1, group_w_bytes, cus, s, kMmStore);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gq
