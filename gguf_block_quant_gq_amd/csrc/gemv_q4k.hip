// gemv_q4k.hip -- y = W x for Q4_K rows wider than one wave: 65..256 units,
// 4096 < cols <= 16384 (the 14336-column down projection of 8B-class models;
// narrower rows run on the row-group kernel of gemv.hip, which measured as
// fast or faster for them).
//
// Decode is bound by the bytes of W (nx_f32_llm_v4 source, model binder:
// bytes moved is the runtime), and for Q4_K the decode arithmetic comes close
// to the same bound: at 8 TB/s the CUs can spend only about 2.8 lane
// operations per weight. This kernel is built around both limits.
//
//  * One workgroup per CU. Output rows are dealt round-robin to the row groups
//    of the whole grid, so every wave has the same number of rows to within
//    one and at any moment the grid reads one compact window of the matrix.
//  * A row group is H waves (H = ceil(units / 64)); lane l of wave h owns unit
//    u = 64h + l of every row it visits -- the 32 code bytes of group g = u & 3
//    of super-block u >> 2 (64 weights) -- and keeps that unit's 64 x values
//    and their two sub-block sums in registers for the whole kernel.
//  * x is staged once per workgroup through LDS with coalesced loads; unit u's
//    sixteen 16-byte chunks sit at slots 17u..17u+15 and its sums at slot
//    17u+16 (the one-slot pad makes the per-lane reads conflict free and lets
//    every read use an immediate offset from one base address).
//  * Every weight row is read with buffer loads whose per-lane part (the
//    unit's header and code offsets) is fixed for the kernel and whose row
//    part is a scalar, so the row loop spends no vector instructions on
//    addressing. D rows per wave are requested before the first one is
//    decoded, and each row's slot is refilled as soon as it is consumed
//    (D = 2 measured fastest; deeper prefetch was slower on MI355X).
//  * The six-bit scale and min codes of the lane's two sub-blocks are
//    gathered into one dword with two v_perm_b32 and three masks, then
//    converted with v_cvt_f32_ubyte; nibbles become exact fp32 values with
//    v_cvt_pk_f32_fp8 (a 4-bit code read as e4m3 is code * 2^-9).
//  * The H*64 lane partial sums of a row are folded with the fixed DPP
//    butterfly and then through LDS in wave order, so the result is
//    deterministic and the same for every epilogue and batch slice.
//
// Prior art: the one-warp-per-row matvec of the "nurllama" README ("What it
// runs"), re-shaped for 64-wide wavefronts.
#include "gemv_common.h"
#include "gq_device.h"
#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kSlotsPerUnit = 17;  // 16 chunks of x + 1 chunk of sums

// A Q4_K unit of one row as it arrives: the super-block header (d, dmin,
// twelve scale bytes) and the 32 code bytes of the lane's group.
struct Q4Raw {
  u32x4 h, q0, q1;
};

// The lane's x: the unit's 64 values (sub-block 2g: a, sub-block 2g + 1: b)
// and their two sums.
struct Q4X {
  float a[32], b[32];
  float sa, sb;
};

// Sum over the unit of w * x, with the min term factored out:
//   d * (sc0 * sum(lo * xa) + sc1 * sum(hi * xb)) - dmin * (m0 * sa + m1 * sb)
// (codes arrive as code * 2^-9, so d carries the factor 2^9).
__device__ __forceinline__ float q4_dot(const Q4Raw& r, const Q4X& x, const Q4Sel& sel) {
  const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
  // four independent accumulation chains (two per sub-block)
  float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
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
  const uint32_t scm = q4_scales(r.h, sel);
  // (one v_cvt_f32_ubyte each)
  const float sc0 = (float)(scm & 0xFFu);
  const float sc1 = (float)((scm >> 8) & 0xFFu);
  const float m0 = (float)((scm >> 16) & 0xFFu);
  const float m1 = (float)(scm >> 24);
  const float d = half_bits_to_float(r.h.x & 0xFFFFu) * kFp8CodeScale;
  const float dmin = half_bits_to_float(r.h.x >> 16);
  const float qs = __builtin_fmaf(sc1, s1, sc0 * s0);
  const float ms = __builtin_fmaf(m1, x.sb, m0 * x.sa);
  return __builtin_fmaf(d, qs, -(dmin * ms));
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, soff, 0));
}

// x is staged in two halves so that its loads can be issued before the
// weight prefetch and written to LDS after it: thread t loads chunks
// t, t + T, ... (C of them, T = threads; a chunk is 4 columns, zero past
// cols), then stores them in the padded layout with the sub-block sums. The
// eight chunks of a sub-block belong to eight consecutive threads (T is a
// multiple of 64), which add them with a DPP butterfly.
template <int C>
struct XChunks {
  f32x4 v[C];
};

template <int C>
__device__ __forceinline__ void issue_x(XChunks<C>& st, const float* x, int cols) {
  // cols is a multiple of 4. No branch and no use of a loaded value before
  // the weight requests (either would make the compiler wait for the x loads
  // first): addresses are clamped here, values past cols zeroed in commit_x.
  const int last = (cols >> 2) - 1;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int q = threadIdx.x + j * blockDim.x;
    st.v[j] = load_f32x4(x + 4 * (q < last ? q : last));
  }
}

// Chunks past the row's units are zeros, so a lane whose unit lies past the
// last one reads zero x.
template <int C>
__device__ __forceinline__ void commit_x(f32x4* xs, const XChunks<C>& st, int cols) {
  const int T = blockDim.x;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int q = threadIdx.x + j * T;
    const f32x4 v = 4 * q < cols ? st.v[j] : zero;
    xs[kSlotsPerUnit * (q >> 4) + (q & 15)] = v;
    // sub-block (8 chunks = 32 columns) sum, every lane of the 8 gets it
    const float sum = group_sum_last<8>((v.x + v.y) + (v.z + v.w));
    if ((q & 7) == 0) {
      float* sums = (float*)&xs[kSlotsPerUnit * (q >> 4) + 16];
      sums[(q >> 3) & 1] = sum;
    }
  }
}

// Unit u's x from the staged layout (16 reads with immediate offsets).
__device__ __forceinline__ void fetch_x(Q4X& x, const f32x4* xs, int u) {
  const f32x4* p = xs + kSlotsPerUnit * u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const f32x4 va = p[k], vb = p[8 + k];
    x.a[4 * k] = va.x; x.a[4 * k + 1] = va.y; x.a[4 * k + 2] = va.z; x.a[4 * k + 3] = va.w;
    x.b[4 * k] = vb.x; x.b[4 * k + 1] = vb.y; x.b[4 * k + 2] = vb.z; x.b[4 * k + 3] = vb.w;
  }
  const f32x4 sm = p[16];
  x.sa = sm.x;
  x.sb = sm.y;
}

// H waves per row group, NW waves per workgroup, D rows (output items) in
// flight per wave. RI = weight rows per output row (2 for SwiGLU: gate row r
// and up row rows + r).
// Kernel arguments: the matvec's (plain or expert-batched) and the row
// split, computed on the host: rows = ng * nlo + rem over ng = gridDim.x *
// (NW / H) row groups; group g owns nlo + (g < rem) output rows.
template <bool EXPERTS>
struct Q4kArgs {
  KernelArgs<EXPERTS> k;
  int nlo, rem;
};

// Output row of item k of row group g: rows are dealt round-robin over the
// ng groups of the grid.
__device__ __forceinline__ int item_row(int g, int k, int ng) { return g + k * ng; }

template <int NW, int H, int D, int EPI, bool EXPERTS>
__global__ __launch_bounds__(NW * 64) void gemv_q4k_kernel(Q4kArgs<EXPERTS> q4) {
  const KernelArgs<EXPERTS>& args = q4.k;
  static_assert(NW % H == 0 && (H == 1 || H == 2 || H == 4), "shape");
  constexpr int NG = NW / H;                       // row groups per workgroup
  constexpr int RI = weight_rows_per_out<EPI>();   // weight rows per output row
  constexpr int kRing = H > 1 ? 8 : 1;             // LDS partial-sum ring (H > 1)
  __shared__ f32x4 xs[kSlotsPerUnit * 64 * H];
  __shared__ float red[kRing][NG][H][RI];

  GemvArgs a = base_args(args);
  if constexpr (EXPERTS) {
    if (!bind_assignment(a, args.e)) return;  // uniform per workgroup
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave / H, hw = wave % H;
  const int u = 64 * hw + lane;
  const int u_ld = u < a.units ? u : a.units - 1;
  const Q4Sel sel = q4_sel(u & 3);

  // Row group gi of ng (over the whole grid) owns nlo or nlo + 1 output
  // rows, so every wave has the same number of rows to within one. n_all is
  // the workgroup's largest count (its first group's), so that the groups of
  // a workgroup meet the same barriers when H > 1.
  const int ng = (int)gridDim.x * NG;
  const int gi0 = (int)blockIdx.x * NG;
  const int gi = gi0 + grp;
  const int n = q4.nlo + (gi < q4.rem ? 1 : 0);
  const int n_all = q4.nlo + (gi0 < q4.rem ? 1 : 0);
  if (n_all == 0) return;  // uniform
  const int n_iter = H > 1 ? n_all : n;

  // weight rows [0, rows) and, for SwiGLU, the up rows [rows, 2 rows) as two
  // buffers; a row's offset is a scalar
  const int row_bytes = (int)a.row_bytes;
  const __amdgpu_buffer_rsrc_t rs0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.W, (short)0, (int)(a.rows * a.row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + (int64_t)a.rows * a.row_bytes), (short)0,
      RI == 2 ? (int)(a.rows * a.row_bytes) : 0, 0x00020000);
  const uint32_t voff_h = (uint32_t)(u_ld >> 2) * kQ4KBytes;
  const uint32_t voff_q = voff_h + 16u + 32u * (uint32_t)(u_ld & 3);
  auto row_of = [&](int k) {  // item k's output row, clamped to a real one
    const int r = item_row(gi, k < n ? k : n - 1, ng);
    return r < a.rows ? (r < 0 ? 0 : r) : a.rows - 1;
  };
  auto row_off = [&](int k) { return row_of(k) * row_bytes; };

  Q4Raw ring[D][RI];
  auto request = [&](int slot, int k) {
    const int so = row_off(k);
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const __amdgpu_buffer_rsrc_t rs = i == 0 ? rs0 : rs1;
      ring[slot][i].h = buf_load16(rs, voff_h, so);
      ring[slot][i].q0 = buf_load16(rs, voff_q, so);
      ring[slot][i].q1 = buf_load16(rs, voff_q + 16u, so);
    }
  };

  // x is requested first (it gates the first dot), then the first D rows;
  // x is written to LDS while the rows are in flight
  constexpr int kXC = (16 * 64 * H) / (NW * 64);  // x chunks per thread
  XChunks<kXC> xst;
  issue_x<kXC>(xst, a.x, a.cols);
#pragma unroll
  for (int j = 0; j < D; ++j) request(j, j);
  commit_x<kXC>(xs, xst, a.cols);
  __syncthreads();
  Q4X x;
  fetch_x(x, xs, u);

  // H > 1: fold the ring's partial sums of items k0 .. k0 + cnt - 1
  auto flush = [&](int k0, int cnt) {
    __syncthreads();
    const int t = threadIdx.x;
    if (t < NG * kRing) {
      const int g = t / kRing, sl = t % kRing;
      const int gg = gi0 + g;
      if (sl < cnt && k0 + sl < q4.nlo + (gg < q4.rem ? 1 : 0)) {
        const int rr = item_row(gg, k0 + sl, ng);
        float v[RI];
#pragma unroll
        for (int i = 0; i < RI; ++i) {
          v[i] = red[sl][g][0][i];
#pragma unroll
          for (int w = 1; w < H; ++w) v[i] += red[sl][g][w][i];
        }
        store_row<EPI>(a.y, rr, v[0], v[RI - 1]);
      }
    }
    __syncthreads();
  };

  // Item k's sums in v: fold the lanes and store (H == 1) or park them in
  // the ring (H > 1, folded every kRing items).
  auto finish = [&](int k, float (&v)[RI]) {
#pragma unroll
    for (int i = 0; i < RI; ++i) v[i] = group_sum_last<64>(v[i]);
    if constexpr (H == 1) {
      if (lane == 63) store_row<EPI>(a.y, item_row(gi, k, ng), v[0], v[RI - 1]);
    } else {
      const int sl = k % kRing;
      if (lane == 63) {
#pragma unroll
        for (int i = 0; i < RI; ++i) red[sl][grp][hw][i] = v[i];
      }
      if (sl == kRing - 1) flush(k - (kRing - 1), kRing);
    }
  };

  // Items are decoded two at a time where possible, so that the two rows'
  // arithmetic and lane reductions interleave (one row alone leaves the
  // SIMD waiting on its dependency chains).
  auto finish2 = [&](int k, float (&v)[RI], float (&w)[RI]) {
    if constexpr (H == 1) {
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        v[i] = group_sum_last<64>(v[i]);
        w[i] = group_sum_last<64>(w[i]);
      }
      if (lane == 63) {
        store_row<EPI>(a.y, item_row(gi, k, ng), v[0], v[RI - 1]);
        store_row<EPI>(a.y, item_row(gi, k + 1, ng), w[0], w[RI - 1]);
      }
    } else {
      finish(k, v);
      finish(k + 1, w);
    }
  };

  if (n_iter <= D) {
    // every item is already requested: decode them in arrival order
#pragma unroll
    for (int j = 0; j < D; j += 2) {
      if (j + 1 < D && j + 1 < n_iter) {
        float v[RI], w[RI];
#pragma unroll
        for (int i = 0; i < RI; ++i) {
          v[i] = q4_dot(ring[j][i], x, sel);
          w[i] = q4_dot(ring[j + 1][i], x, sel);
        }
        finish2(j, v, w);
      } else if (j < n_iter) {
        float v[RI];
#pragma unroll
        for (int i = 0; i < RI; ++i) v[i] = q4_dot(ring[j][i], x, sel);
        finish(j, v);
      }
    }
  } else {
    // steady state: each slot is refilled (with item k + D, clamped to the
    // last item) as soon as it is decoded; the refills are unconditional so
    // every slot keeps its registers
    for (int k0 = 0; k0 < n_iter; k0 += D) {
#pragma unroll
      for (int j = 0; j < D; j += 2) {
        const int k = k0 + j;
        if constexpr (D >= 2) {
          float v[RI], w[RI];
#pragma unroll
          for (int i = 0; i < RI; ++i) {
            v[i] = q4_dot(ring[j][i], x, sel);
            w[i] = q4_dot(ring[j + 1][i], x, sel);
          }
          request(j, k + D);
          request(j + 1, k + 1 + D);
          if (k + 1 < n_iter) finish2(k, v, w);
          else if (k < n_iter) finish(k, v);
        } else {
          float v[RI];
#pragma unroll
          for (int i = 0; i < RI; ++i) v[i] = q4_dot(ring[j][i], x, sel);
          request(j, k + D);
          if (k < n_iter) finish(k, v);
        }
      }
    }
  }
  if constexpr (H > 1) {
    const int used = n_iter % kRing;
    if (used) flush(n_iter - used, used);
  }
}

template <int NW, int H, int D, int EPI>
hipError_t launch_q4k(const GemvArgs& a, int nwg, hipStream_t s, const ExpertArgs* ex) {
  const int ng = nwg * (NW / H);
  const int nlo = a.rows / ng, rem = a.rows % ng;
  if constexpr (EPI == kEpiStore) {
    if (ex) {
      const Q4kArgs<true> qa{GemvExpertArgs{a, *ex}, nlo, rem};
      hipLaunchKernelGGL((gemv_q4k_kernel<NW, H, D, EPI, true>), dim3(nwg, ex->n_assign), dim3(NW * 64), 0, s, qa);
      return hipGetLastError();
    }
  }
  const Q4kArgs<false> qa{a, nlo, rem};
  hipLaunchKernelGGL((gemv_q4k_kernel<NW, H, D, EPI, false>), dim3(nwg), dim3(NW * 64), 0, s, qa);
  return hipGetLastError();
}

// Launch shape (compile-time; defaults are the measured best on MI355X):
// waves per workgroup for one-wave rows, resident workgroups per CU, and the
// largest number of rows a wave requests before decoding the first.
#ifndef GQ_Q4K_NW
#define GQ_Q4K_NW 8
#endif
#ifndef GQ_Q4K_WG_PER_CU
#define GQ_Q4K_WG_PER_CU 1
#endif
#ifndef GQ_Q4K_DMAX
#define GQ_Q4K_DMAX 2
#endif

// Workgroups for a call: GQ_Q4K_WG_PER_CU per CU (shared among the
// assignments of a batched call), but at least four output rows each (two
// for H > 1).
int q4k_workgroups(const GemvArgs& a, int H, int cus, const ExpertArgs* ex) {
  const int n_assign = ex ? ex->n_assign : 1;
  int cap = cus * GQ_Q4K_WG_PER_CU / n_assign;
  if (cap < 1) cap = 1;
  const int min_rows = H == 1 ? 4 : 2;
  int nwg = (a.rows + min_rows - 1) / min_rows;
  return nwg < cap ? nwg : cap;
}

int q4k_waves_per_row(int units) { return units <= 64 ? 1 : units <= 128 ? 2 : 4; }

// D: the smallest power of two >= the rows per wave, at most GQ_Q4K_DMAX
// (4 for SwiGLU, whose items are two rows).
template <int NW, int H, int EPI>
hipError_t launch_depth(const GemvArgs& a, int nwg, int n, hipStream_t s, const ExpertArgs* ex) {
  constexpr int kMax = EPI == kEpiSwiglu && GQ_Q4K_DMAX > 4 ? 4 : GQ_Q4K_DMAX;
  if (n <= 1 || kMax == 1) return launch_q4k<NW, H, 1, EPI>(a, nwg, s, ex);
  if (n <= 2 || kMax == 2) return launch_q4k<NW, H, 2, EPI>(a, nwg, s, ex);
  if (n <= 4 || kMax == 4) return launch_q4k<NW, H, 4, EPI>(a, nwg, s, ex);
  return launch_q4k<NW, H, 8, EPI>(a, nwg, s, ex);
}

template <int EPI>
hipError_t dispatch_q4k(const GemvArgs& a, int cus, hipStream_t s, const ExpertArgs* ex) {
  const int H = q4k_waves_per_row(a.units);
  const int nwg = q4k_workgroups(a, H, cus, ex);
  if (H == 1) {
    // four-wave workgroups when there are too few rows for eight waves each
    if (GQ_Q4K_NW == 4 || a.rows < 8 * nwg) {
      const int n = (a.rows + 4 * nwg - 1) / (4 * nwg);
      return launch_depth<4, 1, EPI>(a, nwg, n, s, ex);
    }
    const int n = (a.rows + 8 * nwg - 1) / (8 * nwg);
    return launch_depth<8, 1, EPI>(a, nwg, n, s, ex);
  }
  const int ng = (8 / H) * nwg;
  const int n = (a.rows + ng - 1) / ng;
  if (H == 2) return launch_depth<8, 2, EPI>(a, nwg, n, s, ex);
  return launch_depth<8, 4, EPI>(a, nwg, n, s, ex);
}

}  // namespace

// Rows of one wave (cols <= 4096) stay on the row-group kernel of gemv.hip:
// on MI355X it measured as fast or faster there (Q4_K 4096 x 4096 4.3 against
// 4.8 us, 14336 x 4096 8.5 against 9.5 us per call); rows of two to four
// waves (the 14336-column down projection: 10.0 against 10.7 us) run here.
#ifndef GQ_Q4K_MIN_UNITS
#define GQ_Q4K_MIN_UNITS 65
#endif

bool gemv_q4k_supports(const GemvArgs& a, int cus, const ExpertArgs* ex) {
  (void)cus;
  (void)ex;
  const int units = 4 * ((a.cols + 255) / 256);
  if (units < GQ_Q4K_MIN_UNITS || units <= 32 || units > 256 || a.rows < 1 || a.cols % 4 != 0)
    return false;
  // row offsets are 31-bit buffer offsets (for SwiGLU, within each half)
  return (int64_t)a.rows * a.row_bytes < ((int64_t)1 << 31);
}

hipError_t launch_gemv_q4k(GemvArgs a, int cus, hipStream_t s, int epi, const ExpertArgs* ex) {
  a.units = 4 * ((a.cols + 255) / 256);
  if (ex && epi != kEpiStore) return hipErrorInvalidValue;
  switch (epi) {
    case kEpiStore: return dispatch_q4k<kEpiStore>(a, cus, s, ex);
    case kEpiAcc: return dispatch_q4k<kEpiAcc>(a, cus, s, nullptr);
    case kEpiSwiglu: return dispatch_q4k<kEpiSwiglu>(a, cus, s, nullptr);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gq
