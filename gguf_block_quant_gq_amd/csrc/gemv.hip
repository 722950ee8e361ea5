// gemv.hip -- y = W x for GGUF Q8_0 / Q4_K / Q5_0 / Q5_K / Q6_K weights on
// gfx950.
//
// The decode-step matrix-vector product is bound by the bytes of W
// (nx_f32_llm_v4 source, model binder: decode is memory-bandwidth bound, so
// bytes moved is the runtime). The kernel streams each packed block once,
// straight from HBM, and decodes it in registers.
//
// Work decomposition ("row groups"): the 256 threads of a workgroup form
// 256/G groups of G lanes (G a power of two, 4..256). A group owns RB rows at
// a time; its lanes split each row into units -- a Q8_0 or Q5_0 block (32
// weights), a pair of Q8_0 blocks, or a quarter of a K-quant super-block (64
// weights; gq_units.h) -- lane l owning unit l. Because a lane always owns the same unit, that unit's x
// values are loaded once into registers and reused for every row the group
// visits. Consecutive lanes own consecutive units, so each load instruction
// of a wave reads one contiguous span of a row.
//
// Workgroups loop over row batches (grid-stride); the bytes of the next batch
// are requested before the current one is decoded, so HBM latency overlaps
// the arithmetic. Loads are never predicated: a row index past the end is
// clamped to the last row (its result is discarded) and a lane whose unit
// lies past the row's last column reads a real unit of the row with zero x.
// Partial sums are folded with a fixed DPP/shuffle butterfly (and for
// G > 64 through LDS), so results are deterministic. Rows wider than G units
// are walked in segments, reloading x per segment.
//
// Prior art: the one-warp-per-row matvec of the "nurllama" README ("What it
// runs": the warp walks the row's blocks, lanes split each block, a shuffle
// reduction folds the partials), re-shaped for 64-wide wavefronts.
#include <type_traits>

#include "gemv_common.h"
#include "gq_device.h"
#include "gq_internal.h"
#include "gq_units.h"

namespace gq {

namespace {

constexpr int kThreads = 256;

// Launch-shape constants (compile-time; the defaults are the measured best
// on MI355X): resident workgroups per CU for RB = 1 and RB > 1 kernels, and
// the rows below which a group takes one row per iteration.
#ifndef GQ_GEMV_WG_PER_CU_RB1
#define GQ_GEMV_WG_PER_CU_RB1 4
#endif
#ifndef GQ_GEMV_WG_PER_CU_RBN
#define GQ_GEMV_WG_PER_CU_RBN 2
#endif
#ifndef GQ_GEMV_RBN
#define GQ_GEMV_RBN 2
#endif
#ifndef GQ_GEMV_Q8_WG_PER_CU
#define GQ_GEMV_Q8_WG_PER_CU GQ_GEMV_WG_PER_CU_RBN
#endif
#ifndef GQ_GEMV_Q8_RBN
#define GQ_GEMV_Q8_RBN GQ_GEMV_RBN
#endif
#ifndef GQ_GEMV_RB1_WAVES_PER_CU
#define GQ_GEMV_RB1_WAVES_PER_CU 8
#endif
// Q8_0 units (packed and split layouts) take one row per group up to
// 12 waves' worth of rows per CU: measured on MI355X, Q8_0 4096 x 4096
// 6.24 -> 5.55 us and 4096 x 14336 15.21 -> 14.57 us against the threshold
// of 8; the Q4_K projections of the same shapes are faster at 8.
#ifndef GQ_GEMV_Q8_RB1_WAVES_PER_CU
#define GQ_GEMV_Q8_RB1_WAVES_PER_CU 12
#endif
// Q5_K and Q6_K (more registers and ALU work per weight)
#ifndef GQ_GEMV_K56_RBN
#define GQ_GEMV_K56_RBN GQ_GEMV_RBN
#endif
#ifndef GQ_GEMV_K56_WG_PER_CU
#define GQ_GEMV_K56_WG_PER_CU GQ_GEMV_WG_PER_CU_RBN
#endif

// Unit traits: kWantsCols (lane() takes the column count and load() the lane
// constants) and kQ8Like (scheduled like the Q8_0 units); false if absent.
template <class F, class = void>
struct wants_cols : std::false_type {};
template <class F>
struct wants_cols<F, std::void_t<decltype(F::kWantsCols)>> : std::integral_constant<bool, F::kWantsCols> {};
template <class F, class = void>
struct q8_like : std::false_type {};
template <class F>
struct q8_like<F, std::void_t<decltype(F::kQ8Like)>> : std::integral_constant<bool, F::kQ8Like> {};

template <class F>
constexpr bool is_q8() {
  return std::is_same<typename F::Base, Q8Unit>::value || std::is_same<typename F::Base, Q8PairUnit>::value ||
         q8_like<F>::value;
}

template <class F>
__device__ __forceinline__ typename F::Lane make_lane(int gl, const GemvArgs& a) {
  if constexpr (wants_cols<F>::value) return F::lane(gl, a.cols);
  else return F::lane(gl);
}

template <class F>
__device__ __forceinline__ void load_unit(typename F::Raw& raw, const uint8_t* row, int unit,
                                          const typename F::Lane& ln) {
  if constexpr (wants_cols<F>::value) F::load(raw, row, unit, ln);
  else F::load(raw, row, unit);
}

template <class F>
constexpr bool is_k56() {
  return std::is_same<typename F::Base, Q5KUnit>::value || std::is_same<typename F::Base, Q6KUnit>::value;
}

// Output rows per group per batch: RB, except for the gate|up epilogue,
// where a group's two weight rows (r and rows + r) make one output.
template <int EPI, int RB>
constexpr int out_rows() {
  return EPI == kEpiSwiglu ? 1 : RB;
}

// The weight rows of a batch whose first output row is obase (clamped to
// the last row: a batch past the end re-reads it and discards the result).
template <class F, int RB, int EPI>
__device__ __forceinline__ void load_rows(typename F::Raw (&raw)[RB], const GemvArgs& a,
                                          int obase, int unit_ld, const typename F::Lane& ln) {
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    int row;
    if constexpr (EPI == kEpiSwiglu) {
      row = (obase < a.rows ? obase : a.rows - 1) + i * a.rows;  // gate, then up
    } else {
      row = obase + i;
      row = row < a.rows ? row : a.rows - 1;
    }
    load_unit<F>(raw[i], a.W + (int64_t)row * a.row_bytes, unit_ld, ln);
  }
}

// Write the finished sums of output rows obase.. (v[i] for weight row i of
// the batch): overwrite, accumulate, or the SwiGLU of the gate|up pair.
template <int EPI, int RB>
__device__ __forceinline__ void epi_store(const GemvArgs& a, int obase, const float (&v)[RB]) {
  if constexpr (EPI == kEpiSwiglu) {
    if (obase < a.rows) a.y[obase] = silu_mul(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (obase + i < a.rows) {
        if constexpr (EPI == kEpiAcc) a.y[obase + i] += v[i];
        else a.y[obase + i] = v[i];
      }
    }
  }
}

template <int G, int RB, int EPI>
__device__ __forceinline__ void reduce_store(float (&acc)[RB], const GemvArgs& a, int obase,
                                             int gl, int grp, float (*red)[RB]) {
  if constexpr (G <= 64) {
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = group_sum_last<G>(acc[i]);
    if (gl == G - 1) epi_store<EPI, RB>(a, obase, acc);
  } else {
    constexpr int kWavesPerGroup = G / 64;
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = group_sum_last<64>(acc[i]);
    const int tid = threadIdx.x;
    if ((tid & 63) == 63) {
#pragma unroll
      for (int i = 0; i < RB; ++i) red[tid >> 6][i] = acc[i];
    }
    __syncthreads();
    if (gl == 0) {
      const int w0 = grp * kWavesPerGroup;
      float v[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        v[i] = red[w0][i];
#pragma unroll
        for (int w = 1; w < kWavesPerGroup; ++w) v[i] += red[w0 + w][i];
      }
      epi_store<EPI, RB>(a, obase, v);
    }
    __syncthreads();
  }
}

// Stage the G*kChunks 16-byte chunks of x that the group's lanes own into
// LDS with coalesced loads (each wave instruction reads 1 KB of consecutive
// columns), zero past `cols`, then give every lane its own chunks. The
// chunks of unit u are stored rotated by u / (16 / kChunks) so that the 16
// lanes served together by a ds_read_b128 hit 16 different bank quads.
template <class F, int G>
__device__ __forceinline__ int x_slot(int q) {
  constexpr int C = F::kChunks;
  const int u = q / C, k = q % C;
  return C * u + ((k + u / (16 / C)) % C);
}

// Staging is split in two so that the x loads can be issued before the
// first W batch: issue_x puts the thread's share of x chunks into registers
// (no wait), commit_x writes them to LDS once they have arrived.
template <class F, int G>
struct XStage {
  static constexpr int kPerThread = (G * F::kChunks + kThreads - 1) / kThreads;
  f32x4 v[kPerThread];
};

template <class F, int G>
__device__ __forceinline__ void issue_x(XStage<F, G>& st, const float* x, int cols, int ubase) {
  constexpr int C = F::kChunks;
  const int c0 = ubase * F::kPerUnitCols;
#pragma unroll
  for (int j = 0; j < XStage<F, G>::kPerThread; ++j) {
    const int q = threadIdx.x + j * kThreads;
    const int col = c0 + 4 * q;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (q < G * C) {
      if (col + 4 <= cols) {
        v = load_f32x4(x + col);
      } else {
        v.x = col < cols ? x[col] : 0.f;
        v.y = col + 1 < cols ? x[col + 1] : 0.f;
        v.z = col + 2 < cols ? x[col + 2] : 0.f;
        v.w = col + 3 < cols ? x[col + 3] : 0.f;
      }
    }
    st.v[j] = v;
  }
}

template <class F, int G>
__device__ __forceinline__ void commit_x(f32x4* xs, const XStage<F, G>& st) {
  constexpr int C = F::kChunks;
#pragma unroll
  for (int j = 0; j < XStage<F, G>::kPerThread; ++j) {
    const int q = threadIdx.x + j * kThreads;
    if (q < G * C) xs[x_slot<F, G>(q)] = st.v[j];
  }
}

template <class F, int G>
__device__ __forceinline__ void fetch_x(typename F::X& xr, const f32x4* xs, int gl) {
  constexpr int C = F::kChunks;
  f32x4 c[C];
#pragma unroll
  for (int k = 0; k < C; ++k) c[k] = xs[x_slot<F, G>(F::x_chunk(gl, k))];
  F::set_x(xr, c);
  F::finish_x(xr);
}

// Row groups wider than a wave (G > 64) would need a barrier per batch to add
// the waves' partial sums; instead each wave parks its partials in an LDS
// ring of kSlots batches and the ring is folded (and y stored) once per
// kSlots batches, so the waves run unsynchronised in between.
template <class F, int G, int RB, int EPI, bool EXPERTS>
__global__ __launch_bounds__(kThreads) void gemv_kernel(KernelArgs<EXPERTS> args) {
  static_assert(G >= 4 && G <= kThreads && (G & (G - 1)) == 0, "G");
  GemvArgs a = base_args(args);
  if constexpr (EXPERTS) {
    if (!bind_assignment(a, args.e)) return;  // uniform per workgroup
  }
  static_assert(EPI != kEpiSwiglu || RB == 2, "the gate|up epilogue pairs two rows");
  constexpr int kGroups = kThreads / G;
  constexpr int kOut = out_rows<EPI, RB>();
  constexpr int kRowsPerIter = kGroups * kOut;  // output rows per batch
  constexpr int kWavesPerGroup = G > 64 ? G / 64 : 1;
  constexpr int kSlots = 8;
  constexpr bool kQ8 = is_q8<F>();
  __shared__ float ring[G > 64 ? kSlots : 1][kThreads / 64][RB];

  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;
  const typename F::Lane ln = make_lane<F>(gl, a);
  const int unit = gl;
  const int unit_ld = unit < a.units ? unit : a.units - 1;

  const int iters = (a.rows + kRowsPerIter - 1) / kRowsPerIter;
  const int it0 = blockIdx.x;
  if (it0 >= iters) return;  // uniform per workgroup
  const int stride = gridDim.x;

  // x is requested first, then the first W batch; x is committed to LDS
  // while the W batch is still in flight.
  __shared__ f32x4 xs[G * F::kChunks];
  XStage<F, G> st;
  issue_x<F, G>(st, a.x, a.cols, 0);
  typename F::Raw buf[RB];
  load_rows<F, RB, EPI>(buf, a, it0 * kRowsPerIter + grp * kOut, unit_ld, ln);
  commit_x<F, G>(xs, st);
  __syncthreads();
  typename F::X xr;
  fetch_x<F, G>(xr, xs, gl);

  // fold the ring: slot s holds batch it0 + (n0 + s) * stride
  auto flush = [&](int n0, int used) {
    __syncthreads();
    const int w0 = grp * kWavesPerGroup;
    if constexpr (EPI == kEpiSwiglu) {
      // one lane per slot: the gate and up sums of its output row
      if (gl < used) {
        const int s = gl;
        float v[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          v[i] = ring[s][w0][i];
#pragma unroll
          for (int w = 1; w < kWavesPerGroup; ++w) v[i] += ring[s][w0 + w][i];
        }
        epi_store<EPI, RB>(a, (it0 + (n0 + s) * stride) * kRowsPerIter + grp * kOut, v);
      }
    } else {
      // one lane per (slot, row)
      if (gl < used * RB) {
        const int s = gl / RB, i = gl % RB;
        float v = ring[s][w0][i];
#pragma unroll
        for (int w = 1; w < kWavesPerGroup; ++w) v += ring[s][w0 + w][i];
        const int row = (it0 + (n0 + s) * stride) * kRowsPerIter + grp * RB + i;
        if (row < a.rows) {
          if constexpr (EPI == kEpiAcc) a.y[row] += v;
          else a.y[row] = v;
        }
      }
    }
    __syncthreads();
  };

  int n = 0;  // batches done by this workgroup
  for (int it = it0; it < iters; it += stride, ++n) {
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = F::dot(buf[i], xr, ln);
    // The next batch's loads are unconditional: past the last batch they
    // re-read the last batch (cached, discarded), so no branch surrounds them.
    // Q4_K issues them before the reduction, Q8_0 (whose short rows make
    // more, smaller batches) after it: each order measured faster for its
    // format.
    const int nx = it + stride < iters ? it + stride : iters - 1;
    if constexpr (!kQ8) load_rows<F, RB, EPI>(buf, a, nx * kRowsPerIter + grp * kOut, unit_ld, ln);
    if constexpr (G <= 64) {
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i] = group_sum_last<G>(acc[i]);
      if (gl == G - 1) epi_store<EPI, RB>(a, it * kRowsPerIter + grp * kOut, acc);
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i] = group_sum_last<64>(acc[i]);
      const int slot = n % kSlots;
      if ((tid & 63) == 63) {
#pragma unroll
        for (int i = 0; i < RB; ++i) ring[slot][tid >> 6][i] = acc[i];
      }
      if (slot == kSlots - 1) flush(n - (kSlots - 1), kSlots);
    }
    if constexpr (kQ8) load_rows<F, RB, EPI>(buf, a, nx * kRowsPerIter + grp * kOut, unit_ld, ln);
  }
  if constexpr (G > 64) {
    const int used = n % kSlots;
    if (used) flush(n - used, used);
  }
}

// Rows wider than G units: each row batch walks the row in segments of G
// units, reloading the lane's x values per segment.
template <class F, int G, int RB, int EPI, bool EXPERTS>
__global__ __launch_bounds__(kThreads) void gemv_seg_kernel(KernelArgs<EXPERTS> args) {
  GemvArgs a = base_args(args);
  if constexpr (EXPERTS) {
    if (!bind_assignment(a, args.e)) return;  // uniform per workgroup
  }
  constexpr int kGroups = kThreads / G;
  constexpr int kOut = out_rows<EPI, RB>();
  constexpr int kRowsPerIter = kGroups * kOut;
  __shared__ float red[kThreads / 64][RB];

  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;
  const typename F::Lane ln = make_lane<F>(gl, a);
  const int nseg = (a.units + G - 1) / G;
  const int iters = (a.rows + kRowsPerIter - 1) / kRowsPerIter;

  for (int it = blockIdx.x; it < iters; it += gridDim.x) {
    const int obase = it * kRowsPerIter + grp * kOut;
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      const int unit = seg * G + gl;
      const int unit_ld = unit < a.units ? unit : a.units - 1;
      typename F::Raw raw[RB];
      load_rows<F, RB, EPI>(raw, a, obase, unit_ld, ln);
      typename F::X xr;
      if (F::valid(unit, a.units, a.cols)) F::load_x(xr, a.x, unit, a.cols);
      else F::zero_x(xr);
      F::finish_x(xr);
#pragma unroll
      for (int i = 0; i < RB; ++i) acc[i] += F::dot(raw[i], xr, ln);
    }
    reduce_store<G, RB, EPI>(acc, a, obase, gl, grp, red);
  }
}

template <class F, int G, int RB, int EPI>
hipError_t launch_one(const GemvArgs& a, int cus, hipStream_t s, const ExpertArgs* ex) {
  constexpr int kRowsPerIter = (kThreads / G) * out_rows<EPI, RB>();
  const int64_t iters = ((int64_t)a.rows + kRowsPerIter - 1) / kRowsPerIter;
  // As many workgroups as can be resident at once (4 per CU at <= 128
  // VGPRs, else 2); each loops over row batches.
  constexpr bool kQ8 = is_q8<F>();
  constexpr int kPerCu = kQ8 ? GQ_GEMV_Q8_WG_PER_CU
                         : RB == 1 ? GQ_GEMV_WG_PER_CU_RB1
                         : is_k56<F>() ? GQ_GEMV_K56_WG_PER_CU : GQ_GEMV_WG_PER_CU_RBN;
  // (expert-batched calls share that many workgroups among their assignments)
  const int n_assign = ex ? ex->n_assign : 1;
  int64_t cap = (int64_t)cus * kPerCu / n_assign;
  if (cap < 1) cap = 1;
  const int blocks = (int)(iters < cap ? iters : cap);
  const dim3 grid(blocks, n_assign);
  // the expert-batched form is a separate instantiation, so the plain
  // matvec's prologue and arguments carry none of its indirection
  if constexpr (EPI == kEpiStore) {
    if (ex) {
      const GemvExpertArgs ea{a, *ex};
      if (a.units <= G)
        hipLaunchKernelGGL((gemv_kernel<F, G, RB, EPI, true>), grid, dim3(kThreads), 0, s, ea);
      else
        hipLaunchKernelGGL((gemv_seg_kernel<typename F::Base, G, RB, EPI, true>), grid, dim3(kThreads), 0, s, ea);
      return hipGetLastError();
    }
  }
  if (a.units <= G)
    hipLaunchKernelGGL((gemv_kernel<F, G, RB, EPI, false>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gemv_seg_kernel<typename F::Base, G, RB, EPI, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// G: the smallest power of two >= the row's units (max 256; wider rows use
// segments). RB: rows per group per iteration -- 1 when the matrix is too
// short to give every CU a few groups, else 2; always 2 (the gate row and
// the up row) for the gate|up epilogue.
template <class F, int G, int EPI>
hipError_t with_g(const GemvArgs& a, int cus, hipStream_t s, const ExpertArgs* ex) {
  if constexpr (EPI == kEpiSwiglu) {
    return launch_one<F, G, 2, EPI>(a, cus, s, ex);
  } else {
    constexpr int kWaves = is_q8<F>() ? GQ_GEMV_Q8_RB1_WAVES_PER_CU : GQ_GEMV_RB1_WAVES_PER_CU;
    const int64_t groups_needed = (int64_t)cus * kWaves * (G >= 64 ? 1 : 64 / G);
    if ((int64_t)a.rows < 2 * groups_needed) return launch_one<F, G, 1, EPI>(a, cus, s, ex);
    // Q5_K / Q6_K on tall matrices (an lm_head, 14336-row projections): one
    // row per group at more workgroups per CU measured faster (more waves to
    // hide latency behind their heavier unpacking); two rows per group stay
    // ahead for shorter matrices and for wide rows.
    if constexpr (is_k56<F>() && G <= 128) {
      if ((int64_t)a.rows >= 4 * groups_needed) return launch_one<F, G, 1, EPI>(a, cus, s, ex);
    }
    constexpr int kRB = is_q8<F>() ? GQ_GEMV_Q8_RBN : is_k56<F>() ? GQ_GEMV_K56_RBN : GQ_GEMV_RBN;
    return launch_one<F, G, kRB, EPI>(a, cus, s, ex);
  }
}

template <class F, int EPI>
hipError_t dispatch_g(const GemvArgs& a, int cus, hipStream_t s, const ExpertArgs* ex) {
  const int n = a.units;
  if (n <= 4) return with_g<F, 4, EPI>(a, cus, s, ex);
  if (n <= 8) return with_g<F, 8, EPI>(a, cus, s, ex);
  if (n <= 16) return with_g<F, 16, EPI>(a, cus, s, ex);
  if (n <= 32) return with_g<F, 32, EPI>(a, cus, s, ex);
  if (n <= 64) return with_g<F, 64, EPI>(a, cus, s, ex);
  if (n <= 128) return with_g<F, 128, EPI>(a, cus, s, ex);
  return with_g<F, 256, EPI>(a, cus, s, ex);
}

// The split-layout unit's column map depends on the group width: in each
// pass of G lanes, lane g takes chunks g, g + G, g + 2G, g + 3G, so the chunks
// of a pass are shared by all G lanes, not by the first `units` of them. The
// unit count is rounded up to whole passes, so that no lane is folded onto
// another lane's unit; the unit's own clamp keeps chunks past the row's end
// in bounds (their x is zero).
template <int G, int EPI>
hipError_t split_with_g(GemvArgs a, int cus, hipStream_t s, const ExpertArgs* ex) {
  a.units = (a.units + G - 1) / G * G;
  return with_g<Q8SplitUnit<G>, G, EPI>(a, cus, s, ex);
}

template <int EPI>
hipError_t dispatch_g_split(const GemvArgs& a, int cus, hipStream_t s, const ExpertArgs* ex) {
  const int n = a.units;
  if (n <= 4) return split_with_g<4, EPI>(a, cus, s, ex);
  if (n <= 8) return split_with_g<8, EPI>(a, cus, s, ex);
  if (n <= 16) return split_with_g<16, EPI>(a, cus, s, ex);
  if (n <= 32) return split_with_g<32, EPI>(a, cus, s, ex);
  if (n <= 64) return split_with_g<64, EPI>(a, cus, s, ex);
  if (n <= 128) return split_with_g<128, EPI>(a, cus, s, ex);
  return split_with_g<256, EPI>(a, cus, s, ex);
}

hipError_t dispatch_split(const GemvArgs& a, int cus, hipStream_t s, int epi, const ExpertArgs* ex) {
  if (ex && epi != kEpiStore) return hipErrorInvalidValue;
  switch (epi) {
    case kEpiStore: return dispatch_g_split<kEpiStore>(a, cus, s, ex);
    case kEpiAcc: return dispatch_g_split<kEpiAcc>(a, cus, s, nullptr);
    case kEpiSwiglu: return dispatch_g_split<kEpiSwiglu>(a, cus, s, nullptr);
    default: return hipErrorInvalidValue;
  }
}

template <class F>
hipError_t dispatch(const GemvArgs& a, int cus, hipStream_t s, int epi, const ExpertArgs* ex) {
  if (ex && epi != kEpiStore) return hipErrorInvalidValue;
  switch (epi) {
    case kEpiStore: return dispatch_g<F, kEpiStore>(a, cus, s, ex);
    case kEpiAcc: return dispatch_g<F, kEpiAcc>(a, cus, s, nullptr);
    case kEpiSwiglu: return dispatch_g<F, kEpiSwiglu>(a, cus, s, nullptr);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(int fmt, GemvArgs a, int cus, hipStream_t s, int epi,
                       const ExpertArgs* ex) {
  if (fmt == kFmtQ8_0) {
    const int blocks = (a.cols + 31) / 32;
    // an even block count keeps every row 4-byte aligned: pairs of blocks
    if (blocks % 2 == 0 && (uintptr_t)a.W % 4 == 0) {
      a.units = blocks / 2;
      return dispatch<Q8PairUnit>(a, cus, s, epi, ex);
    }
    a.units = blocks;
    return dispatch<Q8Unit>(a, cus, s, epi, ex);
  }
  if (fmt == kFmtQ5_0) {
    a.units = (a.cols + 31) / 32;
    return dispatch<Q5_0Unit>(a, cus, s, epi, ex);
  }
  if (fmt == kFmtQ8_0Split) {
    a.units = ((a.cols + 31) / 32 + 1) / 2;  // four 16-code chunks per lane
    return dispatch_split(a, cus, s, epi, ex);
  }
  // K-quants: four units per 256-weight super-block
  if (fmt == kFmtQ4_K && gemv_q4k_supports(a, cus, ex)) return launch_gemv_q4k(a, cus, s, epi, ex);
  a.units = 4 * ((a.cols + 255) / 256);
  if (fmt == kFmtQ5_K) return dispatch<Q5KUnit>(a, cus, s, epi, ex);
  if (fmt == kFmtQ6_K) return dispatch<Q6KUnit>(a, cus, s, epi, ex);
  return dispatch<Q4KUnit>(a, cus, s, epi, ex);
}

}  // namespace gq
