/*
 * gq.h -- C ABI of libgq: block-quantised (GGUF Q8_0 / Q4_K / Q5_0 / Q5_K /
 * Q6_K) weight matrices times fp32 activations on an AMD MI355X (gfx950),
 * dequantised on the fly.
 *
 * The operation: a weight matrix W[out, in] stored row-major as GGUF blocks,
 * each row a whole number of blocks, multiplied by fp32 activations
 * ("nurllama 0.18.1 API", kernels.nu section, layout contract
 * y[r] = sum_c W[r*in + c] * x[c]; model.nu section: weights stay quantised
 * on the device and each block is decoded inside the matmul; the prompt is
 * processed in chunks so each weight is read once per chunk).
 *
 * Shapes and layout
 *   rows = output features, cols = input features.
 *   A row holds ceil(cols / QK) blocks: gq_row_bytes(fmt, cols) bytes.
 *   W holds rows * gq_row_bytes(fmt, cols) bytes in GGUF block order, exactly
 *   as found in the file. Codes at columns >= cols in a row's last block are
 *   ignored (GGUF itself only stores whole blocks, so this only matters for
 *   cols that are not a multiple of QK).
 *   Q8_0 (fmt 8):  34 B per 32 weights: fp16 d, then 32 int8 q; w = d*q.
 *   Q4_K (fmt 12): 144 B per 256 weights: fp16 d, fp16 dmin, 12 bytes of
 *     packed 6-bit scale/min codes (sc_j, m_j, j < 8), 128 bytes of 4-bit
 *     codes; weight 64g+32h+l takes nibble h of code byte 32g+l and belongs
 *     to sub-block j = 2g+h; w = (d*sc_j)*code - dmin*m_j.
 *   Q5_0 (fmt 6):  22 B per 32 weights: fp16 d, a 32-bit little-endian word
 *     qh, 16 bytes of nibbles; weight i < 16 takes the low nibble of byte i,
 *     weight 16 + i the high nibble of byte i, and bit 4 of every code is
 *     bit i of qh; w = d*(code - 16).
 *   Q5_K (fmt 13): 176 B per 256 weights: the 16 header bytes of Q4_K, 32
 *     bytes qh, 128 bytes of nibbles placed as Q4_K's codes; bit 4 of weight
 *     64g+32h+l's code is bit 2g+h of qh[l]; w = (d*sc_j)*code - dmin*m_j.
 *   Q6_K (fmt 14): 210 B per 256 weights: 128 bytes ql, 64 bytes qh, 16 int8
 *     scales, fp16 d; weight 128n+32k+l takes nibble k>>1 of
 *     ql[64n + 32(k&1) + l] as its low four bits and bits 2k, 2k+1 of
 *     qh[32n + l] as its top two, scale number i/16 for weight i;
 *     w = (d*scale)*(code - 32).
 *   Q8_0 split (fmt 1008): the same Q8_0 data repacked per row with the
 *     scales apart from the codes ("nurllama 0.18.1 API", kernels.nu section:
 *     an uploaded q8_0 tensor is repacked into a split per-row layout; the
 *     layout is not printed there, this is the one taken): the ceil(cols/32)
 *     fp16 scales, zero padding to a multiple of 16 bytes, then the codes of
 *     the blocks in order. Made by gq_q8_0_split_repack; the matvec reads its
 *     codes as one contiguous, 16-byte aligned stream.
 *   Q5_0, Q5_K and Q6_K appear next to Q4_K in the model files the pages run
 *   ("nurllama" README, "What it runs"; their per-format matvec kernels are
 *   listed in "nurllama 0.18.1 API", kernels.nu section). The byte layouts
 *   are GGUF's public ones; the pages do not print them.
 *
 * Ownership and threading
 *   All pointers are device pointers owned by the caller; the library never
 *   frees or keeps them. No entry point uses device memory beyond its
 *   arguments: there is no workspace (work split along k stays inside one
 *   workgroup and is added in a fixed order). Global state: a per-device
 *   cache of device properties, filled once. Calls on different streams may
 *   run concurrently.
 *
 * Sizes
 *   rows, cols, M, batch rows, expert assignments and the activation rows of
 *   a grouped product are each at most 2^30 (GQ_ERR_SHAPE beyond; for the
 *   gate|up forms 2 * rows counts): the kernels index them with 32-bit
 *   integers, and this bound keeps every index they form below 2^31.
 *   Byte counts are computed in 64 bits and checked for overflow.
 *
 * Alignment
 *   Q8_0, Q5_0 and Q6_K W: 2-byte aligned (a row range of such a tensor
 *   starts on any block boundary, and their blocks are 34, 22 and 210 bytes).
 *   Q4_K, Q5_K and split Q8_0 W: 4-byte aligned. x, y, X, Y, out: 4-byte
 *   aligned. An output that overlaps an input is rejected (GQ_ERR_OVERLAP).
 *
 * Errors
 *   Every entry point returns a gq_status. Arguments are validated on the
 *   host before any HIP call, so a bad argument never reaches the GPU.
 *   rows == 0 (or M == 0) is an empty product: GQ_OK, nothing is written.
 *   An unsupported fmt returns GQ_ERR_FMT so that a caller can fall back to
 *   another path ("nurllama 0.18.1 API", kernels.nu section: the quantised
 *   matvec dispatch reports a type it has no kernel for).
 *   An asynchronous kernel fault surfaces at the caller's next synchronise.
 *   No C++ exception crosses this interface.
 */
#ifndef GQ_H
#define GQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ggml tensor type ids ("nurllama 0.18.1 API", convert.nu section, gives
 * Q8_0 = 8; the others are GGUF's ids). */
enum gq_fmt {
    GQ_FMT_Q5_0 = 6,
    GQ_FMT_Q8_0 = 8,
    GQ_FMT_Q4_K = 12,
    GQ_FMT_Q5_K = 13,
    GQ_FMT_Q6_K = 14,
    GQ_FMT_Q8_0_SPLIT = 1008, /* Q8_0 in the split per-row layout (not a ggml id) */
    GQ_FMT_Q8_1 = 9,          /* activation blocks of the int8 path only (see
                                 gq_quantize_q8_1); never a weight format */
};

enum gq_status {
    GQ_OK = 0,
    GQ_ERR_NULL = 1,   /* a required pointer is NULL */
    GQ_ERR_FMT = 2,    /* fmt is not one of enum gq_fmt */
    GQ_ERR_SHAPE = 3,  /* rows or M < 0, cols <= 0, or a size that overflows */
    GQ_ERR_ALIGN = 4,  /* a pointer breaks the alignment rules above */
    GQ_ERR_DEVICE = 5, /* the HIP runtime reported an error */
    GQ_ERR_OVERLAP = 6, /* the output range overlaps an input range */
};

/* Bytes of one row of `cols` input features: ceil(cols/QK) * block bytes.
 * Returns a negative value for an unknown fmt or cols < 0. Host only. */
int64_t gq_row_bytes(int fmt, int64_t cols);

/* A static, human-readable name for a status code. */
const char* gq_status_str(int status);

/*
 * out[r*cols + c] = w(r, c) as fp32, for r < rows, c < cols.
 * Bit-exact: w as defined per format above, where every product is exact
 * in fp32 and the Q4_K / Q5_K subtraction rounds once to nearest even;
 * fp16 subnormal scales are decoded exactly. This is the device
 * counterpart of the host dequant fallback ("nurllama 0.18.1 API", model.nu
 * section). Runs on the null stream and returns after it has finished.
 * out: rows*cols floats.
 */
int gq_dequant(int fmt, const void* W, int64_t rows, int64_t cols, float* out);

/*
 * y[r] = sum_{c < cols} w(r, c) * x[c] for r < rows; y is overwritten.
 * The decode-step matrix-vector product ("nurllama" README, "What it runs":
 * the matvec kernels decode GGUF blocks inside the matmul). x: cols floats,
 * y: rows floats. Accumulation is fp32 with exact per-block products; the
 * result is within 2e-4 * sum_c |w*x| of the exact sum, and repeated calls
 * give bit-identical results. Enqueued asynchronously on `stream` (a
 * hipStream_t; NULL = the null stream).
 */
int gq_matvec(int fmt, const void* W, int64_t rows, int64_t cols,
              const float* x, float* y, void* stream);

/*
 * y[r] += sum_{c < cols} w(r, c) * x[c] for r < rows: the matvec with its
 * result added to y (one fp32 addition per output) instead of overwriting
 * it, for a projection that feeds a residual stream (the llama shape has
 * residuals around attention and the feed-forward: "nurllama 0.18.1 API",
 * model.nu section; its kernels.nu section lists the separate vector add
 * this removes, and the Loom inventory has an "acc" mode for its GEMMs). Same arguments, accuracy and stream behaviour as gq_matvec; y
 * must hold the addend.
 */
int gq_matvec_acc(int fmt, const void* W, int64_t rows, int64_t cols,
                  const float* x, float* y, void* stream);

/*
 * The gate|up projection of a SwiGLU feed-forward with its activation fused
 * in: W holds 2*rows weight rows, the gate rows 0..rows-1 followed by the up
 * rows rows..2*rows-1 (one tensor whose parts are row ranges, as the
 * "nurllama" README, "What it runs", describes for phi3's fused ffn_up), and
 *   y[r] = silu(g_r) * u_r,  g_r = sum_c w(r, c) x[c],  u_r = sum_c w(rows+r, c) x[c],
 * silu(g) = g / (1 + exp(-g)) ("nurllama 0.18.1 API", kernels.nu section:
 * the in-place g <- silu(g) * u kernel that follows the two matvecs). One
 * launch: each row group computes its gate and up sums together and applies
 * the activation before the single store. g_r and u_r are bit-identical to
 * what gq_matvec returns for those rows; the activation is evaluated in
 * fp32. W holds 2*rows*gq_row_bytes(fmt, cols) bytes; y: rows floats.
 */
int gq_matvec_swiglu(int fmt, const void* W, int64_t rows, int64_t cols,
                     const float* x, float* y, void* stream);

/*
 * Expert-batched matvec for mixture-of-experts layers: one call over all
 * n_assign (position, expert) assignments ("nurllama 0.18.1 API", kernels.nu
 * section: the batched expert matvec, where output row a uses expert
 * expid[a] and input row a / xk of x):
 *   Y[a*rows + r] = sum_{c < cols} w_e(r, c) * X[(a / xk)*cols + c],  e = expid[a],
 * for a < n_assign, r < rows. W holds the n_expert matrices back to back
 * (a fused 3-D expert tensor: expert e's rows start at byte
 * e * rows * gq_row_bytes(fmt, cols)); X is [ceil(n_assign / xk), cols]
 * (xk = experts per position); expid is a device array of n_assign int32
 * expert ids; Y is [n_assign, rows]. Each assignment is the gq_matvec of its
 * expert and activation row, bit for bit. An id outside [0, n_expert) reads
 * no weights and fills that assignment's output row with NaN (the ids live
 * on the device, so they cannot be checked before the launch). n_assign is
 * at most 2^30 (GQ_ERR_SHAPE beyond). Asynchronous on `stream`.
 */
int gq_matvec_experts(int fmt, const void* W, int64_t n_expert, int64_t rows, int64_t cols,
                      const float* X, int64_t xk, const int32_t* expid, int64_t n_assign,
                      float* Y, void* stream);

/*
 * Batched matvec: `batch` activation rows against one weight matrix, each
 * rounded exactly as a lone gq_matvec call rounds it:
 *   Y[b*rows + r] = sum_{c < cols} w(r, c) * X[b*cols + c],  b < batch, r < rows,
 * and Y's row b equals gq_matvec(fmt, W, rows, cols, X + b*cols, ...) bit for
 * bit, whatever the batch size. The pages' matvec takes a batch count
 * ("nurllama 0.18.1 API", kernels.nu section); a chunked prompt must
 * continue exactly as the unbatched reference does ("nurllama" README, "How
 * it is checked"), and a kernel variant is a dispatch choice, never a change
 * of results (same README, "What it runs"). One launch: every batch row is a slice of the matvec grid, and
 * the slices walk the same rows together, so W is streamed from HBM about
 * once. X: [batch, cols] row-major fp32 (4-byte aligned); Y: [batch, rows],
 * overwritten, must not overlap W or X. batch is at most 2^30 (GQ_ERR_SHAPE
 * beyond); batch == 0 or rows == 0 is a no-op. No workspace. Asynchronous
 * on `stream`.
 */
int gq_matvec_batch(int fmt, const void* W, int64_t rows, int64_t cols, const float* X,
                    int64_t batch, float* Y, void* stream);

/*
 * Repack `rows` rows of Q8_0 blocks (W, rows * gq_row_bytes(GQ_FMT_Q8_0,
 * cols) bytes, 2-byte aligned) into the split per-row layout at `out`
 * (rows * gq_row_bytes(GQ_FMT_Q8_0_SPLIT, cols) bytes, 4-byte aligned, must
 * not overlap W); padding bytes are written as zero. A one-time step after
 * upload ("nurllama 0.18.1 API", kernels.nu section, the q8_0 repack);
 * every entry point then accepts GQ_FMT_Q8_0_SPLIT. Asynchronous on `stream`.
 */
int gq_q8_0_split_repack(const void* W, int64_t rows, int64_t cols, void* out, void* stream);

/*
 * Y[m*rows + r] = sum_{c < cols} w(r, c) * X[m*cols + c], for m < M, r < rows;
 * Y is overwritten. X: [M, cols] row-major fp32; Y: [M, rows] row-major fp32.
 * The batched form used for prompt chunks ("nurllama 0.18.1 API", model.nu
 * section: the matmuls run over up to 64 positions at once, each weight read
 * once per chunk). M == 1 runs the gq_matvec kernel. With M < 16 and
 * M * rows * cols <= 2^28 the call is gq_matvec_batch, so every row of Y
 * equals gq_matvec of its activation row bit for bit. Otherwise, in one
 * launch:
 *   - On the fp16 matrix cores, with exact operands: Q4_K, Q5_K and split
 *     Q8_0 with cols % 4 == 0; Q6_K, and from M = 8 Q8_0 and Q5_0, with
 *     cols % 4 == 0, a row length gq_row_bytes(fmt, cols) that is a multiple
 *     of 4 (an even number of super-blocks or blocks) and W 4-byte aligned.
 *     The weight operand is sc * code (at most 63 * 31), the int8 code, the
 *     Q5_0 code - 16, or for Q6_K the pair 16 sh (q - 32), sl (q - 32) with
 *     sc = 16 sh + sl, all exact in fp16, with d (and dmin) applied in fp32
 *     per super-block or block;
 *     each activation row's 256 values of a 256-column step are scaled by a
 *     power of two and split into fp16 hi and lo parts. They need 64 * 4 * cols < 2^31 and
 *     256 * gq_row_bytes(fmt, cols) < 2^31 (Q4_K: cols < 2^23), else
 *     GQ_ERR_SHAPE before any launch. Accuracy: the gq_matvec bound, except
 *     that activations below about 2^-14 of the largest magnitude max_b in
 *     their row's step b (256 columns) are carried only to an absolute
 *     2^-34 max_b: an extra error of at most 2^-33 * max_b * sum_{c in b}
 *     |w(r, c)|-terms per step (Q4_K / Q5_K: |d sc_j q_c| + |dmin m_j|;
 *     Q8_0: |d q_c|; Q5_0: |d (q_c - 16)|; Q6_K: |d sc_s (q_c - 32)|), none
 *     when every activation is 0 or within that range.
 *   - The other products with M >= 2 of Q4_K, Q5_K, Q6_K and split Q8_0,
 *     and with M >= 8 of Q8_0 and Q5_0 (rows those kernels do not take), run
 *     on the fp32 matrix cores: each
 *     k-chunk of W is dequantised exactly to fp32 and multiplied with the
 *     fp32 activations; same accuracy bound as gq_matvec.
 *   - Q8_0 and Q5_0 with 2 <= M < 8 stream W once per 15 activation rows on
 *     the fp32 vector units; same accuracy bound as gq_matvec. (The
 *     accumulate and SwiGLU forms run these on the matrix cores above.)
 * Repeated calls give bit-identical results. Asynchronous on `stream`.
 */
int gq_matmul(int fmt, const void* W, int64_t rows, int64_t cols,
              const float* X, int64_t M, float* Y, void* stream);

/*
 * The prefill product's other output modes (the Loom porting skill, "What
 * the starter generates": its GEMM generator has store, acc and swiglu
 * modes, as the matvec does here), same arguments, routes, limits and
 * accuracy as gq_matmul:
 *   gq_matmul_acc:    Y[m*rows + r] += sum_c w(r, c) * X[m*cols + c]
 *                     (Y holds the addend; one fp32 addition per output).
 *   gq_matmul_swiglu: W is a gate|up tensor of 2 * rows weight rows (gate
 *                     rows first), Y[m*rows + r] = silu(g) * u with g, u the
 *                     products of gate row r and up row rows + r, evaluated
 *                     in fp32 as g / (1 + e^-g) * u, as gq_matvec_swiglu does.
 * M == 1 runs gq_matvec_acc / gq_matvec_swiglu, and the few-row range (M <
 * 16, M * rows * cols <= 2^28) runs them once per activation row, so those
 * rows equal the matvec forms bit for bit. On the matrix cores the SwiGLU
 * form is two launches on `stream` (Y = up products, then Y = silu(gate
 * products) * Y), with no memory beyond the arguments. Asynchronous.
 */
int gq_matmul_acc(int fmt, const void* W, int64_t rows, int64_t cols,
                  const float* X, int64_t M, float* Y, void* stream);
int gq_matmul_swiglu(int fmt, const void* W, int64_t rows, int64_t cols,
                     const float* X, int64_t M, float* Y, void* stream);

/*
 * Grouped product for the prefill of a mixture-of-experts layer: activation
 * rows already bucketed by expert (the Loom porting skill, "Beyond the
 * starter": tokens bucketed by expert, then one grouped GEMM per expert for
 * prefill; per-assignment matvecs serve decode, gq_matvec_experts). W holds
 * the n_expert matrices back to back as in gq_matvec_experts (expert e's
 * rows start at byte e * rows * gq_row_bytes(fmt, cols)). m_per_expert is a
 * HOST array of n_expert row counts; X is [sum m_e, cols] with expert 0's
 * m_0 rows first, then expert 1's, ...; Y is [sum m_e, rows] in the same
 * order, overwritten:
 *   Y[(o_e + i)*rows + r] = sum_c w_e(r, c) * X[(o_e + i)*cols + c],
 *   o_e = m_0 + ... + m_{e-1}, i < m_e.
 * The layouts that gq_matmul runs on the fp16 matrix cores (whatever the
 * row counts here): one launch per 64 experts on the fp16 matrix cores
 * (every group, whatever its row count, with the accuracy bound and shape
 * limits of that case); each block is deterministic but may differ in the
 * last bits from gq_matmul of the same rows, whose tile is chosen for that
 * call alone. Other layouts: each expert's block is exactly gq_matmul of
 * that expert's matrix and rows (same kernels, same bits), enqueued in
 * expert order.
 * Experts with no rows are skipped. All counts are checked (>= 0, at most
 * 2^30 rows in all, as gq_matmul's M) before the first launch; n_expert == 0, rows == 0 or no
 * rows at all is a no-op. Asynchronous on `stream` (the counts are read
 * during the call and not kept). If a launch fails (GQ_ERR_DEVICE) the
 * launches before it have been enqueued and Y's later blocks are
 * unspecified.
 */
int gq_matmul_experts(int fmt, const void* W, int64_t n_expert, int64_t rows, int64_t cols,
                      const float* X, const int64_t* m_per_expert, float* Y, void* stream);

/*
 * The steps around gq_matmul_experts for a mixture-of-experts prefill, all
 * on the device: bucketing of the assignments by expert (the Loom porting
 * skill, "What the starter generates": the MoE generator buckets the rows
 * before the grouped GEMMs), the gather of the activation rows into bucket
 * order, and the weighted scatter back to the positions ("nurllama 0.18.1
 * API", kernels.nu section: the assignment table holds an expert id and a
 * weight per (position, selected expert) pair, and the scatter adds, for each
 * position, the sum over its k experts of weight times the expert's output
 * row onto the output). An assignment a = t * k + j is slot j of position t.
 *
 * gq_moe_bucket: expid is a device array of n_assign int32 expert ids. A
 * stable counting sort by expert: counts[e] (device, n_expert int64) = the
 * assignments with id e; the bucket of expert e starts at o_e = counts[0] +
 * ... + counts[e-1]; assignment a with id e goes to position pos[a] = o_e +
 * (the assignments a' < a with id e), and order[pos[a]] = a. An id outside
 * [0, n_expert) is dropped: pos[a] = -1, counted nowhere (order then has
 * fewer than n_assign entries written; the rest are left as they were). The
 * same placement on every call (no atomics). One workgroup (1024 threads,
 * an LDS count per expert and wave): n_expert at most 1024, n_assign at most
 * 2^30 (GQ_ERR_SHAPE beyond); sized for the assignments of a prompt chunk,
 * its time grows with n_assign / 1024. n_assign == 0 writes zero counts.
 * counts 8-byte aligned, the int32 arrays 4-byte aligned, no two of the four
 * arrays overlapping. The counts stay on the device: copying them to the
 * host gives gq_matmul_experts its m_per_expert.
 *
 * gq_moe_gather: Xb[pos[a]*cols + c] = X[(a / k)*cols + c] for every a <
 * n_assign with 0 <= pos[a] < n_assign (other rows of Xb are left as they
 * were). X: [ceil(n_assign / k), cols] fp32; Xb: [n_assign, cols] fp32, must
 * not overlap X or pos. A plain copy, bit for bit.
 *
 * gq_moe_scatter: for t < n_assign / k (n_assign a multiple of k), r < rows:
 *   s = 0; for j = 0 .. k-1, a = t*k + j, if 0 <= pos[a] < n_assign:
 *     s = s + w[a] * Yb[pos[a]*rows + r];
 *   out[t*rows + r] = out[t*rows + r] + s,
 * in fp32 with every product and sum rounded on its own (no fused
 * multiply-add), in slot order j. Yb: [n_assign, rows] (gq_matmul_experts
 * on the gathered rows); w: n_assign fp32 weights; out: [n_assign / k, rows],
 * must not overlap Yb, pos or w.
 *
 * All three: asynchronous on `stream`; arguments checked on the host
 * (GQ_ERR_SHAPE / NULL / ALIGN / OVERLAP) before any launch.
 */
int gq_moe_bucket(const int32_t* expid, int64_t n_assign, int64_t n_expert, int64_t* counts,
                  int32_t* order, int32_t* pos, void* stream);
int gq_moe_gather(const float* X, int64_t cols, int64_t k, const int32_t* pos, int64_t n_assign,
                  float* Xb, void* stream);
int gq_moe_scatter(const float* Yb, int64_t rows, const int32_t* pos, const float* w,
                   int64_t n_assign, int64_t k, float* out, void* stream);

/*
 * gq_matmul_experts with the row counts on the device, so that a whole MoE
 * prefill (gq_moe_bucket, gq_moe_gather, this product, gq_moe_scatter) runs
 * without a host synchronisation and can be captured in a HIP graph. m_dev:
 * n_expert int64 counts in device memory (8-byte aligned), such as
 * gq_moe_bucket's; X: [total, cols] and Y: [total, rows] fp32 with expert
 * 0's rows first, then expert 1's, ... as in gq_matmul_experts. The counts
 * are read by the kernels: a negative count counts as 0, and the groups are
 * cut at `total` rows (a count past what is left is clamped), so no group
 * reads or writes past X or Y; rows of Y past the sum of the counts are left
 * as they were. The layouts of the fp16 matrix cores only: cols a multiple
 * of 4, and for Q8_0, Q5_0 and Q6_K rows of whole dwords and a 4-byte
 * aligned W (GQ_ERR_SHAPE / GQ_ERR_ALIGN otherwise). One launch; its grid is
 * sized for the most m-tiles `total` rows can need, the tile is chosen as
 * for one group of `total` rows, and each workgroup finds its group by
 * walking the counts (linear in n_expert, at most 1024). The results obey
 * gq_matmul's accuracy bound per expert; a group's bits may differ from
 * gq_matmul_experts of the same rows, whose tile follows the counts.
 * Asynchronous on `stream`.
 */
int gq_matmul_experts_dev(int fmt, const void* W, int64_t n_expert, int64_t rows, int64_t cols,
                          const float* X, const int64_t* m_dev, int64_t total, float* Y, void* stream);

/*
 * The int8-activation decode path (the Loom porting skill, "What the starter
 * generates": decode-shaped linears with activations in llama.cpp's Q8_1
 * numerics and 4-way integer dot products, an fp32-activation switch kept
 * beside them). The page names the numerics without printing them; the
 * reading taken is the public Q8_1 block.
 *
 * gq_quantize_q8_1: n rows of cols fp32 activations (x, [n, cols] row-major,
 * 4-byte aligned) -> n rows of gq_row_bytes(GQ_FMT_Q8_1, cols) =
 * 36 * ceil(cols / 32) bytes at xq (4-byte aligned, must not overlap x). Per
 * 32 values (columns >= cols count as 0): d = amax / 127 (fp32, to nearest),
 * id = d != 0 ? 1 / d : 0, q_i = round-half-away-from-zero(x_i * id) (fp32
 * product, |q_i| <= 127); bytes 0-1 fp16(d), 2-3 fp16(d * sum q_i), 4..35 the
 * int8 q_i. A block whose 1 / d overflows (largest |x| under about 3.7e-37)
 * has products +-inf, or NaN where x_i = 0: its codes are clamped to +-127
 * and NaN gives 0 (its fp16 scale is 0, so its values are 0 either way).
 * Byte-identical to the CPU oracle's quantiser. n == 0 is a no-op.
 * Asynchronous on `stream`.
 */
int gq_quantize_q8_1(const float* x, int64_t n, int64_t cols, void* xq, void* stream);

/*
 * y[r] = sum_c w(r, c) * x^_c for r < rows, with x^_c = fp16(d) * q_c the
 * values of one quantised activation row xq (gq_quantize_q8_1 of a cols-wide
 * row, 4-byte aligned); y is overwritten. fmt: GQ_FMT_Q8_0 or GQ_FMT_Q4_K
 * (others: GQ_ERR_FMT), W as for gq_matvec. Integer dot products per 32
 * weights (exact int32), scales applied in fp32: the result is within
 * 2e-4 * sum_c |w(r,c) * x^_c| of the exact W x^ (the gq_matvec rule with x^
 * in place of x); against the fp32 activations themselves it differs by the
 * quantisation of x, |x_c - x^_c| <= d/2 + 127 |d - fp16(d)| per value
 * (d of the value's 32-block). cols may be at most 131072 (the quantised row
 * is staged in LDS): GQ_ERR_SHAPE beyond. Asynchronous on `stream`.
 */
int gq_matvec_q8_1(int fmt, const void* W, int64_t rows, int64_t cols, const void* xq, float* y,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
