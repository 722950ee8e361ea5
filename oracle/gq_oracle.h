/*
 * gq_oracle.h -- CPU oracle for block-quantised (GGUF Q8_0 / Q4_K / Q5_0 /
 * Q5_K / Q6_K) dequant,
 * matrix-vector and small matrix-matrix products.
 *
 * TEST INFRASTRUCTURE ONLY. This library defines what the GPU path must
 * compute; it is not part of the product. Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may load it. It shares no code,
 * header, constant or table with the GPU library.
 *
 * Sources for what is computed (page titles as headed in the reference text):
 *  - "nurllama 0.18.1 API" (reg.nurl-lang.org), model.nu section: weights stay
 *    quantised and each block is decoded inside the matmul; a host dequant
 *    path is the correctness fallback.
 *  - same page, kernels.nu section, layout contract: W[out,in] row-major,
 *    y[r] = sum_c W[r*in + c] * x[c].
 *  - "nurllama" README, "What it runs": a row is a whole number of
 *    quantisation blocks; the formats Q8_0, Q4_K, Q5_0, Q5_K and Q6_K are
 *    named there.
 *  - The byte layouts of Q8_0 (34 B), Q4_K (144 B), Q5_0 (22 B), Q5_K (176 B)
 *    and Q6_K (210 B) are not printed on the pages; the public GGUF
 *    definitions are followed (see the .c file).
 *
 * Conventions: rows = output features, cols = input features. A row holds
 * ceil(cols / QK) blocks; codes at columns >= cols are ignored.
 * All functions return 0 on success, a negative value on bad arguments.
 */
#ifndef GQ_ORACLE_H
#define GQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ggml tensor type ids accepted by the oracle. */
#define GQO_TYPE_Q8_0 8
#define GQO_TYPE_Q4_K 12
#define GQO_TYPE_Q5_0 6
#define GQO_TYPE_Q5_K 13
#define GQO_TYPE_Q6_K 14
/* Q8_1 activation blocks (36 bytes per 32 values: fp16 d, fp16 d * sum q,
 * 32 int8 q): only as an activation format, never as weights. */
#define GQO_TYPE_Q8_1 9
/* Q8_0 repacked into the split per-row layout (not a ggml id): per row the
 * nb fp16 scales, zero padding to a multiple of 16 bytes, then the nb * 32
 * int8 codes in block order. */
#define GQO_TYPE_Q8_0_SPLIT 1008

/* Bytes of one row of `cols` input features, or -1 for an unknown type. */
int64_t gqo_row_bytes(int type, int64_t cols);

/* IEEE-754 binary16 -> binary32, decoded field by field. */
float gqo_f16_to_f32(uint16_t h);
void gqo_f16_to_f32_n(const uint16_t* h, int64_t n, float* out);

/* binary32 -> binary16 bits, round to nearest even (used by the test-only
 * quantisers and by tests). */
uint16_t gqo_f32_to_f16_rne(float f);

/* Q4_K: the 8 six-bit scale codes and 8 six-bit min codes of one 12-byte
 * scale field. */
void gqo_q4_k_unpack_scales(const uint8_t s[12], uint8_t sc[8], uint8_t m[8]);

/* out[r*cols + c] = w(r, c) as fp32 (the ragged tail is dropped). */
int gqo_dequant(int type, const void* W, int64_t rows, int64_t cols, float* out);

/* y[r] = sum_c w(r,c) * x[c] accumulated in f64, sequentially in c;
 * S[r] = sum_c |w(r,c) * x[c]| (f64). S may be NULL. Rows are split over
 * `nthreads` threads (each row is still summed in the same order). */
int gqo_matvec(int type, const void* W, int64_t rows, int64_t cols,
               const float* x, double* y, double* S, int nthreads);

/* Y[m*rows + r] = sum_c w(r,c) * X[m*cols + c] (f64), S likewise. */
int gqo_matmul(int type, const void* W, int64_t rows, int64_t cols,
               const float* X, int64_t M, double* Y, double* S, int nthreads);

/* Repack rows of Q8_0 blocks into the split per-row layout (row stride
 * gqo_row_bytes(GQO_TYPE_Q8_0_SPLIT, cols)); padding bytes are zero. */
int gqo_q8_0_split_repack(const void* W, int64_t rows, int64_t cols, void* out);

/* Activations (n rows of cols) -> Q8_1 blocks, row stride
 * gqo_row_bytes(GQO_TYPE_Q8_1, cols); the numerics are spelled out in the .c
 * file. And back: the values x^ = fp16 d * q that the int8 path multiplies. */
int gqo_quantize_q8_1(const float* x, int64_t n, int64_t cols, uint8_t* out);
int gqo_dequant_q8_1(const uint8_t* xq, int64_t n, int64_t cols, float* out);

/* Test-only reference quantisers (the pages print none for Q4_K). */
int gqo_quantize_q8_0(const float* w, int64_t rows, int64_t cols, uint8_t* out);
int gqo_quantize_q4_k(const float* w, int64_t rows, int64_t cols, uint8_t* out);

#ifdef __cplusplus
}
#endif

#endif
