/*
 * gq_oracle.c -- plain, slow CPU oracle for block-quantised GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY (see gq_oracle.h). Built with gcc -O2
 * -ffp-contract=off and no fast-math, so every float expression below is
 * evaluated as written, one IEEE operation at a time.
 *
 * What it follows:
 *  - Dequantise inside the product, weights kept in their block format:
 *    "nurllama 0.18.1 API", model.nu section ("Weights stay QUANTISED on the
 *    device ... decodes each block inside the matmul"; host dequant is the
 *    correctness fallback).
 *  - y[r] = sum_c W[r*in + c] * x[c] with W[out,in] row-major: same page,
 *    kernels.nu section, "Layout contracts".
 *  - A row is a whole number of blocks: "nurllama" README, "What it runs".
 *  - Block layouts: not printed on the pages. The public GGUF definitions are
 *    used and restated here in the form this file implements:
 *      Q8_0, 34 bytes per 32 weights: bytes 0-1 = d (fp16, little endian),
 *        bytes 2..33 = q_0..q_31 (int8). w_i = d * q_i.
 *      Q4_K, 144 bytes per 256 weights: bytes 0-1 = d (fp16), 2-3 = dmin
 *        (fp16), 4..15 = twelve bytes holding eight 6-bit scale codes sc_j and
 *        eight 6-bit min codes m_j, 16..143 = 128 bytes of 4-bit codes.
 *        Weight i = 64g + 32h + l (g<4, h<2, l<32) is in sub-block j = 2g+h;
 *        its code is the low nibble of qs[32g+l] when h = 0, the high nibble
 *        when h = 1. w_i = (d*sc_j)*code - dmin*m_j.
 *      Q5_0, 22 bytes per 32 weights: bytes 0-1 = d (fp16), 2-5 = a 32-bit
 *        little-endian word qh holding bit 4 of every code (bit i for weight
 *        i), 6..21 = sixteen bytes of low nibbles: weight i < 16 takes the
 *        low nibble of byte i, weight 16 + i the high nibble of byte i.
 *        code_i in 0..31, w_i = d * (code_i - 16).
 *      Q5_K, 176 bytes per 256 weights: d, dmin and the twelve 6-bit scale
 *        bytes exactly as in Q4_K (bytes 0..15), then 32 bytes qh (16..47),
 *        then 128 bytes of low nibbles (48..175) placed as in Q4_K. Weight
 *        i = 64g + 32h + l takes bit 2g + h of qh[l] as bit 4 of its code.
 *        w_i = (d*sc_j)*code - dmin*m_j with code in 0..31.
 *      Q6_K, 210 bytes per 256 weights: bytes 0..127 = low nibbles ql,
 *        128..191 = high bit pairs qh, 192..207 = sixteen int8 scales (one per
 *        16 consecutive weights), 208-209 = d (fp16). Weight
 *        i = 128n + 32k + l (n<2, k<4, l<32): low four bits = nibble k>>1 of
 *        ql[64n + 32(k&1) + l], high two bits = bits 2k..2k+1 of qh[32n + l];
 *        code in 0..63, w_i = (d*scale_{i/16})*(code - 32).
 *      Q8_0 split per-row layout (a repack of Q8_0 rows that stores the
 *        scales apart from the quants: "nurllama 0.18.1 API", kernels.nu
 *        section, the q8_0 repack kernel; the layout itself is not printed,
 *        this is the reading taken): per row the nb fp16 scales, zero padding
 *        to a multiple of 16 bytes, then the nb * 32 codes in block order.
 *    Formats other than these are not decoded (the pages list Q5_K, Q6_K and
 *    Q5_0 next to Q4_K: "nurllama" README, "What it runs"; "nurllama 0.18.1
 *    API", kernels.nu section, its per-format kernel list).
 *  - Columns >= cols in a row's last block are ignored (a reading: GGUF
 *    itself only stores whole blocks per row).
 */
#include "gq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's own format constants. */
enum {
    O_Q8_0_WEIGHTS = 32,
    O_Q8_0_BYTES = 34,
    O_Q4_K_WEIGHTS = 256,
    O_Q4_K_BYTES = 144,
    O_Q5_0_WEIGHTS = 32,
    O_Q5_0_BYTES = 22,
    O_Q5_K_WEIGHTS = 256,
    O_Q5_K_BYTES = 176,
    O_Q6_K_WEIGHTS = 256,
    O_Q6_K_BYTES = 210,
    O_Q8_1_VALUES = 32,
    O_Q8_1_BYTES = 36,
};

/* Weights and bytes of one block of `type`; 0 for an unknown type. */
/* Bytes of the scale region of a split Q8_0 row (nb fp16, padded to 16). */
static int64_t split_scale_bytes(int64_t nb)
{
    return ((2 * nb + 15) / 16) * 16;
}

static int block_shape(int type, int* bytes)
{
    switch (type) {
    case GQO_TYPE_Q8_0: *bytes = O_Q8_0_BYTES; return O_Q8_0_WEIGHTS;
    case GQO_TYPE_Q4_K: *bytes = O_Q4_K_BYTES; return O_Q4_K_WEIGHTS;
    case GQO_TYPE_Q5_0: *bytes = O_Q5_0_BYTES; return O_Q5_0_WEIGHTS;
    case GQO_TYPE_Q5_K: *bytes = O_Q5_K_BYTES; return O_Q5_K_WEIGHTS;
    case GQO_TYPE_Q6_K: *bytes = O_Q6_K_BYTES; return O_Q6_K_WEIGHTS;
    case GQO_TYPE_Q8_1: *bytes = O_Q8_1_BYTES; return O_Q8_1_VALUES;
    default: *bytes = 0; return 0;
    }
}

int64_t gqo_row_bytes(int type, int64_t cols)
{
    if (cols < 0)
        return -1;
    if (type == GQO_TYPE_Q8_0_SPLIT) {
        int64_t nb = (cols + O_Q8_0_WEIGHTS - 1) / O_Q8_0_WEIGHTS;
        return split_scale_bytes(nb) + nb * O_Q8_0_WEIGHTS;
    }
    int bytes;
    int weights = block_shape(type, &bytes);
    if (weights == 0)
        return -1;
    return ((cols + weights - 1) / weights) * bytes;
}

/* ---------------------------------------------------------------- fp16 */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float gqo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1F;
    int fraction = h & 0x3FF;
    float magnitude;
    if (exponent == 0) {
        /* zero or subnormal: fraction * 2^-24 (exact in binary32) */
        magnitude = ldexpf((float)fraction, -24);
    } else if (exponent == 31) {
        magnitude = (fraction == 0) ? INFINITY : NAN;
    } else {
        /* normal: (1024 + fraction) * 2^(exponent - 15 - 10) */
        magnitude = ldexpf((float)(1024 + fraction), exponent - 25);
    }
    return sign ? -magnitude : magnitude;
}

void gqo_f16_to_f32_n(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = gqo_f16_to_f32(h[i]);
}

/* Round a non-negative double to binary16, to nearest, ties to even. */
static uint16_t f64_to_f16_rne_mag(double a)
{
    if (a != a)
        return 0x7E00;
    if (a >= 65520.0) /* half-way between 65504 and 2^16 rounds to even = inf */
        return 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24; 1024 quanta encode 2^-14 */
        double q = nearbyint(a * 16777216.0);
        return (uint16_t)q;
    }
    int e;
    (void)frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    double q = nearbyint(ldexp(a, 11 - e)); /* 11 significant bits: [1024, 2048] */
    int biased = e - 1 + 15;
    if (q == 2048.0) {
        q = 1024.0;
        biased += 1;
    }
    if (biased >= 31)
        return 0x7C00;
    return (uint16_t)((biased << 10) | ((int)q - 1024));
}

uint16_t gqo_f32_to_f16_rne(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    return sign | f64_to_f16_rne_mag(fabs((double)f));
}

/* Smallest binary16 >= a (a >= 0, finite result expected). */
static uint16_t f64_to_f16_up(double a)
{
    uint16_t h = f64_to_f16_rne_mag(a);
    if ((double)gqo_f16_to_f32(h) < a && h < 0x7C00)
        h += 1;
    return h;
}

/* ------------------------------------------------------- block decoding */

void gqo_q4_k_unpack_scales(const uint8_t s[12], uint8_t sc[8], uint8_t m[8])
{
    for (int j = 0; j < 4; j++) {
        sc[j] = s[j] & 63;
        m[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; j++) {
        sc[j] = (uint8_t)((s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4));
        m[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
    }
}

static uint16_t read_u16le(const uint8_t* p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

static void dequant_row_q8_0(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q8_0_WEIGHTS - 1) / O_Q8_0_WEIGHTS;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = row + b * O_Q8_0_BYTES;
        float d = gqo_f16_to_f32(read_u16le(blk));
        for (int i = 0; i < O_Q8_0_WEIGHTS; i++) {
            int64_t c = b * O_Q8_0_WEIGHTS + i;
            if (c >= cols)
                break;
            int8_t q = (int8_t)blk[2 + i];
            out[c] = d * (float)q;
        }
    }
}

static void dequant_row_q4_k(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q4_K_WEIGHTS - 1) / O_Q4_K_WEIGHTS;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = row + b * O_Q4_K_BYTES;
        float d = gqo_f16_to_f32(read_u16le(blk));
        float dmin = gqo_f16_to_f32(read_u16le(blk + 2));
        uint8_t sc[8], m[8];
        gqo_q4_k_unpack_scales(blk + 4, sc, m);
        const uint8_t* qs = blk + 16;
        for (int i = 0; i < O_Q4_K_WEIGHTS; i++) {
            int64_t c = b * O_Q4_K_WEIGHTS + i;
            if (c >= cols)
                break;
            int g = i / 64;
            int h = (i / 32) % 2;
            int l = i % 32;
            int j = 2 * g + h;
            uint8_t byte = qs[32 * g + l];
            int code = h ? (byte >> 4) : (byte & 0x0F);
            float scale = d * (float)sc[j];  /* exact: 11-bit x 6-bit */
            float minv = dmin * (float)m[j]; /* exact */
            out[c] = scale * (float)code - minv; /* product exact; one rounding */
        }
    }
}

static void dequant_row_q5_0(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q5_0_WEIGHTS - 1) / O_Q5_0_WEIGHTS;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = row + b * O_Q5_0_BYTES;
        float d = gqo_f16_to_f32(read_u16le(blk));
        uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) |
                      ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
        const uint8_t* qs = blk + 6;
        for (int i = 0; i < O_Q5_0_WEIGHTS; i++) {
            int64_t c = b * O_Q5_0_WEIGHTS + i;
            if (c >= cols)
                break;
            int lo = i < 16 ? (qs[i] & 0x0F) : (qs[i - 16] >> 4);
            int code = lo | (int)(((qh >> i) & 1u) << 4);
            out[c] = d * (float)(code - 16); /* exact: 11-bit x 5-bit */
        }
    }
}

static void dequant_row_q5_k(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q5_K_WEIGHTS - 1) / O_Q5_K_WEIGHTS;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = row + b * O_Q5_K_BYTES;
        float d = gqo_f16_to_f32(read_u16le(blk));
        float dmin = gqo_f16_to_f32(read_u16le(blk + 2));
        uint8_t sc[8], m[8];
        gqo_q4_k_unpack_scales(blk + 4, sc, m);
        const uint8_t* qh = blk + 16;
        const uint8_t* qs = blk + 48;
        for (int i = 0; i < O_Q5_K_WEIGHTS; i++) {
            int64_t c = b * O_Q5_K_WEIGHTS + i;
            if (c >= cols)
                break;
            int g = i / 64;
            int h = (i / 32) % 2;
            int l = i % 32;
            int j = 2 * g + h;
            uint8_t byte = qs[32 * g + l];
            int lo = h ? (byte >> 4) : (byte & 0x0F);
            int code = lo | (((qh[l] >> j) & 1) << 4);
            float scale = d * (float)sc[j];  /* exact: 11-bit x 6-bit */
            float minv = dmin * (float)m[j]; /* exact */
            out[c] = scale * (float)code - minv; /* product exact (22 bits) */
        }
    }
}

static void dequant_row_q6_k(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q6_K_WEIGHTS - 1) / O_Q6_K_WEIGHTS;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = row + b * O_Q6_K_BYTES;
        const uint8_t* ql = blk;
        const uint8_t* qh = blk + 128;
        const int8_t* scales = (const int8_t*)(blk + 192);
        float d = gqo_f16_to_f32(read_u16le(blk + 208));
        for (int i = 0; i < O_Q6_K_WEIGHTS; i++) {
            int64_t c = b * O_Q6_K_WEIGHTS + i;
            if (c >= cols)
                break;
            int n = i / 128;
            int k = (i / 32) % 4;
            int l = i % 32;
            uint8_t lbyte = ql[64 * n + 32 * (k & 1) + l];
            int lo = (k >> 1) ? (lbyte >> 4) : (lbyte & 0x0F);
            int hi = (qh[32 * n + l] >> (2 * k)) & 3;
            int code = lo | (hi << 4);
            float scale = d * (float)scales[i / 16]; /* exact: 11-bit x 8-bit */
            /* exact: |d| significand x |scale*(code-32)| <= 2^11 x 2^12 */
            out[c] = scale * (float)(code - 32);
        }
    }
}

/* Split row: scale of block b at bytes 2b, 2b+1; code i at scale region + i. */
static void dequant_row_q8_0_split(const uint8_t* row, int64_t cols, float* out)
{
    int64_t nb = (cols + O_Q8_0_WEIGHTS - 1) / O_Q8_0_WEIGHTS;
    const uint8_t* codes = row + split_scale_bytes(nb);
    for (int64_t c = 0; c < cols; c++) {
        float d = gqo_f16_to_f32(read_u16le(row + 2 * (c / O_Q8_0_WEIGHTS)));
        out[c] = d * (float)(int8_t)codes[c];
    }
}

static int dequant_row(int type, const uint8_t* row, int64_t cols, float* out)
{
    if (type == GQO_TYPE_Q8_0_SPLIT) {
        dequant_row_q8_0_split(row, cols, out);
        return 0;
    }
    if (type == GQO_TYPE_Q5_0) {
        dequant_row_q5_0(row, cols, out);
        return 0;
    }
    if (type == GQO_TYPE_Q5_K) {
        dequant_row_q5_k(row, cols, out);
        return 0;
    }
    if (type == GQO_TYPE_Q6_K) {
        dequant_row_q6_k(row, cols, out);
        return 0;
    }
    if (type == GQO_TYPE_Q8_0) {
        dequant_row_q8_0(row, cols, out);
        return 0;
    }
    if (type == GQO_TYPE_Q4_K) {
        dequant_row_q4_k(row, cols, out);
        return 0;
    }
    return -1;
}

int gqo_dequant(int type, const void* W, int64_t rows, int64_t cols, float* out)
{
    int64_t rb = gqo_row_bytes(type, cols);
    if (rb < 0 || type == GQO_TYPE_Q8_1 || rows < 0 || cols <= 0 || !W || !out)
        return -1;
    const uint8_t* base = (const uint8_t*)W;
    for (int64_t r = 0; r < rows; r++)
        dequant_row(type, base + r * rb, cols, out + r * cols);
    return 0;
}

/* ------------------------------------------------------------- products */

typedef struct {
    int type;
    const uint8_t* W;
    int64_t row_bytes, rows, cols, M;
    const float* X;
    double* Y;
    double* S;
    int64_t r0, r1;
    int status;
} prod_job;

/* For rows r0..r1-1: dequantise the row once, then for every m the f64 sum
 * over c in increasing order. Products of two binary32 values are exact in
 * binary64 (24 + 24 significant bits < 53). */
static void* prod_worker(void* arg)
{
    prod_job* job = (prod_job*)arg;
    float* w = (float*)malloc((size_t)job->cols * sizeof(float));
    if (!w) {
        job->status = -2;
        return NULL;
    }
    for (int64_t r = job->r0; r < job->r1; r++) {
        dequant_row(job->type, job->W + r * job->row_bytes, job->cols, w);
        for (int64_t m = 0; m < job->M; m++) {
            const float* x = job->X + m * job->cols;
            double acc = 0.0, sabs = 0.0;
            for (int64_t c = 0; c < job->cols; c++) {
                double p = (double)w[c] * (double)x[c];
                acc += p;
                sabs += fabs(p);
            }
            job->Y[m * job->rows + r] = acc;
            if (job->S)
                job->S[m * job->rows + r] = sabs;
        }
    }
    free(w);
    job->status = 0;
    return NULL;
}

int gqo_matmul(int type, const void* W, int64_t rows, int64_t cols,
               const float* X, int64_t M, double* Y, double* S, int nthreads)
{
    int64_t rb = gqo_row_bytes(type, cols);
    if (rb < 0 || type == GQO_TYPE_Q8_1 || rows < 0 || cols <= 0 || M < 0 || !W || !X || !Y)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > rows)
        nthreads = rows > 0 ? (int)rows : 1;
    prod_job jobs[256];
    pthread_t tids[256];
    for (int t = 0; t < nthreads; t++) {
        prod_job* j = &jobs[t];
        j->type = type;
        j->W = (const uint8_t*)W;
        j->row_bytes = rb;
        j->rows = rows;
        j->cols = cols;
        j->M = M;
        j->X = X;
        j->Y = Y;
        j->S = S;
        j->r0 = rows * t / nthreads;
        j->r1 = rows * (t + 1) / nthreads;
        j->status = -3;
    }
    if (nthreads == 1) {
        prod_worker(&jobs[0]);
        return jobs[0].status;
    }
    int started = 0;
    for (int t = 0; t < nthreads; t++) {
        if (pthread_create(&tids[t], NULL, prod_worker, &jobs[t]) != 0)
            break;
        started++;
    }
    for (int t = 0; t < started; t++)
        pthread_join(tids[t], NULL);
    for (int t = started; t < nthreads; t++) /* threads that did not start */
        prod_worker(&jobs[t]);
    for (int t = 0; t < nthreads; t++)
        if (jobs[t].status != 0)
            return jobs[t].status;
    return 0;
}

int gqo_matvec(int type, const void* W, int64_t rows, int64_t cols,
               const float* x, double* y, double* S, int nthreads)
{
    return gqo_matmul(type, W, rows, cols, x, 1, y, S, nthreads);
}

/* ------------------------------------------------ split Q8_0 repack */

int gqo_q8_0_split_repack(const void* W, int64_t rows, int64_t cols, void* out)
{
    int64_t rb = gqo_row_bytes(GQO_TYPE_Q8_0, cols);
    int64_t rs = gqo_row_bytes(GQO_TYPE_Q8_0_SPLIT, cols);
    if (rb < 0 || rows < 0 || cols <= 0 || !W || !out)
        return -1;
    int64_t nb = (cols + O_Q8_0_WEIGHTS - 1) / O_Q8_0_WEIGHTS;
    int64_t sb = split_scale_bytes(nb);
    const uint8_t* src = (const uint8_t*)W;
    uint8_t* dst = (uint8_t*)out;
    for (int64_t r = 0; r < rows; r++) {
        const uint8_t* in = src + r * rb;
        uint8_t* o = dst + r * rs;
        memset(o, 0, (size_t)sb);
        for (int64_t b = 0; b < nb; b++) {
            o[2 * b] = in[b * O_Q8_0_BYTES];
            o[2 * b + 1] = in[b * O_Q8_0_BYTES + 1];
            memcpy(o + sb + b * O_Q8_0_WEIGHTS, in + b * O_Q8_0_BYTES + 2, O_Q8_0_WEIGHTS);
        }
    }
    return 0;
}

/* --------------------------------------------- test-only quantisers */

/* Q8_0: d = fp16_RN(max|w| / 127), q = clamp(RNE(w / d), -127, 127). */
int gqo_quantize_q8_0(const float* w, int64_t rows, int64_t cols, uint8_t* out)
{
    int64_t rb = gqo_row_bytes(GQO_TYPE_Q8_0, cols);
    if (rows < 0 || cols <= 0 || !w || !out)
        return -1;
    int64_t nb = rb / O_Q8_0_BYTES;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t* blk = out + r * rb + b * O_Q8_0_BYTES;
            double amax = 0.0;
            for (int i = 0; i < O_Q8_0_WEIGHTS; i++) {
                int64_t c = b * O_Q8_0_WEIGHTS + i;
                if (c < cols && fabs((double)w[r * cols + c]) > amax)
                    amax = fabs((double)w[r * cols + c]);
            }
            uint16_t d16 = f64_to_f16_rne_mag(amax / 127.0);
            double d = (double)gqo_f16_to_f32(d16);
            blk[0] = (uint8_t)(d16 & 0xFF);
            blk[1] = (uint8_t)(d16 >> 8);
            for (int i = 0; i < O_Q8_0_WEIGHTS; i++) {
                int64_t c = b * O_Q8_0_WEIGHTS + i;
                double q = 0.0;
                if (c < cols && d != 0.0) {
                    q = nearbyint((double)w[r * cols + c] / d);
                    if (q > 127.0)
                        q = 127.0;
                    if (q < -127.0)
                        q = -127.0;
                }
                blk[2 + i] = (uint8_t)(int8_t)q;
            }
        }
    }
    return 0;
}

/* Q4_K, a plain covering quantiser: per sub-block j the grid
 * -dmin*m_j + d*sc_j*{0..15} covers [lo_j, hi_j] with lo_j = min(0, min w),
 * hi_j = max w; d and dmin are rounded up to fp16 so that the 6-bit codes
 * never exceed 63. Codes are rounded to nearest. */
int gqo_quantize_q4_k(const float* w, int64_t rows, int64_t cols, uint8_t* out)
{
    int64_t rb = gqo_row_bytes(GQO_TYPE_Q4_K, cols);
    if (rows < 0 || cols <= 0 || !w || !out)
        return -1;
    int64_t nb = rb / O_Q4_K_BYTES;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t* blk = out + r * rb + b * O_Q4_K_BYTES;
            double lo[8], hi[8];
            for (int j = 0; j < 8; j++) {
                lo[j] = 0.0;
                hi[j] = 0.0;
                int any = 0;
                for (int k = 0; k < 32; k++) {
                    int64_t c = b * O_Q4_K_WEIGHTS + 32 * j + k;
                    if (c >= cols)
                        continue;
                    double v = (double)w[r * cols + c];
                    if (!any || v > hi[j])
                        hi[j] = v;
                    if (v < lo[j])
                        lo[j] = v;
                    any = 1;
                }
            }
            double neg_lo_max = 0.0;
            for (int j = 0; j < 8; j++)
                if (-lo[j] > neg_lo_max)
                    neg_lo_max = -lo[j];
            uint16_t dmin16 = f64_to_f16_up(neg_lo_max / 63.0);
            double dmin = (double)gqo_f16_to_f32(dmin16);
            uint8_t m[8], sc[8];
            double span_max = 0.0, span[8];
            for (int j = 0; j < 8; j++) {
                double mj = (dmin > 0.0) ? ceil(-lo[j] / dmin) : 0.0;
                if (mj > 63.0)
                    mj = 63.0;
                m[j] = (uint8_t)mj;
                span[j] = hi[j] - lo[j] + dmin;
                if (span[j] > span_max)
                    span_max = span[j];
            }
            uint16_t d16 = f64_to_f16_up(span_max / (15.0 * 63.0));
            double d = (double)gqo_f16_to_f32(d16);
            for (int j = 0; j < 8; j++) {
                double s = (d > 0.0) ? ceil(span[j] / (15.0 * d)) : 0.0;
                if (s > 63.0)
                    s = 63.0;
                sc[j] = (uint8_t)s;
            }
            blk[0] = (uint8_t)(d16 & 0xFF);
            blk[1] = (uint8_t)(d16 >> 8);
            blk[2] = (uint8_t)(dmin16 & 0xFF);
            blk[3] = (uint8_t)(dmin16 >> 8);
            uint8_t* s = blk + 4;
            for (int j = 0; j < 4; j++) {
                s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
                s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
                s[j + 8] = (uint8_t)((sc[j + 4] & 0x0F) | ((m[j + 4] & 0x0F) << 4));
            }
            uint8_t codes[256];
            for (int i = 0; i < 256; i++) {
                int j = i / 32;
                int64_t c = b * O_Q4_K_WEIGHTS + i;
                double step = d * (double)sc[j];
                double q = 0.0;
                if (c < cols && step > 0.0) {
                    q = nearbyint(((double)w[r * cols + c] + dmin * (double)m[j]) / step);
                    if (q < 0.0)
                        q = 0.0;
                    if (q > 15.0)
                        q = 15.0;
                }
                codes[i] = (uint8_t)q;
            }
            uint8_t* qs = blk + 16;
            for (int g = 0; g < 4; g++)
                for (int l = 0; l < 32; l++)
                    qs[32 * g + l] = (uint8_t)(codes[64 * g + l] | (codes[64 * g + 32 + l] << 4));
        }
    }
    return 0;
}

/* ------------------------------------------- Q8_1 activation blocks */

/* The int8-activation decode path of the Loom porting skill ("What the
 * starter generates", the gen_llm.py row: activations quantised in
 * llama.cpp's Q8_1 numerics, multiplied with integer dot products). The page
 * names the numerics without printing them; the public Q8_1 block is the
 * reading taken, restated here as this file implements it. Per 32 values
 * (columns >= cols count as 0):
 *   amax = max |x|            (binary32)
 *   d    = amax / 127         (binary32 division, to nearest)
 *   id   = d != 0 ? 1 / d : 0 (binary32 division, to nearest)
 *   q_i  = roundf(x_i * id)   (binary32 product, then to nearest with ties
 *                              away from zero; |q_i| <= 127)
 *   Where 1 / d overflows (d below 2^-128, a block whose largest magnitude
 *   is under about 3.7e-37) the product is +-inf or, for x_i = 0, NaN; the
 *   public block leaves the conversion of those to an integer undefined.
 *   Reading taken: the rounded product is clamped to [-127, 127] and a NaN
 *   product gives 0, so such a block's codes are +-127 (by sign) and 0.
 *   Every other block's products lie within 127 * (1 + 2^-22) and round
 *   to at most 127, so the clamp never changes them. fp16(d) is 0 for
 *   these blocks, so their values x^ are 0 either way.
 *   bytes 0-1: fp16(d), 2-3: fp16(d * sum q_i) (binary32 product, then
 *   binary16, both to nearest even), 4..35: q_0..q_31 (int8).
 * The values the product then uses are x^_i = f32(fp16(d)) * q_i (exact). */
int gqo_quantize_q8_1(const float* x, int64_t n, int64_t cols, uint8_t* out)
{
    int64_t rb = gqo_row_bytes(GQO_TYPE_Q8_1, cols);
    if (n < 0 || cols <= 0 || !x || !out)
        return -1;
    int64_t nb = rb / O_Q8_1_BYTES;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t* blk = out + r * rb + b * O_Q8_1_BYTES;
            float v[O_Q8_1_VALUES];
            float amax = 0.0f;
            for (int i = 0; i < O_Q8_1_VALUES; i++) {
                int64_t c = b * O_Q8_1_VALUES + i;
                v[i] = c < cols ? x[r * cols + c] : 0.0f;
                if (fabsf(v[i]) > amax)
                    amax = fabsf(v[i]);
            }
            float d = amax / 127.0f;
            float id = d != 0.0f ? 1.0f / d : 0.0f;
            int sum = 0;
            for (int i = 0; i < O_Q8_1_VALUES; i++) {
                float p = v[i] * id;
                int q;
                if (p != p)
                    q = 0;
                else if (p >= 127.0f)
                    q = 127;
                else if (p <= -127.0f)
                    q = -127;
                else
                    q = (int)roundf(p);
                blk[4 + i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            float ds = (float)sum * d;
            uint16_t d16 = gqo_f32_to_f16_rne(d);
            uint16_t s16 = gqo_f32_to_f16_rne(ds);
            blk[0] = (uint8_t)(d16 & 0xFF);
            blk[1] = (uint8_t)(d16 >> 8);
            blk[2] = (uint8_t)(s16 & 0xFF);
            blk[3] = (uint8_t)(s16 >> 8);
        }
    }
    return 0;
}

/* out[r*cols + c] = x^ of column c: f32(fp16(d)) * q (exact in binary32:
 * 11 significant bits times 8). */
int gqo_dequant_q8_1(const uint8_t* xq, int64_t n, int64_t cols, float* out)
{
    int64_t rb = gqo_row_bytes(GQO_TYPE_Q8_1, cols);
    if (n < 0 || cols <= 0 || !xq || !out)
        return -1;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t c = 0; c < cols; c++) {
            const uint8_t* blk = xq + r * rb + (c / O_Q8_1_VALUES) * O_Q8_1_BYTES;
            float d = gqo_f16_to_f32(read_u16le(blk));
            out[r * cols + c] = d * (float)(int8_t)blk[4 + c % O_Q8_1_VALUES];
        }
    }
    return 0;
}
