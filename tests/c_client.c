/*
 * A plain C11 client of the C ABI: include/gq.h plus the HIP runtime's C
 * interface for device memory, no Python and no torch. It shows that the
 * boundary is usable from C as declared, and checks results that have a
 * closed form:
 *
 *   Q8_0 blocks with d = 1 (fp16 0x3C00) and integer codes q, integer
 *   activations x: every product q * x and every partial sum is an integer
 *   below 2^24, so y = W x is exact in fp32 and must equal the integer sum
 *   computed here; gq_dequant must return the codes themselves.
 *
 * It runs gq_row_bytes, gq_matvec (default stream and a created stream),
 * gq_matmul with M = 2 and M = 20 (few-row and matrix-core routes),
 * gq_dequant, gq_moe_bucket and gq_moe_scatter on a hand-worked case, and a
 * few calls the host checks reject. Prints "c client ok"
 * and exits 0 on success; any mismatch prints the case and exits 1.
 *
 * Built by __graft_entry__.build() (gcc, linked against libgq.so and
 * libamdhip64); run by tests/test_gpu_c_client.py.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gq.h"

#define ROWS 300
#define COLS 1024 /* 32 blocks of 32 */
#define MMAX 20

static int failures = 0;

static void check(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "c client: FAILED %s\n", what);
        fflush(stderr);
        failures++;
    }
}

static int hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        fprintf(stderr, "c client: %s: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

/* a small deterministic generator (64-bit LCG, top bits) */
static uint64_t state = 0x9E3779B97F4A7C15ull;
static int next_int(int lo, int hi) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (int)((state >> 33) % (uint64_t)(hi - lo + 1));
}

int main(void) {
    const int64_t rb = gq_row_bytes(GQ_FMT_Q8_0, COLS);
    check(rb == (COLS / 32) * 34, "gq_row_bytes(Q8_0)");
    check(gq_row_bytes(GQ_FMT_Q4_K, 4096) == 16 * 144, "gq_row_bytes(Q4_K)");
    check(gq_row_bytes(99, 32) < 0, "gq_row_bytes(unknown format)");

    /* host data: W (Q8_0, d = 1), X (MMAX rows of integers) */
    uint8_t* W = (uint8_t*)malloc((size_t)(ROWS * rb));
    int8_t* codes = (int8_t*)malloc((size_t)ROWS * COLS);
    float* X = (float*)malloc(sizeof(float) * MMAX * COLS);
    float* Y = (float*)malloc(sizeof(float) * MMAX * ROWS);
    float* D = (float*)malloc(sizeof(float) * ROWS * COLS);
    if (!W || !codes || !X || !Y || !D) return 2;
    for (int r = 0; r < ROWS; r++) {
        for (int b = 0; b < COLS / 32; b++) {
            uint8_t* blk = W + r * rb + b * 34;
            blk[0] = 0x00;
            blk[1] = 0x3C; /* fp16 1.0, little-endian */
            for (int i = 0; i < 32; i++) {
                const int q = next_int(-127, 127);
                codes[(size_t)r * COLS + b * 32 + i] = (int8_t)q;
                blk[2 + i] = (uint8_t)(int8_t)q;
            }
        }
    }
    for (int i = 0; i < MMAX * COLS; i++) X[i] = (float)next_int(-8, 8);

    void *dW = NULL, *dX = NULL, *dY = NULL, *dD = NULL;
    if (!hip_ok(hipMalloc(&dW, (size_t)(ROWS * rb)), "hipMalloc W") ||
        !hip_ok(hipMalloc(&dX, sizeof(float) * MMAX * COLS), "hipMalloc X") ||
        !hip_ok(hipMalloc(&dY, sizeof(float) * MMAX * ROWS), "hipMalloc Y") ||
        !hip_ok(hipMalloc(&dD, sizeof(float) * ROWS * COLS), "hipMalloc D"))
        return 2;
    if (!hip_ok(hipMemcpy(dW, W, (size_t)(ROWS * rb), hipMemcpyHostToDevice), "copy W") ||
        !hip_ok(hipMemcpy(dX, X, sizeof(float) * MMAX * COLS, hipMemcpyHostToDevice), "copy X"))
        return 2;

    /* gq_matvec on the default stream (NULL), then on a created stream */
    hipStream_t s = NULL;
    if (!hip_ok(hipStreamCreate(&s), "hipStreamCreate")) return 2;
    for (int pass = 0; pass < 2; pass++) {
        void* stream = pass == 0 ? NULL : (void*)s;
        int st = gq_matvec(GQ_FMT_Q8_0, dW, ROWS, COLS, (const float*)dX, (float*)dY, stream);
        check(st == GQ_OK, "gq_matvec status");
        if (!hip_ok(pass == 0 ? hipDeviceSynchronize() : hipStreamSynchronize(s), "sync")) return 2;
        if (!hip_ok(hipMemcpy(Y, dY, sizeof(float) * ROWS, hipMemcpyDeviceToHost), "copy y")) return 2;
        for (int r = 0; r < ROWS; r++) {
            int64_t want = 0;
            for (int c = 0; c < COLS; c++) want += (int64_t)codes[(size_t)r * COLS + c] * (int64_t)X[c];
            if (Y[r] != (float)want) {
                fprintf(stderr, "c client: matvec pass %d row %d: %g != %lld\n", pass, r, Y[r],
                        (long long)want);
                failures++;
                break;
            }
        }
    }

    /* gq_matmul: M = 2 (few-row route) and M = MMAX (matrix cores) */
    const int ms[2] = {2, MMAX};
    for (int k = 0; k < 2; k++) {
        const int M = ms[k];
        int st = gq_matmul(GQ_FMT_Q8_0, dW, ROWS, COLS, (const float*)dX, M, (float*)dY, (void*)s);
        check(st == GQ_OK, "gq_matmul status");
        if (!hip_ok(hipStreamSynchronize(s), "sync matmul")) return 2;
        if (!hip_ok(hipMemcpy(Y, dY, sizeof(float) * M * ROWS, hipMemcpyDeviceToHost), "copy Y")) return 2;
        int bad = 0;
        for (int m = 0; m < M && !bad; m++) {
            for (int r = 0; r < ROWS; r++) {
                int64_t want = 0;
                for (int c = 0; c < COLS; c++)
                    want += (int64_t)codes[(size_t)r * COLS + c] * (int64_t)X[(size_t)m * COLS + c];
                if (Y[(size_t)m * ROWS + r] != (float)want) {
                    fprintf(stderr, "c client: matmul M=%d row %d col %d: %g != %lld\n", M, m, r,
                            Y[(size_t)m * ROWS + r], (long long)want);
                    bad = 1;
                    break;
                }
            }
        }
        failures += bad;
    }

    /* gq_dequant: the codes themselves (d = 1) */
    check(gq_dequant(GQ_FMT_Q8_0, dW, ROWS, COLS, (float*)dD) == GQ_OK, "gq_dequant status");
    if (!hip_ok(hipMemcpy(D, dD, sizeof(float) * ROWS * COLS, hipMemcpyDeviceToHost), "copy D")) return 2;
    for (int i = 0; i < ROWS * COLS; i++) {
        if (D[i] != (float)codes[i]) {
            fprintf(stderr, "c client: dequant element %d: %g != %d\n", i, D[i], codes[i]);
            failures++;
            break;
        }
    }

    /* gq_moe_bucket / gq_moe_scatter on 4 positions x 2 slots, 4 experts:
     * ids 2 0 | 2 1 | 0 0 | 3 2 give counts 3 1 3 1 and positions
     * 4 0 5 3 1 2 7 6 (a stable sort by id); the scatter then adds to each
     * position w0 * row(pos[2t]) + w1 * row(pos[2t + 1]), exact in small
     * integers */
    {
        const int32_t ids[8] = {2, 0, 2, 1, 0, 0, 3, 2};
        const int32_t want_pos[8] = {4, 0, 5, 3, 1, 2, 7, 6};
        const int64_t want_counts[4] = {3, 1, 3, 1};
        const int R = 3;
        float yb[8 * 3], w[8], out[4 * 3];
        for (int p = 0; p < 8; p++)
            for (int r = 0; r < R; r++) yb[p * R + r] = (float)(10 * p + r);
        for (int a = 0; a < 8; a++) w[a] = (float)(a % 3 + 1);
        for (int i = 0; i < 4 * R; i++) out[i] = 1.0f;
        void *dids = NULL, *dcnt = NULL, *dord = NULL, *dpos = NULL, *dyb = NULL, *dw = NULL, *dout = NULL;
        if (!hip_ok(hipMalloc(&dids, sizeof(ids)), "hipMalloc ids") ||
            !hip_ok(hipMalloc(&dcnt, sizeof(want_counts)), "hipMalloc counts") ||
            !hip_ok(hipMalloc(&dord, sizeof(ids)), "hipMalloc order") ||
            !hip_ok(hipMalloc(&dpos, sizeof(ids)), "hipMalloc pos") ||
            !hip_ok(hipMalloc(&dyb, sizeof(yb)), "hipMalloc yb") ||
            !hip_ok(hipMalloc(&dw, sizeof(w)), "hipMalloc w") ||
            !hip_ok(hipMalloc(&dout, sizeof(out)), "hipMalloc out"))
            return 2;
        if (!hip_ok(hipMemcpy(dids, ids, sizeof(ids), hipMemcpyHostToDevice), "copy ids") ||
            !hip_ok(hipMemcpy(dyb, yb, sizeof(yb), hipMemcpyHostToDevice), "copy yb") ||
            !hip_ok(hipMemcpy(dw, w, sizeof(w), hipMemcpyHostToDevice), "copy w") ||
            !hip_ok(hipMemcpy(dout, out, sizeof(out), hipMemcpyHostToDevice), "copy out"))
            return 2;
        check(gq_moe_bucket((const int32_t*)dids, 8, 4, (int64_t*)dcnt, (int32_t*)dord, (int32_t*)dpos,
                            (void*)s) == GQ_OK, "gq_moe_bucket status");
        check(gq_moe_scatter((const float*)dyb, R, (const int32_t*)dpos, (const float*)dw, 8, 2,
                             (float*)dout, (void*)s) == GQ_OK, "gq_moe_scatter status");
        if (!hip_ok(hipStreamSynchronize(s), "sync moe")) return 2;
        int32_t pos[8];
        int64_t counts[4];
        float got[4 * 3];
        if (!hip_ok(hipMemcpy(pos, dpos, sizeof(pos), hipMemcpyDeviceToHost), "copy pos") ||
            !hip_ok(hipMemcpy(counts, dcnt, sizeof(counts), hipMemcpyDeviceToHost), "copy counts") ||
            !hip_ok(hipMemcpy(got, dout, sizeof(got), hipMemcpyDeviceToHost), "copy out"))
            return 2;
        check(memcmp(pos, want_pos, sizeof(pos)) == 0, "gq_moe_bucket positions");
        check(memcmp(counts, want_counts, sizeof(counts)) == 0, "gq_moe_bucket counts");
        for (int t = 0; t < 4; t++)
            for (int r = 0; r < R; r++) {
                float want = 1.0f;
                for (int j = 0; j < 2; j++) want += w[2 * t + j] * yb[want_pos[2 * t + j] * R + r];
                if (got[t * R + r] != want) {
                    fprintf(stderr, "c client: scatter position %d col %d: %g != %g\n", t, r, got[t * R + r], want);
                    failures++;
                }
            }
        hipFree(dids); hipFree(dcnt); hipFree(dord); hipFree(dpos); hipFree(dyb); hipFree(dw); hipFree(dout);
    }

    /* calls the host checks reject (nothing is launched) */
    check(gq_matvec(7, dW, ROWS, COLS, (const float*)dX, (float*)dY, NULL) == GQ_ERR_FMT, "bad fmt");
    check(gq_matvec(GQ_FMT_Q8_0, NULL, ROWS, COLS, (const float*)dX, (float*)dY, NULL) == GQ_ERR_NULL,
          "null W");
    check(gq_matvec(GQ_FMT_Q8_0, dW, -1, COLS, (const float*)dX, (float*)dY, NULL) == GQ_ERR_SHAPE,
          "negative rows");
    check(gq_matvec(GQ_FMT_Q8_0, dW, ROWS, COLS, (const float*)dX, (float*)dW, NULL) == GQ_ERR_OVERLAP,
          "y overlapping W");
    check(strncmp(gq_status_str(GQ_ERR_NULL), "GQ_ERR_NULL", 11) == 0, "gq_status_str");

    hipStreamDestroy(s);
    hipFree(dW);
    hipFree(dX);
    hipFree(dY);
    hipFree(dD);
    free(W);
    free(codes);
    free(X);
    free(Y);
    free(D);
    if (failures) {
        fprintf(stderr, "c client: %d failure(s)\n", failures);
        return 1;
    }
    printf("c client ok\n");
    return 0;
}
