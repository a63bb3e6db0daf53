/*
 * A plain C99 client of libhkgemm.so: the headers compile as C, and the
 * entry points run from C with HIP's C runtime API for device memory.
 *
 *   hk_c_client          checks argument validation only (no GPU call)
 *   hk_c_client --gpu    also runs hk_gemm_bf16, hk_gemm_fp8 and
 *                        hk_attn_fwd_bf16 on small integer-valued inputs
 *                        and compares with the exact products rounded
 *                        once to bf16 (integer sums far below 2^24 are
 *                        exact in fp32 whatever the order of the sums)
 *
 * Prints one line per check and "hk_c_client OK" at the end; exits 1 on
 * the first mismatch or error.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hk_attn.h"
#include "hk_gemm.h"

static int fail(const char *what) {
    printf("FAIL %s\n", what);
    return 1;
}

/* bf16 bits of a small integer (exact: the fp32 pattern's upper half) */
static uint16_t bf16_of_int(int v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float float_of_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bf16 bits of x rounded to nearest even (x finite and exact in fp32) */
static uint16_t bf16_rne(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP E4M3FN byte of an integer in [-4, 4] */
static uint8_t e4m3_of_int(int v) {
    static const uint8_t mag[5] = {0x00, 0x38, 0x40, 0x44, 0x48}; /* 0, 1, 2, 3, 4 */
    uint8_t b = mag[v < 0 ? -v : v];
    return (uint8_t)(v < 0 ? (b | 0x80) : b);
}

static int validation_checks(void) {
    /* negative sizes, ld below K, a bad dtype: rejected before any HIP call,
     * so the pointers (aligned, never dereferenced) need not be valid */
    void *dummy = (void *)(uintptr_t)0x100000;
    if (hk_gemm_bf16(dummy, dummy, dummy, -1, 8, 8, 8, 8, 8, 0) != HK_ERROR_INVALID_VALUE)
        return fail("negative M");
    if (hk_gemm_bf16(dummy, dummy, dummy, 8, 8, 16, 8, 16, 8, 0) != HK_ERROR_INVALID_VALUE)
        return fail("lda < K");
    if (hk_gemm_ex(7, dummy, dummy, dummy, 8, 8, 8, 8, 8, 8, 1.0f, 1.0f, NULL, 0) !=
        HK_ERROR_INVALID_VALUE)
        return fail("bad dtype");
    if (hk_gemm_fp8(dummy, dummy, dummy, 8, 8, 16, 16, 16, 8, NAN, 1.0f, 0) !=
        HK_ERROR_INVALID_VALUE)
        return fail("NaN scale");
    if (hk_gemm_bf16(dummy, dummy, dummy, 0, 8, 8, 8, 8, 8, 0) != HK_SUCCESS)
        return fail("empty product");
    if (strlen(hk_status_string(HK_ERROR_NOT_SUPPORTED)) == 0) return fail("status string");
    if (hk_version() < 300) return fail("version");
    printf("validation ok (version %d)\n", (int)hk_version());
    return 0;
}

#define M 300
#define N 260
#define K 192

static int gemm_checks(void) {
    static uint16_t a16[M * K], b16[N * K], c16[M * N];
    static uint8_t a8[M * K], b8[N * K];
    static int ai[M * K], bi[N * K];
    unsigned seed = 12345u;
    for (int i = 0; i < M * K; ++i) {
        seed = seed * 1103515245u + 12345u;
        ai[i] = (int)((seed >> 16) % 9u) - 4;
        a16[i] = bf16_of_int(ai[i]);
        a8[i] = e4m3_of_int(ai[i]);
    }
    for (int i = 0; i < N * K; ++i) {
        seed = seed * 1103515245u + 12345u;
        bi[i] = (int)((seed >> 16) % 9u) - 4;
        b16[i] = bf16_of_int(bi[i]);
        b8[i] = e4m3_of_int(bi[i]);
    }
    void *dA = NULL, *dB = NULL, *dC = NULL;
    if (hipMalloc(&dA, sizeof a16) != hipSuccess || hipMalloc(&dB, sizeof b16) != hipSuccess ||
        hipMalloc(&dC, sizeof c16) != hipSuccess)
        return fail("hipMalloc");
    for (int pass = 0; pass < 2; ++pass) {
        const int fp8 = pass == 1;
        const float sa = 0.5f, sb = 4.0f; /* powers of two keep the FP8 results exact */
        if (hipMemcpy(dA, fp8 ? (void *)a8 : (void *)a16, fp8 ? sizeof a8 : sizeof a16,
                      hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(dB, fp8 ? (void *)b8 : (void *)b16, fp8 ? sizeof b8 : sizeof b16,
                      hipMemcpyHostToDevice) != hipSuccess)
            return fail("hipMemcpy in");
        hk_status s = fp8 ? hk_gemm_fp8(dA, dB, dC, M, N, K, K, K, N, sa, sb, 0)
                          : hk_gemm_bf16(dA, dB, dC, M, N, K, K, K, N, 0);
        if (s != HK_SUCCESS) {
            printf("status %s\n", hk_status_string(s));
            return fail(fp8 ? "hk_gemm_fp8" : "hk_gemm_bf16");
        }
        if (hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(c16, dC, sizeof c16, hipMemcpyDeviceToHost) != hipSuccess)
            return fail("hipMemcpy out");
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < N; ++j) {
                long acc = 0;
                for (int k = 0; k < K; ++k) acc += (long)ai[i * K + k] * bi[j * K + k];
                const double exact = fp8 ? (double)acc * sa * sb : (double)acc;
                const uint16_t want = bf16_rne(exact);
                /* +0 and -0 are the same result */
                if (c16[i * N + j] != want && !((c16[i * N + j] | want) == 0x8000u)) {
                    printf("C[%d][%d] = %g, expected %g (exact %g)\n", i, j,
                           (double)float_of_bf16(c16[i * N + j]), (double)float_of_bf16(want),
                           exact);
                    return fail(fp8 ? "fp8 product" : "bf16 product");
                }
            }
        printf("%s %dx%dx%d exact\n", fp8 ? "hk_gemm_fp8" : "hk_gemm_bf16", M, N, K);
    }
    hipFree(dA);
    hipFree(dB);
    hipFree(dC);
    return 0;
}

static int attention_check(void) {
    /* all-zero queries: every weight is equal, so O is the mean of V's rows
     * (exact for 64 keys of integer values) and LSE = log(64) */
    enum { B = 1, H = 2, S = 64, D = 64 };
    static uint16_t q[B * H * S * D], k[B * H * S * D], v[B * H * S * D], o[B * H * S * D];
    static float lse[B * H * S];
    static int vi[B * H * S * D];
    for (int i = 0; i < B * H * S * D; ++i) {
        q[i] = bf16_of_int(0);
        k[i] = bf16_of_int((i % 7) - 3);
        vi[i] = (i * 5 % 9) - 4;
        v[i] = bf16_of_int(vi[i]);
    }
    void *dq, *dk, *dv, *d_o, *dl;
    if (hipMalloc(&dq, sizeof q) != hipSuccess || hipMalloc(&dk, sizeof k) != hipSuccess ||
        hipMalloc(&dv, sizeof v) != hipSuccess || hipMalloc(&d_o, sizeof o) != hipSuccess ||
        hipMalloc(&dl, sizeof lse) != hipSuccess)
        return fail("hipMalloc (attention)");
    if (hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice) != hipSuccess)
        return fail("hipMemcpy in (attention)");
    hk_status s = hk_attn_fwd_bf16(dq, dk, dv, d_o, (float *)dl, B, H, H, S, D, 0.125f, 0, NULL, 0);
    if (s != HK_SUCCESS) return fail("hk_attn_fwd_bf16");
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(o, d_o, sizeof o, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(lse, dl, sizeof lse, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("hipMemcpy out (attention)");
    for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
            long sum = 0;
            for (int t = 0; t < S; ++t) sum += vi[(h * S + t) * D + d];
            const double mean = (double)sum / S;
            for (int t = 0; t < S; ++t)
                if ((double)float_of_bf16(o[(h * S + t) * D + d]) != mean) {
                    printf("O[%d][%d][%d] = %g, expected %g\n", h, t, d,
                           (double)float_of_bf16(o[(h * S + t) * D + d]), mean);
                    return fail("attention mean");
                }
        }
    for (int i = 0; i < B * H * S; ++i)
        if (fabs((double)lse[i] - log(64.0)) > 1e-5 * (1.0 + log(64.0)))
            return fail("attention log-sum-exp");
    printf("hk_attn_fwd_bf16 all-zero queries: O is the mean of V, LSE = log 64\n");
    hipFree(dq);
    hipFree(dk);
    hipFree(dv);
    hipFree(d_o);
    hipFree(dl);
    return 0;
}

int main(int argc, char **argv) {
    const int gpu = argc > 1 && strcmp(argv[1], "--gpu") == 0;
    if (validation_checks()) return 1;
    if (gpu && (gemm_checks() || attention_check())) return 1;
    printf("hk_c_client OK\n");
    return 0;
}
