/*
 * A C program that uses the attention library through its C interface only
 * (include/flash_attn.h): device buffers from the HIP runtime, one causal bf16
 * forward, results checked against the fp64 oracle (oracle/oracle.c, linked
 * as liboracle), and two error paths.  Exit status 0 when every check holds.
 *
 * Inputs: B=1, H=2, N=333 (ragged against every tile size), d=128, values from
 * a 64-bit LCG mapped to roughly uniform(-2, 2), rounded to bf16 (nearest
 * even); the oracle gets the exact values the GPU reads.
 * Tolerances (the library's bf16 bar): max |O - O_ref| <= 2e-2,
 * max |LSE - LSE_ref| <= 1e-2.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flash_attn.h"

void oracle_attn_fwd_rows(const double* q, const double* k, const double* v, int64_t B, int64_t H, int64_t N,
                          int64_t d, int causal, double scale, int p_quant, const int64_t* rows, int64_t nrows,
                          double* o, double* lse);

static uint16_t to_bf16(float x) {  /* round to nearest even (inputs are finite) */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

#define HIP_OK(x)                                                       \
    do {                                                                \
        if ((x) != hipSuccess) {                                        \
            fprintf(stderr, "HIP call failed: %s (line %d)\n", #x, __LINE__); \
            return 2;                                                   \
        }                                                               \
    } while (0)

int main(void) {
    const int64_t B = 1, H = 2, N = 333, d = 128, n = B * H * N * d, rows = B * H * N;
    const double scale = 1.0 / sqrt((double)d);
    uint16_t* hx[3];
    double* rx[3];
    uint64_t state = 0x9E3779B97F4A7C15ull;
    for (int t = 0; t < 3; ++t) {
        hx[t] = malloc(sizeof(uint16_t) * n);
        rx[t] = malloc(sizeof(double) * n);
        for (int64_t i = 0; i < n; ++i) {
            state = state * 6364136223846793005ull + 1442695040888963407ull;
            const float u = (float)((state >> 40) * (1.0 / 16777216.0));  /* [0, 1) */
            hx[t][i] = to_bf16(4.0f * u - 2.0f);
            rx[t][i] = from_bf16(hx[t][i]);
        }
    }

    void* dx[3];
    void* dout;
    float* dlse;
    for (int t = 0; t < 3; ++t) {
        HIP_OK(hipMalloc(&dx[t], sizeof(uint16_t) * n));
        HIP_OK(hipMemcpy(dx[t], hx[t], sizeof(uint16_t) * n, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&dout, sizeof(uint16_t) * n));
    HIP_OK(hipMalloc((void**)&dlse, sizeof(float) * rows));

    const flash_attn_layout lay = {B, H, N, d, H * N * d, N * d, d};
    int fails = 0;

    /* error paths: reported synchronously, nothing launched */
    flash_attn_status st = flash_attn_fwd(NULL, dx[1], dx[2], dout, dlse, lay, FLASH_ATTN_BF16, 1, (float)scale,
                                          NULL, NULL);
    printf("NULL q -> %d (%s)\n", (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_ERR_NULL;
    flash_attn_layout bad = lay;
    bad.head_dim = 96;
    st = flash_attn_fwd(dx[0], dx[1], dx[2], dout, dlse, bad, FLASH_ATTN_BF16, 1, (float)scale, NULL, NULL);
    printf("head_dim 96 -> %d (%s)\n", (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_ERR_UNSUPPORTED;

    st = flash_attn_fwd(dx[0], dx[1], dx[2], dout, dlse, lay, FLASH_ATTN_BF16, 1, (float)scale, NULL, NULL);
    printf("causal bf16 forward B%lld H%lld N%lld d%lld -> %d (%s)\n", (long long)B, (long long)H, (long long)N,
           (long long)d, (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_OK;
    HIP_OK(hipDeviceSynchronize());

    uint16_t* ho = malloc(sizeof(uint16_t) * n);
    float* hl = malloc(sizeof(float) * rows);
    HIP_OK(hipMemcpy(ho, dout, sizeof(uint16_t) * n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dlse, sizeof(float) * rows, hipMemcpyDeviceToHost));

    double* oref = malloc(sizeof(double) * n);
    double* lref = malloc(sizeof(double) * rows);
    oracle_attn_fwd_rows(rx[0], rx[1], rx[2], B, H, N, d, 1, scale, 0, NULL, 0, oref, lref);
    double eo = 0.0, el = 0.0;
    for (int64_t i = 0; i < n; ++i) eo = fmax(eo, fabs(from_bf16(ho[i]) - oref[i]));
    for (int64_t i = 0; i < rows; ++i) el = fmax(el, fabs((double)hl[i] - lref[i]));
    printf("max|dO| = %.3e  max|dLSE| = %.3e\n", eo, el);
    fails += !(eo <= 2e-2) + !(el <= 1e-2);

    for (int t = 0; t < 3; ++t) {
        hipFree(dx[t]);
        free(hx[t]);
        free(rx[t]);
    }
    hipFree(dout);
    hipFree(dlse);
    free(ho);
    free(hl);
    free(oref);
    free(lref);
    printf(fails ? "FAILED (%d checks)\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
