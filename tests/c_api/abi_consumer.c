/*
 * A C program that uses the attention library through its C interface only
 * (include/flash_attn.h): device buffers from the HIP runtime, one causal bf16
 * forward and the backward on its results (workspace sized by
 * flash_attn_bwd_workspace_size), checked against the fp64 oracle
 * (oracle/oracle.c, linked as liboracle), and three error paths.  Exit
 * status 0 when every check holds.
 *
 * Inputs: B=1, H=2, N=333 (ragged against every tile size), d=128; Q, K, V
 * and dO from a 64-bit LCG mapped to roughly uniform(-2, 2), rounded to bf16
 * (nearest even); the oracle gets the exact values the GPU reads.
 * Tolerances (the library's bf16 bar): max |O - O_ref| <= 2e-2,
 * max |LSE - LSE_ref| <= 1e-2; for each of dQ, dK, dV
 * max |g - g_ref| <= 2e-2 * max(1, max |g_ref|) and
 * rms(g - g_ref) <= 1e-2 * rms(g_ref).
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
void oracle_attn_bwd_rows(const double* q, const double* k, const double* v, const double* dout, int64_t B,
                          int64_t H, int64_t N, int64_t d, int causal, double scale, const int64_t* qrows,
                          int64_t nq, const int64_t* krows, int64_t nk, double* dq, double* dk, double* dv);

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
    uint16_t* hx[4];  /* q, k, v, dO */
    double* rx[4];
    uint64_t state = 0x9E3779B97F4A7C15ull;
    for (int t = 0; t < 4; ++t) {
        hx[t] = malloc(sizeof(uint16_t) * n);
        rx[t] = malloc(sizeof(double) * n);
        for (int64_t i = 0; i < n; ++i) {
            state = state * 6364136223846793005ull + 1442695040888963407ull;
            const float u = (float)((state >> 40) * (1.0 / 16777216.0));  /* [0, 1) */
            hx[t][i] = to_bf16(4.0f * u - 2.0f);
            rx[t][i] = from_bf16(hx[t][i]);
        }
    }

    void* dx[4];
    void* dev_o;
    float* dev_lse;
    for (int t = 0; t < 4; ++t) {
        HIP_OK(hipMalloc(&dx[t], sizeof(uint16_t) * n));
        HIP_OK(hipMemcpy(dx[t], hx[t], sizeof(uint16_t) * n, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&dev_o, sizeof(uint16_t) * n));
    HIP_OK(hipMalloc((void**)&dev_lse, sizeof(float) * rows));

    const flash_attn_layout lay = {B, H, N, d, H * N * d, N * d, d};
    int fails = 0;

    /* error paths: reported synchronously, nothing launched */
    flash_attn_status st = flash_attn_fwd(NULL, dx[1], dx[2], dev_o, dev_lse, lay, FLASH_ATTN_BF16, 1, (float)scale,
                                          NULL, NULL);
    printf("NULL q -> %d (%s)\n", (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_ERR_NULL;
    flash_attn_layout bad = lay;
    bad.head_dim = 96;
    st = flash_attn_fwd(dx[0], dx[1], dx[2], dev_o, dev_lse, bad, FLASH_ATTN_BF16, 1, (float)scale, NULL, NULL);
    printf("head_dim 96 -> %d (%s)\n", (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_ERR_UNSUPPORTED;

    st = flash_attn_fwd(dx[0], dx[1], dx[2], dev_o, dev_lse, lay, FLASH_ATTN_BF16, 1, (float)scale, NULL, NULL);
    printf("causal bf16 forward B%lld H%lld N%lld d%lld -> %d (%s)\n", (long long)B, (long long)H, (long long)N,
           (long long)d, (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_OK;
    HIP_OK(hipDeviceSynchronize());

    uint16_t* ho = malloc(sizeof(uint16_t) * n);
    float* hl = malloc(sizeof(float) * rows);
    HIP_OK(hipMemcpy(ho, dev_o, sizeof(uint16_t) * n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dev_lse, sizeof(float) * rows, hipMemcpyDeviceToHost));

    double* oref = malloc(sizeof(double) * n);
    double* lref = malloc(sizeof(double) * rows);
    oracle_attn_fwd_rows(rx[0], rx[1], rx[2], B, H, N, d, 1, scale, 0, NULL, 0, oref, lref);
    double eo = 0.0, el = 0.0;
    for (int64_t i = 0; i < n; ++i) eo = fmax(eo, fabs(from_bf16(ho[i]) - oref[i]));
    for (int64_t i = 0; i < rows; ++i) el = fmax(el, fabs((double)hl[i] - lref[i]));
    printf("max|dO| = %.3e  max|dLSE| = %.3e\n", eo, el);
    fails += !(eo <= 2e-2) + !(el <= 1e-2);

    /* backward on the forward's O and LSE */
    const size_t ws_bytes = flash_attn_bwd_workspace_size(lay, FLASH_ATTN_BF16);
    void* ws;
    void* dg[3];
    HIP_OK(hipMalloc(&ws, ws_bytes));
    for (int t = 0; t < 3; ++t) HIP_OK(hipMalloc(&dg[t], sizeof(uint16_t) * n));
    st = flash_attn_bwd(dx[0], dx[1], dx[2], dev_o, dev_lse, dx[3], dg[0], dg[1], dg[2], lay, FLASH_ATTN_BF16, 1,
                        (float)scale, ws, ws_bytes / 2, NULL);
    printf("workspace %zu of %zu bytes -> %d (%s)\n", ws_bytes / 2, ws_bytes, (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_ERR_WORKSPACE;
    st = flash_attn_bwd(dx[0], dx[1], dx[2], dev_o, dev_lse, dx[3], dg[0], dg[1], dg[2], lay, FLASH_ATTN_BF16, 1,
                        (float)scale, ws, ws_bytes, NULL);
    printf("causal bf16 backward, workspace %zu bytes -> %d (%s)\n", ws_bytes, (int)st, flash_attn_status_str(st));
    fails += st != FLASH_ATTN_OK;
    HIP_OK(hipDeviceSynchronize());

    double* gref[3];
    for (int t = 0; t < 3; ++t) gref[t] = malloc(sizeof(double) * n);
    oracle_attn_bwd_rows(rx[0], rx[1], rx[2], rx[3], B, H, N, d, 1, scale, NULL, 0, NULL, 0, gref[0], gref[1],
                         gref[2]);
    static const char* gname[3] = {"dQ", "dK", "dV"};
    for (int t = 0; t < 3; ++t) {
        HIP_OK(hipMemcpy(ho, dg[t], sizeof(uint16_t) * n, hipMemcpyDeviceToHost));
        double emax = 0.0, rmax = 0.0, e2 = 0.0, r2 = 0.0;
        int finite = 1;
        for (int64_t i = 0; i < n; ++i) {
            const double g = from_bf16(ho[i]), r = gref[t][i];
            finite &= isfinite(g);
            emax = fmax(emax, fabs(g - r));
            rmax = fmax(rmax, fabs(r));
            e2 += (g - r) * (g - r);
            r2 += r * r;
        }
        const double bound = 2e-2 * fmax(1.0, rmax), rel = sqrt(e2 / fmax(r2, 1e-300));
        printf("%s: max|err| = %.3e (bound %.3e)  rms err/ref = %.3e\n", gname[t], emax, bound, rel);
        fails += !finite + !(emax <= bound) + !(rel <= 1e-2);
    }

    for (int t = 0; t < 3; ++t) {
        hipFree(dg[t]);
        free(gref[t]);
    }
    hipFree(ws);
    for (int t = 0; t < 4; ++t) {
        hipFree(dx[t]);
        free(hx[t]);
        free(rx[t]);
    }
    hipFree(dev_o);
    hipFree(dev_lse);
    free(ho);
    free(hl);
    free(oref);
    free(lref);
    printf(fails ? "FAILED (%d checks)\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
