/*
 * oracle.c -- plain fp64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or constant with the HIP library and must never sit on the product path.
 *
 * Everything is computed in double precision with the obvious two-pass
 * definition: a full row of scores is materialised, its maximum taken, then
 * exponentials, their sum and the weighted sum of value rows.  There is no
 * tiling and no online softmax here; the GPU path reaches the same numbers by
 * a different route.
 *
 * Sources (page titles as printed on the pages):
 *  [FA-ja]  "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
 *           sec. 2.1 (S = QK^T, P = softmax(S), O = PV), sec. 6.1 (safe
 *           softmax: subtract the row maximum), sec. 7.2 (the forward keeps
 *           only O and the per-row statistics m, l), sec. 11.3 (causal mask is
 *           the lower triangle, key j allowed iff j <= i).
 *  [FA3]    "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
 *           Low-precision", section 技術 3 (FP8 e4m3, block quantisation with
 *           one scale per B_r x d / B_c x d block, incoherent processing with
 *           M = diag(+-1) * Hadamard) and section 数値誤差 (RMSE against an
 *           FP64 reference, per-tensor FP8 baseline).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - the softmax scale multiplies the scores (the pages' formulas omit it);
 *  - LSE is the natural-log log-sum-exp m + ln(l);
 *  - e4m3 is the OCP "fn" variant: bias 7, max finite 448, no infinities,
 *    round-to-nearest-even, saturating at +-448;
 *  - a block scale is amax(block)/448, 1 when the block is all zero;
 *  - the rotation is x -> (x * signs) H_d / sqrt(d) with Sylvester H_d.
 *
 * Built with gcc -O2 -fopenmp; parallel over independent rows only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of keys query row i may attend to: all N, or i+1 under the causal
 * (lower-triangular) mask of [FA-ja] sec. 11.3. */
static int64_t allowed_keys(int64_t i, int64_t N, int causal) {
    return causal ? i + 1 : N;
}

/*
 * One query row.  q_row: [d]; kh, vh: [N, d] for this (batch, head).
 * s: scratch of N doubles.  Writes o_row[d] and *lse.
 * p_quant: 0 = exact; 1 = the probabilities exp(s - m) are passed through the
 * e4m3 codec as e4m3(p * 256) / 256 before multiplying V (the rule used by the
 * fp8 comparison baselines; the sum l always uses the unquantised p).
 */
static uint8_t e4m3_encode_one(double x);
static double e4m3_decode_one(uint8_t c);

static void attn_row(const double* q_row, const double* kh, const double* vh,
                     int64_t N, int64_t d, int64_t i, int causal, double scale,
                     int p_quant, double* s, double* o_row, double* lse) {
    const int64_t n_allowed = allowed_keys(i, N, causal);
    /* pass 1: scores and their maximum (safe softmax, [FA-ja] sec. 6.1) */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_allowed; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += q_row[c] * kh[j * d + c];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    /* pass 2: exponentials, their sum, weighted sum of V rows */
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
    for (int64_t j = 0; j < n_allowed; ++j) {
        const double p = exp(s[j] - m);
        const double pw = p_quant ? e4m3_decode_one(e4m3_encode_one(p * 256.0)) / 256.0 : p;
        l += p;
        for (int64_t c = 0; c < d; ++c) o_row[c] += pw * vh[j * d + c];
    }
    for (int64_t c = 0; c < d; ++c) o_row[c] /= l;
    *lse = m + log(l);
}

/*
 * Forward attention on selected rows.
 * q, k, v: contiguous [B, H, N, d] doubles.
 * rows: flat row ids r = (b * H + h) * N + i, or NULL for every row in order.
 * o: [nrows, d]; lse: [nrows].
 */
void oracle_attn_fwd_rows(const double* q, const double* k, const double* v,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          int causal, double scale, int p_quant,
                          const int64_t* rows, int64_t nrows,
                          double* o, double* lse) {
    if (!rows) nrows = B * H * N;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            const int64_t bh = flat / N, i = flat % N;
            const double* kh = k + bh * N * d;
            const double* vh = v + bh * N * d;
            attn_row(q + flat * d, kh, vh, N, d, i, causal, scale, p_quant, s,
                     o + r * d, lse + r);
        }
        free(s);
    }
}

/* The probability row P[i, :] of one (b, h) (zeros at masked keys). */
void oracle_attn_probs_row(const double* q, const double* k,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           int causal, double scale, int64_t flat_row,
                           double* p_out) {
    (void)B; (void)H;
    const int64_t bh = flat_row / N, i = flat_row % N;
    const double* kh = k + bh * N * d;
    const int64_t n_allowed = allowed_keys(i, N, causal);
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) p_out[j] = 0.0;
    for (int64_t j = 0; j < n_allowed; ++j) {
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += q[flat_row * d + c] * kh[j * d + c];
        p_out[j] = scale * acc;
        if (p_out[j] > m) m = p_out[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_allowed; ++j) { p_out[j] = exp(p_out[j] - m); l += p_out[j]; }
    for (int64_t j = 0; j < n_allowed; ++j) p_out[j] /= l;
}

/*
 * Backward of the same definition, analytic gradient in fp64.  The pages give
 * no backward formulas; [FA-ja] sec. 7.2 only says S and P are recomputed from
 * Q, K, V and the saved statistics.  Plainest reading: the derivative of
 *   O = softmax(scale * Q K^T) V
 * which is
 *   P = softmax(scale * Q K^T) (masked),  D_i = sum_c dO_ic O_ic,
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 * O and the row statistics are recomputed here from Q, K, V (two-pass).
 *
 * qrows / krows: flat ids (b*H + h)*N + i of the dQ rows and of the dK/dV rows
 * wanted (NULL = all rows, in order).  dq: [nq, d], dk, dv: [nk, d].
 */
void oracle_attn_bwd_rows(const double* q, const double* k, const double* v,
                          const double* dout,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          int causal, double scale,
                          const int64_t* qrows, int64_t nq,
                          const int64_t* krows, int64_t nk,
                          double* dq, double* dk, double* dv) {
    const int64_t BH = B * H;
    if (!qrows) nq = BH * N;
    if (!krows) nk = BH * N;
    /* Which heads are touched. */
    char* need = (char*)calloc((size_t)BH, 1);
    for (int64_t r = 0; r < nq; ++r) need[(qrows ? qrows[r] : r) / N] = 1;
    for (int64_t r = 0; r < nk; ++r) need[(krows ? krows[r] : r) / N] = 1;
    /* Row statistics LSE_i and D_i for every row of every touched head. */
    double* lse = (double*)malloc(sizeof(double) * (size_t)(BH * N));
    double* Dv = (double*)malloc(sizeof(double) * (size_t)(BH * N));
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* orow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < BH * N; ++flat) {
            const int64_t bh = flat / N, i = flat % N;
            if (!need[bh]) continue;
            attn_row(q + flat * d, k + bh * N * d, v + bh * N * d, N, d, i, causal,
                     scale, 0, s, orow, &lse[flat]);
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) acc += dout[flat * d + c] * orow[c];
            Dv[flat] = acc;
        }
        free(s);
        free(orow);
    }
    /* dQ_i = scale * sum_j dS_ij k_j */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nq; ++r) {
        const int64_t flat = qrows ? qrows[r] : r;
        const int64_t bh = flat / N, i = flat % N;
        const double* qi = q + flat * d;
        const double* doi = dout + flat * d;
        double* out = dq + r * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        const int64_t n_allowed = allowed_keys(i, N, causal);
        for (int64_t j = 0; j < n_allowed; ++j) {
            const double* kj = k + (bh * N + j) * d;
            const double* vj = v + (bh * N + j) * d;
            double sij = 0.0, dpij = 0.0;
            for (int64_t c = 0; c < d; ++c) { sij += qi[c] * kj[c]; dpij += doi[c] * vj[c]; }
            const double pij = exp(scale * sij - lse[flat]);
            const double dsij = pij * (dpij - Dv[flat]);
            for (int64_t c = 0; c < d; ++c) out[c] += scale * dsij * kj[c];
        }
    }
    /* dV_j = sum_i P_ij dO_i,  dK_j = scale * sum_i dS_ij q_i */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nk; ++r) {
        const int64_t flat = krows ? krows[r] : r;
        const int64_t bh = flat / N, j = flat % N;
        const double* kj = k + flat * d;
        const double* vj = v + flat * d;
        double* odk = dk + r * d;
        double* odv = dv + r * d;
        for (int64_t c = 0; c < d; ++c) { odk[c] = 0.0; odv[c] = 0.0; }
        for (int64_t i = causal ? j : 0; i < N; ++i) {
            const int64_t fi = bh * N + i;
            const double* qi = q + fi * d;
            const double* doi = dout + fi * d;
            double sij = 0.0, dpij = 0.0;
            for (int64_t c = 0; c < d; ++c) { sij += qi[c] * kj[c]; dpij += doi[c] * vj[c]; }
            const double pij = exp(scale * sij - lse[fi]);
            const double dsij = pij * (dpij - Dv[fi]);
            for (int64_t c = 0; c < d; ++c) {
                odv[c] += pij * doi[c];
                odk[c] += scale * dsij * qi[c];
            }
        }
    }
    free(need);
    free(lse);
    free(Dv);
}

/* ---------------------------------------------------------------------------
 * OCP FP8 E4M3FN codec, written from the format definition:
 *   sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 *   exponent field 0 -> subnormal  (-1)^s * 2^-6 * m/8;
 *   exponent field 1..15 -> normal (-1)^s * 2^(e-7) * (1 + m/8);
 *   code 0x7F / 0xFF (e = 15, m = 7) is NaN; there is no infinity, so the
 *   largest finite magnitude is 2^8 * 1.75 = 448.
 * Encoding rounds to nearest, ties to even, and saturates finite values
 * beyond 448 to +-448 (the reading used for FP8 e4m3 in [FA3] sec. 技術 3).
 * ------------------------------------------------------------------------- */
static double e4m3_decode_one(uint8_t c) {
    const int sign = (c >> 7) & 1;
    const int e = (c >> 3) & 0xF;
    const int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static uint8_t e4m3_encode_one(double x) {
    if (isnan(x)) return 0x7F;
    const uint8_t sign = (signbit(x) ? 0x80 : 0x00);
    double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E; /* saturate (also +-inf) */
    /* Candidates are all non-negative finite codes 0x00..0x7E, whose values
     * increase with the code.  Find the largest code with value <= a, then
     * compare with its successor: nearest wins, ties go to the even code
     * (even mantissa LSB == even code). */
    int lo = 0;
    for (int c = 0; c <= 0x7E; ++c) {
        if (e4m3_decode_one((uint8_t)c) <= a) lo = c; else break;
    }
    if (lo == 0x7E) return sign | 0x7E;
    const double vlo = e4m3_decode_one((uint8_t)lo);
    const double vhi = e4m3_decode_one((uint8_t)(lo + 1));
    int pick;
    if (a - vlo < vhi - a) pick = lo;
    else if (a - vlo > vhi - a) pick = lo + 1;
    else pick = (lo % 2 == 0) ? lo : lo + 1;
    return sign | (uint8_t)pick;
}

void oracle_e4m3_encode(const double* x, int64_t n, uint8_t* codes) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) codes[i] = e4m3_encode_one(x[i]);
}

void oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode_one(codes[i]);
}

/* Sylvester Hadamard entry: H_d[i][j] = (-1)^popcount(i & j), d a power of 2. */
static double hadamard_entry(int64_t i, int64_t j) {
    return (__builtin_popcountll((unsigned long long)(i & j)) & 1) ? -1.0 : 1.0;
}

/*
 * Incoherent processing ([FA3] sec. 技術 3): each row x (length d) becomes
 * x_hat = (x * signs) H_d / sqrt(d), i.e. x_hat_j = sum_i x_i s_i H[i][j] / sqrt(d).
 * Dense O(d^2) matrix product on purpose (no fast transform here).
 */
void oracle_rotate_rows(const double* x, int64_t rows, int64_t d,
                        const int8_t* signs, double* out) {
    const double inv = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d; ++i)
                acc += x[r * d + i] * (double)signs[i] * hadamard_entry(i, j);
            out[r * d + j] = acc * inv;
        }
    }
}

/*
 * Block quantisation ([FA3] sec. 技術 3): x is [BH, N, d]; rows are grouped in
 * blocks of block_rows consecutive rows of one (b, h) (the last block of a
 * head may be short).  scale = amax(block) / 448 (1 when amax is 0), or with
 * pow2 != 0 the smallest power of two >= amax(block) / 448 (a reading: the
 * page fixes no scale format; a power of two lets hardware apply the scale
 * as an exponent); code = e4m3(x / scale).  scales: [BH, ceil(N / block_rows)].
 */
static double pow2_ceil(double t) {
    int e;
    const double m = frexp(t, &e);   /* t = m * 2^e, m in [0.5, 1) */
    return (m == 0.5) ? t : ldexp(1.0, e);
}

void oracle_quantize_blocks(const double* x, int64_t BH, int64_t N, int64_t d,
                            int64_t block_rows, int pow2, uint8_t* codes, double* scales) {
    const int64_t nblk = (N + block_rows - 1) / block_rows;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < BH * nblk; ++t) {
        const int64_t bh = t / nblk, blk = t % nblk;
        const int64_t r0 = blk * block_rows;
        const int64_t r1 = (r0 + block_rows < N) ? r0 + block_rows : N;
        double amax = 0.0;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = 0; c < d; ++c) {
                const double a = fabs(x[(bh * N + r) * d + c]);
                if (a > amax) amax = a;
            }
        double sc = (amax > 0.0) ? amax / 448.0 : 1.0;
        if (pow2 && amax > 0.0) sc = pow2_ceil(sc);
        scales[t] = sc;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = 0; c < d; ++c) {
                const int64_t idx = (bh * N + r) * d + c;
                codes[idx] = e4m3_encode_one(x[idx] / sc);
            }
    }
}
