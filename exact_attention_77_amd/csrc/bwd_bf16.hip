// bwd_bf16.hip -- bf16 backward pass of exact attention for gfx950.
//
// What is computed: the gradients, with respect to Q, K and V, of the
// attention of "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
// sec. 2.1 (causal mask of sec. 11.3).  With s = scale * Q K^T, P = softmax(s)
// row by row and the upstream gradient dO (the pages print no backward
// formulas; these are the analytic derivative of that definition):
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//     dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
// As sec. 7.2 of that page describes, nothing N x N is kept from the forward
// pass: S and P are recomputed tile by tile in on-chip memory from Q, K and
// the per-row statistic the forward stored (its natural-log LSE, so that
// P_ij = exp(s_ij - LSE_i)).
//
// Two kernels, both on the caller's stream, the dQ kernel first:
//  1. dQ   : (below) also forms, per query row, -D_i and LSE_i * log2(e) (fp32)
//            and stores them in the workspace for the dK/dV kernel.
//  2. dK/dV: one workgroup per (batch, head, 128-key tile), four waves of 32
//            keys each (one wave per SIMD); a wave keeps its keys' K and V rows
//            in registers and streams 64-query tiles of Q and dO (with their
//            statistics) through LDS by direct global->LDS loads
//            (double-buffered).  Per tile, with v_mfma_f32_32x32x16_bf16:
//              S = Q K^T and dP - D (the accumulator starts at -D); in the
//              32x32 accumulator layout a lane holds ONE key and 16 queries;
//              P = exp2(S * scale*log2e - LSE*log2e), dS = P (dP - D) -> bf16
//              are, thanks to the query order of the A operand, directly the
//              B operands of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by
//              transposing LDS reads) -- no exchange through LDS.
//  dQ kernel: one workgroup per (batch, head, 256-query tile), eight waves of
//            32 queries, K/V tiles of 128 keys (worked in 64-key blocks)
//            streamed through LDS (the loop order of the forward pass); each
//            query row belongs to exactly one lane pair, which forms D_i from
//            the row's dO (already in its
//            registers) and O.  Per tile the transposed products
//            S^T = K Q^T and dP^T - D = V dO^T (Q^T, dO^T held in registers)
//            put one query per lane, dS^T = P^T (dP^T - D) -> bf16 is, with K
//            rows fed in a permuted order, directly the B operand of
//            dQ^T += K^T dS^T, and dQ is written once at the end.  The dS^T of
//            a block's second 32-key subtile is formed beside the dQ products
//            of its first subtile.
// dQ is thus computed by recomputing S and dP per query tile instead of being
// summed over key tiles with atomic adds: 40% more matrix work, but the fp32
// atomics into a shared accumulator cost more than that on this chip (their
// throughput at the L2 is far below the matrix cores'), and the result is
// deterministic.  "FlashAttention-4" (abstract) likewise names the atomic
// adds of the backward pass as a cost to cut.
// Workgroups run the tiles with the most work first under the causal mask,
// and the tiles of one head share an XCD (ids are dealt round-robin over the
// 8 XCDs), so that head's K/V or Q/dO stream stays in one L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "lds_copy.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int BK = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int BQ = 64;   // queries per tile of the dK/dV inner loop (two 32-query subtiles)
constexpr float kLog2e = 1.4426950408889634f;

// XOR swizzle (16-byte chunk units) of a row of a Q, dO or K tile in LDS.  A
// tile is read two ways: by rows (16 lanes read one chunk of 16 rows) and
// transposed (ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x 64
// bytes).  Both patterns hit 16 distinct bank groups with this swizzle.
template <int D>
__device__ __forceinline__ int swz(int row) {
    return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Row of the A operand that lane row i loads: bits 2 and 3 swapped.  Then
// register g = 4r + t of lane half hh of the accumulator holds query
// 16 * (r >> 1) + 8 * hh + 4 * (r & 1) + t, so registers 8c .. 8c+7 hold
// queries 16c + 8hh .. 16c + 8hh + 7: the B-operand slice of k-step c.
__device__ __forceinline__ int perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Transposing LDS read: within each 16-lane group, destination lane 4p+q gets
// element q of the 8-byte pieces read by source lanes p, 4+p, 8+p, 12+p.
__device__ __forceinline__ short4_t lds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((__attribute__((address_space(3))) char*)(p)));
}

// XOR swizzle of a row of a wave's row slice (32 rows of D bf16): 16 lanes
// reading one chunk of 16 rows hit distinct bank groups.
template <int D>
__device__ __forceinline__ int rswz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// s_waitcnt immediate that waits for LDS (and scalar memory) operations only:
// vmcnt and expcnt at their maxima, lgkmcnt 0.
constexpr int kLgkm0 = 0xC07F;

__device__ __forceinline__ bf16x8 cat(short4_t lo, short4_t hi) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// dK/dV kernel: 4 waves of 32 keys (one wave per
// SIMD).  A wave keeps its keys' K and V rows in registers and, per 64-query
// tile of Q / dO (staged in LDS as above), computes S = Q K^T and dP - D for
// all 64 queries in two 32-query subtiles.  With the Q / dO rows fed in the
// bit-2/3-swapped order, the accumulator registers of subtile qs hold, for
// the lane's key, queries 32qs + 16c' + 8hh .. +7 in registers 8c' .. 8c'+7:
// after exp2 and the bf16 conversion they are directly the B operands of
// dV^T += dO^T P and dK^T += Q^T dS for the 16-query chunks 2qs + c' (A
// operands dO^T, Q^T by transposing LDS reads).  Nothing goes back through
// LDS, and each Q / dO row is read by the 4 waves of the workgroup.  The two
// accumulators (128 registers together at d = 128, in the accumulation
// registers) leave room for the operands only at one wave per SIMD.  The subtiles are pipelined so that the exp/dS work of
// one sits beside the products of the other.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int KS = D / 16;          // k-steps over the head dim
    constexpr int DT = D / 32;          // 32-column head-dim tiles
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int NWV = 4;              // waves: 32 keys each
    constexpr int QT_BYTES = BQ * D * 2;
    constexpr int NQB = QT_BYTES / 1024 / NWV;   // 1 KB copy blocks per wave, Q (and dO) tile
    static_assert(NQB >= 1 && BK == 32 * NWV, "tile shape");

    __shared__ __attribute__((aligned(1024))) char qtile0[QT_BYTES], qtile1[QT_BYTES];   // Q, 64 rows
    __shared__ __attribute__((aligned(1024))) char otile0[QT_BYTES], otile1[QT_BYTES];   // dO, 64 rows
    __shared__ __attribute__((aligned(16))) float stat0[2 * BQ], stat1[2 * BQ];          // LSE*log2e, -D
    // each wave's K and V rows in, its dV and dK rows out (two 32-row slices)
    constexpr int SL = 32 * D * 2;
    __shared__ __attribute__((aligned(1024))) char kvsl[NWV * 2 * SL];

    const int BH = a.B * a.H;
    const int n_kt = (a.N + BK - 1) / BK;
    const int kp = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int lo_kt = CAUSAL ? n_kt - 1 - kp : kp;
    const int n_tiles = (CAUSAL && kp < lo_kt) ? 2 : 1;
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {   // one copy of the tile code
        const int kt = r ? lo_kt : kp;
        const int b = bh / a.H, h = bh % a.H;
        const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
        const u16* Qg = static_cast<const u16*>(a.q) + base;
        const u16* Kg = static_cast<const u16*>(a.k) + base;
        const u16* Vg = static_cast<const u16*>(a.v) + base;
        const u16* Og = static_cast<const u16*>(a.dout) + base;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int j = lane & 31, hh = lane >> 5;
        const int k0 = kt * BK;
        const int kw0 = k0 + 32 * wave;               // first key of this wave
        const int key = kw0 + j;                      // this lane's key

        // K and V rows come in, dV and dK rows go out, through this wave's two
        // LDS slices, so that global memory sees whole rows (1 KB copies in;
        // 16 bytes of a row per lane out); only the registers hold the one-key-
        // per-lane layout.  A wave touches only its own slices: no barrier.
        // The slice addressing starts from an opaque copy of the lane index at
        // each use, so that nothing of it stays live across the main loop.
        char* const sk = kvsl + wave * 2 * SL;
        char* const sv = sk + SL;
        auto fresh_lane = [&]() {
            int l = lane;
            asm volatile("" : "+v"(l));
            return l;
        };
        auto copy_rows = [&](int kt_) {   // keys past the end copy the last row
            const int l = fresh_lane(), r0 = kt_ * BK + 32 * wave;
    #pragma unroll
            for (int i = 0; i < SL / 1024; ++i) {
                const int c = i * 64 + l, row = c / CPR, pch = c % CPR;
                const int64_t off = int64_t(min(r0 + row, a.N - 1)) * a.ss + 8 * (pch ^ rswz<D>(row));
                copy16_to_lds(Kg + off, sk + i * 1024);
                copy16_to_lds(Vg + off, sv + i * 1024);
            }
        };
        // B operands of S = Q K^T and dP = dO V^T: lane (key, half hh), k-step
        // ks holds columns 16ks + 8hh .. +7 of the key's K and V rows
        bf16x8 kreg[KS], vreg[KS];

        auto copy_q = [&](int q0, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
    #pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int blk = wave * NQB + i;
                const int c = blk * 64 + lane;
                const int row = c / CPR, pch = c % CPR;
                const int64_t roff = int64_t(min(q0 + row, a.N - 1)) * a.ss + 8 * (pch ^ swz<D>(row));
                copy16_to_lds(Qg + roff, (buf ? qtile1 : qtile0) + blk * 1024);
                copy16_to_lds(Og + roff, (buf ? otile1 : otile0) + blk * 1024);
            }
            float* st = buf ? stat1 : stat0;
            const int qq = min(q0 + lane, a.N - 1);
            if (wave == 0)       // LSE*log2e of the 64 queries
                copy4_to_lds(a.ws_lse2 + int64_t(bh) * a.N + qq, st);
            else if (wave == 1)  // -D
                copy4_to_lds(a.ws_nd + int64_t(bh) * a.N + qq, st + BQ);
        };

        // ---- per-lane LDS offsets (the swizzle of row 32qs + prow does not depend on qs)
        const int prow = perm_row(j);
        const int tr_row = 8 * hh + ((lane >> 2) & 3);                 // + 16 c  (+4 for the second read)
        const int tr_lch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // + 4 dt
        const int tr_half = 8 * (lane & 1);
        int qo[KS];
    #pragma unroll
        for (int ks = 0; ks < KS; ++ks) qo[ks] = prow * (2 * D) + 16 * ((2 * ks + hh) ^ swz<D>(prow));
        int tro[DT][2];
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int rr = tr_row + 4 * e;
                tro[dt][e] = rr * (2 * D) + tr_half + 16 * ((4 * dt + tr_lch) ^ swz<D>(rr));
            }
        auto ld16 = [](const char* t, int off) { return *reinterpret_cast<const bf16x8*>(t + off); };
        auto ldtr = [](const char* t, int lo, int hi) { return cat(lds_read_tr(t + lo), lds_read_tr(t + hi)); };

        // dV^T and dK^T of this wave's 32 keys.  Started by a product of zeros,
        // so that they live in the accumulation registers from the start (zero
        // vector registers here would make the allocator copy all 128 values
        // into them before every tile's products).
        f32x16 accv[DT], acck[DT];
        {
            const bf16x8 z = {};
            const f32x16 z16 = {};
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                accv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, z16, 0, 0, 0);
                acck[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, z16, 0, 0, 0);
            }
        }

        const float c2 = a.scale_log2;
        const int n_qt = (a.N + BQ - 1) / BQ;
        const int qt0 = CAUSAL ? k0 / BQ : 0;

        // One 64-query tile `it` from buffer `buf`.
        auto tile = [&](int it, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            const char* qt = buf ? qtile1 : qtile0;
            const char* ot = buf ? otile1 : otile0;
            const float* ls = buf ? stat1 : stat0;
            const int q0 = it * BQ;
            // S and dP - D of subtile qs: 2*KS products alternating, LDS
            // operands read two ahead (the first two, `pre`, during the
            // previous phase: `prefetch()` reads the next phase's two beside
            // this phase's second-last product); `beside(m)` is issued after
            // product m
            auto sdp_src = [&](int qs, int m) { return ld16((m & 1) ? ot : qt, 32 * qs * 2 * D + qo[m >> 1]); };
            auto sdp = [&](int qs, f32x16& sc, f32x16& dp, const bf16x8 (&pre)[2], auto&& beside, auto&& prefetch) {
    #pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float4 nd = *reinterpret_cast<const float4*>(ls + BQ + 32 * qs + 16 * (rr >> 1) + 8 * hh + 4 * (rr & 1));
                    dp[4 * rr + 0] = nd.x; dp[4 * rr + 1] = nd.y; dp[4 * rr + 2] = nd.z; dp[4 * rr + 3] = nd.w;
                }
    #pragma unroll
                for (int g = 0; g < 16; ++g) sc[g] = 0.f;
                auto src = [&](int m) { return sdp_src(qs, m); };
                bf16x8 op[3];
                op[0] = pre[0];
                op[1] = pre[1];
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int m = 0; m < 2 * KS; ++m) {
                    if (m + 2 < 2 * KS) op[(m + 2) % 3] = src(m + 2);
                    if (m == 2 * KS - 2) prefetch();
                    if (m & 1)
                        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m % 3], vreg[m >> 1], dp, 0, 0, 0);
                    else
                        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m % 3], kreg[m >> 1], sc, 0, 0, 0);
                    beside(m);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // masked (query, key) pairs of subtile qs get score -inf, hence P = 0
            auto mask = [&](int qs, f32x16& sc) {
                const int q0s = q0 + 32 * qs;
                const bool edge = (CAUSAL && q0s < kw0 + 31) || q0s + 32 > a.N || kw0 + 32 > a.N;
                if (edge) {   // wave-uniform: diagonal or ragged blocks only
                    const int lo = CAUSAL ? key - q0s - 8 * hh : -(1 << 30);
                    const int hi = key < a.N ? a.N - 1 - q0s - 8 * hh : -1;
    #pragma unroll
                    for (int g = 0; g < 16; ++g) {
                        const int rr = g >> 2, t = g & 3;
                        const int off = 16 * (rr >> 1) + 4 * (rr & 1) + t;
                        if (off < lo || off > hi) sc[g] = -INFINITY;
                    }
                }
            };
            // P = exp2(S c - LSE log2 e) and dS = P (dP - D) as bf16 for
            // registers g0 .. g1-1 of subtile qs
            bf16x8 pb[2][2], dsb[2][2];
            float l2v[2][16];
    #pragma unroll
            for (int qs = 0; qs < 2; ++qs)
    #pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float4 v4 = *reinterpret_cast<const float4*>(ls + 32 * qs + 16 * (rr >> 1) + 8 * hh + 4 * (rr & 1));
                    l2v[qs][4 * rr + 0] = v4.x; l2v[qs][4 * rr + 1] = v4.y; l2v[qs][4 * rr + 2] = v4.z; l2v[qs][4 * rr + 3] = v4.w;
                }
            auto softmax = [&](int qs, const f32x16& sc, const f32x16& dp, int g0, int g1) {
    #pragma unroll
                for (int g = g0; g < g1; ++g) {
                    const float l2 = l2v[qs][g];
                    const float pg = __builtin_amdgcn_exp2f(fmaf(sc[g], c2, -l2));
                    pb[qs][g >> 3][g & 7] = static_cast<__bf16>(pg);
                    dsb[qs][g >> 3][g & 7] = static_cast<__bf16>(pg * dp[g]);
                }
            };
            // dV^T and dK^T products of 16-query chunks c0, c0 + 1 (subtile
            // c0 / 2): 4*DT products, A operands read two ahead
            auto dvdk_src = [&](int c0, int n) {   // n: chunk c0 + (n / (2 DT)), tile dt, dO^T or Q^T
                const int c = c0 + n / (2 * DT), dt = (n >> 1) % DT;
                return ldtr((n & 1) ? qt : ot, 32 * D * c + tro[dt][0], 32 * D * c + tro[dt][1]);
            };
            auto dvdk = [&](int c0, const bf16x8 (&pre)[2], auto&& beside, auto&& prefetch) {
                constexpr int NP = 4 * DT;
                auto asrc = [&](int n) { return dvdk_src(c0, n); };
                bf16x8 op[3];
                op[0] = pre[0];
                op[1] = pre[1];
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int n = 0; n < NP; ++n) {
                    if (n + 2 < NP) op[(n + 2) % 3] = asrc(n + 2);
                    if (n == NP - 2) prefetch();
                    const int c = c0 + n / (2 * DT), dt = (n >> 1) % DT;
                    if (n & 1)
                        acck[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n % 3], dsb[c >> 1][c & 1], acck[dt], 0, 0, 0);
                    else
                        accv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n % 3], pb[c >> 1][c & 1], accv[dt], 0, 0, 0);
                    beside(n);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            f32x16 s0, dp0, s1, dp1;
            bf16x8 preA[2], preB[2];
            preA[0] = sdp_src(0, 0);
            preA[1] = sdp_src(0, 1);
            sdp(0, s0, dp0, preA, [](int) {}, [&]() { preB[0] = sdp_src(1, 0); preB[1] = sdp_src(1, 1); });
            mask(0, s0);
            constexpr int G1 = 16 / (2 * KS);   // subtile-0 registers beside each S/dP product of subtile 1
            sdp(1, s1, dp1, preB, [&](int m) { softmax(0, s0, dp0, G1 * m, G1 * (m + 1)); },
                [&]() { preA[0] = dvdk_src(0, 0); preA[1] = dvdk_src(0, 1); });
            mask(1, s1);
            constexpr int G2 = 16 / (4 * DT);   // subtile-1 registers beside each dV/dK product of subtile 0
            dvdk(0, preA, [&](int n) { softmax(1, s1, dp1, G2 * n, G2 * (n + 1)); },
                 [&]() { preB[0] = dvdk_src(2, 0); preB[1] = dvdk_src(2, 1); });
            dvdk(2, preB, [](int) {}, []() {});
        };

        // The first tile's loads are issued here; the second tile's by the
        // first one's end (below).
        if (r == 0) {
            copy_rows(kt);
            if (qt0 < n_qt) copy_q(qt0 * BQ, std::integral_constant<int, 0>{});
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's K and V rows have landed
        {
            const int l = fresh_lane(), jj = l & 31, h2 = l >> 5;
    #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = jj * (2 * D) + 16 * ((2 * ks + h2) ^ rswz<D>(jj));
                kreg[ks] = *reinterpret_cast<const bf16x8*>(sk + off);
                vreg[ks] = *reinterpret_cast<const bf16x8*>(sv + off);
            }
        }
        auto step = [&](int it, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();   // tile it is in LDS; every wave is done with tile it - 1
            if (it + 1 < n_qt) copy_q((it + 1) * BQ, std::integral_constant<int, buf ^ 1>{});
            tile(it, bufc);
        };
        for (int it = qt0; it < n_qt; it += 2) {
            step(it, std::integral_constant<int, 0>{});
            if (it + 1 < n_qt) step(it + 1, std::integral_constant<int, 1>{});
        }

        // ---- handover: the second tile's first Q/dO tile goes out now --------
        const bool hand = r + 1 < n_tiles;
        if (hand) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_s_barrier();   // every wave is done with the Q/dO tiles
            const int qt0n = CAUSAL ? (lo_kt * BK) / BQ : 0;
            if (qt0n < n_qt) copy_q(qt0n * BQ, std::integral_constant<int, 0>{});
        }

        // ---- epilogue: dV and dK = scale * (dK^T)^T, bf16, via the slices ------
        // register g of lane half hh: column 32dt + 8(g>>2) + 4hh + (g&3) of the
        // lane's key, i.e. chunk 4dt + (g>>2), half hh of its row
        const int le = fresh_lane();
        {
            const int jj = le & 31, h2 = le >> 5;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    __bf16 v4[4], k4[4];
    #pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v4[t] = static_cast<__bf16>(accv[dt][4 * rr + t]);
                        k4[t] = static_cast<__bf16>(acck[dt][4 * rr + t] * a.scale);
                    }
                    const int off = jj * (2 * D) + 16 * ((4 * dt + rr) ^ rswz<D>(jj)) + 8 * h2;
                    *reinterpret_cast<uint2*>(sv + off) = __builtin_bit_cast(uint2, v4);
                    *reinterpret_cast<uint2*>(sk + off) = __builtin_bit_cast(uint2, k4);
                }
        }
        {
            constexpr int RPI = 64 / CPR;   // rows per 16-byte-per-lane access
            u16* const dvw = static_cast<u16*>(a.dv) + base + int64_t(kw0) * a.ss;
            u16* const dkw = static_cast<u16*>(a.dk) + base + int64_t(kw0) * a.ss;
    #pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int row = RPI * i + le / CPR, pch = le % CPR;
                const uint4 v = *reinterpret_cast<const uint4*>(sv + row * (2 * D) + 16 * pch);
                const uint4 k = *reinterpret_cast<const uint4*>(sk + row * (2 * D) + 16 * pch);
                if (kw0 + row < a.N) {
                    const int64_t off = int64_t(row) * a.ss + 8 * (pch ^ rswz<D>(row));
                    *reinterpret_cast<uint4*>(dvw + off) = v;
                    *reinterpret_cast<uint4*>(dkw + off) = k;
                }
            }
        }
        if (hand) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);   // this wave's rows are out of its slices
            copy_rows(lo_kt);
        }
    }
}

// ---------------------------------------------------------------------------
// dQ kernel: NW waves of 32 queries, BC-key K/V tiles double-buffered
// (processed in 64-key blocks).
template <int D, bool CAUSAL, int NW, int BC>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdArgs a) {
    constexpr int BR = 32 * NW;
    static_assert(BC % 64 == 0, "key tile");
    constexpr int KS = D / 16, DT = D / 32, CPR = D / 8;
    constexpr int TB = BC * D * 2;              // one K or V tile
    constexpr int NI = TB / 1024 / NW;          // 1 KB copy blocks per wave per tile
    static_assert(NI >= 1, "tile shape");
    __shared__ __attribute__((aligned(1024))) char ktile0[TB], ktile1[TB], vtile0[TB], vtile1[TB];

    // ---- work decomposition: one head per XCD; under the causal mask a
    // workgroup takes the query-tile pair (T-1-p, p), equal work for all ----
    const int n_qt = (a.N + BR - 1) / BR;
    const int per_head = CAUSAL ? (n_qt + 1) / 2 : n_qt;
    const int total = per_head * a.B * a.H;
    int id = blockIdx.x;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        id = (id & 7) * per + (id >> 3);
    }
    const int bh = id / per_head, p = id % per_head;
    const int hi = CAUSAL ? n_qt - 1 - p : p;
    const int n_tiles = (CAUSAL && p < hi) ? 2 : 1;
    static_assert(NW * 32 * D * 2 <= 2 * TB, "dQ rows of all waves fit in one K/V buffer pair");
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {   // one copy of the tile code
        const int qt = r ? p : hi;
        const int b = bh / a.H, h = bh % a.H;
        const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
        const u16* Qg = static_cast<const u16*>(a.q) + base;
        const u16* Kg = static_cast<const u16*>(a.k) + base;
        const u16* Vg = static_cast<const u16*>(a.v) + base;
        const u16* Og = static_cast<const u16*>(a.dout) + base;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int j = lane & 31, hh = lane >> 5;
        const int q0 = qt * BR + 32 * wave;         // first query of this wave
        const int qi = q0 + j;                      // this lane's query
        const int n_kt = (a.N + BC - 1) / BC;
        const int nt = CAUSAL ? min(n_kt, (min(a.N, (qt + 1) * BR) + BC - 1) / BC) : n_kt;
        int wnt = CAUSAL ? min(nt, (min(a.N, q0 + 32) + BC - 1) / BC) : nt;
        if (q0 >= a.N) wnt = 0;

        // ---- K/V tile copy (direct to LDS, swizzled rows; rows past the end
        // re-read the last row, their scores are masked) ---------------------------
        auto copy_kv = [&](int kt, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
    #pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int blk = wave * NI + i;
                const int c = blk * 64 + lane;
                const int row = c / CPR, pch = c % CPR;
                const int64_t off = int64_t(min(kt * BC + row, a.N - 1)) * a.ss + 8 * (pch ^ swz<D>(row));
                copy16_to_lds(Kg + off, (buf ? ktile1 : ktile0) + blk * 1024);
                copy16_to_lds(Vg + off, (buf ? vtile1 : vtile0) + blk * 1024);
            }
        };

        // ---- per-query operands and statistics (zero past the end) --------------
        bf16x8 qreg[KS], oreg[KS];   // B operands of K Q^T / V dO^T: lane (query, half hh)
    #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 xq = make_uint4(0, 0, 0, 0), xo = make_uint4(0, 0, 0, 0);
            if (qi < a.N) {
                const int64_t off = int64_t(qi) * a.ss + 16 * ks + 8 * hh;
                xq = *reinterpret_cast<const uint4*>(Qg + off);
                xo = *reinterpret_cast<const uint4*>(Og + off);
            }
            qreg[ks] = __builtin_bit_cast(bf16x8, xq);
            oreg[ks] = __builtin_bit_cast(bf16x8, xo);
        }
        // -D_i = -sum_c dO_ic O_ic (O as the forward stored it) and LSE_i log2(e):
        // lane half hh holds half of the row's columns of dO, so it sums the
        // products of that half and adds its partner lane's (l ^ 32) sum.
        // Stored for the dK/dV kernel, which runs after this one.
        float dpart = 0.f;
        if (qi < a.N) {
            const u16* Orow = static_cast<const u16*>(a.o) + base + int64_t(qi) * a.ss;
    #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 o8 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Orow + 16 * ks + 8 * hh));
    #pragma unroll
                for (int e = 0; e < 8; ++e) dpart = fmaf(static_cast<float>(o8[e]), static_cast<float>(oreg[ks][e]), dpart);
            }
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart), __float_as_uint(dpart), false, false);
        const float nd = -(__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
        const float lse2 = qi < a.N ? a.lse[int64_t(bh) * a.N + qi] * kLog2e : 0.f;
        if (qi < a.N && hh == 0) {
            a.ws_nd[int64_t(bh) * a.N + qi] = nd;
            a.ws_lse2[int64_t(bh) * a.N + qi] = lse2;
        }

        // ---- per-lane LDS offsets ----------------------------------------------
        const int prow = perm_row(j);                                  // K / V row operand (+32 st)
        const int tr_row = 8 * hh + ((lane >> 2) & 3);                 // + 16 c  (+4 for the second read)
        const int tr_lch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // + 4 dt
        const int tr_half = 8 * (lane & 1);
        int ro[KS];
    #pragma unroll
        for (int ks = 0; ks < KS; ++ks) ro[ks] = prow * (2 * D) + 16 * ((2 * ks + hh) ^ swz<D>(prow));
        int tro[DT][2];
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = tr_row + 4 * e;
                tro[dt][e] = r * (2 * D) + tr_half + 16 * ((4 * dt + tr_lch) ^ swz<D>(r));
            }
        auto ld16 = [](const char* t, int off) { return *reinterpret_cast<const bf16x8*>(t + off); };
        auto ldtr = [](const char* t, int lo, int hi) { return cat(lds_read_tr(t + lo), lds_read_tr(t + hi)); };

        f32x16 acc[DT];   // dQ^T: register g of lane half hh holds column 32dt + 8(g>>2) + 4hh + (g&3)
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int g = 0; g < 16; ++g) acc[dt][g] = 0.f;
        const float c2 = a.scale_log2;

        // One key tile, in 64-key blocks: per 32-key subtile st, S^T and dP^T - D,
        // then P^T and dS^T; register g = 4r + t of lane half hh holds key
        // 32st + 16(r>>1) + 8hh + 4(r&1) + t of the block, so the bf16 dS^T
        // registers are the B operand of the block's 16-key chunk c = 2st + (r>>1).
        auto compute = [&](int kt, const char* kt_lds, const char* vt_lds) __attribute__((always_inline)) {
    #pragma unroll
            for (int kb = 0; kb < BC / 64; ++kb) {
                const int k_lo = kt * BC + 64 * kb;
                if (CAUSAL && kb > 0 && k_lo > q0 + 31) continue;   // wave-uniform: block fully masked
                const bool edge = (k_lo + 64 > a.N) || (CAUSAL && k_lo + 63 > q0);
                const int lim = (CAUSAL ? min(qi, a.N - 1) : a.N - 1) - k_lo - 8 * hh;
                const char* kb_lds = kt_lds + 64 * kb * 2 * D;
                const char* vb_lds = vt_lds + 64 * kb * 2 * D;
                bf16x8 dsb[2][2];
                // S^T and dP^T - D of subtile st (2*KS products alternating;
                // LDS operands read two ahead), with the masked keys' scores
                // set to -inf on diagonal and ragged blocks
                auto scores = [&](int st, f32x16& s, f32x16& dp) {
    #pragma unroll
                    for (int g = 0; g < 16; ++g) { s[g] = 0.f; dp[g] = nd; }
                    auto src = [&](int m) {
                        return ld16((m & 1) ? vb_lds : kb_lds, 32 * st * 2 * D + ro[m >> 1]);
                    };
                    bf16x8 op[3];
                    op[0] = src(0);
                    op[1] = src(1);
    #pragma unroll
                    for (int m = 0; m < 2 * KS; ++m) {
                        if (m + 2 < 2 * KS) op[(m + 2) % 3] = src(m + 2);
                        if (m & 1)
                            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m % 3], oreg[m >> 1], dp, 0, 0, 0);
                        else
                            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m % 3], qreg[m >> 1], s, 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (edge) {
    #pragma unroll
                        for (int g = 0; g < 16; ++g) {
                            const int r = g >> 2, t = g & 3;
                            if (32 * st + 16 * (r >> 1) + 4 * (r & 1) + t > lim) s[g] = -INFINITY;
                        }
                    }
                };
                // dS^T = P^T (dP^T - D) for registers g0 .. g1-1 of subtile st, as bf16
                auto ds_part = [&](int st, const f32x16& s, const f32x16& dp, int g0, int g1) {
    #pragma unroll
                    for (int g = g0; g < g1; ++g)
                        dsb[st][g >> 3][g & 7] =
                            static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[g], c2, -lse2)) * dp[g]);
                };
                {
                    f32x16 s, dp;
                    scores(0, s, dp);
                    ds_part(0, s, dp, 0, 16);
                }
                // dQ^T += K^T dS^T over the block's four 16-key chunks (operands
                // two ahead); chunks 0 and 1 need subtile 0 only, so subtile 1's
                // dS^T is formed beside their products
                f32x16 s1, dp1;
                scores(1, s1, dp1);
                constexpr int NQ = 4 * DT;
                constexpr int G = 16 / (2 * DT);   // subtile-1 registers per early product
                auto tsrc = [&](int n) {
                    const int c = n / DT, dt = n % DT;
                    return ldtr(kb_lds, 16 * c * 2 * D + tro[dt][0], 16 * c * 2 * D + tro[dt][1]);
                };
                bf16x8 top[3];
                top[0] = tsrc(0);
                top[1] = tsrc(1);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int n = 0; n < NQ; ++n) {
                    if (n + 2 < NQ) top[(n + 2) % 3] = tsrc(n + 2);
                    const int c = n / DT, dt = n % DT;
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[n % 3], dsb[c >> 1][c & 1], acc[dt], 0, 0, 0);
                    if (n < 2 * DT) ds_part(1, s1, dp1, G * n, G * (n + 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        // the first tile's first K/V tile; the second tile's is issued by the
        // first one's end (below)
        if (r == 0 && nt > 0) copy_kv(0, std::integral_constant<int, 0>{});
        auto step = [&](int kt, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();   // tile kt is in LDS; everyone is done with tile kt - 1
            if (kt + 1 < nt) copy_kv(kt + 1, std::integral_constant<int, buf ^ 1>{});
            if (kt < wnt) compute(kt, buf ? ktile1 : ktile0, buf ? vtile1 : vtile0);
        };
        for (int kt = 0; kt < nt; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            if (kt + 1 < nt) step(kt + 1, std::integral_constant<int, 1>{});
        }

        // ---- end of tile: every wave is done with the K/V buffers; the second
        // tile's first K/V tile goes out at once (into buffer 0) ----------------
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        if (r + 1 < n_tiles) {
            const int nt2 = CAUSAL ? min(n_kt, (min(a.N, (p + 1) * BR) + BC - 1) / BC) : n_kt;
            if (nt2 > 0) copy_kv(0, std::integral_constant<int, 0>{});
        }

        // ---- epilogue: dQ = scale * (dQ^T)^T, bf16, through buffer 1 ------------
        // Wave w owns 32 rows of buffer 1 (waves 0-3 in the K half, 4-7 in the V
        // half): dQ^T goes in as the lane's row (chunk 4dt + r4, half hh), the
        // rows come out 16 bytes per lane, so that global memory sees whole rows.
        // The next tile's first step copies into buffer 1 only after its
        // barrier, which every wave reaches after reading its rows back.
        {
            constexpr int SL = 32 * D * 2, RPI = 64 / CPR;
            char* const os = ((wave < NW / 2) ? ktile1 : vtile1) + (wave % (NW / 2)) * SL;
            int le = lane;
            asm volatile("" : "+v"(le));
            const int jj = le & 31, h2 = le >> 5;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    __bf16 x4[4];
    #pragma unroll
                    for (int t = 0; t < 4; ++t) x4[t] = static_cast<__bf16>(acc[dt][4 * r4 + t] * a.scale);
                    *reinterpret_cast<uint2*>(os + jj * (2 * D) + 16 * ((4 * dt + r4) ^ rswz<D>(jj)) + 8 * h2) =
                        __builtin_bit_cast(uint2, x4);
                }
            u16* const dqw = static_cast<u16*>(a.dq) + base + int64_t(q0) * a.ss;
    #pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int row = RPI * i + le / CPR, pch = le % CPR;
                const uint4 v = *reinterpret_cast<const uint4*>(os + row * (2 * D) + 16 * pch);
                if (q0 + row < a.N)
                    *reinterpret_cast<uint4*>(dqw + int64_t(row) * a.ss + 8 * (pch ^ rswz<D>(row))) = v;
            }
        }
    }
}

template <int D>
int run(const BwdArgs& a, hipStream_t s) {
    // the dQ kernel first: it also writes the per-row statistics the dK/dV
    // kernel reads
    constexpr int NW = 8, BC = 128;   // dQ kernel: 256 queries per workgroup, 128-key tiles
    const int n_qt = (a.N + 32 * NW - 1) / (32 * NW);
    const unsigned g_q = static_cast<unsigned>(int64_t(a.causal ? (n_qt + 1) / 2 : n_qt) * a.B * a.H);
    if (a.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, NW, BC>), dim3(g_q), dim3(64 * NW), 0, s, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, false, NW, BC>), dim3(g_q), dim3(64 * NW), 0, s, a);
    int err = static_cast<int>(hipGetLastError());
    if (err) return err;
    const int n_kt = (a.N + BK - 1) / BK;
    const unsigned g_kv = static_cast<unsigned>(int64_t(a.causal ? (n_kt + 1) / 2 : n_kt) * a.B * a.H);
    if (a.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(g_kv), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(g_kv), dim3(256), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_bwd_bf16(const BwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.D == 64 ? run<64>(a, s) : run<128>(a, s);
}

}  // namespace fa
