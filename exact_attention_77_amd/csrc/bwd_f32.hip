// bwd_f32.hip -- fp32 backward pass of exact attention for gfx950 on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32).
//
// What is computed: the gradients, with respect to Q, K and V, of the
// attention of "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
// sec. 2.1 (causal mask of sec. 11.3); the pages print no backward formulas,
// these are the analytic derivative of that definition (s = scale Q K^T,
// P = softmax(s) per row, P_ij = exp(s_ij - LSE_i)):
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//     dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
// As sec. 7.2 of that page describes, S and P are recomputed tile by tile on
// chip from Q, K and the forward's LSE; every product and sum is fp32.
//
// The two kernels of the bf16 backward, on the fp32 product: an fp32 product
// takes one value per lane for each operand, so (as in the fp32 forward) the
// contraction over the head dimension pairs columns 8 (s / 4) + 4 h + s % 4
// in k-step s of lane half h -- one 16-byte LDS read of a row feeds four
// products -- and every register of a score accumulator is directly the B
// operand of the next product for the pair of rows it holds, with the
// matching rows of the other operand read 32 consecutive floats per lane half.
//  1. dQ   : one workgroup per (batch, head, query tile), waves of 32 queries
//            (one query per lane), 32-key K/V tiles through LDS:
//            S^T = K Q^T and dP^T - D = V dO^T with Q^T, dO^T in registers,
//            dS^T = P^T o (dP^T - D), dQ^T += K^T dS^T.  It also forms, per
//            query row, -D_i and LSE_i * log2(e) and stores them in the
//            workspace for the second kernel.
//  2. dK/dV: one workgroup per (batch, head, 128-key tile), four waves of 32
//            keys (one key per lane, one wave per SIMD: the two 32 x d
//            accumulators live in the accumulation registers), 32-query tiles
//            of Q, dO and their statistics through LDS:
//            S = Q K^T and dP - D = dO V^T with K^T, V^T in registers,
//            P, dS, then dV^T += dO^T P and dK^T += Q^T dS.
// dQ is recomputed per query tile instead of summed over key tiles with
// atomic adds (their throughput at the L2 is far below the matrix cores'),
// and the result is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "lds_copy.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BT = 32;    // rows per LDS tile: keys (dQ kernel) or queries (dK/dV kernel)
constexpr int BK = 128;   // keys per dK/dV workgroup (four waves of 32)
constexpr float kLog2e = 1.4426950408889634f;

// A tile of BT rows of D floats in LDS.  Rows are read two ways: 32 lanes read
// one 16-byte chunk of 32 different rows (the contraction over the head
// dimension), and 32 lanes read 32 consecutive floats of one row (the second
// product).  The physical chunk is the logical one XOR the row, so that both
// spread over the banks.
template <int D>
struct RowTile {
    static constexpr int CPR = D / 4;          // 16-byte chunks per row
    static constexpr int BYTES = BT * D * 4;
    __device__ static int swz(int row) { return row & (CPR - 1); }
    __device__ static int chunk_off(int row, int c) { return row * (D * 4) + 16 * (c ^ swz(row)); }
    __device__ static int float_off(int row, int col) {
        return row * (D * 4) + 16 * ((col >> 2) ^ swz(row)) + 4 * (col & 3);
    }
};

__device__ __forceinline__ float pair_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows r0 .. r0 + BT - 1 of a [N, D] tensor (row stride ss floats) into an LDS
// tile by direct copies; wave `wave` of nw copies its share of the 1 KB
// blocks.  Rows past the end re-read the last row (callers mask them).
template <int D>
__device__ __forceinline__ void copy_rows(const float* src, int64_t ss, int r0, int n, char* dst, int wave,
                                          int nw, int lane) {
    using TL = RowTile<D>;
    for (int blk = wave; blk < TL::BYTES / 1024; blk += nw) {
        const int c = blk * 64 + lane;
        const int row = c / TL::CPR, pch = c % TL::CPR;
        const float* g = src + int64_t(min(r0 + row, n - 1)) * ss + 4 * (pch ^ TL::swz(row));
        copy16_to_lds(g, dst + blk * 1024);
    }
}

// ---------------------------------------------------------------------------
// dQ kernel (and the per-row statistics)
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1)))
void bwd_f32_dq_kernel(BwdArgs a) {
    static_assert(D == 64 || NW == 4, "d = 128 needs one wave per SIMD");
    using TL = RowTile<D>;
    constexpr int BR = NW * 32;   // queries per workgroup
    constexpr int DT = D / 32;    // head-dim tiles of dQ^T
    constexpr int KU = D / 8;     // 16-byte reads per contraction (four k-steps each)
    __shared__ __attribute__((aligned(1024))) char kt0[TL::BYTES], kt1[TL::BYTES];
    __shared__ __attribute__((aligned(1024))) char vt0[TL::BYTES], vt1[TL::BYTES];

    const int n_qt = (a.N + BR - 1) / BR;
    const int per_head = CAUSAL ? (n_qt + 1) / 2 : n_qt;
    const int total = per_head * a.B * a.H;
    int id = blockIdx.x;
    if ((total & 7) == 0) {   // one head per XCD (ids are dealt round-robin over 8 XCDs)
        const int per = total >> 3;
        id = (id & 7) * per + (id >> 3);
    }
    const int bh = id / per_head, p = id % per_head;
    const int hi = CAUSAL ? n_qt - 1 - p : p;
    const int n_tiles = (CAUSAL && p < hi) ? 2 : 1;   // causal: the pair (T-1-p, p)
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {
        if (r) __syncthreads();   // every wave is done with the first tile's LDS
        const int qt = r ? p : hi;
        const int b = bh / a.H, h = bh % a.H;
        const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
        const float* Qg = static_cast<const float*>(a.q) + base;
        const float* Kg = static_cast<const float*>(a.k) + base;
        const float* Vg = static_cast<const float*>(a.v) + base;
        const float* Og = static_cast<const float*>(a.dout) + base;
        const float* Fo = static_cast<const float*>(a.o) + base;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int j = lane & 31, hh = lane >> 5;
        const int q0 = qt * BR + 32 * wave;
        const int qi = q0 + j;
        const int n_kt = (a.N + BT - 1) / BT;
        const int nt = CAUSAL ? min(n_kt, (min(a.N, (qt + 1) * BR) + BT - 1) / BT) : n_kt;
        int wnt = CAUSAL ? min(nt, (min(a.N, q0 + 32) + BT - 1) / BT) : nt;
        if (q0 >= a.N) wnt = 0;

        // B operands: qreg[4u + i] = Q[qi][8u + 4hh + i], oreg likewise for dO;
        // the lane's half of D_i = sum_c dO_ic O_ic from the same columns
        float qreg[D / 2], oreg[D / 2];
        float dpart = 0.f;
    #pragma unroll
        for (int u = 0; u < KU; ++u) {
            float4 xq = make_float4(0.f, 0.f, 0.f, 0.f), xo = xq, xf = xq;
            if (qi < a.N) {
                const int64_t off = int64_t(qi) * a.ss + 8 * u + 4 * hh;
                xq = *reinterpret_cast<const float4*>(Qg + off);
                xo = *reinterpret_cast<const float4*>(Og + off);
                xf = *reinterpret_cast<const float4*>(Fo + off);
            }
            qreg[4 * u + 0] = xq.x; qreg[4 * u + 1] = xq.y; qreg[4 * u + 2] = xq.z; qreg[4 * u + 3] = xq.w;
            oreg[4 * u + 0] = xo.x; oreg[4 * u + 1] = xo.y; oreg[4 * u + 2] = xo.z; oreg[4 * u + 3] = xo.w;
            dpart = fmaf(xf.x, xo.x, dpart);
            dpart = fmaf(xf.y, xo.y, dpart);
            dpart = fmaf(xf.z, xo.z, dpart);
            dpart = fmaf(xf.w, xo.w, dpart);
        }
        const float nd = -pair_sum32(dpart);
        const float lse2 = qi < a.N ? a.lse[int64_t(bh) * a.N + qi] * kLog2e : 0.f;
        if (qi < a.N && hh == 0) {
            a.ws_nd[int64_t(bh) * a.N + qi] = nd;
            a.ws_lse2[int64_t(bh) * a.N + qi] = lse2;
        }

        f32x16 acc[DT];   // dQ^T: register g of lane half hh is column 32dt + 8(g>>2) + 4hh + (g&3)
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int g = 0; g < 16; ++g) acc[dt][g] = 0.f;
        const float c2 = a.scale_log2;

        // One 32-key tile: register g of lane half hh is key k0 + 8(g>>2) + 4hh + (g&3)
        auto compute = [&](int kt, const char* kl, const char* vl) {
            f32x16 s, dp;
    #pragma unroll
            for (int g = 0; g < 16; ++g) { s[g] = 0.f; dp[g] = nd; }
            // the chunks of read u + 1 are issued before the products of read u
            float4 kn = *reinterpret_cast<const float4*>(kl + TL::chunk_off(j, hh));
            float4 vn = *reinterpret_cast<const float4*>(vl + TL::chunk_off(j, hh));
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int u = 0; u < KU; ++u) {
                const float4 kx = kn, vx = vn;
                if (u + 1 < KU) {
                    kn = *reinterpret_cast<const float4*>(kl + TL::chunk_off(j, 2 * u + 2 + hh));
                    vn = *reinterpret_cast<const float4*>(vl + TL::chunk_off(j, 2 * u + 2 + hh));
                }
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qreg[4 * u + 0], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vx.x, oreg[4 * u + 0], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qreg[4 * u + 1], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vx.y, oreg[4 * u + 1], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qreg[4 * u + 2], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vx.z, oreg[4 * u + 2], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qreg[4 * u + 3], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vx.w, oreg[4 * u + 3], dp, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int k0 = kt * BT;
            if ((k0 + BT > a.N) || (CAUSAL && k0 + BT - 1 > q0)) {   // wave-uniform
                const int lim = (CAUSAL ? min(qi, a.N - 1) : a.N - 1) - k0 - 4 * hh;
    #pragma unroll
                for (int g = 0; g < 16; ++g)
                    if (8 * (g >> 2) + (g & 3) > lim) s[g] = -INFINITY;
            }
            // dS^T = P^T o (dP^T - D), in place of the scores
    #pragma unroll
            for (int g = 0; g < 16; ++g) s[g] = __builtin_amdgcn_exp2f(fmaf(s[g], c2, -lse2)) * dp[g];
            // dQ^T += K^T dS^T: product n takes the key pair of register n / DT
            // (head-dim tile n % DT); its K^T operand is read PF products ahead
            constexpr int NP = 16 * DT, PF = 4;
            auto ksrc = [&](int n) {
                const int t = n / DT, dt = n % DT;
                const int row = 8 * (t >> 2) + 4 * hh + (t & 3);
                return *reinterpret_cast<const float*>(kl + TL::float_off(row, 32 * dt + j));
            };
            float kb[PF];
    #pragma unroll
            for (int n = 0; n < PF; ++n) kb[n] = ksrc(n);
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int n = 0; n < NP; ++n) {
                const float kv = kb[n % PF];
                if (n + PF < NP) kb[n % PF] = ksrc(n + PF);
                acc[n % DT] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv, s[n / DT], acc[n % DT], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        if (nt > 0) {
            copy_rows<D>(Kg, a.ss, 0, a.N, kt0, wave, NW, lane);
            copy_rows<D>(Vg, a.ss, 0, a.N, vt0, wave, NW, lane);
        }
        auto step = [&](int kt, char* kc, char* vc, char* kn, char* vn) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();   // tile kt is in LDS; every wave is done with tile kt - 1
            if (kt + 1 < nt) {
                copy_rows<D>(Kg, a.ss, (kt + 1) * BT, a.N, kn, wave, NW, lane);
                copy_rows<D>(Vg, a.ss, (kt + 1) * BT, a.N, vn, wave, NW, lane);
            }
            if (kt < wnt) compute(kt, kc, vc);
        };
        for (int kt = 0; kt < nt; kt += 2) {
            step(kt, kt0, vt0, kt1, vt1);
            if (kt + 1 < nt) step(kt + 1, kt1, vt1, kt0, vt0);
        }
        __builtin_amdgcn_s_waitcnt(0);

        if (qi < a.N) {
            float* row = static_cast<float*>(a.dq) + base + int64_t(qi) * a.ss;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *reinterpret_cast<float4*>(row + 32 * dt + 8 * r4 + 4 * hh) =
                        make_float4(acc[dt][4 * r4] * a.scale, acc[dt][4 * r4 + 1] * a.scale,
                                    acc[dt][4 * r4 + 2] * a.scale, acc[dt][4 * r4 + 3] * a.scale);
        }
    }
}

// ---------------------------------------------------------------------------
// dK/dV kernel
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_f32_dkdv_kernel(BwdArgs a) {
    using TL = RowTile<D>;
    constexpr int NWV = 4;        // waves: 32 keys each
    constexpr int DT = D / 32;
    constexpr int KU = D / 8;
    static_assert(BK == 32 * NWV, "tile shape");
    __shared__ __attribute__((aligned(1024))) char qt0[TL::BYTES], qt1[TL::BYTES];   // Q, 32 rows
    __shared__ __attribute__((aligned(1024))) char ot0[TL::BYTES], ot1[TL::BYTES];   // dO, 32 rows
    __shared__ __attribute__((aligned(16))) float st0[2 * BT], st1[2 * BT];         // LSE*log2e, -D

    const int BH = a.B * a.H;
    const int n_kt = (a.N + BK - 1) / BK;
    const int kp = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int lo_kt = CAUSAL ? n_kt - 1 - kp : kp;
    const int n_tiles = (CAUSAL && kp < lo_kt) ? 2 : 1;   // causal: the pair (kp, T-1-kp)
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {
        if (r) __syncthreads();
        const int kt = r ? lo_kt : kp;
        const int b = bh / a.H, h = bh % a.H;
        const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
        const float* Qg = static_cast<const float*>(a.q) + base;
        const float* Kg = static_cast<const float*>(a.k) + base;
        const float* Vg = static_cast<const float*>(a.v) + base;
        const float* Og = static_cast<const float*>(a.dout) + base;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int j = lane & 31, hh = lane >> 5;
        const int k0 = kt * BK;
        const int kw0 = k0 + 32 * wave;            // first key of this wave
        const int key = kw0 + j;                   // this lane's key
        const int key_c = min(key, a.N - 1);       // keys past the end re-read the last row

        // B operands of S = Q K^T and dP = dO V^T: kreg[4u + i] = K[key][8u + 4hh + i]
        float kreg[D / 2], vreg[D / 2];
    #pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int64_t off = int64_t(key_c) * a.ss + 8 * u + 4 * hh;
            const float4 xk = *reinterpret_cast<const float4*>(Kg + off);
            const float4 xv = *reinterpret_cast<const float4*>(Vg + off);
            kreg[4 * u + 0] = xk.x; kreg[4 * u + 1] = xk.y; kreg[4 * u + 2] = xk.z; kreg[4 * u + 3] = xk.w;
            vreg[4 * u + 0] = xv.x; vreg[4 * u + 1] = xv.y; vreg[4 * u + 2] = xv.z; vreg[4 * u + 3] = xv.w;
        }

        // dV^T and dK^T of this wave's 32 keys, started by a product of zeros so
        // that they live in the accumulation registers from the start
        f32x16 accv[DT], acck[DT];
        {
            const f32x16 z16 = {};
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                accv[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(0.f, 0.f, z16, 0, 0, 0);
                acck[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(0.f, 0.f, z16, 0, 0, 0);
            }
        }
        const float c2 = a.scale_log2;
        const int n_qt = (a.N + BT - 1) / BT;
        const int qt_first = CAUSAL ? k0 / BT : 0;

        // query tile q0 (with its statistics: LSE*log2e of its 32 rows, then -D)
        auto copy_q = [&](int q0, char* qd, char* od, float* sd) {
            copy_rows<D>(Qg, a.ss, q0, a.N, qd, wave, NWV, lane);
            copy_rows<D>(Og, a.ss, q0, a.N, od, wave, NWV, lane);
            if (wave == 0) {
                const int64_t row = int64_t(bh) * a.N + min(q0 + j, a.N - 1);
                copy4_to_lds((hh ? a.ws_nd : a.ws_lse2) + row, sd);
            }
        };
        // One 32-query tile: register g of lane half hh is query q0 + 8(g>>2) + 4hh + (g&3)
        auto compute = [&](int q0, const char* ql, const char* ol, const float* sl) {
            float l2[16], ndv[16];
    #pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float4 x = *reinterpret_cast<const float4*>(sl + 8 * r4 + 4 * hh);
                const float4 y = *reinterpret_cast<const float4*>(sl + BT + 8 * r4 + 4 * hh);
                l2[4 * r4 + 0] = x.x; l2[4 * r4 + 1] = x.y; l2[4 * r4 + 2] = x.z; l2[4 * r4 + 3] = x.w;
                ndv[4 * r4 + 0] = y.x; ndv[4 * r4 + 1] = y.y; ndv[4 * r4 + 2] = y.z; ndv[4 * r4 + 3] = y.w;
            }
            f32x16 s, dp;
    #pragma unroll
            for (int g = 0; g < 16; ++g) { s[g] = 0.f; dp[g] = ndv[g]; }
            // the chunks of read u + 1 are issued before the products of read u
            float4 qn = *reinterpret_cast<const float4*>(ql + TL::chunk_off(j, hh));
            float4 on = *reinterpret_cast<const float4*>(ol + TL::chunk_off(j, hh));
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int u = 0; u < KU; ++u) {
                const float4 qx = qn, ox = on;
                if (u + 1 < KU) {
                    qn = *reinterpret_cast<const float4*>(ql + TL::chunk_off(j, 2 * u + 2 + hh));
                    on = *reinterpret_cast<const float4*>(ol + TL::chunk_off(j, 2 * u + 2 + hh));
                }
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qx.x, kreg[4 * u + 0], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ox.x, vreg[4 * u + 0], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qx.y, kreg[4 * u + 1], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ox.y, vreg[4 * u + 1], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qx.z, kreg[4 * u + 2], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ox.z, vreg[4 * u + 2], dp, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qx.w, kreg[4 * u + 3], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ox.w, vreg[4 * u + 3], dp, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // masked (query, key) pairs: queries past the end, and under the
            // causal mask queries before the key, get P = 0
            if ((q0 + BT > a.N) || (CAUSAL && q0 < kw0 + 31)) {   // wave-uniform
                const int lo = CAUSAL ? key - q0 - 4 * hh : -(1 << 30);
                const int hi = a.N - 1 - q0 - 4 * hh;
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    const int off = 8 * (g >> 2) + (g & 3);
                    if (off < lo || off > hi) s[g] = -INFINITY;
                }
            }
            f32x16 ds;
    #pragma unroll
            for (int g = 0; g < 16; ++g) {
                s[g] = __builtin_amdgcn_exp2f(fmaf(s[g], c2, -l2[g]));   // P
                ds[g] = s[g] * dp[g];                                   // dS
            }
            // dV^T += dO^T P and dK^T += Q^T dS: product pair n takes the query
            // pair of register n / DT (head-dim tile n % DT); the dO^T and Q^T
            // operands are read PF pairs ahead
            constexpr int NP = 16 * DT, PF = 3;
            auto src = [&](const char* t_lds, int n) {
                const int t = n / DT, dt = n % DT;
                const int row = 8 * (t >> 2) + 4 * hh + (t & 3);
                return *reinterpret_cast<const float*>(t_lds + TL::float_off(row, 32 * dt + j));
            };
            float ob[PF], qb[PF];
    #pragma unroll
            for (int n = 0; n < PF; ++n) { ob[n] = src(ol, n); qb[n] = src(ql, n); }
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int n = 0; n < NP; ++n) {
                const float ov = ob[n % PF], qv = qb[n % PF];
                if (n + PF < NP) { ob[n % PF] = src(ol, n + PF); qb[n % PF] = src(ql, n + PF); }
                accv[n % DT] = __builtin_amdgcn_mfma_f32_32x32x2f32(ov, s[n / DT], accv[n % DT], 0, 0, 0);
                acck[n % DT] = __builtin_amdgcn_mfma_f32_32x32x2f32(qv, ds[n / DT], acck[n % DT], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        if (qt_first < n_qt) copy_q(qt_first * BT, qt0, ot0, st0);
        auto step = [&](int it, char* qc, char* oc, float* sc, char* qn, char* on, float* sn) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();   // tile it is in LDS; every wave is done with tile it - 1
            if (it + 1 < n_qt) copy_q((it + 1) * BT, qn, on, sn);
            compute(it * BT, qc, oc, sc);
        };
        for (int it = qt_first; it < n_qt; it += 2) {
            step(it, qt0, ot0, st0, qt1, ot1, st1);
            if (it + 1 < n_qt) step(it + 1, qt1, ot1, st1, qt0, ot0, st0);
        }
        __builtin_amdgcn_s_waitcnt(0);

        // register g of lane half hh: column 32dt + 8(g>>2) + 4hh + (g&3) of key `key`
        if (key < a.N) {
            float* rv = static_cast<float*>(a.dv) + base + int64_t(key) * a.ss;
            float* rk = static_cast<float*>(a.dk) + base + int64_t(key) * a.ss;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int c = 32 * dt + 8 * r4 + 4 * hh;
                    *reinterpret_cast<float4*>(rv + c) =
                        make_float4(accv[dt][4 * r4], accv[dt][4 * r4 + 1], accv[dt][4 * r4 + 2], accv[dt][4 * r4 + 3]);
                    *reinterpret_cast<float4*>(rk + c) =
                        make_float4(acck[dt][4 * r4] * a.scale, acck[dt][4 * r4 + 1] * a.scale,
                                    acck[dt][4 * r4 + 2] * a.scale, acck[dt][4 * r4 + 3] * a.scale);
                }
        }
    }
}

template <int D>
int run(const BwdArgs& a, hipStream_t s) {
    // the dQ kernel first: it also writes the per-row statistics the dK/dV
    // kernel reads.  At d = 128 the per-query operands (Q^T, dO^T and dQ^T,
    // 3 x 64 registers) need one wave per SIMD: 4-wave workgroups of 128
    // queries.  At d = 64, 8-wave workgroups (two waves per SIMD) unless that
    // grid would leave CUs idle.
    const int64_t n_qt8 = (a.N + 255) / 256;
    const int64_t grid8 = (a.causal ? (n_qt8 + 1) / 2 : n_qt8) * a.B * a.H;
    bool launched = false;
    if constexpr (D == 64) {
        if (grid8 >= 512) {
            const unsigned g = static_cast<unsigned>(grid8);
            if (a.causal) hipLaunchKernelGGL((bwd_f32_dq_kernel<D, 8, true>), dim3(g), dim3(512), 0, s, a);
            else hipLaunchKernelGGL((bwd_f32_dq_kernel<D, 8, false>), dim3(g), dim3(512), 0, s, a);
            launched = true;
        }
    }
    if (!launched) {
        const int64_t n_qt4 = (a.N + 127) / 128;
        const unsigned g = static_cast<unsigned>((a.causal ? (n_qt4 + 1) / 2 : n_qt4) * a.B * a.H);
        if (a.causal) hipLaunchKernelGGL((bwd_f32_dq_kernel<D, 4, true>), dim3(g), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((bwd_f32_dq_kernel<D, 4, false>), dim3(g), dim3(256), 0, s, a);
    }
    int err = static_cast<int>(hipGetLastError());
    if (err) return err;
    const int n_kt = (a.N + BK - 1) / BK;
    const unsigned g_kv = static_cast<unsigned>(int64_t(a.causal ? (n_kt + 1) / 2 : n_kt) * a.B * a.H);
    if (a.causal) hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, true>), dim3(g_kv), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, false>), dim3(g_kv), dim3(256), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_bwd_f32(const BwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.D == 64 ? run<64>(a, s) : run<128>(a, s);
}

}  // namespace fa
