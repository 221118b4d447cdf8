// fwd_f32.hip -- fp32 forward attention for gfx950 on the fp32 matrix cores.
//
// What is computed ("FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析",
// sec. 2.1, 6 and 8): O = softmax(scale * Q K^T) V row by row and the
// natural-log LSE, with the keys/values streamed through LDS in tiles and the
// online softmax update of sec. 6.2 (exact by the rescaling identity of sec.
// 6.3), a single normalisation at the end (sec. 8.1), causal mask of sec. 11.3.
// Scores are taken to base 2 (scale * log2 e folded into one FMA), and the
// running maximum only advances when a tile's maximum exceeds it by more than
// tau ("FlashAttention-4" explainer, 論文 Section 3.3); every product and sum
// stays in fp32.
//
// Layout (the bf16 kernel's, on v_mfma_f32_32x32x2_f32): a wave owns 32
// queries and computes the transposed score tile S^T = K Q^T for 32 keys at a
// time -- lane (query j, half h) ends up holding the scores of its own query
// for keys 8 (g / 4) + 4 h + g % 4 in accumulator register g -- with K rows
// from LDS as the A operand and Q^T in registers as the B operand.  K-step s
// of the contraction pairs head-dim columns 8 (s / 4) + 4 h + s % 4 of lane
// half h, so that one 16-byte LDS read feeds four products.  An fp32 product
// takes one value per lane for each operand, so register g of the score tile
// is directly the B operand of O^T += V^T P for the key pair it holds, and the
// A operand is the matching V row, read 32 consecutive floats per lane half:
// no re-layout of P at all.  Two independent accumulation chains (even and
// odd k-steps) keep consecutive score products independent; the PV products
// of the head-dim tiles are independent by themselves.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>

#include "internal.h"
#include "lds_copy.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WQ = 32;   // queries per wave
constexpr int BC = 32;   // keys per K/V tile

template <int D>
struct TileF {
    static constexpr int CPR = D / 4;          // 16-byte chunks per row
    static constexpr int BYTES = BC * D * 4;   // one K or V tile
    // 32 lanes read one logical chunk of 32 different K rows: the physical
    // chunk is the logical one XOR the row, so that they hit distinct banks.
    __device__ static int kswz(int row) { return row & (CPR - 1); }
};

__device__ __forceinline__ float pair_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One query tile (NW waves of 32 queries) of head bh.
template <int D, int NW, bool CAUSAL>
__device__ __forceinline__ void f32_tile(const FwdArgs& a, char* lds, int bh, int qt) {
    using TL = TileF<D>;
    constexpr int BR = NW * WQ;
    constexpr int DT = D / 32;                  // head-dim tiles of O^T
    constexpr int NI = TL::BYTES / 1024 / NW;   // 1 KB copies per wave per tile
    static_assert(NI >= 1 && TL::BYTES % (1024 * NW) == 0, "tile / wave mismatch");

    const int b = bh / a.H, h = bh % a.H;
    const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
    const float* Qg = static_cast<const float*>(a.q) + base;
    const float* Kg = static_cast<const float*>(a.k) + base;
    const float* Vg = static_cast<const float*>(a.v) + base;
    float* Og = static_cast<float*>(a.o) + base;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31, hh = lane >> 5;
    const int q0 = qt * BR + wave * WQ;   // first query of this wave
    const int qi = q0 + j;                // this lane's query

    const int n_kt_all = (a.N + BC - 1) / BC;
    const int nt = CAUSAL ? min(n_kt_all, (min(a.N, (qt + 1) * BR) + BC - 1) / BC) : n_kt_all;
    int wnt = CAUSAL ? min(nt, (min(a.N, q0 + WQ) + BC - 1) / BC) : nt;
    if (q0 >= a.N) wnt = 0;

    // ---- direct global -> LDS tile copies: lane L of 1 KB block blk fills
    // physical chunk (64 blk + L) % CPR of row (64 blk + L) / CPR; K rows are
    // swizzled (the source chunk is the physical one XOR the swizzle), V rows
    // are stored as they are.  Rows past the end re-read the last row; their
    // scores are masked.
    int crow[NI];
    const float* kp[NI];
    const float* vp[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = (wave * NI + i) * 64 + lane;
        crow[i] = c / TL::CPR;
        const int pch = c % TL::CPR;
        kp[i] = Kg + int64_t(crow[i]) * a.ss + 4 * (pch ^ TL::kswz(crow[i]));
        vp[i] = Vg + int64_t(crow[i]) * a.ss + 4 * pch;
    }
    auto copy_tile = [&](const float* const (&src)[NI], int kt, int lds_off) {
        const int k0 = kt * BC;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t row_off = int64_t(min(k0 + crow[i], a.N - 1) - crow[i]);
            copy16_to_lds(src[i] + row_off * a.ss, lds + lds_off + (wave * NI + i) * 1024);
        }
    };
    constexpr int K_OFF0 = 0, K_OFF1 = TL::BYTES, V_OFF0 = 2 * TL::BYTES, V_OFF1 = 3 * TL::BYTES;

    // ---- Q^T: qreg[4u + i] = Q[qi][8u + 4hh + i], the B operand of k-step 4u + i
    float qreg[D / 2];
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qi < a.N) x = *reinterpret_cast<const float4*>(Qg + int64_t(qi) * a.ss + 8 * u + 4 * hh);
        qreg[4 * u + 0] = x.x; qreg[4 * u + 1] = x.y; qreg[4 * u + 2] = x.z; qreg[4 * u + 3] = x.w;
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 16; ++g) oacc[dt][g] = 0.f;
    float m_ref = -FLT_MAX;   // log2 units
    float lpart = 0.f;        // this lane half's share of the running sum
    const float c2 = a.scale_log2;

    // One K/V tile: scores, the threshold rule, probabilities, O^T += V^T P.
    auto tile = [&](int kt, const char* kt_lds, const char* vt_lds) {
        const float* krow = reinterpret_cast<const float*>(kt_lds + j * (D * 4));
        f32x16 se = {}, so = {};
        // the chunk of read u + 1 is issued before the products of read u
        float4 kn = *reinterpret_cast<const float4*>(krow + 4 * (hh ^ TL::kswz(j)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < D / 8; ++u) {
            const float4 kx = kn;
            if (u + 1 < D / 8) kn = *reinterpret_cast<const float4*>(krow + 4 * ((2 * u + 2 + hh) ^ TL::kswz(j)));
            se = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.x, qreg[4 * u + 0], se, 0, 0, 0);
            so = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.y, qreg[4 * u + 1], so, 0, 0, 0);
            se = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.z, qreg[4 * u + 2], se, 0, 0, 0);
            so = __builtin_amdgcn_mfma_f32_32x32x2f32(kx.w, qreg[4 * u + 3], so, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x16 s = se + so;
        // keys past the query (causal) or past the end score -inf; register g
        // of lane half hh is key k0 + 8 (g / 4) + 4 hh + g % 4
        const int k0 = kt * BC;
        if ((k0 + BC > a.N) || (CAUSAL && k0 + BC - 1 > q0)) {
            const int lim = (CAUSAL ? min(qi, a.N - 1) : a.N - 1) - k0 - 4 * hh;
#pragma unroll
            for (int g = 0; g < 16; ++g)
                if (8 * (g >> 2) + (g & 3) > lim) s[g] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int g = 0; g < 16; ++g) mx = fmaxf(mx, s[g]);
        const float mt = pair_max32(mx) * c2;
        if (__any(mt > m_ref + a.tau)) {
            const float mn = fmaxf(m_ref, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
            lpart *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 16; ++g) oacc[dt][g] *= alpha;
            m_ref = mn;
        }
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            s[g] = __builtin_amdgcn_exp2f(fmaf(s[g], c2, -m_ref));
            lpart += s[g];
        }
        // PV: product n takes the key pair of register t = n / DT (keys
        // 8 (t / 4) + 4 hh + t % 4 in lane half hh) and head-dim tile n % DT;
        // its V operand is read PF products ahead
        const float* vbase = reinterpret_cast<const float*>(vt_lds) + j;
        constexpr int NP = 16 * DT, PF = 4;
        auto vsrc = [&](int n) {
            const int t = n / DT, dt = n % DT;
            return vbase[(8 * (t >> 2) + 4 * hh + (t & 3)) * D + 32 * dt];
        };
        float vb[PF];
#pragma unroll
        for (int n = 0; n < PF; ++n) vb[n] = vsrc(n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const float vv = vb[n % PF];
            if (n + PF < NP) vb[n % PF] = vsrc(n + PF);
            oacc[n % DT] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[n / DT], oacc[n % DT], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: tile 0 in flight ----
    if (nt > 0) {
        copy_tile(kp, 0, K_OFF0);
        copy_tile(vp, 0, V_OFF0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- main loop, unrolled by two so that the buffers alternate ----
    auto step = [&](int kt, int k_cur, int k_nxt, int v_cur, int v_nxt) {
        if (kt + 1 < nt) {
            copy_tile(kp, kt + 1, k_nxt);
            copy_tile(vp, kt + 1, v_nxt);
        }
        if (kt < wnt) tile(kt, lds + k_cur, lds + v_cur);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();   // tile kt+1 is in LDS; every wave is done with tile kt
    };
    for (int kt = 0; kt < nt; kt += 2) {
        step(kt, K_OFF0, K_OFF1, V_OFF0, V_OFF1);
        if (kt + 1 < nt) step(kt + 1, K_OFF1, K_OFF0, V_OFF1, V_OFF0);
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ----
    // register g of head-dim tile dt in lane half hh: column 32 dt + 8 (g / 4) + 4 hh + g % 4
    if (qi < a.N && wnt > 0) {
        const float l = pair_sum32(lpart);
        const float inv = 1.0f / l;
        float* orow = Og + int64_t(qi) * a.ss;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float4 x = make_float4(oacc[dt][4 * r] * inv, oacc[dt][4 * r + 1] * inv,
                                             oacc[dt][4 * r + 2] * inv, oacc[dt][4 * r + 3] * inv);
                *reinterpret_cast<float4*>(orow + 32 * dt + 8 * r + 4 * hh) = x;
            }
        if (hh == 0) a.lse[int64_t(bh) * a.N + qi] = (m_ref + log2f(l)) * 0.69314718055994531f;
    }
}

// Work decomposition as in the bf16 kernel: workgroup ids renumbered so that
// each XCD owns whole heads; under the causal mask a workgroup takes the
// query-tile pair (T-1-p, p) of its head, so all carry the same work.
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_f32_kernel(FwdArgs a) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    constexpr int BR = NW * WQ;
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
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {
        if (r) __syncthreads();   // every wave is done with the first tile's buffers
        f32_tile<D, NW, CAUSAL>(a, lds, bh, r ? p : hi);
    }
}

template <int D, int NW, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = NW * WQ;
    constexpr int LDS = 4 * TileF<D>::BYTES;
    auto kern = fwd_f32_kernel<D, NW, CAUSAL>;
    // set once per process (thread-safe initialisation of a local static)
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return static_cast<int>(attr);
    const int n_qt = (a.N + BR - 1) / BR;
    const int64_t grid = int64_t(CAUSAL ? (n_qt + 1) / 2 : n_qt) * a.B * a.H;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(NW * 64), LDS, stream, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

namespace {
// tile_cfg 1: 8-wave workgroups (256 query rows); 2: 4 waves (128 rows);
// 0 (automatic): 8 waves unless that grid would not give every CU two
// workgroups' worth of work, then 4 (at B1 H16 N2048 the 8-wave grid is 128
// workgroups for 256 CUs).
template <int D>
int dispatch(const FwdArgs& a, hipStream_t s) {
    const int64_t n_qt8 = (a.N + 8 * WQ - 1) / (8 * WQ);
    const int64_t grid8 = (a.causal ? (n_qt8 + 1) / 2 : n_qt8) * a.B * a.H;
    const bool four = a.tile_cfg == 2 || (a.tile_cfg == 0 && grid8 < 512);
    if (four) return a.causal ? launch<D, 4, true>(a, s) : launch<D, 4, false>(a, s);
    return a.causal ? launch<D, 8, true>(a, s) : launch<D, 8, false>(a, s);
}
}  // namespace

int launch_fwd_f32(const FwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.D == 64 ? dispatch<64>(a, s) : dispatch<128>(a, s);
}

}  // namespace fa
