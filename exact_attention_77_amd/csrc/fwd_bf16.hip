// fwd_bf16.hip -- bf16 forward attention for gfx950 on MFMA matrix cores.
//
// The method is the fused tiled attention with online softmax of
// "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析": one workgroup
// per (batch, head, query tile) with the query tile as the outer loop and the
// K/V tiles streamed through on-chip memory (sec. 5 and 8.2), the running
// maximum / sum update of sec. 6.2, and a single normalisation at the end
// (sec. 8.1).  Queries are split across waves, K/V are shared (sec. 8.3).
// The maximum the exponentials refer to only advances when a tile's maximum
// exceeds it by more than tau ("FlashAttention-4" explainer, 論文 Section 3.3);
// the output stays exact by the rescaling identity (sec. 6.3).
//
// gfx950 mapping (designed for CDNA4, not taken from the pages' Hopper or
// Blackwell kernels):
//  * a wave owns 32 query rows.  It computes the TRANSPOSED score tile
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//    B = Q^T held in registers for the whole loop).  In the 32x32 accumulator
//    layout lane l holds column l % 32, i.e. ONE query, and 16 of the keys, so
//    the row maximum and row sum are in-lane reductions plus one exchange
//    between lane l and l ^ 32.
//  * the K rows are fed to the first product in a permuted order (bits 2 and
//    3 of the row index swapped) so that the accumulator registers of S^T are,
//    after exp2 and a bf16 conversion, already the B operand of the second
//    product O^T += V^T P^T: no LDS round trip for P.
//  * O^T stays in registers with one query per lane, so the rescale factor is
//    a per-lane scalar.
//  * K is stored in LDS row-major and V transposed (d-major), both padded so
//    that the 16-byte operand reads of 16 consecutive rows hit distinct banks;
//    two buffers let the global loads of tile j+1 overlap the math of tile j.
//  * workgroups are renumbered so that the tiles of one head run on one XCD
//    (the hardware deals workgroup ids round-robin over the 8 XCDs), which
//    keeps that head's K/V in the XCD's L2; under the causal mask the heaviest
//    query tiles of a head start first.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int BC = 64;  // keys per K/V tile
constexpr int WQ = 32;  // query rows per wave

template <int D>
struct Lds {
    static constexpr int KS = D + 8;   // K row stride (elements)
    static constexpr int VS = BC + 8;  // V^T row stride (elements)
    static constexpr int K_ELEMS = BC * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int BYTES = 2 * BUF * int(sizeof(u16));
};

// Row of the A operand that lane row i loads: bits 2 and 3 swapped.  With this
// order the S^T accumulator register g = 4r + t of lane half hh holds key
//   16 * (r >> 1) + 8 * hh + 4 * (r & 1) + t
// so registers 8c .. 8c+7 hold keys 16c + 8hh .. 16c + 8hh + 7, exactly the
// B-operand slice lane (query, hh) must supply for keys 16c .. 16c+15.
__device__ __forceinline__ int perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
    using L = Lds<D>;
    constexpr int BR = NW * WQ;          // query rows per workgroup
    constexpr int T = NW * 64;           // threads
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int CH = BC * CPR / T;     // chunks per thread per tile (K and V each)
    static_assert(CH >= 1 && BC * CPR % T == 0, "tile / thread mismatch");
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;

    extern __shared__ __attribute__((aligned(16))) u16 smem[];

    // ---- work decomposition -------------------------------------------------
    const int n_qt = (a.N + BR - 1) / BR;
    const int total = n_qt * a.B * a.H;
    int id = blockIdx.x;
    if ((total & 7) == 0) {  // one contiguous range of (head, tile) per XCD
        const int per = total >> 3;
        id = (id & 7) * per + (id >> 3);
    }
    const int bh = id / n_qt;
    int qt = id % n_qt;
    if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest tile of the head first
    const int b = bh / a.H, h = bh % a.H;
    const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
    const u16* Qg = static_cast<const u16*>(a.q) + base;
    const u16* Kg = static_cast<const u16*>(a.k) + base;
    const u16* Vg = static_cast<const u16*>(a.v) + base;
    u16* Og = static_cast<u16*>(a.o) + base;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int j = lane & 31, hh = lane >> 5;
    const int q0 = qt * BR + wave * WQ;  // first query row of this wave
    const int qi = q0 + j;               // this lane's query row

    const int n_kt_all = (a.N + BC - 1) / BC;
    const int kt_end = CAUSAL ? min(n_kt_all, (min(a.N, (qt + 1) * BR) + BC - 1) / BC) : n_kt_all;
    int wave_kt_end = CAUSAL ? min(kt_end, (min(a.N, q0 + WQ) + BC - 1) / BC) : kt_end;
    if (q0 >= a.N) wave_kt_end = 0;

    // ---- Q^T operand: lane (query j, half hh) holds Q[qi][16ks + 8hh .. +7] ----
    bf16x8 qreg[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (qi < a.N) x = *reinterpret_cast<const uint4*>(Qg + int64_t(qi) * a.ss + 16 * ks + 8 * hh);
        qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 16; ++g) oacc[dt][g] = 0.f;
    float m_ref = -FLT_MAX;  // log2 units
    float lsum = 0.f;        // this lane's share of the running sum
    const float c2 = a.scale_log2;

    // ---- K/V tile staging: global -> registers -> LDS ------------------------
    uint4 kreg[CH], vreg[CH];
    auto load_global = [&](int kt) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * T;
            const int row = c / CPR, col = (c % CPR) * 8;
            const int key = kt * BC + row;
            uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
            if (key < a.N) {
                kx = *reinterpret_cast<const uint4*>(Kg + int64_t(key) * a.ss + col);
                vx = *reinterpret_cast<const uint4*>(Vg + int64_t(key) * a.ss + col);
            }
            kreg[i] = kx;
            vreg[i] = vx;
        }
    };
    auto store_lds = [&](int buf) {
        u16* Ks = smem + buf * L::BUF;
        u16* Vts = Ks + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * T;
            const int row = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<uint4*>(Ks + row * L::KS + col) = kreg[i];
            const u16* v8 = reinterpret_cast<const u16*>(&vreg[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) Vts[(col + e) * L::VS + row] = v8[e];
        }
    };

    if (kt_end > 0) {
        load_global(0);
        store_lds(0);
    }
    __syncthreads();

    for (int kt = 0; kt < kt_end; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < kt_end) load_global(kt + 1);

        if (kt < wave_kt_end) {
            const u16* Ks = smem + buf * L::BUF;
            const u16* Vts = Ks + L::K_ELEMS;

            // S^T = K Q^T for keys kt*BC + [0, 32) and [32, 64)
            f32x16 s[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int g = 0; g < 16; ++g) s[st][g] = 0.f;
                const u16* krow = Ks + (32 * st + perm_row(j)) * L::KS + 8 * hh;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 16 * ks);
                    s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s[st], 0, 0, 0);
                }
            }

            // masking: causal diagonal tiles and the ragged end of the keys
            const int k_lo = kt * BC;
            const bool need_mask = (k_lo + BC > a.N) || (CAUSAL && k_lo + BC - 1 > q0);
            if (need_mask) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int g = 0; g < 16; ++g) {
                        const int r = g >> 2, t = g & 3;
                        const int key = k_lo + 32 * st + 16 * (r >> 1) + 8 * hh + 4 * (r & 1) + t;
                        const bool masked = key >= a.N || (CAUSAL && key > qi);
                        if (masked) s[st][g] = -INFINITY;
                    }
            }

            // online softmax, base 2, conditional rescale (wave-uniform decision)
            float mx = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int g = 0; g < 16; ++g) mx = fmaxf(mx, s[st][g]);
            mx = fmaxf(mx, xor32(mx));
            const float mt = mx * c2;
            const bool need = mt > m_ref + a.tau;
            if (__any(need)) {
                const float mn = fmaxf(m_ref, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int g = 0; g < 16; ++g) oacc[dt][g] *= alpha;
                m_ref = mn;
            }
            bf16x8 pb[2][2];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __builtin_amdgcn_exp2f(fmaf(s[st][8 * cc + e], c2, -m_ref));
                        lsum += p;
                        pb[st][cc][e] = static_cast<__bf16>(p);
                    }

            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u16* vrow = Vts + (32 * dt + j) * L::VS + 8 * hh;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + 32 * st + 16 * cc);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st][cc], oacc[dt], 0, 0, 0);
                    }
            }
        }

        if (kt + 1 < kt_end) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------
    if (qi < a.N && wave_kt_end > 0) {
        const float lt = lsum + xor32(lsum);
        const float inv = 1.0f / lt;
        u16* orow = Og + int64_t(qi) * a.ss;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __bf16 o4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) o4[t] = static_cast<__bf16>(oacc[dt][4 * r + t] * inv);
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * r + 4 * hh) = __builtin_bit_cast(uint2, o4);
            }
        if (hh == 0) a.lse[int64_t(bh) * a.N + qi] = (m_ref + __log2f(lt)) * 0.69314718055994531f;
    }
}

template <int D, int NW, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
    using L = Lds<D>;
    constexpr int BR = NW * WQ;
    auto kern = fwd_bf16_kernel<D, NW, CAUSAL>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    const int n_qt = (a.N + BR - 1) / BR;
    const int64_t grid = int64_t(n_qt) * a.B * a.H;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(NW * 64), L::BYTES, stream, a);
    return static_cast<int>(hipGetLastError());
}

template <int D>
int dispatch(const FwdArgs& a, hipStream_t s) {
    // tile_cfg 0/1: 8 waves (256 query rows per workgroup); 2: 4 waves (128 rows).
    if (a.tile_cfg == 2) return a.causal ? launch<D, 4, true>(a, s) : launch<D, 4, false>(a, s);
    return a.causal ? launch<D, 8, true>(a, s) : launch<D, 8, false>(a, s);
}

}  // namespace

int launch_fwd_bf16(const FwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.D == 64 ? dispatch<64>(a, s) : dispatch<128>(a, s);
}

}  // namespace fa
