// fwd_f32.hip -- fp32 forward attention for gfx950: the small-shape,
// full-precision kernel (tiled online softmax, one query row per lane).
//
// Algorithm ("FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析",
// sec. 5-6 and 8): the keys/values are streamed in tiles of KT rows through
// LDS; every lane keeps its query row, its output accumulator and the running
// statistics (m, l) in registers; each tile updates them with the online
// softmax rule and the output is normalised once at the end (sec. 8.1).
// Scores are taken to base 2 (scale * log2 e folded in), and the running
// maximum only advances when a tile's maximum exceeds it by more than tau
// ("FlashAttention-4" explainer, 論文 Section 3.3); the final O / l and
// LSE = ln2 * (m + log2 l) are exact either way (rescaling identity, sec. 6.3).
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>

#include "internal.h"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 64;  // one wave, one query row per lane
constexpr int KT = 32;             // keys per LDS tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRowsPerBlock) void fwd_f32_kernel(FwdArgs a) {
    __shared__ float Ks[KT][D];
    __shared__ float Vs[KT][D];

    const int n_qt = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
    const int bh = blockIdx.x / n_qt;
    const int qt = blockIdx.x % n_qt;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
    const float* Q = static_cast<const float*>(a.q) + base;
    const float* K = static_cast<const float*>(a.k) + base;
    const float* V = static_cast<const float*>(a.v) + base;
    float* O = static_cast<float*>(a.o) + base;

    const int tid = threadIdx.x;
    const int qi = qt * kRowsPerBlock + tid;
    const bool valid = qi < a.N;

    float qr[D];
    float acc[D];
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        float4 x = valid ? *reinterpret_cast<const float4*>(Q + int64_t(qi) * a.ss + c)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        qr[c] = x.x; qr[c + 1] = x.y; qr[c + 2] = x.z; qr[c + 3] = x.w;
        acc[c] = acc[c + 1] = acc[c + 2] = acc[c + 3] = 0.f;
    }
    float m_ref = -FLT_MAX;  // running maximum (log2 units) the exponentials refer to
    float l = 0.f;           // running sum of exp2(score - m_ref)

    const int last_q = min(a.N, (qt + 1) * kRowsPerBlock) - 1;
    const int n_keys = CAUSAL ? last_q + 1 : a.N;
    const float c2 = a.scale_log2;

    for (int k0 = 0; k0 < n_keys; k0 += KT) {
        __syncthreads();
        // Cooperative, coalesced load of K/V rows k0 .. k0+KT-1 (zeros past N).
        for (int e = tid * 4; e < KT * D; e += kRowsPerBlock * 4) {
            const int r = e / D, c = e % D;
            const int key = k0 + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < a.N) {
                kx = *reinterpret_cast<const float4*>(K + int64_t(key) * a.ss + c);
                vx = *reinterpret_cast<const float4*>(V + int64_t(key) * a.ss + c);
            }
            *reinterpret_cast<float4*>(&Ks[r][c]) = kx;
            *reinterpret_cast<float4*>(&Vs[r][c]) = vx;
        }
        __syncthreads();

        float s[KT];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = fmaf(qr[c], Ks[j][c], dot);
            const int key = k0 + j;
            const bool masked = key >= a.N || (CAUSAL && key > qi);
            s[j] = masked ? -INFINITY : dot;
            tmax = fmaxf(tmax, s[j]);
        }
        const float mt = tmax * c2;
        if (mt > m_ref + a.tau) {
            const float mn = fmaxf(m_ref, mt);
            const float alpha = exp2f(m_ref - mn);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] *= alpha;
            m_ref = mn;
        }
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const float p = exp2f(fmaf(s[j], c2, -m_ref));
            l += p;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(p, Vs[j][c], acc[c]);
        }
    }

    if (valid) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            float4 x = make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
            *reinterpret_cast<float4*>(O + int64_t(qi) * a.ss + c) = x;
        }
        a.lse[int64_t(bh) * a.N + qi] = (m_ref + log2f(l)) * 0.69314718055994531f;
    }
}

template <int D, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qt = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t grid = int64_t(n_qt) * a.B * a.H;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(static_cast<unsigned>(grid)),
                       dim3(kRowsPerBlock), 0, stream, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_fwd_f32(const FwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 64) return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
    return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace fa
