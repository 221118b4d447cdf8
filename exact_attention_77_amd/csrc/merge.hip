// merge.hip -- combine attention results over disjoint key sets.
//
// Part s holds, for every query row, the normalised output O_s over its own
// keys and the natural-log LSE_s of its scores.  The result over the union of
// the keys is LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s:
// the rescale-and-add step of the online softmax of "FlashAttention:
// GPUメモリ階層を活用したアテンション最適化の分析" sec. 6.2 (exact by the
// rescaling identity of sec. 6.3), applied to whole partial results.  It is
// the combine step of attention sharded over the sequence (Ring Attention is
// named as the direction for multi-GPU use in the "FlashAttention-4"
// explainer's outlook and as a user of the kernel in the "FlashAttention-3"
// note's strengths).
//
// The operation is a stream over HBM: every part's O is read once and O is
// written once.  A row is handled by D/8 consecutive lanes, each owning 8
// columns (16 or 32 contiguous bytes); every lane of the row reads the S
// LSE values (cached) and forms the weights itself.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;
constexpr float kLog2e = 1.4426950408889634f;

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
    constexpr int LPR = D / 8;
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row = t / LPR;                 // flat (b, h, i)
    const int l = static_cast<int>(t % LPR);
    const int64_t rows = int64_t(a.B) * a.H * a.N;
    if (row >= rows) return;
    const int i = static_cast<int>(row % a.N);
    const int64_t bh = row / a.N;
    const int b = static_cast<int>(bh / a.H), h = static_cast<int>(bh % a.H);
    const int64_t off = int64_t(b) * a.sb + int64_t(h) * a.sh + int64_t(i) * a.ss + 8 * l;

    float m = -INFINITY;
    for (int s = 0; s < a.S; ++s) m = fmaxf(m, a.lse_parts[int64_t(s) * rows + row]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float total = 0.f;
    // the lane's 8 columns of part s, as floats
    auto load = [&](int s, float (&x)[8]) {
        const int64_t po = int64_t(s) * a.part_stride + off;
        if (BF16) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                            static_cast<const u16*>(a.o_parts) + po));
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
        } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.o_parts) + po);
            const float4 x0 = p[0], x1 = p[1];
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
            x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        }
    };
    auto weight = [&](int s) {
        return __builtin_amdgcn_exp2f((a.lse_parts[int64_t(s) * rows + row] - m) * kLog2e);
    };
    // A part of weight 0 (LSE_s = -inf: no key; or a weight that underflows)
    // adds nothing, whatever its O holds -- an empty shard's O may be 0/0.
    auto add = [&](float w, const float (&x)[8]) {
        total += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, w != 0.f ? x[e] : 0.f, acc[e]);
    };
    if (m != -INFINITY) {
        // four parts' loads in flight before their products (the stream is
        // bound by how many bytes each lane keeps outstanding)
        constexpr int U = 4;
        int s = 0;
        for (; s + U <= a.S; s += U) {
            float x[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u) load(s + u, x[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) add(weight(s + u), x[u]);
        }
        for (; s < a.S; ++s) {
            float x[8];
            load(s, x);
            add(weight(s), x);
        }
    }
    // no key in any part: O = 0, LSE = -inf
    const float inv = m != -INFINITY ? 1.0f / total : 0.f;
    if (BF16) {
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = static_cast<__bf16>(acc[e] * inv);
        *reinterpret_cast<uint4*>(static_cast<u16*>(a.o) + off) = __builtin_bit_cast(uint4, y);
    } else {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(a.o) + off);
        p[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        p[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
    if (l == 0) a.lse[row] = m != -INFINITY ? m + logf(total) : -INFINITY;
}

template <int D, bool BF16>
int run(const MergeArgs& a, hipStream_t s) {
    const int64_t threads = int64_t(a.B) * a.H * a.N * (D / 8);
    hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                       s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_merge(const MergeArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 64) return a.bf16 ? run<64, true>(a, s) : run<64, false>(a, s);
    return a.bf16 ? run<128, true>(a, s) : run<128, false>(a, s);
}

}  // namespace fa
