// internal.h -- shared between the host API and the kernel translation units.
// Not part of the public ABI (include/flash_attn.h is).
#pragma once
#include <stdint.h>

namespace fa {

// Arguments of one forward launch, already validated by the host API.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;          // contiguous [B, H, N]
    int64_t sb, sh, ss;  // element strides shared by q, k, v, o (head_dim stride 1)
    int32_t B, H, N, D;
    float scale_log2;    // softmax scale times log2(e): scores go straight to exp2
    float tau;           // conditional-rescale threshold, log2 units
    int32_t causal;
    int32_t tile_cfg;
};

// FP8 pre-pass arguments.
struct QuantArgs {
    const void* x;
    int32_t in_bf16;      // 1: x is bf16, 0: x is f32
    int64_t sb, sh, ss;   // strides of x (elements)
    int32_t B, H, N, D;
    int32_t role;         // 0 Q, 1 K, 2 V
    int32_t rotate;
    const int8_t* signs;  // [D] +-1 (device)
    uint8_t* out;         // Q/K: [B, H, N, D]; V: [B, H, D, N_pad]
    float* scales;        // [B, H, ceil(N / block)]
};

// FP8 attention arguments.
struct Fp8Args {
    const uint8_t* q;
    const uint8_t* k;      // contiguous [B, H, N, D]
    const uint8_t* vt;     // contiguous [B, H, D, N_pad]
    const float* qs;
    const float* ks;
    const float* vs;       // per-block scales
    void* o;               // bf16, strides below
    float* lse;
    int64_t osb, osh, oss;
    int32_t B, H, N, D;
    float scale_log2;
    float tau;
    int32_t causal;
    int32_t tile_cfg;
    int32_t q_terms;       // 1: Q's first e4m3 term only; 2: both terms
};

// Backward arguments (bf16 or fp32 tensors sharing one layout; fp32 workspace
// of two per-row arrays [B, H, N]).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;     // contiguous [B, H, N], natural log
    void* dq;
    void* dk;
    void* dv;
    int64_t sb, sh, ss;   // element strides shared by every tensor above
    int32_t B, H, N, D;
    float scale;
    float scale_log2;
    int32_t causal;
    float* ws_lse2;       // [B, H, N] LSE * log2(e)
    float* ws_nd;         // [B, H, N] -rowsum(dO o O)
};

// Merge of attention results over disjoint key sets.
struct MergeArgs {
    const void* o_parts;   // part s at o_parts + s * part_stride, strides below
    const float* lse_parts;  // contiguous [S, B, H, N]
    void* o;               // same strides as a part
    float* lse;            // contiguous [B, H, N]
    int64_t sb, sh, ss, part_stride;
    int32_t B, H, N, D, S;
    int32_t bf16;
};

// Workspace bytes of the backward pass (each part 256-byte aligned).
inline int64_t bwd_ws_part(int64_t n) { return (n * 4 + 255) / 256 * 256; }
inline int64_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
    return 2 * bwd_ws_part(B * H * N);
}

// Fixed device scratch buffer (scratch.hip) for the allocation-free backward:
// its size bounds B * H * N at 2^21 rows (two fp32 values per row).
constexpr int64_t kScratchBytes = int64_t(16) << 20;
// Device address of the scratch array on the current device (looked up once
// per device); returns a hipError_t value.
int scratch_buffer(void** ptr);

// Launchers: return a hipError_t value (0 = success).
int launch_fwd_bf16(const FwdArgs& a, void* stream);
int launch_fwd_f32(const FwdArgs& a, void* stream);
int launch_fp8_quantize(const QuantArgs& a, void* stream);
int launch_fwd_fp8(const Fp8Args& a, void* stream);
int launch_bwd_bf16(const BwdArgs& a, void* stream);
int launch_bwd_f32(const BwdArgs& a, void* stream);
int launch_merge(const MergeArgs& a, void* stream);

// Rows per scale block the fp8 attention kernel is built for (Q: a wave's
// 32 query rows; K: the 32 keys one lane half holds; V: one 64-key tile), and
// the key padding of the transposed V buffer.
constexpr int kFp8QBlock = 32;
constexpr int kFp8KBlock = 32;
constexpr int kFp8VBlock = 64;
constexpr int64_t fp8_npad(int64_t n) { return (n + kFp8VBlock - 1) / kFp8VBlock * kFp8VBlock; }

}  // namespace fa
