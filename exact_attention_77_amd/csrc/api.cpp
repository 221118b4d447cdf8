// api.cpp -- the C ABI of include/flash_attn.h: host-side validation and
// dispatch to the gfx950 kernels.  Every check runs before the first HIP call,
// so argument errors are reported without touching the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/flash_attn.h"
#include "internal.h"

namespace {

thread_local char g_last_error[256] = "";

flash_attn_status hip_status(int err) {
    if (err == 0) return FLASH_ATTN_OK;
    snprintf(g_last_error, sizeof(g_last_error), "%s (%d)",
             hipGetErrorString(static_cast<hipError_t>(err)), err);
    return FLASH_ATTN_ERR_HIP;
}

constexpr int64_t kMaxRows = int64_t(1) << 24;
constexpr int64_t kMaxTotalRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxMergeParts = 4096;
// Row stride limit: the kernels address a tile's rows with 32-bit byte
// offsets from the tile's first row (64 rows of at most 2^24 elements).
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_empty(const flash_attn_layout& L) {
    return L.batch == 0 || L.heads == 0 || L.seqlen == 0;
}

// Shape checks shared by all entry points.  Returns OK for a valid (possibly
// empty) shape.
flash_attn_status check_shape(const flash_attn_layout& L) {
    if (L.batch < 0 || L.heads < 0 || L.seqlen < 0 || L.head_dim < 0) return FLASH_ATTN_ERR_SHAPE;
    if (L.seqlen > kMaxRows) return FLASH_ATTN_ERR_SHAPE;
    if (L.batch > kMaxRows || L.heads > kMaxRows || L.batch * L.heads > kMaxRows)
        return FLASH_ATTN_ERR_SHAPE;
    // every row index and the kernels' work decompositions stay in int32
    if (L.batch * L.heads * L.seqlen > kMaxTotalRows) return FLASH_ATTN_ERR_SHAPE;
    if (is_empty(L)) return FLASH_ATTN_OK;
    if (L.head_dim != 64 && L.head_dim != 128) return FLASH_ATTN_ERR_UNSUPPORTED;
    return FLASH_ATTN_OK;
}

// Strides must keep every row 16-byte aligned, and the map from (b, h, i, c)
// to the element offset b*stride_b + h*stride_h + i*stride_s + c must be
// one-to-one over the shape, so that no two workgroups ever write the same
// output element.  Sorted by stride, each dimension of extent > 1 must step
// past everything the smaller-stride dimensions span (the head_dim, stride 1,
// is the innermost); this condition is sufficient for a one-to-one map.
flash_attn_status check_strides(const flash_attn_layout& L, int64_t elt_bytes) {
    const int64_t vec = 16 / elt_bytes;
    if (L.stride_s < L.head_dim || L.stride_h < 0 || L.stride_b < 0) return FLASH_ATTN_ERR_LAYOUT;
    if (L.stride_s > kMaxRowStride) return FLASH_ATTN_ERR_LAYOUT;
    if (L.stride_s % vec || L.stride_h % vec || L.stride_b % vec) return FLASH_ATTN_ERR_LAYOUT;
    struct Dim { int64_t stride, extent; } dims[3] = {
        {L.stride_s, L.seqlen}, {L.stride_h, L.heads}, {L.stride_b, L.batch}};
    // insertion sort by stride (three entries)
    for (int a = 1; a < 3; ++a)
        for (int b = a; b > 0 && dims[b].stride < dims[b - 1].stride; --b) {
            const Dim t = dims[b]; dims[b] = dims[b - 1]; dims[b - 1] = t;
        }
    int64_t span = L.head_dim;   // offsets 0 .. span-1 are covered so far
    for (const Dim& d : dims) {
        if (d.extent <= 1) continue;
        if (d.stride < span) return FLASH_ATTN_ERR_LAYOUT;
        // the shape limits keep this below 2^63
        span += d.stride * (d.extent - 1);
    }
    return FLASH_ATTN_OK;
}

flash_attn_status check_opts(const flash_attn_fwd_opts* opts, float* tau, int* tile_cfg,
                             int* q_terms = nullptr) {
    *tau = 8.0f;
    *tile_cfg = 0;
    if (q_terms) *q_terms = 2;
    if (!opts) return FLASH_ATTN_OK;
    if (opts->fp8_q_terms < 0 || opts->fp8_q_terms > 2) return FLASH_ATTN_ERR_ARG;
    if (q_terms && opts->fp8_q_terms != 0) *q_terms = opts->fp8_q_terms;
    if (isnan(opts->tau_log2)) return FLASH_ATTN_ERR_ARG;
    if (opts->tau_log2 >= 0.0f) {
        if (!(opts->tau_log2 <= 64.0f)) return FLASH_ATTN_ERR_ARG;
        *tau = opts->tau_log2;
    }
    if (opts->tile_cfg < 0 || opts->tile_cfg > 2) return FLASH_ATTN_ERR_ARG;
    *tile_cfg = opts->tile_cfg;
    return FLASH_ATTN_OK;
}

flash_attn_status check_scale(float scale) {
    if (!isfinite(scale) || !(scale > 0.0f)) return FLASH_ATTN_ERR_ARG;
    // scale * log2(e) must stay finite.
    if (!isfinite(scale * 1.4426950408889634f)) return FLASH_ATTN_ERR_ARG;
    return FLASH_ATTN_OK;
}

}  // namespace

extern "C" {

flash_attn_status flash_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                 float* lse, flash_attn_layout layout,
                                 flash_attn_dtype dtype, int causal, float scale,
                                 const flash_attn_fwd_opts* opts, void* stream) {
    flash_attn_status st = check_shape(layout);
    if (st != FLASH_ATTN_OK) return st;
    if (dtype != FLASH_ATTN_F32 && dtype != FLASH_ATTN_BF16) return FLASH_ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return FLASH_ATTN_ERR_ARG;
    if ((st = check_scale(scale)) != FLASH_ATTN_OK) return st;
    float tau;
    int tile_cfg;
    if ((st = check_opts(opts, &tau, &tile_cfg)) != FLASH_ATTN_OK) return st;
    if (is_empty(layout)) return FLASH_ATTN_OK;
    if (!q || !k || !v || !o || !lse) return FLASH_ATTN_ERR_NULL;
    const int64_t eb = (dtype == FLASH_ATTN_F32) ? 4 : 2;
    if ((st = check_strides(layout, eb)) != FLASH_ATTN_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return FLASH_ATTN_ERR_LAYOUT;

    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.sb = layout.stride_b; a.sh = layout.stride_h; a.ss = layout.stride_s;
    a.B = static_cast<int32_t>(layout.batch);
    a.H = static_cast<int32_t>(layout.heads);
    a.N = static_cast<int32_t>(layout.seqlen);
    a.D = static_cast<int32_t>(layout.head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.tau = tau;
    a.causal = causal;
    a.tile_cfg = tile_cfg;
    const int err = (dtype == FLASH_ATTN_BF16) ? fa::launch_fwd_bf16(a, stream)
                                               : fa::launch_fwd_f32(a, stream);
    return hip_status(err);
}

flash_attn_status flash_attn_fp8_quantize(const void* x, flash_attn_dtype in_dtype,
                                          flash_attn_layout layout, flash_attn_fp8_role role,
                                          int rotate, const int8_t* signs,
                                          uint8_t* x_fp8, float* scales, void* stream) {
    flash_attn_status st = check_shape(layout);
    if (st != FLASH_ATTN_OK) return st;
    if (in_dtype != FLASH_ATTN_F32 && in_dtype != FLASH_ATTN_BF16) return FLASH_ATTN_ERR_DTYPE;
    if (role != FLASH_ATTN_FP8_Q && role != FLASH_ATTN_FP8_K && role != FLASH_ATTN_FP8_V)
        return FLASH_ATTN_ERR_ARG;
    if (rotate != 0 && rotate != 1) return FLASH_ATTN_ERR_ARG;
    if (rotate && role == FLASH_ATTN_FP8_V) return FLASH_ATTN_ERR_ARG;
    if (is_empty(layout)) return FLASH_ATTN_OK;
    if (!x || !x_fp8 || !scales || (rotate && !signs)) return FLASH_ATTN_ERR_NULL;
    const int64_t eb = (in_dtype == FLASH_ATTN_F32) ? 4 : 2;
    if ((st = check_strides(layout, eb)) != FLASH_ATTN_OK) return st;
    if (!aligned16(x) || !aligned16(x_fp8) || (reinterpret_cast<uintptr_t>(scales) & 3u))
        return FLASH_ATTN_ERR_LAYOUT;
    fa::QuantArgs a;
    a.x = x; a.in_bf16 = (in_dtype == FLASH_ATTN_BF16);
    a.sb = layout.stride_b; a.sh = layout.stride_h; a.ss = layout.stride_s;
    a.B = static_cast<int32_t>(layout.batch);
    a.H = static_cast<int32_t>(layout.heads);
    a.N = static_cast<int32_t>(layout.seqlen);
    a.D = static_cast<int32_t>(layout.head_dim);
    a.role = static_cast<int32_t>(role);
    a.rotate = rotate; a.signs = signs;
    a.out = x_fp8; a.scales = scales;
    return hip_status(fa::launch_fp8_quantize(a, stream));
}

size_t flash_attn_fp8_buffer_bytes(flash_attn_layout layout, flash_attn_fp8_role role) {
    if (layout.batch < 0 || layout.heads < 0 || layout.seqlen < 0 || layout.head_dim < 0) return 0;
    if (role != FLASH_ATTN_FP8_Q && role != FLASH_ATTN_FP8_K && role != FLASH_ATTN_FP8_V) return 0;
    const int64_t rows = (role == FLASH_ATTN_FP8_V) ? fa::fp8_npad(layout.seqlen) : layout.seqlen;
    const int64_t planes = (role == FLASH_ATTN_FP8_Q) ? 2 : 1;   // Q: the code and its residual term
    return static_cast<size_t>(planes * layout.batch * layout.heads * rows * layout.head_dim);
}

int64_t flash_attn_fp8_num_scales(flash_attn_layout layout, flash_attn_fp8_role role) {
    if (layout.batch < 0 || layout.heads < 0 || layout.seqlen < 0) return 0;
    int64_t blk;
    switch (role) {
        case FLASH_ATTN_FP8_Q: blk = fa::kFp8QBlock; break;
        case FLASH_ATTN_FP8_K: blk = fa::kFp8KBlock; break;
        case FLASH_ATTN_FP8_V: blk = fa::kFp8VBlock; break;
        default: return 0;
    }
    return layout.batch * layout.heads * ((layout.seqlen + blk - 1) / blk);
}

flash_attn_status flash_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                     const float* q_scale, const float* k_scale,
                                     const float* v_scale, void* o, float* lse,
                                     flash_attn_layout o_layout, int causal, float scale,
                                     const flash_attn_fwd_opts* opts, void* stream) {
    flash_attn_status st = check_shape(o_layout);
    if (st != FLASH_ATTN_OK) return st;
    if (causal != 0 && causal != 1) return FLASH_ATTN_ERR_ARG;
    if ((st = check_scale(scale)) != FLASH_ATTN_OK) return st;
    float tau;
    int tile_cfg, q_terms;
    if ((st = check_opts(opts, &tau, &tile_cfg, &q_terms)) != FLASH_ATTN_OK) return st;
    if (is_empty(o_layout)) return FLASH_ATTN_OK;
    if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o || !lse)
        return FLASH_ATTN_ERR_NULL;
    if ((st = check_strides(o_layout, 2)) != FLASH_ATTN_OK) return st;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(q_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(k_scale) & 3u) || (reinterpret_cast<uintptr_t>(v_scale) & 3u))
        return FLASH_ATTN_ERR_LAYOUT;
    fa::Fp8Args a;
    a.q = q8; a.k = k8; a.vt = v8t; a.qs = q_scale; a.ks = k_scale; a.vs = v_scale;
    a.o = o; a.lse = lse;
    a.osb = o_layout.stride_b; a.osh = o_layout.stride_h; a.oss = o_layout.stride_s;
    a.B = static_cast<int32_t>(o_layout.batch);
    a.H = static_cast<int32_t>(o_layout.heads);
    a.N = static_cast<int32_t>(o_layout.seqlen);
    a.D = static_cast<int32_t>(o_layout.head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.tau = fminf(tau, 2.5f);  // 64 * 2^tau must stay below 448
    a.causal = causal;
    a.tile_cfg = tile_cfg;
    a.q_terms = q_terms;
    return hip_status(fa::launch_fwd_fp8(a, stream));
}

size_t flash_attn_bwd_workspace_size(flash_attn_layout layout, flash_attn_dtype dtype) {
    if (check_shape(layout) != FLASH_ATTN_OK || (dtype != FLASH_ATTN_BF16 && dtype != FLASH_ATTN_F32))
        return 0;
    if (is_empty(layout)) return 0;
    return static_cast<size_t>(
        fa::bwd_workspace_bytes(layout.batch, layout.heads, layout.seqlen));
}

}  // extern "C"

namespace {

// Validation and dispatch shared by both backward entry points.  With
// from_scratch the workspace is the library's fixed device array instead of
// the caller's (no allocation either way).
flash_attn_status bwd_impl(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           flash_attn_layout layout, flash_attn_dtype dtype, int causal,
                           float scale, void* workspace, size_t workspace_bytes,
                           bool from_scratch, void* stream) {
    flash_attn_status st = check_shape(layout);
    if (st != FLASH_ATTN_OK) return st;
    if (dtype != FLASH_ATTN_BF16 && dtype != FLASH_ATTN_F32) return FLASH_ATTN_ERR_DTYPE;
    if (causal != 0 && causal != 1) return FLASH_ATTN_ERR_ARG;
    if ((st = check_scale(scale)) != FLASH_ATTN_OK) return st;
    if (is_empty(layout)) return FLASH_ATTN_OK;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FLASH_ATTN_ERR_NULL;
    if ((st = check_strides(layout, dtype == FLASH_ATTN_F32 ? 4 : 2)) != FLASH_ATTN_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return FLASH_ATTN_ERR_LAYOUT;
    const int64_t need = fa::bwd_workspace_bytes(layout.batch, layout.heads, layout.seqlen);
    if (from_scratch) {
        if (need > fa::kScratchBytes) return FLASH_ATTN_ERR_WORKSPACE;
        const int err = fa::scratch_buffer(&workspace);
        if (err) return hip_status(err);
        workspace_bytes = static_cast<size_t>(fa::kScratchBytes);
    }
    if (!workspace || workspace_bytes < static_cast<size_t>(need) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return FLASH_ATTN_ERR_WORKSPACE;
    fa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.sb = layout.stride_b; a.sh = layout.stride_h; a.ss = layout.stride_s;
    a.B = static_cast<int32_t>(layout.batch);
    a.H = static_cast<int32_t>(layout.heads);
    a.N = static_cast<int32_t>(layout.seqlen);
    a.D = static_cast<int32_t>(layout.head_dim);
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.causal = causal;
    char* ws = static_cast<char*>(workspace);
    const int64_t rows = layout.batch * layout.heads * layout.seqlen;
    a.ws_lse2 = reinterpret_cast<float*>(ws);
    a.ws_nd = reinterpret_cast<float*>(ws + fa::bwd_ws_part(rows));
    return hip_status(dtype == FLASH_ATTN_BF16 ? fa::launch_bwd_bf16(a, stream) : fa::launch_bwd_f32(a, stream));
}

}  // namespace

extern "C" {

flash_attn_status flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 flash_attn_layout layout, flash_attn_dtype dtype, int causal,
                                 float scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, layout, dtype, causal, scale, workspace,
                    workspace_bytes, false, stream);
}

flash_attn_status flash_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                         const void* o, const float* lse, const void* dout,
                                         void* dq, void* dk, void* dv, flash_attn_layout layout,
                                         flash_attn_dtype dtype, int causal, float scale,
                                         void* stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, layout, dtype, causal, scale, nullptr, 0,
                    true, stream);
}

flash_attn_status flash_attn_merge(const void* o_parts, const float* lse_parts, int64_t n_parts,
                                   int64_t part_stride, void* o, float* lse,
                                   flash_attn_layout layout, flash_attn_dtype dtype, void* stream) {
    flash_attn_status st = check_shape(layout);
    if (st != FLASH_ATTN_OK) return st;
    if (dtype != FLASH_ATTN_F32 && dtype != FLASH_ATTN_BF16) return FLASH_ATTN_ERR_DTYPE;
    if (n_parts < 1 || n_parts > kMaxMergeParts) return FLASH_ATTN_ERR_ARG;
    if (is_empty(layout)) return FLASH_ATTN_OK;
    if (!o_parts || !lse_parts || !o || !lse) return FLASH_ATTN_ERR_NULL;
    const int64_t eb = (dtype == FLASH_ATTN_F32) ? 4 : 2;
    if ((st = check_strides(layout, eb)) != FLASH_ATTN_OK) return st;
    if (n_parts > 1 && (part_stride <= 0 || part_stride % (16 / eb))) return FLASH_ATTN_ERR_LAYOUT;
    if (!aligned16(o_parts) || !aligned16(o) || (reinterpret_cast<uintptr_t>(lse_parts) & 3u) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return FLASH_ATTN_ERR_LAYOUT;
    fa::MergeArgs a;
    a.o_parts = o_parts; a.lse_parts = lse_parts; a.o = o; a.lse = lse;
    a.sb = layout.stride_b; a.sh = layout.stride_h; a.ss = layout.stride_s;
    a.part_stride = part_stride;
    a.B = static_cast<int32_t>(layout.batch);
    a.H = static_cast<int32_t>(layout.heads);
    a.N = static_cast<int32_t>(layout.seqlen);
    a.D = static_cast<int32_t>(layout.head_dim);
    a.S = static_cast<int32_t>(n_parts);
    a.bf16 = (dtype == FLASH_ATTN_BF16);
    return hip_status(fa::launch_merge(a, stream));
}

const char* flash_attn_status_str(flash_attn_status s) {
    switch (s) {
        case FLASH_ATTN_OK: return "FLASH_ATTN_OK";
        case FLASH_ATTN_ERR_NULL: return "FLASH_ATTN_ERR_NULL";
        case FLASH_ATTN_ERR_SHAPE: return "FLASH_ATTN_ERR_SHAPE";
        case FLASH_ATTN_ERR_LAYOUT: return "FLASH_ATTN_ERR_LAYOUT";
        case FLASH_ATTN_ERR_DTYPE: return "FLASH_ATTN_ERR_DTYPE";
        case FLASH_ATTN_ERR_UNSUPPORTED: return "FLASH_ATTN_ERR_UNSUPPORTED";
        case FLASH_ATTN_ERR_ARG: return "FLASH_ATTN_ERR_ARG";
        case FLASH_ATTN_ERR_WORKSPACE: return "FLASH_ATTN_ERR_WORKSPACE";
        case FLASH_ATTN_ERR_HIP: return "FLASH_ATTN_ERR_HIP";
    }
    return "FLASH_ATTN_ERR_UNKNOWN";
}

const char* flash_attn_last_error(void) { return g_last_error; }

int flash_attn_abi_version(void) { return FLASH_ATTN_ABI_VERSION; }

}  // extern "C"
