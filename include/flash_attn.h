/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * What is computed.  For every batch b, head h and query row i:
 *     s_ij  = scale * <q_i, k_j>                  (j allowed)
 *     P_ij  = exp(s_ij - m_i) / l_i,   m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
 *     o_i   = sum_j P_ij v_j,          LSE_i = m_i + ln(l_i)   (natural log)
 * i.e. O = softmax(scale * Q K^T) V plus the per-row log-sum-exp, as defined in
 * "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析" sec. 2.1
 * (standard attention), sec. 6.1-6.3 (safe / online softmax, the rescaling
 * identity) and sec. 7.2 (the forward keeps only O and the row statistics for
 * the backward).  "causal" applies the lower-triangular mask of that page's
 * sec. 11.3: key j is allowed for query i iff j <= i.  The N x N score matrix
 * never reaches device memory: the kernels tile K/V and keep the running
 * maximum and sum on chip (sec. 5, 6.2; FlashAttention-2 loop order, sec. 8.2).
 *
 * Conventions shared by every entry point.
 *  - Pointers to tensors are DEVICE pointers owned by the caller; the library
 *    allocates no device memory and never synchronises: work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and the caller
 *    synchronises.  Its only state is a per-thread last-error message and a
 *    kernel attribute (the bf16 forward's LDS size) set once per process, so
 *    concurrent calls from several host threads are safe.
 *  - Arguments are validated on the host before any HIP call; on any error
 *    return nothing is enqueued and the outputs are untouched.  A failed kernel
 *    launch returns FLASH_ATTN_ERR_HIP; flash_attn_last_error() then describes it.
 *  - Q, K, V and O share one flash_attn_layout: element (b, h, i, c) lives at
 *    base + b*stride_b + h*stride_h + i*stride_s + c (strides in elements, the
 *    head_dim stride is 1).  This expresses both [B, H, N, d] and [B, N, H, d].
 *    Base pointers must be 16-byte aligned and the strides multiples of
 *    16 bytes' worth of elements (8 for bf16, 4 for f32, 16 for fp8);
 *    stride_s is at most 2^24 elements (rows of a tile are addressed with
 *    32-bit offsets).
 *  - LSE is always a contiguous fp32 [B, H, N] array.
 *  - Inputs must be finite.  A NaN or infinite element of Q, K or V leaves the
 *    outputs of the rows that use it (and possibly of other rows whose key
 *    tile contains it) unspecified: the attention kernels are compiled
 *    assuming no NaN operands, which lets a row maximum be one v_max3 per two
 *    scores.  Rows that never load that tile are unaffected.
 *  - Supported v1: head_dim 64 or 128; seqlen_q == seqlen_k == seqlen.
 *    A zero batch, heads or seqlen is a valid empty call (returns OK, no work;
 *    pointers may then be NULL).
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLASH_ATTN_ABI_VERSION 2

typedef enum flash_attn_status {
    FLASH_ATTN_OK = 0,
    FLASH_ATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
    FLASH_ATTN_ERR_SHAPE = 2,       /* a size is negative or beyond the limits below  */
    FLASH_ATTN_ERR_LAYOUT = 3,      /* strides / alignment not supported              */
    FLASH_ATTN_ERR_DTYPE = 4,       /* dtype not accepted by this entry point         */
    FLASH_ATTN_ERR_UNSUPPORTED = 5, /* valid request the library does not implement  */
    FLASH_ATTN_ERR_ARG = 6,         /* scale / option value out of range              */
    FLASH_ATTN_ERR_WORKSPACE = 7,   /* workspace missing or too small                 */
    FLASH_ATTN_ERR_HIP = 8          /* the HIP runtime reported an error              */
} flash_attn_status;

typedef enum flash_attn_dtype {
    FLASH_ATTN_F32 = 0,             /* IEEE binary32                                  */
    FLASH_ATTN_BF16 = 1,            /* bfloat16                                       */
    FLASH_ATTN_FP8_E4M3 = 2         /* OCP FP8 E4M3FN (bias 7, max 448, no inf)        */
} flash_attn_dtype;

/* Shape and strides (in elements) shared by Q, K, V and O.
 * Limits: 0 <= batch*heads <= 2^24, 0 <= seqlen <= 2^24 and
 * batch*heads*seqlen < 2^31 (beyond any tensor the device can hold). */
typedef struct flash_attn_layout {
    int64_t batch, heads, seqlen, head_dim;
    int64_t stride_b, stride_h, stride_s;
} flash_attn_layout;

/* Optional tuning knobs (pass NULL for the defaults).
 * tau_log2: conditional-rescale threshold in log2 units ("FlashAttention-4"
 *   explainer, sec. 論文 Section 3.3: the running output is rescaled only when
 *   the running maximum grows by more than tau).  The result does not depend
 *   on tau (the rescaling identity, FlashAttention page sec. 6.3) beyond fp32
 *   rounding; unnormalised probabilities stay below 2^tau.  Range [0, 64];
 *   a negative value selects the default 8.
 * tile_cfg: 0 = automatic (bf16: 4-wave workgroups of 128 query rows for
 *   head_dim 64, 8-wave workgroups of 256 rows for 128; f32: 8 waves unless
 *   that grid has fewer than 512 workgroups, then 4); 1 and 2 force the 8-
 *   and 4-wave forms of the bf16 and f32 kernels; any other value is an
 *   argument error.  The result does not depend on it beyond fp32 summation
 *   order.
 * fp8_q_terms: flash_attn_fwd_fp8 only (ignored elsewhere): 0 or 2 = use both
 *   e4m3 terms of Q (the default: Q K^T then carries only K's rounding), 1 =
 *   Q's first term only (four fewer fp8 products per 64-key tile at d = 128,
 *   about 11 % faster, the error of a single e4m3 rounding of Q); other
 *   values are an argument error. */
typedef struct flash_attn_fwd_opts {
    float tau_log2;
    int32_t tile_cfg;
    int32_t fp8_q_terms;
} flash_attn_fwd_opts;

/*
 * Forward attention, fp32 or bf16 in and out.
 *   q, k, v : [layout] tensors of `dtype` (read only)
 *   o       : [layout] output of `dtype` (bf16 outputs are rounded to nearest even)
 *   lse     : fp32 [batch, heads, seqlen] natural-log log-sum-exp of the scaled scores
 *   causal  : 0 or 1 (lower-triangular mask, key j <= query i)
 *   scale   : multiplies Q K^T; finite and > 0 (the usual value is 1/sqrt(head_dim))
 * Errors: NULL -> ERR_NULL; sizes -> ERR_SHAPE; head_dim not 64/128 ->
 * ERR_UNSUPPORTED; strides/alignment -> ERR_LAYOUT; dtype other than F32/BF16
 * -> ERR_DTYPE; scale or opts out of range -> ERR_ARG.
 */
flash_attn_status flash_attn_fwd(const void* q, const void* k, const void* v,
                                 void* o, float* lse,
                                 flash_attn_layout layout, flash_attn_dtype dtype,
                                 int causal, float scale,
                                 const flash_attn_fwd_opts* opts, void* stream);

/*
 * FP8 pre-pass ("FlashAttention-3: Fast and Accurate Attention with Asynchrony
 * and Low-precision", sec. 技術 3, accuracy part): optional incoherent
 * processing x -> (x * signs) H_d / sqrt(d) (Sylvester Hadamard H_d, applied as
 * a fast Walsh-Hadamard transform), then block quantisation: rows of one
 * (batch, head) are grouped in blocks of consecutive rows, each block gets one
 * fp32 scale and every element becomes e4m3(x / scale) (round to nearest even,
 * saturating at +-448).  The role fixes the block size, the scale rule and the
 * output layout the fp8 attention kernel consumes:
 *   Q: blocks of 32 rows, scale = amax(block)/448 (1 for an all-zero block),
 *      output two contiguous planes [2][B, H, N, d]: plane 0 holds
 *      hi = e4m3(x / scale), plane 1 the residual term
 *      lo = e4m3(16 (x / scale - hi)), so that x = scale (hi + lo / 16) to
 *      about 2^-8 relative (the attention kernel applies the 1/16 as a matrix
 *      core operand scale; Q K^T then carries the error of K's single term
 *      only);
 *   K: blocks of 32 rows, same scale rule, output contiguous [B, H, N, d];
 *   V: blocks of 64 rows, scale = the smallest power of two >= amax/448 (so the
 *      matrix cores apply it as an exponent), never rotated, output TRANSPOSED
 *      contiguous [B, H, d, N_pad] with N_pad = ceil(N / 64) * 64 (pad columns 0).
 * Q and K must use the same signs (or both rotate = 0): the rotation is
 * orthogonal, so Q K^T is unchanged and V needs no inverse rotation.
 *   x      : [layout] F32 or BF16 input (`in_dtype`)
 *   rotate : 1 = apply the rotation (Q, K only), 0 = none
 *   signs  : device int8[head_dim] of +1/-1 (ignored when rotate == 0)
 *   x_fp8  : output, flash_attn_fp8_buffer_bytes(layout, role) bytes
 *   scales : output, fp32, flash_attn_fp8_num_scales(layout, role) entries,
 *            [B, H, ceil(N / block)]
 * Errors: as flash_attn_fwd, plus ERR_ARG for an unknown role or rotate on V.
 */
typedef enum flash_attn_fp8_role {
    FLASH_ATTN_FP8_Q = 0,
    FLASH_ATTN_FP8_K = 1,
    FLASH_ATTN_FP8_V = 2
} flash_attn_fp8_role;

flash_attn_status flash_attn_fp8_quantize(const void* x, flash_attn_dtype in_dtype,
                                          flash_attn_layout layout, flash_attn_fp8_role role,
                                          int rotate, const int8_t* signs,
                                          uint8_t* x_fp8, float* scales, void* stream);

/* Bytes of the e4m3 buffer and number of fp32 scales the pre-pass writes for a
 * tensor of this shape and role (0 for an invalid role or negative sizes). */
size_t flash_attn_fp8_buffer_bytes(flash_attn_layout layout, flash_attn_fp8_role role);
int64_t flash_attn_fp8_num_scales(flash_attn_layout layout, flash_attn_fp8_role role);

/*
 * FP8 forward attention ("FlashAttention-3: Fast and Accurate Attention with
 * Asynchrony and Low-precision", sec. 技術 3: e4m3 operands with per-block
 * scales, which a blockwise kernel applies at no extra cost; the exp cost
 * relative to the doubled matrix rate is the point of its 考察) on the
 * pre-pass outputs: e4m3 Q (the two planes [2][B, H, N, d]), K (contiguous
 * [B, H, N, d]) and V (transposed [B, H, d, N_pad]) with their block scales;
 * the matrix products run on the fp8 matrix cores with fp32 accumulation.  Q/K
 * block scales fold into the softmax exponent, the power-of-two V scales and
 * the 1/16 of Q's residual term are applied by the matrix cores, and the
 * probabilities enter the second product as e4m3(64 p) (p <= 2^2.5: tau is
 * capped at 2.5 here).  The row sum adds the same e4m3 values that multiply V
 * (so O is normalised by the sum of its own weights), on the matrix core.
 * O is bf16 with the strides of `o_layout`, whose batch, heads, seqlen and
 * head_dim give the shape of everything; LSE is fp32 [B, H, N], the natural
 * log of that row sum (within ln(1 + 2^-4) of the exact one of the
 * quantised scores).
 */
flash_attn_status flash_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                     const float* q_scale, const float* k_scale,
                                     const float* v_scale,
                                     void* o, float* lse, flash_attn_layout o_layout,
                                     int causal, float scale,
                                     const flash_attn_fwd_opts* opts, void* stream);

/*
 * Backward pass, bf16 or fp32.  Gradients of the forward above with respect to Q, K
 * and V for the upstream gradient dO.  The pages give no backward formulas;
 * this is the analytic derivative of the definition (s = scale Q K^T, P =
 * softmax(s) per row, P_ij = exp(s_ij - LSE_i)):
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q.
 * As in "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
 * sec. 7.2, S and P are recomputed tile by tile on chip from Q, K and the
 * forward's LSE; nothing N x N is stored.  bf16: probabilities and dS enter
 * the matrix products as bf16, accumulation is fp32; fp32: every product and
 * sum is fp32.
 *   q, k, v, o, dout : [layout] of `dtype` (o and lse are the forward's outputs)
 *   lse              : fp32 [batch, heads, seqlen] from flash_attn_fwd
 *   dq, dk, dv       : [layout] outputs of `dtype` (bf16: rounded to nearest even)
 *   causal, scale    : as given to the forward
 *   workspace        : device memory of at least
 *                      flash_attn_bwd_workspace_size(layout, dtype) bytes
 *                      (two fp32 values per query row), 256-byte aligned,
 *                      owned by the caller; its contents on entry do not
 *                      matter and are overwritten.
 * The result is deterministic: dK/dV are summed over query tiles and dQ over
 * key tiles inside one workgroup each, in a fixed order (no atomics).
 * Errors: as flash_attn_fwd; a dtype other than BF16 or F32 -> ERR_DTYPE;
 * workspace NULL, too small or misaligned -> ERR_WORKSPACE.
 */
flash_attn_status flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout,
                                 void* dq, void* dk, void* dv,
                                 flash_attn_layout layout, flash_attn_dtype dtype,
                                 int causal, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes flash_attn_bwd needs for this shape and dtype (0 for an
 * empty shape, an invalid one or a dtype the backward does not accept). */
size_t flash_attn_bwd_workspace_size(flash_attn_layout layout, flash_attn_dtype dtype);

/*
 * flash_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid hipMalloc.  The two fp32 values
 * per query row that flash_attn_bwd keeps in the caller's workspace live in
 * a fixed device array of the library instead (16 MiB per GPU, held until
 * the process ends; its address is looked up once per device, with that
 * device current).  The call allocates nothing.
 *   Arguments, results and errors: as flash_attn_bwd (the result is the same,
 *   bit for bit); the stream must belong to the current device.
 *   Limit: batch * heads * seqlen <= 2^21 rows; larger shapes return
 *   FLASH_ATTN_ERR_WORKSPACE (use flash_attn_bwd with a workspace).
 *   Every call on one GPU shares the array: calls that overlap on one GPU
 *   (several streams or host threads at once) race and must be serialised by
 *   the caller.
 */
flash_attn_status flash_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                                         const void* o, const float* lse, const void* dout,
                                         void* dq, void* dk, void* dv,
                                         flash_attn_layout layout, flash_attn_dtype dtype,
                                         int causal, float scale, void* stream);

/*
 * Merge of attention results over disjoint key sets (the combine step of
 * attention sharded along the sequence).  Part s holds, for every row, the
 * normalised output O_s over its keys and the natural-log LSE_s of its scaled
 * scores, as flash_attn_fwd returns them.  The result over the union of the
 * keys is
 *     LSE = ln sum_s exp(LSE_s),    O = sum_s exp(LSE_s - LSE) O_s,
 * the rescale-and-add update of the online softmax
 * ("FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析" sec. 6.2,
 * exact by the rescaling identity of sec. 6.3) applied to whole parts.  A
 * part with LSE_s = -inf (no key) contributes nothing; a row with no key in
 * any part gets O = 0 and LSE = -inf.
 *   o_parts     : n_parts tensors of `dtype` (F32 or BF16), part s at
 *                 o_parts + s * part_stride elements, each with `layout`
 *   lse_parts   : fp32 contiguous [n_parts, batch, heads, seqlen]
 *   n_parts     : 1 .. 4096
 *   part_stride : elements between parts (> 0 and a multiple of 16 bytes'
 *                 worth when n_parts > 1)
 *   o, lse      : outputs, o with `layout` and `dtype`, lse fp32 [B, H, N]
 * Errors: as flash_attn_fwd; n_parts out of range -> ERR_ARG; bad
 * part_stride -> ERR_LAYOUT.
 */
flash_attn_status flash_attn_merge(const void* o_parts, const float* lse_parts, int64_t n_parts,
                                   int64_t part_stride, void* o, float* lse,
                                   flash_attn_layout layout, flash_attn_dtype dtype, void* stream);

/* Human-readable name of a status code (static string). */
const char* flash_attn_status_str(flash_attn_status s);

/* Detail of the last FLASH_ATTN_ERR_HIP on the calling thread ("" if none). */
const char* flash_attn_last_error(void);

/* FLASH_ATTN_ABI_VERSION of the built library. */
int flash_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
