// fp8.hip -- FP8 (OCP e4m3fn) path for gfx950: block-quantising pre-pass with
// incoherent processing, and attention on the fp8 matrix cores.
//
// Method ("FlashAttention-3: Fast and Accurate Attention with Asynchrony and
// Low-precision", sec. 技術 3): Q, K and V are quantised per block of rows with
// one scale each, which a blockwise attention kernel applies at no extra
// cost; before quantising, Q and K are multiplied by M = diag(+-1) H_d / sqrt(d)
// (H_d a Sylvester Hadamard matrix) so that outliers spread over a row; M is
// orthogonal, so (QM)(KM)^T = QK^T.  The attention itself is the tiled online
// softmax of "FlashAttention: GPUメモリ階層を活用したアテンション最適化の分析"
// (sec. 5, 6.2, 8) with fp32 accumulation.
//
// gfx950 mapping:
//  * pre-pass: one workgroup per (batch, head, row block); a row is spread over
//    D/32 lanes (32 elements each); the fast Walsh-Hadamard transform does its
//    five in-lane stages and log2(D/32) cross-lane stages with DPP permutes;
//    conversion uses v_cvt_pk_fp8_f32 (round to nearest even) on values clamped
//    to +-448, which gives the saturating e4m3fn encoding.  Q also gets a
//    second e4m3 term, 16 times its rounding residual (Q = scale (code +
//    residual / 16)), which the attention kernel can add as a second score
//    product.
//    V is written
//    transposed ([d][keys], padded to 64 keys) through an LDS tile, so the
//    attention kernel's PV operand is a plain contiguous LDS read.
//  * attention: like the bf16 kernel, a wave owns 32 queries and computes the
//    transposed score tile S^T = K Q^T, now with v_mfma_scale_f32_32x32x64_f8f6f4
//    (K = 64 fp8 per step).  K rows enter the product in an order that leaves,
//    in lane half h, exactly keys 32h .. 32h+31 of the 64-key tile, so the
//    packed fp8 probabilities are the B operand of O^T += V^T P^T directly.
//    With both Q terms the score is the code product plus the residual
//    product, whose E8M0 B-operand scale is 2^-4 (a second MFMA per k-step
//    on the same K operand).
//    Q and K block scales fold into the exp2 constant (the Q block is the
//    wave's 32 rows, the K block the 32 keys a lane half holds, so both are
//    per-lane scalars); the V block scale is a power of two handed to the
//    matrix core as its E8M0 A-operand scale.  Probabilities enter as e4m3(64 p) with p <= 2^tau (tau capped at
//    2.5, so 64 p stays below e4m3's 448); the row sum and O carry the same factor 64, which cancels in O / l
//    and is removed from the LSE.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "lds_copy.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int kQBlk = kFp8QBlock;  // 32 query rows per Q scale (a wave's rows)
constexpr int kKBlk = kFp8KBlock;  // 32 key rows per K scale (one lane half)
constexpr int kVBlk = kFp8VBlock;  // 64 key rows per V scale (= K/V tile)

// ---------------------------------------------------------------------------
// Pre-pass
// ---------------------------------------------------------------------------

// Two floats -> two e4m3fn bytes in the low (HI = false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ int cvt2(float a, float b, int old) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// One workgroup (4 waves) takes RWG consecutive rows of one (b, h); a lane
// holds 32 consecutive elements of one row (LPR = D / 32 lanes per row), so a
// row's Walsh-Hadamard transform is five butterfly stages inside the lane and
// log2(LPR) stages across neighbouring lanes (DPP quad permutes, no LDS).
// A scale block (32 or 64 rows) is one or more whole waves.
template <int D, bool IN_BF16>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(QuantArgs a) {
    constexpr int LPR = D / 32;       // lanes per row
    constexpr int RPW = 64 / LPR;     // rows per wave
    constexpr int RWG = 4 * RPW;      // rows per workgroup
    static_assert(RPW % kQBlk == 0 || kQBlk % RPW == 0, "scale block / wave mismatch");
    __shared__ float red[4];
    // V^T staging: D rows of RWG key bytes; the keys of head-dim chunk c are
    // rotated by 16c bytes so that the byte writes of one instruction spread
    // over the banks (16-byte groups stay contiguous for the row reads).
    __shared__ __attribute__((aligned(16))) uint8_t vt_tile[D * RWG];

    const int blk_rows = (a.role == 0) ? kQBlk : (a.role == 1) ? kKBlk : kVBlk;
    const int nblk = (a.N + blk_rows - 1) / blk_rows;
    const int nwg = (a.N + RWG - 1) / RWG;
    const int bh = __builtin_amdgcn_workgroup_id_x() / nwg, g = __builtin_amdgcn_workgroup_id_x() % nwg;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63, wave = tid >> 6;
    const int c = lane % LPR;                    // columns 32c .. 32c+31
    const int rw = wave * RPW + lane / LPR;      // row inside the workgroup
    const int row = g * RWG + rw;
    const int64_t xoff = int64_t(b) * a.sb + int64_t(h) * a.sh + int64_t(row) * a.ss + 32 * c;

    float x[32];
    if (row < a.N) {
        if (IN_BF16) {
            const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + xoff);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 r = p[i];
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
                    x[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + xoff);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 r = p[i];
                x[4 * i] = r.x; x[4 * i + 1] = r.y; x[4 * i + 2] = r.z; x[4 * i + 3] = r.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }

    if (a.rotate) {
        // signs of columns 32c .. 32c+31 (byte loads: the vector may have any alignment)
        const int8_t* sp = a.signs + 32 * c;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (sp[i] < 0) x[i] = -x[i];
        // butterflies on index bits 0-4 (inside the lane): (u, v) -> (u + v, u - v)
#pragma unroll
        for (int m = 1; m < 32; m <<= 1)
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (!(i & m)) {
                    const float u = x[i], v = x[i + m];
                    x[i] = u + v;
                    x[i + m] = u - v;
                }
        // index bits 5 and 6: the partner row chunk is lane ^ 1 (and lane ^ 2)
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) {
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int xi = __float_as_int(x[i]);
                const int o = (m == 1) ? __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false)    // quad_perm 1,0,3,2
                                       : __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
                x[i] = upper ? (__int_as_float(o) - x[i]) : (x[i] + __int_as_float(o));
            }
        }
        const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] *= inv_sqrt_d;
    }

    // absolute maximum of each scale block: lane, wave, then the block's waves
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    const int wpb = blk_rows >= RPW ? blk_rows / RPW : 1;   // waves per scale block
    const int w0 = (wave / wpb) * wpb;
    amax = red[w0];
    for (int w = w0 + 1; w < w0 + wpb; ++w) amax = fmaxf(amax, red[w]);
    float scale = (amax > 0.f) ? amax / 448.f : 1.f;
    if (a.role == 2 && amax > 0.f) {  // power-of-two ceiling for V
        int e;
        const float m = frexpf(scale, &e);
        scale = (m == 0.5f) ? scale : ldexpf(1.f, e);
    }
    const int blk = row / blk_rows;
    if (rw % blk_rows == 0 && c == 0 && blk < nblk) a.scales[int64_t(bh) * nblk + blk] = scale;
    const float rcp = 1.0f / scale;

    uint32_t wq[8];   // e4m3 codes of the lane's 32 elements, 4 per word
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int lo = cvt2<false>(x[4 * i] * rcp, x[4 * i + 1] * rcp, 0);
        wq[i] = static_cast<uint32_t>(cvt2<true>(x[4 * i + 2] * rcp, x[4 * i + 3] * rcp, lo));
    }

    if (a.role != 2) {
        if (row < a.N) {
            uint4* op = reinterpret_cast<uint4*>(a.out + (int64_t(bh) * a.N + row) * D + 32 * c);
            op[0] = make_uint4(wq[0], wq[1], wq[2], wq[3]);
            op[1] = make_uint4(wq[4], wq[5], wq[6], wq[7]);
        }
        if (a.role == 0) {
            // Q: a second e4m3 term for the rounding residual, in units of
            // 2^-4 of the scaled value: lo = e4m3(16 (y - hi)), |16 (y - hi)|
            // <= 256 (half an e4m3 step is at most 2^-4 |y| and |y| <= 448),
            // so Q = scale (hi + lo / 16) to about 2^-8 relative.
            uint32_t wl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // decoded hi values: bytes 0-1 and 2-3 of the word
                const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wq[i]), false);
                const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(wq[i]), true);
                const float hv[4] = {h01[0], h01[1], h23[0], h23[1]};
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = fminf(fmaxf(x[4 * i + e] * rcp, -448.f), 448.f);
                    r[e] = (y - hv[e]) * 16.f;
                }
                const int lo = cvt2<false>(r[0], r[1], 0);
                wl[i] = static_cast<uint32_t>(cvt2<true>(r[2], r[3], lo));
            }
            if (row < a.N) {   // the second plane follows the first: [2][B, H, N, D]
                uint4* lp = reinterpret_cast<uint4*>(a.out + int64_t(a.B) * a.H * a.N * D +
                                                     (int64_t(bh) * a.N + row) * D + 32 * c);
                lp[0] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
                lp[1] = make_uint4(wl[4], wl[5], wl[6], wl[7]);
            }
        }
        return;
    }
    // V: [D][RWG] bytes through LDS (rows past N hold zero codes), then rows of
    // V^T written 16 bytes at a time.
    const int col = (rw + 16 * c) % RWG;
#pragma unroll
    for (int i = 0; i < 32; ++i)
        vt_tile[(32 * c + i) * RWG + col] = static_cast<uint8_t>(wq[i >> 2] >> (8 * (i & 3)));
    __syncthreads();
    const int64_t npad = fp8_npad(a.N);
    constexpr int CPRW = RWG / 16;   // 16-byte chunks per staged row
    for (int t = tid; t < D * CPRW; t += 256) {
        const int d = t / CPRW, j = t % CPRW;
        const int64_t k0 = int64_t(g) * RWG + 16 * j;
        if (k0 < npad)
            *reinterpret_cast<uint4*>(a.out + (int64_t(bh) * D + d) * npad + k0) =
                *reinterpret_cast<const uint4*>(vt_tile + d * RWG + (16 * j + 16 * (d / 32)) % RWG);
    }
}

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------

constexpr int BC = kVBlk;   // keys per tile
// s_waitcnt immediate that waits for LDS (and scalar memory) operations only:
// vmcnt and expcnt at their maxima, lgkmcnt 0.
constexpr int kLgkm0 = 0xC07F;
constexpr int WQ = 32;      // query rows per wave

template <int D>
struct Tile8 {
    static constexpr int KBYTES = BC * D;          // K tile [64 keys][D] bytes
    static constexpr int VBYTES = D * BC;          // V^T tile [D][64 keys] bytes
    static constexpr int KCPR = D / 16;            // 16-byte chunks per K row
    // K: the 16 rows read together are keys {0..7, 32..39} (+16 st); the
    // swizzle gives each of them its own bank group.
    __device__ static int kswz(int r) {
        return D == 128 ? (((r >> 1) & 3) | (((r >> 5) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 5) & 1) << 1));
    }
    // V^T: 16 consecutive head-dim rows of 64 bytes.
    __device__ static int vswz(int r) { return (r >> 2) & 3; }
    // A wave's slice: its 32 Q rows (both e4m3 planes, D bytes each) on the
    // way in, its 32 bf16 O rows on the way out.
    static constexpr int SLICE = 32 * D * 2;
    // Q rows of D bytes: lanes of one half-wave read one chunk of 16 rows.
    __device__ static int qswz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
    // O rows of 2 D bytes (the bf16 kernel's K-row swizzle).
    __device__ static int oswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
};

// A-operand row rho of score subtile st loads key
//   32 * ((rho >> 2) & 1) + 16 * st + 4 * (rho >> 3) + (rho & 3)
// so accumulator register g of subtile st in lane half h is key 32h + 16st + g.
__device__ __forceinline__ int krow8(int rho, int st) {
    return 32 * ((rho >> 2) & 1) + 16 * st + 4 * (rho >> 3) + (rho & 3);
}

// A operand of the row-sum product v_mfma_scale_f32_16x16x128_f8f6f4(A, P, 0):
// fed as its B operand, the probabilities of lane l (query l % 32, keys of
// lane half l / 32) are column l % 16 of K-block l / 16 (32 values each).  A
// row m holds e4m3 ones (0x38) in the K-blocks whose parity is that of m / 4
// when m % 4 == 0, zeros elsewhere, so output row 4g, column c -- register 0
// of lane 16g + c -- sums both lane halves of query (16g + c) % 32: every lane
// receives its own query's row sum over the 64-key tile.
__device__ __forceinline__ i32x8 rowsum_ones8(int lane) {
    const int m = lane & 15, kb = lane >> 4;
    const int w = ((m & 3) == 0 && ((m >> 2) & 1) == (kb & 1)) ? 0x38383838 : 0;
    return i32x8{w, w, w, w, w, w, w, w};
}

__device__ __forceinline__ float pair_max8(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum8(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int NW, bool CAUSAL, int QTERMS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(Fp8Args a) {
    using TL = Tile8<D>;
    constexpr int BR = NW * WQ;
    constexpr int KS = D / 64;   // k-steps of the score product
    constexpr int DT = D / 32;   // head-dim tiles of O^T
    constexpr int NBK = TL::KBYTES / 1024, NBV = TL::VBYTES / 1024;

    // Each LDS buffer is its own object and every access names its buffer at
    // compile time, so the compiler can tell an operand read from a pending
    // direct-to-LDS copy into another buffer and does not make it wait.
    __shared__ __attribute__((aligned(1024))) char lds_k0[TL::KBYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k1[TL::KBYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v0[TL::VBYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v1[TL::VBYTES];
    __shared__ __attribute__((aligned(1024))) char lds_qo[NW * TL::SLICE];

    // One head per XCD; under the causal mask a workgroup takes the query-tile
    // pair (T-1-p, p), so that all workgroups carry the same work.
    const int n_qt = (a.N + BR - 1) / BR;
    const int per_head = CAUSAL ? (n_qt + 1) / 2 : n_qt;
    const int total = per_head * a.B * a.H;
    int id = __builtin_amdgcn_workgroup_id_x();
    if ((total & 7) == 0) {
        const int per = total >> 3;
        id = (id & 7) * per + (id >> 3);
    }
    const int bh = id / per_head, p = id % per_head;
    const int hi = CAUSAL ? n_qt - 1 - p : p;
    const int n_tiles = (CAUSAL && p < hi) ? 2 : 1;
    // The first tile's loads are issued and waited for at its start; the
    // second tile's by the first one's end (the handover below), which also
    // carries its Q block scale and first K/V block scales in these.
    float sq_next = 1.f, ks_next = 1.f, vs_next = 1.f;
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r) {   // one copy of the tile code
        const int qt = r ? p : hi;
        const int b = bh / a.H, h = bh % a.H;
        const int64_t npad = fp8_npad(a.N);
        const uint8_t* Qg = a.q + int64_t(bh) * a.N * D;
        const int64_t q_plane = int64_t(a.B) * a.H * a.N * D;   // offset of Q's residual term
        const uint8_t* Kg = a.k + int64_t(bh) * a.N * D;
        const uint8_t* Vg = a.vt + int64_t(bh) * D * npad;
        uint16_t* Og = static_cast<uint16_t*>(a.o) + int64_t(b) * a.osb + int64_t(h) * a.osh;
        const int nqb = (a.N + kQBlk - 1) / kQBlk, nkb = (a.N + kKBlk - 1) / kKBlk;
        const int nvb = (a.N + kVBlk - 1) / kVBlk;

        const int tid = __builtin_amdgcn_workitem_id_x(), lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int j = lane & 31, hh = lane >> 5;
        const int q0 = qt * BR + wave * WQ;
        const int qi = q0 + j;

        const int n_kt_all = (a.N + BC - 1) / BC;
        const int nt = CAUSAL ? min(n_kt_all, (min(a.N, (qt + 1) * BR) + BC - 1) / BC) : n_kt_all;
        int wnt = CAUSAL ? min(nt, (min(a.N, q0 + WQ) + BC - 1) / BC) : nt;
        if (q0 >= a.N) wnt = 0;

        // Outside the main loop, per-lane addresses start from an opaque copy
        // of the lane index: computed once and shared with the other end of
        // the tile they would stay live across the loop, be spilled, and
        // their reloads would wait for every copy in flight.
        auto fresh_lane = [&]() {
            int l = lane;
            asm volatile("" : "+v"(l));
            return l;
        };
        // direct global -> LDS copies (1 KB per wave instruction, XOR-swizzled
        // rows); l is the lane index (or an opaque copy of it)
        auto copy_k = [&](int kt, char* dst, int l) {
            for (int bk = wave; bk < NBK; bk += NW) {
                const int c = bk * 64 + l;
                const int row = c / TL::KCPR, pch = c % TL::KCPR;
                const int key = min(kt * BC + row, a.N - 1);
                const uint8_t* g = Kg + int64_t(key) * D + 16 * (pch ^ TL::kswz(row));
                copy16_to_lds(g, dst + bk * 1024);
            }
        };
        auto copy_v = [&](int kt, char* dst, int l) {
            for (int bk = wave; bk < NBV; bk += NW) {
                const int c = bk * 64 + l;
                const int row = c / 4, pch = c % 4;  // row = head-dim index
                const uint8_t* g = Vg + int64_t(row) * npad + int64_t(kt) * BC + 16 * (pch ^ TL::vswz(row));
                copy16_to_lds(g, dst + bk * 1024);
            }
        };

        // Q in and O out through the wave's own LDS slice, so that global
        // memory sees whole rows (1 KB copies of Q; 16 bytes of an O row per
        // lane) and only the registers hold the transposed layout.  A wave
        // touches only its own slice: no workgroup barrier is involved.
        char* const qo = lds_qo + wave * TL::SLICE;
        constexpr int QCPR = D / 16;                     // 16-byte chunks per e4m3 row
        constexpr int QBLK = 32 * D / 1024;               // 1 KB copies per plane
        // rows past the end copy the last row (never stored)
        auto copy_q = [&](int t) {
            const int r0 = t * BR + wave * WQ, l = fresh_lane();
    #pragma unroll
            for (int pl = 0; pl < QTERMS; ++pl)
    #pragma unroll
                for (int i = 0; i < QBLK; ++i) {
                    const int c = i * 64 + l, row = c / QCPR, pch = c % QCPR;
                    const uint8_t* g = Qg + pl * q_plane + int64_t(min(r0 + row, a.N - 1)) * D + 16 * (pch ^ TL::qswz(row));
                    copy16_to_lds(g, qo + pl * (32 * D) + i * 1024);
                }
        };
        if (r == 0) {
            copy_q(qt);
            if (nt > 0) {
                copy_k(0, lds_k0, lane);
                copy_v(0, lds_v0, lane);
            }
            if (nt > 1) copy_k(1, lds_k1, lane);
        }

        // Q^T operands: lane (query j, half hh) holds Q[qi][64ks + 32hh .. +31],
        // of the first e4m3 term (qhi) and of the residual term (qlo, which
        // the matrix core scales by 2^-4 through its E8M0 B-operand scale).
        i32x8 qhi[KS], qlo[KS];
        auto read_q = [&]() {
            const int l = fresh_lane(), jj = l & 31, h2 = l >> 5;
    #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const char* rp = qo + jj * D;
                const int c0 = (4 * ks + 2 * h2) ^ TL::qswz(jj), c1 = (4 * ks + 2 * h2 + 1) ^ TL::qswz(jj);
                const uint4 h0 = *reinterpret_cast<const uint4*>(rp + 16 * c0);
                const uint4 h1 = *reinterpret_cast<const uint4*>(rp + 16 * c1);
                qhi[ks] = i32x8{int(h0.x), int(h0.y), int(h0.z), int(h0.w), int(h1.x), int(h1.y), int(h1.z), int(h1.w)};
                uint4 l0 = make_uint4(0, 0, 0, 0), l1 = l0;
                if (QTERMS == 2) {
                    l0 = *reinterpret_cast<const uint4*>(rp + 32 * D + 16 * c0);
                    l1 = *reinterpret_cast<const uint4*>(rp + 32 * D + 16 * c1);
                }
                qlo[ks] = i32x8{int(l0.x), int(l0.y), int(l0.z), int(l0.w), int(l1.x), int(l1.y), int(l1.z), int(l1.w)};
            }
        };
        auto qscale = [&](int t) {   // one value per wave: a wave-uniform index
            const int w0 = t * BR + wave * WQ;
            return (w0 < a.N) ? a.qs[__builtin_amdgcn_readfirstlane(bh * nqb + w0 / kQBlk)] : 1.f;
        };
        const float sq = r ? sq_next : qscale(qt);
        const float c2q = a.scale_log2 * sq;

        f32x16 oacc[DT];
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int g = 0; g < 16; ++g) oacc[dt][g] = 0.f;
        float m_ref = -FLT_MAX;  // log2 units of the true scaled score
        float lsum = 0.f;        // the row's sum of the e4m3 values of 64 p

        // K operand of score subtile st, k-step ks (two 16-byte LDS reads)
        auto k_operand = [&](const char* kt_lds, int st, int ks) -> i32x8 {
            const int row = krow8(j, st);
            const char* rp = kt_lds + row * D;
            const int sw = TL::kswz(row);
            const uint4 lo = *reinterpret_cast<const uint4*>(rp + 16 * ((4 * ks + 2 * hh) ^ sw));
            const uint4 hi = *reinterpret_cast<const uint4*>(rp + 16 * ((4 * ks + 2 * hh + 1) ^ sw));
            return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        };
        // V^T operand of head-dim tile dt
        auto v_operand = [&](const char* vt_lds, int dt) -> i32x8 {
            const int row = 32 * dt + j;
            const char* rp = vt_lds + row * BC;
            const int sw = TL::vswz(row);
            const uint4 lo = *reinterpret_cast<const uint4*>(rp + 16 * ((2 * hh) ^ sw));
            const uint4 hi = *reinterpret_cast<const uint4*>(rp + 16 * ((2 * hh + 1) ^ sw));
            return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        };
        // Score product q of a tile (0 .. 4 KS - 1): k-step q / 4, the residual
        // term when bit 1 is set, subtile q & 1 -- consecutive products go to
        // different accumulators, and each K operand serves two of them.
        constexpr int NQK = (QTERMS == 2 ? 4 : 2) * KS;
        auto score_mfma = [&](f32x16 (&s)[2], const i32x8 (&kop)[2], int q) {
            const int st = q & 1, part = QTERMS == 2 ? (q >> 1) & 1 : 0, ks = QTERMS == 2 ? q >> 2 : q >> 1;
            const f32x16 zero = {};
            s[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                kop[st], part ? qlo[ks] : qhi[ks], (q < 2) ? zero : s[st], 0, 0, 0, 127, 0, part ? 123 : 127);
        };
        auto scores = [&](f32x16 (&s)[2], const char* kt_lds) {
            i32x8 kop[2];
    #pragma unroll
            for (int q = 0; q < NQK; ++q) {
                if ((q & (QTERMS == 2 ? 3 : 1)) == 0) {
                    kop[0] = k_operand(kt_lds, 0, q >> (QTERMS == 2 ? 2 : 1));
                    kop[1] = k_operand(kt_lds, 1, q >> (QTERMS == 2 ? 2 : 1));
                }
                score_mfma(s, kop, q);
            }
        };
        const i32x8 ones_a = rowsum_ones8(lane);

        i32x8 pb = {};   // e4m3 probabilities of a tile: the B operand of the PV product
        // Block of tile kt: row maximum of S(kt) and the threshold rule, then
        // the NQK score products of tile kt+1, each with a share of tile kt's
        // probabilities beside it (fma, exp2, e4m3 pack) in fenced chunks; the
        // row sum of the e4m3 values on the matrix core; the PV products.
        auto softmax_pv = [&](f32x16 (&s)[2], int kt, float ksc, float vsc, const char* vt_lds, f32x16 (&nxt)[2],
                              const char* knext) {
            const int k_lo = kt * BC;
            // lane half hh holds keys 32hh .. 32hh+31 of the tile: K block 2kt + hh
            const float ct = c2q * ksc;
            const int e8v = (__float_as_uint(vsc) >> 23) & 0xFF;  // power of two -> E8M0
            if ((k_lo + BC > a.N) || (CAUSAL && k_lo + BC - 1 > q0)) {
                const int lim = (CAUSAL ? min(qi, a.N - 1) : a.N - 1) - k_lo - 32 * hh;
    #pragma unroll
                for (int st = 0; st < 2; ++st)
    #pragma unroll
                    for (int g = 0; g < 16; ++g)
                        if (16 * st + g > lim) s[st][g] = -INFINITY;
            }
            float mx = -INFINITY;
    #pragma unroll
            for (int st = 0; st < 2; ++st)
    #pragma unroll
                for (int g = 0; g < 16; ++g) mx = fmaxf(mx, s[st][g]);
            const float mt = pair_max8(mx * ct);
            if (__any(mt > m_ref + a.tau)) {
                const float mn = fmaxf(m_ref, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
                lsum *= alpha;
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
                    for (int g = 0; g < 16; ++g) oacc[dt][g] *= alpha;
                m_ref = mn;
            }
            const float bias = 6.f - m_ref;  // exp2(s*ct - m + 6) = 64 p
            // probabilities of chunk r4 (4 scores: subtile r4 / 4, elements 4 (r4 % 4) ..)
            auto exp_chunk = [&](int r4) {
                const int st = r4 >> 2, r = r4 & 3;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[st][4 * r + 0], ct, bias));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[st][4 * r + 1], ct, bias));
                const float p2 = __builtin_amdgcn_exp2f(fmaf(s[st][4 * r + 2], ct, bias));
                const float p3 = __builtin_amdgcn_exp2f(fmaf(s[st][4 * r + 3], ct, bias));
                // the low half is written here and the high half below, so the
                // incoming word is irrelevant: it is the previous tile's
                // (already consumed) word of the same register
                const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb[r4], false);
                pb[r4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
            };
            constexpr int CPM = 8 / NQK;   // probability chunks per score product
            // The next k-step's K operands are read two products before they
            // are needed (+1 %), and the first V^T operand during the last two
            // score products (+0.5 %), except in the causal two-term kernel,
            // whose registers do not have room for them (it spilled: -7 %).
            constexpr bool KRA = !(CAUSAL && QTERMS == 2);
            constexpr int QPK = QTERMS == 2 ? 4 : 2;   // score products per k-step
            i32x8 kop[2], kn[2], va0;
            if (KRA) {
                kop[0] = k_operand(knext, 0, 0);
                kop[1] = k_operand(knext, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
            for (int q = 0; q < NQK; ++q) {
                const int ks = q / QPK, pos = q % QPK;
                if (KRA) {
                    if (pos == QPK - 2 && ks + 1 < KS) {
                        kn[0] = k_operand(knext, 0, ks + 1);
                        kn[1] = k_operand(knext, 1, ks + 1);
                    }
                } else if (pos == 0) {
                    kop[0] = k_operand(knext, 0, ks);
                    kop[1] = k_operand(knext, 1, ks);
                }
                if (KRA && q == NQK - 2) va0 = v_operand(vt_lds, 0);   // the first PV operand
                score_mfma(nxt, kop, q);
                if (KRA && pos == QPK - 1 && ks + 1 < KS) {
                    kop[0] = kn[0];
                    kop[1] = kn[1];
                }
    #pragma unroll
                for (int c = 0; c < CPM; ++c) exp_chunk(q * CPM + c);
                __builtin_amdgcn_sched_barrier(0);
            }
            const f32x4 rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                ones_a, pb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            i32x8 va = KRA ? va0 : v_operand(vt_lds, 0);
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const i32x8 vcur = va;
                if (dt + 1 < DT) va = v_operand(vt_lds, dt + 1);
                oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vcur, pb, oacc[dt], 0, 0, 0, e8v, 0, 127);
            }
            lsum += rs[0];
        };

        // Block scales of the tile a step works on are loaded one step ahead,
        // before that step's tile copies: a wait for them is then never a wait
        // for the copies (loads retire in order).  Lane half hh holds the keys
        // of K block 2kt + hh.
        auto kscale = [&](int kt, int l) { return a.ks[int64_t(bh) * nkb + min(2 * kt + (l >> 5), nkb - 1)]; };
        auto vscale = [&](int kt) { return a.vs[int64_t(bh) * nvb + min(kt, nvb - 1)]; };
        float ks_cur = r ? ks_next : kscale(0, lane), vs_cur = r ? vs_next : vscale(0);
        if (r == 0) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        read_q();
        f32x16 sA[2], sB[2];
        if (wnt > 0) scores(sA, lds_k0);
        // every wave is done with K0 before K2 overwrites it (LDS reads only:
        // the previous tile's O stores need not have completed)
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();

        auto step = [&](int kt, f32x16 (&cur)[2], f32x16 (&nxt)[2], char* k_cur, char* k_nxt, char* v_cur,
                        char* v_nxt) {
            const float ks_nxt = kscale(kt + 1, lane), vs_nxt = vscale(kt + 1);
            if (kt + 2 < nt) copy_k(kt + 2, k_cur, lane);
            if (kt + 1 < nt) copy_v(kt + 1, v_nxt, lane);
            if (kt < wnt) softmax_pv(cur, kt, ks_cur, vs_cur, v_cur, nxt, k_nxt);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            ks_cur = ks_nxt;
            vs_cur = vs_nxt;
        };
        for (int kt = 0; kt < nt; kt += 2) {
            step(kt, sA, sB, lds_k0, lds_k1, lds_v0, lds_v1);
            if (kt + 1 < nt) step(kt + 1, sB, sA, lds_k1, lds_k0, lds_v1, lds_v0);
        }

        // Handover: the second tile's K/V copies and block scales go out
        // before this tile's epilogue (the loop's last barrier came after
        // every wave's last LDS read); its Q rows follow once this wave's O
        // rows have left the slice.
        const bool hand = r + 1 < n_tiles;
        if (hand) {
            const int nt2 = CAUSAL ? min(n_kt_all, (min(a.N, (p + 1) * BR) + BC - 1) / BC) : n_kt_all;
            const int l = fresh_lane();
            if (nt2 > 0) {
                copy_k(0, lds_k0, l);
                copy_v(0, lds_v0, l);
            }
            if (nt2 > 1) copy_k(1, lds_k1, l);
            sq_next = qscale(p);
            ks_next = kscale(0, l);
            vs_next = a.vs[__builtin_amdgcn_readfirstlane(bh * nvb)];
        }

        // O = O^T / l into the slice (row j, chunk 4 dt + c4, half hh), then
        // out as whole rows: lane L holds row ORPI i + L / OCPR, chunk L % OCPR.
        const float lt = lsum;   // the row sum already covers both lane halves
        const float inv = 1.0f / lt;
        constexpr int OCPR = D / 8, ORPI = 64 / OCPR;
        const int le = fresh_lane();
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt)
    #pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                __bf16 o4[4];
    #pragma unroll
                for (int t = 0; t < 4; ++t) o4[t] = static_cast<__bf16>(oacc[dt][4 * c4 + t] * inv);
                const int jj = le & 31, h2 = le >> 5;
                *reinterpret_cast<uint2*>(qo + jj * (2 * D) + 16 * ((4 * dt + c4) ^ TL::oswz(jj)) + 8 * h2) =
                    __builtin_bit_cast(uint2, o4);
            }
        if (wnt > 0) {
            uint16_t* const Ow = Og + int64_t(q0) * a.oss;
    #pragma unroll
            for (int i = 0; i < WQ / ORPI; ++i) {
                const int row = ORPI * i + le / OCPR;
                const uint4 v = *reinterpret_cast<const uint4*>(qo + row * (2 * D) + 16 * (le % OCPR));
                if (q0 + row < a.N)
                    *reinterpret_cast<uint4*>(Ow + int64_t(row) * a.oss + 8 * ((le % OCPR) ^ TL::oswz(row))) = v;
            }
            const int qe = q0 + (le & 31);
            if (qe < a.N && le < 32)
                a.lse[int64_t(bh) * a.N + qe] = (m_ref + __log2f(lt) - 6.f) * 0.69314718055994531f;
        }
        if (hand) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);   // this wave's O rows are out of its slice
            copy_q(p);
            __builtin_amdgcn_s_waitcnt(0);        // the second tile's copies and scales have landed
            __builtin_amdgcn_s_barrier();         // ... in every wave
        }
    }
}

template <int D, bool BF>
int launch_q(const QuantArgs& a, hipStream_t s) {
    constexpr int RWG = 4 * (64 / (D / 32));   // rows per workgroup
    const int64_t grid = int64_t(a.B) * a.H * ((a.N + RWG - 1) / RWG);
    hipLaunchKernelGGL((fp8_quantize_kernel<D, BF>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

template <int D, bool CAUSAL>
int launch_a(const Fp8Args& a, hipStream_t s) {
    constexpr int NW = 8;
    const int n_qt = (a.N + NW * WQ - 1) / (NW * WQ);
    const int64_t grid = int64_t(CAUSAL ? (n_qt + 1) / 2 : n_qt) * a.B * a.H;
    if (a.q_terms == 1)
        hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, CAUSAL, 1>), dim3(static_cast<unsigned>(grid)), dim3(NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, CAUSAL, 2>), dim3(static_cast<unsigned>(grid)), dim3(NW * 64), 0, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_fp8_quantize(const QuantArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 64) return a.in_bf16 ? launch_q<64, true>(a, s) : launch_q<64, false>(a, s);
    return a.in_bf16 ? launch_q<128, true>(a, s) : launch_q<128, false>(a, s);
}

int launch_fwd_fp8(const Fp8Args& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 64) return a.causal ? launch_a<64, true>(a, s) : launch_a<64, false>(a, s);
    return a.causal ? launch_a<128, true>(a, s) : launch_a<128, false>(a, s);
}

}  // namespace fa
