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
// the output stays exact by the rescaling identity (sec. 6.3).  The kernel
// does not take every tile's row maximum first: it forms the probabilities
// against the current reference and uses their partial row sums, which bound
// every probability, to detect the rare tile that needs the maximum.  The score
// product of the next tile is issued before the softmax of the current one so
// that matrix-core and vector work overlap (the two-stage GEMM/softmax
// pipelining of the FlashAttention-3 note, section 技術 2).
//
// gfx950 mapping (designed for CDNA4, not taken from the pages' Hopper or
// Blackwell kernels):
//  * a wave owns 32 query rows.  It computes the TRANSPOSED score tile
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS,
//    B = Q^T held in registers for the whole loop).  In the 32x32 accumulator
//    layout lane l holds column l % 32, i.e. ONE query, and 16 of the keys, so
//    the row maximum and row sum are in-lane reductions plus one exchange
//    between lane l and l ^ 32 (v_permlane32_swap).
//  * the K rows are fed to the first product in a permuted order (bits 2 and
//    3 of the row index swapped) so that the accumulator registers of S^T are,
//    after exp2 and a bf16 conversion, already the B operand of the second
//    product O^T += V^T P^T: no LDS round trip for P.
//  * O^T stays in registers with one query per lane, so the rescale factor is
//    a per-lane scalar; the row sum is taken on the matrix core (a product of
//    a constant 0/1 operand with the bf16 probabilities), so it sums exactly
//    the values that multiply V.
//  * K and V tiles are copied global -> LDS by the direct-to-LDS loads of
//    gfx950 (global_load_lds_dwordx4: no registers, no LDS store
//    instructions), row-major and unpadded.  Each lane picks the 16-byte chunk
//    it copies so that the stored tile is XOR-swizzled per row; the operand
//    reads undo the swizzle and hit distinct LDS banks.  V^T is read with the
//    transposing LDS read (ds_read_b64_tr_b16), which hands each lane four
//    consecutive keys of one head-dim column.
//  * K is prefetched two tiles ahead and V one tile ahead (two LDS buffers
//    each), one workgroup barrier per tile.
//  * Q rows come in and O rows go out through each wave's own LDS slice, so
//    that global memory sees whole rows; only the registers hold the
//    transposed (one query per lane) layout.
//  * workgroups are renumbered so that the tiles of one head run on one XCD
//    (the hardware deals workgroup ids round-robin over the 8 XCDs), which
//    keeps that head's K/V in the XCD's L2; under the causal mask a workgroup
//    processes a heavy and a light query tile of one head (tiles T-1-p and
//    p), so all workgroups carry equal work, and the light tile's loads are
//    issued before the heavy tile's epilogue.
//  * workgroup and lane ids come from the compiler builtins: with the IEEE
//    mode bit off (see the build) the device library's id functions cannot
//    be inlined and would become real calls.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "lds_copy.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BC = 64;  // keys per K/V tile
// s_waitcnt immediate that waits for LDS (and scalar memory) operations only:
// vmcnt and expcnt at their maxima, lgkmcnt 0.
constexpr int kLgkm0 = 0xC07F;
constexpr int WQ = 32;  // query rows per wave
constexpr bf16x2 kOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

// Row sums of the probabilities on the matrix core (four small products per
// tile) instead of the vector unit (sixteen v_dot2 per tile): measured +2.1 %
// at head_dim 64 and +0.8 % at 128, where the vector work per score is the
// limit ("FlashAttention-4" explainer, 論文 Section 3.2, moves work off the
// exponential unit; here it moves off the vector unit).
constexpr bool kRowsumMfma = true;

// A operand of the row-sum product v_mfma_f32_16x16x32_bf16(A, P chunk, acc).
// Fed as its B operand, the probability chunk of lane l (query l % 32, keys of
// lane half l / 32) is column l % 16 of K-block l / 16; A row m holds ones in
// the K-blocks whose parity is that of m / 4 when m % 4 == 0 and zeros
// elsewhere, so output row 4g, column c -- register 0 of lane 16g + c -- is
// the sum over both lane halves of query 16 (g % 2) + c = (16g + c) % 32:
// every lane receives its own query's full 64-key row sum.
__device__ __forceinline__ bf16x8 rowsum_ones(int lane) {
    const int m = lane & 15, kb = lane >> 4;
    const __bf16 v = static_cast<__bf16>(((m & 3) == 0 && ((m >> 2) & 1) == (kb & 1)) ? 1.0f : 0.0f);
    return bf16x8{v, v, v, v, v, v, v, v};
}

template <int D>
struct Tile {
    static constexpr int CPR = D / 8;               // 16-byte chunks per row
    static constexpr int BYTES = BC * D * 2;        // one K or V tile
    static constexpr int QS_OFF = 4 * BYTES;        // K0 K1 V0 V1, then the waves' Q/O slices
    static constexpr int SLICE = 32 * D * 2;        // one wave's 32 rows of Q or O
    static constexpr int lds_bytes(int nw) { return QS_OFF + nw * SLICE; }
    // XOR swizzles (in 16-byte chunk units) applied to a row's chunk index.
    // K: 16 lanes read one logical chunk of 16 different rows.
    __device__ static int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
    // V: 16 lanes read 4 rows x 32 bytes (two groups: 4 rows x 64 bytes).
    __device__ static int vswz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

// Row of the A operand that lane row i loads: bits 2 and 3 swapped.  With this
// order the S^T accumulator register g = 4r + t of lane half hh holds key
//   16 * (r >> 1) + 8 * hh + 4 * (r & 1) + t
// so registers 8c .. 8c+7 hold keys 16c + 8hh .. 16c + 8hh + 7, exactly the
// B-operand slice lane (query, hh) must supply for keys 16c .. 16c+15.
__device__ __forceinline__ int perm_row(int i) {
    return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// v_permlane32_swap(x, x) yields {x[lo half] in both halves, x[hi half] in
// both halves}; combining the two gives the pair value in every lane.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read: within each 16-lane group, destination lane 4p+q gets
// element q of the 8-byte rows read by source lanes p, 4+p, 8+p, 12+p.
__device__ __forceinline__ short4_t lds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((__attribute__((address_space(3))) char*)(p)));
}

// One 256-query tile (NW waves of 32 queries) of head bh.  With `issued` the
// tile's Q rows (in the waves' LDS slices) and its first K/V tiles were
// copied by the previous call, which also waited for them and passed a
// barrier.  With next_qt >= 0 the tile ends by starting the K/V copies of
// query tile next_qt of the same head before it normalises and stores its
// own O, then copies the next Q rows into the slices the O rows have left:
// the next tile's loads overlap this tile's epilogue.
template <int D, int NW, bool CAUSAL>
__device__ __forceinline__ void fwd_bf16_tile(const FwdArgs& a, char* smem, int bh, int qt, int next_qt,
                                              bool issued) {
    using TL = Tile<D>;
    constexpr int BR = NW * WQ;                       // query rows per workgroup
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int NI = TL::BYTES / 1024 / NW;         // 1 KB direct loads per wave per tile
    static_assert(NI >= 1 && TL::BYTES % (1024 * NW) == 0, "tile / wave mismatch");

    const int b = bh / a.H, h = bh % a.H;
    const int64_t base = int64_t(b) * a.sb + int64_t(h) * a.sh;
    const u16* Qg = static_cast<const u16*>(a.q) + base;
    const u16* Kg = static_cast<const u16*>(a.k) + base;
    const u16* Vg = static_cast<const u16*>(a.v) + base;
    u16* Og = static_cast<u16*>(a.o) + base;

    const int tid = __builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int j = lane & 31, hh = lane >> 5;
    const int q0 = qt * BR + wave * WQ;  // first query row of this wave
    const int qi = q0 + j;               // this lane's query row

    const int n_kt_all = (a.N + BC - 1) / BC;
    auto n_ktiles = [&](int t) { return CAUSAL ? min(n_kt_all, (min(a.N, (t + 1) * BR) + BC - 1) / BC) : n_kt_all; };
    const int nt = n_ktiles(qt);
    int wnt = CAUSAL ? min(nt, (min(a.N, q0 + WQ) + BC - 1) / BC) : nt;
    if (q0 >= a.N) wnt = 0;

    // ---- direct global -> LDS tile copy ---------------------------------------
    // Wave w copies 1 KB blocks w*NI .. w*NI+NI-1 of the tile; lane L of a block
    // fills LDS chunk 64*blk + L, i.e. row (64*blk + L) / CPR, physical chunk
    // (64*blk + L) % CPR, which holds logical chunk (physical ^ swizzle(row)).
    // The row a lane copies is the same in every tile, so its source address
    // is fixed and a tile adds a wave-uniform offset.  At head_dim 128 a lane
    // keeps a 32-bit byte offset per copy (the tile's first row is a
    // wave-uniform base in scalar registers), which saves the registers that
    // 64-bit addresses would hold (with four waves these spilled, and each
    // reload waited for the copies in flight); at head_dim 64 the 64-bit
    // addresses fit and measured slightly faster.  In the ragged last tile
    // rows past the end re-read the last row: their scores are masked to -inf,
    // so their probabilities are exactly 0.
    constexpr bool OFF = D == 128;
    constexpr int NA = OFF ? 1 : NI;  // 64-bit addresses kept per tensor
    auto fresh_lane0 = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    uint32_t koff[NI], voff[NI];   // OFF: byte offsets from the tile's first row
    const u16* kp[NA];             // !OFF: the lane's source addresses in tile 0
    const u16* vp[NA];
    int crow[NA];                  // !OFF: the rows they copy
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = (wave * NI + i) * 64 + lane;
        const int row = c / TL::CPR, pch = c % TL::CPR;
        if constexpr (OFF) {
            koff[i] = 2u * uint32_t(row * a.ss + 8 * (pch ^ TL::kswz(row)));
            voff[i] = 2u * uint32_t(row * a.ss + 8 * (pch ^ TL::vswz(row)));
        } else {
            crow[i] = row;
            kp[i] = Kg + int64_t(row) * a.ss + 8 * (pch ^ TL::kswz(row));
            vp[i] = Vg + int64_t(row) * a.ss + 8 * (pch ^ TL::vswz(row));
        }
    }
    auto copy_tile = [&](bool is_v, int kt, int lds_off) {
        const int k0 = kt * BC;
        if (k0 + BC <= a.N) {  // full tile: one wave-uniform offset
            if constexpr (OFF) {
                const u16* tb = (is_v ? Vg : Kg) + int64_t(k0) * a.ss;
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    copy16_to_lds_off(tb, is_v ? voff[i] : koff[i], smem + lds_off + (wave * NI + i) * 1024);
            } else {
                const int64_t off = int64_t(k0) * a.ss;
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    copy16_to_lds((is_v ? vp[i] : kp[i]) + off, smem + lds_off + (wave * NI + i) * 1024);
            }
        } else if constexpr (OFF) {
            const int l = fresh_lane0();
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int c = (wave * NI + i) * 64 + l;
                const int row = c / TL::CPR, pch = c % TL::CPR;
                const int sw = is_v ? TL::vswz(row) : TL::kswz(row);
                copy16_to_lds((is_v ? Vg : Kg) + int64_t(min(k0 + row, a.N - 1)) * a.ss + 8 * (pch ^ sw),
                              smem + lds_off + (wave * NI + i) * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int64_t row_off = int64_t(min(k0 + crow[i], a.N - 1) - crow[i]);
                copy16_to_lds((is_v ? vp[i] : kp[i]) + row_off * a.ss, smem + lds_off + (wave * NI + i) * 1024);
            }
        }
    };
    constexpr int K_OFF0 = 0, K_OFF1 = TL::BYTES, V_OFF0 = 2 * TL::BYTES, V_OFF1 = 3 * TL::BYTES;

    // ---- Q in and O out through the wave's own LDS slice (32 rows x D) -------
    // Global memory sees whole rows: Q is copied in 1 KB blocks (lane L of
    // block i fills slice chunk 64 i + L: row (64 i + L) / CPR, physical chunk
    // (64 i + L) % CPR holding logical chunk physical ^ kswz(row)), and O
    // leaves 16 bytes of a row per lane.  Only the registers see the
    // transposed layout (one query per lane).  A wave touches only its own
    // slice, so the slice needs no workgroup barrier.  Rows past the end copy
    // the last row (never stored).
    constexpr int NQ = TL::SLICE / 1024;              // 1 KB copies per slice
    constexpr int RPI = 64 / TL::CPR;                 // rows per 16-byte-per-lane access
    char* const qs = smem + TL::QS_OFF + wave * TL::SLICE;
    // The slice addressing is recomputed at each use from an opaque copy of
    // the lane index: shared with the tile's other end it would stay live
    // across the main loop and cost registers there.
    auto fresh_lane = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    auto copy_q = [&](int t) {
        const int r0 = t * BR + wave * WQ, l = fresh_lane();
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int c = i * 64 + l, row = c / TL::CPR, pch = c % TL::CPR;
            copy16_to_lds(Qg + int64_t(min(r0 + row, a.N - 1)) * a.ss + 8 * (pch ^ TL::kswz(row)), qs + i * 1024);
        }
    };
    // Q^T operand: lane (query j, half hh) holds Q[qi][16ks + 8hh .. +7]
    bf16x8 qreg[KSTEPS];
    auto read_q = [&]() {
        const int l = fresh_lane(), jj = l & 31, h2 = l >> 5;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qreg[ks] = *reinterpret_cast<const bf16x8*>(qs + jj * (2 * D) + 16 * ((2 * ks + h2) ^ TL::kswz(jj)));
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 16; ++g) oacc[dt][g] = 0.f;
    float m_ref = -FLT_MAX;  // log2 units
    float lsum = 0.f;        // running sum: this lane's share, or the row's with kRowsumMfma
    const bf16x8 ones_a = rowsum_ones(lane);
    const float c2 = a.scale_log2;

    // per-lane LDS addressing that does not change across tiles
    const int krow_base = perm_row(j);                              // + 32*st
    const int tr_row = 8 * (lane >> 5) + ((lane >> 2) & 3);         // + 32*st + 16*cc
    const int tr_lch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);   // + 4*dt
    const int tr_half = 8 * (lane & 1);

    // K operand of score MFMA m (subtile m % 2, k-step m / 2: consecutive
    // MFMAs accumulate into different subtiles).
    auto k_operand = [&](const char* kt_lds, int m) -> bf16x8 {
        const int st = m & 1, ks = m >> 1;
        const int row = 32 * st + krow_base;
        return *reinterpret_cast<const bf16x8*>(kt_lds + row * (2 * D) + 16 * ((2 * ks + hh) ^ TL::kswz(row)));
    };
    // V^T operand of PV MFMA n (key chunk c = n / DT, head-dim tile dt = n % DT):
    // two transposing reads; lane 16g + 4a + b addresses key 8*(g >> 1) + a
    // (+4), columns 16*(g & 1) + 4b .. +3 of the row-major V tile.
    auto v_operand = [&](const char* vt_lds, int n) -> bf16x8 {
        const int c = n / DT, dt = n % DT;
        const int row = 32 * (c >> 1) + 16 * (c & 1) + tr_row;
        const char* p = vt_lds + row * (2 * D) + tr_half + 16 * ((4 * dt + tr_lch) ^ TL::vswz(row));
        const short4_t lo = lds_read_tr(p);
        const short4_t hi = lds_read_tr(p + 4 * (2 * D));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // S^T for one K tile (two 32-key subtiles); used outside the main loop.
    auto scores = [&](f32x16 (&s)[2], const char* kt_lds) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int g = 0; g < 16; ++g) s[st][g] = 0.f;
#pragma unroll
        for (int m = 0; m < 2 * KSTEPS; ++m)
            s[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kt_lds, m), qreg[m >> 1], s[m & 1], 0, 0, 0);
    };

    // Causal diagonal / ragged tiles: scores of keys past the query (or past
    // the end) become -inf.  Register g of subtile st in lane half hh holds key
    // k_lo + off(st, g) + 8*hh with a compile-time off, so one per-lane
    // threshold decides every register.
    auto apply_mask = [&](f32x16 (&s)[2], int kt) {
        const int lim = (CAUSAL ? min(qi, a.N - 1) : a.N - 1) - kt * BC - 8 * hh;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int r = g >> 2, t = g & 3;
                const int off = 32 * st + 16 * (r >> 1) + 4 * (r & 1) + t;
                if (off > lim) s[st][g] = -INFINITY;
            }
    };
    auto needs_mask = [&](int kt) {
        const int k_lo = kt * BC;
        return (k_lo + BC > a.N) || (CAUSAL && k_lo + BC - 1 > q0);
    };
    auto tile_max = [&](const f32x16 (&s)[2]) -> float {
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int g = 0; g < 16; ++g) mx = fmaxf(mx, s[st][g]);
        return pair_max(mx);
    };

    // ---- softmax with a speculative reference maximum ------------------------
    // A tile's probabilities are formed with the reference maximum m_ref as it
    // stands, without a pass over the tile's own row maximum.  Every p is
    // non-negative, so a lane's partial row sum bounds each p it holds: while
    // no partial sum exceeds 2^tau, no score exceeds m_ref + tau and the
    // reference may stay (the threshold rule of the "FlashAttention-4"
    // explainer, 論文 Section 3.3).  Otherwise, before any of the tile's
    // probabilities reach O, a slow path takes the tile's true row maximum,
    // applies the same rule (rescale when the maximum exceeds m_ref by more
    // than tau; exact per-lane rescaling of O and l, sec. 6.3) and recomputes
    // the tile's probabilities.  The rescale decisions are those of the
    // max-first formulation (up to the bf16 rounding of a p lying within one
    // bf16 step of 2^tau, where either choice is exact).  An overflowing
    // exp2 gives an infinite sum and so also takes the slow path.
    const float thr = exp2f(a.tau);
    // Does a partial row sum exceed 2^tau?  Compared as unsigned bit patterns,
    // so that an infinite or NaN sum (an overflowing exp2 in the matrix-core
    // row sum meets the zeros of its constant operand: 0 * inf = NaN) also
    // takes the slow path; the sums are never negative.  A float comparison
    // would not do: the kernels are compiled assuming no NaN operands.
    const uint32_t thr_bits = __float_as_uint(thr);
    auto over = [&](float lp) { return __any(__float_as_uint(lp) > thr_bits); };
    auto rescale = [&](const f32x16 (&s)[2]) -> bool {
        const float mt = tile_max(s) * c2;
        if (!__any(mt > m_ref + a.tau)) return false;
        const float mn = fmaxf(m_ref, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 16; ++g) oacc[dt][g] *= alpha;
        m_ref = mn;
        return true;
    };
    // probabilities of score pair p (0..15: chunk p / 4, elements 2*(p % 4), +1)
    auto exp_pair = [&](const f32x16 (&s)[2], int p, bf16x8 (&pb)[4], float& acc) {
        const float neg_m = -m_ref;
        const int c = p >> 2, e = 2 * (p & 3);
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + e], c2, neg_m));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[c >> 1][8 * (c & 1) + e + 1], c2, neg_m));
        const bf16x2 pr = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
        pb[c][e] = pr[0];
        pb[c][e + 1] = pr[1];
        if (!kRowsumMfma) acc = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes, acc, false);
    };
    // the row sum of chunk c on the matrix core (kRowsumMfma)
    auto chunk_sum = [&](const bf16x8 (&pb)[4], int c, f32x4& rs) {
        rs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_a, pb[c], rs, 0, 0, 0);
    };

    // One straight-line block per tile, issued in fenced chunks so that every
    // matrix-core instruction has independent vector work beside it:
    //  phase 1: score MFMAs of the next tile (K operands read NPK MFMAs ahead),
    //           each paired with probabilities of the current tile
    //           (fma, exp2, bf16 pack, and the row-sum product of each
    //           completed chunk); then the check above;
    //  phase 2: PV MFMAs of the current tile (V^T operands read NPV ahead;
    //           the first NPV during the last score products).
    // On a wave's last tile the score product reads a valid but unused buffer.
    constexpr int QKM = 2 * KSTEPS;   // score MFMAs per tile
    constexpr int PVM = 4 * DT;       // PV MFMAs per tile
    constexpr int NPAIR = 16;         // probability pairs per lane per tile
    constexpr int PPM = NPAIR / QKM;  // pairs per score MFMA
    constexpr int NPK = 3, NPV = 2;   // K three ahead: +0.3 % (d = 128), +0.4 % (d = 64)
    static_assert(NPAIR % QKM == 0, "phase split");
    // The last NDEF PV products of a tile are issued at the start of the next
    // tile's block, after the workgroup barrier: the matrix core then has
    // queued work while the next K operands are read from LDS.  Their V^T
    // operands stay in registers (the LDS buffer they came from may be
    // overwritten by then) and their P operand is the last chunk of pb, which
    // the next block rewrites only later.  Before the first tile the deferred
    // operands are zero (a product that adds exactly 0).
    constexpr int NDEF = 2;
    static_assert(NDEF == NPV && PVM - NDEF >= NPV, "deferred PV products");
    bf16x8 pb[4] = {};
    bf16x8 vdef[NDEF] = {};
    auto flush_deferred = [&]() {
#pragma unroll
        for (int i = 0; i < NDEF; ++i) {
            const int n = PVM - NDEF + i;
            oacc[n % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vdef[i], pb[n / DT], oacc[n % DT], 0, 0, 0);
        }
    };
    auto main_block = [&](f32x16 (&s)[2], const char* vt_lds, f32x16 (&nxt)[2], const char* knext) {
        bf16x8 kb[NPK];
#pragma unroll
        for (int i = 0; i < NPK; ++i) kb[i] = k_operand(knext, i);
        float lpart[2] = {0.f, 0.f};  // two independent row-sum chains
        f32x4 rs = {0.f, 0.f, 0.f, 0.f};
        const f32x16 zero = {};
        flush_deferred();
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 vb[NPV];
#pragma unroll
        for (int m = 0; m < QKM; ++m) {
            const bf16x8 ka = kb[m % NPK];
            if (m + NPK < QKM) kb[m % NPK] = k_operand(knext, m + NPK);
            if (m == QKM - 2) {   // the first PV operands, in flight during the check
#pragma unroll
                for (int i = 0; i < NPV; ++i) vb[i] = v_operand(vt_lds, i);
            }
            nxt[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[m >> 1], (m < 2) ? zero : nxt[m & 1], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < PPM; ++q) {
                const int p = m * PPM + q;
                exp_pair(s, p, pb, lpart[p & 1]);
                if (kRowsumMfma && (p & 3) == 3) chunk_sum(pb, p >> 2, rs);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float lp = kRowsumMfma ? rs[0] : lpart[0] + lpart[1];
        if (over(lp) && rescale(s)) {
            lpart[0] = lpart[1] = 0.f;
            rs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                exp_pair(s, p, pb, lpart[p & 1]);
                if (kRowsumMfma && (p & 3) == 3) chunk_sum(pb, p >> 2, rs);
            }
            lp = kRowsumMfma ? rs[0] : lpart[0] + lpart[1];
        }
        lsum += lp;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < PVM - NDEF; ++n) {
            const bf16x8 va = vb[n % NPV];
            if (n + NPV < PVM) vb[n % NPV] = v_operand(vt_lds, n + NPV);
            oacc[n % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[n / DT], oacc[n % DT], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NDEF; ++i) vdef[i] = vb[(PVM - NDEF + i) % NPV];
    };

    // ---- prologue: Q^T, K0, V0, K1 in flight; S(0) -----------------------------
    auto first_copies = [&](int n) {
        if (n > 0) {
            copy_tile(false, 0, K_OFF0);
            copy_tile(true, 0, V_OFF0);
        }
        if (n > 1) copy_tile(false, 1, K_OFF1);
    };
    if (!issued) {
        copy_q(qt);
        first_copies(nt);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    read_q();

    f32x16 sA[2], sB[2];
    if (wnt > 0) {
        scores(sA, smem + K_OFF0);
        if (needs_mask(0)) apply_mask(sA, 0);
        m_ref = tile_max(sA) * c2;  // finite: key 0 is allowed for every query
    }
    // every wave is done with K0 before K2 overwrites it (LDS reads only: the
    // previous tile's O stores need not have completed)
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();

    // ---- main loop, unrolled by two so buffers and score sets alternate ------
    auto step = [&](int kt, f32x16 (&cur)[2], f32x16 (&nxt)[2], int k_cur_off, int k_nxt_off,
                    int v_cur_off, int v_nxt_off) {
        if (kt + 2 < nt) copy_tile(false, kt + 2, k_cur_off);
        if (kt + 1 < nt) copy_tile(true, kt + 1, v_nxt_off);
        if (kt < wnt) {
            main_block(cur, smem + v_cur_off, nxt, smem + k_nxt_off);
            if (needs_mask(kt + 1)) apply_mask(nxt, kt + 1);  // at most the diagonal and the ragged tile
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int kt = 0; kt < nt; kt += 2) {
        step(kt, sA, sB, K_OFF0, K_OFF1, V_OFF0, V_OFF1);
        if (kt + 1 < nt) step(kt + 1, sB, sA, K_OFF1, K_OFF0, V_OFF1, V_OFF0);
    }

    flush_deferred();

    // ---- handover: the next tile's K/V copies go out first ------------------
    // The loop's last barrier came after every wave's last LDS read, so the
    // buffers are free for the next tile's copies.
    if (next_qt >= 0) first_copies(n_ktiles(next_qt));

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------
    // O^T into the slice (row j, logical chunk 4 dt + r, half hh), then back as
    // whole rows: lane L holds row RPI i + L / CPR, physical chunk L % CPR.
    const float lt = kRowsumMfma ? lsum : pair_sum(lsum);
    const float inv = 1.0f / lt;
    const int le = fresh_lane();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            __bf16 o4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) o4[t] = static_cast<__bf16>(oacc[dt][4 * r + t] * inv);
            const int jj = le & 31, h2 = le >> 5;
            *reinterpret_cast<uint2*>(qs + jj * (2 * D) + 16 * ((4 * dt + r) ^ TL::kswz(jj)) + 8 * h2) =
                __builtin_bit_cast(uint2, o4);
        }
    if (wnt > 0) {
#pragma unroll
        for (int i = 0; i < WQ / RPI; ++i) {
            const int row = RPI * i + le / TL::CPR;
            const uint4 orow = *reinterpret_cast<const uint4*>(qs + row * (2 * D) + 16 * (le % TL::CPR));
            if (q0 + row < a.N)
                *reinterpret_cast<uint4*>(Og + int64_t(q0 + row) * a.ss +
                                          8 * ((le % TL::CPR) ^ TL::kswz(row))) = orow;
        }
        if (qi < a.N && hh == 0) a.lse[int64_t(bh) * a.N + qi] = (m_ref + __log2f(lt)) * 0.69314718055994531f;
    }
    // The next tile's Q rows go into the slice once this wave's O rows are
    // out of it; its copies were issued after the O stores, so the wait for
    // them costs little beyond their own latency.
    if (next_qt >= 0) {
        __builtin_amdgcn_s_waitcnt(kLgkm0);   // this wave's O rows are out of its slice
        copy_q(next_qt);
        __builtin_amdgcn_s_waitcnt(0);        // the next tile's copies have landed
        __builtin_amdgcn_s_barrier();         // ... in every wave
    }
}

// Work decomposition.  Workgroup ids are renumbered so that each XCD (the
// hardware deals ids round-robin over the 8 XCDs) owns a contiguous range of
// heads, whose K/V then stay in that XCD's L2.  Under the causal mask tile qt
// needs qt + 1 key tiles; a workgroup takes the pair (T-1-p, p) of a head's T
// query tiles, so every workgroup has the same T + 1 tiles of work (the
// heavier one first) and the grid is balanced without any dynamic queue.
// At most 256 registers per lane so that two waves share each SIMD.
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_kernel(FwdArgs a) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    constexpr int BR = NW * WQ;
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
#pragma nounroll
    for (int r = 0; r < n_tiles; ++r)     // one copy of the tile code
        fwd_bf16_tile<D, NW, CAUSAL>(a, smem, bh, r ? p : hi, r + 1 < n_tiles ? p : -1, r > 0);
}

template <int D, int NW, bool CAUSAL>
int launch(const FwdArgs& a, hipStream_t stream) {
    constexpr int BR = NW * WQ;
    constexpr int LDS = Tile<D>::lds_bytes(NW);
    auto kern = fwd_bf16_kernel<D, NW, CAUSAL>;
    // set once per process (thread-safe initialisation of a local static)
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return static_cast<int>(attr);
    const int n_qt = (a.N + BR - 1) / BR;
    const int64_t grid = int64_t(CAUSAL ? (n_qt + 1) / 2 : n_qt) * a.B * a.H;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(NW * 64), LDS, stream, a);
    return static_cast<int>(hipGetLastError());
}

template <int D>
int dispatch(const FwdArgs& a, hipStream_t s) {
    // tile_cfg 1: 8 waves (256 query rows per workgroup); 2: 4 waves (128 rows);
    // 0 (automatic): 4 waves for d = 64, whose short tiles gain from the smaller
    // workgroups (+1.5 % at B4 H16 N2048), 8 waves for d = 128 (5 % faster there).
    const bool four = a.tile_cfg == 2 || (a.tile_cfg == 0 && D == 64);
    if (four) return a.causal ? launch<D, 4, true>(a, s) : launch<D, 4, false>(a, s);
    return a.causal ? launch<D, 8, true>(a, s) : launch<D, 8, false>(a, s);
}

}  // namespace

int launch_fwd_bf16(const FwdArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return a.D == 64 ? dispatch<64>(a, s) : dispatch<128>(a, s);
}

}  // namespace fa
