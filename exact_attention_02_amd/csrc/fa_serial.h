// Fused exact-attention forward for 16-bit inputs (fp16, bf16) on gfx950:
// each wave works through its 32 x 32 blocks one at a time, and several waves
// share each SIMD.
//
// The computation is the block-by-block loop of the aiinarabic.com
// flash-attention page (load a block of K and V on chip, score it, softmax it,
// multiply by V, merge; the algorithm paragraph under Figure 4), with the
// running max and sum of the FLASHLIGHT summary on gist.science (Methodology
// item 3).
//
// Why one block at a time: on gfx950 the matrix core runs one wave's MFMAs
// while the SIMD issues another wave's VALU work, so the overlap of the two
// comes from the waves sharing the SIMD. At D = 64 a 32 x 32 block costs 8
// MFMAs (256 SIMD cycles) and about 55 VALU instructions of softmax, 16 of
// them exponentials, which take longer than the MFMAs: the VALU is the bound.
// Each wave therefore runs the plain sequence -- scores on MFMA, softmax on
// the VALU, P.V on MFMA -- with as few VALU instructions beside the
// exponentials, sums and conversions as possible, and the register budget is
// held to four waves per SIMD (two at D = 128, where the MFMAs are the bound)
// so that the SIMD always finds a wave with work for each unit.
//
// Per block (wave rows x 32 keys), lane l holds query l mod 32 and 16 of the
// 32 keys (S^T = K Q^T on a 32 x 32 MFMA accumulator):
//   S  = K Q^T                             (D/16 MFMAs)
//   p  = 2^(c s - m), 16 per lane          (one FMA and one exponential each)
//   ts = the lane half's sum of p          (a fixed pairwise order)
//   P  = p rounded to the input type       (8 conversions)
//   O^T += V^T P^T                         (D/16 MFMAs; V read transposed)
// m is a reference per row that moves only when needed: a block whose lane-
// half sum exceeds SUM_LIMIT (a score grew past m), or the row's first block
// (m = -inf makes ts infinite), is formed again exactly against the row max,
// rescaling O and the sum by 2^(m_old - m_new). O / l and the log-sum-exp do
// not depend on which m was used. When a block's sum exceeds a third of the
// lane half's sum so far (the first blocks of a row, peaked rows), P's
// rounding residual (p - P, rounded) also multiplies V, so that a dominant
// weight's rounding does not reach O. Both checks are one compare against
// thr = min(lh / 3, SUM_LIMIT), and both corrections live off the common path;
// the lane half's sum is kept in thirds (one FMA per block), so thr is one
// min.
//
// Score modifiers (the score_mod of fa_fwd_mod in include/fa.h) change only
// the exponent argument. ALiBi adds slope * (key - i') to the scaled score:
// the part that depends on the element's place in the lane's block,
// slope * (8(r/4) + r%4 + 4hh), is the initial value of the score MFMA's
// accumulator (in score units, slope / scale per key), and the rest,
// slope * (32j - i'), is one per-lane term per block, so the bias costs no
// VALU instruction per score. Softcap replaces s by cap * tanh(scale * s /
// cap), through one exponential and one reciprocal.
//
// Tiles of 64 keys go HBM -> LDS by direct-to-LDS buffer loads into two
// slots: tile t+1 is requested at the start of tile t, one barrier per tile.
// The key range of a workgroup runs through four phases: the first
// EARLY_KEYS keys, whose blocks always take the residual pass; tiles with a
// mask edge or skipped blocks before and after the tiles in which every
// block of every wave is fully visible; and those steady tiles, whose blocks
// run with no class checks at all.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace fa {

namespace serial {

// Largest sum of a lane half's 16 weights of one block kept without moving
// the reference: every weight then stays at most 2^10, within fp16's range.
constexpr float SUM_LIMIT = 1024.f;
// e4m3 inputs: the weights are formed as p * 2^LOG2_PRESCALE8 (the scale
// enters the exponent) and stored as e4m3; a lane half's sum of at most
// SUM_LIMIT8 (scaled) keeps every scaled weight at most 256, below the
// format's largest value 448, while weights down to 2^-8 of the reference
// stay in its normal range.
constexpr float LOG2_PRESCALE8 = 2.f;
constexpr float SUM_LIMIT8 = 256.f;
// Keys at the start of a workgroup's range whose blocks always take the
// residual pass (the running sums are small there, so most rows need it).
#ifndef FA_SR_EARLY_KEYS
#define FA_SR_EARLY_KEYS 256
#endif
constexpr int EARLY_KEYS = FA_SR_EARLY_KEYS;
// Waves per SIMD the register budget is held to.
#ifndef FA_SR_WPS_D64
#define FA_SR_WPS_D64 4
#endif
#ifndef FA_SR_WPS_D128
#define FA_SR_WPS_D128 2
#endif
template <int D>
constexpr int waves_per_simd() {
    return D == 64 ? FA_SR_WPS_D64 : FA_SR_WPS_D128;
}

}  // namespace serial

// The workgroup's (batch, head), query tile and split.
__device__ __forceinline__ void serial_wg(const Params& p, int* bh, int* qt, int* split) {
    long long wgid = blockIdx.x;
    *split = 0;
    if (p.n_split > 1) {
        *split = (int)(wgid % p.n_split);
        wgid /= p.n_split;
    }
    decode_wg(wgid, p.n_bh, p.n_qt, p.hg, p.tl, bh, qt);
}

// The kernel's work for one workgroup. FOLD (ALiBi only): the in-block part
// of the bias starts the score accumulator; a compile-time choice, so that
// the loop holds no branch on it.
template <int IN, int OUT, int D, int NW, int TK, int MOD, bool FOLD>
__device__ __forceinline__ void serial_body(const Params& p, uint8_t* smem, int bh, int qt, int split) {
    using namespace serial;
    // e4m3 inputs: Q and K are widened to bf16 (exactly) for the score MFMA,
    // V stays e4m3 and P.V runs on the 8-bit MFMA, 64 keys per step.
    constexpr bool FP8 = IN == IN_E4M3;
    constexpr int QK = FP8 ? IN_BF16 : IN;     // score MFMA operand type
    constexpr int EB = FP8 ? 1 : 2;            // bytes per stored element
    constexpr int NT = 64 * NW;
    constexpr int GRB = D * EB;            // bytes per Q/K/V row in HBM
    constexpr int RB = D * 2;              // bytes per K row in LDS (16-bit)
    constexpr int VRB = D * EB;            // bytes per V row in LDS
    constexpr int CPR = RB / 16;           // 16-byte chunks per LDS K row
    constexpr int VCPR = VRB / 16;         // 16-byte chunks per LDS V row
    static_assert(RB == 128 || RB == 256, "row size");
    static_assert(TK == 64 || TK == 128, "keys per tile");
    static_assert(!FP8 || MOD == MOD_NONE, "e4m3: no score modifier");
    constexpr int SUB = TK / 32;           // 32-key blocks per tile
    constexpr int KTILE = TK * RB;         // bytes of one K tile in LDS
    constexpr int VTILE = TK * VRB;        // bytes of one V tile in LDS
    constexpr int SLOT = KTILE + VTILE;    // K tile, then V tile
    constexpr int NKS = D / 16;            // score MFMA steps over D
    constexpr int ND = D / 32;             // 32-row blocks of O^T
    constexpr int BR = 32 * NW;            // query rows per workgroup
    constexpr int NDMA = VTILE / 16 / NT;  // 16-byte copies per thread per tensor per tile
    static_assert(NDMA >= 1 && VTILE % (16 * NT) == 0, "tile staging");
    constexpr int NK8 = TK * GRB / 16 / NT;   // e4m3: 16-byte K chunks each thread widens per tile

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = lane >> 4, cl = lane & 15;   // 16-lane group of the transposing reads

    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;
    const int r0 = qt * BR;
    const int r1 = min(r0 + BR, Nq);
    int kv_lo, kv_hi;
    kv_range(r0, r1, Nq, Nk, wl, wr, &kv_lo, &kv_hi);
    int t_lo = kv_lo / TK, t_hi = (kv_hi > kv_lo) ? (kv_hi + TK - 1) / TK : kv_lo / TK;
    if (p.n_split > 1) {
        // split s takes tiles [t_lo + nt*s/S, t_lo + nt*(s+1)/S) of the workgroup's range
        const long long nt = t_hi - t_lo;
        const int a = t_lo + (int)(nt * split / p.n_split), b = t_lo + (int)(nt * (split + 1) / p.n_split);
        t_lo = a;
        t_hi = b;
    }
    // Row block of this wave. Waves w and w + 4 share a SIMD; with eight waves
    // the second of each pair takes the mirrored block (7 - w), so that under
    // a causal mask every SIMD carries the same number of the diagonal tiles'
    // blocks (w + 1 and 8 - w).
    const int rblk = (NW == 8 && wave >= 4) ? 11 - wave : wave;
    const int w0 = r0 + rblk * 32;
    const int w1 = min(w0 + 32, Nq);

    const uint8_t* qp = p.q + (size_t)bh * Nq * GRB;
    const uint8_t* kp = p.k + (size_t)bh * Nk * GRB;
    const uint8_t* vp = p.v + (size_t)bh * Nk * GRB;

    // Q fragments, B operand of S^T = K Q^T: lane holds query w0 + l32,
    // head-dim elements [16s + 8hh, +8) (e4m3: widened to bf16). Rows at or
    // past Nq read as zeros.
    i32x4 qf[NKS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)(Nq * GRB));
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            if constexpr (!FP8) {
                qf[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    qrs, (w0 + l32) * GRB + (16 * s + 8 * hh) * 2, 0, 0));
            } else {
                const i32x2 w8 = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(
                    qrs, (w0 + l32) * GRB + 16 * s + 8 * hh, 0, 0));
                const i32x2 a = e4m3x4_to_bf16(w8[0]), b = e4m3x4_to_bf16(w8[1]);
                qf[s] = i32x4{a[0], a[1], b[0], b[1]};
            }
        }
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
    float m = -INFINITY;   // the row's reference (base-2 units); -inf: none yet
    float lh = 0.f;        // this lane half's weight sum (16-bit inputs: a third of it)
    const float c2 = p.c;  // scale * log2(e): scores in base-2 units

    // ---- score modifiers, in base-2 units
    [[maybe_unused]] const float sc_k1 = p.mk1;        // softcap: e^(2x) = 2^(sc_k1 s), x = scale * s / cap
    [[maybe_unused]] const float sc_k2 = p.mk2;        // softcap: cap * log2(e)
    float slope2 = 0.f;                                // ALiBi: this head's slope * log2(e)
    if constexpr (MOD == MOD_ALIBI) slope2 = p.slopes[bh % p.H] * LOG2E;
    // ALiBi: the bias of element r of lane half hh at its place in the block,
    // slope * (8(r/4) + r%4 + 4hh), starts the score accumulator, in score
    // units (the fold), unless slope / scale is too large to stay finite there
    // (alibi_fold); then every exponent argument adds it.
    constexpr bool fold = FOLD;
    f32x16 sinit = {};
    if constexpr (MOD == MOD_ALIBI) {
        const float kb = fold ? slope2 / c2 : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sinit[r] = kb * (float)(8 * (r >> 2) + (r & 3) + 4 * hh);
    }
    // ALiBi with a nonzero slope: the reference is preset from the block with
    // the largest bias (below), and the blocks before it may hold weights that
    // round to zero against it. A row's final sum is at least 1 against its
    // reference, so the residual pass then compares against max(lh, 1).
    // res_floor is a third of that floor (lh is kept in thirds).
    const bool floor1 = (MOD == MOD_ALIBI) && slope2 != 0.f;
    auto res_floor = [&]() __attribute__((always_inline)) { return floor1 ? fmaxf(lh, 1.f / 3.f) : lh; };
    // min(res_floor, SUM_LIMIT): a block whose lane-half sum exceeds it takes the rare path
    float thr = floor1 ? (1.f / 3.f) : 0.f;

    // ---- K/V copies: lane l of a wave fills the l-th 16-byte slot of a 1 KiB
    // run of the tile, fetching the global chunk that belongs there under the
    // swizzled layout; rows at or past Nk read as zeros. e4m3: V's rows are
    // stored permuted (v8_row), so that each lane half's 32 keys are 32
    // consecutive LDS rows for the 8-bit transposing reads, and K passes
    // through registers (stk), to be widened to bf16 on its way into LDS
    // after the tile's blocks (finish_tile).
    const i32x4 kwords = rsrc_words(kp, (unsigned)(Nk * GRB));
    const i32x4 vwords = rsrc_words(vp, (unsigned)(Nk * GRB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    static_assert((NT / CPR) % 16 == 0 && (NT / VCPR) % 8 == 0, "copy rows");
    const unsigned dma_voff = [&] {
        const int slot = 64 * wave + lane;
        const int x = slot / CPR, c = (slot % CPR) ^ swz16<RB>(x);
        return (unsigned)(x * RB + c * 16);
    }();
    // e4m3 V: copy i of a lane fills LDS row xv = slot / VCPR + i * NT / VCPR
    // with key v8_row_inv(xv); the keys of copy i > 0 are those of copy 0
    // moved by a multiple of 4 (xv moves by a multiple of 32), so one
    // per-lane offset serves every copy.
    const unsigned dma_voff8 = [&] {
        const int slot = 64 * wave + lane;
        constexpr int VSW = VCPR < 8 ? VCPR : 8;   // the swizzle of lds_off<VRB>
        const int xv = slot / VCPR, c = (slot % VCPR) ^ (xv & (VSW - 1));
        return (unsigned)(v8_row_inv(xv) * VRB + c * 16);
    }();
    [[maybe_unused]] i32x4 stk[FP8 ? NK8 : 1];
    const __amdgpu_buffer_rsrc_t krs8 = make_rsrc(kp, (unsigned)(Nk * GRB));
    auto issue_tile = [&](int t) {
        const unsigned kb = smem_base + (unsigned)((t & 1) * SLOT);
        if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                const int run = 64 * wave + NT * i;
                const unsigned soff = (unsigned)((t * TK + i * (NT / CPR)) * RB);
                dma16(kwords, kb + run * 16, dma_voff, soff);
                dma16(vwords, kb + KTILE + run * 16, dma_voff, soff);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NK8; ++i) {
                const int ci = tid + NT * i;
                const int x = ci / (GRB / 16), c = ci % (GRB / 16);
                stk[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    krs8, (t * TK + x) * GRB + c * 16, 0, 0));
            }
#pragma unroll
            for (int i = 0; i < NDMA; ++i) {
                const int run = 64 * wave + NT * i;
                // copy i fills LDS rows xv0 + (0 .. NT / VCPR - 1), xv0 a
                // multiple of 32: whole 64-key groups move the keys by 64 each,
                // and 32 rows within a group by 4 (v8_row_inv)
                const int xv0 = i * (NT / VCPR);
                const unsigned soff = (unsigned)((t * TK + ((xv0 >> 6) << 6) + (((xv0 >> 5) & 1) << 2)) * VRB);
                dma16(vwords, kb + KTILE + run * 16, dma_voff8, soff);
            }
        }
    };
    // e4m3: the K chunks of tile t have landed in registers (with the V
    // copies issued beside them); widen them and write them to the tile's
    // slot. Every wave is past tile t-2, the slot's previous tile.
    auto finish_tile = [&](int t) __attribute__((always_inline)) {
        if constexpr (FP8) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            uint8_t* kb = smem + (t & 1) * SLOT;
#pragma unroll
            for (int i = 0; i < NK8; ++i) {
                const int ci = tid + NT * i;
                const int x = ci / (GRB / 16), c = ci % (GRB / 16);
                const i32x2 a = e4m3x4_to_bf16(stk[i][0]), b = e4m3x4_to_bf16(stk[i][1]);
                const i32x2 e = e4m3x4_to_bf16(stk[i][2]), f = e4m3x4_to_bf16(stk[i][3]);
                *reinterpret_cast<i32x4*>(kb + lds_pos<RB>(x, 2 * c)) = i32x4{a[0], a[1], b[0], b[1]};
                *reinterpret_cast<i32x4*>(kb + lds_pos<RB>(x, 2 * c + 1)) = i32x4{e[0], e[1], f[0], f[1]};
            }
        }
    };

    // ---- block classes. Wave: [jf0, jf1) every pair visible, [ju0, ju1) at
    // least one. Workgroup: tiles [ts0, ts1) in which both blocks are fully
    // visible to every wave that holds rows.
    int jf0, jf1, ju0, ju1;
    block_ranges32(w0, w1, Nq, Nk, wl, wr, &jf0, &jf1, &ju0, &ju1);
    int f0 = 0, f1 = 1 << 30;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        const int a0 = r0 + 32 * ww, a1 = min(a0 + 32, Nq);
        if (a1 <= a0) continue;
        int x0, x1, y0, y1;
        block_ranges32(a0, a1, Nq, Nk, wl, wr, &x0, &x1, &y0, &y1);
        f0 = max(f0, x0);
        f1 = min(f1, x1);
    }
    auto block_skip = [&](int j) { return (unsigned)(j - ju0) >= (unsigned)(ju1 - ju0); };
    auto block_full = [&](int j) { return (unsigned)(j - jf0) < (unsigned)(jf1 - jf0); };

    // ---- LDS addresses. Element r of lane (l32, hh) in S^T of sub-tile j is
    // key 32j + 8(r/4) + 4hh + r%4 against query w0 + l32. The per-lane parts
    // of the addresses are fixed; slot, sub-tile and MFMA step are immediate
    // offsets (the swizzle depends on the row mod 16, which those multiples
    // of 16 rows leave unchanged).
    int kofs[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kofs[s] = lds_pos<RB>(l32, 2 * s + hh);
    int vofs[ND][2];   // transposing V reads: rows 4hh + cl/4 and 8 rows further
    if constexpr (!FP8) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) vofs[db][h8] = lds_pos<RB>(4 * hh + (cl >> 2) + 8 * h8, ch) + 8 * (cl & 1);
        }
    } else {
        // e4m3: the 8-bit transposing reads of LDS rows 32hh + 8u + cl/2
        // (u = 0..3, an immediate offset), head-dim columns 32db + 16(g%2)
        // + 8(cl%2) .. +8; the swizzle depends on the row mod 8 only
#pragma unroll
        for (int db = 0; db < ND; ++db)
            vofs[db][0] = lds_off<VRB>(32 * hh + (cl >> 1), (32 * db + 16 * (g & 1)) >> 4) + 8 * (cl & 1);
    }
    const lds_u8* lds0 = (const lds_u8*)smem;

    // S^T of sub-tile jj (0 .. SUB-1) of the tile in slot PAR.
    auto scores = [&](auto par, int jj, f32x16& S) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        const lds_u8* kb = lds0 + PAR * SLOT + 32 * jj * RB;
        i32x4 a[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) a[s] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(kb + kofs[s]);
        if constexpr (MOD == MOD_ALIBI) {
            S = sinit;
        } else {
            S = f32x16{};
        }
#pragma unroll
        for (int s = 0; s < NKS; ++s) S = mfma16(QK, a[s], qf[s], S);
    };
    // V^T operands of sub-tile jj for its two 16-key MFMA steps, in the key
    // order P has: step sp, lane half hh, k-slot e holds key
    // 32j + 16sp + 8(e/4) + 4hh + e%4 (two transposing reads of 4 rows).
    auto v_operands = [&](auto par, int jj, i32x4(&va)[2][ND]) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        const lds_u8* vb = lds0 + PAR * SLOT + KTILE + 32 * jj * RB;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const i32x2 u0 = read_tr16(vb + 16 * sp * RB + vofs[db][0]);
                const i32x2 u1 = read_tr16(vb + 16 * sp * RB + vofs[db][1]);
                va[sp][db] = i32x4{u0[0], u0[1], u1[0], u1[1]};
            }
    };
    auto pv = [&](const i32x4(&va)[2][ND], const i32x4(&P)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[db] = mfma16(IN, va[sp][db], P[sp], oacc[db]);
    };
    // e4m3: O^T += V^T P^T over the 64 keys of the tile in slot PAR; word w
    // of pf holds the e4m3 weights of sub-tile w/4, accumulator elements
    // 4(w%4) .. +3, and the V^T operand comes from four 8-bit transposing
    // reads of the lane half's 32 (permuted) rows.
    auto pv8 = [&](auto par, int grp, const i32x8& pf) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        const lds_u8* vb = lds0 + PAR * SLOT + KTILE + 64 * grp * VRB;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            i32x8 a;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(vb + vofs[db][0] + 8 * u * VRB));
                a[2 * u] = r[0];
                a[2 * u + 1] = r[1];
            }
            oacc[db] = mfma_fp8(a, pf, oacc[db]);
        }
    };

    // Masked scores of sub-tile j become -inf: row i = w0 + l32 sees keys
    // [klo, khi) (none when i is past the wave's rows).
    auto mask = [&](int j, f32x16& S) __attribute__((always_inline)) {
        const int c0 = 32 * j;
        int ln = lane;
        asm volatile("" : "+v"(ln));   // recomputed here, not held across the loop
        const int i = w0 + (ln & 31);
        const int ip = i + (Nk - Nq);
        int klo = ip - wl;
        int khi = ip + wr + 1;
        klo = klo > 0 ? klo : 0;
        khi = khi < Nk ? khi : Nk;
        if (i >= w1) khi = klo;
        const int a = klo - c0 - 4 * (ln >> 5), b = khi - c0 - 4 * (ln >> 5);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            S[r] = (off < a || off >= b) ? -INFINITY : S[r];
        }
    };

    // The exponent arguments of block j against the reference ref: the score
    // in base-2 units, modified, minus ref.
    //   none:    c * s - ref
    //   ALiBi:   c * s' + slope * log2(e) * (32j - i') - ref, where s' holds
    //            the in-block part of the bias (the fold), else that part is
    //            added here
    //   softcap: cap * log2(e) * tanh(scale * s / cap) - ref, with
    //            tanh x = 1 - 2 / (e^(2x) + 1), which holds for every x (u =
    //            e^(2x) may round to 0 or to infinity); its rounding leaves
    //            about 1e-5 in the argument at any x. A masked score (-inf)
    //            would give -cap: in edge blocks it is set to -inf.
    auto alibi_add = [&](int j, float ref) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));   // recomputed here, not held across the loop
        const int ip = w0 + (ln & 31) + (Nk - Nq);
        return fmaf(slope2, (float)(32 * j - ip), -ref);
    };
    auto eargs = [&](const f32x16& S, int j, float ref, bool edge, float(&a)[16]) __attribute__((always_inline)) {
        if constexpr (MOD == MOD_NONE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = fmaf(S[r], c2, -ref);
        } else if constexpr (MOD == MOD_ALIBI) {
            const float na = alibi_add(j, ref);
            if constexpr (fold) {
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = fmaf(S[r], c2, na);
            } else {
                const float nb = fmaf(slope2, (float)(4 * hh), na);
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = fmaf(S[r], c2, fmaf(slope2, (float)(8 * (r >> 2) + (r & 3)), nb));
            }
        } else {
            const float top = sc_k2 - ref;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float u = __builtin_amdgcn_exp2f(S[r] * sc_k1);
                a[r] = fmaf(__builtin_amdgcn_rcpf(u + 1.f), -2.f * sc_k2, top);
            }
            if (edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = (S[r] == -INFINITY) ? -INFINITY : a[r];
            }
        }
    };
    // The row max of block j's modified scores in base-2 units (both lane
    // halves; -inf where the row sees none of its keys).
    auto row_max = [&](const f32x16& S, int j, bool edge) __attribute__((always_inline)) {
        float mx;
        if constexpr (MOD == MOD_NONE || MOD == MOD_ALIBI) {
            mx = S[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        }
        if constexpr (MOD == MOD_NONE) {
            return max_halves(mx) * c2;
        } else {
            if constexpr (MOD == MOD_ALIBI && fold) {
                // the arguments rise with s': the max is that of the largest
                mx = fmaf(mx, c2, alibi_add(j, 0.f));
            } else {
                float a[16];
                eargs(S, j, 0.f, edge, a);
                mx = a[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, a[r]);
            }
            return max_halves(mx);
        }
    };

    // p = 2^(c*s - ms) (modified) for the 16 scores of block j, their sum (a
    // fixed pairwise order) and p rounded to the MFMA type.
    auto softmax = [&](const f32x16& S, int j, float ms, bool edge, float(&pr)[16], float& ts, i32x4(&P)[2])
        __attribute__((always_inline)) {
        {
            float a[16];
            eargs(S, j, FP8 ? ms - LOG2_PRESCALE8 : ms, edge, a);
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(a[r]);
        }
        float s8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) s8[r] = pr[2 * r] + pr[2 * r + 1];
        ts = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
        if constexpr (!FP8) {
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const int o = 8 * sp;
                P[sp] = i32x4{pack2<IN>(pr[o + 0], pr[o + 1]), pack2<IN>(pr[o + 2], pr[o + 3]),
                              pack2<IN>(pr[o + 4], pr[o + 5]), pack2<IN>(pr[o + 6], pr[o + 7])};
            }
        } else {
            // e4m3 of the (scaled) weights, four per word, in P[0]
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                int word = __builtin_amdgcn_cvt_pk_fp8_f32(pr[4 * w], pr[4 * w + 1], 0, false);
                word = __builtin_amdgcn_cvt_pk_fp8_f32(pr[4 * w + 2], pr[4 * w + 3], word, true);
                P[0][w] = word;
            }
            P[1] = i32x4{};
        }
    };
    // The rounding residual of the weights, lo = p - P rounded to the MFMA
    // type (zero where on is false).
    auto residual = [&](const float(&pr)[16], const i32x4(&P)[2], bool on, i32x4(&lo)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int o = 8 * sp;
            const i32x4 h = P[sp];
            const i32x4 d = i32x4{pack2<IN>(pr[o + 0] - unpack_lo<IN>(h[0]), pr[o + 1] - unpack_hi<IN>(h[0])),
                                  pack2<IN>(pr[o + 2] - unpack_lo<IN>(h[1]), pr[o + 3] - unpack_hi<IN>(h[1])),
                                  pack2<IN>(pr[o + 4] - unpack_lo<IN>(h[2]), pr[o + 5] - unpack_hi<IN>(h[2])),
                                  pack2<IN>(pr[o + 6] - unpack_lo<IN>(h[3]), pr[o + 7] - unpack_hi<IN>(h[3]))};
            lo[sp] = i32x4{on ? d[0] : 0, on ? d[1] : 0, on ? d[2] : 0, on ? d[3] : 0};
        }
    };

    // The exact redo of a block for the rows whose reference must move (no
    // reference yet, or a lane half's sum above SUM_LIMIT): their max over
    // the block's visible keys becomes the reference, O and the sums are
    // rescaled, and the weights are formed again. S holds the block's
    // (masked) scores. Rows whose reference does not move form the same bits
    // again, so a row's result depends on its own scores alone.
    auto redo = [&](const f32x16& S, int j, bool edge, bool trig, float(&pr)[16], float& ts, i32x4(&P)[2])
        __attribute__((always_inline)) {
        const unsigned tr = trig ? 1u : 0u;
        auto pw = __builtin_amdgcn_permlane32_swap(tr, tr, false, false);
        const bool row = (pw[0] | pw[1]) != 0;
        const float mx = row_max(S, j, edge);
        const float mnew = row ? fmaxf(m, mx) : m;
        const bool mv = mnew != m;
        const float alpha = mv ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
        m = mnew;
        if (__builtin_amdgcn_ballot_w64(mv) != 0) {
            lh *= alpha;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
        }
        softmax(S, j, (mnew == -INFINITY) ? 0.f : mnew, edge, pr, ts, P);
    };

    // ---- one block: sub-tile jj of the tile in slot PAR, key block j.
    // MODE 0: steady (fully visible, no checks but the one compare);
    // MODE 1: checked (skip / edge classes); MODE 2: checked and early (the
    // residual pass on every lane).
    // e4m3: the tile's weights (pv8's pf) and whether a block of the tile ran
    [[maybe_unused]] i32x8 pf8 = {};
    [[maybe_unused]] bool live8 = false;
    auto block = [&](auto par, auto mode, int jj, int j) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode)::value;
        bool edge = false;
        if constexpr (MODE != 0) {
            if (block_skip(j)) return;
            edge = !block_full(j);
        }
        f32x16 S;
        scores(par, jj, S);
        if constexpr (MODE != 0) {
            if (edge) mask(j, S);
        }
        if constexpr (FP8) {
            // no residual pass; the reference moves when a lane half's sum
            // exceeds SUM_LIMIT8. Sub-tile 0's weights wait for P.V at the end
            // of the tile: before sub-tile 1 moves the reference (and rescales
            // O), they are multiplied in against the reference they were formed
            // with.
            live8 = true;
            float pr[16], ts;
            i32x4 P[2];
            softmax(S, j, m, edge, pr, ts, P);
            // (the register budget of two waves per SIMD keeps the scores, so
            // the redo does not form them again)
            const bool trig = !(ts <= SUM_LIMIT8);
            if (__builtin_amdgcn_ballot_w64(trig) != 0) {
                if (jj & 1) {
                    pv8(par, jj >> 1, i32x8{pf8[0], pf8[1], pf8[2], pf8[3], 0, 0, 0, 0});
                    pf8[0] = pf8[1] = pf8[2] = pf8[3] = 0;
                }
                redo(S, j, edge, trig, pr, ts, P);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) pf8[4 * (jj & 1) + w] = P[0][w];
            lh += ts;
            return;
        }
        i32x4 va[2][ND];
        v_operands(par, jj, va);
        float pr[16], ts;
        i32x4 P[2];
        // m = -inf (no reference yet) gives ts = inf or NaN: the redo runs
        softmax(S, j, m, edge, pr, ts, P);
        if (__builtin_amdgcn_ballot_w64(!(ts <= thr)) != 0) {
            const bool trig = !(ts <= SUM_LIMIT);
            if (__builtin_amdgcn_ballot_w64(trig) != 0) {
                f32x16 S2;
                scores(par, jj, S2);
                if constexpr (MODE != 0) {
                    if (edge) mask(j, S2);
                }
                redo(S2, j, edge, trig, pr, ts, P);
            }
            if constexpr (MODE != 2) {
                const bool sr = ts > res_floor();
                if (__builtin_amdgcn_ballot_w64(sr) != 0) {
                    i32x4 lo[2];
                    residual(pr, P, sr, lo);
                    pv(va, lo);
                }
            }
        }
        if constexpr (MODE == 2) {
            i32x4 lo[2];
            residual(pr, P, true, lo);
            pv(va, lo);
        }
        lh = fmaf(ts, 1.f / 3.f, lh);
        thr = fminf(res_floor(), SUM_LIMIT);
        pv(va, P);
    };

    // ---- tiles: the copies of tile t landed (each wave waits for its own,
    // the barrier for everyone's), every wave is past tile t-1, so tile t+1
    // goes into t-1's slot; then the sub-tiles of tile t.
    auto tile = [&](auto par, auto mode, int t) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
        if (t + 1 < t_hi) issue_tile(t + 1);
        if constexpr (FP8) {
            pf8 = i32x8{};
            live8 = false;
        }
#pragma unroll
        for (int jj = 0; jj < SUB; ++jj) {
            block(par, mode, jj, SUB * t + jj);
            if constexpr (FP8) {
                // P.V of each 64-key group once both its sub-tiles have weights
                if (jj & 1) {
                    if (live8) pv8(par, jj >> 1, pf8);
                    pf8 = i32x8{};
                    live8 = false;
                }
            }
        }
        if constexpr (FP8) {
            if (t + 1 < t_hi) finish_tile(t + 1);
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    auto run = [&](auto mode, int ta, int tb) __attribute__((always_inline)) {
        int t = ta;
        if (t < tb && (t & 1)) {
            tile(P1{}, mode, t);
            ++t;
        }
        for (; t + 1 < tb; t += 2) {
            tile(P0{}, mode, t);
            tile(P1{}, mode, t + 1);
        }
        if (t < tb) tile(P0{}, mode, t);
    };

    // ---- ALiBi: under a bias that grows with the key index the row max climbs
    // by slope * 32 per block, so a reference taken from the first block would
    // be passed, and the exact redo taken, on nearly every block. The
    // reference starts instead at the row max of the wave's block with the
    // largest bias (its last block with a visible key for a positive slope,
    // its first for a negative one), with K read straight from HBM: the same
    // scores, bit for bit, as the loop forms for that block. Rows that see no
    // key of it keep m = -inf.
    if constexpr (MOD == MOD_ALIBI) {
        const int jl = slope2 > 0.f ? ju1 - 1 : ju0;
        if (floor1 && ju1 > ju0 && jl >= SUB * t_lo && jl < SUB * t_hi) {
            const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)(Nk * RB));
            i32x4 a[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                a[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    krs, (32 * jl + l32) * RB + (16 * s + 8 * hh) * 2, 0, 0));
            f32x16 S = sinit;
#pragma unroll
            for (int s = 0; s < NKS; ++s) S = mfma16(QK, a[s], qf[s], S);
            mask(jl, S);
            m = row_max(S, jl, true);
        }
    }

    // e4m3 takes no residual pass: no early tiles
    const int tE = FP8 ? t_lo : min(t_hi, t_lo + (EARLY_KEYS + TK - 1) / TK);
    const int tS0 = min(t_hi, max(tE, (f0 + SUB - 1) / SUB));
    const int tS1 = max(tS0, min(t_hi, f1 / SUB));
    if (t_lo < t_hi) {
        issue_tile(t_lo);
        finish_tile(t_lo);
    }
    if constexpr (!FP8) run(std::integral_constant<int, 2>{}, t_lo, tE);
    if constexpr (MOD == MOD_ALIBI && !FOLD) {
        // the ALiBi form without the fold (rare): every tile checked, which
        // keeps this kernel's code small
        run(std::integral_constant<int, 1>{}, tE, t_hi);
    } else {
        run(std::integral_constant<int, 1>{}, tE, tS0);
        run(std::integral_constant<int, 0>{}, tS0, tS1);
        run(std::integral_constant<int, 1>{}, tS1, t_hi);
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l); a split writes both
    // in fp32 to its slice of the workspace instead
    const float lt = FP8 ? sum_halves(lh) : sum_halves(lh) * 3.f;
    const int i = w0 + l32;
    if (p.n_split > 1) {
        const size_t sl = (size_t)bh * p.n_split + split;
        float* wo = p.ws_o + sl * Nq * D;
        float* wlp = p.ws_lse + sl * Nq;
        if (i < w1) {
            const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
            uint8_t* orow = (uint8_t*)(wo + (size_t)i * D);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x16& a = oacc[db];
                    const int d = 32 * db + 8 * r4 + 4 * hh;
                    Out<OUT_F32>::store4(orow + d * 4, a[4 * r4] * inv, a[4 * r4 + 1] * inv, a[4 * r4 + 2] * inv,
                                         a[4 * r4 + 3] * inv);
                }
            if (hh == 0) wlp[i] = (lt > 0.f) ? (m + __builtin_amdgcn_logf(lt) - (FP8 ? LOG2_PRESCALE8 : 0.f)) * LN2 : -INFINITY;
        }
        clock_stamp(p.clk, p.clk_n, 1);
        return;
    }
    uint8_t* op = p.o + (size_t)bh * Nq * D * Out<OUT>::EB;
    float* lp = p.lse + (size_t)bh * Nq;
    if (i < w1) {
        const float inv = (lt > 0.f) ? p.out_mul / lt : 0.f;
        uint8_t* orow = op + (size_t)i * D * Out<OUT>::EB;
        if constexpr (Out<OUT>::EB == 2) {
            // 16-byte stores: element r of oacc[db] is column 32db + 8(r/4) +
            // 4hh + r%4 of row i, so lanes l and l ^ 32 hold the two 4-column
            // halves of each 8 columns. One exchange of 8 bytes gives lane hh
            // the 8 columns 32db + 16k + 8hh .. +7 of each 16 (k = 0, 1).
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const f32x16& a = oacc[db];
                    const int ra = 8 * k, rb = 8 * k + 4;
                    const i32x2 A = Out<OUT>::pack4(a[ra] * inv, a[ra + 1] * inv, a[ra + 2] * inv, a[ra + 3] * inv);
                    const i32x2 B = Out<OUT>::pack4(a[rb] * inv, a[rb + 1] * inv, a[rb + 2] * inv, a[rb + 3] * inv);
                    // lane hh = 0 takes the other half's A, lane hh = 1 the other half's B
                    const int x0 = __shfl_xor(hh ? A[0] : B[0], 32), x1 = __shfl_xor(hh ? A[1] : B[1], 32);
                    const i32x4 v = hh ? i32x4{x0, x1, B[0], B[1]} : i32x4{A[0], A[1], x0, x1};
                    *reinterpret_cast<i32x4*>(orow + (32 * db + 16 * k + 8 * hh) * 2) = v;
                }
        } else {
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x16& a = oacc[db];
                    const int d = 32 * db + 8 * r4 + 4 * hh;
                    Out<OUT>::store4(orow + d * Out<OUT>::EB, a[4 * r4] * inv, a[4 * r4 + 1] * inv,
                                     a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv);
                }
        }
        if (hh == 0) lp[i] = (lt > 0.f) ? (m + __builtin_amdgcn_logf(lt) - (FP8 ? LOG2_PRESCALE8 : 0.f)) * LN2 : -INFINITY;
    }
    clock_stamp(p.clk, p.clk_n, 1);
}

// Whether head bh's ALiBi bias folds into the score accumulator: slope /
// scale times the largest in-block offset (31) must stay far inside fp32's
// range.
__device__ __forceinline__ bool alibi_fold(const Params& p, int bh) {
    return fabsf(p.slopes[bh % p.H] * LOG2E) <= p.c * 0x1p64f;
}

// With ALiBi the kernel is launched twice on the stream, FOLD true and false,
// so that each kernel holds one form of the loop (a kernel holding both ran
// measurably slower). The FOLD launch has the usual grid and its workgroups
// leave heads without the fold at once; the other launch has one workgroup
// per head, which leaves at once where the head folds (the usual case) and
// otherwise walks the head's query tiles one after another.
template <int IN, int OUT, int D, int NW, int TK, int MOD, bool FOLD>
__global__ __launch_bounds__(64 * NW, serial::waves_per_simd<D>()) void fa_fwd_serial_kernel(Params p) {
    // two slots of a K tile (16-bit in LDS) and a V tile (the input type)
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (TK * D * 2 + TK * D * (IN == IN_E4M3 ? 1 : 2))];
    if constexpr (MOD == MOD_ALIBI && !FOLD) {
        const int bh = blockIdx.x;
        if (alibi_fold(p, bh)) return;
        for (int qt = 0; qt < p.n_qt; ++qt) {
            serial_body<IN, OUT, D, NW, TK, MOD, FOLD>(p, smem, bh, qt, 0);
            __syncthreads();   // every wave is done with the LDS slots before the next tile's copies
        }
    } else {
        int bh, qt, split;
        serial_wg(p, &bh, &qt, &split);
        if constexpr (MOD == MOD_ALIBI) {
            if (!alibi_fold(p, bh)) return;
        }
        clock_stamp(p.clk, p.clk_n, 0);
        serial_body<IN, OUT, D, NW, TK, MOD, FOLD>(p, smem, bh, qt, split);
    }
}

// ---------------------------------------------------------------- host side

template <int IN, int OUT, int D, int NW, int TK, int MOD>
static int launch_serial_one(const Plan& pl, const Params& p, hipStream_t s) {
    const dim3 grid((unsigned)(pl.n_wg * p.n_split)), block(64 * NW);
    if constexpr (MOD == MOD_ALIBI) {
        // ALiBi takes no split (the split-KV entry points have no modifier)
        if (p.n_split != 1) return (int)hipErrorInvalidValue;
        hipLaunchKernelGGL((fa_fwd_serial_kernel<IN, OUT, D, NW, TK, MOD, true>), grid, block, 0, s, p);
        const int e = (int)hipGetLastError();
        if (e != 0) return e;
        hipLaunchKernelGGL((fa_fwd_serial_kernel<IN, OUT, D, NW, TK, MOD, false>), dim3((unsigned)p.n_bh), block, 0,
                           s, p);
        return (int)hipGetLastError();
    }
    hipLaunchKernelGGL((fa_fwd_serial_kernel<IN, OUT, D, NW, TK, MOD, false>), grid, block, 0, s, p);
    return (int)hipGetLastError();
}

// The shapes make_plan (fa_fwd.hip) gives the serial kernel at head size D:
// FA_SR_NW_D64 or FA_SR_NW_D128 waves with their tile size, and four waves
// with 64-key tiles where eight would leave CUs without a workgroup.
template <int IN, int OUT, int D, int MOD>
static int launch_serial_d(const Plan& pl, const Params& p, hipStream_t s) {
    constexpr int NWD = D == 64 ? FA_SR_NW_D64 : FA_SR_NW_D128;
    constexpr int TKD = serial_tile_keys(IN, D, NWD);
    if (pl.nw == NWD && pl.bc == TKD) return launch_serial_one<IN, OUT, D, NWD, TKD, MOD>(pl, p, s);
    if constexpr (NWD == 8) {
        if (pl.nw == 4 && pl.bc == 64) return launch_serial_one<IN, OUT, D, 4, 64, MOD>(pl, p, s);
    }
    return (int)hipErrorInvalidValue;
}

template <int IN, int MOD>
int launch_serial_in(const Plan& pl, const Params& p, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    // 16-bit inputs write their own type or fp32, e4m3 inputs bf16
    constexpr int OUT16 = IN == IN_F16 ? OUT_F16 : OUT_BF16;
    constexpr bool F32 = IN != IN_E4M3;
    if (pl.out != OUT16 && !(F32 && pl.out == OUT_F32)) return (int)hipErrorInvalidValue;
    if (pl.D == 64) {
        if (pl.out == OUT16) return launch_serial_d<IN, OUT16, 64, MOD>(pl, p, s);
        if constexpr (F32) return launch_serial_d<IN, OUT_F32, 64, MOD>(pl, p, s);
    }
    if (pl.D == 128) {
        if (pl.out == OUT16) return launch_serial_d<IN, OUT16, 128, MOD>(pl, p, s);
        if constexpr (F32) return launch_serial_d<IN, OUT_F32, 128, MOD>(pl, p, s);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
