// Fused exact-attention forward for 16-bit inputs (fp16, bf16) on gfx950,
// software-pipelined over blocks of 32 queries x 32 keys.
//
// The computation is the block-by-block loop of the aiinarabic.com
// flash-attention page (load a block of K and V on chip, score it, softmax it,
// multiply by V, merge), with the running max and sum of the FLASHLIGHT
// summary on gist.science (Methodology item 3). It is reorganised so that the
// matrix cores and the vector ALU work at the same time inside one wave.
//
// A wave owns QB blocks of 32 query rows. Its work is a sequence of steps
// u = QB*j + qb, one per (32-key sub-tile j, query block qb). Step u runs, in
// one straight-line block:
//   * the softmax VALU work of block u (exponentials, row sums, rounding to
//     the 16-bit MFMA type), whose scores were formed in step u-1,
//   * the score MFMAs of block u+1 (S^T = K Q^T),
//   * the P.V MFMAs of block u-1 (O^T += V^T P^T).
// The three are independent, so the MFMA pipe and the VALU overlap; per step
// the MFMA work and the VALU work are of similar length.
//
// No row max on the common path. Every row keeps a reference m; a lane forms
// p = 2^(c*s - m) for its 16 scores of the row and sums them. If a lane half's
// sum exceeds SUM_LIMIT (a score has grown well past m) or the lane half has no
// weight yet, the step is redone exactly: the row max is taken across both
// lane halves, m moves up to it (the
// accumulator and the sums are rescaled by 2^(m_old - m_new)) and p is formed
// again. Rows whose m does not move form the same bits again, so a row's
// result depends on its own scores alone; O / l and the log-sum-exp do not
// depend on which m was used. Blocks on a mask edge take the same path after
// their masked scores are set to -inf.
//
// P's rounding residual (P = hi + lo, both 16-bit) also multiplies V in a step
// where a lane half's new weight exceeds a quarter of that half's total so
// far -- the first sub-tiles of a row and peaked rows -- so no dominant
// weight's rounding reaches the output.
//
// K and V tiles of 64 keys go HBM -> LDS with direct-to-LDS buffer loads into
// a ring of three slots: the score look-ahead crosses into tile t+1 before
// tile t is finished, and tile t+2 is copied meanwhile. One barrier per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace fa {

constexpr int NSLOT = 3;

// Operand read-ahead with one query block per wave (see the kernel):
// 0 none, 1 V, 2 K and V.
#ifndef FA_RA_D64
#define FA_RA_D64 2
#endif
#ifndef FA_RA_D128
#define FA_RA_D128 1
#endif
// Largest sum of a lane half's 16 weights of one block kept without moving
// the reference max: every weight is then at most 2^10.
constexpr float SUM_LIMIT = 1024.f;
// Tiles at the start of a wave's key range whose steps keep the fp32 weights
// and take the residual pass on every lane (the running sums are small there,
// so most rows need it).
#ifndef FA_EARLY_TILES
#define FA_EARLY_TILES 4
#endif
constexpr int EARLY_TILES = FA_EARLY_TILES;

// Waves per SIMD the register budget is sized for: three with one query
// block per wave at D = 64 (three workgroups' LDS rings fit a CU), else two.
#ifndef FA_WPS_D64
#define FA_WPS_D64 3
#endif
// The score modifiers need more registers: two waves per SIMD. (Softcap's
// polynomial for small arguments spills inside the step at three; ALiBi at
// three spills inside the loop and loses 7%.)
#ifndef FA_WPS_SOFTCAP
#define FA_WPS_SOFTCAP 2
#endif
#ifndef FA_WPS_ALIBI
#define FA_WPS_ALIBI 2
#endif
template <int D, int QB, int MOD>
constexpr int waves_per_simd() {
    if (D != 64 || QB != 1) return 2;
    return MOD == MOD_NONE ? FA_WPS_D64 : (MOD == MOD_SOFTCAP ? FA_WPS_SOFTCAP : FA_WPS_ALIBI);
}

template <int IN, int OUT, int D, int NW, int QB, int MOD>
__global__ __launch_bounds__(64 * NW, (waves_per_simd<D, QB, MOD>())) void fa_fwd16_kernel(Params p) {
    clock_stamp(p.clk, p.clk_n, 0);
    constexpr int NT = 64 * NW;
    constexpr int RB = D * 2;              // bytes per K/V/Q row, in HBM and in LDS
    constexpr int CPR = RB / 16;           // 16-byte chunks per row
    static_assert(RB == 128 || RB == 256, "row size");
    constexpr int TILE = BC * RB;          // bytes of one K or V tile
    constexpr int SLOT = 2 * TILE;         // K tile, then V tile
    constexpr int NKS = D / 16;            // score MFMA steps over D
    constexpr int ND = D / 32;             // 32-row blocks of O^T
    constexpr int QW = 32 * QB;            // query rows per wave
    constexpr int BR = NW * QW;            // query rows per workgroup
    constexpr int NDMA = TILE / 16 / NT;   // 16-byte copies per thread per tensor per tile
    constexpr int SPT = 2 * QB;            // steps per 64-key tile
    static_assert(NDMA >= 1 && TILE % (16 * NT) == 0, "tile staging");

    __shared__ __attribute__((aligned(16))) uint8_t smem[NSLOT * SLOT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = lane >> 4, cl = lane & 15;   // 16-lane group of the transposing reads

    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;
    int bh, qt, split = 0;
    long long wgid = blockIdx.x;
    if (p.n_split > 1) {
        split = (int)(wgid % p.n_split);
        wgid /= p.n_split;
    }
    decode_wg(wgid, p.n_bh, p.n_qt, p.hg, p.tl, &bh, &qt);
    const int r0 = qt * BR;
    const int r1 = min(r0 + BR, Nq);
    int kv_lo, kv_hi;
    kv_range(r0, r1, Nq, Nk, wl, wr, &kv_lo, &kv_hi);
    int tl = kv_lo / BC, th = (kv_hi > kv_lo) ? (kv_hi + BC - 1) / BC : kv_lo / BC;
    if (p.n_split > 1) {
        // split s takes tiles [tl + nt*s/S, tl + nt*(s+1)/S) of the workgroup's range
        const long long nt = th - tl;
        const int a = tl + (int)(nt * split / p.n_split), b = tl + (int)(nt * (split + 1) / p.n_split);
        tl = a;
        th = b;
    }
    const int t_lo = tl, t_hi = th;
    const int w0 = r0 + wave * QW;
    const int w1 = min(w0 + QW, Nq);

    const uint8_t* qp = p.q + (size_t)bh * Nq * RB;
    const uint8_t* kp = p.k + (size_t)bh * Nk * RB;
    const uint8_t* vp = p.v + (size_t)bh * Nk * RB;

    // Q fragments, B operand of S^T = K Q^T: lane holds query w0+32qb+l32,
    // head-dim elements [16s + 8hh, +8).
    i32x4 qf[QB][NKS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)(Nq * RB));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = w0 + 32 * qb + l32;
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                qf[qb][s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    qrs, row * RB + (16 * s + 8 * hh) * 2, 0, 0));
        }
    }

    f32x16 oacc[ND][QB];
    float m[QB], lh[QB];   // reference max (base-2 units) and this lane half's weight sum
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db][qb] = f32x16{};
        m[qb] = -INFINITY;
        lh[qb] = 0.f;
    }
    const float c2 = p.c;
    // Score modifier (MOD_SOFTCAP, MOD_ALIBI): constants in base-2 units.
    const float sc_k1 = p.mk1;   // softcap: e^(2|x|) = 2^(sc_k1 |s|), x = scale * s / cap
    const float sc_k2 = p.mk2;   // softcap: cap * log2(e)
    const SoftcapPoly scp = p.scp;   // softcap on small arguments (fa_device.h)
    float slope2 = 0.f;          // ALiBi: this head's slope * log2(e)
    if constexpr (MOD == MOD_ALIBI) slope2 = p.slopes[bh % p.H] * LOG2E;
    // ALiBi with a nonzero slope presets the reference (wave-uniform)
    const bool alibi_ref = (MOD == MOD_ALIBI) && slope2 != 0.f;

    // ---- K/V copies: lane l of a wave fills the l-th 16-byte slot of a 1 KiB
    // run of the tile, fetching the global chunk that belongs there under the
    // swizzled layout; rows at or past Nk read as zeros.
    const i32x4 kwords = rsrc_words(kp, (unsigned)(Nk * RB));
    const i32x4 vwords = rsrc_words(vp, (unsigned)(Nk * RB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    // Copy i of a lane fills tile row x + i*NT/CPR: the swizzle depends on the
    // row mod 16 and NT/CPR is a multiple of 16, so one per-lane offset serves
    // every copy and every tile; the rest is a wave-uniform offset.
    static_assert((NT / CPR) % 16 == 0, "copy rows");
    const unsigned dma_voff = [&] {
        const int slot = 64 * wave + lane;
        const int x = slot / CPR, c = (slot % CPR) ^ swz16<RB>(x);
        return (unsigned)(x * RB + c * 16);
    }();
    auto issue_tile = [&](int t) {
        const unsigned kb = smem_base + (unsigned)((t % NSLOT) * SLOT);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int run = 64 * wave + NT * i;
            const unsigned soff = (unsigned)((t * BC + i * (NT / CPR)) * RB);
            dma16(kwords, kb + run * 16, dma_voff, soff);
            dma16(vwords, kb + TILE + run * 16, dma_voff, soff);
        }
    };
    auto tile_lds = [&](int t) { return (const lds_u8*)(smem + (t % NSLOT) * SLOT); };
    // Class of block (j, qb), rows of query block qb x keys of sub-tile j,
    // from two sub-tile ranges per query block: [jf0, jf1) has every pair
    // visible, [ju0, ju1) at least one (the same answers as tile_class).
    int jf0[QB], jf1[QB], ju0[QB], ju1[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int a0 = w0 + 32 * qb;
        block_ranges32(a0, min(a0 + 32, w1), Nq, Nk, wl, wr, &jf0[qb], &jf1[qb], &ju0[qb], &ju1[qb]);
    }
    auto block_skip = [&](int j, int qb) { return (unsigned)(j - ju0[qb]) >= (unsigned)(ju1[qb] - ju0[qb]); };
    auto block_full = [&](int j, int qb) { return (unsigned)(j - jf0[qb]) < (unsigned)(jf1[qb] - jf0[qb]); };

    // S^T of block (j, qb): element r of lane (l32, hh) is key
    // 32j + 8(r/4) + 4hh + r%4 against query w0 + 32qb + l32.
    // Per-lane parts of the LDS addresses; the rest (slot, sub-tile half, MFMA
    // step) is uniform. The swizzle term depends on the row mod 8 only, which
    // the uniform row offsets (multiples of 16) leave unchanged.
    int kofs[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kofs[s] = lds_pos<RB>(l32, 2 * s + hh);
    int vofs[ND][2];   // rows 4hh + cl/4 and 8 rows further
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) vofs[db][h8] = lds_pos<RB>(4 * hh + (cl >> 2) + 8 * h8, ch) + 8 * (cl & 1);
    }
    auto k_read = [&](const lds_u8* tb, int j, i32x4(&a)[NKS]) __attribute__((always_inline)) {
        const lds_u8* kb = tb + 32 * (j & 1) * RB;
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            a[s] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(kb + kofs[s]);
    };
    auto s_mfma = [&](const i32x4(&a)[NKS], int qb, f32x16& S) __attribute__((always_inline)) {
        S = f32x16{};
#pragma unroll
        for (int s = 0; s < NKS; ++s) S = mfma16(IN, a[s], qf[qb][s], S);
    };
    auto scores = [&](const lds_u8* tb, int j, int qb, f32x16& S) __attribute__((always_inline)) {
        i32x4 a[NKS];
        k_read(tb, j, a);
        s_mfma(a, qb, S);
    };

    // V^T operands of sub-tile j for its two 16-key MFMA steps, in the key
    // order P has: step sp, lane half hh, k-slot e holds key
    // 32j + 16sp + 8(e/4) + 4hh + e%4 (two transposing reads of 4 rows).
    auto v_operands = [&](const lds_u8* tb, int j, i32x4(&va)[2][ND]) __attribute__((always_inline)) {
        const lds_u8* vb = tb + TILE + 32 * (j & 1) * RB;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const i32x2 u0 = read_tr16(vb + 16 * sp * RB + vofs[db][0]);
                const i32x2 u1 = read_tr16(vb + 16 * sp * RB + vofs[db][1]);
                va[sp][db] = i32x4{u0[0], u0[1], u1[0], u1[1]};
            }
        }
    };

    // Masked scores become -inf: row i = w0 + 32qb + l32 sees keys [klo, khi)
    // (none when i is past the wave's rows).
    auto mask = [&](int j, int qb, f32x16& S) __attribute__((always_inline)) {
        const int c0 = 32 * j;
        int ln = lane;
        asm volatile("" : "+v"(ln));   // recomputed here, not held across the loop
        const int i = w0 + 32 * qb + (ln & 31);
        const int ip = i + (Nk - Nq);
        int klo = ip - wl;
        int khi = ip + wr + 1;
        klo = klo > 0 ? klo : 0;
        khi = khi < Nk ? khi : Nk;
        if (i >= w1) khi = klo;   // past the last query row: nothing visible
        const int a = klo - c0 - 4 * (ln >> 5), b = khi - c0 - 4 * (ln >> 5);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            S[r] = (off < a || off >= b) ? -INFINITY : S[r];
        }
    };

    // p = 2^(c*s - ms) for the 16 scores, their sum (a fixed pairwise order)
    // and p rounded to the MFMA type.
    // The exponent argument of score s (element r of a lane's block) against
    // the reference ref: the score in base-2 units, modified, minus ref.
    //   none:    c * s - ref
    //   ALiBi:   c * s + slope * log2(e) * (key - i') - ref; key - i' is
    //            32j + 4hh - i' (in abase, with -ref) plus 8(r/4) + r%4
    //   softcap: cap * log2(e) * tanh(scale * s / cap) - ref, with
    //            tanh|x| = 1 - 2 / (e^(2|x|) + 1); a masked score stays -inf
    //            (sc_args takes a polynomial instead on small arguments)
    auto alibi_base = [&](int j, int qb, float ref) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int ipq = w0 + 32 * qb + (ln & 31) + (Nk - Nq);
        return fmaf(slope2, (float)(32 * j + 4 * (ln >> 5) - ipq), -ref);
    };
    auto earg = [&](float s, int r, float abase, float ref) __attribute__((always_inline)) {
        if constexpr (MOD == MOD_ALIBI) {
            return fmaf(s, c2, fmaf(slope2, (float)(8 * (r >> 2) + (r & 3)), abase));
        } else if constexpr (MOD == MOD_SOFTCAP) {
            const float u = __builtin_amdgcn_exp2f(fabsf(s) * sc_k1);
            const float t = fmaf(-2.f, __builtin_amdgcn_rcpf(u + 1.f), 1.f);
            const float a = fmaf(__builtin_copysignf(t, s), sc_k2, -ref);
            return (s == -INFINITY) ? -INFINITY : a;
        } else {
            return fmaf(s, c2, -ref);
        }
    };
    // Softcap: the 16 exponent arguments of a lane's block against ref, by the
    // polynomial when all 16 scores are in its range, else the closed form.
    // The choice depends on the lane's scores alone, so forming a block again
    // (exact redo, residual) repeats it bit for bit.
    auto sc_args = [&](const f32x16& S, float ref, float(&a)[16]) __attribute__((always_inline)) {
        if (softcap_poly_ok(scp, S)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = fmaf(softcap_tanh_poly(scp, S[r]), sc_k2, -ref);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = earg(S[r], r, 0.f, ref);
        }
    };
    auto p_phase_pr = [&](const f32x16& S, float ms, float& ts, i32x4(&hi)[2], float(&pr)[16], int j, int qb)
        __attribute__((always_inline)) {
        if constexpr (MOD == MOD_NONE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c2, -ms));
        } else if constexpr (MOD == MOD_SOFTCAP) {
            float a[16];
            sc_args(S, ms, a);
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(a[r]);
        } else {
            float ab = 0.f;
            if constexpr (MOD == MOD_ALIBI) ab = alibi_base(j, qb, ms);
#pragma unroll
            for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(earg(S[r], r, ab, ms));
        }
        float s8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) s8[r] = pr[2 * r] + pr[2 * r + 1];
        ts = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int o = 8 * sp;
            hi[sp] = i32x4{pack2<IN>(pr[o + 0], pr[o + 1]), pack2<IN>(pr[o + 2], pr[o + 3]),
                           pack2<IN>(pr[o + 4], pr[o + 5]), pack2<IN>(pr[o + 6], pr[o + 7])};
        }
    };
    // The rounding residual of the weights, lo = p - hi rounded to the MFMA
    // type (zero where on is false).
    auto residual = [&](const float(&pr)[16], const i32x4(&hi)[2], bool on, i32x4(&lo)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int o = 8 * sp;
            const i32x4 h = hi[sp];
            const i32x4 d = i32x4{pack2<IN>(pr[o + 0] - unpack_lo<IN>(h[0]), pr[o + 1] - unpack_hi<IN>(h[0])),
                                  pack2<IN>(pr[o + 2] - unpack_lo<IN>(h[1]), pr[o + 3] - unpack_hi<IN>(h[1])),
                                  pack2<IN>(pr[o + 4] - unpack_lo<IN>(h[2]), pr[o + 5] - unpack_hi<IN>(h[2])),
                                  pack2<IN>(pr[o + 6] - unpack_lo<IN>(h[3]), pr[o + 7] - unpack_hi<IN>(h[3]))};
            lo[sp] = i32x4{on ? d[0] : 0, on ? d[1] : 0, on ? d[2] : 0, on ? d[3] : 0};
        }
    };

    auto pv = [&](int qb, const i32x4(&va)[2][ND], const i32x4(&P)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[db][qb] = mfma16(IN, va[sp][db], P[sp], oacc[db][qb]);
    };

    // ---- LDS bases of the slots of tiles t-1, t and t+1 while the loop is at
    // tile t (rotated when t advances)
    const lds_u8* lds_prev = tile_lds(t_lo + 2);
    const lds_u8* lds_cur = tile_lds(t_lo);
    const lds_u8* lds_next = tile_lds(t_lo + 1);
    // With K and V read ahead (RA == 2) the steps read K only from the slot
    // of tile t+1 and V only from the slot of tile t: their per-lane
    // addresses are kept whole and advanced once per tile, so that a read is
    // one register plus an immediate offset.
    const lds_u8* kan[NKS];
    const lds_u8* van[ND][2];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kan[s] = lds_next + kofs[s];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) van[db][h8] = lds_cur + TILE + vofs[db][h8];
    auto k_read_next = [&](int j, i32x4(&a)[NKS]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            a[s] = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(kan[s] + 32 * (j & 1) * RB);
    };
    auto v_operands_cur = [&](int j, i32x4(&va)[2][ND]) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const i32x2 u0 = read_tr16(van[db][0] + (32 * (j & 1) + 16 * sp) * RB);
                const i32x2 u1 = read_tr16(van[db][1] + (32 * (j & 1) + 16 * sp) * RB);
                va[sp][db] = i32x4{u0[0], u0[1], u1[0], u1[1]};
            }
        }
    };

    // ---- per-step state; the buffers alternate between even and odd steps
    f32x16 sbuf[2];        // scores of the current step and of the next
    i32x4 pbuf[2][2];      // rounded weights of the current step and of the previous
    i32x4 va[2][ND];       // V operands of the sub-tile of step u-1
    // With two query blocks per wave, K operands are read a step ahead: at
    // the start of sub-tile j's first step kpf holds K of sub-tile j.
    constexpr bool PF = QB == 2;
    i32x4 kpf[NKS];
    // With one query block per wave, operands are read a step ahead of their
    // MFMAs: RA >= 1 reads V of sub-tile j in step j (vb[j % 2]) for the
    // P.V of step j+1; RA == 2 also keeps kpf = K of sub-tile j+1 at the
    // start of step j, read in step j-1.
    constexpr int RA = (QB == 1) ? ((D == 64) ? FA_RA_D64 : FA_RA_D128) : 0;
    i32x4 vb[2][2][ND];

    // After the first p_phase of block (j, qb): masking of edge blocks, the
    // exact redo for flagged rows, the residual pass and the row sums (a
    // skipped block changes nothing: its weights and ts are zero). The common
    // path keeps no scores: the rare path forms the block's scores again from
    // K in LDS (sub-tile j lies in the loop's current tile), the same bits.
    // In the first sub-tiles of a row (EARLY) the residual pass is taken by
    // every lane from the weights pr kept by the step; later it is taken by
    // the rows whose new weight exceeds a quarter of their sum so far.
    // "No reference yet" and the share of the row's sum above which a block
    // takes the residual pass. Normally a lane half with no weight has no
    // reference, and the share is of the lane half's sum so far. With an
    // ALiBi reference preset from the largest-bias block (alibi_ref below),
    // the blocks before it may have weights that round to 0 against it:
    // "no reference" is then m = -inf, and since the row's final sum is at
    // least 1 against that reference, shares are of max(sum so far, 1).
    auto no_ref = [&](int qb) __attribute__((always_inline)) {
        return alibi_ref ? (m[qb] == -INFINITY) : (lh[qb] == 0.f);
    };
    auto res_floor = [&](int qb) __attribute__((always_inline)) {
        return alibi_ref ? fmaxf(lh[qb], 1.f) : lh[qb];
    };
    auto tail = [&](auto early, int j, int qb, bool skip, float& ms, float& ts, i32x4(&hi)[2], float(&pr)[16])
        __attribute__((always_inline)) {
        constexpr bool EARLY = decltype(early)::value;
        const bool edge = !skip & !block_full(j, qb);
        const bool first = no_ref(qb) | !(ts <= SUM_LIMIT);
        const bool flag = !skip & (EARLY ? first : (first | (ts * 3.f > res_floor(qb))));
        if (edge || __builtin_amdgcn_ballot_w64(flag) != 0) {
            f32x16 S;
            scores(lds_cur, j, qb, S);
            bool trig = !skip & first;
            if (edge) {
                // the weights so far saw every key of the sub-tile: mask, form
                // them again, and decide on the visible keys alone
                mask(j, qb, S);
                p_phase_pr(S, ms, ts, hi, pr, j, qb);
                trig = no_ref(qb) | !(ts <= SUM_LIMIT);
            }
            if (__builtin_amdgcn_ballot_w64(trig) != 0) {
                const unsigned tr = trig ? 1u : 0u;
                auto pw = __builtin_amdgcn_permlane32_swap(tr, tr, false, false);
                const bool row = (pw[0] | pw[1]) != 0;
                float mx;
                if constexpr (MOD == MOD_NONE) {
                    mx = S[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
                    mx = max_halves(mx);
                } else if constexpr (MOD == MOD_SOFTCAP) {
                    float a[16];
                    sc_args(S, 0.f, a);
                    mx = a[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, a[r]);
                    mx = max_halves(mx);
                } else {
                    float ab = 0.f;
                    if constexpr (MOD == MOD_ALIBI) ab = alibi_base(j, qb, 0.f);
                    mx = earg(S[0], 0, ab, 0.f);
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, earg(S[r], r, ab, 0.f));
                    mx = max_halves(mx);
                }
                // the row max in base-2 units (the modified scores are already)
                const float mnew = row ? fmaxf(m[qb], (MOD == MOD_NONE) ? mx * c2 : mx) : m[qb];
                const bool mv = mnew != m[qb];
                const float alpha = mv ? __builtin_amdgcn_exp2f(m[qb] - mnew) : 1.f;
                m[qb] = mnew;
                if (__builtin_amdgcn_ballot_w64(mv) != 0) {
                    lh[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha;
                }
                ms = (mnew == -INFINITY) ? 0.f : mnew;
                p_phase_pr(S, ms, ts, hi, pr, j, qb);
            }
            if constexpr (!EARLY) {
                const bool sr = !skip & (ts * 3.f > res_floor(qb));
                if (__builtin_amdgcn_ballot_w64(sr) != 0) {
                    float pe[16];
                    if constexpr (MOD == MOD_NONE) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c2, -ms));
                    } else if constexpr (MOD == MOD_SOFTCAP) {
                        float a[16];
                        sc_args(S, ms, a);
#pragma unroll
                        for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(a[r]);
                    } else {
                        float ab = 0.f;
                        if constexpr (MOD == MOD_ALIBI) ab = alibi_base(j, qb, ms);
#pragma unroll
                        for (int r = 0; r < 16; ++r) pe[r] = __builtin_amdgcn_exp2f(earg(S[r], r, ab, ms));
                    }
                    i32x4 lo[2];
                    residual(pe, hi, sr, lo);
                    if constexpr (RA >= 1) {
                        if (j & 1) pv(qb, vb[1], lo); else pv(qb, vb[0], lo);   // V of sub-tile j, read this step
                    } else {
                        i32x4 vt[2][ND];
                        v_operands(lds_cur, j, vt);
                        pv(qb, vt, lo);
                    }
                }
            }
        }
        if constexpr (EARLY) {
            if (!skip) {
                i32x4 lo[2];
                residual(pr, hi, true, lo);
                if (j & 1) pv(qb, vb[1], lo); else pv(qb, vb[0], lo);   // V of sub-tile j, read this step
            }
        }
        lh[qb] += ts;   // zero for a skipped block
    };

    // ---- one step (see the file comment); KP = u % 2 picks the buffers.
    // Branch-free apart from the rare exact path: the look-ahead scores and
    // the softmax are formed on every step, and a skipped step's weights are
    // zeroed, so the next step's P.V adds exactly nothing for it.
    auto step = [&](auto kp, int u, auto early) __attribute__((always_inline)) {
        constexpr int KP = decltype(kp)::value;
        constexpr bool EARLY = decltype(early)::value;   // only with RA == 2
        const int j = u / QB;
        constexpr int qb = KP % QB;                 // steps alternate query blocks when QB = 2
        constexpr int qn = (KP + 1) % QB;           // query block of step u+1
        constexpr int qpv = (KP + QB - 1) % QB;     // query block of step u-1
        constexpr bool load_v = qpv == 0;           // step u-1 is the first of its sub-tile
        const int jn = (qn == 0) ? j + 1 : j;       // sub-tile of step u+1
        // sub-tile of step u-1; before the first sub-tile, any loaded one will
        // do (its weights are zero)
        const int jp = max((qb == 0) ? j - 1 : j, 2 * t_lo);
        f32x16& S = sbuf[KP];
        f32x16& Sn = sbuf[KP ^ 1];
        i32x4(&Pc)[2] = pbuf[KP];
        i32x4(&Pp)[2] = pbuf[KP ^ 1];
        const bool skip = block_skip(j, qb);
        // a skipped block's weights are 2^-inf = 0: the next step's P.V of
        // them adds exactly nothing and the sums are unchanged. Before a row's
        // first reference (m = -inf) the weights come out +inf or NaN; such
        // a row has no weight yet and always takes the exact redo.
        float ms = skip ? INFINITY : m[qb];
        float ts;
        const int t = j >> 1;   // the loop's current tile
        if constexpr (RA == 2) {
            v_operands_cur(j, vb[KP]);        // for the next step's P.V (and an early residual)
        } else if constexpr (RA == 1) {
            v_operands(lds_cur, j, vb[KP]);   // for the next step's P.V
        } else if (load_v) {
            v_operands(((jp >> 1) == t) ? lds_cur : lds_prev, jp, va);
        }
        if constexpr (PF) {
            // qb 0: scores of (j, 1) from K(j), then K(j+1) is requested;
            // qb 1: scores of (j+1, 0) from K(j+1), read a step ago
            s_mfma(kpf, qn, Sn);
            if (KP == 0) k_read(((j + 1) >> 1 == t) ? lds_cur : lds_next, j + 1, kpf);
        } else if constexpr (RA == 2 && EARLY) {
            // no read-ahead: the registers hold the weights for the residual
            scores((KP == 0) ? lds_cur : lds_next, j + 1, 0, Sn);
        } else if constexpr (RA == 2) {
            s_mfma(kpf, 0, Sn);              // K of sub-tile j+1, read a step ago
            k_read_next(j + 2, kpf);         // K of sub-tile j+2 lies in tile t+1
        } else {
            scores(((jn >> 1) == t) ? lds_cur : lds_next, jn, qn, Sn);
        }
        float pr[16];
        p_phase_pr(S, ms, ts, Pc, pr, j, qb);
        if constexpr (RA >= 1) pv(qpv, vb[KP ^ 1], Pp);
        else pv(qpv, va, Pp);
        if constexpr (RA == 2) {
            // operands are in registers already: each MFMA is followed by
            // two exponentials (a wave overlaps transcendental work with its
            // own MFMA; MFMA and VALU work of different waves on one SIMD do
            // not overlap) and a share of the other VALU work
#pragma unroll
            for (int g = 0; g < NKS + 2 * ND; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);   // transcendental
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
            }
        }
        tail(early, j, qb, skip, ms, ts, Pc, pr);
    };

    // ---- ALiBi: under a bias that grows with the key index the row max climbs
    // by slope * 32 per sub-tile, so a reference taken from the first block
    // would be passed, and the exact redo taken, on nearly every block. The
    // reference starts instead at the row max of the modified scores of the
    // query block's last visible sub-tile, where the bias is largest (K read
    // straight from HBM; the same scores, bit for bit, as the loop forms for
    // that sub-tile). Rows that see no key of it keep m = -inf.
    if constexpr (MOD == MOD_ALIBI) {
        if (alibi_ref) {
            const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)(Nk * RB));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                if (ju1[qb] <= ju0[qb] || ju1[qb] - 1 < 2 * t_lo || ju1[qb] - 1 >= 2 * t_hi) continue;
                const int jl = ju1[qb] - 1;
                i32x4 a[NKS];
#pragma unroll
                for (int s = 0; s < NKS; ++s)
                    a[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (32 * jl + l32) * RB + (16 * s + 8 * hh) * 2, 0, 0));
                f32x16 S;
                s_mfma(a, qb, S);
                mask(jl, qb, S);
                const float ab = alibi_base(jl, qb, 0.f);
                float mx = earg(S[0], 0, ab, 0.f);
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, earg(S[r], r, ab, 0.f));
                m[qb] = max_halves(mx);
            }
        }
    }

    // ---- prologue: Q and tile t_lo land, tile t_lo+1 is requested (with
    // RA == 2 it lands too and tile t_lo+2 is requested), the first block's
    // scores are formed; no weights are pending yet
    if (t_lo < t_hi) issue_tile(t_lo);
    if (RA == 2 && t_lo + 1 < t_hi) issue_tile(t_lo + 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (RA != 2 && t_lo + 1 < t_hi) issue_tile(t_lo + 1);
    if (RA == 2 && t_lo + 2 < t_hi) issue_tile(t_lo + 2);
    if (t_lo < t_hi) {
        if constexpr (PF) {
            k_read(lds_cur, 2 * t_lo, kpf);
            s_mfma(kpf, 0, sbuf[0]);
        } else if constexpr (RA == 2) {
            scores(lds_cur, 2 * t_lo, 0, sbuf[0]);   // the early steps read K just in time
        } else {
            scores(lds_cur, 2 * t_lo, 0, sbuf[0]);
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            pbuf[b][sp] = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                va[sp][db] = i32x4{0, 0, 0, 0};
                vb[b][sp][db] = i32x4{0, 0, 0, 0};
            }
        }

    // ---- main loop: iteration i runs steps 2i and 2i+1 (sub-tile i's two
    // query blocks when QB = 2, tile i's two sub-tiles when QB = 1). A
    // barrier publishes tile t+1 before its first read -- the K read-ahead
    // of sub-tile 2t+1's first step when QB = 2, the score look-ahead of tile
    // t's last step when QB = 1 -- and follows every use of tile t-1, whose
    // slot then receives tile t+2.
    const int i_lo = SPT * t_lo / 2, i_hi = SPT * t_hi / 2;
    auto tile_barrier = [&](int t) __attribute__((always_inline)) {
        if (t + 1 < t_hi) __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's copies of tile t+1 landed
        __syncthreads();
        if (t + 2 < t_hi) issue_tile(t + 2);
    };
    auto rotate = [&]() __attribute__((always_inline)) {
        if constexpr (RA == 2) {
            const int dk = (int)(lds_prev - lds_next), dv = (int)(lds_next - lds_cur);
#pragma unroll
            for (int s = 0; s < NKS; ++s) kan[s] += dk;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int h8 = 0; h8 < 2; ++h8) van[db][h8] += dv;
        }
        const lds_u8* x = lds_prev;
        lds_prev = lds_cur;
        lds_cur = lds_next;
        lds_next = x;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using NotEarly = std::false_type;
    if constexpr (RA == 2) {
        // the K read-ahead of tile t's first step already reads tile t+1, and
        // tile t-1 was last read in the step before: one barrier before the
        // tile does both (tile t_lo+1 landed in the prologue). The first
        // EARLY_TILES tiles take the early steps.
        const int t_e = min(t_hi, t_lo + EARLY_TILES);
        int t = t_lo;
        for (; t < t_e; ++t) {
            if (t > t_lo) tile_barrier(t);
            step(I0{}, 2 * t, std::true_type{});
            step(I1{}, 2 * t + 1, std::true_type{});
            rotate();
        }
        if (t < t_hi) k_read(lds_cur, 2 * t + 1, kpf);   // the read-ahead of the first later step
        for (; t < t_hi; ++t) {
            if (t > t_lo) tile_barrier(t);
            step(I0{}, 2 * t, NotEarly{});
            step(I1{}, 2 * t + 1, NotEarly{});
            rotate();
        }
    } else {
        for (int i = i_lo; i < i_hi; ++i) {
            if constexpr (PF) {
                if (i & 1) tile_barrier(i >> 1);
                step(I0{}, 2 * i, NotEarly{});
                step(I1{}, 2 * i + 1, NotEarly{});
                if (i & 1) rotate();
            } else {
                step(I0{}, 2 * i, NotEarly{});
                tile_barrier(i);
                step(I1{}, 2 * i + 1, NotEarly{});
                rotate();
            }
        }
    }
    // ---- the last step's P.V (zero weights if that step was skipped)
    if (t_lo < t_hi) {
        if constexpr (RA >= 1) {
            pv(0, vb[1], pbuf[1]);   // V of the last sub-tile, read in its step
        } else {
            v_operands(tile_lds(t_hi - 1), 2 * t_hi - 1, va);
            pv(QB - 1, va, pbuf[1]);
        }
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l); a split writes both
    // in fp32 to its slice of the workspace instead
    if (p.n_split > 1) {
        const size_t sl = (size_t)bh * p.n_split + split;
        float* wo = p.ws_o + sl * Nq * D;
        float* wlp = p.ws_lse + sl * Nq;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = sum_halves(lh[qb]);
            const int i = w0 + 32 * qb + l32;
            if (i < w1) {
                const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
                uint8_t* orow = (uint8_t*)(wo + (size_t)i * D);
#pragma unroll
                for (int db = 0; db < ND; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const f32x16& a = oacc[db][qb];
                        const int d = 32 * db + 8 * r4 + 4 * hh;
                        Out<OUT_F32>::store4(orow + d * 4, a[4 * r4] * inv, a[4 * r4 + 1] * inv, a[4 * r4 + 2] * inv,
                                             a[4 * r4 + 3] * inv);
                    }
                if (hh == 0) wlp[i] = (lt > 0.f) ? (m[qb] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
            }
        }
        clock_stamp(p.clk, p.clk_n, 1);
        return;
    }
    uint8_t* op = p.o + (size_t)bh * Nq * D * Out<OUT>::EB;
    float* lp = p.lse + (size_t)bh * Nq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum_halves(lh[qb]);
        const int i = w0 + 32 * qb + l32;
        if (i < w1) {
            const float inv = (lt > 0.f) ? p.out_mul / lt : 0.f;
            uint8_t* orow = op + (size_t)i * D * Out<OUT>::EB;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x16& a = oacc[db][qb];
                    const int d = 32 * db + 8 * r4 + 4 * hh;
                    Out<OUT>::store4(orow + d * Out<OUT>::EB, a[4 * r4] * inv, a[4 * r4 + 1] * inv,
                                     a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv);
                }
            if (hh == 0) lp[i] = (lt > 0.f) ? (m[qb] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
        }
    }
    clock_stamp(p.clk, p.clk_n, 1);
}

// ---------------------------------------------------------------- host side

template <int IN, int OUT, int D, int NW, int QB, int MOD>
static int launch16_one(const Plan& pl, const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((fa_fwd16_kernel<IN, OUT, D, NW, QB, MOD>), dim3((unsigned)(pl.n_wg * p.n_split)), dim3(64 * NW),
                       0, s, p);
    return (int)hipGetLastError();
}

template <int IN, int OUT, int D, int NW, int QB>
static int launch16_mod(const Plan& pl, const Params& p, hipStream_t s) {
    if (p.mod == MOD_SOFTCAP) return launch16_one<IN, OUT, D, NW, QB, MOD_SOFTCAP>(pl, p, s);
    if (p.mod == MOD_ALIBI) return launch16_one<IN, OUT, D, NW, QB, MOD_ALIBI>(pl, p, s);
    return launch16_one<IN, OUT, D, NW, QB, MOD_NONE>(pl, p, s);
}

template <int IN, int OUT>
static int launch16_io(const Plan& pl, const Params& p, hipStream_t s) {
    if (pl.D == 64) {
        if (pl.qb == 2) return launch16_mod<IN, OUT, 64, 4, 2>(pl, p, s);
        return launch16_mod<IN, OUT, 64, 4, 1>(pl, p, s);
    }
    return launch16_mod<IN, OUT, 128, 8, 1>(pl, p, s);
}

// Merge of the splits of each row (the online-softmax identity of the
// FLASHLIGHT summary, Methodology item 3, across splits): with each split's
// O_s (normalised by its own sum) and LSE_s,
//   LSE = ln sum_s e^(LSE_s),   O = sum_s e^(LSE_s - LSE) O_s.
// One thread per 4 consecutive columns of a row; rows whose splits all saw no
// key get O = 0 and LSE = -inf.
template <int OUT>
__global__ __launch_bounds__(256) void fa_combine_kernel(Params p, int D) {
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const int q4 = D / 4;
    const long long rows = (long long)p.n_bh * p.Nq;
    if (t >= rows * q4) return;
    const long long row = t / q4;
    const int d = (int)(t % q4) * 4;
    const long long bh = row / p.Nq, i = row % p.Nq;
    const int S = p.n_split;
    const float* wl = p.ws_lse + (size_t)bh * S * p.Nq + i;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, wl[(size_t)s * p.Nq]);
    uint8_t* orow = p.o + (size_t)row * D * Out<OUT>::EB;
    if (mx == -INFINITY) {
        Out<OUT>::store4(orow + d * Out<OUT>::EB, 0.f, 0.f, 0.f, 0.f);
        if (d == 0) p.lse[row] = -INFINITY;
        return;
    }
    float wsum = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    const float* wo = p.ws_o + ((size_t)bh * S * p.Nq + i) * D + d;
    for (int s = 0; s < S; ++s) {
        const float w = expf(wl[(size_t)s * p.Nq] - mx);
        const float4 v = *reinterpret_cast<const float4*>(wo + (size_t)s * p.Nq * D);
        wsum += w;
        o0 = fmaf(w, v.x, o0);
        o1 = fmaf(w, v.y, o1);
        o2 = fmaf(w, v.z, o2);
        o3 = fmaf(w, v.w, o3);
    }
    const float inv = 1.f / wsum;
    Out<OUT>::store4(orow + d * Out<OUT>::EB, o0 * inv, o1 * inv, o2 * inv, o3 * inv);
    if (d == 0) p.lse[row] = mx + logf(wsum);
}

int launch_combine(const Plan& pl, const Params& p, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const long long n = (long long)p.n_bh * p.Nq * (pl.D / 4);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (blocks == 0) return 0;
    if (pl.out == OUT_F16) hipLaunchKernelGGL((fa_combine_kernel<OUT_F16>), dim3(blocks), dim3(256), 0, s, p, pl.D);
    else if (pl.out == OUT_BF16) hipLaunchKernelGGL((fa_combine_kernel<OUT_BF16>), dim3(blocks), dim3(256), 0, s, p, pl.D);
    else hipLaunchKernelGGL((fa_combine_kernel<OUT_F32>), dim3(blocks), dim3(256), 0, s, p, pl.D);
    return (int)hipGetLastError();
}

int launch16(const Plan& pl, const Params& p, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (pl.in == IN_F16 && pl.out == OUT_F16) return launch16_io<IN_F16, OUT_F16>(pl, p, s);
    if (pl.in == IN_F16 && pl.out == OUT_F32) return launch16_io<IN_F16, OUT_F32>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_BF16) return launch16_io<IN_BF16, OUT_BF16>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_F32) return launch16_io<IN_BF16, OUT_F32>(pl, p, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
