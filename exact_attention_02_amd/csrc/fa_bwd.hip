// Attention backward for 16-bit inputs on gfx950: dQ, dK and dV of
// O = softmax(scale Q K^T) V, given the upstream gradient dO, the forward's O
// and its log-sum-exp.
//
// The softmax weights are not stored by the forward; they are formed again
// here from Q, K and the stored normaliser, tile by tile (aiinarabic.com
// flash-attention page, the recomputation paragraph: the backward pass
// recomputes the attention matrix instead of reading it from memory). With
// P = exp(scale S - LSE):
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - Dvec),
//   dQ = scale dS K,   dK = scale dS^T Q,
// where Dvec_i = dO_i . O_i is the row sum of P o dP. With a score modifier f
// (softcap s <- cap tanh(s / cap), ALiBi s <- s + slope (j - i'); the
// FLASHLIGHT summary's score_mod variants) P is the softmax of the modified
// scores and dS picks up f'(s) by the chain rule: 1 - tanh^2 for softcap.
//
// Three kernels:
//   * fa_bwd_rowstat_kernel: -Dvec and the LSE in base-2 units per row;
//   * fa_bwd_dq_kernel: one workgroup per 128 query rows walks their keys.
//     Scores are kept transposed as in the forward (lane = query): S^T = K Q^T
//     and dP^T = V dO^T on MFMA, dS^T formed in registers, dQ^T += K^T dS^T
//     with K^T read by transposing LDS reads;
//   * fa_bwd_dkdv_kernel: one workgroup per 128 keys walks the query rows
//     that see them, in the mirrored layout (lane = key): S = Q K^T and
//     dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
//     read by transposing LDS reads.
// Both stream 64-row tiles through two LDS slots with direct-to-LDS copies,
// in the layout of the forward kernels (swizzled 16-byte chunks), one barrier
// per tile. P and dS are rounded to the input type for the MFMAs.
//
// On this chip the MFMAs and the vector ALU work of the waves on one SIMD do
// not overlap, so the loops are shaped to issue few vector instructions per
// MFMA: the dP accumulator starts at -Dvec (dP - Dvec comes out of the MFMA),
// masks are applied only on edge blocks, and the tile loop is unrolled over
// the two LDS slots so that every LDS address is a loop-invariant register
// plus an immediate. Each sub-tile runs its scores, softmax and products in
// turn; holding two sub-tiles' scores to overlap one's softmax with the
// other's MFMAs costs a wave per SIMD (3 -> 2 at D = 64) and measured slower.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

// dQ kernel: 1 starts each dP^T accumulator at -Dvec from 16 loop-invariant
// registers (no subtraction per score); 0 subtracts per score.
#ifndef FA_BWD_DQ_DINIT
#define FA_BWD_DQ_DINIT 1
#endif


namespace fa {

// ---------------------------------------------------------------- row statistics

// TPR threads per row, each reading 16 bytes of O and of dO per step; the
// padding rows of a head (Nq <= i < nqp) get -Dvec = 0 and l2 = +inf.
template <int IN, int D>
__global__ __launch_bounds__(256) void fa_bwd_rowstat_kernel(BwdParams p) {
    constexpr int TPR = D / 8;
    constexpr int RPB = 256 / TPR;
    const int sub = threadIdx.x % TPR;
    const long long idx = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const bool live = idx < (long long)p.n_bh * p.nqp;
    const int bh = live ? (int)(idx / p.nqp) : 0, i = live ? (int)(idx % p.nqp) : p.Nq;
    float acc = 0.f;
    if (i < p.Nq) {
        const size_t row = (size_t)bh * p.Nq + i;
        const i32x4 a = *reinterpret_cast<const i32x4*>(p.o + row * D * 2 + 16 * sub);
        const i32x4 b = *reinterpret_cast<const i32x4*>(p.dout + row * D * 2 + 16 * sub);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(unpack_lo<IN>(a[e]), unpack_lo<IN>(b[e]), acc);
            acc = fmaf(unpack_hi<IN>(a[e]), unpack_hi<IN>(b[e]), acc);
        }
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (!live || sub != 0) return;
    float l2 = INFINITY;
    if (i < p.Nq) {
        const float l = p.lse[(size_t)bh * p.Nq + i];
        // a row that sees no key: every weight of its row must come out 0
        if (l != -INFINITY) l2 = l * LOG2E;
    }
    p.ndvec[idx] = -acc;
    p.l2[idx] = l2;
}

// Shared pieces of the two tiled kernels: tile shape, the LDS row and
// transposing reads of a 64-row tile (the forward's layout), the copies.
template <int D>
struct TileShape {
    static constexpr int NW = 4;
    static constexpr int NT = 64 * NW;
    static constexpr int RB = D * 2;
    static constexpr int CPR = RB / 16;
    static constexpr int TILE = BC * RB;     // one tensor's 64-row tile
    static constexpr int SLOT = 2 * TILE;    // two tensors
    static constexpr int NKS = D / 16;
    static constexpr int ND = D / 32;
    static constexpr int NDMA = TILE / 16 / NT;
};

using Slot0 = std::integral_constant<int, 0>;
using Slot1 = std::integral_constant<int, 1>;

__device__ __forceinline__ i32x4 lds_read16(const lds_u8* a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(a);
}
__device__ __forceinline__ f32x4v lds_readf4(const lds_u8* a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4v*>(a);
}

// The weight 2^(f(s) - LSE) of a score s (base-2 units: the scaled score is
// c s) and the chain factor g = f'. e is the exponent's additive part: -LSE
// in base-2 units, plus the ALiBi bias. Softcap: u = e^(2|x|) with
// x = scale s / cap (k1 = 2 c / cap), tanh|x| = 1 - 2 r with r = 1 / (u + 1),
// f = cap log2(e) tanh(x) (k2 = cap log2(e)), and 1 - tanh^2 = 4 r (1 - r),
// which has no cancellation and is 0 where u overflows. A masked score
// (-inf) has weight 0 under every modifier.
// Softcap on small arguments (all 16 scores of the lane's block within the
// range of softcap_tanh_poly): the weight and f' from the polynomial's tanh.
__device__ __forceinline__ float softcap_weight_poly(const SoftcapPoly& P, float s, float k2, float e, float& g) {
    const float t = softcap_tanh_poly(P, s);
    g = fmaf(-t, t, 1.f);
    return __builtin_amdgcn_exp2f(fmaf(t, k2, e));
}

template <int MOD>
__device__ __forceinline__ float mod_weight(float s, float c2, float k1, float k2, float e, float& g) {
    if constexpr (MOD == MOD_SOFTCAP) {
        const float u = __builtin_amdgcn_exp2f(fabsf(s) * k1);
        const float r = __builtin_amdgcn_rcpf(u + 1.f);
        const float t = fmaf(-2.f, r, 1.f);
        g = 4.f * r * (1.f - r);
        const float a = fmaf(__builtin_copysignf(t, s), k2, e);
        return (s == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(a);
    } else {
        g = 1.f;
        return __builtin_amdgcn_exp2f(fmaf(s, c2, e));
    }
}

// ---------------------------------------------------------------- dQ

template <int IN, int D, int MOD>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(BwdParams p) {
    using T = TileShape<D>;
    constexpr int RB = T::RB, CPR = T::CPR, TILE = T::TILE, SLOT = T::SLOT, NKS = T::NKS, ND = T::ND;
    constexpr int NT = T::NT, NDMA = T::NDMA, BR = 32 * T::NW;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SLOT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int g = lane >> 4, cl = lane & 15;
    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;

    int bh, qt;
    decode_wg((long long)blockIdx.x, p.n_bh, p.n_qt, p.hg, p.tl, &bh, &qt);
    const int r0 = qt * BR, r1 = min(r0 + BR, Nq);
    int kv_lo, kv_hi;
    kv_range(r0, r1, Nq, Nk, wl, wr, &kv_lo, &kv_hi);
    const int t_lo = kv_lo / BC, t_hi = (kv_hi > kv_lo) ? (kv_hi + BC - 1) / BC : kv_lo / BC;
    const int w0 = r0 + wave * 32, w1 = min(w0 + 32, Nq);
    const int row = w0 + l32;

    // Q and dO rows of the lane's query: B operands of S^T = K Q^T and dP^T = V dO^T
    i32x4 qf[NKS], dof[NKS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + (size_t)bh * Nq * RB, (unsigned)(Nq * RB));
        const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.dout + (size_t)bh * Nq * RB, (unsigned)(Nq * RB));
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int off = row * RB + (16 * s + 8 * hh) * 2;
            qf[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
            dof[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0));
        }
    }
    const float l2 = (row < Nq) ? p.l2[(size_t)bh * p.nqp + row] : INFINITY;
    const float ndv = (row < Nq) ? p.ndvec[(size_t)bh * p.nqp + row] : 0.f;
    const float c2 = p.c;
    const float k1 = p.mk1, k2 = p.mk2;   // softcap constants
    const SoftcapPoly scp = p.scp;        // softcap on small arguments (fa_device.h)
    float slope2 = 0.f;                   // ALiBi: this head's slope * log2(e)
    if constexpr (MOD == MOD_ALIBI) slope2 = p.slopes[bh % p.H] * LOG2E;
#if FA_BWD_DQ_DINIT
    f32x16 dinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) dinit[r] = ndv;
#endif

    int jf0, jf1, ju0, ju1;
    block_ranges32(w0, w1, Nq, Nk, wl, wr, &jf0, &jf1, &ju0, &ju1);

    const i32x4 kwords = rsrc_words(p.k + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
    const i32x4 vwords = rsrc_words(p.v + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    static_assert((NT / CPR) % 16 == 0, "copy rows");
    const unsigned dma_voff = [&] {
        const int slot = 64 * wave + lane;
        const int x = slot / CPR, c = (slot % CPR) ^ swz16<RB>(x);
        return (unsigned)(x * RB + c * 16);
    }();
    // K and V tile t into LDS slot `slot`
    auto issue_tile = [&](int t, int slot) {
        const unsigned kb = smem_base + (unsigned)(slot * SLOT);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int run = 64 * wave + NT * i;
            const unsigned soff = (unsigned)((t * BC + i * (NT / CPR)) * RB);
            dma16(kwords, kb + run * 16, dma_voff, soff);
            dma16(vwords, kb + TILE + run * 16, dma_voff, soff);
        }
    };

    const lds_u8* lds = (const lds_u8*)smem;
    int kofs[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kofs[s] = lds_pos<RB>(l32, 2 * s + hh);
    int tofs[ND][2];   // transposing reads: rows 4hh + cl/4 and 8 rows further
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) tofs[db][h8] = lds_pos<RB>(4 * hh + (cl >> 2) + 8 * h8, ch) + 8 * (cl & 1);
    }

    f32x16 dq[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) dq[db] = f32x16{};

    auto tile = [&](int t, auto slot_c) {
        constexpr int SL = decltype(slot_c)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's copies of tile t (and the rows above) landed
        __syncthreads();                       // ... and every wave's; the other slot is free
        if (t + 1 < t_hi) issue_tile(t + 1, 1 - SL);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int j = 2 * t + sub;
            if ((unsigned)(j - ju0) >= (unsigned)(ju1 - ju0)) continue;   // no visible pair
            const bool full = (unsigned)(j - jf0) < (unsigned)(jf1 - jf0);
            constexpr int KB = SL * SLOT, VB = SL * SLOT + TILE;
            f32x16 S = f32x16{};
#if FA_BWD_DQ_DINIT
            f32x16 dP = dinit;   // dP^T - Dvec
#else
            f32x16 dP = f32x16{};
#endif
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                S = mfma16(IN, lds_read16(lds + kofs[s] + (KB + 32 * sub * RB)), qf[s], S);
                dP = mfma16(IN, lds_read16(lds + kofs[s] + (VB + 32 * sub * RB)), dof[s], dP);
            }
            if (!full) {
                // element r of the lane holds key 32j + 8(r/4) + 4hh + r%4 against query row
                const int ip = row + (Nk - Nq);
                int klo = ip - wl, khi = ip + wr + 1;
                klo = klo > 0 ? klo : 0;
                khi = khi < Nk ? khi : Nk;
                if (row >= w1) khi = klo;
                const int a = klo - 32 * j - 4 * hh, b = khi - 32 * j - 4 * hh;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    S[r] = (off < a || off >= b) ? -INFINITY : S[r];
                }
            }
            // ALiBi: key - i' = 32j + 4hh - i' (per lane) + 8(r/4) + r%4
            float ab = -l2;
            if constexpr (MOD == MOD_ALIBI) ab = fmaf(slope2, (float)(32 * j + 4 * hh - (row + Nk - Nq)), -l2);
            float ds[16];
            // POLY: softcap by the polynomial (all 16 of the lane's scores in range)
            auto weights = [&](auto poly_c) __attribute__((always_inline)) {
                constexpr bool POLY = decltype(poly_c)::value;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float e = ab, g;
                    if constexpr (MOD == MOD_ALIBI) e = fmaf(slope2, (float)(8 * (r >> 2) + (r & 3)), ab);
                    const float pr = POLY ? softcap_weight_poly(scp, S[r], k2, e, g) : mod_weight<MOD>(S[r], c2, k1, k2, e, g);
#if FA_BWD_DQ_DINIT
                    ds[r] = pr * dP[r];
#else
                    ds[r] = pr * (dP[r] + ndv);
#endif
                    if constexpr (MOD == MOD_SOFTCAP) ds[r] *= g;
                }
            };
            if constexpr (MOD == MOD_SOFTCAP) {
                if (softcap_poly_ok(scp, S)) weights(std::true_type{});
                else weights(std::false_type{});
            } else {
                weights(std::false_type{});
            }
            i32x4 dsb[2];
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const int o = 8 * sp;
                dsb[sp] = i32x4{pack2<IN>(ds[o + 0], ds[o + 1]), pack2<IN>(ds[o + 2], ds[o + 3]),
                                pack2<IN>(ds[o + 4], ds[o + 5]), pack2<IN>(ds[o + 6], ds[o + 7])};
            }
            // dQ^T += K^T dS^T: K^T of the sub-tile in the key order dS^T has
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    const int base = KB + (32 * sub + 16 * sp) * RB;
                    const i32x2 u0 = read_tr16(lds + tofs[db][0] + base);
                    const i32x2 u1 = read_tr16(lds + tofs[db][1] + base);
                    dq[db] = mfma16(IN, i32x4{u0[0], u0[1], u1[0], u1[1]}, dsb[sp], dq[db]);
                }
        }
    };

    if (t_lo < t_hi) issue_tile(t_lo, 0);
    for (int t = t_lo; t < t_hi; t += 2) {
        tile(t, Slot0{});
        if (t + 1 < t_hi) tile(t + 1, Slot1{});
    }

    // dQ = scale * dQ^T, row `row`, columns 32db + 8r4 + 4hh .. +3
    if (row < w1) {
        uint8_t* orow = p.dq + ((size_t)bh * Nq + row) * RB;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * hh;
                Out<(IN == IN_BF16) ? OUT_BF16 : OUT_F16>::store4(orow + d * 2, dq[db][4 * r4] * sc,
                                                                  dq[db][4 * r4 + 1] * sc, dq[db][4 * r4 + 2] * sc,
                                                                  dq[db][4 * r4 + 3] * sc);
            }
    }
}

// ---------------------------------------------------------------- dK, dV

// D = 128 holds 128 accumulator registers for dK^T and dV^T: one wave per SIMD.
template <int IN, int D, int MOD>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void fa_bwd_dkdv_kernel(BwdParams p) {
    using T = TileShape<D>;
    constexpr int RB = T::RB, CPR = T::CPR, TILE = T::TILE, SLOT = T::SLOT, NKS = T::NKS, ND = T::ND;
    constexpr int NT = T::NT, NDMA = T::NDMA, BK = 32 * T::NW;
    // a slot: the Q tile, the dO tile, then the tile rows' -Dvec and base-2 LSE
    // (1 KB each: one 64-lane copy, of which the first 256 bytes are the rows')
    constexpr int SLOTK = SLOT + 2048;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SLOTK];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int g = lane >> 4, cl = lane & 15;
    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;
    const int dlt = Nk - Nq;

    // key blocks in increasing order: under a causal mask the first ones see
    // the most query rows, so the heaviest work starts first
    int bh, kt;
    decode_wg((long long)blockIdx.x, p.n_bh, p.n_kt, p.hg, p.tl, &bh, &kt);
    kt = p.n_kt - 1 - kt;
    const int c0 = kt * BK, c1 = min(c0 + BK, Nk);
    // query rows that see a key of [c0, c1): key j is visible to row i when
    // j - wr <= i' <= j + wl, i' = i + Nk - Nq
    long long qlo = (long long)c0 - wr - dlt, qhi = (long long)(c1 - 1) + wl - dlt + 1;
    if (qlo < 0) qlo = 0;
    if (qhi > Nq) qhi = Nq;
    if (qhi < qlo) qhi = qlo;
    const int t_lo = (int)(qlo / BC), t_hi = (qhi > qlo) ? (int)((qhi + BC - 1) / BC) : t_lo;
    const int kw0 = c0 + wave * 32, kw1 = min(kw0 + 32, Nk);
    const int key = kw0 + l32;

    // K and V rows of the lane's key: B operands of S = Q K^T and dP = dO V^T
    i32x4 kf[NKS], vf[NKS];
    {
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int off = key * RB + (16 * s + 8 * hh) * 2;
            kf[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
            vf[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
        }
    }
    // The per-row statistics of a tile's 64 rows go to LDS with the tile: wave
    // 0 copies -Dvec, wave 1 the base-2 LSE, lanes 0-15 4 rows each. The head's
    // rows start 16-byte aligned (padded to nqp); lanes 16-63 and rows past
    // the head read 0 (their offsets lie beyond the descriptor's range: 2^30
    // plus at most 4 Nq < 2^25 bytes). Only masked pairs use a row past Nq.
    const i32x4 swords = (wave == 0) ? rsrc_words(p.ndvec + (size_t)bh * p.nqp, (unsigned)(p.nqp * 4))
                                     : rsrc_words(p.l2 + (size_t)bh * p.nqp, (unsigned)(p.nqp * 4));
    const unsigned stat_voff = (lane < 16) ? (unsigned)(16 * lane) : (1u << 30);
    const float c2 = p.c;
    const float k1 = p.mk1, k2 = p.mk2;   // softcap constants
    const SoftcapPoly scp = p.scp;        // softcap on small arguments (fa_device.h)
    float slope2 = 0.f;                   // ALiBi: this head's slope * log2(e)
    if constexpr (MOD == MOD_ALIBI) slope2 = p.slopes[bh % p.H] * LOG2E;
    // the lane's key sees the rows [klo_q, khi_q)
    int klo_q = key - wr - dlt, khi_q = key + wl - dlt + 1;
    klo_q = klo_q > 0 ? klo_q : 0;
    khi_q = khi_q < Nq ? khi_q : Nq;
    if (key >= kw1) khi_q = klo_q;

    const i32x4 qwords = rsrc_words(p.q + (size_t)bh * Nq * RB, (unsigned)(Nq * RB));
    const i32x4 dwords = rsrc_words(p.dout + (size_t)bh * Nq * RB, (unsigned)(Nq * RB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    static_assert((NT / CPR) % 16 == 0, "copy rows");
    const unsigned dma_voff = [&] {
        const int slot = 64 * wave + lane;
        const int x = slot / CPR, c = (slot % CPR) ^ swz16<RB>(x);
        return (unsigned)(x * RB + c * 16);
    }();
    // Q, dO and the statistics of tile t into LDS slot `slot`
    auto issue_tile = [&](int t, int slot) {
        const unsigned qb = smem_base + (unsigned)(slot * SLOTK);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int run = 64 * wave + NT * i;
            const unsigned soff = (unsigned)((t * BC + i * (NT / CPR)) * RB);
            dma16(qwords, qb + run * 16, dma_voff, soff);
            dma16(dwords, qb + TILE + run * 16, dma_voff, soff);
        }
        if (wave < 2) dma16(swords, qb + SLOT + 1024 * wave, stat_voff, (unsigned)(t * BC * 4));
    };

    const lds_u8* lds = (const lds_u8*)smem;
    int rofs[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) rofs[s] = lds_pos<RB>(l32, 2 * s + hh);
    int tofs[ND][2];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) tofs[db][h8] = lds_pos<RB>(4 * hh + (cl >> 2) + 8 * h8, ch) + 8 * (cl & 1);
    }
    const int sofs = 16 * hh;   // the lane half's 4 rows in each group of 8

    f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    // Pieces of one 32-row sub-tile `sub` of the tile in slot SL.
    // -Dvec of the sub-tile's rows, the starting value of its dP accumulator:
    // element r of the lane holds query q0 + 8(r/4) + 4hh + r%4 against the lane's key
    auto dp_init = [&](auto slot_c, int sub) __attribute__((always_inline)) {
        constexpr int SB = decltype(slot_c)::value * SLOTK + SLOT;
        f32x16 d;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const f32x4v nd = lds_readf4(lds + sofs + (SB + 4 * (32 * sub + 8 * gq)));
#pragma unroll
            for (int e = 0; e < 4; ++e) d[4 * gq + e] = nd[e];
        }
        return d;
    };
    // S = Q K^T and dP - Dvec = dO V^T - Dvec of the sub-tile
    auto scores = [&](auto slot_c, int sub, f32x16& S, f32x16& dP) __attribute__((always_inline)) {
        constexpr int QB = decltype(slot_c)::value * SLOTK, DB = QB + TILE;
        S = f32x16{};
        dP = dp_init(slot_c, sub);
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            S = mfma16(IN, lds_read16(lds + rofs[s] + (QB + 32 * sub * RB)), kf[s], S);
            dP = mfma16(IN, lds_read16(lds + rofs[s] + (DB + 32 * sub * RB)), vf[s], dP);
        }
    };
    auto mask = [&](int q0, f32x16& S) __attribute__((always_inline)) {
        const int a = klo_q - q0 - 4 * hh, b = khi_q - q0 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            S[r] = (off < a || off >= b) ? -INFINITY : S[r];
        }
    };
    // P = 2^(f(c S) - LSE) and dS = P (dP - Dvec) f', rounded to the MFMA type;
    // rows q0 .. q0 + 31 of the sub-tile
    auto softmax = [&](auto slot_c, int sub, int q0, const f32x16& S, const f32x16& dP, i32x4(&pb)[2],
                       i32x4(&db2)[2]) __attribute__((always_inline)) {
        constexpr int SB = decltype(slot_c)::value * SLOTK + SLOT;
        // ALiBi: key - i' = key - q0 - 4hh - (Nk - Nq) (per lane) - 8(r/4) - r%4
        float bb = 0.f;
        if constexpr (MOD == MOD_ALIBI) bb = slope2 * (float)(key - q0 - 4 * hh - dlt);
        float pr[16], ds[16];
        // POLY: softcap by the polynomial (all 16 of the lane's scores in range)
        auto weights = [&](auto poly_c) __attribute__((always_inline)) {
            constexpr bool POLY = decltype(poly_c)::value;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4v L = lds_readf4(lds + sofs + (SB + 1024 + 4 * (32 * sub + 8 * gq)));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * gq + e;
                    float ex = -L[e], g;
                    if constexpr (MOD == MOD_ALIBI) ex = fmaf(-slope2, (float)(8 * gq + e), bb) - L[e];
                    pr[r] = POLY ? softcap_weight_poly(scp, S[r], k2, ex, g) : mod_weight<MOD>(S[r], c2, k1, k2, ex, g);
                    ds[r] = pr[r] * dP[r];
                    if constexpr (MOD == MOD_SOFTCAP) ds[r] *= g;
                }
            }
        };
        if constexpr (MOD == MOD_SOFTCAP) {
            if (softcap_poly_ok(scp, S)) weights(std::true_type{});
            else weights(std::false_type{});
        } else {
            weights(std::false_type{});
        }
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int o = 8 * sp;
            pb[sp] = i32x4{pack2<IN>(pr[o + 0], pr[o + 1]), pack2<IN>(pr[o + 2], pr[o + 3]),
                           pack2<IN>(pr[o + 4], pr[o + 5]), pack2<IN>(pr[o + 6], pr[o + 7])};
            db2[sp] = i32x4{pack2<IN>(ds[o + 0], ds[o + 1]), pack2<IN>(ds[o + 2], ds[o + 3]),
                            pack2<IN>(ds[o + 4], ds[o + 5]), pack2<IN>(ds[o + 6], ds[o + 7])};
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS, dO^T and Q^T in the query order P has
    auto accumulate = [&](auto slot_c, int sub, const i32x4(&pb)[2], const i32x4(&db2)[2])
        __attribute__((always_inline)) {
        constexpr int QB = decltype(slot_c)::value * SLOTK, DB = QB + TILE;
#pragma unroll
        for (int d0 = 0; d0 < ND; ++d0)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const int rowoff = (32 * sub + 16 * sp) * RB;
                const i32x2 o0 = read_tr16(lds + tofs[d0][0] + (DB + rowoff));
                const i32x2 o1 = read_tr16(lds + tofs[d0][1] + (DB + rowoff));
                const i32x2 u0 = read_tr16(lds + tofs[d0][0] + (QB + rowoff));
                const i32x2 u1 = read_tr16(lds + tofs[d0][1] + (QB + rowoff));
                dv[d0] = mfma16(IN, i32x4{o0[0], o0[1], o1[0], o1[1]}, pb[sp], dv[d0]);
                dk[d0] = mfma16(IN, i32x4{u0[0], u0[1], u1[0], u1[1]}, db2[sp], dk[d0]);
            }
    };
    // Class of 32-row sub-tile n (rows 32n .. 32n+31) against the wave's keys,
    // from two ranges of n computed once: the mask read with keys as rows --
    // key j sees the rows i with i + Nk - Nq in [j - wr, j + wl] -- is the
    // forward's with (Nq, Nk) and (wl, wr) swapped. A full sub-tile lies
    // inside [0, Nq).
    int nf0, nf1, nu0, nu1;
    block_ranges32(kw0, kw1, Nk, Nq, wr, wl, &nf0, &nf1, &nu0, &nu1);
    auto sub_class = [&](int n) __attribute__((always_inline)) {
        if ((unsigned)(n - nu0) >= (unsigned)(nu1 - nu0)) return (int)TILE_SKIP;
        return ((unsigned)(n - nf0) < (unsigned)(nf1 - nf0)) ? (int)TILE_FULL : (int)TILE_EDGE;
    };

    auto tile = [&](int t, auto slot_c) {
        constexpr int SL = decltype(slot_c)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (t + 1 < t_hi) issue_tile(t + 1, 1 - SL);
        const int cls0 = sub_class(2 * t), cls1 = sub_class(2 * t + 1);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int cls = sub ? cls1 : cls0;
            if (cls == TILE_SKIP) continue;
            f32x16 S, dP;
            i32x4 pb[2], db2[2];
            scores(slot_c, sub, S, dP);
            if (cls != TILE_FULL) mask(BC * t + 32 * sub, S);
            softmax(slot_c, sub, BC * t + 32 * sub, S, dP, pb, db2);
            accumulate(slot_c, sub, pb, db2);
        }
    };

    if (t_lo < t_hi) issue_tile(t_lo, 0);
    for (int t = t_lo; t < t_hi; t += 2) {
        tile(t, Slot0{});
        if (t + 1 < t_hi) tile(t + 1, Slot1{});
    }

    // dK = scale * dK^T, dV = dV^T: key row `key`, columns 32db + 8r4 + 4hh .. +3
    if (key < kw1) {
        uint8_t* krow = p.dk + ((size_t)bh * Nk + key) * RB;
        uint8_t* vrow = p.dv + ((size_t)bh * Nk + key) * RB;
        const float sc = p.scale;
        constexpr int OT = (IN == IN_BF16) ? OUT_BF16 : OUT_F16;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * hh;
                Out<OT>::store4(krow + d * 2, dk[db][4 * r4] * sc, dk[db][4 * r4 + 1] * sc, dk[db][4 * r4 + 2] * sc,
                                dk[db][4 * r4 + 3] * sc);
                Out<OT>::store4(vrow + d * 2, dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2],
                                dv[db][4 * r4 + 3]);
            }
    }
}

// ---------------------------------------------------------------- host side

template <int IN, int D, int MOD>
static int launch_bwd_d(const BwdParams& p, hipStream_t s) {
    const long long rows = (long long)p.n_bh * p.nqp;
    constexpr int RPB = 256 / (D / 8);
    if (rows > 0)
        hipLaunchKernelGGL((fa_bwd_rowstat_kernel<IN, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s,
                           p);
    if (p.n_bh * (long long)p.n_qt > 0)
        hipLaunchKernelGGL((fa_bwd_dq_kernel<IN, D, MOD>), dim3((unsigned)(p.n_bh * (long long)p.n_qt)), dim3(256), 0, s,
                           p);
    if (p.n_bh * (long long)p.n_kt > 0)
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<IN, D, MOD>), dim3((unsigned)(p.n_bh * (long long)p.n_kt)), dim3(256), 0,
                           s, p);
    return (int)hipGetLastError();
}

template <int IN, int MOD>
static int launch_bwd_m(int D, const BwdParams& p, hipStream_t s) {
    return D == 64 ? launch_bwd_d<IN, 64, MOD>(p, s) : launch_bwd_d<IN, 128, MOD>(p, s);
}

template <int IN>
static int launch_bwd_i(int D, const BwdParams& p, hipStream_t s) {
    if (p.mod == MOD_SOFTCAP) return launch_bwd_m<IN, MOD_SOFTCAP>(D, p, s);
    if (p.mod == MOD_ALIBI) return launch_bwd_m<IN, MOD_ALIBI>(D, p, s);
    return launch_bwd_m<IN, MOD_NONE>(D, p, s);
}

int launch_bwd(int in, int D, const BwdParams& p, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (in == IN_BF16) return launch_bwd_i<IN_BF16>(D, p, s);
    if (in == IN_F16) return launch_bwd_i<IN_F16>(D, p, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
