// Fused exact-attention forward for gfx950 (MI355X, CDNA4).
//
// One workgroup = 4 waves = one logical tile of BR query rows of one
// (batch, head); each wave owns 32*QB consecutive query rows. The loop walks
// the workgroup's key range in tiles of BC = 64 keys, which is the per-block
// order the aiinarabic.com flash-attention page lists: load a block of K and V
// on chip, form the block's scores, apply softmax to them, multiply by V and
// merge with what came before, then move to the next block. Nothing of size
// Nq x Nk is ever written to HBM (same page, kernel fusion; inskillml module 9).
//
// gfx950 mapping:
//  * Q lives in VGPRs for the whole loop as the B operand of the score MFMA.
//  * K and V tiles are double-buffered in LDS: the global loads of tile t+1 are
//    in flight while tile t is multiplied, with one barrier per tile.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,
//    f16} (or v_mfma_f32_32x32x64_f8f6f4 for e4m3). In the 32x32 accumulator
//    layout lane l holds column l%32 -- one query -- and 16 of the 32 key rows,
//    so the row max and row sum are in-lane, plus one v_permlane32_swap to
//    meet the other lane half.
//  * Online softmax (FLASHLIGHT summary, Methodology item 3: running max and
//    running sum, rescaled with e^(x-y) = e^x / e^y when the max moves), in
//    base 2 with v_exp_f32. The rescale is lazy: the accumulator is only
//    rescaled when a tile's max exceeds the max in use by more than TAU (in
//    log2 units), which keeps every exponentiated score <= 2^TAU; the final
//    division by the row sum is unchanged by the choice of reference max.
//  * P goes straight from the score accumulator into the B operand of the
//    P.V MFMA (no LDS round trip). The key order inside the MFMA reduction is
//    free, so V's rows are read from LDS with ds_read_b64_tr_b16 / _tr_b8
//    (transposing reads) in the order P already has.
//  * O^T accumulates in registers (fp32); the epilogue divides by the row sum,
//    converts with round-to-nearest-even and writes O and the row LSE.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace fa {

constexpr int WAVES = 4;
constexpr int NTHREADS = 64 * WAVES;

// Rounding P to 16 bits costs up to 2^-9 (bf16) of each weight. Averaged over
// many comparable weights that is negligible (the output's own rounding
// dominates), but a row whose tile holds a weight above a quarter of the row's
// sum so far, this tile included -- its first tile, rows with few keys, peaked
// rows -- also multiplies V by P's rounding residual, P = hi + lo, so no
// dominant weight's rounding reaches the output. The decision is taken before
// the tile's exponentials: the tile adds at least pmax to the sum, so
// 3 * pmax > (sum before the tile) covers every case of 4 * pmax > (sum with
// the tile). Other rows get lo = 0, an exact no-op. pmax is the tile's
// largest exponentiated score, lhalf this lane half's share of the rescaled
// sum before the tile.
__device__ __forceinline__ bool split_row(float pmax, float lhalf) {
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(lhalf), __float_as_uint(lhalf), false, false);
    const float l = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    return pmax * 3.f > l;
}

template <int IN, int OUT, int D, int QB>
__global__ __launch_bounds__(NTHREADS) void fa_fwd_kernel(Params p) {
    typedef In<IN> I;
    constexpr int QK = I::QK;
    constexpr bool FP8 = (IN == IN_E4M3);
    constexpr int GRB = D * I::EB;             // bytes per row in HBM (q, k, v)
    constexpr int KRB = D * 2;                 // bytes per K row in LDS (16-bit)
    constexpr int VRB = D * I::EB;             // bytes per V row in LDS
    constexpr int KTILE = BC * KRB, VTILE = BC * VRB, STAGE = KTILE + VTILE;
    constexpr int GCPR = GRB / 16;             // 16-byte chunks per HBM row
    constexpr int GLD = BC * GCPR / NTHREADS;  // chunks per tensor each thread stages per tile
    constexpr int NKS = D / 16;                // steps of the score MFMA over D
    constexpr int ND = D / 32;                 // 32-wide blocks of the head dim
    constexpr int QW = 32 * QB;                // query rows per wave
    constexpr int BR = WAVES * QW;
    static_assert(GLD >= 1 && (BC * GCPR) % NTHREADS == 0, "tile staging");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;
    int bh, qt;
    decode_wg((long long)blockIdx.x, p.n_bh, p.n_qt, p.hg, p.tl, &bh, &qt);
    const int r0 = qt * BR;
    const int r1 = min(r0 + BR, Nq);
    int kv_lo, kv_hi;
    kv_range(r0, r1, Nq, Nk, wl, wr, &kv_lo, &kv_hi);
    const int t_lo = kv_lo / BC;
    const int t_hi = (kv_hi > kv_lo) ? (kv_hi + BC - 1) / BC : t_lo;
    clock_stamp(p.clk, p.clk_n, 0);

    const int w0 = r0 + wave * QW;
    const int w1 = min(w0 + QW, Nq);

    const uint8_t* qp = p.q + (size_t)bh * Nq * GRB;
    const uint8_t* kp = p.k + (size_t)bh * Nk * GRB;
    const uint8_t* vp = p.v + (size_t)bh * Nk * GRB;

    // ---- per-row state. Row i = w0 + 32qb + l32 sees keys [klo, khi).
    int klo[QB], khi[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int i = w0 + 32 * qb + l32;
        klo[qb] = 0;
        khi[qb] = 0;
        if (i < w1) kv_range(i, i + 1, Nq, Nk, wl, wr, &klo[qb], &khi[qb]);
    }

    // ---- Q fragments, B operand of S^T = K Q^T: lane holds query
    // w0+32qb+l32, head-dim elements [16s + 8hh, +8), as 16-bit values.
    i32x4 qf[QB][NKS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qp, (unsigned)(Nq * GRB));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = w0 + 32 * qb + l32;
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                if constexpr (!FP8) {
                    qf[qb][s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        qrs, row * GRB + (16 * s + 8 * hh) * 2, 0, 0));
                } else {
                    const i32x2 w8 = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(
                        qrs, row * GRB + 16 * s + 8 * hh, 0, 0));
                    const i32x2 a = e4m3x4_to_bf16(w8[0]), b = e4m3x4_to_bf16(w8[1]);
                    qf[qb][s] = i32x4{a[0], a[1], b[0], b[1]};
                }
            }
        }
        // Q has landed before the loop, so no wait inside the loop is left
        // for the compiler to place (where it would also cover the K/V copies).
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }

    f32x16 oacc[ND][QB];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = f32x16{};
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }

    // ---- K/V tile staging, issued a tile ahead. 16-bit K and V, and e4m3 V,
    // go HBM -> LDS directly (buffer_load ... lds: lane l of a wave fills the
    // l-th 16-byte slot of a 1 KiB run), each lane fetching the global chunk
    // that belongs in its slot under the swizzled layout. e4m3 K passes
    // through registers to be widened to bf16 on its way into LDS.
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (unsigned)(Nk * GRB));
    const i32x4 kwords = rsrc_words(kp, (unsigned)(Nk * GRB));
    const i32x4 vwords = rsrc_words(vp, (unsigned)(Nk * GRB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    constexpr int KSLOTS = KTILE / 16, VSLOTS = VTILE / 16;
    constexpr int KCPR = KRB / 16, VCPR = VRB / 16;
    constexpr int KSW = KCPR < 8 ? KCPR : 8, VSW = VCPR < 8 ? VCPR : 8;
    i32x4 stk[FP8 ? GLD : 1];
    auto issue_tile = [&](int t, int buf) {
        const int kv0 = t * BC;
        const unsigned kb = smem_base + buf * STAGE;
        const unsigned vb = kb + KTILE;
        if constexpr (!FP8) {
#pragma unroll
            for (int i = 0; i < KSLOTS / NTHREADS; ++i) {
                const int run = 64 * wave + NTHREADS * i;     // first slot of this wave's run
                const int slot = run + lane;
                const int x = slot / KCPR, c = (slot % KCPR) ^ (x & (KSW - 1));
                dma16(kwords, kb + run * 16, (kv0 + x) * GRB + c * 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < GLD; ++i) {
                const int ci = tid + NTHREADS * i;
                const int x = ci / GCPR, c = ci % GCPR;
                stk[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (kv0 + x) * GRB + c * 16, 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < VSLOTS / NTHREADS; ++i) {
            const int run = 64 * wave + NTHREADS * i;
            const int slot = run + lane;
            const int xv = slot / VCPR, c = (slot % VCPR) ^ (xv & (VSW - 1));
            const int x = FP8 ? v8_row_inv(xv) : xv;
            dma16(vwords, vb + run * 16, (kv0 + x) * GRB + c * 16);
        }
    };
    // e4m3 K: widen the staged chunks to bf16 and write them to LDS.
    auto finish_tile = [&](int buf) {
        if constexpr (FP8) {
            uint8_t* kb = smem + buf * STAGE;
#pragma unroll
            for (int i = 0; i < GLD; ++i) {
                const int ci = tid + NTHREADS * i;
                const int x = ci / GCPR, c = ci % GCPR;
                const i32x2 a = e4m3x4_to_bf16(stk[i][0]), b = e4m3x4_to_bf16(stk[i][1]);
                const i32x2 e = e4m3x4_to_bf16(stk[i][2]), f = e4m3x4_to_bf16(stk[i][3]);
                *reinterpret_cast<i32x4*>(kb + lds_off<KRB>(x, 2 * c)) = i32x4{a[0], a[1], b[0], b[1]};
                *reinterpret_cast<i32x4*>(kb + lds_off<KRB>(x, 2 * c + 1)) = i32x4{e[0], e[1], f[0], f[1]};
            }
        }
        // the direct-to-LDS loads of this tile have landed (vmcnt(0)); the
        // barrier that follows publishes them to the other waves
        __builtin_amdgcn_s_waitcnt(0x0F70);
    };

    if (t_lo < t_hi) {
        issue_tile(t_lo, t_lo & 1);
        finish_tile(t_lo & 1);
    }
    __syncthreads();

    const float c2 = p.c;
    const int g = lane >> 4, cl = lane & 15;   // 16-lane group of the transposing reads
    for (int t = t_lo; t < t_hi; ++t) {
        const bool more = (t + 1 < t_hi);
        if (more) issue_tile(t + 1, (t + 1) & 1);

        const int c0 = t * BC;
        const int cls = tile_class(w0, w1, c0, c0 + BC, Nq, Nk, wl, wr);
        if (cls != TILE_SKIP) {
            const lds_u8* kbuf = (const lds_u8*)(smem + (t & 1) * STAGE);
            const lds_u8* vbuf = kbuf + KTILE;

            // ---- S^T = K Q^T over the tile's 64 keys (2 blocks of 32)
            f32x16 sacc[2][QB];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const i32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
                        kbuf + lds_off<KRB>(32 * kb + l32, 2 * s + hh));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma16(QK, a, qf[qb][s], sacc[kb][qb]);
                }
            }

            // ---- mask (edge tiles only). Element r of block kb holds key
            // c0 + 4hh + off with off = 32kb + 8(r/4) + r%4.
            if (cls == TILE_EDGE) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int a = klo[qb] - c0 - 4 * hh, b = khi[qb] - c0 - 4 * hh;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                            if (off < a || off >= b) sacc[kb][qb][r] = -INFINITY;
                        }
                }
            }

            // ---- online softmax (base 2). A row rescales only when its own
            // tile max passes its reference max by more than TAU; the other
            // rows keep alpha = 1 (an exact no-op), so each row's arithmetic
            // depends on its own scores alone.
            float alpha[QB], mt[QB];
            bool need = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = sacc[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
                mx = max_halves(mx);
                mt[qb] = mx * c2;
                const bool nd = mt[qb] > m_run[qb] + I::TAU;
                alpha[qb] = nd ? __builtin_amdgcn_exp2f(m_run[qb] - mt[qb]) : 1.f;
                m_run[qb] = nd ? mt[qb] : m_run[qb];
                need |= nd;
            }
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    l_run[qb] *= alpha[qb];
#pragma unroll
                    for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha[qb];
                }
            }
            bool sr[QB];
            bool sp_any = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float ms = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
                sr[qb] = !FP8 && split_row(__builtin_amdgcn_exp2f(mt[qb] - ms), l_run[qb]);
                sp_any |= sr[qb];
            }
            const bool split = __builtin_amdgcn_ballot_w64(sp_any) != 0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float ms = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
                float sum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][r], c2, -ms));
                        sacc[kb][qb][r] = e;
                        sum += e;
                    }
                l_run[qb] += sum;
            }

            // ---- O^T += V^T P^T
            if constexpr (!FP8) {
                // k-step s covers the tile's keys 16s..16s+15: lane half hh
                // supplies accumulator elements r = 8(s%2)+e of block s/2,
                // i.e. keys 16s + 8(e/4) + 4hh + e%4, and the V^T operand is
                // read in that order by two ds_read_b64_tr_b16 (4 rows x 16
                // columns per 16-lane group; lane receives one column).
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    i32x4 pf[QB], pl[QB];
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const f32x16& e = sacc[s >> 1][qb];
                        const int o = 8 * (s & 1);
                        pf[qb] = i32x4{pack2<IN>(e[o + 0], e[o + 1]), pack2<IN>(e[o + 2], e[o + 3]),
                                       pack2<IN>(e[o + 4], e[o + 5]), pack2<IN>(e[o + 6], e[o + 7])};
                        if (split) {
                            const i32x4 h = pf[qb];
                            pl[qb] = sr[qb] ? i32x4{pack2<IN>(e[o + 0] - unpack_lo<IN>(h[0]), e[o + 1] - unpack_hi<IN>(h[0])),
                                                pack2<IN>(e[o + 2] - unpack_lo<IN>(h[1]), e[o + 3] - unpack_hi<IN>(h[1])),
                                                pack2<IN>(e[o + 4] - unpack_lo<IN>(h[2]), e[o + 5] - unpack_hi<IN>(h[2])),
                                                pack2<IN>(e[o + 6] - unpack_lo<IN>(h[3]), e[o + 7] - unpack_hi<IN>(h[3]))}
                                        : i32x4{};
                        }
                    }
#pragma unroll
                    for (int db = 0; db < ND; ++db) {
                        const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
                        const int x0 = 16 * s + 4 * hh + (cl >> 2);
                        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(vbuf + lds_off<VRB>(x0, ch) + 8 * (cl & 1)));
                        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(vbuf + lds_off<VRB>(x0 + 8, ch) + 8 * (cl & 1)));
                        const i32x2 u0 = __builtin_bit_cast(i32x2, v0), u1 = __builtin_bit_cast(i32x2, v1);
                        const i32x4 a = i32x4{u0[0], u0[1], u1[0], u1[1]};
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) {
                            oacc[db][qb] = mfma16(IN, a, pf[qb], oacc[db][qb]);
                            if (split) oacc[db][qb] = mfma16(IN, a, pl[qb], oacc[db][qb]);
                        }
                    }
                }
            } else {
                // One k-step of 64 keys: element t of lane half hh is
                // accumulator element (block t/16, r = t%16); V^T comes from
                // 4 ds_read_b64_tr_b8 of LDS rows 32hh + 8u + 0..7.
                i32x8 pf[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const f32x16& e = sacc[w >> 2][qb];
                        const int o = 4 * (w & 3);
                        int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[o + 0] * I::PRESCALE, e[o + 1] * I::PRESCALE, 0, false);
                        word = __builtin_amdgcn_cvt_pk_fp8_f32(e[o + 2] * I::PRESCALE, e[o + 3] * I::PRESCALE, word, true);
                        pf[qb][w] = word;
                    }
                }
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const int ch = (32 * db + 16 * (g & 1)) >> 4;
                    i32x8 a;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int x = 32 * hh + 8 * u + (cl >> 1);
                        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) i32x2*)(vbuf + lds_off<VRB>(x, ch) + 8 * (cl & 1)));
                        a[2 * u] = r[0];
                        a[2 * u + 1] = r[1];
                    }
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = mfma_fp8(a, pf[qb], oacc[db][qb]);
                }
            }
        }

        if (more) finish_tile((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
    uint8_t* op = p.o + (size_t)bh * Nq * D * Out<OUT>::EB;
    float* lp = p.lse + (size_t)bh * Nq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum_halves(l_run[qb]);
        const int i = w0 + 32 * qb + l32;
        if (i < w1) {
            const float inv = (lt > 0.f) ? p.out_mul / (lt * I::PRESCALE) : 0.f;
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
            if (hh == 0) lp[i] = (lt > 0.f) ? (m_run[qb] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
        }
    }
    clock_stamp(p.clk, p.clk_n, 1);
}

// ---------------------------------------------------------------- host side

#ifndef FA_KS_MAX_WG
#define FA_KS_MAX_WG 128
#endif
Plan make_plan(int in, int out, int D, int B, int H, int Nq, int mod, bool splitkv) {
    Plan pl;
    pl.in = in;
    pl.out = out;
    pl.D = D;
    pl.bc = BC;
    const long long n_bh = (long long)B * H;
    // The serial kernel (below) takes most problems. Otherwise 16-bit inputs
    // use the pipelined kernel (4 waves at D = 64, 8 at D = 128) and e4m3
    // inputs the 64-key-tile kernel. FA_KNOB_KERNEL forces one (tuning).
    int kernel = (in == IN_E4M3) ? KERNEL_TILE64 : KERNEL_PIPE16;
    // 16-bit inputs at D = 64 go to the key-split kernel where the pipelined
    // kernel would leave waves idle: with at most 64 query rows per head (two
    // or three of its four waves would hold no row), or when it would launch
    // at most FA_KS_MAX_WG workgroups (a CU would hold at most one, and the
    // heaviest tile would walk its keys alone). Elsewhere the key-split
    // kernel's 32-row workgroups copy each K/V tile into LDS four times as
    // often and lose (measured: c2, 384 workgroups, 29.7 against 23.3 us;
    // B8 H32 Nq128, 256 workgroups, 95 against 78 us).
    const bool ks_ok = in != IN_E4M3 && D == 64 && mod == MOD_NONE;
    // The serial kernel (four waves per SIMD at D = 64): 16-bit inputs with
    // or without a score modifier, except on the small grids above, and e4m3
    // inputs without one (not split).
    const bool sr_ok = in != IN_E4M3 || (mod == MOD_NONE && !splitkv);
    if (sr_ok) kernel = KERNEL_SERIAL;
    if (ks_ok && (Nq <= 64 || n_bh * ((Nq + 127) / 128) <= FA_KS_MAX_WG)) kernel = KERNEL_KSPLIT;
    {
        const int f = knob(1);   // FA_KNOB_KERNEL
        if (f == KERNEL_TILE64 || (f == KERNEL_PIPE16 && in != IN_E4M3) || (f == KERNEL_KSPLIT && ks_ok) ||
            (f == KERNEL_SERIAL && sr_ok))
            kernel = f;
    }
    // score modifiers: the serial or the pipelined kernel; split-KV: the
    // serial, the pipelined or the key-split kernel (16-bit inputs)
    if ((mod != MOD_NONE && kernel != KERNEL_SERIAL) || (splitkv && kernel == KERNEL_TILE64)) kernel = KERNEL_PIPE16;
    // 64-key-tile kernel: two 32-row query blocks per wave halve LDS traffic
    // per MFMA and the K/V re-reads per query; one block keeps the grid large
    // on small problems and keeps D = 128 within the register file.
    // Pipelined kernel: one block per wave, so that three waves fit per SIMD
    // (their LDS latency then overlaps) -- measured faster than two blocks.
    int qb = (D == 64 && kernel == KERNEL_TILE64) ? 2 : 1;
    if (qb == 2) {
        const long long wg2 = n_bh * ((Nq + 255) / 256);
        if (wg2 < 512) qb = 1;
    }
    // Tuning override: FA_KNOB_TILE_QB = 1 or 2 forces the query blocks per
    // wave (D = 64 only; D = 128 keeps one block within the register file).
    {
        const int f = knob(2);   // FA_KNOB_TILE_QB
        if ((f == 1 || f == 2) && (D == 64 || f == 1)) qb = f;
    }
    pl.kernel = kernel;
    if (kernel == KERNEL_SERIAL) qb = 1;
    pl.nw = (kernel == KERNEL_PIPE16 && D == 128) ? 8 : WAVES;
    if (kernel == KERNEL_SERIAL) {
        pl.nw = D == 64 ? FA_SR_NW_D64 : FA_SR_NW_D128;
        if (pl.nw == 8 && n_bh * ((Nq + 255) / 256) < 256) pl.nw = 4;
        pl.bc = serial_tile_keys(in, D, pl.nw);
    }
    pl.qb = qb;
    pl.br = pl.nw * 32 * qb;
    if (kernel == KERNEL_KSPLIT) {
        pl.qb = 1;
        pl.br = 32;     // one 32-row block per workgroup, its keys split over the waves
        pl.bc = 128;    // keys per tile: one 32-key sub-tile per wave
    }
    pl.n_qt = (Nq + pl.br - 1) / pl.br;
    pl.n_wg = n_bh * pl.n_qt;
    return pl;
}

template <int IN, int OUT, int D, int QB>
static int launch_one(const Plan& pl, const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((fa_fwd_kernel<IN, OUT, D, QB>), dim3((unsigned)pl.n_wg), dim3(NTHREADS), 0, s, p);
    return (int)hipGetLastError();
}

template <int IN, int OUT, int D>
static int launch_d(const Plan& pl, const Params& p, hipStream_t s) {
    if constexpr (D == 64) {
        if (pl.qb == 2) return launch_one<IN, OUT, D, 2>(pl, p, s);
    }
    return launch_one<IN, OUT, D, 1>(pl, p, s);
}

template <int IN, int OUT>
static int launch_io(const Plan& pl, const Params& p, hipStream_t s) {
    return pl.D == 64 ? launch_d<IN, OUT, 64>(pl, p, s) : launch_d<IN, OUT, 128>(pl, p, s);
}

int launch(const Plan& pl, const Params& p, void* stream) {
    if (pl.kernel == KERNEL_PIPE16) return launch16(pl, p, stream);
    if (pl.kernel == KERNEL_KSPLIT) return launch_ks(pl, p, stream);
    if (pl.kernel == KERNEL_SERIAL) return launch_serial(pl, p, stream);
    hipStream_t s = (hipStream_t)stream;
    if (pl.in == IN_F16 && pl.out == OUT_F16) return launch_io<IN_F16, OUT_F16>(pl, p, s);
    if (pl.in == IN_F16 && pl.out == OUT_F32) return launch_io<IN_F16, OUT_F32>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_BF16) return launch_io<IN_BF16, OUT_BF16>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_F32) return launch_io<IN_BF16, OUT_F32>(pl, p, s);
    if (pl.in == IN_E4M3 && pl.out == OUT_BF16) return launch_io<IN_E4M3, OUT_BF16>(pl, p, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
