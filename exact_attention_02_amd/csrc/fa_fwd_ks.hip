// Small-grid forward for 16-bit inputs at D = 64: one workgroup per 32 query
// rows, whose 4 waves split those rows' keys.
//
// When a problem has few query tiles (a GPT-2-sized layer: 384 tiles of 128
// rows), the pipelined kernel leaves most SIMDs with one or two waves, and the
// heaviest causal tile walks all of its keys alone. Here a workgroup holds
// only 32 rows: the grid is four times larger, and wave w takes the 32-key
// sub-tiles 4T + w of each 128-key tile, so each wave walks a quarter of the
// keys. Each wave keeps its own running max, sum and output (the per-block
// loop of the aiinarabic.com flash-attention page, the algorithm paragraph
// under Figure 4), and the four partial results are merged at the end in LDS
// with the online-softmax identity (gist.science summary of FLASHLIGHT,
// Methodology item 3):
//     M = max_w m_w,   L = sum_w l_w 2^(m_w - M),   O = sum_w O_w 2^(m_w - M) / L.
//
// Per 32 x 32 block a wave forms S^T = K Q^T (lane = query, as in the
// pipelined kernel), masks edge blocks, moves its max to the block's (an
// exact online softmax, no deferred reference), and multiplies V^T by the
// weights split as hi + lo, each rounded to the input type, so the rounding
// of P never reaches O. Skipped sub-tiles cost a wave nothing but the
// barrier. K and V tiles of 128 keys stream through two LDS slots by
// direct-to-LDS copies, in the pipelined kernel's swizzled layout.
//
// Split-KV (p.n_split > 1): workgroup (tile, split) takes a contiguous share of
// the tile's 128-key tiles and writes its O (divided by its own sum) and its
// LSE in fp32 to the workspace, which the merge kernel combines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_sched.h"

namespace fa {

template <int IN, int OUT>
__global__ __launch_bounds__(256, 2) void fa_fwd_ks_kernel(Params p) {
    clock_stamp(p.clk, p.clk_n, 0);
    constexpr int D = 64, RB = 128, CPR = RB / 16, NKS = D / 16, ND = D / 32;
    constexpr int NT = 256, TK = 128;       // threads; keys per tile (4 sub-tiles)
    constexpr int TILE = TK * RB;           // one tensor's tile: 16 KiB
    constexpr int SLOT = 2 * TILE;          // K and V
    constexpr int NDMA = TILE / 16 / NT;    // copies per tensor per tile
    // the merge reuses the slots: per wave O^T (64 x 32 floats), m and the
    // two lane halves' sums (32 floats each)
    constexpr int MO = 0, MM = 4 * D * 32 * 4, ML = MM + 4 * 32 * 4;
    static_assert(ML + 4 * 2 * 32 * 4 <= 2 * SLOT, "merge fits the slots");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SLOT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int g = lane >> 4, cl = lane & 15;
    const int Nq = p.Nq, Nk = p.Nk, wl = p.wl, wr = p.wr;

    int bh, qt, split = 0;
    long long wgid = blockIdx.x;
    if (p.n_split > 1) {
        split = (int)(wgid % p.n_split);
        wgid /= p.n_split;
    }
    decode_wg(wgid, p.n_bh, p.n_qt, p.hg, p.tl, &bh, &qt);
    const int r0 = qt * 32, r1 = min(r0 + 32, Nq);
    int kv_lo, kv_hi;
    kv_range(r0, r1, Nq, Nk, wl, wr, &kv_lo, &kv_hi);
    int t_lo = kv_lo / TK, t_hi = (kv_hi > kv_lo) ? (kv_hi + TK - 1) / TK : kv_lo / TK;
    if (p.n_split > 1) {
        // split s takes tiles [t_lo + nt*s/S, t_lo + nt*(s+1)/S) of the range
        const long long nt = t_hi - t_lo;
        const int a = t_lo + (int)(nt * split / p.n_split), b = t_lo + (int)(nt * (split + 1) / p.n_split);
        t_lo = a;
        t_hi = b;
    }
    int jf0, jf1, ju0, ju1;
    block_ranges32(r0, r1, Nq, Nk, wl, wr, &jf0, &jf1, &ju0, &ju1);
    const int row = r0 + l32;

    // Q of the lane's row, B operand of S^T = K Q^T (every wave holds the same rows)
    i32x4 qf[NKS];
    {
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + (size_t)bh * Nq * RB, (unsigned)(Nq * RB));
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            qf[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                qrs, row * RB + (16 * s + 8 * hh) * 2, 0, 0));
    }
    // the lane's row sees the keys [klo, khi)
    int klo, khi;
    {
        const int ip = row + (Nk - Nq);
        klo = ip - wl;
        khi = ip + wr + 1;
        klo = klo > 0 ? klo : 0;
        khi = khi < Nk ? khi : Nk;
        if (row >= r1) khi = klo;
    }

    const i32x4 kwords = rsrc_words(p.k + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
    const i32x4 vwords = rsrc_words(p.v + (size_t)bh * Nk * RB, (unsigned)(Nk * RB));
    const unsigned smem_base = (unsigned)(unsigned long long)(lds_u8*)smem;
    static_assert((NT / CPR) % 16 == 0, "copy rows");
    const unsigned dma_voff = [&] {
        const int slot = 64 * wave + lane;
        const int x = slot / CPR, c = (slot % CPR) ^ swz16<RB>(x);
        return (unsigned)(x * RB + c * 16);
    }();
    auto issue_tile = [&](int t) {
        const unsigned kb = smem_base + (unsigned)((t & 1) * SLOT);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int run = 64 * wave + NT * i;
            const unsigned soff = (unsigned)((t * TK + i * (NT / CPR)) * RB);
            dma16(kwords, kb + run * 16, dma_voff, soff);
            dma16(vwords, kb + TILE + run * 16, dma_voff, soff);
        }
    };

    int kofs[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kofs[s] = lds_pos<RB>(l32, 2 * s + hh);
    int vofs[ND][2];   // transposing reads: rows 4hh + cl/4 and 8 rows further
#pragma unroll
    for (int db = 0; db < ND; ++db) {
        const int ch = (2 * (32 * db + 16 * (g & 1)) + 8 * (cl & 3)) >> 4;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) vofs[db][h8] = lds_pos<RB>(4 * hh + (cl >> 2) + 8 * h8, ch) + 8 * (cl & 1);
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
    float m = -INFINITY, lh = 0.f;   // running max (base-2 units) and this lane half's sum
    const float c2 = p.c;

    if (t_lo < t_hi) issue_tile(t_lo);
    for (int t = t_lo; t < t_hi; ++t) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's copies of tile t landed
        __syncthreads();                       // ... and every wave's; the other slot is free
        if (t + 1 < t_hi) issue_tile(t + 1);
        const int j = 4 * t + wave;            // this wave's 32-key sub-tile
        if ((unsigned)(j - ju0) >= (unsigned)(ju1 - ju0)) continue;   // no visible pair
        const lds_u8* kt = (const lds_u8*)(smem + (t & 1) * SLOT) + 32 * wave * RB;
        const lds_u8* vt = kt + TILE;
        // S^T: element r of the lane holds key 32j + 8(r/4) + 4hh + r%4 against the lane's row
        f32x16 S = f32x16{};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const i32x4 a = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(kt + kofs[s]);
            S = mfma16(IN, a, qf[s], S);
        }
        if ((unsigned)(j - jf0) >= (unsigned)(jf1 - jf0)) {
            const int a = klo - 32 * j - 4 * hh, b = khi - 32 * j - 4 * hh;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = 8 * (r >> 2) + (r & 3);
                S[r] = (off < a || off >= b) ? -INFINITY : S[r];
            }
        }
        // the row max moves to the block's; O and the sum follow
        float bm = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) bm = fmaxf(bm, S[r]);
        const float mnew = fmaxf(m, max_halves(bm) * c2);
        const float alpha = (mnew == m) ? 1.f : __builtin_amdgcn_exp2f(m - mnew);   // m = -inf: 0
        if (__builtin_amdgcn_ballot_w64(mnew != m) != 0) {
            lh *= alpha;
#pragma unroll
            for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
        }
        m = mnew;
        const float ms = (mnew == -INFINITY) ? 0.f : mnew;   // a row with nothing visible yet
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c2, -ms));
        float s8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) s8[r] = pr[2 * r] + pr[2 * r + 1];
        lh += ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
        // O^T += V^T (hi + lo): the weights and their rounding residuals
        i32x4 hi[2], lo[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int o = 8 * sp;
            hi[sp] = i32x4{pack2<IN>(pr[o + 0], pr[o + 1]), pack2<IN>(pr[o + 2], pr[o + 3]),
                           pack2<IN>(pr[o + 4], pr[o + 5]), pack2<IN>(pr[o + 6], pr[o + 7])};
            const i32x4 h = hi[sp];
            lo[sp] = i32x4{pack2<IN>(pr[o + 0] - unpack_lo<IN>(h[0]), pr[o + 1] - unpack_hi<IN>(h[0])),
                           pack2<IN>(pr[o + 2] - unpack_lo<IN>(h[1]), pr[o + 3] - unpack_hi<IN>(h[1])),
                           pack2<IN>(pr[o + 4] - unpack_lo<IN>(h[2]), pr[o + 5] - unpack_hi<IN>(h[2])),
                           pack2<IN>(pr[o + 6] - unpack_lo<IN>(h[3]), pr[o + 7] - unpack_hi<IN>(h[3]))};
        }
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const i32x2 u0 = read_tr16(vt + 16 * sp * RB + vofs[db][0]);
                const i32x2 u1 = read_tr16(vt + 16 * sp * RB + vofs[db][1]);
                const i32x4 va = i32x4{u0[0], u0[1], u1[0], u1[1]};
                oacc[db] = mfma16(IN, va, hi[sp], oacc[db]);
                oacc[db] = mfma16(IN, va, lo[sp], oacc[db]);
            }
    }

    // ---- merge the four waves' (m, l, O) in LDS
    __syncthreads();   // every wave is done with the tiles
    float* wo = (float*)smem + (MO / 4);
    float* wm = (float*)(smem + MM);
    float* wlh = (float*)(smem + ML);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
            wo[(wave * D + d) * 32 + l32] = oacc[db][r];
        }
    if (hh == 0) wm[wave * 32 + l32] = m;
    wlh[(wave * 2 + hh) * 32 + l32] = lh;
    __syncthreads();
    // thread: row tid / 8, dimensions 8 (tid % 8) .. +7
    const int mr = tid >> 3, d0 = 8 * (tid & 7);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w * 32 + mr]);
    float f[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float mw = wm[w * 32 + mr];
        f[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += f[w] * (wlh[(w * 2) * 32 + mr] + wlh[(w * 2 + 1) * 32 + mr]);
    }
    const int orow = r0 + mr;
    if (orow < r1) {
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        float o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) a = fmaf(f[w], wo[(w * D + d0 + e) * 32 + mr], a);
            o8[e] = a * inv;
        }
        const float lse = (L > 0.f) ? (M + __builtin_amdgcn_logf(L)) * LN2 : -INFINITY;
        if (p.n_split > 1) {
            const size_t sl = (size_t)bh * p.n_split + split;
            uint8_t* dst = (uint8_t*)(p.ws_o + (sl * Nq + orow) * D + d0);
            Out<OUT_F32>::store4(dst, o8[0], o8[1], o8[2], o8[3]);
            Out<OUT_F32>::store4(dst + 16, o8[4], o8[5], o8[6], o8[7]);
            if (d0 == 0) p.ws_lse[sl * Nq + orow] = lse;
        } else {
            uint8_t* dst = p.o + ((size_t)bh * Nq + orow) * D * Out<OUT>::EB + d0 * Out<OUT>::EB;
            Out<OUT>::store4(dst, o8[0], o8[1], o8[2], o8[3]);
            Out<OUT>::store4(dst + 4 * Out<OUT>::EB, o8[4], o8[5], o8[6], o8[7]);
            if (d0 == 0) p.lse[(size_t)bh * Nq + orow] = lse;
        }
    }
    clock_stamp(p.clk, p.clk_n, 1);
}

template <int IN, int OUT>
static int launch_ks_io(const Plan& pl, const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((fa_fwd_ks_kernel<IN, OUT>), dim3((unsigned)(pl.n_wg * p.n_split)), dim3(256), 0, s, p);
    return (int)hipGetLastError();
}

int launch_ks(const Plan& pl, const Params& p, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (pl.in == IN_F16 && pl.out == OUT_F16) return launch_ks_io<IN_F16, OUT_F16>(pl, p, s);
    if (pl.in == IN_F16 && pl.out == OUT_F32) return launch_ks_io<IN_F16, OUT_F32>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_BF16) return launch_ks_io<IN_BF16, OUT_BF16>(pl, p, s);
    if (pl.in == IN_BF16 && pl.out == OUT_F32) return launch_ks_io<IN_BF16, OUT_F32>(pl, p, s);
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
