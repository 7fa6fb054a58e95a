// Logical-grid tile scheduler for the fused attention forward.
//
// The grid is logical (FLASHLIGHT summary on gist.science, Methodology item 4:
// logical grid dimensions decouple the problem's structure from the hardware
// grid, with a tile size per dimension and small dimensions kept whole in one
// tile). Here the logical dimensions are (batch*head, query tile); the head
// dimension D (64 or 128) is never split. Each workgroup decodes its logical
// tile from its hardware id, and the kv range it visits follows from the mask,
// so fully masked key tiles are never loaded or computed (the same summary's
// Results: skipping masked blocks is what makes block-mask variants fast).
//
// Pure integer code, shared by the host launcher, the kernel and the CPU
// tests (through the fa_plan_* exports).
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

// The mask as one key interval per query row. With delta = Nk - Nq
// (bottom-right alignment) and i' = i + delta, row i sees the keys
//   max(0, i' - wl) <= j <= min(Nk - 1, i' + wr).
// Causal is wr = 0; the causal window of w keys is (wl, wr) = (w - 1, 0); the
// symmetric window |i - j| <= w is (w, w); no mask is wl = wr >= Nq + Nk.
// The entry points clamp wl and wr to Nq + Nk, so every sum below stays far
// inside 32 bits.
FA_HD bool visible(long long i, long long j, int Nq, int Nk, int wl, int wr) {
    const long long ip = i + (long long)Nk - Nq;
    if (j < 0 || j >= Nk) return false;
    return j >= ip - wl && j <= ip + wr;
}

// Keys [lo, hi) visible to at least one row of [r0, r1) (r1 exclusive, r1 > r0).
// Both interval ends grow with the row, so the union runs from row r0's start
// to row r1-1's end.
FA_HD void kv_range(int r0, int r1, int Nq, int Nk, int wl, int wr, int* lo, int* hi) {
    const long long d = (long long)Nk - Nq;
    long long l = (long long)r0 + d - wl, h = (long long)(r1 - 1) + d + wr + 1;
    if (l < 0) l = 0;
    if (h > Nk) h = Nk;
    if (h < 0) h = 0;
    if (l > h) l = h;
    *lo = (int)l;
    *hi = (int)h;
}

// Class of the block rows [w0, w1) x keys [c0, c1):
//   0: no pair visible (the block is skipped),
//   1: every pair visible (no mask is evaluated),
//   2: mixed (the element-wise predicate is applied).
enum { TILE_SKIP = 0, TILE_FULL = 1, TILE_EDGE = 2 };

FA_HD int tile_class(int w0, int w1, int c0, int c1, int Nq, int Nk, int wl, int wr) {
    if (w1 <= w0 || c1 <= c0) return TILE_SKIP;
    const long long d = (long long)Nk - Nq;
    // union over the rows of the visible key interval, [ulo, uhi)
    long long ulo = (long long)w0 + d - wl, uhi = (long long)(w1 - 1) + d + wr + 1;
    if (ulo < 0) ulo = 0;
    if (uhi > Nk) uhi = Nk;
    if ((long long)c1 <= ulo || (long long)c0 >= uhi || uhi <= ulo) return TILE_SKIP;
    // intersection over the rows, [ilo, ihi)
    long long ilo = (long long)(w1 - 1) + d - wl, ihi = (long long)w0 + d + wr + 1;
    if (ilo < 0) ilo = 0;
    if (ihi > Nk) ihi = Nk;
    if ((long long)c0 >= ilo && (long long)c1 <= ihi) return TILE_FULL;
    return TILE_EDGE;
}

// tile_class in 32-bit arithmetic, for the kernels: exact whenever Nq and Nk
// are below 2^28 and wl, wr <= Nq + Nk (the entry points keep every tensor
// below 2^31 bytes for the buffer descriptors and clamp wl and wr).
FA_HD int tile_class32(int w0, int w1, int c0, int c1, int Nq, int Nk, int wl, int wr) {
    if (w1 <= w0 || c1 <= c0) return TILE_SKIP;
    const int d = Nk - Nq;
    int ulo = w0 + d - wl, uhi = w1 - 1 + d + wr + 1;
    if (ulo < 0) ulo = 0;
    if (uhi > Nk) uhi = Nk;
    if (c1 <= ulo || c0 >= uhi || uhi <= ulo) return TILE_SKIP;
    int ilo = w1 - 1 + d - wl, ihi = w0 + d + wr + 1;
    if (ilo < 0) ilo = 0;
    if (ihi > Nk) ihi = Nk;
    if (c0 >= ilo && c1 <= ihi) return TILE_FULL;
    return TILE_EDGE;
}

// The same classes for the blocks rows [a0, a1) x keys [32j, 32j + 32), as
// two ranges of j: every pair visible for j in [*jf0, *jf1), at least one for
// j in [*ju0, *ju1) (outside it the block is skipped). 32-bit arithmetic, under
// the same limits as tile_class32.
FA_HD void block_ranges32(int a0, int a1, int Nq, int Nk, int wl, int wr, int* jf0, int* jf1, int* ju0, int* ju1) {
    const int d = Nk - Nq;
    // union and intersection of the rows' key ranges
    int ulo = a0 + d - wl, uhi = a1 - 1 + d + wr + 1, ilo = a1 - 1 + d - wl, ihi = a0 + d + wr + 1;
    if (ulo < 0) ulo = 0;
    if (uhi > Nk) uhi = Nk;
    if (ilo < 0) ilo = 0;
    if (ihi > Nk) ihi = Nk;
    if (a1 <= a0 || uhi <= ulo) {
        *jf0 = *jf1 = *ju0 = *ju1 = 0;
        return;
    }
    *ju0 = ulo / 32;                      // first j with 32j + 32 > ulo
    *ju1 = (uhi + 31) / 32;               // past the last j with 32j < uhi
    *jf0 = (ilo + 31) / 32;               // first j with 32j >= ilo
    *jf1 = (ihi > 0) ? ihi / 32 : 0;      // past the last j with 32j + 32 <= ihi
    if (*jf1 < *jf0) *jf1 = *jf0;
}

// (causal, window) of fa_fwd as the interval extents: causal is wr = 0, a
// window of w > 0 keys is wl = w - 1; unbounded sides become Nq + Nk.
FA_HD void mask_extents(int causal, int window, int Nq, int Nk, int* wl, int* wr) {
    const int big = Nq + Nk;
    *wr = causal ? 0 : big;
    *wl = (window > 0 && window - 1 < big) ? window - 1 : big;
}

// Heads per group in phase 1 of the workgroup order (decode_wg): as many as
// keep the K and V of the heads in flight on the 8 XCDs within kv_budget
// bytes (the XCDs' L2 caches together), at least 1. per_head_kv is one head's
// K plus V in bytes.
FA_HD int wg_head_group(long long n_bh, long long per_head_kv, long long kv_budget) {
    const bool by_xcd = n_bh % 8 == 0;
    const long long hp = by_xcd ? n_bh / 8 : n_bh;
    const long long in_flight = by_xcd ? 8 * per_head_kv : per_head_kv;
    long long g = in_flight > 0 ? kv_budget / in_flight : hp;
    if (g > hp) g = hp;
    if (g < 1) g = 1;
    return (int)g;
}

// Hardware workgroup id -> (batch*head, query tile).
//
// Workgroups are handed to the 8 XCDs of the chip round-robin by id, and each
// XCD has its own L2. When the head count is a multiple of 8, XCD x gets a
// contiguous block of heads (otherwise the whole grid is one sequence), and
// walks them in two phases:
//   1. the query tiles qt >= tl, in groups of hg heads (the last group may be
//      smaller): within a group the tiles go from last to first across the
//      group's heads;
//   2. the tiles qt < tl of all its heads, from last to first across them.
// Under a causal mask the last tiles carry the most key tiles, so every phase
// starts with its heaviest work. Phase 2 keeps long tiles from starting near
// the end: a long tile dispatched late shares its CU with other workgroups
// for its whole run, and the launch ends in a tail. Its tiles stream only
// short K/V prefixes, so interleaving all heads there costs little cache;
// phase 1 keeps the resident workgroups on few heads, whose K and V the L2
// then serves. hg = 1 and tl = 0 walk one head at a time.
FA_HD void decode_wg(long long wg, int n_bh, int n_qt, int hg, int tl, int* bh, int* qt) {
    long long x = 0, s = wg, hp = n_bh;
    if (n_bh % 8 == 0) {
        x = wg % 8;
        s = wg / 8;
        hp = n_bh / 8;
    }
    const long long T = tl < 0 ? 0 : (tl > n_qt ? n_qt : tl);
    const long long nh = n_qt - T;          // phase-1 tiles per head
    if (s < hp * nh) {
        const long long g = hg < 1 ? 1 : (hg > hp ? hp : hg);
        const long long span = g * nh;      // workgroups of a full group
        const long long gi = s / span, r = s % span;
        const long long gs = (hp - gi * g < g) ? hp - gi * g : g;   // heads in this group
        *bh = (int)(x * hp + gi * g + r % gs);
        *qt = n_qt - 1 - (int)(r / gs);
    } else {
        const long long s2 = s - hp * nh;
        *bh = (int)(x * hp + s2 % hp);
        *qt = (int)(T - 1 - s2 / hp);
    }
}

}  // namespace fa
