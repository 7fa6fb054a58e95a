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

// Visibility of key j to query row i, with delta = Nk - Nq (bottom-right
// causal alignment): j < Nk, and j <= i + delta if causal, and
// j > i + delta - window if window > 0.
FA_HD bool visible(long long i, long long j, int Nq, int Nk, int causal, int window) {
    const long long ip = i + (long long)Nk - Nq;
    if (j < 0 || j >= Nk) return false;
    if (causal && j > ip) return false;
    if (window > 0 && j <= ip - window) return false;
    return true;
}

// Keys [lo, hi) visible to at least one row of [r0, r1) (r1 exclusive, r1 > r0).
FA_HD void kv_range(int r0, int r1, int Nq, int Nk, int causal, int window, int* lo, int* hi) {
    const long long d = (long long)Nk - Nq;
    long long l = 0, h = Nk;
    if (causal) {
        const long long c = (long long)(r1 - 1) + d + 1;
        h = c < Nk ? c : Nk;
    }
    if (window > 0) {
        const long long c = (long long)r0 + d - window + 1;
        l = c > 0 ? c : 0;
    }
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

FA_HD int tile_class(int w0, int w1, int c0, int c1, int Nq, int Nk, int causal, int window) {
    if (w1 <= w0 || c1 <= c0) return TILE_SKIP;
    const long long d = (long long)Nk - Nq;
    // union over the rows of the visible key interval
    long long ulo = 0, uhi = Nk;  // [ulo, uhi)
    if (causal) {
        const long long c = (long long)(w1 - 1) + d + 1;
        if (c < uhi) uhi = c;
    }
    if (window > 0) {
        const long long c = (long long)w0 + d - window + 1;
        if (c > ulo) ulo = c;
    }
    if ((long long)c1 <= ulo || (long long)c0 >= uhi) return TILE_SKIP;
    // intersection over the rows
    long long ilo = 0, ihi = Nk;
    if (causal) {
        const long long c = (long long)w0 + d + 1;
        if (c < ihi) ihi = c;
    }
    if (window > 0) {
        const long long c = (long long)(w1 - 1) + d - window + 1;
        if (c > ilo) ilo = c;
    }
    if ((long long)c0 >= ilo && (long long)c1 <= ihi) return TILE_FULL;
    return TILE_EDGE;
}

// tile_class in 32-bit arithmetic, for the kernels: exact whenever Nq, Nk
// and window are below 2^30 (the entry points keep every tensor below 2^31
// bytes for the buffer descriptors, and pass window < Nk).
FA_HD int tile_class32(int w0, int w1, int c0, int c1, int Nq, int Nk, int causal, int window) {
    if (w1 <= w0 || c1 <= c0) return TILE_SKIP;
    const int d = Nk - Nq;
    int ulo = 0, uhi = Nk;
    if (causal && w1 + d < uhi) uhi = w1 + d;
    if (window > 0 && w0 + d - window + 1 > ulo) ulo = w0 + d - window + 1;
    if (c1 <= ulo || c0 >= uhi) return TILE_SKIP;
    int ilo = 0, ihi = Nk;
    if (causal && w0 + d + 1 < ihi) ihi = w0 + d + 1;
    if (window > 0 && w1 + d - window > ilo) ilo = w1 + d - window;
    if (c0 >= ilo && c1 <= ihi) return TILE_FULL;
    return TILE_EDGE;
}

// The same classes for the blocks rows [a0, a1) x keys [32j, 32j + 32), as
// two ranges of j: every pair visible for j in [*jf0, *jf1), at least one for
// j in [*ju0, *ju1) (outside it the block is skipped). 32-bit arithmetic, under
// the same limits as tile_class32.
FA_HD void block_ranges32(int a0, int a1, int Nq, int Nk, int causal, int window, int* jf0, int* jf1, int* ju0,
                          int* ju1) {
    const int d = Nk - Nq;
    int ulo = 0, uhi = Nk, ilo = 0, ihi = Nk;   // union and intersection of the rows' key ranges
    if (causal) {
        if (a1 + d < uhi) uhi = a1 + d;
        if (a0 + d + 1 < ihi) ihi = a0 + d + 1;
    }
    if (window > 0) {
        if (a0 + d - window + 1 > ulo) ulo = a0 + d - window + 1;
        if (a1 + d - window > ilo) ilo = a1 + d - window;
    }
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

// Hardware workgroup id -> (batch*head, query tile).
//
// Workgroups are handed to the 8 XCDs of the chip round-robin by id, and each
// XCD has its own L2. When the head count is a multiple of 8, XCD x gets a
// contiguous block of heads and walks them one head at a time, so the
// workgroups resident on one XCD share one head's K and V in that L2. Within
// a head the query tiles go from last to first: under a causal mask the last
// tiles carry the most key tiles, so the heaviest work starts first and the
// light tiles fill the tail.
FA_HD void decode_wg(long long wg, int n_bh, int n_qt, int* bh, int* qt) {
    if (n_bh % 8 == 0) {
        const long long x = wg % 8, s = wg / 8;
        const long long hp = n_bh / 8;
        *bh = (int)(x * hp + s / n_qt);
        *qt = n_qt - 1 - (int)(s % n_qt);
    } else {
        *bh = (int)(wg / n_qt);
        *qt = n_qt - 1 - (int)(wg % n_qt);
    }
}

}  // namespace fa
