"""The logical-grid scheduler, exhaustively on small shapes (CPU).

Checks against the mask predicate written out here: every visible
(query, key) pair lies in its workgroup's key range; the workgroup ids map
one-to-one onto (batch*head, query tile); the block classes the kernel uses
are exact (skipped blocks hold no visible pair, unmasked blocks no hidden one).
"""
import itertools

import numpy as np
import pytest

import exact_attention_02_amd as fa


def vis(i, j, Nq, Nk, causal, window):
    ip = i + Nk - Nq
    return 0 <= j < Nk and (not causal or j <= ip) and (window == 0 or j > ip - window)


def vis_matrix(Nq, Nk, causal, window):
    ip = np.arange(Nq)[:, None] + (Nk - Nq)
    j = np.arange(Nk)[None, :]
    m = np.ones((Nq, Nk), dtype=bool)
    if causal:
        m &= j <= ip
    if window:
        m &= j > ip - window
    return m


SHAPES = [(1, 1, 1, 1), (2, 3, 5, 7), (1, 2, 130, 130), (2, 1, 300, 257), (1, 1, 257, 300), (1, 8, 256, 256),
          (3, 8, 513, 513), (1, 1, 70, 1), (1, 1, 1, 200), (1, 16, 1000, 1000), (2, 4, 40, 0)]
MODES = [(False, 0), (True, 0), (True, 1), (True, 63), (True, 200)]


@pytest.mark.parametrize("B,H,Nq,Nk", SHAPES)
@pytest.mark.parametrize("causal,window", MODES)
@pytest.mark.parametrize("D,dtype", [(64, fa.FA_BF16), (128, fa.FA_BF16), (128, fa.FA_E4M3), (64, fa.FA_F16)])
def test_grid_covers_every_visible_pair_once(B, H, Nq, Nk, causal, window, D, dtype):
    n_wg, br, qw, bc = fa.plan_grid(B, H, Nq, Nk, D, causal, window, dtype)
    n_qt = (Nq + br - 1) // br
    assert n_wg == B * H * n_qt and br % qw == 0 and bc in (64, 128)
    seen = set()
    vm = vis_matrix(Nq, Nk, causal, window)
    for wg in range(n_wg):
        bh, qt, lo, hi = fa.plan_tile(B, H, Nq, Nk, D, causal, window, dtype, wg)
        assert 0 <= bh < B * H and 0 <= qt < n_qt
        assert (bh, qt) not in seen
        seen.add((bh, qt))
        r0, r1 = qt * br, min(qt * br + br, Nq)
        assert 0 <= lo <= hi <= Nk
        cols = np.nonzero(vm[r0:r1].any(axis=0))[0]
        if cols.size:
            # every visible key of the tile's rows is in range, and the range is
            # tight: its first and last keys are visible to some row
            assert lo == cols.min() and hi == cols.max() + 1, (wg, lo, hi)
        else:
            assert lo == hi
    assert len(seen) == n_wg


@pytest.mark.parametrize("Nq,Nk", [(64, 64), (100, 37), (37, 100), (128, 200)])
@pytest.mark.parametrize("causal,window", MODES)
def test_block_class_is_exact(Nq, Nk, causal, window):
    for w0, c0 in itertools.product(range(0, Nq, 13), range(0, Nk + 20, 17)):
        for w1, c1 in [(w0 + 1, c0 + 1), (min(w0 + 32, Nq), c0 + 64), (min(w0 + 64, Nq), c0 + 9)]:
            if w1 <= w0:
                continue
            cls = fa.plan_block_class(w0, w1, c0, c1, Nq, Nk, causal, window)
            pairs = [vis(i, j, Nq, Nk, causal, window) for i in range(w0, w1) for j in range(c0, c1)]
            if cls == 0:
                assert not any(pairs)
            elif cls == 1:
                assert all(pairs)
            else:
                assert cls == 2 and any(pairs) and not all(pairs)


def vis_window(i, j, Nq, Nk, wl, wr):
    """fa_fwd_window's predicate: i' - wl <= j <= i' + wr, a side with extent -1 open."""
    ip = i + Nk - Nq
    return 0 <= j < Nk and (wl < 0 or j >= ip - wl) and (wr < 0 or j <= ip + wr)


EXTENTS = [(-1, -1), (-1, 0), (0, 0), (1, 1), (5, 0), (0, 9), (16, 16), (40, 3), (-1, 7), (12, -1), (500, 500)]


@pytest.mark.parametrize("Nq,Nk", [(64, 64), (130, 97), (97, 130), (300, 300), (1, 50)])
@pytest.mark.parametrize("wl,wr", EXTENTS)
def test_window_range_is_the_tight_union_of_visible_keys(Nq, Nk, wl, wr):
    for r0 in range(0, Nq, 37):
        for r1 in {min(Nq, r0 + 1), min(Nq, r0 + 32), min(Nq, r0 + 128), Nq}:
            lo, hi = fa.plan_window_range(r0, r1, Nq, Nk, wl, wr)
            cols = [j for j in range(Nk) if any(vis_window(i, j, Nq, Nk, wl, wr) for i in range(r0, r1))]
            if cols:
                assert (lo, hi) == (min(cols), max(cols) + 1)
                assert hi - lo == len(cols)   # the visible keys of a row range are contiguous
            else:
                assert lo == hi


@pytest.mark.parametrize("Nq,Nk", [(64, 64), (100, 37), (37, 100), (128, 200)])
@pytest.mark.parametrize("wl,wr", EXTENTS)
def test_block_class_window_is_exact(Nq, Nk, wl, wr):
    for w0, c0 in itertools.product(range(0, Nq, 13), range(0, Nk + 20, 17)):
        for w1, c1 in [(w0 + 1, c0 + 1), (min(w0 + 32, Nq), c0 + 64), (min(w0 + 64, Nq), c0 + 9)]:
            if w1 <= w0:
                continue
            cls = fa.plan_block_class_window(w0, w1, c0, c1, Nq, Nk, wl, wr)
            pairs = [vis_window(i, j, Nq, Nk, wl, wr) for i in range(w0, w1) for j in range(c0, c1)]
            if cls == 0:
                assert not any(pairs)
            elif cls == 1:
                assert all(pairs)
            else:
                assert cls == 2 and any(pairs) and not all(pairs)


def test_window_extents_reproduce_fa_fwd_masks():
    """(causal, window) and their extents give the same ranges and classes."""
    for Nq, Nk in [(64, 64), (100, 37), (37, 100)]:
        for causal, window in MODES:
            wl = window - 1 if window > 0 else -1
            wr = 0 if causal else -1
            for w0, c0 in itertools.product(range(0, Nq, 9), range(0, Nk + 20, 11)):
                w1, c1 = min(w0 + 32, Nq), c0 + 32
                assert fa.plan_block_class(w0, w1, c0, c1, Nq, Nk, causal, window) == \
                    fa.plan_block_class_window(w0, w1, c0, c1, Nq, Nk, wl, wr)


def test_window_extent_below_minus_one_is_rejected():
    assert fa.plan_block_class_window(0, 32, 0, 32, 64, 64, -2, 0) == -1
    with pytest.raises(fa.FaError):
        fa.plan_window_range(0, 32, 64, 64, 0, -2)


def test_heads_stay_on_one_xcd_and_tiles_go_heavy_first():
    # 48 heads (B4 H12), 32 query tiles: workgroups with the same id mod 8
    # (the same XCD under round-robin dispatch) cover 6 whole heads, and
    # within a head the causal query tiles come last-first.
    B, H, N = 4, 12, 8192
    n_wg, br, qw, bc = fa.plan_grid(B, H, N, N, 64, True, 0, fa.FA_BF16)
    heads_of_xcd = {x: set() for x in range(8)}
    order = {}
    for wg in range(n_wg):
        bh, qt, lo, hi = fa.plan_tile(B, H, N, N, 64, True, 0, fa.FA_BF16, wg)
        heads_of_xcd[wg % 8].add(bh)
        order.setdefault(bh, []).append(qt)
    assert all(len(s) == 6 for s in heads_of_xcd.values())
    assert set().union(*heads_of_xcd.values()) == set(range(48))
    for bh, qts in order.items():
        assert qts == sorted(qts, reverse=True)


def test_32bit_block_class_equals_64bit(tmp_path):
    """The kernels classify blocks in 32-bit arithmetic, one block at a time or
    as ranges of 32-key sub-tiles; both must agree with the 64-bit classifier
    everywhere the entry points allow (sizes below 2^28, extents clamped to
    Nq + Nk), for fa_fwd's masks and fa_fwd_window's extents, including the
    extremes of that range."""
    import subprocess
    src = tmp_path / "cls.cpp"
    hdr = fa.LIB_PATH.replace("libfa.so", "csrc/fa_sched.h")
    src.write_text(f'''
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include "{hdr}"
int main() {{
    long long n = 0, bad = 0;
    const int sizes[] = {{1, 2, 31, 32, 33, 64, 100, 257, 1000}};
    auto check = [&](int w0, int w1, int c0, int Nq, int Nk, int wl, int wr) {{
        const int a = fa::tile_class(w0, w1, c0, c0 + 32, Nq, Nk, wl, wr);
        const int b = fa::tile_class32(w0, w1, c0, c0 + 32, Nq, Nk, wl, wr);
        int jf0, jf1, ju0, ju1;
        fa::block_ranges32(w0, w1, Nq, Nk, wl, wr, &jf0, &jf1, &ju0, &ju1);
        const int j = c0 / 32;
        const int r = (j >= jf0 && j < jf1) ? 1 : ((j >= ju0 && j < ju1) ? 2 : 0);
        ++n; if (a != b || a != r) {{ if (bad < 5) std::printf("mismatch %d %d %d %d %d %d %d: %d vs %d vs %d\\n", w0, w1, c0, Nq, Nk, wl, wr, a, b, r); ++bad; }}
    }};
    // The backward's key-parallel kernel classifies 32-row sub-tiles n against
    // its keys [k0, k1) from block_ranges32 with (Nq, Nk) and (wl, wr)
    // swapped; a sub-tile that reaches past Nq must not count as full.
    auto check_t = [&](int k0, int k1, int Nq, int Nk, int wl, int wr) {{
        int nf0, nf1, nu0, nu1;
        fa::block_ranges32(k0, k1, Nk, Nq, wr, wl, &nf0, &nf1, &nu0, &nu1);
        for (int q0 = 0; q0 < Nq + 64; q0 += 32) {{
            int a = (q0 >= Nq) ? 0 : fa::tile_class(q0, q0 + 32 < Nq ? q0 + 32 : Nq, k0, k1, Nq, Nk, wl, wr);
            if (a == 1 && q0 + 32 > Nq) a = 2;
            const int nn = q0 / 32;
            const int r = (nn >= nf0 && nn < nf1) ? 1 : ((nn >= nu0 && nn < nu1) ? 2 : 0);
            ++n; if (a != r) {{ if (bad < 5) std::printf("transposed mismatch %d %d %d %d %d %d %d: %d vs %d\\n", k0, k1, q0, Nq, Nk, wl, wr, a, r); ++bad; }}
        }}
    }};
    for (int Nq : sizes) for (int Nk : sizes) {{
        for (int wl0 : {{-1, 0, 1, 5, 31, 32, 100}}) for (int wr0 : {{-1, 0, 1, 7, 33, 200}}) {{
            const int big = Nq + Nk;
            const int wl = (wl0 < 0 || wl0 > big) ? big : wl0, wr = (wr0 < 0 || wr0 > big) ? big : wr0;
            for (int k0 = 0; k0 < Nk; k0 += 32) check_t(k0, k0 + 32 < Nk ? k0 + 32 : Nk, Nq, Nk, wl, wr);
        }}
    }}
    for (int Nq : sizes) for (int Nk : sizes) {{
        // fa_fwd's (causal, window) masks
        for (int causal = 0; causal < 2; ++causal)
        for (int window = 0; window < Nk + 3; window += (window < 3 ? 1 : 37)) {{
            if (window > 0 && !causal) continue;
            int wl, wr;
            fa::mask_extents(causal, window, Nq, Nk, &wl, &wr);
            for (int w0 = 0; w0 < Nq; w0 += 7) for (int w1 = w0 + 1; w1 <= Nq; w1 += 13)
            for (int c0 = 0; c0 < Nk + 40; c0 += 32) check(w0, w1, c0, Nq, Nk, wl, wr);
        }}
        // fa_fwd_window's extents, clamped as the entry point clamps them
        for (int wl0 : {{-1, 0, 1, 5, 31, 32, 100}}) for (int wr0 : {{-1, 0, 1, 7, 33, 200}}) {{
            const int big = Nq + Nk;
            const int wl = (wl0 < 0 || wl0 > big) ? big : wl0, wr = (wr0 < 0 || wr0 > big) ? big : wr0;
            for (int w0 = 0; w0 < Nq; w0 += 11) for (int w1 = w0 + 1; w1 <= Nq; w1 += 17)
            for (int c0 = 0; c0 < Nk + 40; c0 += 32) check(w0, w1, c0, Nq, Nk, wl, wr);
        }}
    }}
    // extremes: sizes near 2^28, extents up to Nq + Nk
    const int big = (1 << 28) - 64;
    const int ext[][4] = {{{{big, big, big - 2, 0}}, {{big, 64, 2 * big, 2 * big}}, {{64, big, 1, 2 * big}}, {{big, big, 0, 0}}, {{big, big, 2 * big, 0}}, {{big, big, 1000, 1000}}}};
    for (const auto& e : ext) for (int w0 : {{0, 64, e[0] - 64}}) for (int c0 : {{0, 32, e[1] - 32, e[1] - 64}}) {{
        if (w0 < 0 || c0 < 0) continue;
        const int w1 = w0 + 64 < e[0] ? w0 + 64 : e[0];
        const int a = fa::tile_class(w0, w1, c0, c0 + 32, e[0], e[1], e[2], e[3]);
        const int b = fa::tile_class32(w0, w1, c0, c0 + 32, e[0], e[1], e[2], e[3]);
        ++n; if (a != b) {{ std::printf("extreme mismatch %d %d %d\\n", w0, c0, e[0]); ++bad; }}
    }}
    std::printf("%lld cases, %lld mismatches\\n", n, bad);
    return bad != 0;
}}
''')
    exe = tmp_path / "cls"
    subprocess.run(["g++", "-O1", "-std=c++17", "-o", str(exe), str(src)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout


@pytest.mark.parametrize("B,H,N", [(4, 12, 8192), (1, 12, 1000), (3, 5, 700), (2, 8, 300)])
@pytest.mark.parametrize("group", ["1", "2", "4", "5", "64"])
def test_grouped_order_is_a_bijection_heavy_first_per_group(B, H, N, group, knobs):
    # FA_WG_GROUP forces the heads an XCD interleaves (the last group may be
    # smaller). Every (head, tile) appears once; heads stay on their XCD when
    # B*H is a multiple of 8; per XCD the workgroups run group by group, and
    # within a group the tiles go from last to first across its heads.
    knobs.set("FA_WG_GROUP", group)
    knobs.set("FA_WG_LIGHT", "0")   # no interleaved light phase
    n_wg, br, qw, bc = fa.plan_grid(B, H, N, N, 64, True, 0, fa.FA_BF16)
    n_bh = B * H
    n_qt = (N + br - 1) // br
    by_xcd = n_bh % 8 == 0
    hp = n_bh // 8 if by_xcd else n_bh
    g = min(max(int(group), 1), hp)
    seen = set()
    seq = {}
    for wg in range(n_wg):
        bh, qt, lo, hi = fa.plan_tile(B, H, N, N, 64, True, 0, fa.FA_BF16, wg)
        assert (bh, qt) not in seen
        seen.add((bh, qt))
        x = wg % 8 if by_xcd else 0
        if by_xcd:
            assert x * hp <= bh < (x + 1) * hp
        seq.setdefault(x, []).append((bh, qt))
    assert len(seen) == n_bh * n_qt == n_wg
    for x, items in seq.items():
        pos = 0
        for g0 in range(0, hp, g):
            gs = min(g, hp - g0)
            chunk = items[pos:pos + gs * n_qt]
            pos += gs * n_qt
            assert {bh - x * hp for bh, _ in chunk} == set(range(g0, g0 + gs))
            qts = [qt for _, qt in chunk]
            assert qts == sorted(qts, reverse=True)


@pytest.mark.parametrize("B,H,N", [(4, 12, 8192), (3, 5, 700), (2, 8, 300)])
@pytest.mark.parametrize("group,light", [("1", "3"), ("2", "16"), ("4", "0"), ("1", "1000"), ("3", "1")])
def test_two_phase_order_is_a_bijection(B, H, N, group, light, knobs):
    # FA_WG_LIGHT = T: per XCD, the tiles qt >= T go first, group by group
    # (tiles last-first across a group's heads); then the tiles qt < T of all
    # the XCD's heads, last-first across them. T is clamped to the tile count.
    knobs.set("FA_WG_GROUP", group)
    knobs.set("FA_WG_LIGHT", light)
    n_wg, br, qw, bc = fa.plan_grid(B, H, N, N, 64, True, 0, fa.FA_BF16)
    n_bh = B * H
    n_qt = (N + br - 1) // br
    by_xcd = n_bh % 8 == 0
    hp = n_bh // 8 if by_xcd else n_bh
    g = min(max(int(group), 1), hp)
    T = min(int(light), n_qt)
    seen, seq = set(), {}
    for wg in range(n_wg):
        bh, qt, lo, hi = fa.plan_tile(B, H, N, N, 64, True, 0, fa.FA_BF16, wg)
        assert (bh, qt) not in seen
        seen.add((bh, qt))
        x = wg % 8 if by_xcd else 0
        seq.setdefault(x, []).append((bh - x * hp, qt))
    assert len(seen) == n_bh * n_qt == n_wg
    for x, items in seq.items():
        nh = n_qt - T
        heavy, rest = items[:hp * nh], items[hp * nh:]
        assert all(qt >= T for _, qt in heavy) and all(qt < T for _, qt in rest)
        pos = 0
        for g0 in range(0, hp if nh else 0, g):
            gs = min(g, hp - g0)
            chunk = heavy[pos:pos + gs * nh]
            pos += gs * nh
            assert {h for h, _ in chunk} == set(range(g0, g0 + gs))
            assert [qt for _, qt in chunk] == sorted((qt for _, qt in chunk), reverse=True)
        assert [qt for _, qt in rest] == sorted((qt for _, qt in rest), reverse=True)
        for k in range(0, len(rest), hp):
            assert {h for h, _ in rest[k:k + hp]} == set(range(hp))
