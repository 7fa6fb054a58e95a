"""Pins of the float64 CPU oracle to facts other than itself.

Each test checks the oracle against something the pages or the mathematics
fix: closed forms of softmax(QK^T/sqrt(d)) V (aiinarabic.com flash-attention
page, equation (1)), invariants of a convex combination, brute force at 50
significant digits, an independent library routine (torch's float64 SDPA with
an explicit boolean mask), and the page's own worked-example figures. The last
test plants plausible mistakes into copies of oracle.c and checks that the
pins catch every one.
"""
import json
import math
import os
import shutil
import tempfile

import mpmath
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def rnd(shape, seed, tid=0):
    n = 1
    for s in shape:
        n *= s
    return synth.normal(seed, tid, n).view(shape)


def mask_matrix(Nq, Nk, causal, window):
    """Boolean [Nq, Nk] keep-mask built from the predicate, independently of the oracle."""
    i = torch.arange(Nq).view(-1, 1) + (Nk - Nq)
    j = torch.arange(Nk).view(1, -1)
    keep = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        keep &= j <= i
    if window > 0:
        keep &= j > i - window
    return keep


def mask_matrix_window(Nq, Nk, wl, wr):
    """Boolean [Nq, Nk] keep-mask of the extents mask, independently of the oracle:
    row i keeps j with i' - wl <= j <= i' + wr (i' = i + Nk - Nq; a negative extent is open)."""
    i = torch.arange(Nq).view(-1, 1) + (Nk - Nq)
    j = torch.arange(Nk).view(1, -1)
    keep = torch.ones(Nq, Nk, dtype=torch.bool)
    if wl >= 0:
        keep &= j >= i - wl
    if wr >= 0:
        keep &= j <= i + wr
    return keep


def page_sliding_window_mask(n, window):
    """The sliding-window mask exactly as the inskillml module's sparse-patterns
    example builds it: row i keeps columns max(0, i - window) .. min(n, i + window + 1) - 1."""
    mask = torch.zeros(n, n, dtype=torch.bool)
    for i in range(n):
        lo = max(0, i - window)
        hi = min(n, i + window + 1)
        mask[i, lo:hi] = True
    return mask


# ---------------------------------------------------------------- brute force

def mp_attention(Q, K, V, scale, keep):
    """Softmax attention at 50 significant digits; inputs are exact binary floats."""
    mpmath.mp.dps = 50
    Nq, D = Q.shape
    Nk = K.shape[0]
    O = [[mpmath.mpf(0)] * D for _ in range(Nq)]
    L = []
    sc = mpmath.mpf(scale)
    for i in range(Nq):
        js = [j for j in range(Nk) if keep[i, j]]
        if not js:
            L.append(-mpmath.inf)
            continue
        s = {j: sc * mpmath.fsum(mpmath.mpf(float(Q[i, d])) * mpmath.mpf(float(K[j, d])) for d in range(D)) for j in js}
        den = mpmath.fsum(mpmath.exp(s[j]) for j in js)
        for d in range(D):
            O[i][d] = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(float(V[j, d])) for j in js) / den
        L.append(mpmath.log(den))
    return O, L


@pytest.mark.parametrize("Nq,Nk,D,causal,window", [
    (1, 1, 3, False, 0), (3, 3, 4, False, 0), (4, 4, 4, True, 0), (5, 3, 3, True, 0),
    (3, 5, 3, True, 0), (5, 5, 4, True, 2), (4, 6, 3, True, 3), (5, 5, 8, False, 0),
])
def test_bruteforce_50_digits(Nq, Nk, D, causal, window):
    Q = rnd((1, 1, Nq, D), 11, 0) * 1.7
    K = rnd((1, 1, Nk, D), 11, 1) * 1.3
    V = rnd((1, 1, Nk, D), 11, 2)
    scale = 0.61
    O, L = oracle.attention(Q, K, V, scale, causal, window)
    keep = mask_matrix(Nq, Nk, causal, window)
    s32 = float(torch.tensor(scale, dtype=torch.float32))
    Om, Lm = mp_attention(Q[0, 0], K[0, 0], V[0, 0], s32, keep)
    for i in range(Nq):
        if Lm[i] == -mpmath.inf:
            assert L[0, 0, i].item() == -math.inf
            assert torch.all(O[0, 0, i] == 0)
            continue
        assert abs(L[0, 0, i].item() - float(Lm[i])) <= 1e-13 * max(1.0, abs(float(Lm[i])))
        for d in range(D):
            assert abs(O[0, 0, i, d].item() - float(Om[i][d])) <= 1e-13


@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [
    (4, 4, 3, 1, 1), (5, 5, 4, 0, 2), (5, 5, 3, 2, 0), (4, 4, 4, 0, 0), (3, 6, 3, 3, -1),
    (6, 3, 3, -1, 1), (5, 5, 3, 1, 1),
])
def test_bruteforce_50_digits_window_extents(Nq, Nk, D, wl, wr):
    Q = rnd((1, 1, Nq, D), 12, 0) * 1.7
    K = rnd((1, 1, Nk, D), 12, 1) * 1.3
    V = rnd((1, 1, Nk, D), 12, 2)
    scale = 0.61
    O, L = oracle.attention(Q, K, V, scale, window_left=wl, window_right=wr)
    keep = mask_matrix_window(Nq, Nk, wl, wr)
    Om, Lm = mp_attention(Q[0, 0], K[0, 0], V[0, 0], float(torch.tensor(scale, dtype=torch.float32)), keep)
    for i in range(Nq):
        if Lm[i] == -mpmath.inf:
            assert L[0, 0, i].item() == -math.inf
            assert torch.all(O[0, 0, i] == 0)
            continue
        assert abs(L[0, 0, i].item() - float(Lm[i])) <= 1e-13 * max(1.0, abs(float(Lm[i])))
        for d in range(D):
            assert abs(O[0, 0, i, d].item() - float(Om[i][d])) <= 1e-13


# ------------------------------------------------------- independent library

@pytest.mark.parametrize("Nq,Nk,D,causal,window", [
    (17, 17, 64, False, 0), (65, 65, 64, True, 0), (129, 129, 128, True, 0),
    (64, 100, 64, True, 0), (100, 64, 64, True, 0), (129, 129, 64, True, 16),
    (33, 200, 128, False, 0), (257, 257, 64, True, 100),
])
def test_against_torch_sdpa_float64(Nq, Nk, D, causal, window):
    B, H = 2, 2
    Q = rnd((B, H, Nq, D), 21, 0)
    K = rnd((B, H, Nk, D), 21, 1)
    V = rnd((B, H, Nk, D), 21, 2)
    scale = 1.0 / math.sqrt(D)
    s32 = float(torch.tensor(scale, dtype=torch.float32))
    O, L = oracle.attention(Q, K, V, scale, causal, window)
    keep = mask_matrix(Nq, Nk, causal, window)
    Oref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=keep, scale=s32)
    S = torch.matmul(Q, K.transpose(-1, -2)) * s32
    Lref = torch.logsumexp(S.masked_fill(~keep, -math.inf), dim=-1)
    rows_ok = keep.any(dim=1)
    assert torch.allclose(O[:, :, rows_ok], Oref[:, :, rows_ok], rtol=0, atol=1e-12)
    assert torch.allclose(L[:, :, rows_ok], Lref[:, :, rows_ok], rtol=1e-13, atol=1e-13)
    assert torch.all(O[:, :, ~rows_ok] == 0)
    assert torch.all(L[:, :, ~rows_ok] == -math.inf)


@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [
    (129, 129, 64, 16, 16), (200, 200, 64, 8, 40), (100, 64, 128, -1, 5), (64, 100, 64, 10, -1),
    (257, 257, 64, 100, 100), (90, 90, 64, 0, 0),
])
def test_window_extents_against_torch_sdpa_float64(Nq, Nk, D, wl, wr):
    B, H = 1, 2
    Q, K, V = rnd((B, H, Nq, D), 22, 0), rnd((B, H, Nk, D), 22, 1), rnd((B, H, Nk, D), 22, 2)
    s32 = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    O, L = oracle.attention(Q, K, V, 1.0 / math.sqrt(D), window_left=wl, window_right=wr)
    keep = mask_matrix_window(Nq, Nk, wl, wr)
    Oref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=keep, scale=s32)
    Lref = torch.logsumexp((torch.matmul(Q, K.transpose(-1, -2)) * s32).masked_fill(~keep, -math.inf), dim=-1)
    rows_ok = keep.any(dim=1)
    assert torch.allclose(O[:, :, rows_ok], Oref[:, :, rows_ok], rtol=0, atol=1e-12)
    assert torch.allclose(L[:, :, rows_ok], Lref[:, :, rows_ok], rtol=1e-13, atol=1e-13)
    assert torch.all(L[:, :, ~rows_ok] == -math.inf)


def test_sliding_window_matches_the_pages_mask_example():
    """The pages' own sliding-window example (n = 1024, window = 128), mask built as the page builds it."""
    n, window, D = 1024, 128, 64
    keep = page_sliding_window_mask(n, window)
    assert torch.equal(keep, mask_matrix_window(n, n, window, window))
    Q, K, V = rnd((1, 1, n, D), 23, 0), rnd((1, 1, n, D), 23, 1), rnd((1, 1, n, D), 23, 2)
    s32 = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    O, L = oracle.attention(Q, K, V, 1.0 / math.sqrt(D), window_left=window, window_right=window)
    Oref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=keep, scale=s32)
    assert torch.allclose(O, Oref, rtol=0, atol=1e-12)
    assert oracle.pair_count_window(n, n, window, window) == int(keep.sum())


# ------------------------------------------------------- score modifiers

def alibi_bias(Nq, Nk, slopes):
    """[H, Nq, Nk] additive ALiBi bias slope_h * (j - i'), built independently of the oracle."""
    i = torch.arange(Nq, dtype=torch.float64).view(-1, 1) + (Nk - Nq)
    j = torch.arange(Nk, dtype=torch.float64).view(1, -1)
    return torch.stack([s * (j - i) for s in slopes])


@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [(65, 65, 64, -1, 0), (100, 64, 64, -1, 0), (64, 100, 128, -1, -1),
                                           (129, 129, 64, 20, 20), (90, 90, 64, 10, 0)])
def test_alibi_against_torch_sdpa_float_mask(Nq, Nk, D, wl, wr):
    B, H = 1, 3
    Q, K, V = rnd((B, H, Nq, D), 24, 0), rnd((B, H, Nk, D), 24, 1), rnd((B, H, Nk, D), 24, 2)
    slopes = [0.5, 0.125, 0.03125]
    s32 = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    O, L = oracle.attention(Q, K, V, 1.0 / math.sqrt(D), window_left=wl, window_right=wr,
                            score_mod="alibi", alibi_slopes=slopes)
    keep = mask_matrix_window(Nq, Nk, wl, wr)
    bias = alibi_bias(Nq, Nk, slopes).masked_fill(~keep, -math.inf).unsqueeze(0)
    Oref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=bias, scale=s32)
    Lref = torch.logsumexp(torch.matmul(Q, K.transpose(-1, -2)) * s32 + bias, dim=-1)
    ok = keep.any(dim=1)
    assert torch.allclose(O[:, :, ok], Oref[:, :, ok], rtol=0, atol=1e-12)
    assert torch.allclose(L[:, :, ok], Lref[:, :, ok], rtol=1e-13, atol=1e-12)


def test_alibi_zero_query_is_a_geometric_series():
    """With Q = 0 the causal ALiBi weights of row i are e^(-slope*k), k = i - j: a geometric series."""
    N, D, slope = 60, 64, 0.3
    Q = torch.zeros(1, 1, N, D, dtype=torch.float64)
    K, V = rnd((1, 1, N, D), 25, 1), rnd((1, 1, N, D), 25, 2)
    O, L = oracle.attention(Q, K, V, 0.125, True, 0, score_mod="alibi", alibi_slopes=[slope])
    r = math.exp(-slope)
    for i in range(N):
        lse = math.log((1 - r ** (i + 1)) / (1 - r))
        assert abs(L[0, 0, i].item() - lse) <= 1e-13 * max(1.0, abs(lse))
        w = torch.tensor([r ** (i - j) for j in range(i + 1)], dtype=torch.float64)
        assert torch.allclose(O[0, 0, i], (w[:, None] * V[0, 0, : i + 1]).sum(0) / w.sum(), atol=1e-13)


def test_alibi_with_zero_slope_and_softcap_limits_are_plain_attention():
    N, D = 80, 64
    Q, K, V = rnd((1, 2, N, D), 26, 0), rnd((1, 2, N, D), 26, 1), rnd((1, 2, N, D), 26, 2)
    O0, L0 = oracle.attention(Q, K, V, 0.125, True, 0)
    O1, L1 = oracle.attention(Q, K, V, 0.125, True, 0, score_mod="alibi", alibi_slopes=[0.0, 0.0])
    assert torch.equal(O0, O1) and torch.equal(L0, L1)
    O2, L2 = oracle.attention(Q, K, V, 0.125, True, 0, score_mod="softcap", softcap=1e7)
    assert torch.allclose(O2, O0, atol=1e-10) and torch.allclose(L2, L0, atol=1e-10)
    # a tiny cap flattens every score to (almost) the same value: the weights become uniform
    O3, L3 = oracle.attention(Q, K, V, 0.125, True, 0, score_mod="softcap", softcap=1e-9)
    cnt = torch.arange(1, N + 1, dtype=torch.float64)
    assert torch.allclose(O3, V.cumsum(dim=2) / cnt.view(1, 1, N, 1), atol=1e-8)
    assert torch.allclose(L3, torch.log(cnt).expand_as(L3), atol=1e-8)


@pytest.mark.parametrize("Nq,Nk,D,causal,cap", [(4, 4, 3, True, 0.8), (5, 3, 4, True, 2.5), (3, 5, 3, False, 0.3)])
def test_softcap_bruteforce_50_digits(Nq, Nk, D, causal, cap):
    Q, K, V = rnd((1, 1, Nq, D), 27, 0) * 2.0, rnd((1, 1, Nk, D), 27, 1) * 1.5, rnd((1, 1, Nk, D), 27, 2)
    scale = 0.61
    O, L = oracle.attention(Q, K, V, scale, causal, 0, score_mod="softcap", softcap=cap)
    mpmath.mp.dps = 50
    keep = mask_matrix(Nq, Nk, causal, 0)
    sc = mpmath.mpf(float(torch.tensor(scale, dtype=torch.float32)))
    cp = mpmath.mpf(cap)
    for i in range(Nq):
        js = [j for j in range(Nk) if keep[i, j]]
        if not js:
            continue
        s = {j: cp * mpmath.tanh(sc * mpmath.fsum(mpmath.mpf(float(Q[0, 0, i, d])) * mpmath.mpf(float(K[0, 0, j, d]))
                                                   for d in range(D)) / cp) for j in js}
        den = mpmath.fsum(mpmath.exp(s[j]) for j in js)
        assert abs(L[0, 0, i].item() - float(mpmath.log(den))) <= 1e-13
        for d in range(D):
            ref = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(float(V[0, 0, j, d])) for j in js) / den
            assert abs(O[0, 0, i, d].item() - float(ref)) <= 1e-13


# ------------------------------------------------------------- backward

def fwd_loss(Q, K, V, dO, scale, wl, wr):
    """sum(dO * O) through the (pinned) forward oracle."""
    O, _ = oracle.attention(Q, K, V, scale, window_left=wl, window_right=wr)
    return float((O * dO).sum())


@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [(6, 6, 8, -1, 0), (5, 9, 8, -1, -1), (9, 5, 8, -1, 0), (8, 8, 4, 2, 1),
                                           (7, 7, 16, 0, 0)])
def test_bwd_matches_finite_differences_of_the_forward(Nq, Nk, D, wl, wr):
    B, H = 1, 2
    Q, K, V = rnd((B, H, Nq, D), 41, 0), rnd((B, H, Nk, D), 41, 1), rnd((B, H, Nk, D), 41, 2)
    dO = rnd((B, H, Nq, D), 41, 3)
    scale = 0.7
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, scale, wl, wr)
    h = 1e-5
    for X, G, tid in [(Q, dQ, 4), (K, dK, 5), (V, dV, 6)]:
        E = rnd(X.shape, 42, tid)
        X0 = X.clone()
        X.add_(h * E)
        fp = fwd_loss(Q, K, V, dO, scale, wl, wr)
        X.copy_(X0 - h * E)
        fm = fwd_loss(Q, K, V, dO, scale, wl, wr)
        X.copy_(X0)
        fd = (fp - fm) / (2 * h)
        an = float((G * E).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (tid, fd, an)


@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [(33, 33, 64, -1, 0), (40, 70, 64, -1, -1), (70, 40, 128, -1, 0),
                                           (64, 64, 64, 10, 10), (50, 50, 64, 5, 0)])
def test_bwd_matches_torch_autograd_float64(Nq, Nk, D, wl, wr):
    B, H = 1, 2
    Q, K, V = rnd((B, H, Nq, D), 43, 0), rnd((B, H, Nk, D), 43, 1), rnd((B, H, Nk, D), 43, 2)
    dO = rnd((B, H, Nq, D), 43, 3)
    scale = 1.0 / math.sqrt(D)
    s32 = float(torch.tensor(scale, dtype=torch.float32))
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, scale, wl, wr)
    keep = mask_matrix_window(Nq, Nk, wl, wr)
    Qg, Kg, Vg = (t.clone().requires_grad_(True) for t in (Q, K, V))
    S = torch.matmul(Qg, Kg.transpose(-1, -2)) * s32
    P = torch.softmax(S.masked_fill(~keep, -math.inf), dim=-1)
    P = torch.nan_to_num(P, nan=0.0)   # rows with no visible key contribute nothing
    O = torch.matmul(P, Vg)
    O.backward(dO)
    assert torch.allclose(dQ, Qg.grad, rtol=0, atol=1e-12)
    assert torch.allclose(dK, Kg.grad, rtol=0, atol=1e-12)
    assert torch.allclose(dV, Vg.grad, rtol=0, atol=1e-12)


def test_bwd_uniform_weights_give_mean_upstream_for_dv():
    """Q = 0 without a mask: every weight is 1/Nk, so dV_j is the mean of dO over the rows."""
    Nq, Nk, D = 30, 20, 64
    Q = torch.zeros(1, 1, Nq, D, dtype=torch.float64)
    K, V, dO = rnd((1, 1, Nk, D), 44, 1), rnd((1, 1, Nk, D), 44, 2), rnd((1, 1, Nq, D), 44, 3)
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, 0.125, -1, -1)
    assert torch.allclose(dV[0, 0], dO[0, 0].sum(0, keepdim=True).expand(Nk, D) / Nk, atol=1e-13)


def fwd_loss_mod(Q, K, V, dO, scale, wl, wr, **mod):
    """sum(dO * O) through the (pinned) forward oracle with a score modifier."""
    O, _ = oracle.attention(Q, K, V, scale, window_left=wl, window_right=wr, **mod)
    return float((O * dO).sum())


BWD_MODS = [dict(score_mod="softcap", softcap=0.9), dict(score_mod="softcap", softcap=3.0),
            dict(score_mod="alibi", alibi_slopes=[0.7, 0.05])]


@pytest.mark.parametrize("mod", BWD_MODS, ids=["softcap0.9", "softcap3", "alibi"])
@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [(6, 6, 8, -1, 0), (5, 9, 8, -1, -1), (9, 5, 8, 2, 1)])
def test_bwd_mod_matches_finite_differences_of_the_forward(mod, Nq, Nk, D, wl, wr):
    B, H = 1, 2
    Q, K, V = rnd((B, H, Nq, D), 45, 0), rnd((B, H, Nk, D), 45, 1), rnd((B, H, Nk, D), 45, 2)
    dO = rnd((B, H, Nq, D), 45, 3)
    scale = 0.7
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, scale, wl, wr, **mod)
    h = 1e-5
    for X, G, tid in [(Q, dQ, 4), (K, dK, 5), (V, dV, 6)]:
        E = rnd(X.shape, 46, tid)
        X0 = X.clone()
        X.add_(h * E)
        fp = fwd_loss_mod(Q, K, V, dO, scale, wl, wr, **mod)
        X.copy_(X0 - h * E)
        fm = fwd_loss_mod(Q, K, V, dO, scale, wl, wr, **mod)
        X.copy_(X0)
        fd = (fp - fm) / (2 * h)
        an = float((G * E).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (tid, fd, an)


@pytest.mark.parametrize("mod", BWD_MODS, ids=["softcap0.9", "softcap3", "alibi"])
@pytest.mark.parametrize("Nq,Nk,D,wl,wr", [(33, 33, 64, -1, 0), (40, 70, 64, -1, -1), (70, 40, 128, 5, 3)])
def test_bwd_mod_matches_torch_autograd_float64(mod, Nq, Nk, D, wl, wr):
    """The modifier written out in torch (cap tanh(S / cap); S + slope (j - i')) and differentiated by autograd."""
    B, H = 1, 2
    Q, K, V = rnd((B, H, Nq, D), 47, 0), rnd((B, H, Nk, D), 47, 1), rnd((B, H, Nk, D), 47, 2)
    dO = rnd((B, H, Nq, D), 47, 3)
    scale = 1.0 / math.sqrt(D)
    s32 = float(torch.tensor(scale, dtype=torch.float32))
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, scale, wl, wr, **mod)
    keep = mask_matrix_window(Nq, Nk, wl, wr)
    Qg, Kg, Vg = (t.clone().requires_grad_(True) for t in (Q, K, V))
    S = torch.matmul(Qg, Kg.transpose(-1, -2)) * s32
    if mod["score_mod"] == "softcap":
        S = mod["softcap"] * torch.tanh(S / mod["softcap"])
    else:
        S = S + alibi_bias(Nq, Nk, mod["alibi_slopes"]).unsqueeze(0)
    P = torch.nan_to_num(torch.softmax(S.masked_fill(~keep, -math.inf), dim=-1), nan=0.0)
    torch.matmul(P, Vg).backward(dO)
    for a, b in ((dQ, Qg.grad), (dK, Kg.grad), (dV, Vg.grad)):
        assert torch.allclose(a, b, rtol=0, atol=1e-12)


def test_bwd_mod_limits_reduce_to_plain_attention():
    """Zero ALiBi slopes give the plain gradients bit for bit; a cap far above every score gives them to rounding."""
    Q, K, V, dO = rnd((1, 2, 20, 16), 48, 0), rnd((1, 2, 25, 16), 48, 1), rnd((1, 2, 25, 16), 48, 2), \
        rnd((1, 2, 20, 16), 48, 3)
    plain = oracle.attention_bwd(Q, K, V, dO, 0.3, -1, 0)
    zero = oracle.attention_bwd(Q, K, V, dO, 0.3, -1, 0, score_mod="alibi", alibi_slopes=[0.0, 0.0])
    big = oracle.attention_bwd(Q, K, V, dO, 0.3, -1, 0, score_mod="softcap", softcap=1e8)
    for a, b, c in zip(plain, zero, big):
        assert torch.equal(a, b)
        assert torch.allclose(a, c, rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("Nq,Nk,causal,window", [(40, 40, False, 0), (40, 40, True, 0), (40, 40, True, 7), (30, 50, True, 0)])
def test_zero_query_gives_mean_of_visible_values(Nq, Nk, causal, window):
    D = 64
    Q = torch.zeros(1, 2, Nq, D, dtype=torch.float64)
    K = rnd((1, 2, Nk, D), 31, 1)
    V = rnd((1, 2, Nk, D), 31, 2)
    O, L = oracle.attention(Q, K, V, 0.125, causal, window)
    for i in range(Nq):
        lo, hi = oracle.visible_keys(i, Nq, Nk, causal, window)
        n = hi - lo
        mean = V[:, :, lo:hi].mean(dim=2)
        assert torch.allclose(O[:, :, i], mean, atol=1e-14, rtol=0)
        assert abs(L[0, 0, i].item() - math.log(n)) <= 1e-14
    # the page-level special cases: non-causal -> log Nk; causal -> log(i+1); window -> log(min(i+1, w))
    if not causal:
        assert torch.allclose(L, torch.full_like(L, math.log(Nk)), atol=1e-14)
    elif window and Nq == Nk:
        ref = torch.tensor([math.log(min(i + 1, window)) for i in range(Nq)], dtype=torch.float64)
        assert torch.allclose(L[0, 0], ref, atol=1e-14)
    elif Nq == Nk:
        ref = torch.tensor([math.log(i + 1) for i in range(Nq)], dtype=torch.float64)
        assert torch.allclose(L[0, 0], ref, atol=1e-14)


@pytest.mark.parametrize("D,a", [(64, 80.0), (128, 96.0)])
@pytest.mark.parametrize("t", [0, 31, 64, 127])
def test_one_hot_score_selects_value_row(D, a, t):
    N = 128
    scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))
    Q = torch.zeros(1, 1, N, D, dtype=torch.float64)
    Q[..., 0] = a
    K = torch.zeros(1, 1, N, D, dtype=torch.float64)
    K[0, 0, t, 0] = a
    V = rnd((1, 1, N, D), 41, 2)
    O, L = oracle.attention(Q, K, V, scale, False, 0)
    assert torch.equal(O[0, 0], V[0, 0, t].expand(N, D))
    assert torch.allclose(L[0, 0], torch.full((N,), a * a * scale, dtype=torch.float64), rtol=1e-15, atol=0)


@pytest.mark.parametrize("Nq,Nk,wl,wr", [(40, 40, 5, 5), (40, 40, 0, 7), (30, 50, -1, 3), (50, 30, 4, -1)])
def test_zero_query_window_extents_gives_mean_of_visible_values(Nq, Nk, wl, wr):
    D = 64
    Q = torch.zeros(1, 1, Nq, D, dtype=torch.float64)
    K, V = rnd((1, 1, Nk, D), 32, 1), rnd((1, 1, Nk, D), 32, 2)
    O, L = oracle.attention(Q, K, V, 0.125, window_left=wl, window_right=wr)
    ip = torch.arange(Nq) + (Nk - Nq)
    for i in range(Nq):
        lo = max(0, int(ip[i]) - wl) if wl >= 0 else 0
        hi = min(Nk, int(ip[i]) + wr + 1) if wr >= 0 else Nk
        if hi <= lo:
            assert L[0, 0, i].item() == -math.inf
            continue
        assert abs(L[0, 0, i].item() - math.log(hi - lo)) <= 1e-13
        assert torch.allclose(O[0, 0, i], V[0, 0, lo:hi].mean(0), atol=1e-13)


def test_window_one_sees_only_itself():
    N, D = 50, 64
    Q, K, V = rnd((1, 2, N, D), 51, 0), rnd((1, 2, N, D), 51, 1), rnd((1, 2, N, D), 51, 2)
    O, L = oracle.attention(Q, K, V, 0.125, True, 1)
    assert torch.equal(O, V)
    ref = 0.125 * (Q * K).sum(-1)
    assert torch.allclose(L, ref, rtol=1e-14, atol=1e-14)


def test_causal_first_row_is_first_value():
    N, D = 70, 128
    Q, K, V = rnd((2, 1, N, D), 61, 0), rnd((2, 1, N, D), 61, 1), rnd((2, 1, N, D), 61, 2)
    O, L = oracle.attention(Q, K, V, 0.088, True, 0)
    s32 = float(torch.tensor(0.088, dtype=torch.float32))
    assert torch.equal(O[:, :, 0], V[:, :, 0])
    assert torch.allclose(L[:, :, 0], s32 * (Q[:, :, 0] * K[:, :, 0]).sum(-1), rtol=1e-14)


def test_affine_values_and_constant_column():
    N, D = 60, 64
    Q, K, V = rnd((1, 1, N, D), 71, 0), rnd((1, 1, N, D), 71, 1), rnd((1, 1, N, D), 71, 2)
    V[..., 5] = 0.75
    O, _ = oracle.attention(Q, K, V, 0.125, True, 0)
    assert torch.allclose(O[..., 5], torch.full_like(O[..., 5], 0.75), atol=1e-15, rtol=0)
    O2, _ = oracle.attention(Q, K, 3.0 * V - 2.0, 0.125, True, 0)
    assert torch.allclose(O2, 3.0 * O - 2.0, atol=1e-13, rtol=0)
    ones, _ = oracle.attention(Q, K, torch.ones_like(V), 0.125, True, 0)   # softmax rows sum to one
    assert torch.allclose(ones, torch.ones_like(ones), atol=1e-15, rtol=0)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 9)])
def test_output_lies_in_convex_hull_of_visible_values(causal, window):
    N, D = 80, 64
    Q, K, V = rnd((1, 1, N, D), 81, 0) * 3, rnd((1, 1, N, D), 81, 1), rnd((1, 1, N, D), 81, 2)
    O, _ = oracle.attention(Q, K, V, 0.125, causal, window)
    for i in range(N):
        lo, hi = oracle.visible_keys(i, N, N, causal, window)
        vmin = V[0, 0, lo:hi].min(dim=0).values
        vmax = V[0, 0, lo:hi].max(dim=0).values
        assert torch.all(O[0, 0, i] >= vmin - 1e-12) and torch.all(O[0, 0, i] <= vmax + 1e-12)


def test_empty_rows_when_queries_outnumber_keys():
    Nq, Nk, D = 10, 4, 64
    Q, K, V = rnd((1, 1, Nq, D), 91, 0), rnd((1, 1, Nk, D), 91, 1), rnd((1, 1, Nk, D), 91, 2)
    O, L = oracle.attention(Q, K, V, 0.125, True, 0)
    # bottom-right alignment: row i sees keys j <= i - 6, so rows 0..5 see nothing
    assert torch.all(O[0, 0, :6] == 0) and torch.all(L[0, 0, :6] == -math.inf)
    assert torch.equal(O[0, 0, 6], V[0, 0, 0])
    assert torch.all(torch.isfinite(L[0, 0, 6:]))


def test_wide_window_equals_plain_causal_and_keys_permute():
    N, D = 64, 64
    Q, K, V = rnd((1, 2, N, D), 101, 0), rnd((1, 2, N, D), 101, 1), rnd((1, 2, N, D), 101, 2)
    Oc, Lc = oracle.attention(Q, K, V, 0.125, True, 0)
    Ow, Lw = oracle.attention(Q, K, V, 0.125, True, N)
    assert torch.equal(Oc, Ow) and torch.equal(Lc, Lw)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(5))
    O1, L1 = oracle.attention(Q, K, V, 0.125, False, 0)
    O2, L2 = oracle.attention(Q, K[:, :, perm], V[:, :, perm], 0.125, False, 0)
    assert torch.allclose(O1, O2, atol=1e-14, rtol=0) and torch.allclose(L1, L2, atol=1e-14, rtol=0)


def test_sampled_rows_match_full_run():
    B, H, N, D = 2, 3, 100, 64
    Q, K, V = rnd((B, H, N, D), 111, 0), rnd((B, H, N, D), 111, 1), rnd((B, H, N, D), 111, 2)
    O, L = oracle.attention(Q, K, V, 0.125, True, 30)
    rows = [0, 5, 99, 100, 250, 599, 301]
    Os, Ls = oracle.attention(Q, K, V, 0.125, True, 30, rows=rows)
    assert torch.equal(Os, O.reshape(-1, D)[rows]) and torch.equal(Ls, L.reshape(-1)[rows])


# ----------------------------------------------------- storage-format decode

def e4m3fn_value(code: int) -> float:
    """OCP 8-bit E4M3 ('FN' variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    S.1111.111 is NaN, there is no infinity, exponent 0 encodes subnormals."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_e4m3_decode_matches_the_format_definition():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    dec = oracle.decode(codes)
    for c in range(256):
        ref = e4m3fn_value(c)
        got = dec[c].item()
        assert (math.isnan(ref) and math.isnan(got)) or got == ref, (c, ref, got)
    assert max(e4m3fn_value(c) for c in range(256) if not math.isnan(e4m3fn_value(c))) == synth.E4M3_MAX


def test_e4m3_quantizer_rounds_to_nearest_even_with_saturation():
    finite = sorted({e4m3fn_value(c) for c in range(256) if not math.isnan(e4m3fn_value(c))})
    x = torch.cat([synth.normal(7, 0, 4000) * 3, torch.tensor([1000.0, -1000.0, 448.0, 0.0])])
    codes, ds = synth.quantize_e4m3(x)
    assert ds == float(torch.tensor(1000.0 / 448.0, dtype=torch.float32))
    y = (x.to(torch.float32) / torch.tensor(ds, dtype=torch.float32)).to(torch.float64)
    got = oracle.decode(codes)
    for yi, gi in zip(y.tolist(), got.tolist()):
        yc = max(-448.0, min(448.0, yi))
        best = min(finite, key=lambda f: (abs(f - yc), 0))
        ties = [f for f in finite if abs(f - yc) == abs(best - yc)]
        if len(ties) > 1:   # round half to even mantissa bit
            best = [f for f in ties if (int(torch.tensor(f, dtype=torch.float8_e4m3fn).view(torch.uint8)) & 1) == 0][0]
        assert gi == best, (yi, gi, best)


# ---------------------------------------------------- the pages' figures

def test_worked_example_figures_from_the_pages():
    g = json.load(open(os.path.join(HERE, "golden", "pages_worked_example.json")))
    B, h, n, d = g["B"], g["h"], g["n"], g["d_k"]
    assert 2 * B * h * n * n == g["weights_bytes_fp16"]
    assert round(g["weights_bytes_fp16"] / 1e9, 2) == g["weights_gb_fp16_printed"]
    assert round(g["layers_example"] * g["weights_bytes_fp16"] / 1e9) == g["weights_gb_fp16_32_layers_printed"]
    assert g["weights_bytes_fp16"] * g["layers_example"] / 1e9 > g["gpu_memory_gb_printed"]
    assert 2 * B * h * n * n * d == g["product_flops"]
    # the oracle's visible-key count agrees with the closed forms of the two mask shapes
    assert oracle.pair_count(n, n, False, 0) == n * n
    assert oracle.pair_count(n, n, True, 0) == n * (n + 1) // 2


# --------------------------------------------------------- planted mistakes

MUTANTS = {
    "dropped_scale": ("s[j - lo] = jb->scale * dot;", "s[j - lo] = dot;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "causal_off_by_one": ("hi = ip + 1 < Nk ? ip + 1 : Nk;", "hi = ip < Nk ? ip : Nk;"),
    "window_off_by_one": ("lo = ip - jb->window + 1 > 0 ? ip - jb->window + 1 : 0;", "lo = ip - jb->window > 0 ? ip - jb->window : 0;"),
    "top_left_alignment": ("const long ip = i + (Nk - Nq);", "const long ip = i;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "lse_base_two": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "not_normalised": ("s[j] = s[j] / l;", "s[j] = s[j];"),
    "value_for_key": ("const double *kj = K + j * D;", "const double *kj = V + j * D;"),
    "value_index_transposed": ("const double *vj = V + j * D;", "const double *vj = V + (j % D) * D;"),
    "dot_drops_last_dim": ("for (long d = 0; d < D; ++d) dot += qi[d] * kj[d];",
                           "for (long d = 0; d < D - 1; ++d) dot += qi[d] * kj[d];"),
    "sum_drops_first_key": ("l += s[j];", "if (j > 0) l += s[j];"),
    "output_drops_last_key": ("for (long j = lo; j < hi; ++j) {\n        const double p", "for (long j = lo; j < hi - 1; ++j) {\n        const double p"),
    "extent_left_off_by_one": ("if (jb->wl >= 0) lo = ip - jb->wl > 0 ? ip - jb->wl : 0;",
                               "if (jb->wl >= 0) lo = ip - jb->wl + 1 > 0 ? ip - jb->wl + 1 : 0;"),
    "extent_right_off_by_one": ("if (jb->wr >= 0) hi = ip + jb->wr + 1 < Nk ? ip + jb->wr + 1 : Nk;",
                                "if (jb->wr >= 0) hi = ip + jb->wr < Nk ? ip + jb->wr : Nk;"),
    "extents_swapped": ("if (jb->wl >= 0) lo = ip - jb->wl > 0 ? ip - jb->wl : 0;",
                        "if (jb->wr >= 0) lo = ip - jb->wr > 0 ? ip - jb->wr : 0;"),
    "alibi_sign": ("s[j - lo] += slope * (double)(j - ip);", "s[j - lo] += slope * (double)(ip - j);"),
    "alibi_top_left": ("s[j - lo] += slope * (double)(j - ip);", "s[j - lo] += slope * (double)(j - i);"),
    "alibi_wrong_head": ("const double slope = jb->slopes[bh % jb->H];",
                         "const double slope = jb->slopes[(bh + 1) % jb->H];"),
    "softcap_no_outer": ("s[j - lo] = jb->cap * tanh(s[j - lo] / jb->cap);", "s[j - lo] = tanh(s[j - lo] / jb->cap);"),
    "softcap_no_inner": ("s[j - lo] = jb->cap * tanh(s[j - lo] / jb->cap);", "s[j - lo] = jb->cap * tanh(s[j - lo]);"),
    "bwd_ds_sign": ("const double dsm = s[j - lo] * (dp[j - lo] - dv_row);",
                    "const double dsm = s[j - lo] * (dv_row - dp[j - lo]);"),
    "bwd_softcap_no_chain": ("g[j - lo] = 1.0 - t * t;", "g[j - lo] = 1.0;"),
    "bwd_softcap_chain_sign": ("g[j - lo] = 1.0 - t * t;", "g[j - lo] = 1.0 + t * t;"),
    "bwd_softcap_no_outer": ("s[j - lo] = jb->cap * t;", "s[j - lo] = t;"),
    "bwd_alibi_dropped": ("s[j - lo] += jb->slopes[bh % jb->H] * (double)(j - ip);", "s[j - lo] += 0.0;"),
    "bwd_alibi_sign": ("s[j - lo] += jb->slopes[bh % jb->H] * (double)(j - ip);",
                       "s[j - lo] += jb->slopes[bh % jb->H] * (double)(ip - j);"),
    "bwd_dq_no_scale": ("dQ[i * D + d] += jb->scale * ds * K[j * D + d];", "dQ[i * D + d] += ds * K[j * D + d];"),
    "bwd_dk_uses_k": ("dK[j * D + d] += jb->scale * ds * qi[d];", "dK[j * D + d] += jb->scale * ds * K[j * D + d];"),
    "bwd_dv_no_weight": ("for (long d = 0; d < D; ++d) dV[j * D + d] += p * doi[d];",
                         "for (long d = 0; d < D; ++d) dV[j * D + d] += doi[d];"),
    "bwd_rowsum_unweighted": ("dv_row += p * x;", "dv_row += x;"),
}


def pin_suite(lib) -> bool:
    """A compact run of the pins above against a given oracle build; True if all hold."""
    try:
        # brute force at 50 digits, causal window with unequal lengths
        Q, K, V = rnd((1, 1, 4, 3), 13, 0), rnd((1, 1, 6, 3), 13, 1), rnd((1, 1, 6, 3), 13, 2)
        for causal, window in [(False, 0), (True, 0), (True, 3)]:
            O, L = oracle.attention(Q, K, V, 0.7, causal, window, lib=lib, threads=1)
            Om, Lm = mp_attention(Q[0, 0], K[0, 0], V[0, 0], float(torch.tensor(0.7, dtype=torch.float32)),
                                  mask_matrix(4, 6, causal, window))
            for i in range(4):
                if abs(L[0, 0, i].item() - float(Lm[i])) > 1e-12:
                    return False
                for d in range(3):
                    if abs(O[0, 0, i, d].item() - float(Om[i][d])) > 1e-12:
                        return False
        # closed forms
        N, D = 20, 64
        Qz = torch.zeros(1, 1, N, D, dtype=torch.float64)
        K2, V2 = rnd((1, 1, N, D), 14, 1), rnd((1, 1, N, D), 14, 2)
        O, L = oracle.attention(Qz, K2, V2, 0.125, True, 0, lib=lib, threads=1)
        for i in range(N):
            if abs(L[0, 0, i].item() - math.log(i + 1)) > 1e-13:
                return False
            if not torch.allclose(O[0, 0, i], V2[0, 0, : i + 1].mean(0), atol=1e-13):
                return False
        Q2 = rnd((1, 1, N, D), 14, 0)
        O, L = oracle.attention(Q2, K2, V2, 0.125, True, 1, lib=lib, threads=1)
        if not torch.equal(O, V2):
            return False
        # the extents mask at 50 digits, both sides bounded and unequal
        for wl, wr in [(1, 2), (2, 0)]:
            O, L = oracle.attention(Q, K, V, 0.7, lib=lib, threads=1, window_left=wl, window_right=wr)
            Om, Lm = mp_attention(Q[0, 0], K[0, 0], V[0, 0], float(torch.tensor(0.7, dtype=torch.float32)),
                                  mask_matrix_window(4, 6, wl, wr))
            for i in range(4):
                if Lm[i] == -mpmath.inf:
                    if L[0, 0, i].item() != -math.inf:
                        return False
                    continue
                if abs(L[0, 0, i].item() - float(Lm[i])) > 1e-12:
                    return False
        # ALiBi against torch's SDPA with the bias as an additive mask (two heads, Nq != Nk)
        Qa, Ka, Va = rnd((1, 2, 5, 8), 15, 0), rnd((1, 2, 9, 8), 15, 1), rnd((1, 2, 9, 8), 15, 2)
        slopes = [0.7, 0.2]
        O, L = oracle.attention(Qa, Ka, Va, 0.5, True, 0, score_mod="alibi", alibi_slopes=slopes, lib=lib, threads=1)
        keep = mask_matrix(5, 9, True, 0)
        bias = alibi_bias(5, 9, slopes).masked_fill(~keep, -math.inf).unsqueeze(0)
        Oref = torch.nn.functional.scaled_dot_product_attention(Qa, Ka, Va, attn_mask=bias, scale=0.5)
        Lref = torch.logsumexp(torch.matmul(Qa, Ka.transpose(-1, -2)) * 0.5 + bias, dim=-1)
        if not torch.allclose(O, Oref, atol=1e-12) or not torch.allclose(L, Lref, atol=1e-12):
            return False
        # softcap at 50 digits
        O, L = oracle.attention(Q, K, V, 0.7, True, 0, score_mod="softcap", softcap=0.9, lib=lib, threads=1)
        mpmath.mp.dps = 50
        sc, cp = mpmath.mpf(float(torch.tensor(0.7, dtype=torch.float32))), mpmath.mpf(0.9)
        for i in range(4):
            js = [j for j in range(6) if mask_matrix(4, 6, True, 0)[i, j]]
            sv = [cp * mpmath.tanh(sc * mpmath.fsum(mpmath.mpf(float(Q[0, 0, i, d])) * mpmath.mpf(float(K[0, 0, j, d]))
                                                     for d in range(3)) / cp) for j in js]
            if abs(L[0, 0, i].item() - float(mpmath.log(mpmath.fsum(mpmath.exp(x) for x in sv)))) > 1e-12:
                return False
        # the backward against central differences of the (possibly mutated) oracle forward
        Qb, Kb, Vb, dOb = rnd((1, 1, 5, 4), 16, 0), rnd((1, 1, 6, 4), 16, 1), rnd((1, 1, 6, 4), 16, 2), \
            rnd((1, 1, 5, 4), 16, 3)
        dQ, dK, dV = oracle.attention_bwd(Qb, Kb, Vb, dOb, 0.7, -1, 0, lib=lib, threads=1)
        for X, G, tid in [(Qb, dQ, 4), (Kb, dK, 5), (Vb, dV, 6)]:
            E = rnd(X.shape, 17, tid)
            X0 = X.clone()
            vals = []
            for sgn in (1, -1):
                X.copy_(X0 + sgn * 1e-5 * E)
                O, _ = oracle.attention(Qb, Kb, Vb, 0.7, window_left=-1, window_right=0, lib=lib, threads=1)
                vals.append(float((O * dOb).sum()))
            X.copy_(X0)
            if abs((vals[0] - vals[1]) / 2e-5 - float((G * E).sum())) > 1e-6:
                return False
        # the backward with each score modifier against central differences of the modified forward
        for mod in (dict(score_mod="softcap", softcap=0.9), dict(score_mod="alibi", alibi_slopes=[0.7])):
            dQ, dK, dV = oracle.attention_bwd(Qb, Kb, Vb, dOb, 0.7, -1, 0, lib=lib, threads=1, **mod)
            for X, G, tid in [(Qb, dQ, 4), (Kb, dK, 5), (Vb, dV, 6)]:
                E = rnd(X.shape, 18, tid)
                X0 = X.clone()
                vals = []
                for sgn in (1, -1):
                    X.copy_(X0 + sgn * 1e-5 * E)
                    O, _ = oracle.attention(Qb, Kb, Vb, 0.7, window_left=-1, window_right=0, lib=lib, threads=1,
                                            **mod)
                    vals.append(float((O * dOb).sum()))
                X.copy_(X0)
                if abs((vals[0] - vals[1]) / 2e-5 - float((G * E).sum())) > 1e-6:
                    return False
        return True
    except RuntimeError:
        return False


def test_planted_mistakes_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    tmp = tempfile.mkdtemp()
    try:
        good = os.path.join(tmp, "good.so")
        shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "oracle.c"), os.path.join(tmp, "good.c"))
        oracle.build(good, os.path.join(tmp, "good.c"))
        assert pin_suite(oracle.load(good)), "the unmodified oracle must pass the pin suite"
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, name
            path_c = os.path.join(tmp, name + ".c")
            open(path_c, "w").write(src.replace(old, new))
            so = oracle.build(os.path.join(tmp, name + ".so"), path_c)
            assert not pin_suite(oracle.load(so)), f"mutant {name} passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
