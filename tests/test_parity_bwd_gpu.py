"""Parity of the HIP backward (fa_bwd, through the C ABI) with the float64
CPU oracle's dQ, dK, dV.

Bound, derived from the kernel's arithmetic (u = 2^-8 for bfloat16, 2^-11 for
float16, the unit roundoff of the input type). Every product in the kernel is
formed by MFMA from stored 16-bit values and summed in fp32; the roundings
that matter are:
  * P rounded to the input type for dV = P^T dO (relative u per weight);
  * dS rounded to the input type for dQ = scale dS K and dK = scale dS^T Q
    (relative u per entry);
  * D_i = dO_i . O_i formed from the forward's stored O, whose error per
    element is at most about u (P|V|)_id + u |O_id| (the forward rounds P and
    O), so |dD_i| <= u A_i with A_i = sum_d |dO_id| ((P|V|)_id + |O_id|); it
    enters dS as P_ij dD_i;
  * the outputs rounded to the input type (relative u).
Below the smallest normal number a rounding is off by up to eta absolute
instead (half the smallest subnormal: 2^-25 for float16; negligible for
bfloat16, whose range is float32's); small weights and dS entries reach it
under steep ALiBi biases. With V_ij = 1 for a visible pair, to first order,
elementwise,
  |dV - dV_ref| <= u (P^T|dO|) + eta (V^T|dO|) + u |dV_ref| + eta
  |dQ - dQ_ref| <= u scale (|dS||K| + A o (P|K|)) + eta scale (V|K|) + u |dQ_ref| + eta
  |dK - dK_ref| <= u scale (|dS|^T|Q| + (P o A)^T |Q|) + eta scale (V^T|Q|) + u |dK_ref| + eta
fp32 accumulation and the fp32 exponential add terms below 1e-5 of these.
The test allows twice the first-order bound plus 1e-6. The magnitude arrays
P, dS, A are evaluated here in float64 from the inputs; they set the
tolerance only, the expected values are the oracle's.

With a score modifier f (softcap, ALiBi) P is the softmax of f(scale S) and
dS carries g = f'(scale S): the same bound holds with |dS| the modified
gradient and P o g in place of P in the stored-O term. The fp32 tanh and bias
add exponent errors below 1e-5 relative to the weights at the caps and slopes
tested, well inside u.

Rows that see no key must give dQ = 0 exactly; keys that no row sees must give
dK = dV = 0 exactly.
"""
import math

import pytest
import torch

import exact_attention_02_amd as fa
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
ETA = {"bf16": 0.0, "f16": 2.0 ** -25}


def visible(Nq, Nk, wl, wr):
    i = torch.arange(Nq)[:, None] + (Nk - Nq)
    j = torch.arange(Nk)[None, :]
    vis = torch.ones(Nq, Nk, dtype=torch.bool)
    if wl >= 0:
        vis &= j >= i - wl
    if wr >= 0:
        vis &= j <= i + wr
    return vis


def head_tolerance(Q, K, V, O, dO, dQr, dKr, dVr, scale, wl, wr, u, mod=None, cap=0.0, slope=0.0, eta=0.0):
    """Elementwise allowed |error| of dQ, dK, dV for one head (float64 2-D inputs)."""
    Nq, Nk = Q.shape[0], K.shape[0]
    vis = visible(Nq, Nk, wl, wr)
    S = (Q @ K.T) * scale
    g = torch.ones_like(S)
    if mod == "softcap":
        t = torch.tanh(S / cap)
        S, g = cap * t, 1.0 - t * t
    elif mod == "alibi":
        i = torch.arange(Nq, dtype=torch.float64)[:, None] + (Nk - Nq)
        j = torch.arange(Nk, dtype=torch.float64)[None, :]
        S = S + slope * (j - i)
    S = S.masked_fill(~vis, -math.inf)
    m = S.max(dim=1, keepdim=True).values
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    E = torch.exp(S - m)
    del S
    P = E / E.sum(dim=1, keepdim=True).clamp_min(1e-300)
    del E
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(dim=1, keepdim=True)) * g
    del dP
    A = (dO.abs() * (P @ V.abs() + O.abs())).sum(dim=1)
    bV = P.T @ dO.abs()
    Pg = P * g
    bQ = scale * (dS.abs() @ K.abs() + A[:, None] * (Pg @ K.abs()))
    bK = scale * (dS.abs().T @ Q.abs() + (Pg * A[:, None]).T @ Q.abs())
    Vm = vis.to(torch.float64)
    fQ = scale * (Vm @ K.abs()) + 1.0
    fK = scale * (Vm.T @ Q.abs()) + 1.0
    fV = Vm.T @ dO.abs() + 1.0
    return [2.0 * (u * (b + r.abs()) + eta * f) + 1e-6
            for b, r, f in ((bQ, dQr, fQ), (bK, dKr, fK), (bV, dVr, fV))]


def mod_args(w):
    """The score modifier of a workload as attention() / attention_bwd() keyword arguments."""
    if w.score_mod is None:
        return {}
    m = dict(score_mod=w.score_mod, softcap=w.softcap)
    if w.score_mod == "alibi":
        m["alibi"] = torch.tensor(synth.alibi_slopes(w.H), dtype=torch.float32, device=DEV)
    return m


def run(w, wl, wr, q, k, v, do):
    """Forward (for O and LSE) then backward on the GPU; returns host tensors."""
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    o, lse = fa.attention(qd, kd, vd, scale=w.scale, window_left=wl, window_right=wr, **mod_args(w))
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale=w.scale, window_left=wl, window_right=wr,
                                  **mod_args(w))
    torch.cuda.synchronize()
    return o.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def check(w, wl, wr, q, k, v, do, o, dq, dk, dv, heads=None, ref=None):
    """Compare (b, h) heads (default all) with the oracle under the derived bound."""
    u = UNIT[w.in_dtype]
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    worst = 0.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        om = {}
        if w.score_mod is not None:
            om = dict(score_mod=w.score_mod, softcap=w.softcap,
                      alibi_slopes=[synth.alibi_slopes(w.H)[h]] if w.score_mod == "alibi" else None)
        if ref is None:
            dQr, dKr, dVr = oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], w.scale, wl, wr, **om)
        else:
            dQr, dKr, dVr = (t[sl] for t in ref)
        dQr, dKr, dVr = dQr[0, 0], dKr[0, 0], dVr[0, 0]
        Q, K, V, dO = (oracle.decode(t[b, h]) for t in (q, k, v, do))
        s32 = float(torch.tensor(w.scale, dtype=torch.float32))
        slope = synth.alibi_slopes(w.H)[h] if w.score_mod == "alibi" else 0.0
        tq, tk, tv = head_tolerance(Q, K, V, oracle.decode(o[b, h]), dO, dQr, dKr, dVr, s32, wl, wr, u,
                                    mod=w.score_mod, cap=w.softcap, slope=slope, eta=ETA[w.in_dtype])
        for name, got, exp, tol in (("dQ", dq[b, h], dQr, tq), ("dK", dk[b, h], dKr, tk),
                                    ("dV", dv[b, h], dVr, tv)):
            err = (got.double() - exp).abs()
            ratio = (err / tol).max().item() if err.numel() else 0.0
            worst = max(worst, ratio)
            assert torch.isfinite(got.double()).all(), f"{w.name} {name} ({b},{h}) not finite"
            assert ratio <= 1.0, (f"{w.name} {name} head ({b},{h}): max err/tol {ratio:.3f}, "
                                  f"max err {err.max().item():.3e}")
        # exact zeros: rows that see no key, keys that no row sees
        vis = visible(w.Nq, w.Nk, wl, wr)
        empty_rows = ~vis.any(dim=1)
        unseen = ~vis.any(dim=0)
        assert (dq[b, h][empty_rows] == 0).all(), f"{w.name}: dQ of a row that sees no key"
        assert (dk[b, h][unseen] == 0).all() and (dv[b, h][unseen] == 0).all(), \
            f"{w.name}: dK/dV of a key that no row sees"
    print(f"{w.name}: worst error / tolerance {worst:.3f}", flush=True)
    return worst


# (name, B, H, Nq, Nk, D, window_left, window_right, dtype): several 128-row
# blocks and 64-row tiles with ragged tails, every mask family, both dtypes,
# both head dims, and the degenerate shapes.
CASES = [
    ("causal_sq", 1, 2, 300, 300, 64, -1, 0, "bf16"),
    ("causal_sq_f16", 1, 2, 300, 300, 64, -1, 0, "f16"),
    ("full_d128", 1, 2, 300, 300, 128, -1, -1, "bf16"),
    ("causal_d128_f16", 2, 1, 257, 257, 128, -1, 0, "f16"),
    ("causal_nq_lt_nk", 2, 1, 200, 333, 64, -1, 0, "bf16"),
    ("causal_nq_gt_nk", 1, 1, 333, 200, 64, -1, 0, "bf16"),       # 133 rows see no key
    ("window_sym_f16", 1, 2, 400, 400, 64, 50, 50, "f16"),
    ("window_causal_d128", 1, 2, 400, 400, 128, 63, 0, "bf16"),
    ("diagonal", 1, 1, 130, 130, 64, 0, 0, "bf16"),
    ("left_only_f16", 1, 1, 300, 280, 64, 10, -1, "f16"),
    ("unseen_keys", 1, 2, 100, 400, 64, 10, 0, "bf16"),          # keys below 290 are seen by no row
    ("one_row", 1, 3, 1, 1000, 64, -1, 0, "bf16"),
    ("one_key", 1, 2, 150, 1, 64, -1, -1, "bf16"),
    ("one_by_one_f16", 1, 1, 1, 1, 64, -1, -1, "f16"),
    ("ragged_batch", 3, 2, 129, 65, 64, -1, -1, "bf16"),
    ("causal_1k", 1, 2, 1100, 1100, 64, -1, 0, "bf16"),
    ("causal_1k_d128_f16", 1, 1, 1100, 1100, 128, -1, 0, "f16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    name, B, H, Nq, Nk, D, wl, wr, dt = case
    w = synth.small_workload("bwd_" + name, B, H, Nq, Nk, D, False, 0, dt, dt, 31 + len(name), backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    print(f"case {name} B{B} H{H} Nq{Nq} Nk{Nk} D{D} wl{wl} wr{wr} {dt}", flush=True)
    o, dq, dk, dv = run(w, wl, wr, inp.q, inp.k, inp.v, do)
    ref = oracle.attention_bwd(inp.q, inp.k, inp.v, do, w.scale, wl, wr)
    check(w, wl, wr, inp.q, inp.k, inp.v, do, o, dq, dk, dv, ref=ref)


@pytest.mark.parametrize("Nq,Nk", [(0, 70), (70, 0)])
def test_bwd_empty_sides(Nq, Nk):
    """No rows: dK = dV = 0 (nothing flows back). No keys: dQ = 0."""
    w = synth.small_workload("bwd_empty", 1, 2, Nq, Nk, 64, False, 0, "bf16", "bf16", 5, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    q, k, v, dod = (t.to(DEV) for t in (inp.q, inp.k, inp.v, do))
    o = torch.zeros_like(q)
    lse = torch.full((1, 2, Nq), -math.inf, device=DEV)
    dq = torch.full_like(q, 7.0)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    fa.attention_bwd(q, k, v, o, lse, dod, scale=w.scale, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_bwd_workspace_contents_do_not_matter_and_calls_repeat_bitwise():
    """The workspace is fully written before it is read (padding rows included),
    and the kernels use no atomics: a NaN-filled workspace gives the same bits."""
    w = synth.small_workload("bwd_ws", 2, 3, 203, 190, 64, False, 0, "bf16", "bf16", 9, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    q, k, v, dod = (t.to(DEV) for t in (inp.q, inp.k, inp.v, do))
    o, lse = fa.attention(q, k, v, scale=w.scale, causal=True)
    need = fa.bwd_workspace_bytes(w.B, w.H, w.Nq)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    a = fa.attention_bwd(q, k, v, o, lse, dod, scale=w.scale, causal=True, workspace=ws)
    b = fa.attention_bwd(q, k, v, o, lse, dod, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        assert torch.isfinite(x.float()).all()


def test_bwd_full_size_sampled_heads():
    """The backward workload at full size (causal B4 H12 N8192 D64 bf16) in the
    launch configuration the benchmark times; two heads compared in full."""
    w = synth.WORKLOADS["c3bwd"]
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    wl, wr = -1, 0
    print(f"full size {w.name}", flush=True)
    o, dq, dk, dv = run(w, wl, wr, inp.q, inp.k, inp.v, do)
    check(w, wl, wr, inp.q, inp.k, inp.v, do, o, dq, dk, dv, heads=[(0, 0), (w.B - 1, w.H - 1)])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_bwd_masked_positions_are_exact(dt):
    """Masked pairs contribute exactly nothing: under a causal mask, scaling the
    K and V rows that rows 0..150 cannot see leaves their dQ bitwise unchanged,
    and scaling the Q and dO rows 0..99 (which cannot see keys 100..) leaves dK
    and dV of those keys bitwise unchanged."""
    w = synth.small_workload("bwd_maskexact", 1, 2, 300, 300, 64, True, 0, dt, dt, 12, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)

    def grads(q, k, v, dout):
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
        o, lse = fa.attention(qd, kd, vd, scale=w.scale, causal=True)
        g = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale=w.scale, causal=True)
        torch.cuda.synchronize()
        return [t.cpu() for t in g]

    base = grads(inp.q, inp.k, inp.v, do)
    k2, v2 = inp.k.clone(), inp.v.clone()
    k2[:, :, 151:] = (k2[:, :, 151:].float() * 100).to(k2.dtype)
    v2[:, :, 151:] = (v2[:, :, 151:].float() * 100).to(v2.dtype)
    pk = grads(inp.q, k2, v2, do)
    assert torch.equal(base[0][:, :, :151].view(torch.int16), pk[0][:, :, :151].view(torch.int16))
    q2, do2 = inp.q.clone(), do.clone()
    q2[:, :, :100] = (q2[:, :, :100].float() * 100).to(q2.dtype)
    do2[:, :, :100] = (do2[:, :, :100].float() * 100).to(do2.dtype)
    pq = grads(q2, inp.k, inp.v, do2)
    for a, b in ((base[1], pq[1]), (base[2], pq[2])):
        assert torch.equal(a[:, :, 100:].view(torch.int16), b[:, :, 100:].view(torch.int16))


# (name, B, H, Nq, Nk, D, window_left, window_right, dtype, modifier, cap)
MOD_CASES = [
    ("softcap50_causal", 1, 2, 300, 300, 64, -1, 0, "bf16", "softcap", 50.0),
    # cap 20: lanes inside and outside the range of the kernels' polynomial for tanh
    ("softcap20_causal", 1, 2, 300, 300, 64, -1, 0, "bf16", "softcap", 20.0),
    ("softcap20_window_f16_d128", 1, 2, 260, 300, 128, 70, 30, "f16", "softcap", 20.0),
    ("softcap2_full_f16", 1, 2, 257, 300, 64, -1, -1, "f16", "softcap", 2.0),
    ("softcap0.5_window_d128", 1, 2, 300, 300, 128, 40, 40, "bf16", "softcap", 0.5),
    ("softcap3_nq_gt_nk_f16", 1, 1, 333, 200, 64, -1, 0, "f16", "softcap", 3.0),
    ("alibi_causal", 1, 3, 300, 300, 64, -1, 0, "bf16", "alibi", 0.0),
    ("alibi_full_f16_d128", 1, 2, 200, 333, 128, -1, -1, "f16", "alibi", 0.0),
    ("alibi_window", 2, 2, 129, 400, 64, 50, 0, "bf16", "alibi", 0.0),
    ("alibi_1k_f16", 1, 2, 1100, 1100, 64, -1, 0, "f16", "alibi", 0.0),
]


@pytest.mark.parametrize("case", MOD_CASES, ids=[c[0] for c in MOD_CASES])
def test_bwd_mod_parity(case):
    name, B, H, Nq, Nk, D, wl, wr, dt, mod, cap = case
    w = synth.small_workload("bwd_" + name, B, H, Nq, Nk, D, False, 0, dt, dt, 51 + len(name), score_mod=mod,
                             softcap=cap, backward=True)
    inp = synth.make_inputs(w)
    if mod == "softcap" and cap == 20.0:
        # about 5% of the scaled scores past 20 * 0.2: roughly half the lanes'
        # blocks leave the range of the kernels' polynomial for tanh
        inp = synth.Inputs((inp.q.double() * 2.0).to(inp.q.dtype), inp.k, inp.v)
    do = synth.make_grad_out(w)
    print(f"case {name} B{B} H{H} Nq{Nq} Nk{Nk} D{D} wl{wl} wr{wr} {dt} {mod} {cap}", flush=True)
    o, dq, dk, dv = run(w, wl, wr, inp.q, inp.k, inp.v, do)
    check(w, wl, wr, inp.q, inp.k, inp.v, do, o, dq, dk, dv)


def test_bwd_alibi_with_zero_slopes_is_bitwise_plain():
    w = synth.small_workload("bwd_alibi0", 1, 2, 300, 300, 64, True, 0, "bf16", "bf16", 13, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    q, k, v, dod = (t.to(DEV) for t in (inp.q, inp.k, inp.v, do))
    o, lse = fa.attention(q, k, v, scale=w.scale, causal=True)
    plain = fa.attention_bwd(q, k, v, o, lse, dod, scale=w.scale, causal=True)
    zero = torch.zeros(2, dtype=torch.float32, device=DEV)
    mod = fa.attention_bwd(q, k, v, o, lse, dod, scale=w.scale, causal=True, score_mod="alibi", alibi=zero)
    torch.cuda.synchronize()
    for a, b in zip(plain, mod):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["c3sc", "c3al"])
def test_bwd_mod_full_size_sampled_heads(name):
    """The c3 softcap and ALiBi workloads' backward at full size, two heads compared in full
    (ALiBi: the steepest and the shallowest slope)."""
    base = synth.WORKLOADS[name]
    w = synth.Workload(base.name + "_backward", base.B, base.H, base.Nq, base.Nk, base.D, True, 0, base.in_dtype,
                       base.out_dtype, base.seed, score_mod=base.score_mod, softcap=base.softcap, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w)
    print(f"full size {w.name}", flush=True)
    o, dq, dk, dv = run(w, -1, 0, inp.q, inp.k, inp.v, do)
    check(w, -1, 0, inp.q, inp.k, inp.v, do, o, dq, dk, dv, heads=[(0, 0), (w.B - 1, w.H - 1)])


@pytest.mark.parametrize("mod", [None, "softcap", "alibi"])
def test_flash_attention_autograd_matches_the_c_calls(mod):
    """flash_attention's autograd backward is fa_bwd / fa_bwd_mod on the saved O and LSE, bit for bit."""
    w = synth.small_workload("autograd", 1, 2, 200, 200, 64, True, 0, "bf16", "bf16", 14, score_mod=mod,
                             softcap=5.0 if mod == "softcap" else 0.0, backward=True)
    inp = synth.make_inputs(w)
    do = synth.make_grad_out(w).to(DEV)
    q, k, v = (t.to(DEV).requires_grad_(True) for t in (inp.q, inp.k, inp.v))
    m = mod_args(w)
    o = fa.flash_attention(q, k, v, scale=w.scale, causal=True, **m)
    o.backward(do)
    with torch.no_grad():
        o2, lse = fa.attention(q.detach(), k.detach(), v.detach(), scale=w.scale, window_left=-1, window_right=0, **m)
        ref = fa.attention_bwd(q.detach(), k.detach(), v.detach(), o2, lse, do, scale=w.scale, causal=True, **m)
    torch.cuda.synchronize()
    assert torch.equal(o.detach().view(torch.int16), o2.view(torch.int16))
    for g, r in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(g.view(torch.int16), r.view(torch.int16))
