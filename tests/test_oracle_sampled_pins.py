"""Pins of the oracle's sampled-row path and its e4m3 decode.

Full-size parity compares the kernels with `oracle.attention(rows=...)`, which
decodes one (batch, head) slice at a time, hands the C oracle that head's own
ALiBi slope and the e4m3 descales, and computes the listed rows only. Every
row of the plain definition (aiinarabic.com flash-attention page, eq. (1)) is
independent of the others, so those rows must be bit for bit the rows of one
call over the whole tensor, under every mask and score modifier. The e4m3
decode is pinned to the format's definition times the fp32 descale in exact
rational arithmetic, and the whole e4m3 path to torch's float64 SDPA on
inputs dequantised independently here. The last test plants plausible
mistakes into copies of the oracle's Python layer and checks that these pins
catch each one.
"""
import math
import os
import types
from fractions import Fraction

import pytest
import torch

import oracle
import synth

ORACLE_PY = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")


def rnd(shape, seed, tid=0):
    n = 1
    for s in shape:
        n *= s
    return synth.normal(seed, tid, n).reshape(shape).to(torch.float64)


def rows_across_heads(B, H, Nq):
    """Rows from every head: the first, last and a middle row of each, plus a few more."""
    rows = []
    for bh in range(B * H):
        base = bh * Nq
        rows += [base, base + Nq // 2, base + Nq - 1, base + (7 * bh + 3) % Nq]
    return sorted(set(rows))


def e4m3fn_fraction(code: int):
    """OCP E4M3FN value of a code as an exact Fraction (None for NaN)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return None
    if e == 0:
        return s * Fraction(m, 1 << 9)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def dequant_exact(codes: torch.Tensor, descale: float) -> torch.Tensor:
    """Independent dequantisation: the format's value times the fp32 descale, exactly, as float64."""
    d = Fraction(float(torch.tensor(descale, dtype=torch.float32)))
    table = [e4m3fn_fraction(c) for c in range(256)]
    flat = codes.view(torch.uint8).reshape(-1).tolist()
    out = [float(table[c] * d) if table[c] is not None else math.nan for c in flat]
    return torch.tensor(out, dtype=torch.float64).reshape(codes.shape)


def e4m3_inputs(B, H, Nq, Nk, D, seed):
    q, dq = synth.quantize_e4m3(synth.normal(seed, 0, B * H * Nq * D).reshape(B, H, Nq, D) * 3.0)
    k, dk = synth.quantize_e4m3(synth.normal(seed, 1, B * H * Nk * D).reshape(B, H, Nk, D) * 0.5)
    v, dv = synth.quantize_e4m3(synth.normal(seed, 2, B * H * Nk * D).reshape(B, H, Nk, D) * 7.0)
    return (q, k, v), (dq, dk, dv)


# ------------------------------------------- sampled rows against the full run

SAMPLED_CASES = {
    "extents": dict(window_left=5, window_right=17),
    "extents_open_left": dict(window_left=-1, window_right=3),
    "softcap": dict(causal=True, score_mod="softcap", softcap=2.5),
    "softcap_extents": dict(window_left=20, window_right=0, score_mod="softcap", softcap=0.7),
    "alibi": dict(causal=True, score_mod="alibi", alibi_slopes=[0.9, 0.25, 0.0625]),
    "alibi_extents": dict(window_left=11, window_right=6, score_mod="alibi", alibi_slopes=[0.5, 0.125, 0.03125]),
}


@pytest.mark.parametrize("case", list(SAMPLED_CASES))
def test_sampled_rows_are_the_full_run_bitwise(case, lib=None):
    B, H, Nq, Nk, D = 2, 3, 45, 60, 64
    Q, K, V = rnd((B, H, Nq, D), 201, 0), rnd((B, H, Nk, D), 201, 1), rnd((B, H, Nk, D), 201, 2)
    kw = dict(SAMPLED_CASES[case])
    causal = kw.pop("causal", False)
    O, L = oracle.attention(Q, K, V, 0.125, causal, 0, lib=lib, **kw)
    rows = rows_across_heads(B, H, Nq)
    Os, Ls = oracle.attention(Q, K, V, 0.125, causal, 0, rows=rows, lib=lib, **kw)
    assert torch.equal(Os, O.reshape(-1, D)[rows]) and torch.equal(Ls, L.reshape(-1)[rows])


def test_sampled_rows_e4m3_with_descales_are_the_full_run_bitwise(mod=oracle, lib=None):
    B, H, Nq, Nk, D = 2, 3, 40, 52, 128
    (q, k, v), ds = e4m3_inputs(B, H, Nq, Nk, D, 202)
    assert all(d != 1.0 for d in ds)
    O, L = mod.attention(q, k, v, 0.0884, True, 0, descales=ds, lib=lib)
    rows = rows_across_heads(B, H, Nq)
    Os, Ls = mod.attention(q, k, v, 0.0884, True, 0, descales=ds, rows=rows, lib=lib)
    assert torch.equal(Os, O.reshape(-1, D)[rows]) and torch.equal(Ls, L.reshape(-1)[rows])


# ----------------------------------------------------------- the e4m3 decode

@pytest.mark.parametrize("descale", [1.0, 0.0123, 3.7, 1000.0 / 448.0, 2.0 ** -9])
def test_decode_is_the_exact_rational_product(descale, mod=oracle):
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = mod.decode(codes, float(torch.tensor(descale, dtype=torch.float32)))
    ref = dequant_exact(codes, descale)
    nan = torch.isnan(ref)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], ref[~nan])


def test_e4m3_attention_matches_sdpa_on_independently_dequantised_inputs(mod=oracle, lib=None):
    B, H, Nq, Nk, D = 1, 2, 33, 47, 128
    (q, k, v), ds = e4m3_inputs(B, H, Nq, Nk, D, 203)
    O, L = mod.attention(q, k, v, 0.0884, True, 0, descales=ds, lib=lib)
    Qd, Kd, Vd = dequant_exact(q, ds[0]), dequant_exact(k, ds[1]), dequant_exact(v, ds[2])
    scale = float(torch.tensor(0.0884, dtype=torch.float32))
    i = torch.arange(Nq).unsqueeze(1) + (Nk - Nq)
    keep = torch.arange(Nk).unsqueeze(0) <= i
    Oref = torch.nn.functional.scaled_dot_product_attention(Qd, Kd, Vd, attn_mask=keep, scale=scale)
    Lref = torch.logsumexp((torch.matmul(Qd, Kd.transpose(-1, -2)) * scale).masked_fill(~keep, -math.inf), dim=-1)
    assert torch.allclose(O, Oref, atol=1e-12, rtol=0) and torch.allclose(L, Lref, atol=1e-12, rtol=0)


# --------------------------------------- planted mistakes in the Python layer

PY_MUTANTS = {
    "sampled_alibi_first_head_slope": ('cur["slopes"] = slopes_all[h:h + 1]', 'cur["slopes"] = slopes_all[0:1]'),
    "descale_applied_twice": ("y = y * float(descale)", "y = y * float(descale) * float(descale)"),
    "sampled_row_off_by_one": ("local = (rows[sel] % Nq).contiguous()", "local = ((rows[sel] + 1) % Nq).contiguous()"),
    "sampled_head_transposed": ("b, h = divmod(bh, H)", "h, b = divmod(bh, B)"),
    "fp32_scale_dropped": ("scale64 = float(torch.tensor(scale, dtype=torch.float32))\n    if rows is None:",
                           "scale64 = float(scale)\n    if rows is None:"),
}


def mutated_oracle(old, new):
    src = open(ORACLE_PY).read()
    assert src.count(old) == 1, old
    m = types.ModuleType("oracle_mutant")
    m.__file__ = ORACLE_PY
    exec(compile(src.replace(old, new), ORACLE_PY, "exec"), m.__dict__)
    return m


def py_pin_suite(mod) -> bool:
    """The pins above, run against a (possibly mutated) copy of the Python layer; True if all hold."""
    lib = oracle.load()
    saved = oracle.attention, oracle.decode
    try:
        oracle.attention, oracle.decode = mod.attention, mod.decode
        for case in SAMPLED_CASES:
            test_sampled_rows_are_the_full_run_bitwise(case, lib=lib)
        test_sampled_rows_e4m3_with_descales_are_the_full_run_bitwise(mod, lib)
        for d in (0.0123, 3.7):
            test_decode_is_the_exact_rational_product(d, mod)
        test_e4m3_attention_matches_sdpa_on_independently_dequantised_inputs(mod, lib)
        # an odd fp32 scale, whose float64 and fp32 values differ
        Q, K, V = rnd((1, 2, 9, 64), 204, 0), rnd((1, 2, 9, 64), 204, 1), rnd((1, 2, 9, 64), 204, 2)
        O, L = mod.attention(Q, K, V, 0.1, True, 0, lib=lib)
        s32 = float(torch.tensor(0.1, dtype=torch.float32))
        Lref = torch.logsumexp((torch.matmul(Q, K.transpose(-1, -2)) * s32).masked_fill(
            torch.ones(9, 9, dtype=torch.bool).triu(1), -math.inf), dim=-1)
        assert (L - Lref).abs().max().item() < 1e-14
        return True
    except AssertionError:
        return False
    finally:
        oracle.attention, oracle.decode = saved


def test_python_layer_planted_mistakes_are_caught():
    assert py_pin_suite(oracle), "the unmodified oracle must pass its Python-layer pins"
    for name, (old, new) in PY_MUTANTS.items():
        assert not py_pin_suite(mutated_oracle(old, new)), f"mutant {name} passed every pin"
