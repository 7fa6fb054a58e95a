"""The largest problems the entry points accept, on the GPU, against the oracle.

One head's rows of any tensor must stay below 2^31 bytes (max(Nq, Nk) * D * 4
< 2^31: the kernels address a head through 32-bit buffer descriptors and
offsets), so at D = 64 a head holds at most 2^23 - 1 keys or query rows. These
tests run at that size, with a ragged last tile, so that every offset near the
top of the 32-bit range is exercised:
  * the forward (fa_fwd, and fa_fwd_splitkv with the recommended split count)
    with 40 query rows against 2^23 - 1 keys, every row compared;
  * the forward with 2^23 - 1 query rows against 100 keys, sampled rows
    compared (the first and last rows, tile boundaries, random rows);
  * the backward with 4 query rows against 2^23 - 1 keys, every element of
    dQ, dK and dV compared under the bound of test_parity_bwd_gpu.
"""
import pytest
import torch

import exact_attention_02_amd as fa
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NMAX = (1 << 23) - 1
_cache = {}


def inputs(name, Nq, Nk):
    if name not in _cache:
        w = synth.small_workload(name, 1, 1, Nq, Nk, 64, False, 0, "bf16", "bf16", 21, backward=True)
        print(f"generating {name} Nq{Nq} Nk{Nk}", flush=True)
        _cache[name] = (w, synth.make_inputs(w))
    return _cache[name]


def compare_rows(w, o, lse, rows, Oref, Lref):
    O = o.reshape(-1, w.D)[rows.to(DEV)].double().cpu()
    L = lse.reshape(-1)[rows.to(DEV)].double().cpu()
    err = (O - Oref).abs().max().item()
    lerr = ((L - Lref).abs() / Lref.abs().clamp(min=1.0)).max().item()
    print(f"{w.name}: max |O - O_ref| {err:.3e}, LSE rel {lerr:.3e}", flush=True)
    assert err <= 1e-2 and lerr <= 1e-4


@pytest.mark.parametrize("path", ["fa_fwd", "splitkv"])
def test_forward_at_the_maximum_key_count(path):
    w, inp = inputs("maxkeys", 40, NMAX)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    extra = dict(num_splits="auto") if path == "splitkv" else {}
    o, lse = fa.attention(q, k, v, scale=w.scale, **extra)
    torch.cuda.synchronize()
    rows = torch.arange(40)
    if "maxkeys_ref" not in _cache:
        _cache["maxkeys_ref"] = oracle.attention(inp.q, inp.k, inp.v, w.scale, False, 0, rows=rows)
    Oref, Lref = _cache["maxkeys_ref"]
    compare_rows(w, o, lse, rows, Oref, Lref)


def test_forward_at_the_maximum_query_count():
    w, inp = inputs("maxrows", NMAX, 100)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    o, lse = fa.attention(q, k, v, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(3)
    rows = sorted(set([0, 1, 127, 128, NMAX // 2, NMAX - 129, NMAX - 128, NMAX - 2, NMAX - 1]
                      + torch.randint(0, NMAX, (1000,), generator=g).tolist()))
    rows = torch.tensor(rows)
    Oref, Lref = oracle.attention(inp.q, inp.k, inp.v, w.scale, False, 0, rows=rows)
    compare_rows(w, o, lse, rows, Oref, Lref)


def test_backward_at_the_maximum_key_count():
    from test_parity_bwd_gpu import check
    w0, inp0 = inputs("maxkeys", 40, NMAX)
    # the first 4 query rows of the same inputs (the oracle's backward streams
    # dK and dV once per row)
    w = synth.small_workload("maxkeys_bwd", 1, 1, 4, NMAX, 64, False, 0, "bf16", "bf16", 21, backward=True)
    q = inp0.q[:, :, :4].contiguous()
    do = synth.make_grad_out(w)
    qd, kd, vd, dod = q.to(DEV), inp0.k.to(DEV), inp0.v.to(DEV), do.to(DEV)
    o, lse = fa.attention(qd, kd, vd, scale=w.scale, window_left=-1, window_right=-1)
    dq, dk, dv = fa.attention_bwd(qd, kd, vd, o, lse, dod, scale=w.scale, window_left=-1, window_right=-1)
    torch.cuda.synchronize()
    check(w, -1, -1, q, inp0.k, inp0.v, do, o.cpu(), dq.cpu(), dk.cpu(), dv.cpu())
