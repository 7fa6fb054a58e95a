"""fa_fwd_splitkv_noalloc, the split-KV forward that allocates nothing: its
split results go to the library's static scratch array instead of a caller's
workspace. Through the C ABI, two calls in a row (the second smaller) must
give bitwise the outputs of fa_fwd_splitkv with a workspace, and meet the
oracle's bounds."""
import pytest
import torch

import exact_attention_02_amd as fa
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_pair(B, H, Nq, Nk, D, causal, din, splits, seed):
    w = synth.small_workload(f"noalloc_B{B}H{H}q{Nq}k{Nk}D{D}_{din}", B, H, Nq, Nk, D, causal, 0, din, din, seed)
    inp = synth.make_inputs(w)
    q, k, v = inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)
    dt = q.dtype
    code = fa.dtype_code(dt, dt)
    if splits == "auto":
        splits = fa.splitkv_num_splits(B, H, Nq, Nk, D, code)
    wl, wr = -1, (0 if causal else -1)
    stream = torch.cuda.current_stream().cuda_stream
    o1, l1 = torch.empty_like(q), torch.empty(B, H, Nq, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, fa.splitkv_workspace_bytes(B, H, Nq, D, splits)), dtype=torch.uint8, device=DEV)
    st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(), B, H, Nq, Nk, D,
                           w.scale, wl, wr, code, stream, splits, ws.data_ptr(), ws.numel())
    assert st == fa.FA_OK
    o2, l2 = torch.full_like(q, float("nan")), torch.full((B, H, Nq), float("nan"), device=DEV)
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), B, H, Nq,
                                   Nk, D, w.scale, wl, wr, code, stream, splits)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    Oref, Lref = oracle.attention(inp.q, inp.k, inp.v, w.scale, causal, 0)
    bound = {"f16": 2e-3, "bf16": 1e-2}[din]
    assert (o2.double().cpu() - Oref).abs().max().item() <= bound
    assert ((l2.double().cpu() - Lref).abs() / Lref.abs().clamp(min=1.0)).max().item() <= 1e-4
    return splits


@pytest.mark.parametrize("din,D", [("bf16", 64), ("f16", 128)])
def test_noalloc_splitkv_matches_the_workspace_call_twice(din, D):
    # a large call, then a smaller one: the scratch keeps the first call's
    # contents, and the second must not depend on them
    s1 = run_pair(4, 8, 5, 6000, D, True, din, "auto", 8100 + D)
    s2 = run_pair(1, 3, 2, 2100, D, True, din, 7, 8200 + D)
    assert s1 > 1 and s2 > 1
    run_pair(2, 2, 1, 4000, D, False, din, 64, 8300 + D)
