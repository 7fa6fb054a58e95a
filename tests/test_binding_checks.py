"""The Python binding rejects misuse before any C call (CPU only).

A host tensor beside a device q, a caller's out of the wrong shape or type, or
an out_dtype that disagrees with out would otherwise hand the kernels host
pointers or buffers smaller than they write. Each case must raise ValueError
and never reach libfa.
"""
import pytest
import torch

import exact_attention_02_amd as fa

B, H, Nq, Nk, D = 2, 3, 40, 56, 64


@pytest.fixture
def no_lib(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("libfa was called")
    monkeypatch.setattr(fa, "load", boom)


def qkv(dt=torch.bfloat16, dev="cpu"):
    return (torch.zeros(B, H, Nq, D, dtype=dt, device=dev), torch.zeros(B, H, Nk, D, dtype=dt, device=dev),
            torch.zeros(B, H, Nk, D, dtype=dt, device=dev))


def test_host_tensors_are_rejected_by_attention(no_lib):
    q, k, v = qkv()
    with pytest.raises(ValueError, match="device"):
        fa.attention(q, k, v, causal=True)


def test_host_tensors_are_rejected_by_attention_bwd(no_lib):
    q, k, v = qkv()
    o, lse = torch.zeros_like(q), torch.zeros(B, H, Nq)
    with pytest.raises(ValueError, match="device"):
        fa.attention_bwd(q, k, v, o, lse, torch.zeros_like(q), causal=True)


# The shape, dtype and placement rules themselves, on host tensors (require_gpu=False).

def fwd(**kw):
    q, k, v = kw.pop("qkv", qkv())
    return fa.check_forward_args(q, k, v, require_gpu=False, **kw)


def test_output_dtype_follows_out():
    assert fwd() == torch.bfloat16
    assert fwd(out=torch.zeros(B, H, Nq, D, dtype=torch.float32)) == torch.float32
    assert fwd(out_dtype=torch.float32) == torch.float32
    assert fwd(qkv=qkv(torch.float8_e4m3fn)) == torch.bfloat16


@pytest.mark.parametrize("kw,match", [
    (dict(out=torch.zeros(B, H, Nq, D, dtype=torch.bfloat16), out_dtype=torch.float32), "disagrees"),
    (dict(out=torch.zeros(B, H, Nq + 1, D, dtype=torch.bfloat16)), "shape"),
    (dict(out=torch.zeros(B, H, D, Nq, dtype=torch.bfloat16).transpose(2, 3)), "contiguous"),
    (dict(out=torch.zeros(B, H, Nq, D, dtype=torch.bfloat16, device="meta")), "meta"),
    (dict(out=torch.zeros(B, H, Nq, D, dtype=torch.float16)), "unsupported"),
    (dict(lse=torch.zeros(B, H, Nq, dtype=torch.float64)), "dtype"),
    (dict(lse=torch.zeros(B, H, Nq - 1)), "shape"),
    (dict(alibi=torch.zeros(H + 1)), "shape"),
    (dict(alibi=torch.zeros(H, dtype=torch.float64)), "dtype"),
    (dict(workspace=torch.zeros(64, dtype=torch.float32)), "dtype"),
    (dict(workspace=torch.zeros(64, dtype=torch.uint8, device="meta")), "meta"),
])
def test_forward_misuse_raises(kw, match):
    with pytest.raises(ValueError, match=match):
        fwd(**kw)


def test_forward_inputs_must_agree():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="meta"):
        fa.check_forward_args(q, k.to("meta"), v, require_gpu=False)
    with pytest.raises(ValueError, match="dtype"):
        fa.check_forward_args(q, k, v.to(torch.float16), require_gpu=False)
    with pytest.raises(ValueError, match="shape"):
        fa.check_forward_args(q, k, v[:, :, :-1].contiguous(), require_gpu=False)
    with pytest.raises(ValueError, match="contiguous"):
        fa.check_forward_args(q, k.transpose(2, 3).contiguous().transpose(2, 3), v, require_gpu=False)


def bwd(**kw):
    q, k, v = qkv()
    args = dict(out=torch.zeros_like(q), lse=torch.zeros(B, H, Nq), dout=torch.zeros_like(q))
    args.update(kw)
    return fa.check_backward_args(q, k, v, args.pop("out"), args.pop("lse"), args.pop("dout"), require_gpu=False,
                                  **args)


def test_backward_accepts_matching_tensors():
    bwd(dq=torch.zeros(B, H, Nq, D, dtype=torch.bfloat16), dk=torch.zeros(B, H, Nk, D, dtype=torch.bfloat16),
        dv=torch.zeros(B, H, Nk, D, dtype=torch.bfloat16), workspace=torch.zeros(16, dtype=torch.uint8))


@pytest.mark.parametrize("kw,match", [
    (dict(dq=torch.zeros(B, H, Nk, D, dtype=torch.bfloat16)), "shape"),
    (dict(dk=torch.zeros(B, H, Nk, D, dtype=torch.float16)), "dtype"),
    (dict(dv=torch.zeros(B, H, Nk, D, dtype=torch.bfloat16, device="meta")), "meta"),
    (dict(dq=torch.zeros(B, H, D, Nq, dtype=torch.bfloat16).transpose(2, 3)), "contiguous"),
    (dict(out=torch.zeros(B, H, Nq, D, dtype=torch.float16)), "dtype"),
    (dict(lse=torch.zeros(B, H, Nq, dtype=torch.float16)), "dtype"),
    (dict(dout=torch.zeros(B, H, Nq, D - 1, dtype=torch.bfloat16)), "shape"),
    (dict(alibi=torch.zeros(H - 1)), "shape"),
    (dict(workspace=torch.zeros(8, dtype=torch.int32)), "dtype"),
])
def test_backward_misuse_raises(kw, match):
    with pytest.raises(ValueError, match=match):
        bwd(**kw)
