"""The C ABI on the host: the library loads, exports what include/fa.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

import exact_attention_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+(?:\s+\w+)*\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS), names
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_enums_match_header():
    text = open(HEADER).read()
    for name in ["FA_F16", "FA_BF16", "FA_F16_F32OUT", "FA_E4M3", "FA_BF16_F32OUT", "FA_OK", "FA_ERR_NULL",
                 "FA_ERR_SHAPE", "FA_ERR_HEADDIM", "FA_ERR_DTYPE", "FA_ERR_MASK", "FA_ERR_SCALE",
                 "FA_ERR_ALIGN", "FA_ERR_DEVICE", "FA_ERR_LAUNCH", "FA_ERR_MOD", "FA_ERR_SCRATCH", "FA_MOD_NONE", "FA_MOD_SOFTCAP",
                 "FA_MOD_ALIBI", "FA_KNOB_KERNEL", "FA_KNOB_TILE_QB", "FA_KNOB_WG_GROUP", "FA_KNOB_WG_LIGHT",
                 "FA_KNOB_DEBUG"]:
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(fa, name), name


def test_status_strings():
    for s in range(11):
        assert fa.fa_status_str(s) and fa.fa_status_str(s) != "unknown status"
    assert fa.fa_status_str(99) == "unknown status"


P = 0x100000  # a 16-byte aligned dummy address; never dereferenced on these paths


def call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=64, Nk=64, D=64, scale=0.125, causal=0, window=0,
             dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"],
                     a["scale"], a["causal"], a["window"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), fa.FA_ERR_SHAPE), (dict(Nq=-3), fa.FA_ERR_SHAPE), (dict(Nk=-1), fa.FA_ERR_SHAPE),
    (dict(D=96), fa.FA_ERR_HEADDIM), (dict(D=0), fa.FA_ERR_HEADDIM), (dict(D=256), fa.FA_ERR_HEADDIM),
    (dict(dtype=0), fa.FA_ERR_DTYPE), (dict(dtype=6), fa.FA_ERR_DTYPE),
    (dict(window=16), fa.FA_ERR_MASK), (dict(window=-1, causal=1), fa.FA_ERR_MASK),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(scale=float("inf")), fa.FA_ERR_SCALE), (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(q=0), fa.FA_ERR_NULL), (dict(o=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL),
    (dict(k=0), fa.FA_ERR_NULL), (dict(v=0), fa.FA_ERR_NULL),
    (dict(q=P + 8), fa.FA_ERR_ALIGN), (dict(v=P + 4), fa.FA_ERR_ALIGN), (dict(lse=P + 2), fa.FA_ERR_ALIGN),
    (dict(B=1 << 20, H=1 << 12, Nq=1 << 20), fa.FA_ERR_SHAPE),
])
def test_argument_errors_before_any_device_work(kw, code):
    assert call(**kw) == code


def test_fp8_entry_checks_dtype_and_descales():
    args = (P, P, P, P, P, 1, 1, 64, 64, 128, 0.088, 0, 0)
    assert fa.fa_fwd_fp8(*args, fa.FA_BF16, None, 1.0, 1.0, 1.0) == fa.FA_ERR_DTYPE
    assert fa.fa_fwd_fp8(*args, fa.FA_E4M3, None, 0.0, 1.0, 1.0) == fa.FA_ERR_SCALE
    assert fa.fa_fwd_fp8(*args, fa.FA_E4M3, None, 1.0, float("nan"), 1.0) == fa.FA_ERR_SCALE


def test_window_entry_checks_extents_and_descales():
    args = (P, P, P, P, P, 1, 1, 64, 64, 64, 0.125)
    assert fa.fa_fwd_window(*args, -2, 0, fa.FA_BF16, None) == fa.FA_ERR_MASK
    assert fa.fa_fwd_window(*args, 0, -5, fa.FA_BF16, None) == fa.FA_ERR_MASK
    assert fa.fa_fwd_window(*args, 4, 4, fa.FA_BF16, None, 2.0, 1.0, 1.0) == fa.FA_ERR_SCALE
    assert fa.fa_fwd_window(*args, 4, 4, fa.FA_E4M3, None, 0.0, 1.0, 1.0) == fa.FA_ERR_SCALE
    assert fa.fa_fwd_window(P, P, P, P, P, 1, 1, 64, 64, 96, 0.125, -2, 0, fa.FA_BF16, None) == fa.FA_ERR_HEADDIM
    assert fa.fa_fwd_window(P, P, P, P, P, 0, 1, 64, 64, 64, 0.125, 4, 4, fa.FA_BF16, None) == fa.FA_OK
    assert fa.fa_fwd_window(0, P, P, P, P, 1, 1, 64, 64, 64, 0.125, 4, 4, fa.FA_BF16, None) == fa.FA_ERR_NULL


def test_mod_entry_checks_modifier_and_parameters():
    args = (P, P, P, P, P, 1, 1, 64, 64, 64, 0.125, -1, 0)
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, 3, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, -1, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, fa.FA_MOD_SOFTCAP, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, fa.FA_MOD_SOFTCAP, float("inf"), None) == fa.FA_ERR_MOD
    assert fa.fa_fwd_mod(*args, fa.FA_E4M3, None, fa.FA_MOD_SOFTCAP, 30.0, None) == fa.FA_ERR_MOD
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, fa.FA_MOD_ALIBI, 0.0, None) == fa.FA_ERR_NULL
    assert fa.fa_fwd_mod(*args, fa.FA_BF16, None, fa.FA_MOD_ALIBI, 0.0, P + 2) == fa.FA_ERR_ALIGN
    assert fa.fa_fwd_mod(P, P, P, P, P, 1, 1, 64, 64, 64, 0.125, -3, 0, fa.FA_BF16, None, 0, 0.0, None) == \
        fa.FA_ERR_MASK
    assert fa.fa_fwd_mod(P, P, P, P, P, 1, 1, 64, 64, 96, 0.125, -1, 0, fa.FA_BF16, None, 9, 0.0, None) == \
        fa.FA_ERR_HEADDIM
    assert fa.fa_fwd_mod(P, P, P, P, P, 0, 1, 64, 64, 64, 0.125, -1, 0, fa.FA_BF16, None, fa.FA_MOD_ALIBI, 0.0,
                         None) == fa.FA_OK


def test_splitkv_entry_checks_and_workspace_size():
    assert fa.splitkv_workspace_bytes(2, 3, 5, 64, 1) == 0
    assert fa.splitkv_workspace_bytes(2, 3, 5, 64, 4) == 2 * 3 * 4 * 5 * (64 + 1) * 4
    assert fa.splitkv_workspace_bytes(2, 3, 5, 64, 0) == -1
    assert fa.splitkv_num_splits(1, 32, 1, 32768, 64, fa.FA_BF16) > 1
    assert fa.splitkv_num_splits(4, 12, 8192, 8192, 64, fa.FA_BF16) == 1
    assert fa.splitkv_num_splits(1, 1, 1, 100, 64, fa.FA_BF16) == 1      # too few key tiles to split
    assert fa.splitkv_num_splits(1, 1, 1, 100000, 64, fa.FA_E4M3) == 1
    need = fa.splitkv_workspace_bytes(1, 2, 1, 64, 8)
    args = (P, P, P, P, P, 1, 2, 1, 4096, 64, 0.125, -1, 0)
    assert fa.fa_fwd_splitkv(*args, fa.FA_BF16, None, 0, P, need) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_splitkv(*args, fa.FA_BF16, None, 2000, P, need) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_splitkv(*args, fa.FA_E4M3, None, 8, P, need) == fa.FA_ERR_DTYPE
    assert fa.fa_fwd_splitkv(*args, fa.FA_BF16, None, 8, None, need) == fa.FA_ERR_NULL
    assert fa.fa_fwd_splitkv(*args, fa.FA_BF16, None, 8, P + 8, need) == fa.FA_ERR_ALIGN
    assert fa.fa_fwd_splitkv(*args, fa.FA_BF16, None, 8, P, need - 1) == fa.FA_ERR_SHAPE
    assert fa.fa_fwd_splitkv(P, P, P, P, P, 1, 2, 1, 4096, 64, 0.125, -2, 0, fa.FA_BF16, None, 8, P, need) == \
        fa.FA_ERR_MASK
    assert fa.fa_fwd_splitkv(P, P, P, P, P, 0, 2, 1, 4096, 64, 0.125, -1, 0, fa.FA_BF16, None, 8, None, 0) == fa.FA_OK


def bwd_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2, Nq=64, Nk=96, D=64, scale=0.125,
             wl=-1, wr=0, dtype=fa.FA_BF16, stream=None, ws=P, ws_bytes=fa.bwd_workspace_bytes(1, 2, 64))
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                     a["H"], a["Nq"], a["Nk"], a["D"], a["scale"], a["wl"], a["wr"], a["dtype"], a["stream"],
                     a["ws"], a["ws_bytes"])


def test_bwd_workspace_size():
    assert fa.bwd_workspace_bytes(2, 3, 5) == 2 * 2 * 3 * 8 * 4      # rows padded to a multiple of 4
    assert fa.bwd_workspace_bytes(1, 1, 8) == 2 * 8 * 4
    assert fa.bwd_workspace_bytes(1, 1, 0) == 0
    assert fa.bwd_workspace_bytes(-1, 1, 8) == -1
    assert fa.bwd_workspace_bytes(4, 12, 8192) == 2 * 4 * 12 * 8192 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), fa.FA_ERR_SHAPE), (dict(Nk=-1), fa.FA_ERR_SHAPE), (dict(D=96), fa.FA_ERR_HEADDIM),
    (dict(dtype=fa.FA_E4M3), fa.FA_ERR_DTYPE), (dict(dtype=fa.FA_F16_F32OUT), fa.FA_ERR_DTYPE),
    (dict(dtype=fa.FA_BF16_F32OUT), fa.FA_ERR_DTYPE), (dict(dtype=0), fa.FA_ERR_DTYPE),
    (dict(wl=-2), fa.FA_ERR_MASK), (dict(wr=-7), fa.FA_ERR_MASK),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(q=0), fa.FA_ERR_NULL), (dict(o=0), fa.FA_ERR_NULL), (dict(dout=0), fa.FA_ERR_NULL),
    (dict(lse=0), fa.FA_ERR_NULL), (dict(dq=0), fa.FA_ERR_NULL), (dict(ws=0), fa.FA_ERR_NULL),
    (dict(k=0), fa.FA_ERR_NULL), (dict(v=0), fa.FA_ERR_NULL), (dict(dk=0), fa.FA_ERR_NULL),
    (dict(dv=0), fa.FA_ERR_NULL),
    (dict(dout=P + 8), fa.FA_ERR_ALIGN), (dict(dk=P + 2), fa.FA_ERR_ALIGN), (dict(ws=P + 4), fa.FA_ERR_ALIGN),
    (dict(lse=P + 2), fa.FA_ERR_ALIGN),
    (dict(ws_bytes=fa.bwd_workspace_bytes(1, 2, 64) - 1), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 12, Nq=1 << 20), fa.FA_ERR_SHAPE),
])
def test_bwd_argument_errors_before_any_device_work(kw, code):
    assert bwd_call(**kw) == code


def test_bwd_mod_entry_checks_modifier_and_parameters():
    a = (P, P, P, P, P, P, P, P, P, 1, 2, 64, 96, 64, 0.125, -1, 0, fa.FA_BF16, None, P,
         fa.bwd_workspace_bytes(1, 2, 64))
    assert fa.fa_bwd_mod(*a, 3, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_bwd_mod(*a, -1, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_SOFTCAP, 0.0, None) == fa.FA_ERR_MOD
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_SOFTCAP, float("nan"), None) == fa.FA_ERR_MOD
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_ALIBI, 0.0, None) == fa.FA_ERR_NULL
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_ALIBI, 0.0, P + 2) == fa.FA_ERR_ALIGN
    b = list(a)
    b[17] = fa.FA_E4M3
    assert fa.fa_bwd_mod(*b, fa.FA_MOD_SOFTCAP, 30.0, None) == fa.FA_ERR_DTYPE
    c = list(a)
    c[9] = 0   # B = 0: nothing to do, no pointer needed
    assert fa.fa_bwd_mod(*c, fa.FA_MOD_ALIBI, 0.0, None) == fa.FA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_bwd_mod_valid_call_without_gpu_reports_device_error():
    a = (P, P, P, P, P, P, P, P, P, 1, 2, 64, 96, 64, 0.125, -1, 0, fa.FA_BF16, None, P,
         fa.bwd_workspace_bytes(1, 2, 64))
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_SOFTCAP, 30.0, None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_mod(*a, fa.FA_MOD_ALIBI, 0.0, P) == fa.FA_ERR_DEVICE


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_largest_head_is_accepted_and_one_more_row_is_not():
    """One head's rows must stay below 2^31 bytes at 4 bytes per element: at D = 64 that is 2^23 - 1 rows."""
    n = (1 << 23) - 1
    assert call(Nq=64, Nk=n) == fa.FA_ERR_DEVICE
    assert call(Nq=64, Nk=n + 1) == fa.FA_ERR_SHAPE
    assert call(Nq=n, Nk=64) == fa.FA_ERR_DEVICE
    assert call(Nq=n + 1, Nk=64) == fa.FA_ERR_SHAPE
    assert call(Nq=64, Nk=(1 << 22) - 1, D=128) == fa.FA_ERR_DEVICE
    assert call(Nq=64, Nk=1 << 22, D=128) == fa.FA_ERR_SHAPE
    assert bwd_call(Nq=64, Nk=n) == fa.FA_ERR_DEVICE
    assert bwd_call(Nq=64, Nk=n + 1) == fa.FA_ERR_SHAPE


def test_bwd_empty_problems_need_no_device():
    assert bwd_call(B=0) == fa.FA_OK
    assert bwd_call(H=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, ws=0) == fa.FA_OK
    assert bwd_call(Nq=0, Nk=0, q=0, k=0, v=0, ws=0) == fa.FA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_bwd_valid_call_without_gpu_reports_device_error():
    assert bwd_call() == fa.FA_ERR_DEVICE
    # no rows: dK = dV = 0 must still be written, so the call needs the device
    assert bwd_call(Nq=0, q=0, o=0, dout=0, lse=0, dq=0, ws=0, ws_bytes=0) == fa.FA_ERR_DEVICE
    assert bwd_call(Nk=0, k=0, v=0, dk=0, dv=0) == fa.FA_ERR_DEVICE


def test_empty_problems_need_no_device():
    assert call(B=0) == fa.FA_OK
    assert call(H=0, q=0, k=0, v=0, o=0, lse=0) == fa.FA_OK
    assert call(Nq=0) == fa.FA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_valid_call_without_gpu_reports_device_error():
    assert call() == fa.FA_ERR_DEVICE
    assert call(Nk=0, k=0, v=0) == fa.FA_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        fa.load(str(tmp_path / "libfa.so"))


def test_knobs_reject_unknown_names_and_values_and_restore():
    lib = fa.load()
    for knob in (0, 6, -1):
        assert lib.fa_set_knob(knob, 1) == fa.FA_ERR_SHAPE
    assert lib.fa_set_knob(fa.FA_KNOB_KERNEL, -2) == fa.FA_ERR_SHAPE
    try:
        assert fa.plan_kernel(4, 12, 8192, 8192, 64, fa.FA_BF16) == 3
        fa.set_knob(fa.FA_KNOB_KERNEL, 1)
        assert fa.plan_kernel(4, 12, 8192, 8192, 64, fa.FA_BF16) == 1
        fa.set_knob(fa.FA_KNOB_KERNEL, 2)   # key-split needs D = 64 and no modifier: honoured here
        assert fa.plan_kernel(4, 12, 8192, 8192, 64, fa.FA_BF16) == 2
        assert fa.plan_kernel(4, 12, 8192, 8192, 128, fa.FA_BF16) == 3   # ... and ignored here
    finally:
        fa.set_knob(fa.FA_KNOB_KERNEL, -1)
    assert fa.plan_kernel(4, 12, 8192, 8192, 64, fa.FA_BF16) == 3


def test_environment_variables_do_not_change_the_plan(monkeypatch):
    for name in ("FA_KERNEL", "FA_TILE_QB", "FA_WG_GROUP", "FA_WG_LIGHT", "FA_DEBUG"):
        monkeypatch.setenv(name, "1")
    assert fa.plan_kernel(4, 12, 8192, 8192, 64, fa.FA_BF16) == 3
    assert fa.plan_grid(4, 12, 8192, 8192, 64, 1, 0, fa.FA_BF16) == (3072, 128, 32, 64)


def test_plan_kernel_choices_and_errors():
    K = fa.plan_kernel
    assert K(4, 16, 8192, 8192, 128, fa.FA_E4M3) == 3                         # e4m3: serial kernel
    assert K(1, 1, 64, 1000, 64, fa.FA_E4M3) == 3
    assert K(4, 12, 8192, 8192, 64, fa.FA_BF16, fa.FA_MOD_SOFTCAP) == 3       # score modifiers: serial
    assert K(4, 12, 8192, 8192, 64, fa.FA_BF16, fa.FA_MOD_ALIBI) == 3
    assert K(1, 32, 32768, 32768, 128, fa.FA_BF16, fa.FA_MOD_ALIBI) == 3
    assert K(1, 1, 128, 128, 64, fa.FA_F16_F32OUT, fa.FA_MOD_SOFTCAP) == 3   # ... also where plain goes key-split
    assert K(1, 1, 128, 128, 64, fa.FA_F16_F32OUT) == 2                      # one workgroup: key-split
    assert K(8, 32, 1, 16384, 64, fa.FA_BF16, splitkv=True) == 2             # decode: key-split splits
    assert K(1, 32, 32768, 32768, 128, fa.FA_BF16) == 3                      # long context: serial
    with pytest.raises(fa.FaError):
        K(1, 1, 128, 128, 96, fa.FA_BF16)
    with pytest.raises(fa.FaError):
        K(1, 1, 128, 128, 128, fa.FA_E4M3, fa.FA_MOD_ALIBI)
    with pytest.raises(fa.FaError):
        K(1, 1, 128, 128, 128, fa.FA_E4M3, splitkv=True)


def test_clock_telemetry_checks_arguments():
    lib = fa.load()
    buf = (ctypes.c_ulonglong * 8)()
    assert lib.fa_set_clock_telemetry(None, 2) == fa.FA_ERR_NULL
    assert lib.fa_set_clock_telemetry(buf, 0) == fa.FA_ERR_SHAPE
    assert lib.fa_set_clock_telemetry(buf, -1) == fa.FA_ERR_SHAPE
    assert lib.fa_set_clock_telemetry(ctypes.addressof(buf) + 4, 1) == fa.FA_ERR_ALIGN
    assert lib.fa_set_clock_telemetry(None, 0) == fa.FA_OK


def test_noalloc_splitkv_checks_arguments_and_the_scratch_limit():
    lib = fa.load()
    A = 1 << 20   # a 16-byte-aligned stand-in address; nothing is launched in these cases
    args = dict(B=2, H=8, Nq=3, Nk=5000, D=64)

    def call(B, H, Nq, Nk, D, scale=0.125, wl=-1, wr=0, dtype=fa.FA_BF16, splits=4, q=A, o=A, lse=A):
        return lib.fa_fwd_splitkv_noalloc(q, A, A, o, lse, B, H, Nq, Nk, D, scale, wl, wr, dtype, None, splits)

    m = re.search(r"#define\s+FA_NOALLOC_SCRATCH_BYTES\s+\((\d+)LL\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES
    # the largest decode problem that fits, and one more head than fits
    per_head = fa.splitkv_workspace_bytes(1, 1, 4, 128, 64)
    heads = fa.FA_NOALLOC_SCRATCH_BYTES // per_head
    assert call(1, heads + 1, 4, 8192, 128, splits=64) == fa.FA_ERR_SCRATCH
    assert call(1, heads, 4, 8192, 128, splits=64) in (fa.FA_ERR_DEVICE, fa.FA_OK)
    # argument errors come first, before any device work
    assert call(**args, scale=-1.0) == fa.FA_ERR_SCALE
    assert call(**{**args, "D": 96}) == fa.FA_ERR_HEADDIM
    assert call(**args, wl=-2) == fa.FA_ERR_MASK
    assert call(**args, dtype=fa.FA_E4M3) == fa.FA_ERR_DTYPE
    assert call(**args, splits=0) == fa.FA_ERR_SHAPE
    assert call(**args, q=None) == fa.FA_ERR_NULL
    assert call(**args, lse=A + 2) == fa.FA_ERR_ALIGN
    assert call(2, 8, 0, 5000, 64) == fa.FA_OK          # empty problem: nothing to do
    if not torch.cuda.is_available():
        assert call(**args) == fa.FA_ERR_DEVICE
