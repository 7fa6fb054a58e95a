"""Python binding of libfa.so, the gfx950 fused exact-attention forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI in include/fa.h. The functions fa_fwd, fa_fwd_fp8 and
fa_status_str carry the C names and arguments (device pointers as ints, the
stream as an int handle). `attention()` is a convenience wrapper that takes
torch tensors on a ROCm device, allocates the outputs with torch and calls
fa_fwd / fa_fwd_fp8 on torch's current stream.

There is no fallback: if libfa.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

# Mirrors of the enums in include/fa.h.
FA_F16, FA_BF16, FA_F16_F32OUT, FA_E4M3, FA_BF16_F32OUT = 1, 2, 3, 4, 5
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_DTYPE = 0, 1, 2, 3, 4
FA_ERR_MASK, FA_ERR_SCALE, FA_ERR_ALIGN, FA_ERR_DEVICE, FA_ERR_LAUNCH = 5, 6, 7, 8, 9
FA_ERR_MOD = 10
FA_ERR_SCRATCH = 11
FA_NOALLOC_SCRATCH_BYTES = 32 << 20
FA_MOD_NONE, FA_MOD_SOFTCAP, FA_MOD_ALIBI = 0, 1, 2
FA_KNOB_KERNEL, FA_KNOB_TILE_QB, FA_KNOB_WG_GROUP, FA_KNOB_WG_LIGHT, FA_KNOB_DEBUG = 1, 2, 3, 4, 5

EXPORTS = ("fa_fwd", "fa_fwd_fp8", "fa_fwd_window", "fa_fwd_mod", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
           "fa_splitkv_workspace_bytes",
           "fa_splitkv_num_splits", "fa_bwd", "fa_bwd_mod", "fa_bwd_workspace_bytes", "fa_status_str", "fa_plan_grid", "fa_plan_tile", "fa_plan_block_class",
           "fa_plan_window_range", "fa_plan_block_class_window", "fa_plan_kernel", "fa_set_clock_telemetry", "fa_set_knob")

# fa_plan_kernel's kinds and the kernels each runs (split-KV adds the merge kernel).
KERNEL_NAMES = {0: "fa_fwd_kernel", 1: "fa_fwd16_kernel", 2: "fa_fwd_ks_kernel", 3: "fa_fwd_serial_kernel"}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({fa_status_str(status)})")


def load(path: str = LIB_PATH):
    """Loads libfa.so and declares the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    # torch's ROCm build carries its own HIP runtime under a file name other
    # than ROCm's. Loaded first, libfa.so would bring in ROCm's runtime, and
    # torch would then load its own beside it: two runtimes in one process, and
    # the library's calls would not see the device and streams torch set up.
    # With torch loaded first, libfa.so's libamdhip64.so.7 resolves to torch's.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I, F, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
    pI, pLL = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_longlong)
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, F, F, F]
    lib.fa_fwd_fp8.restype = I
    lib.fa_fwd_window.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, F, F, F]
    lib.fa_fwd_window.restype = I
    lib.fa_fwd_mod.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, I, F, P]
    lib.fa_fwd_mod.restype = I
    lib.fa_fwd_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, I, P, LL]
    lib.fa_fwd_splitkv.restype = I
    lib.fa_fwd_splitkv_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, I]
    lib.fa_fwd_splitkv_noalloc.restype = I
    lib.fa_splitkv_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_splitkv_workspace_bytes.restype = LL
    lib.fa_splitkv_num_splits.argtypes = [I, I, I, I, I, I]
    lib.fa_splitkv_num_splits.restype = I
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, P, LL]
    lib.fa_bwd.restype = I
    lib.fa_bwd_mod.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, P, LL, I, F, P]
    lib.fa_bwd_mod.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.fa_bwd_workspace_bytes.restype = LL
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_plan_grid.argtypes = [I, I, I, I, I, I, I, I, pLL, pI, pI, pI]
    lib.fa_plan_grid.restype = I
    lib.fa_plan_tile.argtypes = [I, I, I, I, I, I, I, I, LL, pI, pI, pI, pI]
    lib.fa_plan_tile.restype = I
    lib.fa_plan_block_class.argtypes = [I, I, I, I, I, I, I, I]
    lib.fa_plan_block_class.restype = I
    lib.fa_plan_window_range.argtypes = [I, I, I, I, I, I, pI, pI]
    lib.fa_plan_window_range.restype = I
    lib.fa_plan_block_class_window.argtypes = [I, I, I, I, I, I, I, I]
    lib.fa_plan_block_class_window.restype = I
    lib.fa_plan_kernel.argtypes = [I, I, I, I, I, I, I, I]
    lib.fa_plan_kernel.restype = I
    lib.fa_set_clock_telemetry.argtypes = [P, I]
    lib.fa_set_clock_telemetry.restype = I
    lib.fa_set_knob.argtypes = [I, I]
    lib.fa_set_knob.restype = I
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, dtype, stream=None) -> int:
    """The C call, unchanged: pointers are ints (device addresses); returns the status."""
    return load().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(causal), int(window), dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, window, dtype, stream,
               descale_q, descale_k, descale_v) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(causal), int(window), dtype, stream,
                             descale_q, descale_k, descale_v)


def fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream,
                  descale_q=1.0, descale_k=1.0, descale_v=1.0) -> int:
    return load().fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(window_left), int(window_right), dtype,
                                stream, descale_q, descale_k, descale_v)


def fa_fwd_mod(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream,
               score_mod, softcap=0.0, alibi_slopes=None) -> int:
    return load().fa_fwd_mod(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(window_left), int(window_right), dtype,
                             stream, int(score_mod), float(softcap), alibi_slopes)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream,
                   num_splits, workspace, workspace_bytes) -> int:
    return load().fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(window_left), int(window_right), dtype,
                                 stream, int(num_splits), workspace, int(workspace_bytes))


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream,
                           num_splits) -> int:
    return load().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, scale, int(window_left),
                                         int(window_right), dtype, stream, int(num_splits))


def splitkv_workspace_bytes(B, H, Nq, D, num_splits) -> int:
    return load().fa_splitkv_workspace_bytes(B, H, Nq, D, num_splits)


def splitkv_num_splits(B, H, Nq, Nk, D, dtype) -> int:
    return load().fa_splitkv_num_splits(B, H, Nq, Nk, D, dtype)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, window_left, window_right, dtype, stream,
           workspace, workspace_bytes) -> int:
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, int(window_left),
                         int(window_right), dtype, stream, workspace, int(workspace_bytes))


def fa_bwd_mod(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, window_left, window_right, dtype,
               stream, workspace, workspace_bytes, score_mod, softcap=0.0, alibi_slopes=None) -> int:
    return load().fa_bwd_mod(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, scale, int(window_left),
                             int(window_right), dtype, stream, workspace, int(workspace_bytes), int(score_mod),
                             float(softcap), alibi_slopes)


def bwd_workspace_bytes(B, H, Nq) -> int:
    return load().fa_bwd_workspace_bytes(B, H, Nq)


def alibi_slopes(H: int):
    """The geometric ALiBi slopes 2^(-8 (h+1) / H), h = 0 .. H-1, as a list of floats."""
    return [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]


def fa_status_str(status: int) -> str:
    return load().fa_status_str(status).decode()


def plan_grid(B, H, Nq, Nk, D, causal, window, dtype):
    """(n_wg, br, qw, bc) of the launch fa_fwd would make."""
    n = ctypes.c_longlong()
    br, qw, bc = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = load().fa_plan_grid(B, H, Nq, Nk, D, int(causal), int(window), dtype, ctypes.byref(n), ctypes.byref(br),
                             ctypes.byref(qw), ctypes.byref(bc))
    if st != FA_OK:
        raise FaError(st, "fa_plan_grid")
    return n.value, br.value, qw.value, bc.value


def plan_tile(B, H, Nq, Nk, D, causal, window, dtype, wg):
    """(bh, qtile, kv_lo, kv_hi) of workgroup wg."""
    bh, qt, lo, hi = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = load().fa_plan_tile(B, H, Nq, Nk, D, int(causal), int(window), dtype, wg, ctypes.byref(bh),
                             ctypes.byref(qt), ctypes.byref(lo), ctypes.byref(hi))
    if st != FA_OK:
        raise FaError(st, "fa_plan_tile")
    return bh.value, qt.value, lo.value, hi.value


def plan_kernel(B, H, Nq, Nk, D, dtype, score_mod=FA_MOD_NONE, splitkv=False) -> int:
    """The forward kernel kind (KERNEL_NAMES) a call would launch."""
    k = load().fa_plan_kernel(B, H, Nq, Nk, D, dtype, int(score_mod), int(bool(splitkv)))
    if k < 0:
        raise FaError(-k, "fa_plan_kernel")
    return k


def set_knob(knob: int, value: int) -> None:
    """A tuning override of the launch planning (FA_KNOB_*; -1 restores the default)."""
    st = load().fa_set_knob(int(knob), int(value))
    if st != FA_OK:
        raise FaError(st, "fa_set_knob")


def fa_set_clock_telemetry(buf, n) -> int:
    return load().fa_set_clock_telemetry(buf, int(n))


def plan_block_class(w0, w1, c0, c1, Nq, Nk, causal, window) -> int:
    return load().fa_plan_block_class(w0, w1, c0, c1, Nq, Nk, int(causal), int(window))


def plan_window_range(r0, r1, Nq, Nk, window_left, window_right):
    """Keys [lo, hi) visible to at least one row of [r0, r1) under fa_fwd_window's mask."""
    lo, hi = ctypes.c_int(), ctypes.c_int()
    st = load().fa_plan_window_range(r0, r1, Nq, Nk, window_left, window_right, ctypes.byref(lo), ctypes.byref(hi))
    if st != FA_OK:
        raise FaError(st, "fa_plan_window_range")
    return lo.value, hi.value


def plan_block_class_window(w0, w1, c0, c1, Nq, Nk, window_left, window_right) -> int:
    return load().fa_plan_block_class_window(w0, w1, c0, c1, Nq, Nk, window_left, window_right)


def dtype_code(in_dtype, out_dtype) -> int:
    import torch
    table = {
        (torch.float16, torch.float16): FA_F16,
        (torch.bfloat16, torch.bfloat16): FA_BF16,
        (torch.float16, torch.float32): FA_F16_F32OUT,
        (torch.float8_e4m3fn, torch.bfloat16): FA_E4M3,
        (torch.bfloat16, torch.float32): FA_BF16_F32OUT,
    }
    if (in_dtype, out_dtype) not in table:
        raise ValueError(f"unsupported dtypes {in_dtype} -> {out_dtype}")
    return table[(in_dtype, out_dtype)]


def _check(t, name, device, shape=None, dtype=None):
    """One tensor argument: on `device`, contiguous, and of the given shape and dtype."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _device_of(q, require_gpu=True):
    """q's device, which every other tensor argument must share; a GPU device unless require_gpu is False."""
    import torch
    if not isinstance(q, torch.Tensor):
        raise ValueError("q must be a torch tensor")
    if require_gpu and q.device.type != "cuda":
        raise ValueError(f"q is on {q.device}: the kernels take device tensors (a ROCm GPU)")
    return q.device


def check_forward_args(q, k, v, out=None, lse=None, out_dtype=None, alibi=None, workspace=None,
                       require_gpu=True):
    """Validates attention()'s tensors before any C call and returns the output dtype.

    Every tensor must be contiguous and on q's device (a GPU device unless
    require_gpu is False, which the CPU tests use); k and v [B,H,Nk,D] of q's
    dtype; a given out [B,H,Nq,D], whose dtype is the output type (out_dtype,
    when also given, must agree); a given lse [B,H,Nq] float32; alibi H float32
    slopes; workspace a uint8 tensor.
    """
    import torch
    dev = _device_of(q, require_gpu)
    if q.dim() != 4:
        raise ValueError("q must be [B,H,Nq,D]")
    B, H, Nq, D = q.shape
    _check(q, "q", dev)
    if k.dim() != 4:
        raise ValueError("k must be [B,H,Nk,D]")
    Nk = k.shape[2]
    _check(k, "k", dev, (B, H, Nk, D), q.dtype)
    _check(v, "v", dev, (B, H, Nk, D), q.dtype)
    if out is not None:
        if out_dtype is not None and out_dtype != out.dtype:
            raise ValueError(f"out_dtype {out_dtype} disagrees with out.dtype {out.dtype}")
        out_dtype = out.dtype
        _check(out, "out", dev, (B, H, Nq, D))
    if out_dtype is None:
        out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    dtype_code(q.dtype, out_dtype)   # raises on an unsupported pair
    if lse is not None:
        _check(lse, "lse", dev, (B, H, Nq), torch.float32)
    if alibi is not None:
        _check(alibi, "alibi", dev, (H,), torch.float32)
    if workspace is not None:
        _check(workspace, "workspace", dev, None, torch.uint8)
    return out_dtype


def check_backward_args(q, k, v, out, lse, dout, dq=None, dk=None, dv=None, alibi=None, workspace=None,
                        require_gpu=True):
    """Validates attention_bwd()'s tensors before any C call (as check_forward_args)."""
    import torch
    dev = _device_of(q, require_gpu)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,H,Nq,D] and k [B,H,Nk,D]")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check(q, "q", dev)
    for t, name in ((k, "k"), (v, "v")):
        _check(t, name, dev, (B, H, Nk, D), q.dtype)
    for t, name in ((out, "out"), (dout, "dout")):
        _check(t, name, dev, (B, H, Nq, D), q.dtype)
    _check(lse, "lse", dev, (B, H, Nq), torch.float32)
    for t, name, shp in ((dq, "dq", (B, H, Nq, D)), (dk, "dk", (B, H, Nk, D)), (dv, "dv", (B, H, Nk, D))):
        if t is not None:
            _check(t, name, dev, shp, q.dtype)
    if alibi is not None:
        _check(alibi, "alibi", dev, (H,), torch.float32)
    if workspace is not None:
        _check(workspace, "workspace", dev, None, torch.uint8)


def attention(q, k, v, scale=None, causal=False, window=0, out=None, lse=None, out_dtype=None,
              descales=None, stream=None, window_left=None, window_right=None,
              score_mod=None, softcap=0.0, alibi=None, num_splits=None, workspace=None):
    """O [B,H,Nq,D] and LSE [B,H,Nq] (float32) of softmax(scale Q K^T) V via libfa.

    q [B,H,Nq,D], k and v [B,H,Nk,D]: contiguous device tensors of one dtype
    (float16, bfloat16 or float8_e4m3fn). The output dtype is out.dtype when
    out is given, else out_dtype, else the input dtype (bfloat16 for e4m3).
    descales = (dq, dk, dv) for e4m3 inputs. Every tensor argument is checked
    (check_forward_args) before any C call.
    The mask is (causal, window) as in fa_fwd, or, when window_left or
    window_right is given, the key interval [i' - window_left, i' + window_right]
    of fa_fwd_window (None or -1: that side unbounded; causal and window are then
    ignored).
    score_mod: None, "softcap" (s <- softcap * tanh(s / softcap)) or "alibi"
    (s <- s + slope_h * (j - i')); alibi is a float32 device tensor of H slopes
    (default: alibi_slopes(H)). Score modifiers go through fa_fwd_mod.
    num_splits: split-KV through fa_fwd_splitkv ("auto": fa_splitkv_num_splits);
    workspace: a uint8 device tensor of at least splitkv_workspace_bytes(...)
    bytes (allocated here when None).
    """
    import torch
    out_dtype = check_forward_args(q, k, v, out, lse, out_dtype, alibi, workspace)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    code = dtype_code(q.dtype, out_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, Nq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    if num_splits is not None:
        if score_mod is not None:
            raise ValueError("split-KV takes no score modifier")
        if window_left is not None or window_right is not None:
            wl = -1 if window_left is None else int(window_left)
            wr = -1 if window_right is None else int(window_right)
        else:
            wl = int(window) - 1 if window > 0 else -1
            wr = 0 if causal else -1
        ns = splitkv_num_splits(B, H, Nq, Nk, D, code) if num_splits == "auto" else int(num_splits)
        need = splitkv_workspace_bytes(B, H, Nq, D, ns)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        st = fa_fwd_splitkv(*ptrs, B, H, Nq, Nk, D, float(scale), wl, wr, code, stream, ns, workspace.data_ptr(),
                            workspace.numel() * workspace.element_size())
        if st != FA_OK:
            raise FaError(st, "fa_fwd_splitkv")
        return out, lse
    if score_mod is not None:
        if window_left is not None or window_right is not None:
            wl = -1 if window_left is None else int(window_left)
            wr = -1 if window_right is None else int(window_right)
        else:
            wl = int(window) - 1 if window > 0 else -1
            wr = 0 if causal else -1
        mod = {"softcap": FA_MOD_SOFTCAP, "alibi": FA_MOD_ALIBI, "none": FA_MOD_NONE}[score_mod]
        slopes_ptr = None
        if mod == FA_MOD_ALIBI:
            if alibi is None:
                alibi = torch.tensor(alibi_slopes(H), dtype=torch.float32, device=q.device)
            slopes_ptr = alibi.data_ptr()
        st = fa_fwd_mod(*ptrs, B, H, Nq, Nk, D, float(scale), wl, wr, code, stream, mod, float(softcap), slopes_ptr)
        if st != FA_OK:
            raise FaError(st, "fa_fwd_mod")
        return out, lse
    if window_left is not None or window_right is not None:
        wl = -1 if window_left is None else int(window_left)
        wr = -1 if window_right is None else int(window_right)
        ds = [float(x) for x in descales] if (code == FA_E4M3 and descales is not None) else [1.0, 1.0, 1.0]
        st = fa_fwd_window(*ptrs, B, H, Nq, Nk, D, float(scale), wl, wr, code, stream, *ds)
        if st != FA_OK:
            raise FaError(st, "fa_fwd_window")
        return out, lse
    args = (*ptrs, B, H, Nq, Nk, D, float(scale), int(bool(causal)), int(window), code, stream)
    if code == FA_E4M3 and descales is not None:
        st = fa_fwd_fp8(*args, *[float(x) for x in descales])
        where = "fa_fwd_fp8"
    else:
        st = fa_fwd(*args)
        where = "fa_fwd"
    if st != FA_OK:
        raise FaError(st, where)
    return out, lse


def attention_bwd(q, k, v, out, lse, dout, scale=None, causal=False, window_left=None, window_right=None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None, score_mod=None, softcap=0.0, alibi=None):
    """dQ, dK, dV of O = softmax(scale Q K^T) V contracted with dout, via fa_bwd.

    q, out, dout [B,H,Nq,D], k and v [B,H,Nk,D]: contiguous float16 or bfloat16
    device tensors of one dtype; out and lse [B,H,Nq] (float32) are the
    forward's outputs for the same arguments. The mask is causal (window_left
    unbounded, window_right 0) or the extents of fa_fwd_window (None or -1:
    unbounded). workspace: a uint8 device tensor of at least
    bwd_workspace_bytes(B, H, Nq) bytes (allocated here when None). Every
    tensor argument is checked (check_backward_args) before any C call.
    score_mod, softcap, alibi: as in attention() (then through fa_bwd_mod; out
    and lse must come from the forward with the same modifier).
    """
    import torch
    check_backward_args(q, k, v, out, lse, dout, dq, dk, dv, alibi, workspace)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    code = {torch.float16: FA_F16, torch.bfloat16: FA_BF16}[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if window_left is not None or window_right is not None:
        wl = -1 if window_left is None else int(window_left)
        wr = -1 if window_right is None else int(window_right)
    else:
        wl, wr = -1, (0 if causal else -1)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = bwd_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if score_mod is None:
        st = fa_bwd(*ptrs, B, H, Nq, Nk, D, float(scale), wl, wr, code, stream, *ws)
        where = "fa_bwd"
    else:
        mod = {"softcap": FA_MOD_SOFTCAP, "alibi": FA_MOD_ALIBI, "none": FA_MOD_NONE}[score_mod]
        slopes_ptr = None
        if mod == FA_MOD_ALIBI:
            if alibi is None:
                alibi = torch.tensor(alibi_slopes(H), dtype=torch.float32, device=q.device)
            slopes_ptr = alibi.data_ptr()
        st = fa_bwd_mod(*ptrs, B, H, Nq, Nk, D, float(scale), wl, wr, code, stream, *ws, mod, float(softcap),
                        slopes_ptr)
        where = "fa_bwd_mod"
    if st != FA_OK:
        raise FaError(st, where)
    return dq, dk, dv


_autograd_fn = None


def _flash_fn():
    """The autograd Function (built on first use, so that importing the package does not import torch)."""
    global _autograd_fn
    if _autograd_fn is None:
        import torch

        class FlashAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, window_left, window_right, score_mod, softcap, alibi):
                o, lse = attention(q, k, v, scale=scale, window_left=window_left, window_right=window_right,
                                   score_mod=score_mod, softcap=softcap, alibi=alibi)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.args = (scale, window_left, window_right, score_mod, softcap, alibi)
                return o

            @staticmethod
            def backward(ctx, dout):
                q, k, v, o, lse = ctx.saved_tensors
                scale, wl, wr, score_mod, softcap, alibi = ctx.args
                dq, dk, dv = attention_bwd(q, k, v, o, lse, dout.contiguous(), scale=scale, window_left=wl,
                                           window_right=wr, score_mod=score_mod, softcap=softcap, alibi=alibi)
                return dq, dk, dv, None, None, None, None, None, None

        _autograd_fn = FlashAttention
    return _autograd_fn


def flash_attention(q, k, v, scale=None, causal=False, window_left=None, window_right=None, score_mod=None,
                    softcap=0.0, alibi=None):
    """O = softmax(f(scale Q K^T)) V as a differentiable torch operation: the
    forward through fa_fwd_window / fa_fwd_mod, the backward through fa_bwd /
    fa_bwd_mod with the saved O and LSE. float16 or bfloat16 inputs
    [B,H,Nq,D], [B,H,Nk,D]; the mask is causal or the extents (None or -1:
    open side); score_mod, softcap, alibi as in attention()."""
    import math as _m
    if scale is None:
        scale = 1.0 / _m.sqrt(q.shape[-1])
    if window_left is None and window_right is None:
        wl, wr = -1, (0 if causal else -1)
    else:
        wl = -1 if window_left is None else int(window_left)
        wr = -1 if window_right is None else int(window_right)
    if score_mod == "alibi" and alibi is None:
        import torch
        alibi = torch.tensor(alibi_slopes(q.shape[1]), dtype=torch.float32, device=q.device)
    return _flash_fn().apply(q, k, v, float(scale), wl, wr, score_mod, float(softcap), alibi)
