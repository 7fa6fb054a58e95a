"""CPU oracle for the exact attention forward pass (float64).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package. The product path (the HIP library and
its binding) never imports, links or runs it, and shares no code with it.

`attention()` decodes the stored inputs exactly to float64 (float16, bfloat16
and E4M3FN values are all exactly representable; an e4m3 value is then
multiplied by its fp32 descale in float64, which is exact too), then calls the
plain C implementation in oracle.c of softmax(scale * Q K^T) V and the
per-row log-sum-exp, with each softmax row materialised.

Parity pins: tests/test_oracle_pins.py (closed forms, invariants, brute force
at 50 significant digits, an independent library routine, planted mistakes in
oracle.c) and tests/test_oracle_sampled_pins.py (the sampled-row path bit for
bit against the full run under every mask and score modifier, the e4m3 decode
against exact rational arithmetic, the e4m3 path against torch's SDPA on
independently dequantised inputs, planted mistakes in this file).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out: str = _LIB, src: str = _SRC, extra=()) -> str:
    """Compile oracle.c with gcc into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = _LIB):
    lib = ctypes.CDLL(path)
    fn = lib.oracle_attn_fwd
    P = ctypes.c_void_p
    L = ctypes.c_long
    fn.argtypes = [P, P, P, P, P, L, L, L, L, L, ctypes.c_double, ctypes.c_int, L, P, L, ctypes.c_int]
    fn.restype = ctypes.c_int
    fw = lib.oracle_attn_fwd_window
    fw.argtypes = [P, P, P, P, P, L, L, L, L, L, ctypes.c_double, L, L, P, L, ctypes.c_int]
    fw.restype = ctypes.c_int
    fm = lib.oracle_attn_fwd_mod
    fm.argtypes = [P, P, P, P, P, L, L, L, L, L, ctypes.c_double, L, L, ctypes.c_int, ctypes.c_double, P, P, L,
                   ctypes.c_int]
    fm.restype = ctypes.c_int
    fb = lib.oracle_attn_bwd
    fb.argtypes = [P, P, P, P, P, P, P, L, L, L, L, L, ctypes.c_double, L, L, ctypes.c_int]
    fb.restype = ctypes.c_int
    fbm = lib.oracle_attn_bwd_mod
    fbm.argtypes = [P, P, P, P, P, P, P, L, L, L, L, L, ctypes.c_double, L, L, ctypes.c_int, ctypes.c_double, P,
                    ctypes.c_int]
    fbm.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load()
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def decode(x: torch.Tensor, descale: float = 1.0) -> torch.Tensor:
    """Exact float64 value of each stored element, times its descale."""
    y = x.detach().to("cpu").to(torch.float64)
    if descale != 1.0:
        y = y * float(descale)
    return y.contiguous()


MODS = {None: 0, "softcap": 1, "alibi": 2}


def attention(q, k, v, scale, causal=False, window=0, descales=(1.0, 1.0, 1.0),
              rows=None, threads=None, lib=None, window_left=None, window_right=None,
              score_mod=None, softcap=0.0, alibi_slopes=None):
    """float64 O and LSE of softmax(scale * Q K^T) V.

    q [B,H,Nq,D], k and v [B,H,Nk,D] (CPU or device tensors of any float dtype).
    scale is used as float64(fp32(scale)) -- the fp32 value the kernel gets.
    rows: None for every row (O [B,H,Nq,D], LSE [B,H,Nq]); otherwise an
    iterable of flattened row ids (b*H + h)*Nq + i (O [n,D], LSE [n]).
    The mask is (causal, window), or, when window_left or window_right is
    given, the keys [i' - window_left, i' + window_right] of row i (None or a
    negative extent: that side open); causal and window are then ignored.
    score_mod: None, "softcap" (s <- softcap * tanh(s / softcap)) or "alibi"
    (s <- s + alibi_slopes[h] * (j - i'), alibi_slopes a sequence of H floats).
    """
    lib = lib or _get()
    if score_mod is not None:
        mod = MODS[score_mod]
        if window_left is not None or window_right is not None:
            wl = -1 if window_left is None else int(window_left)
            wr = -1 if window_right is None else int(window_right)
        else:
            wl = window - 1 if window > 0 else -1
            wr = 0 if causal else -1
        Hn = q.shape[1]
        slopes_all = torch.zeros(Hn, dtype=torch.float64)
        if mod == 2:
            slopes_all = torch.as_tensor([float(x) for x in alibi_slopes], dtype=torch.float64)
            assert slopes_all.numel() == Hn
        cap = float(softcap)
        cur = {"slopes": slopes_all}

        def call(Qp, Kp, Vp, Op, Lp, B_, H_, rows_p, nrows):
            sl = cur["slopes"].contiguous()
            return lib.oracle_attn_fwd_mod(Qp, Kp, Vp, Op, Lp, B_, H_, Nq, Nk, D, scale64, wl, wr, mod, cap,
                                           sl.data_ptr(), rows_p, nrows, threads)
    elif window_left is not None or window_right is not None:
        wl = -1 if window_left is None else int(window_left)
        wr = -1 if window_right is None else int(window_right)

        def call(Qp, Kp, Vp, Op, Lp, B_, H_, rows_p, nrows):
            return lib.oracle_attn_fwd_window(Qp, Kp, Vp, Op, Lp, B_, H_, Nq, Nk, D, scale64, wl, wr,
                                              rows_p, nrows, threads)
    else:
        def call(Qp, Kp, Vp, Op, Lp, B_, H_, rows_p, nrows):
            return lib.oracle_attn_fwd(Qp, Kp, Vp, Op, Lp, B_, H_, Nq, Nk, D, scale64, int(bool(causal)),
                                       int(window), rows_p, nrows, threads)
    threads = threads or default_threads()
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale64 = float(torch.tensor(scale, dtype=torch.float32))
    if rows is None:
        Q = decode(q, descales[0])
        K = decode(k, descales[1])
        V = decode(v, descales[2])
        O = torch.empty((B, H, Nq, D), dtype=torch.float64)
        LSE = torch.empty((B, H, Nq), dtype=torch.float64)
        rc = call(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), LSE.data_ptr(), B, H, None, 0)
        if rc != 0:
            raise RuntimeError(f"oracle_attn_fwd returned {rc}")
        return O, LSE
    # Sampled rows: decode one head at a time so full-size workloads fit.
    rows = torch.as_tensor(list(rows) if not torch.is_tensor(rows) else rows, dtype=torch.int64)
    O = torch.empty((rows.numel(), D), dtype=torch.float64)
    LSE = torch.empty((rows.numel(),), dtype=torch.float64)
    bh_of = rows // Nq
    for bh in torch.unique(bh_of).tolist():
        sel = (bh_of == bh).nonzero().flatten()
        b, h = divmod(bh, H)
        if score_mod is not None:
            cur["slopes"] = slopes_all[h:h + 1]   # this head's slope, for a one-head call
        Q = decode(q[b, h], descales[0])
        K = decode(k[b, h], descales[1])
        V = decode(v[b, h], descales[2])
        local = (rows[sel] % Nq).contiguous()
        Oh = torch.empty((sel.numel(), D), dtype=torch.float64)
        Lh = torch.empty((sel.numel(),), dtype=torch.float64)
        rc = call(Q.data_ptr(), K.data_ptr(), V.data_ptr(), Oh.data_ptr(), Lh.data_ptr(), 1, 1,
                  local.data_ptr(), local.numel())
        if rc != 0:
            raise RuntimeError(f"oracle_attn_fwd returned {rc}")
        O[sel] = Oh
        LSE[sel] = Lh
    return O, LSE


def attention_bwd(q, k, v, dout, scale, window_left=-1, window_right=-1, threads=None, lib=None,
                  score_mod=None, softcap=0.0, alibi_slopes=None):
    """float64 (dQ, dK, dV) of O = softmax(f(scale Q K^T)) V under the extents mask, given dO.

    q, dout [B,H,Nq,D]; k, v [B,H,Nk,D] (any float dtype, decoded exactly);
    window_left/right as in attention() (-1: open side). scale is used as
    float64(fp32(scale)). score_mod: None, "softcap" or "alibi" as in
    attention() (f the modifier; its derivative enters by the chain rule).
    """
    lib = lib or _get()
    threads = threads or default_threads()
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale64 = float(torch.tensor(scale, dtype=torch.float32))
    Q, K, V, dO = decode(q), decode(k), decode(v), decode(dout)
    dQ = torch.empty((B, H, Nq, D), dtype=torch.float64)
    dK = torch.empty((B, H, Nk, D), dtype=torch.float64)
    dV = torch.empty((B, H, Nk, D), dtype=torch.float64)
    if score_mod is None:
        rc = lib.oracle_attn_bwd(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dO.data_ptr(), dQ.data_ptr(),
                                 dK.data_ptr(), dV.data_ptr(), B, H, Nq, Nk, D, scale64, int(window_left),
                                 int(window_right), threads)
    else:
        mod = MODS[score_mod]
        sl = torch.zeros(max(H, 1), dtype=torch.float64)
        if mod == 2:
            sl = torch.as_tensor([float(x) for x in alibi_slopes], dtype=torch.float64)
            assert sl.numel() == H
        sl = sl.contiguous()
        rc = lib.oracle_attn_bwd_mod(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dO.data_ptr(), dQ.data_ptr(),
                                     dK.data_ptr(), dV.data_ptr(), B, H, Nq, Nk, D, scale64, int(window_left),
                                     int(window_right), mod, float(softcap), sl.data_ptr(), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd returned {rc}")
    return dQ, dK, dV


def visible_keys(i: int, Nq: int, Nk: int, causal: bool, window: int):
    """[lo, hi) of the keys query row i sees (bottom-right causal alignment)."""
    ip = i + (Nk - Nq)
    lo, hi = 0, Nk
    if causal:
        hi = min(Nk, ip + 1)
    if window > 0:
        lo = max(0, ip - window + 1)
    hi = max(hi, 0)
    lo = min(lo, hi)
    return lo, hi


def visible_keys_window(i: int, Nq: int, Nk: int, window_left: int, window_right: int):
    """[lo, hi) of the keys row i sees under the extents mask (negative: open side)."""
    ip = i + (Nk - Nq)
    lo = max(0, ip - window_left) if window_left >= 0 else 0
    hi = min(Nk, ip + window_right + 1) if window_right >= 0 else Nk
    hi = max(hi, 0)
    lo = min(lo, hi)
    return lo, hi


def pair_count_window(Nq: int, Nk: int, window_left: int, window_right: int) -> int:
    """Number of (query, key) pairs the extents mask keeps, per (b, h)."""
    total = 0
    for i in range(Nq):
        lo, hi = visible_keys_window(i, Nq, Nk, window_left, window_right)
        total += hi - lo
    return total


def pair_count(Nq: int, Nk: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs the mask keeps, per (b, h)."""
    total = 0
    for i in range(Nq):
        lo, hi = visible_keys(i, Nq, Nk, causal, window)
        total += hi - lo
    return total
