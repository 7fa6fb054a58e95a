"""Seeded synthetic inputs for the attention forward workloads.

This module is shared by the tests, the benchmark and the smoke check. It
produces the Q, K, V tensors (and, for e4m3, their per-tensor descales) on the
host; both the CPU oracle and the HIP library then read the very same bytes.
It holds no attention arithmetic.

Generator (a plain statement of a published method):
  * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) used counter-style: word i of stream
    (seed, tensor_id) is mix64(base + (i + 1) * GAMMA), with
    base = mix64(mix64(seed) ^ tensor_id) and GAMMA the golden-ratio constant.
  * Box-Muller in float64: words 2i and 2i+1 give u1 in (0, 1] and u2 in
    [0, 1); the normals are r*cos(2*pi*u2) and r*sin(2*pi*u2) with
    r = sqrt(-2 ln u1).

The pages draw Q, K, V with torch.randn over (B, h, n, d) in their worked
example (page 4, "Where n^2 comes from" and the SDPA listing); these inputs
have that distribution, i.i.d. N(0, 1), but from a counter-based generator so
they are identical across processes, machines and library versions.

Storage dtypes: float16 and bfloat16 are the float64 normals rounded by
torch's conversion; e4m3 inputs follow the per-tensor recipe in
`quantize_e4m3`.
"""
from __future__ import annotations

import math
from typing import Optional
from dataclasses import dataclass, field

import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1

# Tensor ids of the streams (fixed, never tuned).
TID_Q, TID_K, TID_V = 0, 1, 2
TID_OUTLIER_Q, TID_OUTLIER_K, TID_OUTLIER_V = 3, 4, 5
TID_DOUT = 6

E4M3_MAX = 448.0


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _to_i64(x: int) -> int:
    x &= _MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _srl(z: torch.Tensor, n: int) -> torch.Tensor:
    """Logical right shift of int64 lanes holding uint64 bit patterns."""
    return (z >> n) & ((1 << (64 - n)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    # int64 multiplication wraps modulo 2**64, which is the uint64 product.
    z = (z ^ _srl(z, 30)) * _to_i64(_M1)
    z = (z ^ _srl(z, 27)) * _to_i64(_M2)
    return z ^ _srl(z, 31)


def words(seed: int, tensor_id: int, start: int, count: int) -> torch.Tensor:
    """SplitMix64 words start .. start+count-1 of stream (seed, tensor_id), as int64 bit patterns."""
    base = _mix64_int(_mix64_int(seed) ^ tensor_id)
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64)
    z = idx * _to_i64(_GAMMA) + _to_i64(base)
    return _mix64(z)


def uniform53(w: torch.Tensor) -> torch.Tensor:
    """Top 53 bits of each word as a float64 in [0, 1)."""
    return _srl(w, 11).to(torch.float64) * (2.0 ** -53)


_CHUNK = 1 << 24


def normal(seed: int, tensor_id: int, numel: int) -> torch.Tensor:
    """numel i.i.d. N(0, 1) float64 values of stream (seed, tensor_id)."""
    out = torch.empty(numel, dtype=torch.float64)
    npairs = (numel + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        w = words(seed, tensor_id, 2 * p0, 2 * (p1 - p0)).view(-1, 2)
        u1 = 1.0 - uniform53(w[:, 0])          # (0, 1]
        u2 = uniform53(w[:, 1])                # [0, 1)
        r = torch.sqrt(-2.0 * torch.log(u1))
        t = (2.0 * math.pi) * u2
        pair = torch.stack((r * torch.cos(t), r * torch.sin(t)), dim=1).reshape(-1)
        n0 = 2 * p0
        n1 = min(numel, 2 * p1)
        out[n0:n1] = pair[: n1 - n0]
    return out


def uniform(seed: int, tensor_id: int, numel: int) -> torch.Tensor:
    """numel i.i.d. U[0, 1) float64 values of stream (seed, tensor_id)."""
    out = torch.empty(numel, dtype=torch.float64)
    for i0 in range(0, numel, _CHUNK):
        i1 = min(numel, i0 + _CHUNK)
        out[i0:i1] = uniform53(words(seed, tensor_id, i0, i1 - i0))
    return out


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor scaling of a float64 tensor to OCP E4M3FN.

    descale = fp32(amax(|x|) / 448); codes = round-to-nearest-even of
    fp32(x) / descale, clamped to +-448 first (E4M3FN has no infinity; 448 is
    its largest finite value). Returns (codes as torch.float8_e4m3fn, descale
    as a Python float that is exactly an fp32 value).
    """
    amax = float(x.abs().max()) if x.numel() else 1.0
    if amax == 0.0:
        amax = 1.0
    descale = float(torch.tensor(amax / E4M3_MAX, dtype=torch.float32))
    y = x.to(torch.float32) / torch.tensor(descale, dtype=torch.float32)
    y = y.clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), descale


DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "e4m3": torch.float8_e4m3fn,
}


@dataclass
class Workload:
    """One attention forward problem: shapes, mode, storage dtypes and seed."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    causal: bool
    window: int          # 0 = no window; w > 0 keeps keys j with i - w < j <= i
    in_dtype: str        # "f16" | "bf16" | "e4m3"
    out_dtype: str       # "f32" | "f16" | "bf16"
    seed: int
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    scale: float = field(default=0.0)
    # The mask as key extents instead of (causal, window): row i keeps keys
    # [i' - window_left, i' + window_right], i' = i + Nk - Nq, -1 an open side.
    window_left: Optional[int] = None
    window_right: Optional[int] = None
    # Score modifier: None, "softcap" (s <- softcap * tanh(s / softcap)) or
    # "alibi" (s <- s + slope_h * (j - i') with the slopes alibi_slopes(H)).
    score_mod: Optional[str] = None
    softcap: float = 0.0
    splitkv: bool = False   # run through split-KV with the recommended split count
    backward: bool = False  # the workload is the backward pass (dQ, dK, dV given dO)

    def __post_init__(self):
        if self.scale == 0.0:
            # 1/sqrt(D) rounded to fp32: both sides receive this fp32 value.
            self.scale = float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def delta(self) -> int:
        return self.Nk - self.Nq


# The five workloads: shapes, modes and dtypes of the attention forward
# configurations this library is measured on. Seeds are the workload numbers.
WORKLOADS = {
    "c1": Workload("c1_noncausal_B1H1N128D64_f16_f32out", 1, 1, 128, 128, 64, False, 0, "f16", "f32", 1),
    "c2": Workload("c2_causal_B4H12N1024D64_f16", 4, 12, 1024, 1024, 64, True, 0, "f16", "f16", 2),
    "c3": Workload("c3_causal_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16", "bf16", 3),
    "c4c": Workload("c4_causal_B1H32N32768D128_bf16", 1, 32, 32768, 32768, 128, True, 0, "bf16", "bf16", 4),
    "c4w": Workload("c4_window4096_B1H32N32768D128_bf16", 1, 32, 32768, 32768, 128, True, 4096, "bf16", "bf16", 4),
    "c5": Workload("c5_noncausal_B4H16N8192D128_e4m3", 4, 16, 8192, 8192, 128, False, 0, "e4m3", "bf16", 5,
                   outlier_frac=0.001, outlier_mult=20.0),
    # The sliding window |i - j| <= w of the sparse-attention-patterns section
    # at c3's shape, w = 1024 (the page's example uses w = n / 8).
    "c3sw": Workload("c3_slidingwindow1024_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, False, 0, "bf16", "bf16", 3,
                     window_left=1024, window_right=1024),
    # c3 with FLASHLIGHT's score_mod variants: softcap (cap 50) and ALiBi.
    "c3sc": Workload("c3_causal_softcap50_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16", "bf16", 3,
                     score_mod="softcap", softcap=50.0),
    "c3al": Workload("c3_causal_alibi_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16", "bf16", 3,
                     score_mod="alibi"),
    # Decode: one new query per sequence against a long context (LLaMa-3.2-1B
    # serving: 32 heads of 64), run with split-KV. Seed 6.
    "c6": Workload("c6_decode_B8H32Nq1Nk16384D64_bf16", 8, 32, 1, 16384, 64, True, 0, "bf16", "bf16", 6,
                   splitkv=True),
    # The backward pass at c3's shape: dQ, dK, dV of the causal forward given
    # an upstream gradient dO (make_grad_out), O and the LSE.
    "c3bwd": Workload("c3_backward_causal_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16", "bf16", 3,
                      backward=True),
    # The backward of the softcap and ALiBi workloads.
    "c3scbwd": Workload("c3_backward_causal_softcap50_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16",
                        "bf16", 3, score_mod="softcap", softcap=50.0, backward=True),
    "c3albwd": Workload("c3_backward_causal_alibi_B4H12N8192D64_bf16", 4, 12, 8192, 8192, 64, True, 0, "bf16", "bf16",
                        3, score_mod="alibi", backward=True),
}


def alibi_slopes(H: int):
    """The geometric ALiBi slopes 2^(-8 (h+1) / H), h = 0 .. H-1 (an input of the alibi workloads)."""
    return [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    descale_q: float = 1.0
    descale_k: float = 1.0
    descale_v: float = 1.0


def make_inputs(w: Workload) -> Inputs:
    """Q [B,H,Nq,D], K and V [B,H,Nk,D] on the host, contiguous, in w.in_dtype."""
    shapes = {TID_Q: (w.B, w.H, w.Nq, w.D), TID_K: (w.B, w.H, w.Nk, w.D), TID_V: (w.B, w.H, w.Nk, w.D)}
    outl = {TID_Q: TID_OUTLIER_Q, TID_K: TID_OUTLIER_K, TID_V: TID_OUTLIER_V}
    out = {}
    descales = {}
    for tid, shp in shapes.items():
        n = shp[0] * shp[1] * shp[2] * shp[3]
        x = normal(w.seed, tid, n)
        if w.outlier_frac > 0.0:
            hit = uniform(w.seed, outl[tid], n) < w.outlier_frac
            x = torch.where(hit, x * w.outlier_mult, x)
        x = x.view(shp)
        if w.in_dtype == "e4m3":
            codes, ds = quantize_e4m3(x)
            out[tid] = codes.contiguous()
            descales[tid] = ds
        else:
            out[tid] = x.to(DTYPES[w.in_dtype]).contiguous()
            descales[tid] = 1.0
        del x
    return Inputs(out[TID_Q], out[TID_K], out[TID_V], descales[TID_Q], descales[TID_K], descales[TID_V])


def make_grad_out(w: Workload) -> torch.Tensor:
    """The upstream gradient dO [B,H,Nq,D] of a backward workload: i.i.d.
    N(0, 1) from stream (seed, TID_DOUT), on the host, in w.in_dtype."""
    shp = (w.B, w.H, w.Nq, w.D)
    return normal(w.seed, TID_DOUT, w.B * w.H * w.Nq * w.D).view(shp).to(DTYPES[w.in_dtype]).contiguous()


def small_workload(name, B, H, Nq, Nk, D, causal, window, in_dtype, out_dtype, seed,
                   outlier_frac=0.0, outlier_mult=1.0, window_left=None, window_right=None,
                   score_mod=None, softcap=0.0, backward=False) -> Workload:
    """A workload of the same recipe at other sizes (parity and edge cases)."""
    return Workload(name, B, H, Nq, Nk, D, causal, window, in_dtype, out_dtype, seed,
                    outlier_frac=outlier_frac, outlier_mult=outlier_mult,
                    window_left=window_left, window_right=window_right, score_mod=score_mod, softcap=softcap,
                    backward=backward)
