"""Benchmark of the fused attention forward on one MI355X.

Default workload: causal self-attention forward, B=4 H=12 N=8192 D=64, bf16
inputs and output, fp32 LSE -- the worked shape of the pages (inskillml course
module 9). A step is one fa_fwd call over the whole batch, inputs resident in
HBM. Prints one JSON line:

  value      algorithmic TFLOP/s = 4*D*B*H*(visible query-key pairs) / time
             (two products of 2*D flops per visible pair: Q K^T and P V)
  roofline   the kernel against the dense bf16 MFMA peak (2516.6 TFLOP/s =
             256 CU x 2.4 GHz x 4096 flop/CU/clk), timed with HIP events on
             the launch stream; traffic = HBM bytes per launch from rocprofv3
             FETCH_SIZE/WRITE_SIZE counters (profiles/), when the kernel source
             is the one those counters were taken on
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
             workload's rows, on this host's cores (reported, not a target)

The backward workload (--workload c3bwd) times one fa_bwd call (its three
kernels) given O and the LSE of one earlier forward call: 10*D flops per
visible pair (the recomputed Q K^T, dO V^T, P^T dO, dS K and dS^T Q).
"""
import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2}
HBM_PEAK_GBS = 8000.0
METRIC = "attention fwd TFLOPS + % MFMA peak, B4 H12 N8192 D64 causal bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def visible_pairs(Nq, Nk, causal, window):
    """Visible (query, key) pairs per (batch, head)."""
    import numpy as np
    i = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    hi = np.minimum(i + 1, Nk) if causal else np.full(Nq, Nk, dtype=np.int64)
    lo = np.maximum(i - window + 1, 0) if window > 0 else np.zeros(Nq, dtype=np.int64)
    return int(np.clip(hi - lo, 0, None).sum())


def visible_pairs_window(Nq, Nk, wl, wr):
    """Visible pairs per (batch, head) when row i keeps keys [i' - wl, i' + wr] (-1: open side)."""
    import numpy as np
    i = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    lo = np.maximum(i - wl, 0) if wl >= 0 else np.zeros(Nq, dtype=np.int64)
    hi = np.minimum(i + wr + 1, Nk) if wr >= 0 else np.full(Nq, Nk, dtype=np.int64)
    return int(np.clip(hi - lo, 0, None).sum())


def pairs(w):
    if w.window_left is not None or w.window_right is not None:
        return visible_pairs_window(w.Nq, w.Nk, -1 if w.window_left is None else w.window_left,
                                    -1 if w.window_right is None else w.window_right)
    return visible_pairs(w.Nq, w.Nk, w.causal, w.window)


def flops(w):
    return 4.0 * w.D * w.B * w.H * pairs(w)


def flops_bwd(w):
    return 10.0 * w.D * w.B * w.H * pairs(w)


def algorithmic_bytes(w):
    eb = {"f16": 2, "bf16": 2, "e4m3": 1}[w.in_dtype]
    ob = {"f32": 4, "f16": 2, "bf16": 2}[w.out_dtype]
    n_bh = w.B * w.H
    return n_bh * (w.Nq * w.D * eb + 2 * w.Nk * w.D * eb + w.Nq * w.D * ob + w.Nq * 4)


# The sources that decide what a workload's kernels do: the kernels, their
# headers and the launch planning (tile shapes, workgroup order) in fa_api.hip.
FWD_SOURCES = ("fa_fwd.hip", "fa_fwd16.hip", "fa_fwd_ks.hip", "fa_fwd_serial.hip", "fa_serial.h", "fa_fwd_serial_inst.hip",
               "fa_device.h", "fa_sched.h", "fa_launch.h",
               "fa_api.hip")
BWD_SOURCES = ("fa_bwd.hip", "fa_device.h", "fa_sched.h", "fa_launch.h", "fa_api.hip")


def _code_only(text):
    """C++ source without comments, whitespace collapsed: an edit of a comment
    leaves the kernels, and so the hash, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_hash(backward=False):
    """Hash of the code of the kernel sources a workload runs (the forward's or
    the backward's), comments and layout ignored."""
    h = hashlib.sha256()
    for name in (BWD_SOURCES if backward else FWD_SOURCES):
        with open(os.path.join(ROOT, "exact_attention_02_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(w):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(w.name)
    if not e or e.get("kernel_sha") != kernel_hash(w.backward):
        return None
    return e.get("hbm_bytes_per_launch")


def host_cores():
    """The cores this process may run on: sched_getaffinity, capped by a cgroup CPU quota if one is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n)


def cpu_baseline(w, inp, target_s=15.0):
    """The oracle, as it is, on random rows of the workload, scaled to TFLOP/s."""
    import torch
    import oracle
    import synth
    threads = host_cores()
    g = torch.Generator().manual_seed(1234)
    n_rows_total = w.B * w.H * w.Nq

    ext = w.window_left is not None or w.window_right is not None
    wl = -1 if w.window_left is None else w.window_left
    wr = -1 if w.window_right is None else w.window_right
    mask = dict(window_left=wl, window_right=wr) if ext else {}
    if w.score_mod is not None:
        mask.update(score_mod=w.score_mod, softcap=w.softcap,
                    alibi_slopes=synth.alibi_slopes(w.H) if w.score_mod == "alibi" else None)

    def row_pairs(rows):
        i = rows % w.Nq + (w.Nk - w.Nq)
        if ext:
            lo = torch.clamp(i - wl, min=0) if wl >= 0 else torch.zeros_like(i)
            hi = torch.clamp(i + wr + 1, max=w.Nk) if wr >= 0 else torch.full_like(i, w.Nk)
        else:
            hi = torch.clamp(i + 1, max=w.Nk) if w.causal else torch.full_like(i, w.Nk)
            lo = torch.clamp(i - w.window + 1, min=0) if w.window > 0 else torch.zeros_like(i)
        return int(torch.clamp(hi - lo, min=0).sum())

    n = 256
    while True:
        rows = torch.randint(0, n_rows_total, (n,), generator=g)
        t0 = time.perf_counter()
        oracle.attention(inp.q, inp.k, inp.v, w.scale, w.causal, w.window,
                         descales=(inp.descale_q, inp.descale_k, inp.descale_v), rows=rows, threads=threads,
                         **mask)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= n_rows_total:
            pr = row_pairs(rows)
            fl = 4.0 * w.D * pr
            if w.splitkv:
                # the metric's unit: algorithmic bytes (each row's visible K and V
                # rows, its q, o and LSE) per second
                eb = {"f16": 2, "bf16": 2, "e4m3": 1}[w.in_dtype]
                ob = {"f32": 4, "f16": 2, "bf16": 2}[w.out_dtype]
                nb = 2.0 * w.D * eb * pr + n * (w.D * eb + w.D * ob + 4)
                return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                        "sample": f"{n} random query rows of the workload ({nb / 1e9:.2f} GB of K, V, q, o and "
                                  f"LSE), float64, {dt:.1f} s wall"}
            return {"value": fl / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
                    "sample": f"{n} random query rows of the workload ({fl / 1e9:.1f} GFLOP), float64, "
                              f"{dt:.1f} s wall"}
        n = min(n_rows_total, max(2 * n, int(n * target_s / max(dt, 1e-3))))


def cpu_baseline_bwd(w, inp, dout, target_s=15.0):
    """The oracle's backward, as it is, on whole heads of the workload, scaled to TFLOP/s."""
    import oracle
    import synth
    threads = host_cores()
    wl = -1 if w.window_left is None else w.window_left
    wr = -1 if w.window_right is None else w.window_right
    if w.window_left is None and w.window_right is None:
        wl, wr = (w.window - 1 if w.window > 0 else -1), (0 if w.causal else -1)
    n_heads, spent = 0, 0.0
    while spent < 0.5 * target_s and n_heads < w.B * w.H:
        b, h = divmod(n_heads, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        om = {}
        if w.score_mod is not None:
            om = dict(score_mod=w.score_mod, softcap=w.softcap,
                      alibi_slopes=[synth.alibi_slopes(w.H)[h]] if w.score_mod == "alibi" else None)
        oracle.attention_bwd(inp.q[sl], inp.k[sl], inp.v[sl], dout[sl], w.scale, wl, wr, threads=threads, **om)
        spent += time.perf_counter() - t0
        n_heads += 1
    fl = 10.0 * w.D * n_heads * visible_pairs_window(w.Nq, w.Nk, wl, wr)
    return {"value": fl / spent / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{n_heads} whole (batch, head) slices of the workload ({fl / 1e9:.1f} GFLOP), float64, "
                      f"{spent:.1f} s wall"}


def kernel_label(w):
    """The kernels one step launches, from the library's launch plan."""
    import exact_attention_02_amd as fa
    if w.backward:
        return "fa_bwd_rowstat_kernel + fa_bwd_dq_kernel + fa_bwd_dkdv_kernel (one call)"
    code = {("f16", "f16"): fa.FA_F16, ("bf16", "bf16"): fa.FA_BF16, ("f16", "f32"): fa.FA_F16_F32OUT,
            ("e4m3", "bf16"): fa.FA_E4M3, ("bf16", "f32"): fa.FA_BF16_F32OUT}[(w.in_dtype, w.out_dtype)]
    mod = {None: fa.FA_MOD_NONE, "softcap": fa.FA_MOD_SOFTCAP, "alibi": fa.FA_MOD_ALIBI}[w.score_mod]
    name = fa.KERNEL_NAMES[fa.plan_kernel(w.B, w.H, w.Nq, w.Nk, w.D, code, mod, w.splitkv)]
    if w.splitkv and fa.splitkv_num_splits(w.B, w.H, w.Nq, w.Nk, w.D, code) > 1:
        name += " + fa_combine_kernel"
    return name


def timed_launches(step, stream, n, between=None):
    """Per-launch times (ms) of n launches, each bracketed by HIP events on the
    launch stream; `between` runs before each launch, outside its events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        if between is not None:
            between()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def measured_clock_ghz(step, n_launches, n_wg):
    """Mean shader clock during the kernel, from its own workgroups: with
    fa_set_clock_telemetry on, each workgroup records the shader-clock and the
    100 MHz counters at its start and end. The clock of each launch is the sum
    of its workgroups' shader-clock advances over the sum of their 100 MHz
    advances; the median over n_launches launches is returned."""
    import torch
    import exact_attention_02_amd as fa
    dev = torch.device("cuda:0")
    buf = torch.zeros(n_launches, 4 * n_wg, dtype=torch.int64, device=dev)
    clocks = []
    torch.cuda.synchronize()
    try:
        for i in range(n_launches):
            st = fa.fa_set_clock_telemetry(buf[i].data_ptr(), n_wg)
            if st != fa.FA_OK:
                raise fa.FaError(st, "fa_set_clock_telemetry")
            step()
        torch.cuda.synchronize()
    finally:
        fa.fa_set_clock_telemetry(None, 0)
    v = buf.view(n_launches, n_wg, 4).cpu().double()
    for i in range(n_launches):
        cyc, ticks = (v[i, :, 2] - v[i, :, 0]).sum().item(), (v[i, :, 3] - v[i, :, 1]).sum().item()
        if ticks > 0:
            clocks.append(cyc / ticks * 0.1)
    clocks.sort()
    return clocks[len(clocks) // 2] if clocks else None


def launch_trace(step, stream, n, w, in_t, out_t, n_splits):
    """The first n launches of the process, one event pair each, with the
    shader clock of each from the kernel's own telemetry (the clock records
    of measured_clock_ghz). Under sustained load the part's power management
    moves the clock over the first launches; this shows where and by how much."""
    import torch
    import exact_attention_02_amd as fa
    dev = torch.device("cuda:0")
    code = fa.dtype_code(in_t, out_t)
    n_wg = max(1, 4 * fa.plan_grid(w.B, w.H, w.Nq, w.Nk, w.D, True, 0, code)[0] * max(1, n_splits))
    buf = torch.zeros(n, 4 * n_wg, dtype=torch.int64, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    try:
        for i in range(n):
            st = fa.fa_set_clock_telemetry(buf[i].data_ptr(), n_wg)
            if st != fa.FA_OK:
                raise fa.FaError(st, "fa_set_clock_telemetry")
            evs[i][0].record(stream)
            step()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
    finally:
        fa.fa_set_clock_telemetry(None, 0)
    v = buf.view(n, n_wg, 4).cpu().double()
    us, ghz = [], []
    for i in range(n):
        us.append(round(evs[i][0].elapsed_time(evs[i][1]) * 1000.0, 1))
        cyc, ticks = (v[i, :, 2] - v[i, :, 0]).sum().item(), (v[i, :, 3] - v[i, :, 1]).sum().item()
        ghz.append(round(cyc / ticks * 0.1, 3) if ticks > 0 else None)

    def mean(a, b):
        x = us[a:b]
        return round(sum(x) / len(x), 1) if x else None
    return {"workload": w.name, "launches": n, "us": us, "shader_ghz": ghz,
            "mean_us": {"1-5": mean(0, 5), "6-25": mean(5, 25), "26-45": mean(25, 45), "46-": mean(45, n)},
            "note": "launch i of a fresh process: HIP event pair on the launch stream; clock from the kernel's "
                    "per-workgroup clock records (fa_set_clock_telemetry)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The shader clock keeps settling over about the first 100 launches of a
    # fresh process (c3 measures 881 TFLOP/s over launches 11-60 and 950 over
    # launches 101-300), so the default timed region starts after that.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c3", help="c1 c2 c3 c4c c4w c5 c3sw c3sc c3al c6 c3bwd c3scbwd c3albwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true", help="skip the shader-clock pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device-to-device copy (to scale the FETCH_SIZE/WRITE_SIZE "
                         "counters of a profiler run)")
    ap.add_argument("--launch-trace", type=int, default=0, metavar="N",
                    help="instead of the bench line: time each of the first N launches of this process "
                         "(an event pair each) with the shader clock each ran at, and print them (forward "
                         "workloads)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                                   "(sharding the heads across GPUs is not implemented)"}))
        sys.exit(2)

    import torch
    import exact_attention_02_amd as fa
    import synth

    if args.copy_calibration:
        n = 512 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))
        return

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    out_t = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.out_dtype]
    o = torch.empty((w.B, w.H, w.Nq, w.D), dtype=out_t, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    descales = (inp.descale_q, inp.descale_k, inp.descale_v) if w.in_dtype == "e4m3" else None
    stream = torch.cuda.current_stream(dev)
    mod = {}
    if w.score_mod is not None:
        mod = dict(score_mod=w.score_mod, softcap=w.softcap)
        if w.score_mod == "alibi":
            mod["alibi"] = torch.tensor(synth.alibi_slopes(w.H), dtype=torch.float32, device=dev)
    n_splits = 1
    if w.splitkv:
        code = fa.dtype_code(q.dtype, out_t)
        n_splits = fa.splitkv_num_splits(w.B, w.H, w.Nq, w.Nk, w.D, code)
        ws = torch.empty(max(16, fa.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.D, n_splits)), dtype=torch.uint8,
                         device=dev)
        mod = dict(num_splits=n_splits, workspace=ws)

    def step():
        fa.attention(q, k, v, scale=w.scale, causal=w.causal, window=w.window, out=o, lse=lse,
                     window_left=w.window_left, window_right=w.window_right, **mod,
                     descales=descales, stream=stream.cuda_stream)

    if w.backward:
        # O and the LSE come from one forward call outside the timed region.
        step()
        dout = synth.make_grad_out(w)
        do_d = dout.to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_b = torch.empty(max(16, fa.bwd_workspace_bytes(w.B, w.H, w.Nq)), dtype=torch.uint8, device=dev)

        bmod = {}
        if w.score_mod is not None:
            bmod = dict(score_mod=w.score_mod, softcap=w.softcap, alibi=mod.get("alibi"))

        def step():
            fa.attention_bwd(q, k, v, o, lse, do_d, scale=w.scale, causal=w.causal,
                             window_left=w.window_left, window_right=w.window_right,
                             dq=dq, dk=dk, dv=dv, workspace=ws_b, stream=stream.cuda_stream, **bmod)

    if args.launch_trace > 0 and not w.backward:
        print(json.dumps(launch_trace(step, stream, args.launch_trace, w, q.dtype, out_t, n_splits)), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps

    # After the timed region (which alone gives `value`): per-launch times of
    # as many launches again, a cold-cache pass with a 512 MiB write between
    # launches, and the shader clock measured beside the kernel.
    per = timed_launches(step, stream, args.steps)
    per_sorted = sorted(per)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = sorted(timed_launches(step, stream, max(3, min(args.steps, 20)), between=lambda: scratch.fill_(1)))
    del scratch
    clock = None
    if not args.no_clock and not w.backward:
        import exact_attention_02_amd as fa_
        code = fa_.dtype_code(q.dtype, out_t)
        # records for every workgroup with room to spare (unused records stay zero and add nothing)
        n_wg = 4 * fa_.plan_grid(w.B, w.H, w.Nq, w.Nk, w.D, True, 0, code)[0] * max(1, n_splits)
        clock = measured_clock_ghz(step, max(8, min(args.steps, 40)), max(1, n_wg))

    fl = flops(w)
    tflops = fl / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_dtype]
    res = {
        "metric": METRIC if args.workload == "c3" else f"attention fwd TFLOPS, {w.name}",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "window": w.window, "window_left": w.window_left,
                   "window_right": w.window_right, "score_mod": w.score_mod, "softcap": w.softcap,
                   "in": w.in_dtype, "out": w.out_dtype,
                   "parallelism": "single GPU"},
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic_for(w),
                     "kernel": kernel_label(w), "flop_per_launch": fl,
                     "algorithmic_hbm_bytes": algorithmic_bytes(w),
                     "timing": "HIP events on the launch stream, mean over the timed steps"},
        "wall_s_timed_region": round(wall, 4),
        "per_launch_ms": {"mean": round(sum(per) / len(per), 5), "median": round(per_sorted[len(per) // 2], 5),
                          "min": round(per_sorted[0], 5), "launches": len(per),
                          "note": "one event pair per launch, after the timed region"},
        "cold_cache_ms": {"median": round(cold[len(cold) // 2], 5), "min": round(cold[0], 5), "launches": len(cold),
                          "note": "a 512 MiB device write before each launch, outside its events"},
    }
    if clock is not None:
        peak_at_clock = peak * clock / 2.4
        # A launch takes the same number of shader cycles whatever the clock
        # (--launch-trace), so the timed region's mean clock follows from the
        # cycles of a launch after it and the timed mean duration.
        timed_ghz = clock * res["per_launch_ms"]["median"] / ms
        res["clock"] = {"shader_ghz": round(clock, 3), "nominal_ghz": 2.4,
                        "peak_at_clock": round(peak_at_clock, 1),
                        "frac_at_clock": round(tflops / peak_at_clock, 4),
                        "note": "median over launches after the timed region; each launch's workgroups record "
                                "the shader-clock and 100 MHz counters at their start and end "
                                "(fa_set_clock_telemetry)",
                        "timed_region_ghz_est": round(timed_ghz, 3),
                        "frac_at_timed_region_clock_est": round(tflops / (peak * timed_ghz / 2.4), 4),
                        "timed_region_note": "shader_ghz x the per-launch median duration / ms_per_step: the "
                                             "cycles of one launch after the timed region over the timed "
                                             "region's mean launch time"}
    if w.splitkv:
        # A decode step reads the whole K/V once for a handful of queries: HBM
        # bound. The time covers both kernels of the call (splits and merge).
        gbs = algorithmic_bytes(w) / (ms * 1e-3) / 1e9
        res.update({
            "metric": f"attention decode GB/s (algorithmic HBM bytes / time), {w.name}",
            "value": round(gbs, 1), "unit": "GB/s", "num_splits": n_splits,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(w),
                         "kernel": kernel_label(w),
                         "algorithmic_hbm_bytes": algorithmic_bytes(w), "flop_per_launch": fl,
                         "timing": "HIP events on the launch stream, mean over the timed steps"},
        })
        res.pop("pct_mfma_peak", None)
        res.pop("clock", None)
    if w.backward:
        fl = flops_bwd(w)
        tflops = fl / (ms * 1e-3) / 1e12
        res.update({
            "metric": f"attention bwd TFLOPS (10*D flops per visible pair / time), {w.name}",
            "value": round(tflops, 2), "pct_mfma_peak": round(100.0 * tflops / peak, 2),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(tflops / peak, 4), "traffic": traffic_for(w),
                         "kernel": kernel_label(w),
                         "flop_per_launch": fl,
                         "timing": "HIP events on the launch stream, mean over the timed steps"},
        })
    if not args.no_cpu_baseline and w.backward:
        res["cpu_baseline"] = cpu_baseline_bwd(w, inp, dout)
    elif not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
