"""Builds libfa.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Each source compiles to its own object in parallel, then one link step."""
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_fwd.hip", "fa_fwd16.hip", "fa_fwd_ks.hip", "fa_fwd_serial.hip", "fa_bwd.hip", "fa_api.hip"]
# The serial forward kernel's instantiation sets: fa_fwd_serial_inst.hip once
# per (input type, score modifier), as FA_SR_IN and FA_SR_MOD (fa_launch.h);
# e4m3 inputs (2) take no modifier.
SERIAL_SETS = [(i, m) for i in (0, 1) for m in (0, 1, 2)] + [(2, 0)]

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32.
HIPFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(out: str = LIB, extra=()) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    jobs = max(1, min(len(SOURCES) + len(SERIAL_SETS), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc, *HIPFLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        for i, m in SERIAL_SETS:
            o = os.path.join(tmpd, f"fa_fwd_serial_inst_{i}_{m}.o")
            objs.append(o)
            cmds.append([hipcc, *HIPFLAGS, *extra, f"-DFA_SR_IN={i}", f"-DFA_SR_MOD={m}", "-c", "-o", o,
                         os.path.join(CSRC, "fa_fwd_serial_inst.hip")])
        # the slowest compiles first
        cmds.sort(key=lambda c: 0 if "fa_fwd_serial_inst.hip" in c[-1] or c[-1].endswith(("fa_fwd16.hip", "fa_bwd.hip")) else 1)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out
