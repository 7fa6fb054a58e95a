"""The binding loads the library into a process with one HIP runtime.

torch's ROCm build carries its own copy of the HIP runtime. If libfa.so were
loaded before torch, the process would map ROCm's runtime and torch's side by
side, and the library's calls would not see torch's device context. load()
imports torch first; this checks, in a fresh process and in the order that
would go wrong, that only one libamdhip64 is mapped. No GPU is needed.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import re
import exact_attention_02_amd as fa
fa.load()
import torch
maps = open('/proc/self/maps').read()
print(len(set(re.findall(r'\S*libamdhip64\S*', maps))))
"""


def test_library_loaded_before_torch_shares_torchs_hip_runtime():
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout
