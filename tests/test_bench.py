"""Host-side logic of bench.py, without a GPU: the visible-pair, FLOP and byte
counts against closed forms and brute force, the kernel-source hash behind the
stored HBM counters, the lookup of those counters, and the one-GPU guard."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_visible_pairs_closed_forms():
    # causal N x N: N(N+1)/2; no mask: Nq*Nk; causal window w keeps the keys
    # i - w < j <= i of row i: min(i + 1, w) of them
    assert bench.visible_pairs(8192, 8192, True, 0) == 8192 * 8193 // 2
    assert bench.visible_pairs(100, 37, False, 0) == 3700
    assert bench.visible_pairs(300, 300, True, 64) == sum(min(i + 1, 64) for i in range(300))


@pytest.mark.parametrize("Nq,Nk,wl,wr", [(50, 70, 5, 3), (70, 50, -1, 0), (33, 33, 0, 0), (40, 90, 10, -1),
                                         (60, 20, -1, -1), (1, 1, 0, 0)])
def test_visible_pairs_of_extents_match_brute_force(Nq, Nk, wl, wr):
    # row i sees the keys [i' - wl, i' + wr], i' = i + Nk - Nq, -1 an open side
    d = Nk - Nq
    want = sum(1 for i in range(Nq) for j in range(Nk)
               if (wl < 0 or j >= i + d - wl) and (wr < 0 or j <= i + d + wr))
    assert bench.visible_pairs_window(Nq, Nk, wl, wr) == want


def test_c3_flops_and_algorithmic_bytes():
    w = synth.WORKLOADS["c3"]
    # two products of 2 D flops per visible pair, 48 heads
    assert bench.flops(w) == 4 * 64 * 48 * (8192 * 8193 // 2) == 412367192064
    # Q, K, V read once and O written once (bf16), the LSE written once (fp32)
    assert bench.algorithmic_bytes(w) == 48 * (4 * 8192 * 64 * 2 + 8192 * 4) == 202899456
    # the backward counts five products per pair
    assert bench.flops_bwd(synth.WORKLOADS["c3bwd"]) == 2.5 * bench.flops(w)


@pytest.fixture
def source_copy(tmp_path, monkeypatch):
    dst = tmp_path / "exact_attention_02_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "exact_attention_02_amd", "csrc"), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.o"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return dst


def test_kernel_hash_follows_code_not_comments(source_copy):
    fwd0, bwd0 = bench.kernel_hash(False), bench.kernel_hash(True)
    f16 = source_copy / "fa_fwd16.hip"
    text = f16.read_text()
    f16.write_text("// a note\n" + text.replace("\n", "\n\n", 3) + "/* more\n   notes */\n")
    assert bench.kernel_hash(False) == fwd0
    f16.write_text(text.replace("SUM_LIMIT = 1024.f", "SUM_LIMIT = 512.f"))
    assert bench.kernel_hash(False) != fwd0
    assert bench.kernel_hash(True) == bwd0          # the backward does not run that file
    api = source_copy / "fa_api.hip"
    api.write_text(api.read_text().replace("return (int)((3LL * n_tiles) / 8);", "return n_tiles / 2;"))
    assert bench.kernel_hash(True) != bwd0          # launch planning counts for both


def test_traffic_is_reported_only_for_the_hashed_build(tmp_path, monkeypatch):
    w = synth.WORKLOADS["c3"]
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({w.name: {"kernel_sha": bench.kernel_hash(False), "hbm_bytes_per_launch": 123}}))
    assert bench.traffic_for(w) == 123
    f.write_text(json.dumps({w.name: {"kernel_sha": "0" * 16, "hbm_bytes_per_launch": 123}}))
    assert bench.traffic_for(w) is None
    f.write_text("not json")
    assert bench.traffic_for(w) is None
    f.unlink()
    assert bench.traffic_for(w) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_roofline_kernel_label_follows_the_launch_plan(name):
    import exact_attention_02_amd as fa
    w = synth.WORKLOADS[name]
    label = bench.kernel_label(w)
    if w.backward:
        assert label.startswith("fa_bwd_")
        return
    kinds = {v: k for k, v in fa.KERNEL_NAMES.items()}
    first = label.split(" + ")[0]
    assert first in kinds
    code = {("f16", "f16"): fa.FA_F16, ("bf16", "bf16"): fa.FA_BF16, ("f16", "f32"): fa.FA_F16_F32OUT,
            ("e4m3", "bf16"): fa.FA_E4M3}[(w.in_dtype, w.out_dtype)]
    mod = {None: 0, "softcap": 1, "alibi": 2}[w.score_mod]
    assert kinds[first] == fa.plan_kernel(w.B, w.H, w.Nq, w.Nk, w.D, code, mod, w.splitkv)
    assert ("fa_combine_kernel" in label) == (w.splitkv and fa.splitkv_num_splits(w.B, w.H, w.Nq, w.Nk, w.D, code) > 1)


def test_host_cores_is_positive_and_within_affinity():
    n = bench.host_cores()
    assert 1 <= n <= len(os.sched_getaffinity(0))
