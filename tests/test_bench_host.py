"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic bytes the roofline divides by, and the rule that the measured
traffic is reported only for the kernel sources it was taken on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# Llama-3-8B linear stack: (name, N, K, per-128-group activation scales)
SHAPES = [("qkv", 6144, 4096, False), ("o_proj", 4096, 4096, True),
          ("gate_up", 28672, 4096, False), ("down", 4096, 14336, False)]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _stack(layers):
    s = bench.Stack.__new__(bench.Stack)          # the byte counts need no tensors
    s.linears = [(n, N, K, 128 if g else 0) for (n, N, K, g) in SHAPES]
    s.layers = layers
    return s


def test_algorithmic_bytes_per_launch():
    # counted here launch by launch: a draft launch (M = 1, fused) reads the
    # hi plane, the fp16 scales and the fp32 row, writes the int8 codes, the
    # activation scale(s) and y; a verify launch (M = 4, after its own
    # quantisation) reads both planes, the scales, 4 rows of codes and their
    # scales, and writes y
    total, launches = 0, 0
    for (_, N, K, g) in SHAPES:
        groups = K // 128
        n_scales = groups if g else 1
        draft = N * K // 2 + 2 * N * groups + 4 * K + K + 4 * n_scales + 4 * N
        verify = 2 * (N * K // 2) + 2 * N * groups + 4 * K + 4 * 4 * n_scales + 4 * 4 * N
        total += 3 * draft + verify
        launches += 4
    s = _stack(32)
    assert s.gemv_launches_per_round() == 32 * launches
    assert s.gemv_algorithmic_bytes_per_round() == 32 * total
    assert int(s.gemv_algorithmic_bytes_per_round() / s.gemv_launches_per_round()) == 35037629
    # plane bytes of the round: three hi-only passes and one hi+lo pass
    assert s.plane_bytes_per_round() == 32 * 5 * sum(N * K // 2 for (_, N, K, _) in SHAPES)


def test_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    src_json = os.path.join(ROOT, "profiles", "gemv_planes_round_traffic.json")
    with open(src_json) as f:
        prof = json.load(f)
    for rel in prof["sources"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copyfile(os.path.join(ROOT, rel), dst)
    (tmp_path / "profiles").mkdir()
    shutil.copyfile(src_json, tmp_path / "profiles" / "gemv_planes_round_traffic.json")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == prof["traffic_bytes_per_launch"]
    changed = tmp_path / prof["sources"][0]
    changed.write_bytes(changed.read_bytes() + b"\n")
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("gpus", ["0", "8"])
def test_gpu_count_other_than_one_exits_before_touching_a_gpu(gpus):
    assert bench.main(["--gpus", gpus]) == 2
