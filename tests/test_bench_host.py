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
    # activation scale(s) and y; a verify launch (M = 4) reads both planes
    # and the scales and writes y, and either quantises in the same launch
    # (K <= 4096 and N <= 8192: reads 4 fp32 rows, writes their codes and
    # scales) or reads the codes and scales of its own earlier quantisation
    # launch (gate_up, down)
    total, launches = 0, 0
    for (_, N, K, g) in SHAPES:
        groups = K // 128
        n_scales = groups if g else 1
        draft = N * K // 2 + 2 * N * groups + 4 * K + K + 4 * n_scales + 4 * N
        verify = 2 * (N * K // 2) + 2 * N * groups + 4 * 4 * N
        if K <= 4096 and N <= 8192:
            verify += 4 * 4 * K + 4 * K + 4 * 4 * n_scales
        else:
            verify += 4 * K + 4 * 4 * n_scales
        total += 3 * draft + verify
        launches += 4
    s = _stack(32)
    assert s.gemv_launches_per_round() == 32 * launches
    assert s.gemv_algorithmic_bytes_per_round() == 32 * total
    assert int(s.gemv_algorithmic_bytes_per_round() / s.gemv_launches_per_round()) == 35045821
    # the whole round adds the quantisation launches of the verify calls that
    # take two launches (gate_up, down): 4 fp32 rows read, codes and scales
    # written
    quant = sum(4 * 4 * K + 4 * K + 4 * 4 * (K // 128 if g else 1)
                for (_, N, K, g) in SHAPES if not (K <= 4096 and N <= 8192))
    assert s.algorithmic_bytes_per_round() == 32 * (total + quant)
    # plane bytes of the round: three hi-only passes and one hi+lo pass
    assert s.plane_bytes_per_round() == 32 * 5 * sum(N * K // 2 for (_, N, K, _) in SHAPES)


def test_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    # a profile recorded with the hash of the sources it was taken on: its
    # traffic is reported while they are unchanged, and not after an edit
    import hashlib
    src_json = os.path.join(ROOT, "profiles", "gemv_planes_round_traffic.json")
    with open(src_json) as f:
        prof = json.load(f)
    h = hashlib.sha256()
    for rel in prof["sources"]:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copyfile(os.path.join(ROOT, rel), dst)
        h.update(dst.read_bytes())
    prof["sources_sha256"] = h.hexdigest()
    (tmp_path / "profiles").mkdir()
    with open(tmp_path / "profiles" / "gemv_planes_round_traffic.json", "w") as f:
        json.dump(prof, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == prof["traffic_bytes_per_launch"]
    changed = tmp_path / prof["sources"][0]
    changed.write_bytes(changed.read_bytes() + b"\n")
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("gpus", ["0", "8"])
def test_gpu_count_other_than_one_exits_before_touching_a_gpu(gpus):
    assert bench.main(["--gpus", gpus]) == 2


def test_cold_weight_cycles_cover_the_requested_bytes():
    # the stack's layers first, then extra seeded layers of the same shape,
    # until the plane bytes of the cycle reach the requested amount
    import bench
    from w8_quantized_linear_amd import synth
    st = bench.Stack.__new__(bench.Stack)
    st.linears = [("a", 8, 256, 0), ("b", 16, 128, 0)]
    st.layers, st.seed, st.device, st.extra = 2, 5, "cpu", {}
    st.w = [[synth.make_weights(N, K, seed=5, layer=l, linear=i) for i, (_, N, K, _) in enumerate(st.linears)]
            for l in range(2)]
    one = 8 * 256 // 2
    ws = st.cold_weights(0, 1, at_least=5 * one)
    assert len(ws) == 5 and ws[0] is st.w[0][0] and ws[1] is st.w[1][0]
    assert len({w.hi.data_ptr() for w in ws}) == 5
    extra = synth.make_weights(8, 256, seed=5, layer=2, linear=0)
    assert (ws[2].hi == extra.hi).all() and (ws[2].scale == extra.scale).all()
    # target cycles count both planes; the extra layers are reused
    wt = st.cold_weights(0, 2, at_least=5 * one)
    assert len(wt) == 3 and wt[2] is ws[2]
    assert len(st.cold_weights(1, 1, at_least=1)) == 1
