"""The benchmark's output contract, on the GPU: bench.py run end to end on a
two-layer stack (a child process, small settings) prints one JSON line with
the metric, the round's timing, the roofline of the linear kernel, the read
ceiling, the per-linear timings against it, and the CPU baseline (all host
threads and one)."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_prints_the_contract_line():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--layers", "2", "--steps", "2", "--warmup", "1",
           "--cpu-seconds", "0.2", "--no-r4", "--no-pack", "--no-accept", "--no-kv", "--verify-batches", "8"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=110)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    out = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict), ("read_ceiling", dict), ("per_linear", dict)):
        assert isinstance(out[key], kind), key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["vs_baseline"] is None
    assert "workload" in out["config"] and out["config"]["layers"] == 2
    assert out["config"]["algorithmic_bytes_per_round"] > out["config"]["plane_bytes_per_round"]
    assert out["algorithmic_GBps"] > out["value"]
    roof = out["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    assert cpu["one_thread"]["cores"] == 1 and cpu["one_thread"]["value"] > 0
    ceil = out["read_ceiling"]
    assert set(ceil) == {"8MiB", "12MiB", "16MiB", "24MiB", "28MiB", "56MiB", "112MiB", "2048MiB"}
    assert all(v["GBps"] > 0 and 0 < v["frac"] < 1 for v in ceil.values())
    lin = out["per_linear"]
    assert set(lin) == {"draft_M1", "target_M1", "target_M4", "quant_M4", "verify_M4"}
    for mode in ("draft_M1", "target_M1", "target_M4"):
        assert set(lin[mode]) == {"qkv", "o_proj", "gate_up", "down"}
        for v in lin[mode].values():
            assert v["us"] > 0 and v["cold_set"]["plane_bytes"] >= 512 << 20
            assert 0 < v["of_read_ceiling"]
    # the one-launch M = 4 call covers the shapes the library fuses
    assert set(lin["verify_M4"]) == {"qkv", "o_proj"}
    assert set(out["batched_verify"]) == {"8"}
