"""The profile summariser (bench_profile.py) on a synthetic rocprofv3 trace:
dispatches in the round's launch order with known durations, so the shape
labels, the quantiles and the per-round accounting can be checked exactly."""
import csv
import io
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench_profile as bp  # noqa: E402

NS = "void bitnest::(anonymous namespace)::"
GEMV = NS + "gemv_planes_kernel<%s>(bitnest::LinearArgs)"
QUANT = NS + "quant_token_kernel<%d>(float const*, int, signed char*, float*)"

# (kernel name, label, duration ns) of one layer of one round, in launch order
DRAFT = [(GEMV % "1, 1, false, false, 4, 8, 1, 0", "draft qkv", 4800),
         (GEMV % "1, 1, true, false, 4, 8, 1, 0", "draft o_proj", 4000),
         (GEMV % "1, 1, false, false, 4, 8, 1, 0", "draft gate_up", 11500),
         (GEMV % "1, 1, false, false, 4, 8, 4, 0", "draft down", 7800)]
VERIFY = [(GEMV % "2, 4, false, false, 2, 8, 1, 0", "verify qkv", 9400),
          (GEMV % "2, 4, true, false, 2, 8, 1, 0", "verify o_proj", 7800),
          (QUANT % 2, "quant gate_up", 3000),
          (GEMV % "2, 4, false, false, 2, 8, 0, 0", "verify gate_up", 22200),
          (QUANT % 7, "quant down", 4500),
          (GEMV % "2, 4, false, false, 2, 8, 0, 0", "verify down", 13000)]
GAP = 250


def launches(layers, rounds):
    seq = []
    for r in range(rounds):
        for p in range(4):
            for _ in range(layers):
                seq.extend(VERIFY if p == 3 else DRAFT)
    # the batched-verify section that follows the rounds
    seq.append((NS + "verify_mfma_kernel<2, 1, false, false, 1>(bitnest::LinearArgs, int)", "mfma", 16000))
    seq.append((QUANT % 2, "quant gate_up", 3000))
    return seq


def write_trace(d, seq, jitter):
    t = 1_000_000
    rows = []
    for i, (name, _, ns) in enumerate(seq):
        ns += jitter(i)
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + ns})
        t += ns + GAP
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "TotalDurationNs"])
        w.writeheader()
        w.writerow({"Name": GEMV % "1, 1, false, false, 4, 8, 1, 0", "Calls": 2, "AverageNs": 5000.0,
                    "TotalDurationNs": 10000})


def test_quantile_is_nearest_rank():
    v = list(range(1, 11))
    assert bp.quantile(v, 0.1) == 1 and bp.quantile(v, 0.5) == 5 and bp.quantile(v, 0.9) == 9
    assert bp.quantile([7], 0.1) == 7 and bp.quantile([7], 0.9) == 7
    w = list(range(1, 12))
    assert bp.quantile(w, 0.5) == 6 and bp.quantile(w, 0.9) == 10


def test_labels_follow_the_round_launch_order(tmp_path):
    layers, rounds = 2, 3
    seq = launches(layers, rounds)
    write_trace(tmp_path, seq, lambda i: 0)
    trace = bp.read_csv(str(tmp_path), "kernel_trace.csv")
    lab = bp.label_rows(trace, lambda r: int(r["Start_Timestamp"]))
    want = {}
    for name, label, ns in seq:
        if label != "mfma":
            want.setdefault(label, set()).add(ns)
    for label, durs in want.items():
        got = {int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in lab[label]}
        assert got == durs, label
    assert len(lab["draft qkv"]) == 3 * layers * rounds
    assert len(lab["verify down"]) == layers * rounds
    assert len(lab["verify_mfma_kernel<2, 1, false, false, 1>"]) == 1


def test_round_accounting(tmp_path):
    layers, rounds = 2, 3
    seq = launches(layers, rounds)
    write_trace(tmp_path, seq, lambda i: i % 3)     # a few ns of jitter, known per dispatch
    trace = bp.read_csv(str(tmp_path), "kernel_trace.csv")
    got = bp.round_accounting(trace, layers)
    assert len(got) == rounds                        # stops at the batched-verify section
    n = 18 * layers
    for r, (busy, span) in enumerate(got):
        idx = range(r * n, (r + 1) * n)
        want_busy = sum(seq[i][2] + i % 3 for i in idx)
        assert abs(busy * 1e3 - want_busy) < 1e-6
        assert abs(span * 1e3 - (want_busy + (n - 1) * GAP)) < 1e-6
    out = io.StringIO()
    with redirect_stdout(out):
        bp.cmd_trace(str(tmp_path), layers)
    text = out.getvalue()
    assert "| shape | dispatches | mean us | p10 us | median us | p90 us | min us |" in text
    assert "## Rounds" in text and "| 2 |" in text


def test_ceiling_sweep_labels_and_spans(tmp_path):
    # two sizes x two configurations; per (size, config): an eager pass, a
    # warm replay and `reps` timed replays over ceil(cold / size) buffers
    sizes, configs, cold, reps = [1, 4], [(2, 0), (4, 8)], 4 << 20, 3
    seq = []
    want = {}
    for mib in sizes:
        count = max(1, -(-cold // (mib << 20)))
        for ci, (depth, wpc) in enumerate(configs):
            base = 1000 * mib + 100 * ci
            for p in range(2 + reps):
                for c in range(count):
                    seq.append((NS + "stream_read_kernel<%d>(unsigned char const*, unsigned int)" % depth, "sr",
                                base + p + c))
            timed = [base + p + c for p in range(2, 2 + reps) for c in range(count)]
            spans = sorted((sum(base + p + c for c in range(count)) + (count - 1) * GAP) / count
                           for p in range(2, 2 + reps))
            want[(mib, depth, wpc)] = (bp.quantile(sorted(timed), 0.5) / 1e3, spans[len(spans) // 2] / 1e3)
    write_trace(tmp_path, seq, lambda i: 0)
    got = bp.ceiling_sweep(bp.read_csv(str(tmp_path), "kernel_trace.csv"), sizes, configs, cold, reps)
    assert set(got) == set(want)
    for k in want:
        assert abs(got[k][0] - want[k][0]) < 1e-9 and abs(got[k][1] - want[k][1]) < 1e-9, k


def _counter_run(d, counter, seq, values, copy_value):
    os.makedirs(d, exist_ok=True)
    rows = [{"Dispatch_Id": 1, "Kernel_Name": "void at::native::elementwise_copy_kernel<float>(...)",
             "Counter_Name": counter, "Counter_Value": copy_value}]
    for i, (name, label, _) in enumerate(seq):
        rows.append({"Dispatch_Id": i + 2, "Kernel_Name": name, "Counter_Name": counter,
                     "Counter_Value": values[label]})
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def test_traffic_scaling_and_launch_weighting(tmp_path):
    # FETCH_SIZE and WRITE_SIZE per dispatch (KiB) scaled by what a copy of
    # known size reads (here: half its bytes) and writes (all of them), then
    # weighted 3 : 1 over the draft and verify launches of each shape
    import json
    seq = launches(2, 2)[:-2]                        # the rounds only
    labels = [l for _, l, _ in DRAFT + VERIFY]
    fetch = {l: 1000.0 + 37 * i for i, l in enumerate(labels)}
    write = {l: 10.0 + 3 * i for i, l in enumerate(labels)}
    copy_mib = 16
    _counter_run(str(tmp_path / "f"), "FETCH_SIZE", seq, fetch, copy_mib * 1024 / 2)
    _counter_run(str(tmp_path / "w"), "WRITE_SIZE", seq, write, copy_mib * 1024)
    out_json = str(tmp_path / "t.json")
    buf = io.StringIO()
    with redirect_stdout(buf):
        bp.cmd_traffic(str(tmp_path / "f"), str(tmp_path / "w"), out_json, copy_mib)
    got = json.load(open(out_json))
    assert abs(got["fetch_factor"] - 2.0) < 1e-12 and abs(got["write_factor"] - 1.0) < 1e-12
    per_shape = {s: fetch[s] * 1024 * 2 + write[s] * 1024 for s in bp.ROUND_SHAPES}
    for s in bp.ROUND_SHAPES:
        assert got["per_shape_bytes"][s] == round(per_shape[s])
    want = sum((3 if s.startswith("draft") else 1) * per_shape[s] for s in bp.ROUND_SHAPES) / 16
    assert got["traffic_bytes_per_launch"] == round(want)
    assert got["sources"] == bp.KERNEL_SOURCES and len(got["sources_sha256"]) == 64


def _pmc_rows(d, entries):
    # entries: (dispatch id, kernel name, duration ns, grid, {counter: value})
    os.makedirs(d, exist_ok=True)
    rows = []
    for did, name, dur, grid, counters in entries:
        for c, v in counters.items():
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": 1000 * did,
                         "End_Timestamp": 1000 * did + dur, "Grid_Size": grid * 512, "Workgroup_Size": 512,
                         "Counter_Name": c, "Counter_Value": v})
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _table(text):
    return [[c.strip() for c in line.strip().strip("|").split("|")] for line in text.splitlines()
            if line.startswith("| ") and not line.startswith("| kernel")]


def test_mfma_busy_share(tmp_path):
    name = NS + "verify_mfma_kernel<2, 1, false, false, 1>(bitnest::LinearArgs, int)"
    # 448 MFMAs per workgroup x 256 workgroups, 32768 int8 ops each; busy
    # cycles summed over the 1024 SIMDs: 1792 per SIMD in a 16 us dispatch
    c = {"SQ_INSTS_VALU_MFMA_MOPS_I8": 114688 * 32768 / 512, "SQ_INSTS_VALU_MFMA_I8": 114688,
         "SQ_VALU_MFMA_BUSY_CYCLES": 1792 * 1024, "GRBM_GUI_ACTIVE": 1.0}
    _pmc_rows(str(tmp_path), [(1, name, 16000, 256, c), (2, name, 16000, 256, c)])
    out = io.StringIO()
    with redirect_stdout(out):
        bp.cmd_mfma(str(tmp_path))
    (row,) = _table(out.getvalue())
    assert row[0] == "verify_mfma_kernel<2, 1, false, false, 1>" and row[1] == "2" and row[2] == "256"
    assert row[3] == "16.00" and float(row[4]) == float("%.4g" % (114688 * 32768)) and row[5] == "114688"
    assert row[6] == "1792"
    assert row[7] == "%.2f %%" % (100.0 * 1792 / (16000 * 2.4))


def test_counters_derived_rates(tmp_path):
    qkv = NS + "gemv_planes_kernel<1, 1, false, false, 4, 8, 1, 0>(bitnest::LinearArgs)"
    # SQ_INSTS_VALU: 1200 (2400) cycles' worth per SIMD at 4 cycles each over
    # 5 us (12 us) at 2.4 GHz = 10 % (8.33 %)
    c1 = {"TCC_HIT_sum": 300.0, "TCC_MISS_sum": 100.0, "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 60.0,
          "SQ_INSTS_VALU": 1200 / 4 * 1024}
    c2 = {"TCC_HIT_sum": 100.0, "TCC_MISS_sum": 300.0, "SQ_LDS_BANK_CONFLICT": 30.0, "SQ_LDS_IDX_ACTIVE": 100.0,
          "SQ_INSTS_VALU": 2400 / 4 * 1024}
    # launch order qkv, gate_up, qkv, gate_up for this instantiation
    _pmc_rows(str(tmp_path), [(1, qkv, 5000, 256, c1), (2, qkv, 12000, 256, c2),
                              (3, qkv, 5000, 256, c1), (4, qkv, 12000, 256, c2)])
    out = io.StringIO()
    with redirect_stdout(out):
        bp.cmd_counters(str(tmp_path))
    rows = {r[0]: r for r in _table(out.getvalue())}
    assert set(rows) == {"draft qkv", "draft gate_up"}
    assert rows["draft qkv"][1] == "2" and rows["draft qkv"][2] == "5.00"
    assert rows["draft qkv"][-3] == "75.0" and rows["draft gate_up"][-3] == "25.0"       # L2 hit %
    assert rows["draft qkv"][-2] == "0.2000" and rows["draft gate_up"][-2] == "0.4286"   # c / (a - c)
    assert rows["draft qkv"][-1] == "10.0" and rows["draft gate_up"][-1] == "8.3"        # VALU issue share


def test_counters_scale_fetch_by_the_copy(tmp_path):
    # a 16 MiB copy that FETCH_SIZE counts as 8192 KiB: 2 bytes per KiB x 1024
    name = NS + "verify_mfma_kernel<2, 1, false, false, 1>(bitnest::LinearArgs, int)"
    copy = "void at::native::elementwise_copy_kernel<float>(...)"
    entries = [(1, copy, 1000, 256, {"FETCH_SIZE": 8192.0}),
               (2, name, 16000, 256, {"FETCH_SIZE": 30000.0}), (3, name, 16000, 256, {"FETCH_SIZE": 32000.0})]
    _pmc_rows(str(tmp_path), entries)
    out = io.StringIO()
    with redirect_stdout(out):
        bp.cmd_counters(str(tmp_path), copy_mib=16)
    text = out.getvalue()
    assert "bytes = 2.0000 x FETCH_SIZE KiB x 1024" in text
    (row,) = _table(text)
    assert row[0] == "verify_mfma_kernel<2, 1, false, false, 1>"
    assert row[-1] == "%.3f" % (31000.0 * 1024 * 2 / 1e6)


def test_kv_blocks_follow_the_section_order(tmp_path):
    # two contexts x (draft, verify), 2 layers, 1 timed replay: blocks of
    # 2 x (2 + 1) split dispatches; combine dispatches interleaved and ignored
    contexts, layers, reps = [64, 128], 2, 1
    entries, did = [], 1
    want = []
    for T in contexts:
        for m, base in (("draft KV4", 10.0), ("verify KV8", 20.0)):
            for p in range(2 + reps):
                for l in range(layers):
                    v = base * T + (100.0 if p < 2 else 0.0) + l      # eager and warm passes differ
                    entries.append((did, NS + "kv_attn_split_kernel<false, 4>(bitnest::KvArgs, int)", 1000, 8,
                                    {"FETCH_SIZE": v}))
                    entries.append((did + 1, NS + "kv_attn_combine_kernel(bitnest::KvArgs, int)", 500, 8,
                                    {"FETCH_SIZE": 1.0}))
                    did += 2
            want.append((T, m, base * T + 0.5))
    _pmc_rows(str(tmp_path), entries)
    got = bp.kv_blocks(bp.read_csv(str(tmp_path), "counter_collection.csv"), "FETCH_SIZE", contexts, layers, reps)
    assert got == want


def test_pack_blocks_follow_the_section_order(tmp_path):
    # two shapes with 3 and 2 rotating buffers, 1 timed replay: blocks of
    # nbuf x (2 + 1) dispatches, the timed replay averaged
    import bench
    shapes = [("a", 8192, 16384), ("b", 16384, 16384)]
    nb = [bench.pack_buffers(N, K) for _, N, K in shapes]
    assert nb == [2, 2]
    entries, did, want = [], 1, []
    for (name, N, K), n in zip(shapes, nb):
        for p in range(3):
            for j in range(n):
                entries.append((did, NS + "pack_nested_kernel(float const*, long long, ...)", 1000, 8,
                                {"FETCH_SIZE": float(N + (7 if p < 2 else j))}))
                did += 1
        want.append((name, N + (n - 1) / 2))
    _pmc_rows(str(tmp_path), entries)
    got = bp.pack_blocks(bp.read_csv(str(tmp_path), "counter_collection.csv"), "FETCH_SIZE", shapes, 1)
    assert got == want
