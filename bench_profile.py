"""Summaries of rocprofv3 runs of bench.py, for the files under profiles/.

Runs on the host and reads rocprofv3 CSV output only (plain or gzipped):

  python bench_profile.py trace DIR
      DIR holds the output of
        rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python -u bench.py ...
      Prints markdown tables: the --stats summary of the library's kernels,
      the average duration over all gemv_planes_kernel dispatches,
      per-shape durations of the round's launches (mean, p10, median, p90,
      min), and per round the sum of its dispatch durations against the
      span from its first start to its last end (--layers: the run's layer
      count, default 32).

  python bench_profile.py traffic FETCH_DIR WRITE_DIR [--json PATH]
      The two directories hold
        rocprofv3 --pmc FETCH_SIZE ... / rocprofv3 --pmc WRITE_SIZE ...
      runs of bench.py with --copy-calibration MIB (a device copy of known
      size). Prints the per-shape counter table scaled by the factors the copy
      measures, and writes the JSON that bench.py reads (traffic per launch of
      the round's linear kernel, with the hash of the kernel sources).

  python bench_profile.py counters DIR
      DIR holds the output of one rocprofv3 --pmc pass (any counters) of
      bench.py. Prints, per round shape and per batched-verify
      instantiation, the mean of each counter per dispatch, and the derived
      L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)), LDS bank conflicts per
      access (SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE -
      SQ_LDS_BANK_CONFLICT), rocprofv3's LdsBankConflict) and the VALU issue
      share (SQ_INSTS_VALU x 4 cycles over all SIMDs' cycles of the
      dispatch at the peak clock) where the counters are present; with
      --copy-mib MIB (the run's --copy-calibration), FETCH_SIZE and
      WRITE_SIZE scaled to bytes by what that copy reads and writes.

  python bench_profile.py ceiling DIR
      DIR holds the output of
        rocprofv3 --kernel-trace --output-format csv -d DIR -o run -- python -u bench.py ...
      of a run that times the read ceiling. Prints, per buffer size and
      configuration (items in flight per wave, waves per CU) of the sweep,
      the median dispatch duration of the timed graph replays with its GB/s
      (the fastest configuration of each size marked).

  python bench_profile.py pack FETCH_DIR WRITE_DIR [--copy-mib 256]
      The same for bench.py's packer section: per Llama-3-8B shape, the
      scaled reads and writes per dispatch against the fp32 weights read and
      the planes and scales written.

  python bench_profile.py kv FETCH_DIR WRITE_DIR [--copy-mib 256]
      The two directories hold --pmc FETCH_SIZE / --pmc WRITE_SIZE runs of
      bench.py's nested-KV attention section (with --copy-calibration).
      Prints, per context length and mode, the split kernel's scaled HBM
      reads and writes per dispatch against the cache bytes it must read.

  python bench_profile.py mfma DIR
      DIR holds the output of
        rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_VALU_MFMA_BUSY_CYCLES
                  SQ_INSTS_VALU_MFMA_I8 GRBM_GUI_ACTIVE --output-format csv -d DIR -o run -- python -u bench.py ...
      Prints, per batched-verify instantiation, the int8 matrix-core work per
      dispatch and the share of the kernel's duration the matrix cores were
      busy.

Shapes are told apart by the round's fixed launch order: each draft pass
launches qkv, o_proj, gate_up, down per layer, the verify pass a quantisation
launch and a linear launch per linear, so every kernel instantiation sees its
shapes in a fixed cycle (LABELS below; it follows the instantiations the
library picks for the Llama-3-8B shapes).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import gzip
import hashlib
import json
import math
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

# (pattern on the demangled kernel name, labels in launch order; the last
# template argument of gemv_planes_kernel is the rotation block, 0 = none)
LABELS = [
    (r"^gemv_planes_kernel<1, 1, false, false, \d+, \d+, 1, 0>", ["draft qkv", "draft gate_up"]),
    (r"^gemv_planes_kernel<1, 1, true, false, \d+, \d+, 1, 0>", ["draft o_proj"]),
    (r"^gemv_planes_kernel<1, 1, false, false, \d+, \d+, 4, 0>", ["draft down"]),
    # the verify pass quantises inside the linear's launch for qkv and o_proj
    # and takes a quantisation launch before gate_up's and down_proj's
    # linears
    (r"^gemv_planes_kernel<2, 4, false, false, \d+, \d+, 1, 0>", ["verify qkv"]),
    (r"^gemv_planes_kernel<2, 4, true, false, \d+, \d+, 1, 0>", ["verify o_proj"]),
    (r"^gemv_planes_kernel<2, 4, false, false, \d+, \d+, 0, 0>", ["verify gate_up", "verify down"]),
    (r"^quant_token_kernel<2>", ["quant gate_up"]),
    (r"^quant_token_kernel<7>", ["quant down"]),
]
ROUND_SHAPES = ["draft qkv", "draft o_proj", "draft gate_up", "draft down",
                "verify qkv", "verify o_proj", "verify gate_up", "verify down"]
# launches of each linear shape per layer in one round: 3 draft passes, 1 verify pass
ROUND_WEIGHT = {s: (3 if s.startswith("draft") else 1) for s in ROUND_SHAPES}
KERNEL_SOURCES = ["w8_quantized_linear_amd/csrc/gemv_planes.hip",
                  "w8_quantized_linear_amd/csrc/gemv_common.h",
                  "w8_quantized_linear_amd/csrc/device_common.h",
                  "w8_quantized_linear_amd/csrc/bitnest_internal.h"]


def short(name: str) -> str:
    name = re.sub(r"bitnest::\(anonymous namespace\)::", "", name)
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*\)$", "", name).strip()


def read_csv(directory: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True) +
                   glob.glob(os.path.join(directory, "**", "*" + suffix + ".gz"), recursive=True))
    if not paths:
        sys.exit("no *%s under %s" % (suffix, directory))
    rows = []
    for p in paths:
        with (gzip.open(p, "rt") if p.endswith(".gz") else open(p)) as f:
            rows.extend(csv.DictReader(f))
    return rows


def label_rows(rows, order_key):
    """{label: [rows]} for the library's kernels, each instantiation's
    dispatches (in `order_key` order) assigned to its cycle of shapes."""
    by_name = collections.defaultdict(list)
    for r in rows:
        if "bitnest" in r["Kernel_Name"]:
            by_name[short(r["Kernel_Name"])].append(r)
    out = collections.defaultdict(list)
    for name, rs in by_name.items():
        rs.sort(key=order_key)
        for pattern, cycle in LABELS:
            if re.match(pattern, name):
                for i, r in enumerate(rs):
                    out[cycle[i % len(cycle)]].append(r)
                break
        else:
            out[name].extend(rs)
    return out


def quantile(v, q):
    """Nearest-rank quantile of the sorted list v (0 < q < 1)."""
    return v[min(len(v) - 1, max(0, math.ceil(q * len(v)) - 1))]


def round_accounting(trace, layers):
    """[(busy us, span us)] per round: the library dispatches in start order,
    cut into rounds of 18 * layers launches from the first one while every
    dispatch of a round is one of the round's kernels (LABELS)."""
    rows = sorted((r for r in trace if "bitnest" in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
    n = 18 * layers
    out = []
    for i in range(0, len(rows) - n + 1, n):
        chunk = rows[i:i + n]
        if not all(any(re.match(p, short(r["Kernel_Name"])) for p, _ in LABELS) for r in chunk):
            break
        starts = [int(r["Start_Timestamp"]) for r in chunk]
        ends = [int(r["End_Timestamp"]) for r in chunk]
        busy = sum(e - b for b, e in zip(starts, ends)) / 1e3
        out.append((busy, (max(ends) - min(starts)) / 1e3))
    return out


def ceiling_sweep(trace, sizes_mib, configs, cold_bytes, reps):
    """{(MiB, depth, waves per CU): (median dispatch us, us per launch over
    the timed replays' spans)} from the stream_read dispatches of bench.py's
    read-ceiling sweep, in its order: per size and configuration, one eager
    pass and 1 + reps graph replays over ceil(cold_bytes / size) buffers."""
    rows = sorted((r for r in trace if re.match(r"^stream_read_kernel<\d+>", short(r["Kernel_Name"]))),
                  key=lambda r: int(r["Start_Timestamp"]))
    plan = []
    for mib in sizes_mib:
        count = max(1, -(-cold_bytes // (mib << 20)))
        plan.extend((mib, depth, wpc, count) for depth, wpc in configs)
    need = sum(count * (2 + reps) for *_, count in plan)
    if len(rows) != need:
        sys.exit("expected %d stream_read dispatches, found %d" % (need, len(rows)))
    out = {}
    i = 0
    for mib, depth, wpc, count in plan:
        block = rows[i:i + count * (2 + reps)]
        i += len(block)
        assert all(short(r["Kernel_Name"]) == "stream_read_kernel<%d>" % depth for r in block)
        timed = block[2 * count:]
        durs = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed)
        spans = sorted((int(timed[k * count + count - 1]["End_Timestamp"]) - int(timed[k * count]["Start_Timestamp"]))
                       / 1e3 / count for k in range(reps))
        out[(mib, depth, wpc)] = (quantile(durs, 0.5), spans[len(spans) // 2])
    return out


def cmd_ceiling(directory: str):
    sys.path.insert(0, ROOT)
    import inspect
    import bench
    trace = read_csv(directory, "kernel_trace.csv")
    reps = inspect.signature(bench.read_ceiling).parameters["reps"].default
    sweep = ceiling_sweep(trace, bench.READ_CEILING_MIB, bench.READ_CONFIGS, bench.COLD_BYTES, reps)
    print("| size | depth | waves per CU | median dispatch us | GB/s |")
    print("|---|---:|---:|---:|---:|")
    for mib in bench.READ_CEILING_MIB:
        cands = {k: v for k, v in sweep.items() if k[0] == mib}
        best = min(cands, key=lambda k: cands[k][0])
        for k in sorted(cands, key=lambda k: bench.READ_CONFIGS.index(k[1:])):
            d = cands[k][0]
            print("| %d MiB | %d | %s | %.3f%s | %.0f |"
                  % (mib, k[1], k[2] or "all", d, " **best**" if k == best else "", (mib << 20) / d / 1e3))


def cmd_trace(directory: str, layers: int = 32):
    stats = read_csv(directory, "kernel_stats.csv")
    print("## rocprofv3 --stats (kernel_stats.csv, library kernels)\n")
    print("| kernel | calls | average ns | total ns |")
    print("|---|---:|---:|---:|")
    gemv_calls = gemv_total = 0
    for r in stats:
        if "bitnest" not in r["Name"]:
            continue
        n, calls, avg, tot = short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"])
        print("| %s | %d | %.1f | %.0f |" % (n, calls, avg, tot))
        if n.startswith("gemv_planes_kernel"):
            gemv_calls += calls
            gemv_total += tot
    if gemv_calls:
        print("\nAll gemv_planes_kernel dispatches together: %.0f ns over %d launches = **%.2f us average "
              "per launch**.\n" % (gemv_total, gemv_calls, gemv_total / gemv_calls / 1e3))
    trace = read_csv(directory, "kernel_trace.csv")
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lab = label_rows(trace, lambda r: int(r["Start_Timestamp"]))
    print("## Per shape (kernel_trace.csv)\n")
    print("| shape | dispatches | mean us | p10 us | median us | p90 us | min us |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k in sorted(lab):
        v = sorted(dur(r) for r in lab[k])
        print("| %s | %d | %.3f | %.3f | %.3f | %.3f | %.3f |"
              % (k, len(v), sum(v) / len(v), quantile(v, 0.1), quantile(v, 0.5), quantile(v, 0.9), v[0]))
    rounds = round_accounting(trace, layers)
    if rounds:
        print("\n## Rounds (kernel_trace.csv)\n")
        print("The first %d x %d dispatches, taken in rounds of %d (%d layers x 18: three draft passes of 4 "
              "linears, 4 verify linears and 2 verify quantisation launches); round 0 is the eager run on the "
              "capture stream, the others are graph replays. busy = sum of the round's dispatch durations, "
              "span = first start to last end.\n" % (len(rounds), 18 * layers, 18 * layers, layers))
        print("| round | busy ms | span ms | span - busy, us per launch |")
        print("|---|---:|---:|---:|")
        for i, (busy, span) in enumerate(rounds):
            print("| %d | %.3f | %.3f | %.3f |" % (i, busy / 1e3, span / 1e3, (span - busy) / (18 * layers)))


def copy_factor(rows, counter: str, copy_bytes: float):
    """Bytes per counter unit: the largest device-copy dispatch of the run is
    the known-size calibration copy."""
    cp = [r for r in rows if "copy" in r["Kernel_Name"].lower() and r["Counter_Name"] == counter]
    if not cp:
        sys.exit("no copy kernel with %s in the run (use bench.py --copy-calibration)" % counter)
    big = max(float(r["Counter_Value"]) for r in cp)
    return copy_bytes / (big * 1024.0), big


def per_dispatch(rows, counter):
    rows = [r for r in rows if r["Counter_Name"] == counter]
    agg = {}
    for r in rows:       # one row per dispatch (a counter summed over its instances)
        agg.setdefault(r["Dispatch_Id"], r)
    return list(agg.values())


def cmd_traffic(fetch_dir: str, write_dir: str, json_path: str | None, copy_mib: int):
    res = {}
    factors = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(read_csv(d, "counter_collection.csv"), counter)
        f, raw = copy_factor(rows, counter, copy_mib * 1048576.0)
        factors[counter] = (f, raw)
        lab = label_rows(rows, lambda r: int(r["Dispatch_Id"]))
        res[counter] = {k: sum(float(r["Counter_Value"]) for r in v) / len(v) for k, v in lab.items()}
    ff, fraw = factors["FETCH_SIZE"]
    wf, wraw = factors["WRITE_SIZE"]
    print("Calibration: the %d MiB copy reads FETCH_SIZE = %.1f KiB and WRITE_SIZE = %.1f KiB, so "
          "bytes = %.4f x FETCH_SIZE KiB x 1024 and %.4f x WRITE_SIZE KiB x 1024.\n" % (copy_mib, fraw, wraw, ff, wf))
    print("| shape | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic (scaled) MB |")
    print("|---|---:|---:|---:|")
    per_shape = {}
    for k in sorted(res["FETCH_SIZE"]):
        fk, wk = res["FETCH_SIZE"][k], res["WRITE_SIZE"].get(k, 0.0)
        b = fk * 1024 * ff + wk * 1024 * wf
        per_shape[k] = b
        print("| %s | %.1f | %.1f | %.2f |" % (k, fk, wk, b / 1e6))
    missing = [s for s in ROUND_SHAPES if s not in per_shape]
    if missing:
        sys.exit("shapes missing from the counters: %s" % missing)
    n = sum(ROUND_WEIGHT.values())
    per_launch = sum(ROUND_WEIGHT[s] * per_shape[s] for s in ROUND_SHAPES) / n
    print("\nLaunch-weighted over the round (3 draft launches per verify launch of each shape): "
          "**%.0f bytes per launch**." % per_launch)
    if json_path:
        h = hashlib.sha256()
        for src in KERNEL_SOURCES:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        out = {"kernel": "gemv_planes_kernel (the round's linear launches)",
               "sources_sha256": h.hexdigest(), "sources": KERNEL_SOURCES,
               "fetch_factor": ff, "write_factor": wf,
               "traffic_bytes_per_launch": int(round(per_launch)),
               "per_shape_bytes": {s: int(round(per_shape[s])) for s in ROUND_SHAPES},
               "note": "FETCH_SIZE/WRITE_SIZE per dispatch (KiB) x the factor a %d MiB device copy measures "
                       "in the same runs" % copy_mib}
        with open(json_path, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        print("\nwrote %s" % json_path)


# MI355X: 256 CUs x 4 SIMDs, each with its own matrix core; the engine clock
# the busy share is taken against (the part's peak clock, so the share can
# only be understated)
SIMDS = 1024
CLOCK_GHZ = 2.4


def cmd_mfma(directory: str):
    rows = [r for r in read_csv(directory, "counter_collection.csv") if "verify_mfma_kernel" in r["Kernel_Name"]]
    if not rows:
        sys.exit("no verify_mfma_kernel dispatches in %s" % directory)
    per = {}
    for r in rows:
        d = per.setdefault((short(r["Kernel_Name"]), r["Dispatch_Id"]),
                           {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                            "grid": int(r["Grid_Size"]) // int(r["Workgroup_Size"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    by_kernel = {}
    for (name, _), d in per.items():
        by_kernel.setdefault(name, []).append(d)
    print("| kernel | dispatches | workgroups | mean us | int8 MFMA ops per dispatch | MFMA instructions | "
          "busy cycles per SIMD | busy share of the duration |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    for name in sorted(by_kernel):
        ds = by_kernel[name]
        n = len(ds)
        mean = lambda key: sum(d[key] for d in ds) / n
        dur = mean("dur_ns")
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / SIMDS
        print("| %s | %d | %d | %.2f | %.4g | %.0f | %.0f | %.2f %% |" % (
            name, n, ds[0]["grid"], dur / 1e3, mean("SQ_INSTS_VALU_MFMA_MOPS_I8") * 512,
            mean("SQ_INSTS_VALU_MFMA_I8"), busy, 100.0 * busy / (dur * CLOCK_GHZ)))


def cmd_counters(directory: str, copy_mib: int = 0):
    rows = read_csv(directory, "counter_collection.csv")
    names = sorted({r["Counter_Name"] for r in rows})
    scaled = {}
    if copy_mib:
        # bytes per counter KiB from the run's known-size device copy, as for
        # the traffic summary
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in names:
                f, raw = copy_factor(per_dispatch(rows, c), c, copy_mib * 1048576.0)
                scaled[c] = f
                print("Calibration: the %d MiB copy reads %s = %.1f KiB: bytes = %.4f x %s KiB x 1024.\n"
                      % (copy_mib, c, raw, f, c))
    per = {}
    for r in rows:
        if "bitnest" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"row": r, "dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lab = label_rows([d["row"] for d in per.values()], lambda r: int(r["Dispatch_Id"]))
    by_id = {d["row"]["Dispatch_Id"]: d for d in per.values()}
    derived = []
    if "TCC_HIT" in " ".join(names) and "TCC_MISS" in " ".join(names):
        derived.append("L2 hit %")
    if "SQ_LDS_BANK_CONFLICT" in names and "SQ_LDS_IDX_ACTIVE" in names:
        derived.append("LDS conflicts per access")
    if "SQ_INSTS_VALU" in names:
        derived.append("VALU issue share %")
    for c in sorted(scaled):
        derived.append("%s MB (scaled)" % c)
    print("| kernel / shape | dispatches | mean us | " + " | ".join(names + derived) + " |")
    print("|---|---:|---:|" + "---:|" * (len(names) + len(derived)))
    hit = next((n for n in names if n.startswith("TCC_HIT")), None)
    miss = next((n for n in names if n.startswith("TCC_MISS")), None)
    for k in sorted(lab):
        ds = [by_id[r["Dispatch_Id"]] for r in lab[k]]
        n = len(ds)
        mean = lambda key: sum(d.get(key, 0.0) for d in ds) / n
        cells = ["%.4g" % mean(c) for c in names]
        if "L2 hit %" in derived:
            h, m = mean(hit), mean(miss)
            cells.append("%.1f" % (100.0 * h / (h + m)) if h + m else "-")
        if "LDS conflicts per access" in derived:
            c, a = mean("SQ_LDS_BANK_CONFLICT"), mean("SQ_LDS_IDX_ACTIVE")
            cells.append("%.4f" % (c / (a - c)) if a > c else "-")
        if "VALU issue share %" in derived:
            # wave64 VALU instructions take 4 cycles of a 16-lane SIMD; against
            # every SIMD over the dispatch at the peak clock (an understatement
            # where the clock runs lower)
            cells.append("%.1f" % (100.0 * mean("SQ_INSTS_VALU") * 4 / (SIMDS * mean("dur_ns") * CLOCK_GHZ)))
        for c in sorted(scaled):
            cells.append("%.3f" % (mean(c) * 1024 * scaled[c] / 1e6))
        print("| %s | %d | %.2f | %s |" % (k, n, mean("dur_ns") / 1e3, " | ".join(cells)))



def kv_blocks(rows, counter, contexts, layers, reps):
    """[(T, mode, mean counter value per split dispatch)] from bench.py's KV
    section: the split-kernel dispatches in start order, one block of
    layers x (2 + reps) per (context, mode), draft KV4 then verify KV8; the
    eager pass and the warm replay of each block are left out."""
    split = sorted((r for r in per_dispatch(rows, counter) if "kv_attn_split_kernel" in r["Kernel_Name"]),
                   key=lambda r: int(r["Dispatch_Id"]))
    n = layers * (2 + reps)
    if len(split) != n * 2 * len(contexts):
        sys.exit("expected %d split dispatches, found %d" % (n * 2 * len(contexts), len(split)))
    out = []
    for i, (T, mode) in enumerate((T, m) for T in contexts for m in ("draft KV4", "verify KV8")):
        timed = split[i * n + 2 * layers:(i + 1) * n]
        out.append((T, mode, sum(float(r["Counter_Value"]) for r in timed) / len(timed)))
    return out


def cmd_kv(fetch_dir: str, write_dir: str, copy_mib: int, contexts, layers: int, reps: int, hkv: int):
    print("| T | mode | cache bytes read (algorithmic) MB | FETCH (scaled) MB | ratio | WRITE (scaled) MB |")
    print("|---:|---|---:|---:|---:|---:|")
    res = {}
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_csv(d, "counter_collection.csv")
        f, _ = copy_factor(per_dispatch(rows, c), c, copy_mib * 1048576.0)
        res[c] = [(T, m, v * 1024 * f) for T, m, v in kv_blocks(rows, c, contexts, layers, reps)]
    for (T, mode, fb), (_, _, wb) in zip(res["FETCH_SIZE"], res["WRITE_SIZE"]):
        planes = 2 if mode.startswith("verify") else 1
        alg = 2 * T * hkv * (64 * planes + 2)
        print("| %d | %s | %.3f | %.3f | %.3f | %.3f |" % (T, mode, alg / 1e6, fb / 1e6, fb / alg, wb / 1e6))


def pack_blocks(rows, counter, shapes, reps):
    """[(name, mean counter value per dispatch)] from bench.py's packer
    section: pack_nested_kernel dispatches in start order, per shape
    pack_buffers(N, K) x (2 + reps) of them (eager pass, warm replay, timed
    replays); the timed ones are averaged."""
    sys.path.insert(0, ROOT)
    import bench
    pk = sorted((r for r in per_dispatch(rows, counter) if "pack_nested_kernel" in r["Kernel_Name"]),
                key=lambda r: int(r["Dispatch_Id"]))
    sizes = [bench.pack_buffers(N, K) for (_, N, K) in shapes]
    if len(pk) != sum(n * (2 + reps) for n in sizes):
        sys.exit("expected %d pack dispatches, found %d" % (sum(n * (2 + reps) for n in sizes), len(pk)))
    out, i = [], 0
    for (name, _, _), n in zip(shapes, sizes):
        timed = pk[i + 2 * n:i + n * (2 + reps)]
        out.append((name, sum(float(r["Counter_Value"]) for r in timed) / len(timed)))
        i += n * (2 + reps)
    return out


def cmd_pack(fetch_dir: str, write_dir: str, copy_mib: int, reps: int):
    from w8_quantized_linear_amd import synth
    shapes = [(name, N, K) for (name, N, K, _) in synth.LLAMA3_8B_LINEARS]
    res = {}
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_csv(d, "counter_collection.csv")
        f, _ = copy_factor(per_dispatch(rows, c), c, copy_mib * 1048576.0)
        res[c] = {name: v * 1024 * f for name, v in pack_blocks(rows, c, shapes, reps)}
    print("| shape | fp32 read MB | FETCH (scaled) MB | ratio | planes + scales written MB | WRITE (scaled) MB | ratio |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for name, N, K in shapes:
        rd, wr = 4 * N * K, N * K + 2 * N * (K // 128)
        fb, wb = res["FETCH_SIZE"][name], res["WRITE_SIZE"][name]
        print("| %s | %.2f | %.2f | %.3f | %.2f | %.2f | %.3f |" % (name, rd / 1e6, fb / 1e6, fb / rd, wr / 1e6,
                                                                  wb / 1e6, wb / wr))

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--layers", type=int, default=32, help="layers of the profiled bench.py run")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--json", default=None)
    c.add_argument("--copy-mib", type=int, default=256)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    k = sub.add_parser("counters")
    k.add_argument("dir")
    k.add_argument("--copy-mib", type=int, default=0,
                   help="the run's --copy-calibration size: scale FETCH_SIZE / WRITE_SIZE to bytes")
    r = sub.add_parser("ceiling")
    r.add_argument("dir")
    pk = sub.add_parser("pack")
    pk.add_argument("fetch_dir")
    pk.add_argument("write_dir")
    pk.add_argument("--copy-mib", type=int, default=256)
    pk.add_argument("--reps", type=int, default=5)
    v = sub.add_parser("kv")
    v.add_argument("fetch_dir")
    v.add_argument("write_dir")
    v.add_argument("--copy-mib", type=int, default=256)
    v.add_argument("--contexts", default="2048,8192,32768")
    v.add_argument("--layers", type=int, default=32)
    v.add_argument("--reps", type=int, default=5)
    v.add_argument("--hkv", type=int, default=8)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        cmd_trace(a.dir, a.layers)
    elif a.cmd == "mfma":
        cmd_mfma(a.dir)
    elif a.cmd == "counters":
        cmd_counters(a.dir, a.copy_mib)
    elif a.cmd == "ceiling":
        cmd_ceiling(a.dir)
    elif a.cmd == "pack":
        cmd_pack(a.fetch_dir, a.write_dir, a.copy_mib, a.reps)
    elif a.cmd == "kv":
        cmd_kv(a.fetch_dir, a.write_dir, a.copy_mib, [int(t) for t in a.contexts.split(",")], a.layers, a.reps,
               a.hkv)
    else:
        cmd_traffic(a.fetch_dir, a.write_dir, a.json, a.copy_mib)


if __name__ == "__main__":
    main()
