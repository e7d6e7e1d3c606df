"""Summaries of rocprofv3 runs of bench.py, for the files under profiles/.

Runs on the host and reads rocprofv3 CSV output only (plain or gzipped):

  python bench_profile.py trace DIR
      DIR holds the output of
        rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- python -u bench.py ...
      Prints markdown tables: the --stats summary of the library's kernels,
      the average duration over all gemv_planes_kernel dispatches, and
      per-shape durations of the round's launches.

  python bench_profile.py traffic FETCH_DIR WRITE_DIR [--json PATH]
      The two directories hold
        rocprofv3 --pmc FETCH_SIZE ... / rocprofv3 --pmc WRITE_SIZE ...
      runs of bench.py with --copy-calibration MIB (a device copy of known
      size). Prints the per-shape counter table scaled by the factors the copy
      measures, and writes the JSON that bench.py reads (traffic per launch of
      the round's linear kernel, with the hash of the kernel sources).

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
    (r"^gemv_planes_kernel<2, 4, false, false, \d+, \d+, 0, 0>", ["verify qkv", "verify gate_up", "verify down"]),
    (r"^gemv_planes_kernel<2, 4, true, false, \d+, \d+, 0, 0>", ["verify o_proj"]),
    (r"^quant_token_kernel<2>", ["quant qkv", "quant gate_up"]),
    (r"^quant_token_kernel<7>", ["quant down"]),
    (r"^quant_group_kernel", ["quant o_proj"]),
]
ROUND_SHAPES = ["draft qkv", "draft o_proj", "draft gate_up", "draft down",
                "verify qkv", "verify o_proj", "verify gate_up", "verify down"]
# launches of each linear shape per layer in one round: 3 draft passes, 1 verify pass
ROUND_WEIGHT = {s: (3 if s.startswith("draft") else 1) for s in ROUND_SHAPES}
KERNEL_SOURCES = ["w8_quantized_linear_amd/csrc/gemv_planes.hip",
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


def cmd_trace(directory: str):
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
    print("| shape | dispatches | mean us | median us | min us |")
    print("|---|---:|---:|---:|---:|")
    for k in sorted(lab):
        v = sorted(dur(r) for r in lab[k])
        print("| %s | %d | %.3f | %.3f | %.3f |" % (k, len(v), sum(v) / len(v), v[len(v) // 2], v[0]))


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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--json", default=None)
    c.add_argument("--copy-mib", type=int, default=256)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        cmd_trace(a.dir)
    elif a.cmd == "mfma":
        cmd_mfma(a.dir)
    else:
        cmd_traffic(a.fetch_dir, a.write_dir, a.json, a.copy_mib)


if __name__ == "__main__":
    main()
