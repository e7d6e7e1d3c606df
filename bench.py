#!/usr/bin/env python3
"""Benchmark of the bit-nested W4/W8 linear on one MI355X.

Workload (one "step"): one speculative decoding round over the linear stack of
Llama-3-8B (32 decoder layers, linears qkv 6144x4096, o_proj 4096x4096 with
per-128-group activation scales, gate_up 28672x4096, down 4096x14336; the
base model and the default draft length gamma = 3 of the BitNest-Llama-3-8B
model card): three draft passes at M = 1 (hi plane only) and one target
(verify) pass at M = gamma + 1 = 4 (hi and lo planes). Every linear is an
activation quantisation followed by the nested linear, 4 passes x 32 layers
x 4 linears; the quantisation runs inside the linear's launch except for the
verify pass's gate_up and down_proj (four tokens; N = 28672, K = 14336), which
take a quantisation launch first: 576 launches per round, replayed from one
HIP graph. Weights are seeded synthetic tensors in the layout and with
the distributions of the weight package (generated on the GPU, 3.49 GB per
plane, so the stream is far larger than the 256 MB Infinity Cache); they are
resident in HBM before timing starts.

Printed: one JSON line with the aggregate plane GB/s of the round (plane bytes
read / time per round), the roofline of the dominant kernel (the
plane-streaming GEMV, timed per launch with HIP events on the launch stream),
the measured read ceiling per plane size, per-linear timings against it, the
next rows' timings, and the CPU oracle's throughput (all host threads and
one thread) on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
COLD_BYTES = 512 << 20         # distinct bytes a cold-read cycle covers (2x the 256 MiB Infinity Cache)
# buffer sizes of the read ceiling: each linear's plane bytes (draft: hi,
# target: hi + lo) of the Llama-3-8B shapes, and a large buffer
READ_CEILING_MIB = (8, 12, 16, 24, 28, 56, 112, 2048)
GAMMA = 3


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-baseline", dest="cpu_baseline", action="store_true", default=True)
    p.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU work for the oracle baseline sample")
    p.add_argument("--no-kernel-timing", dest="kernel_timing", action="store_false", default=True)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run one plain device copy of MIB MiB before timing (a known-size "
                        "reference dispatch for hardware byte counters)")
    p.add_argument("--verify-batches", default="8,16,32",
                   help="token counts for the batched-verify (matrix-core) layer timing; empty to skip")
    p.add_argument("--no-read-ceiling", dest="read_ceiling", action="store_false", default=True,
                   help="skip the streaming-read ceiling (bitnest_stream_read per buffer size)")
    p.add_argument("--no-per-linear", dest="per_linear", action="store_false", default=True,
                   help="skip the per-linear timing (each shape on its own, draft/target M=1, target M=4)")
    p.add_argument("--no-r4", dest="r4", action="store_false", default=True,
                   help="skip the R4 (rotated down_proj input) timing")
    p.add_argument("--no-pack", dest="pack", action="store_false", default=True,
                   help="skip the offline packer timing")
    p.add_argument("--no-accept", dest="accept", action="store_false", default=True,
                   help="skip the greedy-verification timing")
    p.add_argument("--no-kv", dest="kv", action="store_false", default=True,
                   help="skip the nested-KV attention timing")
    p.add_argument("--unfused", action="store_true",
                   help="quantise with its own launch before each linear instead of the fused call")
    p.add_argument("--verbose", action="store_true")
    return p.parse_args(argv)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Stack:
    """Weights of every layer and the per-pass activation inputs, on the GPU."""

    def __init__(self, layers, seed, device):
        import torch
        from w8_quantized_linear_amd import synth
        self.linears = synth.LLAMA3_8B_LINEARS
        self.layers = layers
        self.seed = seed
        self.device = device
        self.extra = {}          # linear index -> weights past the stack's layers (cold cycles)
        self.w = []
        for l in range(layers):
            self.w.append([synth.make_weights(N, K, seed=seed, layer=l, linear=i, device=device)
                           for i, (_, N, K, _) in enumerate(self.linears)])
        # activation inputs: draft pass p (M = 1) and the verify pass (M = gamma + 1)
        self.x_draft = [[[synth.make_activations(1, K, seed=seed, layer=l, linear=i, step=p, device=device)
                          for i, (_, _, K, _) in enumerate(self.linears)] for l in range(layers)]
                        for p in range(GAMMA)]
        self.x_verify = [[synth.make_activations(GAMMA + 1, K, seed=seed, layer=l, linear=i, step=GAMMA,
                                                 device=device)
                          for i, (_, _, K, _) in enumerate(self.linears)] for l in range(layers)]
        # per-shape work buffers (reused across layers, as a decoder would)
        self.buf = {}
        for M in (1, GAMMA + 1):
            for i, (_, N, K, g) in enumerate(self.linears):
                self.buf[(M, i)] = (
                    torch.empty((M, K), dtype=torch.int8, device=device),
                    torch.empty((M,) if g == 0 else (M, K // 128), dtype=torch.float32, device=device),
                    torch.empty((M, N), dtype=torch.float32, device=device))
        torch.cuda.synchronize()

    def plane_bytes_per_round(self):
        per_layer = sum(N * K // 2 for (_, N, K, _) in self.linears)
        return self.layers * per_layer * (GAMMA * 1 + 2)

    def gemv_algorithmic_bytes_per_round(self):
        """Bytes the round's linear launches must move at least, summed: plane
        bytes, fp16 scales, the activation input (fp32 x for a fused launch,
        int8 codes otherwise), the codes and scales a fused launch writes,
        and the fp32 outputs."""
        import w8_quantized_linear_amd as bn
        tot = 0
        for M, planes, passes in ((1, 1, GAMMA), (GAMMA + 1, 2, 1)):
            for (_, N, K, g) in self.linears:
                S = 1 if g == 0 else K // 128
                b = planes * N * K // 2 + N * (K // 128) * 2 + M * N * 4
                if bn.fused_in_one_launch(M, N, K):
                    b += 4 * M * K + M * K + 4 * M * S
                else:
                    b += M * K + 4 * M * S
                tot += passes * self.layers * b
        return tot

    def algorithmic_bytes_per_round(self):
        """All bytes the round must move at least: the linear launches'
        (gemv_algorithmic_bytes_per_round) plus those of the separate
        quantisation launches of the calls that take two launches (fp32 rows
        read, codes and activation scales written)."""
        import w8_quantized_linear_amd as bn
        tot = self.gemv_algorithmic_bytes_per_round()
        for M, passes in ((1, GAMMA), (GAMMA + 1, 1)):
            for (_, N, K, g) in self.linears:
                if not bn.fused_in_one_launch(M, N, K):
                    S = 1 if g == 0 else K // 128
                    tot += passes * self.layers * (4 * M * K + M * K + 4 * M * S)
        return tot

    def gemv_launches_per_round(self):
        return (GAMMA + 1) * self.layers * len(self.linears)

    def cold_weights(self, i, planes, at_least=COLD_BYTES):
        """Distinct weights of linear i whose `planes` plane bytes add up to
        at least `at_least` (the stack's layers first, then extra seeded
        layers of the same shape), so that cycling through them reads every
        byte from HBM: twice the 256 MiB Infinity Cache."""
        from w8_quantized_linear_amd import synth
        _, N, K, _ = self.linears[i]
        need = -(-at_least // (planes * N * K // 2))
        ws = [self.w[l][i] for l in range(min(need, self.layers))]
        extra = self.extra.setdefault(i, [])
        while len(ws) + len(extra) < need:
            extra.append(synth.make_weights(N, K, seed=self.seed, layer=self.layers + len(extra), linear=i,
                                            device=self.device))
        return ws + extra[:need - len(ws)]


def run_round(stack, bn, mode="fused", rot_block=0):
    """One speculative round: 3 draft passes at M = 1, one verify pass at M = 4.

    mode "fused": each linear quantises its fp32 input and runs the nested
    linear in one call (bitnest_quant_linear_*); "unfused": bitnest_quant_act
    then bitnest_linear_*; "linear_only": the linear launches of the fused
    round and nothing else (linears whose fused call is two launches run only
    their linear, on the codes already in the buffers) - used to time the
    dominant kernel on its own. rot_block > 0 (with mode "fused"): the
    down_proj input also takes the R4 rotation (blocks of rot_block columns)
    before its quantisation, as the model card's recipe does."""
    for p in range(GAMMA + 1):
        verify = p == GAMMA
        M = GAMMA + 1 if verify else 1
        for l in range(stack.layers):
            for i, (name, N, K, g) in enumerate(stack.linears):
                xq, xs, y = stack.buf[(M, i)]
                w = stack.w[l][i]
                x = stack.x_verify[l][i] if verify else stack.x_draft[p][l][i]
                one = bn.fused_in_one_launch(M, N, K)
                if rot_block and mode == "fused" and name == "down":
                    if verify:
                        bn.bitnest_hadamard_quant_linear_target(x, rot_block, w.hi, w.lo, w.scale, y=y, xq=xq, xs=xs)
                    else:
                        bn.bitnest_hadamard_quant_linear_draft(x, rot_block, w.hi, w.scale, y=y, xq=xq, xs=xs)
                    continue
                if mode == "fused" or (mode == "linear_only" and one):
                    if verify:
                        bn.bitnest_quant_linear_target(x, w.hi, w.lo, w.scale, g, y=y, xq=xq, xs=xs)
                    else:
                        bn.bitnest_quant_linear_draft(x, w.hi, w.scale, g, y=y, xq=xq, xs=xs)
                    continue
                if mode == "unfused":
                    bn.bitnest_quant_act(x, g, xq=xq, xs=xs)
                if verify:
                    bn.bitnest_linear_target(xq, xs, w.hi, w.lo, w.scale, g, y=y)
                else:
                    bn.bitnest_linear_draft(xq, xs, w.hi, w.scale, g, y=y)


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def gemv_kernel_timing(stack, bn, steps):
    """Average launch duration of the linear kernel: the round's 512 linear
    launches (same shapes, weights and order as the timed round, without the
    separate quantisation launches of the linears that need one) replayed
    back to back from a HIP graph, timed with HIP events on the stream they
    run on, divided by the number of launches. Gaps between dispatches are
    included, so this can only overstate the duration."""
    import torch
    n = stack.gemv_launches_per_round()
    g = capture(lambda: run_round(stack, bn, mode="linear_only"))
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(max(3, steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / n)
    per.sort()
    return per[len(per) // 2] * 1e-3     # seconds per launch, median over replays


INT8_DENSE_PEAK_OPS = 5.0e15       # MI355X dense int8 matrix-core peak, ops/s


READ_CONFIGS = ((2, 0), (4, 0), (8, 0), (4, 8), (8, 8), (4, 16), (8, 16))   # (depth, waves per CU; 0 = all)


def read_ceiling(bn, reps=5):
    """The HBM read ceiling per buffer size: bitnest_stream_read (the plane
    stream's loads, no arithmetic) over a cycle of distinct buffers of that
    size covering at least 512 MiB (one buffer of 2 GiB), so every launch
    reads cold memory, replayed from a HIP graph and timed with HIP events,
    launch overhead included as it is for a linear of the same plane bytes.
    Every (items in flight per wave, waves per CU) of READ_CONFIGS is timed;
    the ceiling is the fastest, reported with its configuration."""
    import torch
    out = {}
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    for mib in READ_CEILING_MIB:
        size = mib << 20
        count = max(1, -(-COLD_BYTES // size))
        pool = torch.empty((count, size), dtype=torch.uint8, device="cuda")
        best = None
        for depth, wpc in READ_CONFIGS:
            def fn(pool=pool, count=count, depth=depth, wpc=wpc):
                for c in range(count):
                    bn.bitnest_stream_read(pool[c], sink, depth=depth, waves_per_cu=wpc)
            g = capture(fn)
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3 / count)
            t = sorted(ts)[len(ts) // 2]
            if best is None or t < best[0]:
                best = (t, depth, wpc)
            del g
        t, depth, wpc = best
        out["%dMiB" % mib] = {"us": round(t * 1e6, 3), "GBps": round(size / t / 1e9, 1),
                              "frac": round(size / t / 1e9 / HBM_PEAK_GBS, 4), "buffers": count,
                              "depth": depth, "waves_per_cu": wpc or "max"}
        del pool
        torch.cuda.empty_cache()
    log("read ceiling: %s" % ", ".join("%s %.0f GB/s (%.2f us)" % (k, v["GBps"], v["us"]) for k, v in out.items()))
    return out


def per_linear(stack, bn, ceiling=None, reps=5):
    """Each linear shape on its own: a cycle of launches over distinct
    weights of that shape covering at least 512 MiB of plane bytes (the
    stack's layers, then extra seeded layers), so that every launch reads
    cold weights, replayed from a HIP graph and timed with HIP events; us per
    launch and plane GB/s with its fraction of the 8 TB/s peak and of the
    measured read ceiling at the same number of bytes. Modes: draft M=1 and
    target M=1 (the fused call, one launch), target M=4 (the linear on ready
    codes; its separate quantisation launch is timed on its own as
    quant_M4, one launch per layer), and verify_M4: the fused call at M=4 as
    the round makes it where that is one launch (K <= 4096: qkv, o_proj,
    gate_up)."""
    import torch
    out = {}
    L = stack.layers

    def timed(fn, n):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / n)
        return sorted(ts)[len(ts) // 2]

    for mode in ("draft_M1", "target_M1", "target_M4", "quant_M4", "verify_M4"):
        res = {}
        for i, (name, N, K, g) in enumerate(stack.linears):
            M = 4 if "M4" in mode else 1
            if mode == "verify_M4" and not bn.fused_in_one_launch(M, N, K):
                continue
            xq, xs, y = stack.buf[(M, i)]

            planes = 1 if mode == "draft_M1" else 2
            ws = stack.cold_weights(i, planes) if mode != "quant_M4" else []
            n = len(ws) if ws else L

            def fn(i=i, g=g, xq=xq, xs=xs, y=y, ws=ws):
                for l in range(n):
                    w = ws[l] if ws else None
                    if mode == "draft_M1":
                        bn.bitnest_quant_linear_draft(stack.x_draft[0][l % L][i], w.hi, w.scale, g,
                                                      y=y, xq=xq, xs=xs)
                    elif mode == "target_M1":
                        bn.bitnest_quant_linear_target(stack.x_draft[0][l % L][i], w.hi, w.lo, w.scale, g,
                                                       y=y, xq=xq, xs=xs)
                    elif mode == "target_M4":
                        bn.bitnest_linear_target(xq, xs, w.hi, w.lo, w.scale, g, y=y)
                    elif mode == "verify_M4":
                        bn.bitnest_quant_linear_target(stack.x_verify[l % L][i], w.hi, w.lo, w.scale, g,
                                                       y=y, xq=xq, xs=xs)
                    else:
                        bn.bitnest_quant_act(stack.x_verify[l][i], g, xq=xq, xs=xs)
            if mode == "target_M4":
                bn.bitnest_quant_act(stack.x_verify[0][i], g, xq=xq, xs=xs)
            t = timed(fn, n)
            entry = {"us": round(t * 1e6, 3)}
            if mode != "quant_M4":
                plane = N * K // 2 * planes
                gbs = plane / t / 1e9
                entry.update({"plane_GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                              "cold_set": {"launches": n, "plane_bytes": n * plane}})
                ceil = (ceiling or {}).get("%dMiB" % (plane >> 20))
                if ceil and plane % (1 << 20) == 0:
                    entry["of_read_ceiling"] = round(gbs / ceil["GBps"], 4)
            res[name] = entry
        out[mode] = res
        log("per linear %s: %s" % (mode, ", ".join("%s %.2f us%s" % (k, v["us"], (" %.0f GB/s" % v["plane_GBps"])
                                                                      if "plane_GBps" in v else "")
                                                     for k, v in res.items())))
    return out


def batched_verify(stack, bn, batches, reps=20):
    """Target linears of one layer at M in `batches` (several sequences of
    gamma + 1 verify tokens), on the int8 matrix-core kernel. Each M is
    timed as a HIP graph of `reps` passes over distinct layers (cold weights)
    with HIP events; reports per-layer time, plane GB/s and the matrix-core
    utilisation implied by the method's integer ops (2 M N K per plane)."""
    import torch
    from w8_quantized_linear_amd import synth
    out = {}
    layers = list(range(min(stack.layers, reps)))
    for M in batches:
        xs_in = [synth.make_activations(M, K, seed=7, layer=l, linear=i, step=M, device="cuda")
                 for l in layers for i, (_, _, K, _) in enumerate(stack.linears)]
        bufs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"),
                 torch.empty((M,) if g == 0 else (M, K // 128), dtype=torch.float32, device="cuda"),
                 torch.empty((M, N), dtype=torch.float32, device="cuda")) for (_, N, K, g) in stack.linears]
        xq_all = []
        for j, x in enumerate(xs_in):
            i = j % len(stack.linears)
            g = stack.linears[i][3]
            xq_all.append(bn.bitnest_quant_act(x, g))

        def layer_pass():
            for j, l in enumerate(layers):
                for i, (_, N, K, g) in enumerate(stack.linears):
                    xq, xs = xq_all[j * len(stack.linears) + i]
                    w = stack.w[l][i]
                    bn.bitnest_linear_target(xq, xs, w.hi, w.lo, w.scale, g, y=bufs[i][2])
        graph = capture(layer_pass)
        graph.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / len(layers))
        t = sorted(times)[len(times) // 2]
        plane = sum(N * K for (_, N, K, _) in stack.linears)          # both planes: 2 * N*K/2
        ops = 2 * M * 2 * sum(N * K for (_, N, K, _) in stack.linears)
        out[str(M)] = {"layer_us": round(t * 1e6, 2), "plane_GBps": round(plane / t / 1e9, 1),
                       "pct_hbm_peak": round(100 * plane / t / 1e9 / HBM_PEAK_GBS, 2),
                       "int_ops_per_s": float("%.4g" % (ops / t)),
                       "mfma_util_pct": round(100 * ops / t / INT8_DENSE_PEAK_OPS, 2)}
        log("batched verify M=%d: %.2f us/layer, %.1f GB/s, MFMA util %.2f%%"
            % (M, t * 1e6, plane / t / 1e9, 100 * ops / t / INT8_DENSE_PEAK_OPS))
    return out


def r4_timing(stack, bn, block=512, steps=10, reps=5):
    """The down_proj input with the R4 rotation (model card recipe: an online
    Hadamard on the down_proj inputs; here blocks of `block` columns): the
    fused one-token draft and target launches, the rotation + quantisation
    launch at M=4, each over the stack's layers from a HIP graph; and the
    whole round with the rotation on every down_proj input."""
    import torch
    i = [n for (n, _, _, _) in stack.linears].index("down")
    _, N, K, _ = stack.linears[i]
    L = stack.layers
    out = {"block": block}

    def timed(fn, n):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / n)
        return sorted(ts)[len(ts) // 2]

    xq1, xs1, y1 = stack.buf[(1, i)]
    xq4, xs4, y4 = stack.buf[(GAMMA + 1, i)]
    for mode in ("draft_M1", "target_M1"):
        def fn(mode=mode):
            for l in range(L):
                w = stack.w[l][i]
                if mode == "draft_M1":
                    bn.bitnest_hadamard_quant_linear_draft(stack.x_draft[0][l][i], block, w.hi, w.scale,
                                                           y=y1, xq=xq1, xs=xs1)
                else:
                    bn.bitnest_hadamard_quant_linear_target(stack.x_draft[0][l][i], block, w.hi, w.lo, w.scale,
                                                            y=y1, xq=xq1, xs=xs1)
        t = timed(fn, L)
        plane = N * K // 2 * (1 if mode == "draft_M1" else 2)
        out["down_" + mode] = {"us": round(t * 1e6, 3), "plane_GBps": round(plane / t / 1e9, 1),
                               "frac": round(plane / t / 1e9 / HBM_PEAK_GBS, 4)}
    t = timed(lambda: [bn.bitnest_hadamard_quant_act(stack.x_verify[l][i], block, xq=xq4, xs=xs4)
                       for l in range(L)], L)
    out["rotate_quant_M4_us"] = round(t * 1e6, 3)
    g = capture(lambda: run_round(stack, bn, mode="fused", rot_block=block))
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = stack.plane_bytes_per_round() / (ms * 1e-3) / 1e9
    out["round_ms"] = round(ms, 4)
    out["round_plane_GBps"] = round(gbs, 1)
    out["round_pct_hbm_peak"] = round(100 * gbs / HBM_PEAK_GBS, 2)
    log("R4 (block %d): down draft M=1 %.2f us, target M=1 %.2f us, rotate+quant M=4 %.2f us; round %.3f ms"
        % (block, out["down_draft_M1"]["us"], out["down_target_M1"]["us"], out["rotate_quant_M4_us"], ms))
    return out


def pack_buffers(N, K):
    """Distinct fp32 weight buffers the packer timing rotates through for an
    [N, K] shape: more than 512 MiB of inputs, at least two."""
    return max(2, -(-(512 << 20) // (4 * N * K)))


def pack_timing(stack, bn, reps=5):
    """The offline nested packer on each Llama-3-8B linear shape: fp32
    weights (cold: buffers rotate through more memory than the caches hold)
    -> hi / lo planes and fp16 scales. us per linear and GB/s of its
    algorithmic bytes (4 N K read, N K planes + 2 N K/128 scales written)
    with the fraction of the 8 TB/s peak."""
    import torch
    out = {}
    g = torch.Generator(device="cuda").manual_seed(1234)
    for (name, N, K, _) in stack.linears:
        nbuf = pack_buffers(N, K)
        Ws = [torch.randn((N, K), generator=g, device="cuda") * 0.02 for _ in range(nbuf)]
        hi = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
        lo = torch.empty_like(hi)
        sc = torch.empty((N, K // 128), dtype=torch.int16, device="cuda")

        def fn():
            for W in Ws:
                bn.bitnest_pack_nested(W, hi, lo, sc)
        graph = capture(fn)
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3 / nbuf)
        t = sorted(ts)[len(ts) // 2]
        nbytes = 4 * N * K + N * K + 2 * N * (K // 128)
        gbs = nbytes / t / 1e9
        out[name] = {"us": round(t * 1e6, 2), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bytes": nbytes}
        del Ws
        torch.cuda.empty_cache()
    log("pack: " + ", ".join("%s %.1f us %.0f GB/s" % (k, v["us"], v["GBps"]) for k, v in out.items()))
    return out


def accept_timing(bn, V=128256, calls=32, reps=5):
    """Greedy verification of one round (gamma + 1 = 4 verify rows over the
    Llama-3 vocabulary, fp32 logits, cold: a different logits buffer each
    call) replayed from a HIP graph: us per call and GB/s of logits read."""
    import torch
    R = GAMMA + 1
    g = torch.Generator(device="cuda").manual_seed(99)
    logits = [torch.randn((R, V), generator=g, device="cuda") for _ in range(calls)]
    draft = torch.zeros((R - 1,), dtype=torch.int32, device="cuda")
    targ = torch.empty((R,), dtype=torch.int32, device="cuda")
    res = torch.empty((2,), dtype=torch.int32, device="cuda")
    work = torch.empty((bn.bitnest_greedy_accept_workspace_bytes(R, V),), dtype=torch.uint8, device="cuda")
    graph = capture(lambda: [bn.bitnest_greedy_accept(lg, draft, targ, res, work) for lg in logits])
    graph.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3 / calls)
    t = sorted(ts)[len(ts) // 2]
    out = {"rows": R, "vocab": V, "us": round(t * 1e6, 3), "GBps": round(4 * R * V / t / 1e9, 1)}
    log("greedy accept: %.2f us per call (%d x %d fp32 logits)" % (t * 1e6, R, V))
    return out


def kv_timing(bn, layers=32, contexts=(2048, 8192, 32768), Hq=32, Hkv=8, reps=5):
    """Decode attention over the nested KV cache at the Llama-3-8B head layout
    (32 query heads, 8 KV heads, head dimension 128): the draft step (M=1,
    KV4: hi planes) and the verify pass (M=4, KV8: hi+lo planes), one call
    per layer over `layers` distinct caches (cold) from a HIP graph; each
    cache is head-major, exactly T positions per head. us per call and GB/s
    of cache bytes read (planes + fp16 scales of K and V)."""
    import torch
    out = {}
    g = torch.Generator(device="cuda").manual_seed(77)
    for T in contexts:
        caches = []
        for _ in range(layers):
            planes = [torch.randint(0, 256, (Hkv, T, 64), dtype=torch.uint8, device="cuda", generator=g)
                      for _ in range(4)]                 # k_hi, k_lo, v_hi, v_lo
            scales = [(torch.rand((Hkv, T), device="cuda", generator=g) * 0.02 + 0.005).half().view(torch.int16)
                      for _ in range(2)]
            caches.append((planes, scales))
        res = {}
        for M, kv8 in ((1, False), (GAMMA + 1, True)):
            q = torch.randn((M, Hq, 128), device="cuda", generator=g)
            o = torch.empty((M, Hq, 128), device="cuda")
            work = torch.empty((bn.bitnest_kv_attention_workspace_bytes(M, Hq, T),), dtype=torch.uint8, device="cuda")

            def fn(q=q, o=o, work=work, kv8=kv8):
                for (kh, kl, vh, vl), (ks, vs) in caches:
                    bn.bitnest_kv_attention(q, kh, ks, vh, vs, kl if kv8 else None, vl if kv8 else None,
                                            out=o, work=work)
            graph = capture(fn)
            graph.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3 / layers)
            t = sorted(ts)[len(ts) // 2]
            nbytes = 2 * T * Hkv * (64 * (2 if kv8 else 1) + 2)
            key = "draft_M1_KV4" if not kv8 else "verify_M4_KV8"
            res[key] = {"us": round(t * 1e6, 2), "cache_bytes": nbytes, "GBps": round(nbytes / t / 1e9, 1),
                        "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        out[str(T)] = res
        del caches
        torch.cuda.empty_cache()
        log("nested KV attention T=%d: %s" % (T, ", ".join("%s %.2f us %.0f GB/s" % (k, v["us"], v["GBps"])
                                                            for k, v in res.items())))
    return out


def measured_traffic():
    """HBM bytes per linear launch from the committed hardware-counter
    profile (rocprofv3 FETCH_SIZE and WRITE_SIZE of the round's launches,
    scaled by a known-size copy), or None when the kernel sources have
    changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_planes_round_traffic.json")
    try:
        with open(path) as f:
            prof = json.load(f)
        h = hashlib.sha256()
        for src in prof["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return prof["traffic_bytes_per_launch"] if h.hexdigest() == prof["sources_sha256"] else None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(stack, budget_s, threads=None):
    """The oracle on the machine's host cores over a bounded sample of the round:
    the first layer(s) of the stack, 3 draft passes + 1 verify pass each,
    quantisation plus linear, until about `budget_s` seconds of CPU work
    (at least one layer). `threads`: the oracle's thread count (default: all
    it may use)."""
    import oracle
    threads = oracle.max_threads() if threads is None else threads
    done_bytes = 0
    t_total = 0.0
    layers_done = 0
    for l in range(stack.layers):
        host = [w.numpy() for w in stack.w[l]]
        t0 = time.perf_counter()
        for p in range(GAMMA + 1):
            verify = p == GAMMA
            for i, (_, N, K, g) in enumerate(stack.linears):
                x = (stack.x_verify[l][i] if verify else stack.x_draft[p][l][i]).cpu().numpy()
                hi, lo, sc = host[i]
                q, s = oracle.quant_act(x, g)
                oracle.linear(q, s, hi, sc, lo if verify else None, g, threads=threads)
                done_bytes += N * K // 2 * (2 if verify else 1)
        t_total += time.perf_counter() - t0
        layers_done += 1
        if t_total >= budget_s:
            break
    gbs = done_bytes / t_total / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d layers of the round (3 draft passes at M=1 + 1 verify pass at M=4 per layer, "
                      "activation quant + dequantise-then-multiply in fp64), %.1f s; plane bytes %d"
                      % (layers_done, stack.layers, t_total, done_bytes)}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2
    import torch
    import w8_quantized_linear_amd as bn
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    bn.lib()                            # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    t0 = time.perf_counter()
    stack = Stack(args.layers, args.seed, dev)
    log("stack ready: %d layers, %.2f GB of planes per round, %.1f s"
        % (args.layers, stack.plane_bytes_per_round() / 1e9, time.perf_counter() - t0))

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    fused = not args.unfused
    graph = capture(lambda: run_round(stack, bn, mode="fused" if fused else "unfused"))
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    plane_bytes = stack.plane_bytes_per_round()
    alg_bytes = stack.algorithmic_bytes_per_round()
    value = plane_bytes / (ms_per_step * 1e-3) / 1e9
    log("timed %d rounds: %.3f ms/round wall, %.3f ms/round events" % (args.steps, ms_per_step, ev_ms))

    roofline = None
    if args.kernel_timing:
        t_gemv = gemv_kernel_timing(stack, bn, min(args.steps, 10))
        per_launch_bytes = stack.gemv_algorithmic_bytes_per_round() / stack.gemv_launches_per_round()
        achieved = per_launch_bytes / t_gemv / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                    "kernel": "gemv_planes_kernel (draft M=1 and target M=4 instantiations, fused "
                              "quantisation where the round uses it)",
                    "avg_launch_us": round(t_gemv * 1e6, 3),
                    "algorithmic_bytes_per_launch": int(per_launch_bytes)}
        log("GEMV: %.3f us per launch (events), %.1f GB/s algorithmic" % (t_gemv * 1e6, achieved))

    ceiling = read_ceiling(bn) if args.read_ceiling else None
    linears = per_linear(stack, bn, ceiling) if args.per_linear else None
    r4 = r4_timing(stack, bn, steps=min(args.steps, 10)) if args.r4 else None
    pack = pack_timing(stack, bn) if args.pack else None
    accept = accept_timing(bn) if args.accept else None
    kv = kv_timing(bn) if args.kv else None

    verify = None
    batches = [int(v) for v in args.verify_batches.split(",") if v.strip()]
    if batches:
        verify = batched_verify(stack, bn, batches)

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(stack, args.cpu_seconds)
        cpu["cpu_model"] = cpu_model()
        log("cpu oracle: %s GB/s on %d threads (%s)" % (cpu["value"], cpu["cores"], cpu["cpu_model"]))
        one = cpu_baseline(stack, args.cpu_seconds / 2, threads=1)
        cpu["one_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
        log("cpu oracle: %s GB/s on 1 thread" % one["value"])

    out = {
        "metric": "nested W4/W8 linear: plane GB/s (% HBM peak), draft M=1 & verify M=4",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B linear stack (%d layers x qkv/o_proj/gate_up/down), one speculative "
                               "round: %d draft passes M=1 (hi plane) + 1 verify pass M=%d (hi+lo planes), "
                               "act quant + nested linear per linear" % (args.layers, GAMMA, GAMMA + 1),
                   "layers": args.layers, "gamma": GAMMA, "plane_bytes_per_round": plane_bytes,
                   "algorithmic_bytes_per_round": alg_bytes,
                   "quant": "fused into the linear launch" if fused else "separate launch",
                   "replay": "hip_graph"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "algorithmic_GBps": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "roofline": roofline,
        "read_ceiling": ceiling,
        "per_linear": linears,
        "r4": r4,
        "pack": pack,
        "accept": accept,
        "kv_attention": kv,
        "batched_verify": verify,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
