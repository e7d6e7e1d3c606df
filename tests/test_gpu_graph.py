"""Graph replay of the calls a speculative round makes, through the C ABI.

The benchmark times a round as one captured HIP graph of quantise + linear
calls. This checks that such a graph computes what the same calls compute
eagerly, bit for bit (same kernels, same launch shapes, deterministic
reductions), on every replay: the graph is replayed several times, with the
outputs poisoned before each replay (NaN outputs and scales, codes of -128,
a value the quantiser never writes), with eager launches and
synchronisation between replays, and with new inputs copied into the
captured input buffers between replays (the replay must read them, not
values seen at capture). The calls cover every kernel variant the round
uses: the fused single-token draft and target (per-token and per-group
activation scales, rows of 4096 and 14336 columns), the fused four-token
target, the four-token target taken as a quantisation launch plus a linear
launch (N above the fused rule's limit, K = 14336), the eight-token target
on the matrix cores, and the R4-rotated down_proj input.
"""
import pytest
import torch

import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

# (name, N, K, act_group): the four linear kinds at reduced N, full K
SHAPES = [("qkv", 1536, 4096, 0), ("o_proj", 1024, 4096, 128), ("gate_up", 9216, 4096, 0),
          ("down", 1024, 14336, 0)]
ROT = 512
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _calls():
    """[(kind, M, shape index)]: the launches of one round-like sequence."""
    out = []
    for i, (name, N, K, g) in enumerate(SHAPES):
        out += [("draft", 1, i), ("target", 1, i), ("target", 4, i), ("target", 8, i)]
        if name == "down":
            out += [("rot_draft", 1, i), ("rot_target", 4, i)]
    return out


def _outputs(calls, dev):
    bufs = []
    for kind, M, i in calls:
        _, N, K, g = SHAPES[i]
        gg = 0 if kind.startswith("rot") else g
        bufs.append({"y": torch.empty((M, N), dtype=torch.float32, device=dev),
                     "xq": torch.empty((M, K), dtype=torch.int8, device=dev),
                     "xs": torch.empty((M,) if gg == 0 else (M, K // 128), dtype=torch.float32, device=dev)})
    return bufs


def _run(calls, w, xs_in, bufs):
    for (kind, M, i), b in zip(calls, bufs):
        g = SHAPES[i][3]
        x = xs_in[(M, i)]
        hi, lo, sc = w[i].hi, w[i].lo, w[i].scale
        if kind == "draft":
            bn.bitnest_quant_linear_draft(x, hi, sc, g, y=b["y"], xq=b["xq"], xs=b["xs"])
        elif kind == "target":
            bn.bitnest_quant_linear_target(x, hi, lo, sc, g, y=b["y"], xq=b["xq"], xs=b["xs"])
        elif kind == "rot_draft":
            bn.bitnest_hadamard_quant_linear_draft(x, ROT, hi, sc, y=b["y"], xq=b["xq"], xs=b["xs"])
        else:
            bn.bitnest_hadamard_quant_linear_target(x, ROT, hi, lo, sc, y=b["y"], xq=b["xq"], xs=b["xs"])


def _poison(bufs):
    for b in bufs:
        b["y"].fill_(float("nan"))
        b["xs"].fill_(float("nan"))
        b["xq"].fill_(-128)


def _same(bufs, ref):
    for j, (b, r) in enumerate(zip(bufs, ref)):
        for k in ("y", "xq", "xs"):
            assert torch.equal(_bits(b[k]), _bits(r[k])), (j, k)


def test_round_calls_replayed_from_a_graph():
    dev = torch.device("cuda", 0)
    calls = _calls()
    assert any(not bn.fused_in_one_launch(M, SHAPES[i][1], SHAPES[i][2])
               for kind, M, i in calls if kind == "target" and M == 4)      # a two-launch call is covered
    assert any(bn.fused_in_one_launch(M, SHAPES[i][1], SHAPES[i][2])
               for kind, M, i in calls if kind == "target" and M == 4)      # and a fused one
    w = [synth.make_weights(N, K, seed=31, linear=i, device=dev) for i, (_, N, K, _) in enumerate(SHAPES)]
    keys = sorted({(M, i) for _, M, i in calls})
    xs_in = {(M, i): synth.make_activations(M, SHAPES[i][2], seed=31, linear=i, step=M, device=dev)
             for (M, i) in keys}

    graph_bufs = _outputs(calls, dev)
    eager_bufs = _outputs(calls, dev)
    # warm-up on the capture stream, then capture
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(calls, w, xs_in, graph_bufs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _run(calls, w, xs_in, graph_bufs)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        if r % 2 == 1:
            # new inputs, written into the buffers the graph captured
            for (M, i), x in xs_in.items():
                x.copy_(synth.make_activations(M, SHAPES[i][2], seed=31, linear=i, step=100 + r, device=dev))
        _poison(eager_bufs)
        _run(calls, w, xs_in, eager_bufs)        # eager reference on the current inputs
        torch.cuda.synchronize()
        _poison(graph_bufs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(graph_bufs, eager_bufs)
        assert all(torch.isfinite(b["y"]).all() for b in graph_bufs)
