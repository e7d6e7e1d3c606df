"""GPU parity of the linear chain (bitnest_linear_chain: a sequence of
quantise + linear steps in one launch with device-side waits between the
links) through the C ABI.

Bars: every output of the chain (codes, activation scales, y) is bit for bit
that of the single calls bitnest_quant_linear_draft / _target made one after
another on the same tensors (which are checked against the oracle in
test_gpu_parity.py); y of small chains is also compared with the oracle
(within 1e-5 * max|y|, codes exact). A link whose input is the previous
link's output checks that the waits order the links; the workspace's
arrival counter is back at zero after every call.
"""
import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t


def _links(shapes, M, target, seed, outs=True):
    """Links over independent seeded inputs: shapes = [(N, K, act_group)]."""
    links = []
    for i, (N, K, g) in enumerate(shapes):
        w = synth.make_weights(N, K, seed=seed, layer=i, linear=N % 89, with_lo=target, device="cuda")
        x = synth.make_activations(M, K, seed=seed, layer=i, linear=K % 97, device="cuda")
        d = dict(x=x, hi=w.hi, scale=w.scale, y=torch.empty((M, N), device="cuda"), act_group=g, w=w)
        if target:
            d["lo"] = w.lo
        if outs:
            d["xq"] = torch.empty((M, K), dtype=torch.int8, device="cuda")
            d["xs"] = torch.empty((M,) if g == 0 else (M, K // 128), device="cuda")
        links.append(d)
    return links


def _single_calls(links, target):
    """The same steps as single calls, one after another: (y, xq, xs) per link."""
    out = []
    for d in links:
        if target:
            y, q, s = bn.bitnest_quant_linear_target(d["x"], d["hi"], d["lo"], d["scale"], d["act_group"])
        else:
            y, q, s = bn.bitnest_quant_linear_draft(d["x"], d["hi"], d["scale"], d["act_group"])
        out.append((y, q, s))
    return out


def _check_same(links, ref):
    for j, (d, (y, q, s)) in enumerate(zip(links, ref)):
        assert torch.equal(_bits(d["y"]), _bits(y)), "link %d: y" % j
        if "xq" in d:
            assert torch.equal(d["xq"], q), "link %d: codes" % j
            assert torch.equal(_bits(d["xs"]), _bits(s)), "link %d: scales" % j


def _counter_words(chain):
    w = chain.work[:8].view(torch.int32).cpu().tolist()
    return w[0], w[1]


LAYER = [(n, k, g) for (_, n, k, g) in synth.LLAMA3_8B_LINEARS]


@pytest.mark.parametrize("M,target", [(1, False), (1, True), (2, True), (3, False), (4, True), (4, False)])
def test_chain_of_llama_layers_equals_single_calls(M, target):
    # two Llama-3-8B decoder layers (qkv, o_proj with per-group activation
    # scales, gate_up, down): 8 links, every output bit-identical
    links = _links(LAYER * 2, M, target, seed=11)
    chain = bn.LinearChain(links)
    chain.run()
    ref = _single_calls(links, target)
    torch.cuda.synchronize()
    _check_same(links, ref)
    assert _counter_words(chain) == (0, 0)


def _oracle_y(d, target):
    hi, lo, sc = d["w"].numpy()
    q, s = oracle.quant_act(d["x"].cpu().numpy(), d["act_group"])
    return q, s, oracle.linear(q, s, hi, sc, lo if target else None, d["act_group"])


# ragged N (fewer rows than waves, a ragged last wave), K from one group to
# the widest input, one link with no rows (quantisation only), mixed widths
SMALL = [(256, 512, 0), (37, 640, 128), (0, 384, 0), (1000, 2176, 0), (5, 128, 128), (2049, 16384, 0),
         (129, 4096, 128), (70, 14336, 0), (4096, 256, 0)]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("target", [False, True])
def test_chain_small_shapes_match_oracle(M, target):
    links = _links(SMALL, M, target, seed=12)
    chain = bn.LinearChain(links)
    chain.run()
    ref = _single_calls(links, target)
    torch.cuda.synchronize()
    _check_same(links, ref)
    for j, d in enumerate(links):
        q, s, y64 = _oracle_y(d, target)
        assert np.array_equal(d["xq"].cpu().numpy(), q), j
        assert np.array_equal(d["xs"].cpu().numpy(), s), j
        y = d["y"].double().cpu().numpy()
        if y.size:
            assert np.abs(y - y64).max() <= TOL * np.abs(y64).max() + 1e-30, j
    assert _counter_words(chain) == (0, 0)


@pytest.mark.parametrize("M,target", [(1, False), (4, True), (2, False)])
def test_chain_link_reads_previous_output(M, target):
    # x of link j + 1 IS y of link j (square shapes): the chain must read each
    # input only after the previous link has written all of it; the result is
    # the single calls' one after another, bit for bit
    shapes = [(4096, 4096, 128), (4096, 4096, 0), (2048, 4096, 0), (2048, 2048, 128), (4096, 2048, 0),
              (4096, 4096, 0)]
    links = _links(shapes, M, target, seed=13, outs=False)
    for j in range(1, len(links)):
        links[j]["x"] = links[j - 1]["y"]
    chain = bn.LinearChain(links)
    chain.run()
    torch.cuda.synchronize()
    got = [d["y"].clone() for d in links]
    # the same steps one after another on fresh outputs
    prev = links[0]["x"]
    for j, d in enumerate(links):
        x = prev if j else d["x"]
        if target:
            y, _, _ = bn.bitnest_quant_linear_target(x, d["hi"], d["lo"], d["scale"], d["act_group"])
        else:
            y, _, _ = bn.bitnest_quant_linear_draft(x, d["hi"], d["scale"], d["act_group"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(got[j])), "link %d" % j
        prev = y
    assert _counter_words(chain) == (0, 0)


def test_chain_runs_again_on_the_same_workspace():
    links = _links(LAYER, 1, False, seed=14)
    chain = bn.LinearChain(links)
    chain.run()
    torch.cuda.synchronize()
    first = [d["y"].clone() for d in links]
    for d in links:
        d["y"].fill_(float("nan"))
    for _ in range(3):
        chain.run()
    torch.cuda.synchronize()
    for d, y in zip(links, first):
        assert torch.equal(_bits(d["y"]), _bits(y))
    assert _counter_words(chain) == (0, 0)


def test_chain_replayed_from_a_graph():
    # captured once, replayed with eager work and synchronisation between the
    # replays; every replay equals the eager result
    links = _links(LAYER, 4, True, seed=15, outs=False)
    chain = bn.LinearChain(links)
    chain.run()
    torch.cuda.synchronize()
    ref = [d["y"].clone() for d in links]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain.run()
    for _ in range(3):
        for d in links:
            d["y"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for d, y in zip(links, ref):
            assert torch.equal(_bits(d["y"]), _bits(y))
    assert _counter_words(chain) == (0, 0)


def test_chain_with_one_poll_per_wait_still_ends():
    # every wait may give up after a single poll (forced from the host): the
    # kernel must still end normally, with the counter back at zero; a wait
    # that ran out is reported in word 1, and a later call on a fresh
    # workspace is exact again
    links = _links(LAYER * 4, 1, False, seed=16, outs=False)
    chain = bn.LinearChain(links, max_polls=1)
    chain.run()
    torch.cuda.synchronize()
    arrivals, flag = _counter_words(chain)
    assert arrivals == 0 and flag in (0, 1)
    ok = bn.LinearChain(links)
    ok.run()
    ref = _single_calls(links, False)
    torch.cuda.synchronize()
    _check_same(links, ref)
    assert _counter_words(ok) == (0, 0)


def test_chain_built_on_one_stream_runs_on_another():
    # the constructor's table copy and workspace fill are complete before it
    # returns, so a first run() on an unrelated stream, with no ordering
    # between the two streams, sees them
    links = _links(LAYER, 1, True, seed=17)
    ref = _single_calls(links, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    chain = bn.LinearChain(links)
    with torch.cuda.stream(s):
        chain.run()
    s.synchronize()
    _check_same(links, ref)
    assert _counter_words(chain) == (0, 0)
