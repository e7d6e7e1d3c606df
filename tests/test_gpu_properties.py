"""GPU parity over drawn problems: derandomized Hypothesis draws of the
token count (1 to 32: the GEMV and the matrix-core kernel), ragged N, K (one
to forty 128-column groups), per-token or per-group activation scales, draft
or target, and activation magnitudes over many orders, through the C ABI;
then drawn problems for the packer, greedy verification, the KV attention
and the R4 rotation, each against the oracle to its own bar, and drawn
chains of linears against the single calls.

Bars (BitNest-Llama-3-8B model card, "Files", planes.safetensors: the W4 and
W8 dequantisation; recipe table row "Activations"): codes and scales bit for
bit against the oracle; each y within 1e-5 of the sum of the magnitudes of
its group terms |P * scale * f * s_a| (fp32 sums of at most 128 terms stay
within 130 * 2^-24 of that); the fused quantise + linear call bit for bit
equal to the two calls.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


@st.composite
def problems(draw):
    M = draw(st.sampled_from([1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 32]))
    N = draw(st.integers(1, 700))
    K = 128 * draw(st.integers(1, 40))
    g = draw(st.sampled_from([0, 128]))
    target = draw(st.booleans())
    mag = draw(st.sampled_from([1.0, 1e-20, 1e20, 1e-38]))
    seed = draw(st.integers(0, 2**16))
    return M, N, K, g, target, mag, seed


@settings(max_examples=250, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(p=problems())
def test_drawn_problems_match_the_oracle(p):
    M, N, K, g, target, mag, seed = p
    w = synth.make_weights(N, K, seed=seed, layer=M, linear=g)
    x = (synth.make_activations(M, K, seed=seed, layer=M, linear=g).double() * mag).float()
    xd = x.cuda()
    hi, lo, sc = w.hi.cuda(), w.lo.cuda(), w.scale.cuda()
    planes = (hi, lo, sc) if target else (hi, sc)
    xq, xs = bn.bitnest_quant_act(xd, g)
    y = (bn.bitnest_linear_target if target else bn.bitnest_linear_draft)(xq, xs, *planes, g)
    yf, fq, fs = (bn.bitnest_quant_linear_target if target else bn.bitnest_quant_linear_draft)(xd, *planes, g)
    torch.cuda.synchronize()
    q, s = oracle.quant_act(x.numpy(), g)
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert torch.equal(fq, xq) and torch.equal(fs.view(torch.int32), xs.view(torch.int32))
    assert torch.equal(yf.view(torch.int32), y.view(torch.int32))
    hn, ln, scn = w.numpy()
    y64 = oracle.linear(q, s, hn, scn, ln if target else None, g)
    P = oracle.partials(q, hn, ln)[2] if target else oracle.partials(q, hn)
    sa = s[:, None, None] if g == 0 else s[:, None, :]
    terms = np.abs(P.astype(np.float64) * scn.view(np.float16).astype(np.float64)[None]
                   * (1 / 16 if target else 1.0) * sa)
    bound = 1e-5 * terms.sum(axis=2) + 1e-38
    err = np.abs(y.double().cpu().numpy() - y64)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert (err <= bound).all(), (p, worst, err[worst], bound[worst])


# --------------------------------------------------------------------------- the rows ranked next

@st.composite
def pack_problems(draw):
    N = draw(st.integers(1, 300))
    K = 128 * draw(st.integers(1, 24))
    mag = draw(st.sampled_from([1.0, 1e-3, 1e4, 1e-7, 3e-8]))     # the last: subnormal fp16 scales
    seed = draw(st.integers(0, 2**16))
    return N, K, mag, seed


@settings(max_examples=120, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(p=pack_problems())
def test_drawn_packs_match_the_oracle(p):
    # the offline packer (model card introduction: the hi nibble the W4 fit,
    # the lo nibble the closed-form residual): planes and scale bits exact
    N, K, mag, seed = p
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * mag * rng.uniform(0.1, 3.0, size=(N, 1))).astype(np.float32)
    W[rng.random((N, K)) < 0.01] = 0.0
    hi, lo, sc = bn.bitnest_pack_nested(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    h_ref, l_ref, s_ref = oracle.pack_nested(W)
    assert np.array_equal(hi.cpu().numpy(), h_ref)
    assert np.array_equal(lo.cpu().numpy(), l_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), s_ref)


@st.composite
def accept_problems(draw):
    R = draw(st.integers(1, 32))
    V = draw(st.one_of(st.integers(1, 5000), st.integers(5000, 300000)))
    ties = draw(st.sampled_from(["none", "top", "flat", "negative"]))
    seed = draw(st.integers(0, 2**16))
    return R, V, ties, seed


@settings(max_examples=120, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(p=accept_problems())
def test_drawn_greedy_rounds_match_the_oracle(p):
    # greedy verification (model card introduction: every draft token is
    # checked against the target): argmax with ties to the smallest index,
    # accepted count and next token exact
    from test_gpu_accept import _case
    R, V, ties, seed = p
    logits, draft = _case(R, V, seed=seed, ties=ties)
    targ, res = bn.bitnest_greedy_accept(torch.from_numpy(logits).cuda(), torch.from_numpy(draft).cuda())
    torch.cuda.synchronize()
    t_ref, n_ref, next_ref = oracle.greedy_accept(logits, draft)
    assert np.array_equal(targ.cpu().numpy(), t_ref)
    assert res.cpu().numpy().tolist() == [n_ref, next_ref]


@st.composite
def kv_problems(draw):
    Hkv = draw(st.sampled_from([1, 2, 4, 8]))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    M = draw(st.integers(1, max(1, min(4, 16 // G))))
    T = draw(st.integers(M, 3000))
    t_cap = T + draw(st.integers(0, 200))
    kv8 = draw(st.booleans())
    seed = draw(st.integers(0, 2**16))
    return M, G * Hkv, Hkv, T, t_cap, kv8, seed


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(p=kv_problems())
def test_drawn_kv_attention_matches_the_oracle(p):
    # nested KV decode attention (model card recipe table row "KV cache"):
    # each (token, query head) output within 1e-5 of its own largest
    # magnitude, plus 1e-8 of max|V|
    from test_gpu_kv import _cache, _check, _ref, _run, _vmax
    M, Hq, Hkv, T, t_cap, kv8, seed = p
    assert M * Hq // Hkv <= 16
    kc, vc = _cache(T, Hkv, seed=seed, spread=0.5)
    q = np.random.default_rng(seed).standard_normal((M, Hq, 128)).astype(np.float32)
    got = _run(q, kc, vc, kv8, t_cap=t_cap)
    _check(got, _ref(q, kc, vc, kv8), _vmax(vc, kv8))


@st.composite
def rotation_problems(draw):
    block = 2 ** draw(st.integers(1, 9))                 # 2 .. 512
    K = 128 * draw(st.integers(1, 112))
    if K % block:
        K = block * (K // block + 1)
    M = draw(st.integers(1, 8))
    N = draw(st.integers(1, 200))
    mag = draw(st.sampled_from([1.0, 1e-30, 1e30]))
    target = draw(st.booleans())
    seed = draw(st.integers(0, 2**16))
    return M, N, K, block, mag, target, seed


@settings(max_examples=80, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(p=rotation_problems())
def test_drawn_rotations_match_the_oracle(p):
    # the R4 rotation of the down_proj input (model card recipe table row
    # "Rotation"): rotated values, codes and scales bit for bit; the rotating
    # quantise + linear call bit for bit equal to the rotation call followed
    # by the linear
    M, N, K, block, mag, target, seed = p
    x = (synth.make_activations(M, K, seed=seed, layer=block).double() * mag).float()
    xd = x.cuda()
    xq, xs, xr = bn.bitnest_hadamard_quant_act(xd, block, rotated=True)
    w = synth.make_weights(N, K, seed=seed, layer=block)
    hi, lo, sc = w.hi.cuda(), w.lo.cuda(), w.scale.cuda()
    if target:
        y_ref = bn.bitnest_linear_target(xq, xs, hi, lo, sc)
        y, fq, fs = bn.bitnest_hadamard_quant_linear_target(xd, block, hi, lo, sc)
    else:
        y_ref = bn.bitnest_linear_draft(xq, xs, hi, sc)
        y, fq, fs = bn.bitnest_hadamard_quant_linear_draft(xd, block, hi, sc)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.hadamard_quant_act(x.numpy(), block)
    assert np.array_equal(xr.cpu().numpy().view(np.uint32), r_ref.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert torch.equal(fq, xq) and torch.equal(fs.view(torch.int32), xs.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))


@st.composite
def chain_problems(draw):
    M = draw(st.integers(1, 4))
    target = draw(st.booleans())
    links = []
    for j in range(draw(st.integers(1, 8))):
        prev_n = links[-1][0] if links else 0
        chained = bool(links) and prev_n >= 128 and prev_n % 128 == 0 and draw(st.booleans())
        N = draw(st.one_of(st.just(0), st.integers(1, 3000), st.sampled_from([128, 256, 1024, 4096])))
        K = prev_n if chained else 128 * draw(st.integers(1, 32))
        links.append((N, K, draw(st.sampled_from([0, 128])), chained))
    return M, target, links, draw(st.integers(0, 2**16))


@settings(max_examples=40, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(p=chain_problems())
def test_drawn_chains_equal_single_calls(p):
    # a chain of quantise + linear steps in one launch, some links reading the
    # previous link's output: every y, code and scale bit for bit that of the
    # single calls made one after another
    M, target, spec, seed = p
    links = []
    for i, (N, K, g, chained) in enumerate(spec):
        w = synth.make_weights(N, K, seed=seed, layer=i, with_lo=target, device="cuda")
        x = links[-1]["y"] if chained else synth.make_activations(M, K, seed=seed, layer=i, device="cuda")
        d = dict(x=x, hi=w.hi, scale=w.scale, y=torch.empty((M, N), device="cuda"), act_group=g,
                 xq=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                 xs=torch.empty((M,) if g == 0 else (M, K // 128), device="cuda"))
        if target:
            d["lo"] = w.lo
        links.append(d)
    chain = bn.LinearChain(links)
    chain.run()
    torch.cuda.synchronize()
    got = [(d["y"].clone(), d["xq"].clone(), d["xs"].clone()) for d in links]
    prev = None
    for j, (d, (N, K, g, chained)) in enumerate(zip(links, spec)):
        x = prev if chained else d["x"]
        if target:
            y, q, s = bn.bitnest_quant_linear_target(x, d["hi"], d["lo"], d["scale"], g)
        else:
            y, q, s = bn.bitnest_quant_linear_draft(x, d["hi"], d["scale"], g)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), got[j][0].view(torch.int32)), ("y", j)
        assert torch.equal(q, got[j][1]), ("codes", j)
        assert torch.equal(s.view(torch.int32), got[j][2].view(torch.int32)), ("scales", j)
        prev = y
    assert chain.work[:8].view(torch.int32).cpu().tolist() == [0, 0]
