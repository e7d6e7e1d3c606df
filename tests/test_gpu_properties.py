"""GPU parity over drawn problems: derandomized Hypothesis draws of the
token count (1 to 32: the GEMV and the matrix-core kernel), ragged N, K (one
to forty 128-column groups), per-token or per-group activation scales, draft
or target, and activation magnitudes over many orders, through the C ABI.

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
