"""GPU parity of the offline nested packer (fp32 weights -> hi / lo planes
and fp16 scales) against the CPU oracle, through the C ABI: planes and scale
bits identical (the codes are integer decisions taken in fp32 on both
sides), and the packed weights feed the linear like any other planes.
"""
import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _weights(N, K, seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        W = rng.standard_normal((N, K)) * 0.02
    elif kind == "heavy":
        W = rng.standard_t(3, size=(N, K)) * 0.01
    elif kind == "grid":
        # values on and half-way between the W4 / W8 grids of s = 0.25: ties everywhere
        W = rng.integers(-16 * 8, 16 * 7, size=(N, K)) * (0.25 / 16) + rng.integers(0, 2, size=(N, K)) * (0.25 / 32)
        W[:, ::128] = 1.875
    elif kind == "tiny":
        W = rng.standard_normal((N, K)) * 1e-6          # fp16 scales in the subnormal range
    else:
        raise ValueError(kind)
    W = W.astype(np.float32)
    W[0, :128] = 0.0                                     # an all-zero group
    return W


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (37, 640), (64, 4096), (5, 14336), (130, 1024)])
@pytest.mark.parametrize("kind", ["normal", "heavy", "grid", "tiny"])
def test_pack_bit_exact(N, K, kind):
    W = _weights(N, K, seed=N * 7 + K, kind=kind)
    hi, lo, sc = bn.bitnest_pack_nested(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    hi_r, lo_r, sc_r = oracle.pack_nested(W)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), sc_r)
    assert np.array_equal(hi.cpu().numpy(), hi_r)
    assert np.array_equal(lo.cpu().numpy(), lo_r)


def test_pack_full_layer_shape_sampled_rows():
    # the Llama-3-8B gate_up shape; rows sampled for the oracle
    N, K = 28672, 4096
    g = torch.Generator(device="cuda").manual_seed(5)
    W = torch.randn((N, K), generator=g, device="cuda") * 0.02
    hi, lo, sc = bn.bitnest_pack_nested(W)
    torch.cuda.synchronize()
    rows = np.random.default_rng(1).choice(N, 64, replace=False)
    Wn = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    hi_r, lo_r, sc_r = oracle.pack_nested(Wn)
    assert np.array_equal(hi.cpu().numpy()[rows], hi_r)
    assert np.array_equal(lo.cpu().numpy()[rows], lo_r)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16)[rows], sc_r)


def test_packed_weights_through_the_linear():
    # pack fp32 weights on the GPU, run the target linear on them, compare
    # with the fp32 product of the original weights (the nesting error bound)
    N, K = 256, 4096
    W = _weights(N, K, seed=3, kind="normal")
    hi, lo, sc = bn.bitnest_pack_nested(torch.from_numpy(W).cuda())
    x = synth.make_activations(1, K, seed=3, outliers=False)
    xq, xs = bn.bitnest_quant_act(x.cuda())
    y8 = bn.bitnest_linear_target(xq, xs, hi, lo, sc).double().cpu().numpy()
    y4 = bn.bitnest_linear_draft(xq, xs, hi, sc).double().cpu().numpy()
    torch.cuda.synchronize()
    xhat = xq.cpu().numpy().astype(np.float64) * xs.cpu().numpy().astype(np.float64)[:, None]
    yref = xhat @ W.astype(np.float64).T
    s = sc.cpu().numpy().view(np.float16).astype(np.float64)
    # |W8 - W| <= s/32 (and s/16 where the residual clamps), |W4 - W| <= s/2 per element
    bound8 = (np.abs(xhat).reshape(1, K // 128, 128).sum(axis=2) @ (s / 16).T).ravel()
    bound4 = (np.abs(xhat).reshape(1, K // 128, 128).sum(axis=2) @ (s / 2 * 1.0001).T).ravel()
    assert np.all(np.abs(y8 - yref).ravel() <= bound8 + 1e-6)
    assert np.all(np.abs(y4 - yref).ravel() <= bound4 + 1e-6)
    assert np.abs(y8 - yref).mean() < np.abs(y4 - yref).mean() / 8


def test_pack_empty():
    W = torch.zeros((0, 256), dtype=torch.float32, device="cuda")
    hi, lo, sc = bn.bitnest_pack_nested(W)
    assert hi.shape == (0, 128) and sc.shape == (0, 2)
