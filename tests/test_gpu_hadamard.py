"""GPU parity of the R4 rotation path (down_proj input: block Sylvester-
Hadamard rotation, then per-token int8 quantisation, then the nested linear)
against the CPU oracle, through the C ABI.

Bars: the rotated fp32 values, the int8 codes and the fp32 scales bit-exact
(both sides run the same fp32 transform in the same stage order, so the
values and the codes they decide agree to the bit); fp32 outputs of the
linear within max|y - y_oracle| <= 1e-5 * max|y_oracle|; the fused calls
bit-identical to the rotation call followed by the plain linear.
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


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("M,K,block", [
    (1, 14336, 512), (4, 14336, 512), (3, 4096, 512), (2, 512, 512), (1, 16384, 512),
    (5, 128, 2), (2, 256, 4), (7, 1024, 8), (32, 2048, 64), (2, 640, 128), (9, 4096, 256),
    (1, 128, 128), (8, 14336, 256),
])
def test_rotation_and_codes_bit_exact(M, K, block):
    x = synth.make_activations(M, K, seed=21, layer=block, linear=M)
    if M > 2:
        x[1] = 0.0                                   # a zero token: s = 0, codes 0
    xq, xs, xr = bn.bitnest_hadamard_quant_act(x.cuda(), block, rotated=True)
    torch.cuda.synchronize()
    q_ref, s_ref, r_ref = oracle.hadamard_quant_act(x.numpy(), block)
    assert np.array_equal(_bits(xr.cpu().numpy()), _bits(r_ref))
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(_bits(xs.cpu().numpy()), _bits(s_ref))



@pytest.mark.parametrize("block", [512, 64])
def test_rotation_of_extreme_magnitudes_bit_exact(block):
    # tokens whose maxima span the fp32 range (1e34 down to subnormal values
    # whose scale underflows to 0), a single nonzero value and a zero token:
    # the rotated values, codes and scales bit for bit on the rotation
    # kernel and on the rotating one-token fused launch
    K = 14336
    rng = np.random.default_rng(block)
    base = rng.standard_normal((8, K))
    x = np.zeros((8, K), np.float32)
    for i, f in enumerate([1.0, 1e34, 1e30, 1e-30, 1e-37, 1e-44]):
        x[i] = (base[i] * f).astype(np.float32)
    x[6, 5] = 3.0
    q_ref, s_ref, r_ref = oracle.hadamard_quant_act(x, block)
    xq, xs, xr = bn.bitnest_hadamard_quant_act(torch.from_numpy(x).cuda(), block, rotated=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(xr.cpu().numpy()), _bits(r_ref))
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(_bits(xs.cpu().numpy()), _bits(s_ref))
    w = synth.make_weights(64, K, seed=24)
    for m in range(8):
        xd = torch.from_numpy(x[m:m + 1].copy()).cuda()
        _, fq, fs = bn.bitnest_hadamard_quant_linear_draft(xd, block, w.hi.cuda(), w.scale.cuda())
        torch.cuda.synchronize()
        assert np.array_equal(fq.cpu().numpy(), q_ref[m:m + 1]), m
        assert np.array_equal(_bits(fs.cpu().numpy()), _bits(s_ref[m:m + 1])), m

def test_rotation_without_rotated_output_gives_same_codes():
    x = synth.make_activations(4, 14336, seed=22)
    xq1, xs1 = bn.bitnest_hadamard_quant_act(x.cuda(), 512)
    xq2, xs2, _ = bn.bitnest_hadamard_quant_act(x.cuda(), 512, rotated=True)
    torch.cuda.synchronize()
    assert torch.equal(xq1, xq2) and torch.equal(xs1, xs2)


FUSED = [(64, 14336, 512), (37, 512, 512), (129, 4096, 512), (33, 1024, 8), (17, 16384, 512),
         (65, 2048, 256), (9, 1024, 64)]


@pytest.mark.parametrize("N,K,block", FUSED)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
@pytest.mark.parametrize("target", [False, True])
def test_fused_rotation_linear(M, N, K, block, target):
    w = synth.make_weights(N, K, seed=23, layer=M, linear=block)
    x = synth.make_activations(M, K, seed=23, layer=M, linear=block)
    xd, hi, lo, sc = x.cuda(), w.hi.cuda(), w.lo.cuda(), w.scale.cuda()
    xq, xs = bn.bitnest_hadamard_quant_act(xd, block)
    if target:
        y_ref = bn.bitnest_linear_target(xq, xs, hi, lo, sc)
        y, fq, fs = bn.bitnest_hadamard_quant_linear_target(xd, block, hi, lo, sc)
    else:
        y_ref = bn.bitnest_linear_draft(xq, xs, hi, sc)
        y, fq, fs = bn.bitnest_hadamard_quant_linear_draft(xd, block, hi, sc)
    torch.cuda.synchronize()
    assert torch.equal(fq, xq)
    assert torch.equal(fs.view(torch.int32), xs.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    q, s, _ = oracle.hadamard_quant_act(x.numpy(), block)
    assert np.array_equal(fq.cpu().numpy(), q)
    hi_n, lo_n, sc_n = w.numpy()
    y64 = oracle.linear(q, s, hi_n, sc_n, lo_n if target else None, 0)
    err = np.abs(y.double().cpu().numpy() - y64).max()
    assert err <= TOL * np.abs(y64).max()


@pytest.mark.parametrize("target", [False, True])
def test_full_size_down_proj_with_rotation(target):
    # Llama-3-8B down_proj (4096 x 14336, 28 blocks of 512), one token (the
    # fused launch a pass times, every row checked) and the verify batch
    # (sampled rows); codes bit-exact, fused y bit-identical to the rotation
    # call followed by the plain linear, y within the bar of the oracle
    N, K, block = 4096, 14336, 512
    w = synth.make_weights(N, K, seed=24, layer=0, linear=3)
    hi_n, lo_n, sc_n = w.numpy()
    hi, lo, sc = w.hi.cuda(), w.lo.cuda(), w.scale.cuda()
    for M in (1, 4):
        x = synth.make_activations(M, K, seed=24, layer=0, linear=3, step=M)
        xd = x.cuda()
        xq, xs = bn.bitnest_hadamard_quant_act(xd, block)
        if target:
            y_ref = bn.bitnest_linear_target(xq, xs, hi, lo, sc)
            y, fq, fs = bn.bitnest_hadamard_quant_linear_target(xd, block, hi, lo, sc)
        else:
            y_ref = bn.bitnest_linear_draft(xq, xs, hi, sc)
            y, fq, fs = bn.bitnest_hadamard_quant_linear_draft(xd, block, hi, sc)
        torch.cuda.synchronize()
        assert torch.equal(fq, xq) and torch.equal(fs.view(torch.int32), xs.view(torch.int32))
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
        q, s, _ = oracle.hadamard_quant_act(x.numpy(), block)
        assert np.array_equal(fq.cpu().numpy(), q)
        assert np.array_equal(_bits(fs.cpu().numpy()), _bits(s))
        rows = np.arange(N) if M == 1 else np.sort(np.random.default_rng(0).choice(N, 48, replace=False))
        y64 = oracle.linear(q, s, np.ascontiguousarray(hi_n[rows]), np.ascontiguousarray(sc_n[rows]),
                            np.ascontiguousarray(lo_n[rows]) if target else None, 0)
        err = np.abs(y.double().cpu().numpy()[:, rows] - y64).max()
        assert err <= TOL * np.abs(y64).max()


def test_rotation_empty_and_zero():
    x = torch.zeros((0, 512), dtype=torch.float32, device="cuda")
    xq, xs = bn.bitnest_hadamard_quant_act(x, 512)
    assert xq.shape == (0, 512) and xs.shape == (0,)
    z = torch.zeros((3, 1024), dtype=torch.float32, device="cuda")
    xq, xs, xr = bn.bitnest_hadamard_quant_act(z, 512, rotated=True)
    torch.cuda.synchronize()
    assert not xq.any() and not xs.any() and not xr.any()
