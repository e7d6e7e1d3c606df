"""Linears at the largest plane the library accepts, through the C ABI.

A plane may hold at most BITNEST_MAX_PLANE_BYTES = 2^31 - 1 bytes, because
the kernels address a plane with 32-bit byte offsets. At K = 16384 that is
N = 262143 rows (2,147,475,456 bytes per plane); one row more is refused
before any launch. Every path is run at that size: the single-token fused
draft and target, the four-token target GEMV, the batched target and draft
on the matrix cores (one and two token tiles), the partials export of
both kernel families, and the offline packer (whose fp32 input then has more
than 2^32 elements). Greedy verification is run at its largest vocabulary
(BITNEST_ACCEPT_MAX_V = 2^30 logits per row) with planted maxima and ties. The rows checked against the oracle are a spread over
the whole plane plus the last 64 rows, whose offsets come closest to the
limit; y within 1e-5 * max|y| of the fp64 oracle (BitNest-Llama-3-8B model
card, "Files", planes.safetensors: W4 and W8 dequantisation), codes, scales,
partials and packed planes exact.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

K = 16384
MAX_PLANE = 2**31 - 1
N = MAX_PLANE // (K // 2)
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


@pytest.fixture(scope="module")
def big():
    assert N * (K // 2) <= MAX_PLANE < (N + 1) * (K // 2)
    w = synth.make_weights(N, K, seed=41, device="cuda")
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 192).astype(int), np.arange(N - 64, N)]))
    ridx = torch.from_numpy(rows).cuda()
    host = (w.hi[ridx].cpu().numpy(), w.lo[ridx].cpu().numpy(), w.scale[ridx].cpu().numpy().view(np.uint16))
    yield w, rows, ridx, host
    del w
    torch.cuda.empty_cache()


def _check_y(y_rows, y64, what):
    y = y_rows.double().cpu().numpy()
    ref = np.abs(y64).max()
    err = np.abs(y - y64).max()
    assert err <= TOL * ref, "%s: max err %.3e vs bound %.3e" % (what, err, TOL * ref)


def test_one_row_more_is_refused(big):
    w, _, _, _ = big
    lib = bn.lib()
    p = ctypes.c_void_p(w.hi.data_ptr())
    st = lib.bitnest_linear_draft(p, p, 0, p, p, p, 1, N + 1, K, None)
    assert st == 3      # BITNEST_EUNSUPPORTED, before any launch


@pytest.mark.parametrize("M,target,fused", [(1, False, True), (1, True, True), (4, True, False),
                                            (8, True, False), (32, False, False)])
def test_largest_plane_matches_oracle(big, M, target, fused):
    w, rows, ridx, (hi, lo, sc) = big
    x = synth.make_activations(M, K, seed=41, linear=M, step=int(target))
    xd = x.cuda()
    if fused:
        assert bn.fused_in_one_launch(M, N, K)
        f = bn.bitnest_quant_linear_target if target else bn.bitnest_quant_linear_draft
        args = (xd, w.hi, w.lo, w.scale) if target else (xd, w.hi, w.scale)
        y, xq, xs = f(*args)
    else:
        xq, xs = bn.bitnest_quant_act(xd, 0)
        if target:
            y = bn.bitnest_linear_target(xq, xs, w.hi, w.lo, w.scale)
        else:
            y = bn.bitnest_linear_draft(xq, xs, w.hi, w.scale)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act(x.numpy(), 0)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    y64 = oracle.linear(q_ref, s_ref, hi, sc, lo if target else None, 0)
    _check_y(y[:, ridx], y64, "M=%d target=%s" % (M, target))
    assert torch.isfinite(y).all()


@pytest.mark.parametrize("M", [1, 8])
def test_largest_plane_partials_exact(big, M):
    w, rows, ridx, (hi, lo, sc) = big
    x = synth.make_activations(M, K, seed=42, linear=M)
    xq, xs = bn.bitnest_quant_act(x.cuda(), 0)
    p = bn.bitnest_linear_partials(xq, w.hi, w.lo)
    torch.cuda.synchronize()
    r = oracle.partials(xq.cpu().numpy(), hi, lo)
    for got, want in zip(p, r):
        assert np.array_equal(got[:, ridx].cpu().numpy(), want)
    del p
    torch.cuda.empty_cache()


def test_largest_plane_pack_bit_exact():
    # the offline packer over fp32 weights [N, K] with N * K / 2 just under
    # 2^31 (about 4.3e9 weights, 17 GB of input: element offsets beyond 32
    # bits); sampled rows bit for bit against the oracle's packing
    g = torch.Generator(device="cuda")
    g.manual_seed(43)
    W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)
    W[N - 1, :128] = 0.0                        # an all-zero group in the last row
    hi, lo, sc = bn.bitnest_pack_nested(W)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 64).astype(int), np.arange(N - 16, N)]))
    ridx = torch.from_numpy(rows).cuda()
    want = oracle.pack_nested(W[ridx].cpu().numpy())
    del W
    torch.cuda.empty_cache()
    assert np.array_equal(hi[ridx].cpu().numpy(), want[0])
    assert np.array_equal(lo[ridx].cpu().numpy(), want[1])
    assert np.array_equal(sc[ridx].cpu().numpy().view(np.uint16), want[2])


@pytest.mark.parametrize("noalloc", [False, True])
def test_greedy_accept_at_the_largest_vocabulary(noalloc):
    # V = BITNEST_ACCEPT_MAX_V = 2^30 logits per row (4 GiB): the slices of
    # the last workgroups end at the row's last column. The answer is fixed by
    # construction: row 0 peaks at V - 5 and V - 3 (tie: the smaller index),
    # row 1 at 7 and at V - 1 (tie: 7)
    V = 1 << 30
    logits = torch.full((2, V), -1.0, dtype=torch.float32, device="cuda")
    logits[0, V - 5] = logits[0, V - 3] = 5.0
    logits[1, 7] = logits[1, V - 1] = 3.0
    f = bn.bitnest_greedy_accept_noalloc if noalloc else bn.bitnest_greedy_accept
    for draft, want in (([V - 5], [1, 7]), ([V - 3], [0, V - 5])):
        targ, result = f(logits, torch.tensor(draft, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert targ.cpu().tolist() == [V - 5, 7]
        assert result.cpu().tolist() == want
    del logits
    torch.cuda.empty_cache()
