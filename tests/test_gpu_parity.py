"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: int8 activation codes, fp32 activation scales and int32 per-group
partials bit-exact; fp32 outputs within max|y - y_oracle| <= 1e-5 * max|y_oracle|
(y_oracle is the oracle's fp64 dequantise-then-multiply result). Invariants of
the format are checked on the GPU bit for bit: lo == 8 makes the target equal
the draft, an M-token call equals single-token calls row by row.
"""
import numpy as np
import pytest
import torch

import oracle
import w8_quantized_linear_amd as bn
from w8_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

GROUP = 128
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bn.lib()


def _dev(t):
    return t.to("cuda")


def _problem(M, N, K, seed=0, outliers=True, lo=True):
    w = synth.make_weights(N, K, seed=seed, layer=M, linear=N % 97, with_lo=lo)
    x = synth.make_activations(M, K, seed=seed, layer=M, linear=N % 97, outliers=outliers)
    return w, x


def _check_y(y_gpu, y64, what=""):
    y = y_gpu.double().cpu().numpy()
    ref = np.abs(y64).max()
    err = np.abs(y - y64).max() if y.size else 0.0
    assert err <= TOL * ref + 1e-30, "%s: max err %.3e vs bound %.3e" % (what, err, TOL * ref)


def _run(w, x, act_group, target, M=None):
    xd = _dev(x)
    xq, xs = bn.bitnest_quant_act(xd, act_group)
    hi, lo, sc = _dev(w.hi), (_dev(w.lo) if target else None), _dev(w.scale)
    if target:
        y = bn.bitnest_linear_target(xq, xs, hi, lo, sc, act_group)
    else:
        y = bn.bitnest_linear_draft(xq, xs, hi, sc, act_group)
    torch.cuda.synchronize()
    return xq, xs, y


# --------------------------------------------------------------------------- activation quant

@pytest.mark.parametrize("M,K,act_group", [
    (1, 512, 0), (1, 4096, 0), (4, 4096, 0), (3, 14336, 0), (32, 4096, 0), (7, 16384, 0),
    (1, 128, 0), (1, 4096, 128), (4, 4096, 128), (13, 640, 128), (32, 14336, 128), (5, 128, 128),
])
def test_quant_act_bit_exact(M, K, act_group):
    x = synth.make_activations(M, K, seed=1, layer=K, linear=M)
    if M > 2:
        x[1] = 0.0                                   # a zero token: s = 0, q = 0
    xq, xs = bn.bitnest_quant_act(_dev(x), act_group)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quant_act_ties_golden_on_gpu(golden_dir):
    import json, os
    fx = json.load(open(os.path.join(golden_dir, "act_quant.json")))
    rows = []
    for case in fx["per_token"]:
        r = np.zeros(GROUP, np.float32)
        r[:len(case["x"])] = case["x"]
        rows.append(r)
    x = torch.from_numpy(np.stack(rows))
    xq, xs = bn.bitnest_quant_act(_dev(x))
    torch.cuda.synchronize()
    for i, case in enumerate(fx["per_token"]):
        assert xs[i].item() == case["s"]
        assert xq[i, :len(case["q"])].cpu().tolist() == case["q"]


# --------------------------------------------------------------------------- partials

SHAPES = [(256, 512), (37, 640), (70, 2176), (33, 14336), (5, 128), (129, 4096), (17, 16384)]
MS = [1, 2, 3, 4, 5, 7, 8, 13, 16, 17, 32]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", MS)
def test_partials_bit_exact(M, N, K):
    w, x = _problem(M, N, K)
    q, _ = oracle.quant_act(x.numpy())
    xq = _dev(torch.from_numpy(q))
    hi, lo, _ = w.numpy()
    g_hi, g_lo, g_8 = bn.bitnest_linear_partials(xq, _dev(w.hi), _dev(w.lo))
    d_hi = bn.bitnest_linear_partials(xq, _dev(w.hi))
    torch.cuda.synchronize()
    r_hi, r_lo, r_8 = oracle.partials(q, hi, lo)
    assert np.array_equal(g_hi.cpu().numpy(), r_hi)
    assert np.array_equal(g_lo.cpu().numpy(), r_lo)
    assert np.array_equal(g_8.cpu().numpy(), r_8)
    assert np.array_equal(d_hi.cpu().numpy(), r_hi)


def test_partials_reach_their_bounds():
    # every code -8 (nibble 0) against codes -127: |P_hi| = 127*8*128 and
    # |P8| = 127*136*128 exactly, on both kernels
    for M in (1, 4, 8, 32):
        xq = torch.full((M, 256), -127, dtype=torch.int8, device="cuda")
        z = torch.zeros((3, 128), dtype=torch.uint8, device="cuda")
        p_hi, p_lo, p8 = bn.bitnest_linear_partials(xq, z, z)
        torch.cuda.synchronize()
        assert int(p_hi.min()) == int(p_hi.max()) == 127 * 8 * 128
        assert int(p8.min()) == int(p8.max()) == 127 * 136 * 128
        assert int(p_lo.max()) == 127 * 8 * 128


# --------------------------------------------------------------------------- fp32 outputs

@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 3, 4, 7, 8, 16, 32])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_linear_matches_oracle(M, N, K, act_group, target):
    w, x = _problem(M, N, K, seed=2)
    xq, xs, y = _run(w, x, act_group, target)
    hi, lo, sc = w.numpy()
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q)
    y64 = oracle.linear(q, s, hi, sc, lo if target else None, act_group)
    _check_y(y, y64, "M=%d N=%d K=%d g=%d t=%s" % (M, N, K, act_group, target))


@pytest.mark.parametrize("N", [16390, 32770])   # 2 and 4 row tiles per workgroup on 256 CUs, ragged last tile
@pytest.mark.parametrize("M", [8, 17, 32])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_batched_verify_several_row_tiles(M, N, act_group, target):
    # the batched-verify kernel gives a workgroup several 16-row tiles when N
    # is large (activation loads shared by the tiles); every row is checked
    w, x = _problem(M, N, 256, seed=3)
    xq, xs, y = _run(w, x, act_group, target)
    hi, lo, sc = w.numpy()
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q)
    y64 = oracle.linear(q, s, hi, sc, lo if target else None, act_group)
    _check_y(y, y64, "M=%d N=%d g=%d t=%s" % (M, N, act_group, target))


# rows per workgroup on 256 CUs: 8 (tiles half empty), 24 with a ragged last
# workgroup, 24 (the qkv shape), 40 (three tiles, the last with 8 rows), 64,
# 80, 112 (the gate_up shape, seven tiles) and 120 (eight tiles, the most a
# workgroup holds, with one or two token tiles)
@pytest.mark.parametrize("N", [1000, 5001, 6144, 10000, 16000, 20000, 28672, 30000])
@pytest.mark.parametrize("M", [8, 32])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_batched_verify_rows_per_workgroup(M, N, act_group, target):
    # where N spread over one workgroup per CU fits the tile limit, a
    # workgroup owns ceil(N / CUs) rows rounded up to 8, and the rows past it
    # in its last tile read as zero; every row is checked
    w, x = _problem(M, N, 256, seed=4)
    xq, xs, y = _run(w, x, act_group, target)
    hi, lo, sc = w.numpy()
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q)
    y64 = oracle.linear(q, s, hi, sc, lo if target else None, act_group)
    _check_y(y, y64, "M=%d N=%d g=%d t=%s" % (M, N, act_group, target))


# one 16-row tile per workgroup (at most 16 rows per CU on 256 CUs): the
# row-contiguous order, 1 KiB chunks of each row staged through LDS. N = 4090
# leaves 10 rows in the last workgroup, N = 2000 gives 8-row workgroups; K =
# 6016 ends in a partial chunk (15 of 16 groups), K = 14336 has an odd number
# of chunks
@pytest.mark.parametrize("N,K", [(4090, 6016), (2000, 14336), (4096, 1152)])
@pytest.mark.parametrize("M", [8, 17])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_batched_verify_row_contiguous(M, N, K, act_group, target):
    w, x = _problem(M, N, K, seed=6)
    xq, xs, y = _run(w, x, act_group, target)
    hi, lo, sc = w.numpy()
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q)
    y64 = oracle.linear(q, s, hi, sc, lo if target else None, act_group)
    _check_y(y, y64, "M=%d N=%d K=%d g=%d t=%s" % (M, N, K, act_group, target))


@pytest.mark.parametrize("M", [1, 4, 8, 32])
@pytest.mark.parametrize("act_group", [0, 128])
def test_target_equals_draft_when_lo_is_8(M, act_group):
    N, K = 96, 2176
    w, x = _problem(M, N, K, seed=3)
    xd = _dev(x)
    xq, xs = bn.bitnest_quant_act(xd, act_group)
    hi, sc = _dev(w.hi), _dev(w.scale)
    lo8 = torch.full_like(hi, 0x88)
    yd = bn.bitnest_linear_draft(xq, xs, hi, sc, act_group)
    yt = bn.bitnest_linear_target(xq, xs, hi, lo8, sc, act_group)
    torch.cuda.synchronize()
    assert torch.equal(yd.view(torch.int32), yt.view(torch.int32))


@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_verify_batch_rows_equal_single_token_calls(act_group, target):
    # GEMV: one M = 4 call == four M = 1 calls, bit for bit (y and partials).
    N, K = 200, 4096
    w, x = _problem(4, N, K, seed=4)
    _, _, y4 = _run(w, x, act_group, target)
    for m in range(4):
        _, _, y1 = _run(w, x[m:m + 1], act_group, target)
        assert torch.equal(y1[0].view(torch.int32), y4[m].view(torch.int32)), m
    xq, _ = bn.bitnest_quant_act(_dev(x))
    p4 = bn.bitnest_linear_partials(xq, _dev(w.hi), _dev(w.lo))
    for m in range(4):
        p1 = bn.bitnest_linear_partials(xq[m:m + 1].contiguous(), _dev(w.hi), _dev(w.lo))
        for a, b in zip(p1, p4):
            assert torch.equal(a[0], b[m])



def _special_scales(N, G, seed):
    # fp16 bit patterns, 16 rows per class: negative normals; subnormals of
    # both signs; zeros of both signs between normals; the extremes (largest
    # finite 65504, smallest normal 2^-14) of both signs
    rng = np.random.default_rng(seed)
    sc = np.empty((N, G), np.uint16)
    normal = lambda n: (np.exp(np.log(0.01) + 0.3 * rng.standard_normal(n))).astype(np.float16).view(np.uint16)
    for r in range(N):
        kind = (r // 16) % 4
        if kind == 0:
            sc[r] = normal(G) | 0x8000
        elif kind == 1:
            sc[r] = rng.integers(1, 0x400, G).astype(np.uint16) | (rng.integers(0, 2, G) << 15).astype(np.uint16)
        elif kind == 2:
            sc[r] = np.where(rng.integers(0, 2, G) == 1, normal(G), np.where(rng.integers(0, 2, G) == 1, 0x8000, 0))
        else:
            sc[r] = rng.choice(np.array([0x7BFF, 0xFBFF, 0x0400, 0x8400], np.uint16), G)
    return sc


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_special_weight_scales(M, act_group, target):
    # Any finite fp16 scale: each output within 1e-5 of the sum of the
    # magnitudes of its group terms |P * scale * f * s_a| (the fp32 sum of at
    # most 128 terms stays within 130 * 2^-24 of that; rows whose terms
    # cancel are not held to a bound relative to their own small value)
    N, K = 64, 4096
    G = K // 128
    w, x = _problem(M, N, K, seed=31)
    sc = _special_scales(N, G, seed=31)
    xd = _dev(x)
    xq, xs = bn.bitnest_quant_act(xd, act_group)
    hi, lo, scd = _dev(w.hi), _dev(w.lo), torch.from_numpy(sc.view(np.int16)).cuda()
    if target:
        y = bn.bitnest_linear_target(xq, xs, hi, lo, scd, act_group)
    else:
        y = bn.bitnest_linear_draft(xq, xs, hi, scd, act_group)
    torch.cuda.synchronize()
    q, s = oracle.quant_act(x.numpy(), act_group)
    hn, ln, _ = w.numpy()
    y64 = oracle.linear(q, s, hn, sc, ln if target else None, act_group)
    P = oracle.partials(q, hn, ln)[2] if target else oracle.partials(q, hn)
    f = 1.0 / 16 if target else 1.0
    sa = s[:, None, None] if act_group == 0 else s[:, None, :]
    terms = np.abs(P.astype(np.float64) * sc.view(np.float16).astype(np.float64)[None] * f * sa)
    bound = 1e-5 * terms.sum(axis=2) + 1e-38
    got = y.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - y64)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert (err <= bound).all(), ("token, row", worst, err[worst], bound[worst])

@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_batched_verify_rows_do_not_depend_on_batch(target, act_group):
    # The matrix-core kernel: rows of an M = 32 call equal those of M = 8, 9,
    # 16, 17 and 23 calls on the same tokens (one and two token tiles, full
    # and ragged), bit for bit.
    N, K = 160, 4096
    w, x = _problem(32, N, K, seed=5)
    _, _, y32 = _run(w, x, act_group, target)
    for a, b in ((0, 8), (8, 24), (3, 12), (15, 32), (0, 17), (9, 32)):
        _, _, y = _run(w, x[a:b], act_group, target)
        assert torch.equal(y.view(torch.int32), y32[a:b].view(torch.int32)), (a, b)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_repeated_calls_are_bit_identical(M):
    N, K = 1000, 4096
    w, x = _problem(M, N, K, seed=6)
    xq, xs = bn.bitnest_quant_act(_dev(x))
    hi, lo, sc = _dev(w.hi), _dev(w.lo), _dev(w.scale)
    ref = bn.bitnest_linear_target(xq, xs, hi, lo, sc)
    for _ in range(10):
        y = bn.bitnest_linear_target(xq, xs, hi, lo, sc)
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32))


def test_zero_activations_give_zero_outputs():
    for M in (1, 8):
        x = torch.zeros((M, 512), device="cuda")
        xq, xs = bn.bitnest_quant_act(x)
        w = synth.make_weights(64, 512)
        y = bn.bitnest_linear_target(xq, xs, _dev(w.hi), _dev(w.lo), _dev(w.scale))
        torch.cuda.synchronize()
        assert float(xs.abs().max()) == 0.0 and int(xq.abs().max()) == 0
        assert float(y.abs().max()) == 0.0


def test_empty_calls_are_noops():
    xq = torch.zeros((0, 256), dtype=torch.int8, device="cuda")
    xs = torch.zeros((0,), dtype=torch.float32, device="cuda")
    w = synth.make_weights(8, 256)
    y = bn.bitnest_linear_draft(xq, xs, _dev(w.hi), _dev(w.scale))
    assert y.shape == (0, 8)
    xq1 = torch.zeros((2, 256), dtype=torch.int8, device="cuda")
    xs1 = torch.ones((2,), dtype=torch.float32, device="cuda")
    hi0 = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    sc0 = torch.zeros((0, 2), dtype=torch.int16, device="cuda")
    y0 = bn.bitnest_linear_target(xq1, xs1, hi0, hi0, sc0)
    assert y0.shape == (2, 0)


def test_misaligned_pointer_is_rejected_on_gpu():
    buf = torch.zeros(4096 + 16, dtype=torch.uint8, device="cuda")
    hi = buf[4:4 + 8 * 64].view(8, 64)              # offset 4 bytes: misaligned
    xq = torch.zeros((1, 128), dtype=torch.int8, device="cuda")
    xs = torch.ones((1,), dtype=torch.float32, device="cuda")
    sc = torch.zeros((8, 1), dtype=torch.int16, device="cuda")
    with pytest.raises(bn.BitnestError) as e:
        bn.bitnest_linear_draft(xq, xs, hi, sc)
    assert e.value.status == bn.EALIGN


def test_runs_on_a_side_stream():
    N, K, M = 300, 4096, 4
    w, x = _problem(M, N, K, seed=7)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xd = _dev(x)
        xq, xs = bn.bitnest_quant_act(xd)
        y = bn.bitnest_linear_target(xq, xs, _dev(w.hi), _dev(w.lo), _dev(w.scale))
    s.synchronize()
    hi, lo, sc = w.numpy()
    q, sa = oracle.quant_act(x.numpy())
    assert np.array_equal(xq.cpu().numpy(), q)
    _check_y(y, oracle.linear(q, sa, hi, sc, lo), "side stream")



def test_calls_on_two_streams_run_concurrently():
    # Calls keep no state between them (outside the no-allocation scratch
    # and caller workspaces), so work enqueued on two streams with no order
    # between them gives what the same calls give one after another: the
    # fused one-token path, the two-launch four-token path and the matrix
    # cores, alternately enqueued on both streams
    cases = [(1, 1536, 4096, 0, False), (4, 9216, 4096, 0, True), (1, 1024, 14336, 0, True),
             (8, 512, 4096, 128, True), (4, 1024, 4096, 128, False), (1, 2048, 4096, 128, True)]
    probs = []
    for i, (M, N, K, g, target) in enumerate(cases):
        w = synth.make_weights(N, K, seed=40 + i, device="cuda")
        x = synth.make_activations(M, K, seed=40 + i, device="cuda")
        probs.append((x, w, g, target))

    def call(x, w, g, target):
        if target:
            return bn.bitnest_quant_linear_target(x, w.hi, w.lo, w.scale, g)
        return bn.bitnest_quant_linear_draft(x, w.hi, w.scale, g)

    serial = [call(*p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    out = []
    for rep in range(3):
        for i, p in enumerate(probs):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                out.append((i, call(*p)))
    torch.cuda.synchronize()
    for i, (y, q, s) in out:
        y0, q0, s0 = serial[i]
        assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32)), i
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32)), i

# --------------------------------------------------------------------------- full-size layers

@pytest.fixture(scope="module")
def llama_layer():
    """One Llama-3-8B decoder layer's four linears (seed 0, layer 0), both planes."""
    out = []
    for li, (name, N, K, g) in enumerate(synth.LLAMA3_8B_LINEARS):
        w = synth.make_weights(N, K, seed=0, layer=0, linear=li)
        out.append((name, N, K, g, w, w.to("cuda")))
    return out


def _rows_sample(N, n=384):
    idx = np.unique(np.concatenate([np.linspace(0, N - 1, n).astype(int), np.arange(N - 16, N)]))
    return idx


@pytest.mark.parametrize("N", [6144, 10000])     # 24 and 40 rows per workgroup on 256 CUs
@pytest.mark.parametrize("K", [4096, 6016, 14336])     # 2, 3 (the last partial) and 7 chunks of 16 groups
@pytest.mark.parametrize("M", [8, 32])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_batched_verify_several_tiles_full_k(M, K, N, act_group, target):
    # several row tiles per workgroup at full width: the batched-verify
    # kernel takes each chunk of K for all its tiles in turn, the chunk's
    # activations loaded once (an odd chunk count ends in an empty chunk);
    # sampled rows against the oracle
    w, x = _problem(M, N, K, seed=5)
    xq, xs, y = _run(w, x, act_group, target)
    hi, lo, sc = w.numpy()
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(xq.cpu().numpy(), q)
    rows = _rows_sample(N)
    y64 = oracle.linear(q, s, np.ascontiguousarray(hi[rows]), np.ascontiguousarray(sc[rows]),
                        np.ascontiguousarray(lo[rows]) if target else None, act_group)
    _check_y(y[:, torch.from_numpy(rows).cuda()], y64, "M=%d N=%d g=%d t=%s" % (M, N, act_group, target))


@pytest.mark.parametrize("M,target", [(1, False), (1, True), (4, True), (8, False), (8, True), (16, True), (32, True)])
def test_llama_layer_full_size(llama_layer, M, target):
    for li, (name, N, K, g, w, wd) in enumerate(llama_layer):
        x = synth.make_activations(M, K, seed=0, layer=0, linear=li)
        xq, xs = bn.bitnest_quant_act(_dev(x), g)
        if target:
            y = bn.bitnest_linear_target(xq, xs, wd.hi, wd.lo, wd.scale, g)
        else:
            y = bn.bitnest_linear_draft(xq, xs, wd.hi, wd.scale, g)
        torch.cuda.synchronize()
        q_ref, s_ref = oracle.quant_act(x.numpy(), g)
        assert np.array_equal(xq.cpu().numpy(), q_ref), name
        assert np.array_equal(xs.cpu().numpy(), s_ref), name
        hi, lo, sc = w.numpy()
        rows = _rows_sample(N) if M > 1 else np.arange(N)
        y64 = oracle.linear(q_ref, s_ref, np.ascontiguousarray(hi[rows]), np.ascontiguousarray(sc[rows]),
                            np.ascontiguousarray(lo[rows]) if target else None, g)
        _check_y(y[:, torch.from_numpy(rows).cuda()], y64, "%s M=%d target=%s" % (name, M, target))
        if M in (1, 4, 8):
            p = bn.bitnest_linear_partials(xq, wd.hi[:64].contiguous(), wd.lo[:64].contiguous())
            r = oracle.partials(q_ref, hi[:64], lo[:64])
            for a, b in zip(p, r):
                assert np.array_equal(a.cpu().numpy(), b), name


# --------------------------------------------------------------------------- fused quant + linear

FUSED_SHAPES = [(256, 512), (37, 640), (70, 2176), (33, 14336), (129, 4096), (17, 16384), (9, 128), (300, 256),
                (8192, 384)]


@pytest.mark.parametrize("N,K", FUSED_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 32])
@pytest.mark.parametrize("act_group", [0, 128])
@pytest.mark.parametrize("target", [False, True])
def test_fused_quant_linear_equals_two_calls(M, N, K, act_group, target):
    # One fused call must give the codes, scales and y of quant_act followed by
    # the linear, bit for bit (one launch for one token up to K = 16384 and
    # for up to four tokens up to K = 4096 and N = 8192, else two).
    one = (M == 1 and K <= 16384) or (M <= 4 and K <= 4096 and N <= 8192)
    assert bn.fused_in_one_launch(M, N, K) == one
    w, x = _problem(M, N, K, seed=9)
    xd, hi, lo, sc = _dev(x), _dev(w.hi), _dev(w.lo), _dev(w.scale)
    xq, xs = bn.bitnest_quant_act(xd, act_group)
    if target:
        y_ref = bn.bitnest_linear_target(xq, xs, hi, lo, sc, act_group)
        y, fq, fs = bn.bitnest_quant_linear_target(xd, hi, lo, sc, act_group)
    else:
        y_ref = bn.bitnest_linear_draft(xq, xs, hi, sc, act_group)
        y, fq, fs = bn.bitnest_quant_linear_draft(xd, hi, sc, act_group)
    torch.cuda.synchronize()
    assert torch.equal(fq, xq)
    assert torch.equal(fs.view(torch.int32), xs.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    q, s = oracle.quant_act(x.numpy(), act_group)
    assert np.array_equal(fq.cpu().numpy(), q)
    hi_n, lo_n, sc_n = w.numpy()
    _check_y(y, oracle.linear(q, s, hi_n, sc_n, lo_n if target else None, act_group), "fused")


@pytest.mark.parametrize("M,target", [(1, False), (1, True), (4, True), (4, False), (2, True)])
def test_fused_single_token_full_layer(llama_layer, M, target):
    # The launches a round times: quantisation and the linear in one launch
    # (one token: a draft pass, all four shapes; four tokens: the verify pass's
    # qkv and o_proj, while gate_up (N above 8192) and down (K = 14336) take
    # two launches) at the Llama-3-8B shapes, o_proj with per-group activation
    # scales. Codes,
    # scales and y are bit-identical to the two-call path; every row of y is
    # within the bar of the oracle.
    for li, (name, N, K, g, w, wd) in enumerate(llama_layer):
        x = synth.make_activations(M, K, seed=0, layer=1, linear=li)
        xd = _dev(x)
        xq, xs = bn.bitnest_quant_act(xd, g)
        if target:
            y_ref = bn.bitnest_linear_target(xq, xs, wd.hi, wd.lo, wd.scale, g)
            y, fq, fs = bn.bitnest_quant_linear_target(xd, wd.hi, wd.lo, wd.scale, g)
        else:
            y_ref = bn.bitnest_linear_draft(xq, xs, wd.hi, wd.scale, g)
            y, fq, fs = bn.bitnest_quant_linear_draft(xd, wd.hi, wd.scale, g)
        torch.cuda.synchronize()
        assert torch.equal(fq, xq), name
        assert torch.equal(fs.view(torch.int32), xs.view(torch.int32)), name
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), name
        q, s = oracle.quant_act(x.numpy(), g)
        assert np.array_equal(fq.cpu().numpy(), q), name
        assert np.array_equal(fs.cpu().numpy(), s), name
        hi, lo, sc = w.numpy()
        _check_y(y, oracle.linear(q, s, hi, sc, lo if target else None, g), "%s fused t=%s" % (name, target))



@pytest.mark.parametrize("target", [True, False])
def test_verify_rows_equal_one_token_calls_full_layer(llama_layer, target):
    # The verify pass's call (four tokens, quantised in the call: one launch
    # for qkv and o_proj, two for gate_up and down) at the Llama-3-8B shapes:
    # each token's codes, scale and y are bit for bit those of a one-token call
    # on that token, so the verify rows are exactly what one-token target
    # steps compute.
    for li, (name, N, K, g, w, wd) in enumerate(llama_layer):
        xd = _dev(synth.make_activations(4, K, seed=3, layer=2, linear=li))
        f = bn.bitnest_quant_linear_target if target else bn.bitnest_quant_linear_draft
        planes = (wd.hi, wd.lo, wd.scale) if target else (wd.hi, wd.scale)
        y4, q4, s4 = f(xd, *planes, g)
        for m in range(4):
            y1, q1, s1 = f(xd[m:m + 1].contiguous(), *planes, g)
            torch.cuda.synchronize()
            assert torch.equal(q1[0], q4[m]), (name, m)
            assert torch.equal(s1[0].view(torch.int32), s4[m].view(torch.int32)), (name, m)
            assert torch.equal(y1[0].view(torch.int32), y4[m].view(torch.int32)), (name, m)

def test_fused_quant_linear_with_no_rows_still_quantises():
    x = synth.make_activations(3, 512, seed=10)
    xd = _dev(x)
    hi0 = torch.zeros((0, 256), dtype=torch.uint8, device="cuda")
    sc0 = torch.zeros((0, 4), dtype=torch.int16, device="cuda")
    y, fq, fs = bn.bitnest_quant_linear_draft(xd, hi0, sc0)
    torch.cuda.synchronize()
    q, s = oracle.quant_act(x.numpy())
    assert y.shape == (3, 0)
    assert np.array_equal(fq.cpu().numpy(), q) and np.array_equal(fs.cpu().numpy(), s)



def _extreme_tokens(K, seed):
    # fp32 tokens whose maxima span the range: ordinary, 1e34 and 1e30 times
    # larger, 1e-30 and 1e-37 times smaller (s = amax / 127 subnormal), 1e-44
    # (the values themselves subnormal; s underflows to 0, so every code is
    # 0), a single nonzero value, and all zeros
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((8, K)).astype(np.float32)
    x = np.empty((8, K), np.float32)
    for i, f in enumerate([1.0, 1e34, 1e30, 1e-30, 1e-37, 1e-44]):
        x[i] = (base[i].astype(np.float64) * f).astype(np.float32)
    x[6] = 0.0
    x[6, K // 3] = -1.0
    x[7] = 0.0
    return x


@pytest.mark.parametrize("act_group", [0, 128])
def test_extreme_activation_magnitudes(act_group):
    # Codes and scales bit for bit against the oracle on every quantising
    # path (the quantisation kernel, the fused one-token launch, the fused
    # four-token launch), and y of the linears (GEMV at four tokens and in the
    # fused calls, matrix cores at eight) within 1e-5 of the sum of its group
    # terms' magnitudes
    N, K = 96, 4096
    x = _extreme_tokens(K, seed=21)
    w = synth.make_weights(N, K, seed=21)
    hn, ln, sc = w.numpy()
    q, s = oracle.quant_act(x, act_group)
    assert (q[5] == 0).all() and (s[5] == 0).all()          # the scale underflows: codes 0
    xd = torch.from_numpy(x).cuda()
    hi, lo, scd = _dev(w.hi), _dev(w.lo), _dev(w.scale)
    xq, xs = bn.bitnest_quant_act(xd, act_group)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), q)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s.view(np.uint32))

    def bound(P, f, qi, si):
        sa = si[:, None, None] if act_group == 0 else si[:, None, :]
        t = np.abs(P.astype(np.float64) * sc.view(np.float16).astype(np.float64)[None] * f * sa)
        return 1e-5 * t.sum(axis=2) + 1e-38

    def check(y, rows, target):
        qi, si = q[rows], s[rows]
        y64 = oracle.linear(qi, si, hn, sc, ln if target else None, act_group)
        P = oracle.partials(qi, hn, ln)[2] if target else oracle.partials(qi, hn)
        got = y.double().cpu().numpy()
        assert np.isfinite(got).all()
        assert (np.abs(got - y64) <= bound(P, 1 / 16 if target else 1.0, qi, si)).all(), (rows, target)

    for target in (False, True):
        planes = (hi, lo, scd) if target else (hi, scd)
        lin = bn.bitnest_linear_target if target else bn.bitnest_linear_draft
        fused = bn.bitnest_quant_linear_target if target else bn.bitnest_quant_linear_draft
        check(lin(xq, xs, *planes, act_group), list(range(8)), target)            # matrix cores
        check(lin(xq[:4].contiguous(), xs[:4].contiguous(), *planes, act_group), [0, 1, 2, 3], target)
        for m in range(8):                                                       # fused, one token
            y, fq, fs = fused(xd[m:m + 1].contiguous(), *planes, act_group)
            torch.cuda.synchronize()
            assert np.array_equal(fq.cpu().numpy(), q[m:m + 1]), m
            assert np.array_equal(fs.cpu().numpy().view(np.uint32), s[m:m + 1].view(np.uint32)), m
            check(y, [m], target)
        y, fq, fs = fused(xd[4:8].contiguous(), *planes, act_group)             # fused, four tokens
        torch.cuda.synchronize()
        assert bn.fused_in_one_launch(4, N, K)
        assert np.array_equal(fq.cpu().numpy(), q[4:8])
        assert np.array_equal(fs.cpu().numpy().view(np.uint32), s[4:8].view(np.uint32))
        check(y, [4, 5, 6, 7], target)

def _near_tie_rows(K=512):
    """Rows whose elements sit within a few ulps of (k + 1/2) * s, s = amax/127:
    the places where a reciprocal-multiply rounds differently from x / s."""
    rows = []
    for amax in (139.7, 3.3, 5.7, 0.91, 77.77, 1234.5, 17.0, 101.3):
        a = np.float32(amax)
        s = a / np.float32(127)
        vals = [a]
        for k in range(0, 126):
            x = np.float32((k + 0.5) * np.float64(s))
            for _ in range(3):
                x = np.nextafter(x, np.float32(-np.inf))
            for _ in range(7):
                vals.append(x if k % 2 else -x)
                x = np.nextafter(x, np.float32(np.inf))
        row = np.zeros(K * ((len(vals) + K - 1) // K), np.float32)
        row[:len(vals)] = vals
        rows.append(row)
    width = max(len(r) for r in rows)
    return np.stack([np.pad(r, (0, width - len(r))) for r in rows])


def test_quant_near_ties_bit_exact():
    x = _near_tie_rows()
    q_ref, s_ref = oracle.quant_act(x)
    xq, xs = bn.bitnest_quant_act(_dev(torch.from_numpy(x)))
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    # the fused prologue, one token at a time (M * K within one launch)
    for m in range(x.shape[0]):
        xm = torch.from_numpy(x[m:m + 1].copy())
        K = xm.shape[1]
        w = synth.make_weights(16, K)
        _, fq, fs = bn.bitnest_quant_linear_draft(_dev(xm), _dev(w.hi), _dev(w.scale))
        torch.cuda.synchronize()
        assert np.array_equal(fq.cpu().numpy()[0], q_ref[m])
        assert fs.item() == s_ref[m]


def test_quant_grouped_near_ties_bit_exact():
    x = _near_tie_rows(K=128)[:, :1024]
    q_ref, s_ref = oracle.quant_act(x, 128)
    xq, xs = bn.bitnest_quant_act(_dev(torch.from_numpy(x)), 128)
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
