"""Pins of the CPU oracle against what the pages and the mathematics fix.

Sources (BitNest-Llama-3-8B model card): section "Files", entry
planes.safetensors (plane layout, nibble order, fp16 [N, K/128] scales, draft
and target dequantisation formulas); recipe table rows "Weights" (group size
128) and "Activations" (symmetric int8 per token, o_proj per 128-group).

Each pin is chosen so that a plausible slip in the oracle fails it: swapped
nibble order, wrong byte index, wrong offset (8 vs 7 or 128), a dropped 16 or
/16, a wrong group index, a transposed operand, round-half-away instead of
round-half-even, a missing clamp or a wrong activation scale.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GROUP = 128


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- fp16

def test_half_decoder_matches_ieee_binary16_everywhere():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(ref[np.isinf(ref)], got[np.isinf(ref)])
    assert np.all(np.isnan(got[np.isnan(ref)]))


# --------------------------------------------------------------------------- packing

def test_nibble_order_golden(golden_dir):
    fx = _load(golden_dir, "packing.json")
    rows = fx["rows"]
    plane = np.array([[int(r[0], 16) for r in rows]], dtype=np.uint8)
    u = oracle.unpack_plane(plane, 2 * len(rows))
    for j, r in enumerate(rows):
        assert u[0, 2 * j] == r[1], r
        assert u[0, 2 * j + 1] == r[2], r
        assert int(u[0, 2 * j]) - 8 == r[3]
        assert int(u[0, 2 * j + 1]) - 8 == r[4]


def test_unpack_every_byte_value_and_position():
    # 256 rows, each row's byte j is (row + 37 j) mod 256: every byte value at
    # many positions. Expected nibbles come from the hex spelling of the byte
    # (second hex digit = low nibble = even column), a route independent of
    # the oracle's shifts and masks.
    N, K = 256, 256
    plane = ((np.arange(N)[:, None] + 37 * np.arange(K // 2)[None, :]) % 256).astype(np.uint8)
    u = oracle.unpack_plane(plane, K)
    for n in range(0, N, 17):
        for j in range(K // 2):
            h = "%02x" % plane[n, j]
            assert u[n, 2 * j] == int(h[1], 16)
            assert u[n, 2 * j + 1] == int(h[0], 16)


# --------------------------------------------------------------------------- dequantisation

def _single_column_planes(pairs, K=GROUP):
    """Row i holds (hi, lo) nibble pair i in column 0; every other nibble is 8 (code 0)."""
    N = len(pairs)
    hi = np.full((N, K // 2), 0x88, np.uint8)
    lo = np.full((N, K // 2), 0x88, np.uint8)
    for i, (h, l) in enumerate(pairs):
        hi[i, 0] = 0x80 | h       # column 0 = low nibble of byte 0
        lo[i, 0] = 0x80 | l
    return hi, lo


def test_dequant_golden(golden_dir):
    fx = _load(golden_dir, "dequant.json")
    pairs = [(r[0], r[1]) for r in fx["rows"]]
    hi, lo = _single_column_planes(pairs)
    for sc in fx["scales"]:
        bits = int(sc["fp16_bits"], 16)
        scale = np.full((len(pairs), 1), bits, np.uint16)
        w4 = oracle.dequant(hi, scale)
        w8 = oracle.dequant(hi, scale, lo)
        for i, r in enumerate(fx["rows"]):
            assert w4[i, 0] == r[2] * sc["value"], (r, sc)
            assert w8[i, 0] == r[3] * sc["value"] / 16.0, (r, sc)
            assert np.all(w4[i, 1:] == 0) and np.all(w8[i, 1:] == 0)


def test_w8_codes_are_a_bijection_onto_minus136_119():
    # 16 * (hi - 8) + (lo - 8) over all 256 (hi, lo) pairs is every integer of
    # [-136, 119] exactly once; a zero point of 128 or a dropped factor fails.
    pairs = [(h, l) for h in range(16) for l in range(16)]
    hi, lo = _single_column_planes(pairs)
    scale = np.full((256, 1), 0x4C00, np.uint16)        # 16.0: W8 = code exactly
    w8 = oracle.dequant(hi, scale, lo)[:, 0]
    assert sorted(w8.astype(int).tolist()) == list(range(-136, 120))
    w4 = oracle.dequant(hi, np.full((256, 1), 0x3C00, np.uint16))[:, 0]
    vals, counts = np.unique(w4, return_counts=True)
    assert vals.tolist() == list(range(-8, 8)) and set(counts.tolist()) == {16}
    # Nesting: the target code's top part is the draft code, refined by lo.
    assert np.array_equal(np.floor((w8 + 136) / 16) - 8, w4)


def test_scale_groups_follow_columns_of_128():
    N, K = 2, 3 * GROUP
    hi = np.full((N, K // 2), 0x99, np.uint8)            # every code = +1
    scale = np.array([[0x3C00, 0x4000, 0x3400],         # 1, 2, 0.25
                      [0x3800, 0x3C00, 0x4400]], np.uint16)  # 0.5, 1, 4
    W = oracle.dequant(hi, scale)
    expect = np.repeat(np.array([[1.0, 2.0, 0.25], [0.5, 1.0, 4.0]]), GROUP, axis=1)
    assert np.array_equal(W, expect)


# --------------------------------------------------------------------------- activation quant

def test_act_quant_golden_ties_to_even(golden_dir):
    fx = _load(golden_dir, "act_quant.json")
    for case in fx["per_token"]:
        x = np.array([case["x"]], np.float32)   # act_group 0 takes any K
        q, s = oracle.quant_act(x)
        assert s[0] == np.float32(case["s"])
        assert q[0].tolist() == case["q"], case


def test_act_quant_grouped_golden(golden_dir):
    g = _load(golden_dir, "act_quant.json")["grouped"]
    K = g["K"]
    x = np.zeros((1, K), np.float32)
    x[0, 0] = g["group0"]["amax_value"]
    x[0, GROUP] = g["group1"]["amax_value"]
    for grp in ("group0", "group1"):
        for col, val, _ in g[grp]["probe"]:
            x[0, col] = val
    q, s = oracle.quant_act(x, act_group=GROUP)
    assert s.shape == (1, 2)
    assert s[0, 0] == g["group0"]["s"] and s[0, 1] == g["group1"]["s"]
    assert q[0, 0] == 127 and q[0, GROUP] == 127
    for grp in ("group0", "group1"):
        for col, _, code in g[grp]["probe"]:
            assert q[0, col] == code


def _rand_x(rng, M, K, outliers=True):
    x = rng.standard_normal((M, K)).astype(np.float32)
    if outliers:
        idx = rng.choice(K, size=max(1, K // 200), replace=False)
        x[:, idx] *= 20
    return x


@pytest.mark.parametrize("act_group", [0, GROUP])
def test_act_quant_equals_library_rounding(act_group):
    # numpy's fp32 division and np.rint (IEEE round half to even) give the
    # textbook form of the rule; the oracle must agree code for code.
    rng = np.random.default_rng(1)
    M, K = 5, 1024
    x = _rand_x(rng, M, K)
    x[2] = 0.0
    q, s = oracle.quant_act(x, act_group)
    R = K if act_group == 0 else GROUP
    xr = x.reshape(M, K // R, R)
    amax = np.abs(xr).max(axis=2)
    s_ref = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = (xr / s_ref[:, :, None]).astype(np.float32)
    q_ref = np.where(s_ref[:, :, None] == 0, 0, np.clip(np.rint(t), -127, 127)).astype(np.int8)
    assert np.array_equal(q, q_ref.reshape(M, K))
    assert np.array_equal(s.reshape(M, -1), s_ref)


def test_act_quant_near_ties_divide_not_reciprocal():
    # Elements within a few ulps of (k + 1/2) * s, kept only where the IEEE
    # quotient x / s and the product x * fl(1/s) round to different codes.
    # numpy's fp32 division and np.rint (the library form of the rule) decide
    # the expected code; an oracle that multiplies by a reciprocal fails here.
    rows, expect = [], []
    for amax in (139.7, 3.3, 5.7, 0.91, 77.77, 1234.5, 17.0, 101.3):
        a = np.float32(amax)
        s = a / np.float32(127)
        r = np.float32(1) / s
        row, codes = [a], [127]
        for k in range(0, 126):
            x = np.float32((k + 0.5) * np.float64(s))
            for _ in range(4):
                x = np.nextafter(x, np.float32(-np.inf))
            for _ in range(9):
                if np.rint(x / s) != np.rint(x * r):
                    row.append(x)
                    codes.append(int(np.rint(x / s)))
                x = np.nextafter(x, np.float32(np.inf))
        rows.append(np.array(row, np.float32))
        expect.append(codes)
    assert sum(len(c) - 1 for c in expect) >= 10
    for row, codes in zip(rows, expect):
        q, s = oracle.quant_act(row[None, :])
        assert s[0] == row[0] / np.float32(127)
        assert q[0].tolist() == codes


@pytest.mark.parametrize("act_group", [0, GROUP])
def test_act_quant_properties(act_group):
    rng = np.random.default_rng(2)
    M, K = 4, 2048
    x = _rand_x(rng, M, K)
    q, s = oracle.quant_act(x, act_group)
    R = K if act_group == 0 else GROUP
    s2 = s.reshape(M, -1)
    qr = q.reshape(M, K // R, R).astype(np.float64)
    xr = x.reshape(M, K // R, R).astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    # the largest-magnitude element of each set maps to +-127
    i = np.abs(xr).argmax(axis=2)
    top = np.take_along_axis(qr, i[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == 127)
    # reconstruction error within half a step (plus fp32 division rounding)
    err = np.abs(qr * s2[:, :, None] - xr)
    assert np.all(err <= s2[:, :, None] * (0.5 + 1e-5))
    # symmetric: negating x negates the codes and keeps the scales
    qn, sn = oracle.quant_act(-x, act_group)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # power-of-two scaling of x leaves the codes unchanged and scales s exactly
    q4, s4 = oracle.quant_act(x * np.float32(4.0), act_group)
    assert np.array_equal(q4, q) and np.array_equal(s4, s * np.float32(4.0))


# --------------------------------------------------------------------------- partials and linear

def _onehot_problem(golden_dir):
    fx = _load(golden_dir, "onehot_linear.json")
    N, K = fx["N"], fx["K"]
    fill = int(fx["fill_byte"], 16)
    hi = np.full((N, K // 2), fill, np.uint8)
    lo = np.full((N, K // 2), fill, np.uint8)
    for e in fx["hi_bytes"]:
        hi[e["row"], e["byte"]] = int(e["value"], 16)
    for e in fx["lo_bytes"]:
        lo[e["row"], e["byte"]] = int(e["value"], 16)
    scale = np.array([[int(b, 16) for b in r] for r in fx["scale_bits"]], np.uint16)
    x = np.zeros((1, K), np.float32)
    x[0, fx["x_nonzero"]["column"]] = fx["x_nonzero"]["value"]
    return fx, x, hi, lo, scale


def test_onehot_linear_golden(golden_dir):
    fx, x, hi, lo, scale = _onehot_problem(golden_dir)
    q, s = oracle.quant_act(x)
    assert s[0] == fx["act_scale"]
    assert q[0, fx["x_nonzero"]["column"]] == fx["act_code"]
    assert np.count_nonzero(q) == 1
    p_hi, p_lo, p8 = oracle.partials(q, hi, lo)
    assert p_hi.tolist() == fx["p_hi"]
    assert p_lo.tolist() == fx["p_lo"]
    assert p8.tolist() == fx["p8"]
    assert oracle.partials(q, hi).tolist() == fx["p_hi"]
    assert oracle.linear(q, s, hi, scale).tolist() == fx["y_draft"]
    assert oracle.linear(q, s, hi, scale, lo).tolist() == fx["y_target"]


def _random_problem(seed, M, N, K, lo_const=None):
    rng = np.random.default_rng(seed)
    hi = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    lo = rng.integers(0, 256, (N, K // 2), dtype=np.uint8) if lo_const is None else \
        np.full((N, K // 2), lo_const, np.uint8)
    scale = np.exp(np.log(0.01) + 0.3 * rng.standard_normal((N, K // GROUP))) \
        .astype(np.float16).view(np.uint16)
    x = _rand_x(rng, M, K)
    return x, hi, lo, scale


def test_brute_force_exact_rationals_tiny():
    # An independent route: nibbles from the hex spelling of each byte, fp16
    # from numpy, and exact rational arithmetic for the whole sum. The oracle's
    # fp64 result must be the exact value to within a few fp64 roundings.
    M, N, K = 2, 3, 2 * GROUP
    x, hi, lo, scale = _random_problem(11, M, N, K)
    for act_group in (0, GROUP):
        q, s = oracle.quant_act(x, act_group)
        for target in (False, True):
            y = oracle.linear(q, s, hi, scale, lo if target else None, act_group)
            for m in range(M):
                for n in range(N):
                    tot = Fraction(0)
                    absum = Fraction(0)
                    for k in range(K):
                        hx = "%02x" % hi[n, k // 2]
                        lx = "%02x" % lo[n, k // 2]
                        pos = 1 if k % 2 == 0 else 0
                        ch = int(hx[pos], 16) - 8
                        cl = int(lx[pos], 16) - 8
                        sw = Fraction(float(scale[n, k // GROUP:k // GROUP + 1].view(np.float16)[0]))
                        w = sw * (Fraction(16 * ch + cl, 16) if target else ch)
                        sa = Fraction(float(s[m] if act_group == 0 else s[m, k // GROUP]))
                        term = int(q[m, k]) * sa * w
                        tot += term
                        absum += abs(term)
                    # K fp64 additions and two products per term: |err| <= (K + 3) u sum|terms|
                    bound = (K + 3) * 2.0 ** -53 * float(absum)
                    assert abs(float(tot) - y[m, n]) <= bound, (m, n, target, act_group)


@pytest.mark.parametrize("act_group", [0, GROUP])
def test_target_equals_draft_when_lo_is_8(act_group):
    # lo == 8 everywhere means every lo code is 0: W8 = 16 (hi - 8) scale / 16
    # = W4 exactly, so the two linears must agree bit for bit.
    M, N, K = 3, 40, 4 * GROUP
    x, hi, lo, scale = _random_problem(3, M, N, K, lo_const=0x88)
    q, s = oracle.quant_act(x, act_group)
    assert np.array_equal(oracle.linear(q, s, hi, scale, lo, act_group),
                          oracle.linear(q, s, hi, scale, None, act_group))
    p_hi, p_lo, p8 = oracle.partials(q, hi, lo)
    assert not p_lo.any()
    assert np.array_equal(p8, 16 * p_hi)


def test_combined_partial_identity_and_bounds():
    M, N, K = 4, 33, 5 * GROUP
    x, hi, lo, scale = _random_problem(4, M, N, K)
    q, _ = oracle.quant_act(x)
    p_hi, p_lo, p8 = oracle.partials(q, hi, lo)
    assert np.array_equal(p8.astype(np.int64), 16 * p_hi.astype(np.int64) + p_lo)
    assert np.abs(p_hi).max() <= 127 * 8 * GROUP
    assert np.abs(p8).max() <= 127 * 136 * GROUP
    # extreme inputs reach the bounds exactly
    qx = np.full((1, GROUP), -127, np.int8)
    h0 = np.zeros((1, GROUP // 2), np.uint8)              # every code -8
    ph, pl, pe = oracle.partials(qx, h0, h0)
    assert ph[0, 0, 0] == 127 * 8 * GROUP and pe[0, 0, 0] == 127 * 136 * GROUP


@pytest.mark.parametrize("act_group", [0, GROUP])
def test_verify_batch_rows_equal_single_token_calls(act_group):
    # Per-token quantisation makes rows independent: an M = 4 call is four
    # M = 1 calls stacked, bit for bit.
    M, N, K = 4, 24, 3 * GROUP
    x, hi, lo, scale = _random_problem(5, M, N, K)
    q, s = oracle.quant_act(x, act_group)
    y4 = oracle.linear(q, s, hi, scale, lo, act_group)
    p4 = oracle.partials(q, hi, lo)
    for m in range(M):
        q1, s1 = oracle.quant_act(x[m:m + 1], act_group)
        assert np.array_equal(q1, q[m:m + 1])
        assert np.array_equal(oracle.linear(q1, s1, hi, scale, lo, act_group), y4[m:m + 1])
        p1 = oracle.partials(q1, hi, lo)
        for a, b in zip(p1, p4):
            assert np.array_equal(a[0], b[m])


@pytest.mark.parametrize("act_group", [0, GROUP])
def test_factorised_form_equals_dequantise_then_multiply(act_group):
    # sum_g P[m,n,g] * scale[n,g] * f * s_a equals the plain definition.
    M, N, K = 3, 20, 4 * GROUP
    x, hi, lo, scale = _random_problem(6, M, N, K)
    q, s = oracle.quant_act(x, act_group)
    p_hi, p_lo, p8 = oracle.partials(q, hi, lo)
    sw = scale.view(np.float16).astype(np.float64)
    sa = s.astype(np.float64)[:, None, None] if act_group == 0 else s.astype(np.float64)[:, None, :]
    yd = (p_hi * sw[None] * sa).sum(axis=2)
    yt = (p8 * (sw[None] / 16.0) * sa).sum(axis=2)
    np.testing.assert_allclose(oracle.linear(q, s, hi, scale, None, act_group), yd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.linear(q, s, hi, scale, lo, act_group), yt, rtol=1e-12, atol=1e-12)
    # and the dense dequantised matrices under a library matmul
    xhat = q.astype(np.float64) * (np.repeat(s.astype(np.float64), GROUP, axis=1) if act_group else
                                   s.astype(np.float64)[:, None])
    np.testing.assert_allclose(xhat @ oracle.dequant(hi, scale).T, yd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(xhat @ oracle.dequant(hi, scale, lo).T, yt, rtol=1e-12, atol=1e-12)


def test_linear_is_transposed_correctly_on_non_square_shapes():
    # A one-hot token at column k must return column k of W [N, K] (length N).
    M, N, K = 1, 7, 3 * GROUP
    _, hi, lo, scale = _random_problem(8, M, N, K)
    W = oracle.dequant(hi, scale, lo)
    for k in (0, 1, 200, K - 1):
        q = np.zeros((1, K), np.int8)
        q[0, k] = 1
        y = oracle.linear(q, np.ones(1, np.float32), hi, scale, lo)
        assert y.shape == (1, N)
        assert np.array_equal(y[0], W[:, k])


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.unpack_plane(np.zeros((2, 3), np.uint8), 4)
    with pytest.raises(oracle.OracleError):
        oracle.quant_act(np.zeros((1, 100), np.float32), act_group=GROUP)


# --------------------------------------------------------------------------- R4 rotation (down_proj input)
# Reading (model card, recipe table row "Rotation": an online Hadamard, R4, on
# the down_proj inputs; the matrices themselves are not given): block-diagonal
# normalised Sylvester-Hadamard H_b / sqrt(b), fp32 fast transform, one
# multiply by the fp32 value nearest 1/sqrt(b).

def _f32_bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def _sylvester(b):
    """H_b by the closed form H[i][j] = (-1)^popcount(i & j) (int64)."""
    i = np.arange(b)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def test_hadamard_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hadamard.json")))
    for case in g["cases"]:
        b = case["block"]
        x = np.array([case["x"]], np.float32)
        y = oracle.hadamard_rotate(x, b)
        if "y" in case:
            assert np.array_equal(y[0], np.array(case["y"], np.float32))
        r = np.array([int(case.get("r_bits", "0x3f000000"), 16)], np.uint32).view(np.float32)[0]
        want = (np.array(case["Hx"], np.float32) * r).astype(np.float32)
        assert np.array_equal(y[0], want), (b, y, want)
    # the normalisation constant for the Llama-3-8B block
    e0 = np.zeros((1, 512), np.float32)
    e0[0, 0] = 1.0
    assert _f32_bits(oracle.hadamard_rotate(e0, 512)[0, 0]) == int(g["r_512_bits"], 16)


@pytest.mark.parametrize("b", [2, 8, 16, 64, 512])
def test_hadamard_columns_closed_form(b):
    # the transform of a one-hot vector e_j is column j of H_b times r_b, exactly
    H = _sylvester(b)
    r = oracle.hadamard_rotate(np.eye(1, b, 0, dtype=np.float32), b)[0, 0]
    js = range(b) if b <= 64 else [0, 1, 2, 3, 5, 64, 255, 256, 300, 511]
    for j in js:
        e = np.zeros((1, b), np.float32)
        e[0, j] = 1.0
        y = oracle.hadamard_rotate(e, b)[0]
        assert np.array_equal(y, (H[:, j] * r).astype(np.float32)), j


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 4096])
def test_hadamard_constant_is_nearest_fp32(b):
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    r = oracle.hadamard_rotate(np.eye(1, b, 0, dtype=np.float32), b)[0, 0]
    exact = Decimal(1) / Decimal(b).sqrt()
    bits = _f32_bits(r)
    err = abs(Decimal(float(r)) - exact)
    for nb in (bits - 1, bits + 1):
        other = float(np.array([nb], np.uint32).view(np.float32)[0])
        assert err <= abs(Decimal(other) - exact)


@pytest.mark.parametrize("b", [4, 16, 64, 256])
def test_hadamard_involution_exact(b):
    # for even log2(b) the constant is a power of two, so small integer inputs
    # stay exact: R applied twice is the identity (H_b^2 = b I)
    rng = np.random.default_rng(b)
    x = rng.integers(-8, 9, size=(3, 4 * b)).astype(np.float32)
    y = oracle.hadamard_rotate(oracle.hadamard_rotate(x, b), b)
    assert np.array_equal(y, x)


def test_hadamard_dense_fp64_and_norm():
    # Llama-3-8B down_proj input: 28 blocks of 512, with outlier channels
    b, K = 512, 14336
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, K)).astype(np.float32)
    x[:, rng.choice(K, 72, replace=False)] *= 20
    y = oracle.hadamard_rotate(x, b).astype(np.float64)
    H = _sylvester(b).astype(np.float64) / np.sqrt(b)
    ref = np.concatenate([x[:, i:i + b].astype(np.float64) @ H.T for i in range(0, K, b)], axis=1)
    u = 2.0 ** -24
    for i in range(0, K, b):
        bound = (np.log2(b) + 2) * u * np.abs(x[:, i:i + b]).sum(axis=1, keepdims=True).astype(np.float64) / np.sqrt(b)
        assert np.all(np.abs(y[:, i:i + b] - ref[:, i:i + b]) <= bound)
        nx = np.linalg.norm(x[:, i:i + b].astype(np.float64), axis=1)
        ny = np.linalg.norm(y[:, i:i + b], axis=1)
        assert np.allclose(nx, ny, rtol=1e-5)


def test_hadamard_blocks_independent_and_scaling():
    b, K = 512, 14336
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, K)).astype(np.float32)
    y = oracle.hadamard_rotate(x, b)
    for i in (0, 512, 13824):
        assert np.array_equal(y[:, i:i + b], oracle.hadamard_rotate(np.ascontiguousarray(x[:, i:i + b]), b))
    assert np.array_equal(oracle.hadamard_rotate(x * 4, b), y * 4)
    assert np.array_equal(oracle.hadamard_rotate(-x, b), -y)


def test_hadamard_bad_args():
    x = np.zeros((1, 96), np.float32)
    for b in (0, 1, 3, 12, 64, 128):
        with pytest.raises(oracle.OracleError):
            oracle.hadamard_rotate(x, b)


# --------------------------------------------------------------------------- offline nested packing
# Reading (model card introduction and planes.safetensors): symmetric 15-step
# RTN high nibble with fp16 scale amax / 7.5, closed-form residual low nibble.

def test_float_to_half_matches_ieee_library():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(20000) * 1000, rng.standard_normal(20000) * 1e-6,
                         [0.0, 6.1035156e-05, 5.96e-08, 2.98e-08, 65504.0, 65519.0, 1e-10, -3.0e-6, 0.5,
                          1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]]).astype(np.float32)
    got = np.array([oracle.float_to_half_bits(x) for x in xs], np.uint16)
    assert np.array_equal(got, xs.astype(np.float16).view(np.uint16))


def test_pack_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pack.json")))
    W = np.zeros((g["N"], g["K"]), np.float32)
    for k, v in g["group0_values"].items():
        W[0, int(k)] = v
    hi, lo, sc = oracle.pack_nested(W)
    fill = int(g["fill_byte"], 16)
    want_hi = np.full(g["K"] // 2, fill, np.uint8)
    want_lo = np.full(g["K"] // 2, fill, np.uint8)
    want_hi[:4] = [int(b, 16) for b in g["hi_bytes_group0_first4"]]
    want_lo[:4] = [int(b, 16) for b in g["lo_bytes_group0_first4"]]
    assert np.array_equal(hi[0], want_hi)
    assert np.array_equal(lo[0], want_lo)
    assert [int(v) for v in sc[0]] == [int(b, 16) for b in g["scale_bits"]]


def _packed_codes(W):
    hi, lo, sc = oracle.pack_nested(W)
    K = W.shape[1]
    ch = oracle.unpack_plane(hi, K).astype(np.int64) - 8
    cl = oracle.unpack_plane(lo, K).astype(np.int64) - 8
    s = np.repeat(sc.view(np.float16).astype(np.float64), 128, axis=1)
    return hi, lo, sc, ch, cl, s


def test_pack_error_bounds_and_formulas():
    rng = np.random.default_rng(12)
    W = (rng.standard_t(4, size=(24, 1024)) * 0.02).astype(np.float32)
    W[3, :128] = 0.0                                      # an all-zero group
    hi, lo, sc, ch, cl, s = _packed_codes(W)
    w = W.astype(np.float64)
    # the scale is fp16(amax / 7.5) of its group
    amax = np.abs(W).reshape(24, 8, 128).max(axis=2)
    assert np.array_equal(sc, (amax / np.float32(7.5)).astype(np.float32).astype(np.float16).view(np.uint16))
    # codes in range; a zero group gives zero codes
    assert ch.min() >= -8 and ch.max() <= 7 and cl.min() >= -8 and cl.max() <= 7
    assert not ch[3, :128].any() and not cl[3, :128].any()
    # the model card's formulas: W4 = c_hi s, W8 = (16 c_hi + c_lo) s / 16
    W4 = ch * s
    W8 = (16 * ch + cl) * s / 16
    assert np.allclose(oracle.dequant(hi, sc), W4, rtol=0, atol=0)
    assert np.allclose(oracle.dequant(hi, sc, lo), W8, rtol=0, atol=0)
    # where no clamp acts: |W4 - W| <= s/2 and |W8 - W| <= s/32
    ss = np.where(s > 0, s, 1.0)
    u = w / ss
    t = (w - W4) * 16 / ss
    free_hi = (s > 0) & (u > -8.5) & (u < 7.5)
    free = free_hi & (t > -8.5) & (t < 7.5)
    assert free_hi.mean() > 0.99 and free.mean() > 0.9
    tol = 1 + 2.0 ** -20
    assert np.all(np.abs(W4 - w)[free_hi] <= s[free_hi] / 2 * tol)
    assert np.all(np.abs(W8 - w)[free] <= s[free] / 32 * tol)
    # W8 is never worse than W4 by more than the residual clamp allows
    assert np.all(np.abs(W8 - w) <= np.abs(W4 - w) + 1e-12)


def test_pack_on_the_w4_grid_gives_lo_8():
    # a group with amax 1.875 has s = fp16(0.25) exactly; values k * 0.25 for
    # |k| <= 7 are on the W4 grid, so their residual code is 0 (lo = 8)
    rng = np.random.default_rng(13)
    W = (rng.integers(-7, 8, size=(4, 256)) * 0.25).astype(np.float32)
    W[:, 0] = 1.875
    W[:, 128] = -1.875
    hi, lo, sc, ch, cl, s = _packed_codes(W)
    assert np.all(sc == np.float16(0.25).view(np.uint16))
    grid = np.ones(W.shape, bool)
    grid[:, [0, 128]] = False
    assert np.all(cl[grid] == 0)
    assert np.array_equal(ch[grid], (W[grid] / 0.25).astype(np.int64))


def test_pack_sign_and_power_of_two_symmetry():
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((6, 512)) * 0.03).astype(np.float32)
    hi, lo, sc, ch, cl, s = _packed_codes(W)
    # doubling W doubles every scale exactly and keeps every code
    hi2, lo2, sc2 = oracle.pack_nested(W * 2)
    assert np.array_equal(hi2, hi) and np.array_equal(lo2, lo)
    assert np.array_equal(sc2.view(np.float16), (sc.view(np.float16).astype(np.float32) * 2).astype(np.float16))
    # negating W negates the codes except where the asymmetric range clamps
    _, _, scn, chn, cln, _ = _packed_codes(-W)
    assert np.array_equal(scn, sc)
    ok = (ch > -8) & (ch < 7) & (cl > -8) & (cl < 7) & (np.abs((W / s).astype(np.float64) % 1) != 0.5)
    assert np.array_equal(chn[ok], -ch[ok])


# --------------------------------------------------------------------------- greedy verification
# Reading (model card introduction: the output is exactly the target's greedy
# output): argmax per verify row, ties to the smallest index, accept the
# longest matching prefix, emit the target's token after it.

def test_accept_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "accept.json")))
    logits = np.array(g["logits"], np.float32)
    for case in g["cases"]:
        targ, n, nxt = oracle.greedy_accept(logits, np.array(case["draft"], np.int32))
        assert list(targ) == g["targ"]
        assert (n, nxt) == (case["n"], case["next"]), case["why"]


def test_accept_argmax_is_the_library_argmax():
    # numpy's argmax returns the first maximum: the same tie rule
    rng = np.random.default_rng(15)
    for V in (1, 2, 7, 1000, 128256):
        logits = rng.standard_normal((4, V)).astype(np.float32)
        if V > 10:
            logits[1, [3, V - 1]] = logits[1].max() + 1.0          # a tie at the maximum
            logits[2] = np.round(logits[2])                          # many ties
        targ, _, _ = oracle.greedy_accept(logits, np.zeros(3, np.int32))
        assert np.array_equal(targ, np.argmax(logits, axis=1))


def test_accept_emits_the_target_greedy_sequence():
    # whatever the drafts, the emitted tokens (accepted drafts + next) are the
    # target's argmax tokens t_0 .. t_n
    rng = np.random.default_rng(16)
    for _ in range(200):
        R = int(rng.integers(1, 9))
        logits = rng.standard_normal((R, 50)).astype(np.float32)
        t = np.argmax(logits, axis=1)
        draft = t[:R - 1].copy()
        if R > 1 and rng.random() < 0.7:
            k = int(rng.integers(0, R - 1))
            draft[k] = (draft[k] + 1 + int(rng.integers(0, 48))) % 50
        targ, n, nxt = oracle.greedy_accept(logits, draft.astype(np.int32))
        emitted = list(draft[:n]) + [nxt]
        assert emitted == list(t[:n + 1])
        assert n == R - 1 or draft[n] != t[n]


# --------------------------------------------------------------------------- nested KV cache attention
# Reading (recipe table row "KV cache": the draft reads KV4, the target KV8):
# every (token, KV head) vector of 128 values packed like one weight group;
# grouped-query heads, causal visibility for the M query tokens, scores / sqrt(128).

def _kv_cache(Kf, Vf):
    """fp32 [T, Hkv, 128] K and V -> nested planes [T, Hkv, 64] and scales [T, Hkv] (the packer)."""
    T, Hkv, d = Kf.shape
    out = []
    for X in (Kf, Vf):
        hi, lo, sc = oracle.pack_nested(np.ascontiguousarray(X.reshape(T * Hkv, d)))
        out.append((hi.reshape(T, Hkv, d // 2), lo.reshape(T, Hkv, d // 2), sc.reshape(T, Hkv)))
    return out


def _kv_dequant(planes, lo=True):
    hi, lo_p, sc = planes
    T, Hkv, half = hi.shape
    W = oracle.dequant(hi.reshape(T * Hkv, half), sc.reshape(T * Hkv, 1), lo_p.reshape(T * Hkv, half) if lo else None)
    return W.reshape(T, Hkv, 2 * half)


def _attn(q, kc, vc, lo=True):
    return oracle.kv_attention(q, kc[0], kc[2], vc[0], vc[2], kc[1] if lo else None, vc[1] if lo else None)


def test_kv_single_visible_position_returns_its_value():
    rng = np.random.default_rng(20)
    Kf = rng.standard_normal((4, 2, 128)).astype(np.float32)
    Vf = rng.standard_normal((4, 2, 128)).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vf)
    q = rng.standard_normal((4, 4, 128)).astype(np.float32)       # M = T = 4: token 0 sees position 0 only
    for lo in (False, True):
        out = _attn(q, kc, vc, lo)
        V = _kv_dequant(vc, lo)
        for h in range(4):
            assert np.array_equal(out[0, h], V[0, h // 2])


def test_kv_equal_keys_average_the_values():
    rng = np.random.default_rng(21)
    T, Hkv = 37, 2
    Kf = np.repeat(rng.standard_normal((1, Hkv, 128)), T, axis=0).astype(np.float32)
    Vf = (rng.standard_normal((T, Hkv, 128)) * rng.uniform(0.1, 3, size=(T, Hkv, 1))).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vf)
    q = rng.standard_normal((3, 8, 128)).astype(np.float32)
    out = _attn(q, kc, vc)
    V = _kv_dequant(vc)
    for i in range(3):
        vis = T - 3 + i + 1
        for h in range(8):
            assert np.allclose(out[i, h], V[:vis, h // 4].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_kv_two_positions_closed_form_weights():
    # softmax over two scores: weights 1 / (1 + r) and r / (1 + r) with
    # r = exp((q.k1 - q.k0) / sqrt(128))
    rng = np.random.default_rng(22)
    Kf = (rng.standard_normal((2, 1, 128)) * 0.2).astype(np.float32)
    Vf = rng.standard_normal((2, 1, 128)).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vf)
    q = rng.standard_normal((1, 1, 128)).astype(np.float32)
    K, V = _kv_dequant(kc), _kv_dequant(vc)
    qd = q[0, 0].astype(np.float64)
    r = np.exp((qd @ K[1, 0] - qd @ K[0, 0]) / np.sqrt(128.0))
    want = (V[0, 0] + r * V[1, 0]) / (1 + r)
    assert np.allclose(_attn(q, kc, vc)[0, 0], want, rtol=1e-12, atol=1e-12)


def test_kv_peaked_score_selects_one_position():
    rng = np.random.default_rng(23)
    T = 50
    Kf = np.zeros((T, 1, 128), np.float32)
    Kf[17, 0, :] = 2.0                                  # only position 17 aligns with q
    Vf = rng.standard_normal((T, 1, 128)).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vf)
    q = np.full((1, 1, 128), 2.0, np.float32)           # score of 17: 512 / sqrt(128) = 45
    out = _attn(q, kc, vc)
    assert np.allclose(out[0, 0], _kv_dequant(vc)[17, 0], rtol=0, atol=1e-12)


def test_kv_grouped_heads_and_causality():
    rng = np.random.default_rng(24)
    T, Hkv, Hq, M = 40, 2, 8, 4
    Kf = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    Vf = np.zeros((T, Hkv, 128), np.float32)
    Vf[:, 0, :] = 1.5                                   # KV head 0's values all 1.5, head 1's all -0.75
    Vf[:, 1, :] = -0.75
    kc, vc = _kv_cache(Kf, Vf)
    q = rng.standard_normal((M, Hq, 128)).astype(np.float32)
    out = _attn(q, kc, vc)
    V = _kv_dequant(vc)
    for h in range(Hq):                                  # query heads 0-3 read KV head 0, 4-7 KV head 1
        assert np.allclose(out[:, h], V[0, h // 4, 0], rtol=1e-12)
    # token i of an M-token call equals a one-token call on the cache cut after position T - M + i
    Vr = rng.standard_normal((T, Hkv, 128)).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vr)
    out = _attn(q, kc, vc)
    for i in range(M):
        n = T - M + i + 1
        cut = [tuple(a[:n] for a in kc), tuple(a[:n] for a in vc)]
        one = _attn(q[i:i + 1], cut[0], cut[1])
        assert np.array_equal(out[i], one[0])


def test_kv4_equals_kv8_when_lo_is_8_and_value_scaling():
    rng = np.random.default_rng(25)
    Kf = rng.standard_normal((30, 2, 128)).astype(np.float32)
    Vf = rng.standard_normal((30, 2, 128)).astype(np.float32)
    kc, vc = _kv_cache(Kf, Vf)
    q = rng.standard_normal((2, 4, 128)).astype(np.float32)
    k8 = (kc[0], np.full_like(kc[1], 0x88), kc[2])
    v8 = (vc[0], np.full_like(vc[1], 0x88), vc[2])
    assert np.array_equal(_attn(q, k8, v8, lo=True), _attn(q, kc, vc, lo=False))
    # doubling every value scale doubles the output exactly
    v2 = (vc[0], vc[1], (vc[2].view(np.float16) * np.float16(2)).view(np.uint16))
    assert np.array_equal(_attn(q, kc, v2), 2 * _attn(q, kc, vc))
