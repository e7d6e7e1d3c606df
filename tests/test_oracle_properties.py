"""Property-based pins of the CPU oracle: random shapes and arbitrary finite
values (subnormal, negative, zero, extreme) against routes that share nothing
with it.

Sources (BitNest-Llama-3-8B model card): section "Files", entry
planes.safetensors (plane layout, nibble order, fp16 scales, the draft and
target dequantisation formulas); recipe table row "Activations" (symmetric
int8 per token, o_proj per 128-group).

- the activation codes and scales against numpy's IEEE fp32 division and
  round-half-even, element by element (the library form of the rule);
- the integer partials against sums taken here in Python integers, with the
  nibbles read from the hex spelling of each byte;
- y against exact rational arithmetic (Python fractions) within the fp64
  rounding bound of the oracle's sum.
Draws are derandomized, so the examples are the same on every run.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from hypothesis.extra import numpy as hnp

import oracle

GROUP = 128
SETTINGS = settings(max_examples=120, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

finite32 = st.floats(width=32, allow_nan=False, allow_infinity=False, allow_subnormal=True)


@st.composite
def activations(draw, max_m=3, max_groups=2):
    M = draw(st.integers(1, max_m))
    K = GROUP * draw(st.integers(1, max_groups))
    scale = draw(st.sampled_from([1.0, 1e30, 1e-30, 1e-39, 3e35]))
    base = draw(hnp.arrays(np.float32, (M, K), elements=st.floats(-100, 100, width=32)))
    x = (base.astype(np.float64) * scale).astype(np.float32)
    # a few arbitrary finite values anywhere in the row
    for _ in range(draw(st.integers(0, 4))):
        x[draw(st.integers(0, M - 1)), draw(st.integers(0, K - 1))] = draw(finite32)
    return x


def _numpy_rule(x, act_group):
    M, K = x.shape
    cols = K if act_group == 0 else GROUP
    xg = x.reshape(M, K // cols, cols)
    amax = np.abs(xg).max(axis=2)
    s = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s[:, :, None] == 0, np.float32(0),
                      np.rint(xg / s[:, :, None]).astype(np.float32))
    q = np.clip(qf, -127, 127).astype(np.int8).reshape(M, K)
    return q, (s[:, 0] if act_group == 0 else s)


@SETTINGS
@given(x=activations(), act_group=st.sampled_from([0, GROUP]))
def test_quant_act_is_numpy_ieee_rule(x, act_group):
    q, s = oracle.quant_act(x, act_group)
    q_np, s_np = _numpy_rule(x, act_group)
    assert np.array_equal(s.view(np.uint32), s_np.view(np.uint32))
    assert np.array_equal(q, q_np)
    assert q.min() >= -127


def _nibble(b, k):
    # column 2j is the low nibble of byte j, 2j + 1 the high one: read from
    # the hex spelling of the byte
    hx = "%02x" % int(b)
    return int(hx[1 if k % 2 == 0 else 0], 16)


@st.composite
def problems(draw):
    M = draw(st.integers(1, 2))
    N = draw(st.integers(1, 3))
    K = GROUP * draw(st.integers(1, 2))
    q = draw(hnp.arrays(np.int8, (M, K), elements=st.integers(-127, 127)))
    hi = draw(hnp.arrays(np.uint8, (N, K // 2)))
    lo = draw(hnp.arrays(np.uint8, (N, K // 2)))
    # any finite fp16 scale bit pattern (exponent field 31 excluded)
    sc = draw(hnp.arrays(np.uint16, (N, K // GROUP),
                         elements=st.integers(0, 0xFFFF).filter(lambda v: (v >> 10) & 0x1F != 0x1F)))
    g = draw(st.sampled_from([0, GROUP]))
    s = draw(hnp.arrays(np.float32, (M,) if g == 0 else (M, K // GROUP),
                        elements=st.floats(0, 1e3, width=32, allow_subnormal=True)))
    return q, hi, lo, sc, g, s


@SETTINGS
@given(p=problems())
def test_partials_are_integer_sums_of_the_nibbles(p):
    q, hi, lo, sc, g, s = p
    M, K = q.shape
    N = hi.shape[0]
    P_hi, P_lo, P8 = oracle.partials(q, hi, lo)
    for m in range(M):
        for n in range(N):
            for gg in range(K // GROUP):
                ph = pl = 0
                for k in range(gg * GROUP, (gg + 1) * GROUP):
                    ph += int(q[m, k]) * (_nibble(hi[n, k // 2], k) - 8)
                    pl += int(q[m, k]) * (_nibble(lo[n, k // 2], k) - 8)
                assert (P_hi[m, n, gg], P_lo[m, n, gg], P8[m, n, gg]) == (ph, pl, 16 * ph + pl)


@SETTINGS
@given(p=problems(), target=st.booleans())
def test_linear_is_the_exact_rational_sum(p, target):
    q, hi, lo, sc, g, s = p
    M, K = q.shape
    N = hi.shape[0]
    y = oracle.linear(q, s, hi, sc, lo if target else None, g)
    for m in range(M):
        for n in range(N):
            tot = absum = Fraction(0)
            for k in range(K):
                ch = _nibble(hi[n, k // 2], k) - 8
                cl = _nibble(lo[n, k // 2], k) - 8
                sw = Fraction(float(sc[n, k // GROUP:k // GROUP + 1].view(np.float16)[0]))
                w = sw * (Fraction(16 * ch + cl, 16) if target else ch)
                sa = Fraction(float(s[m] if g == 0 else s[m, k // GROUP]))
                term = int(q[m, k]) * sa * w
                tot += term
                absum += abs(term)
            # K fp64 additions and two products per term
            bound = (K + 3) * 2.0 ** -53 * float(absum)
            assert abs(float(tot) - y[m, n]) <= bound, (m, n)
