"""The fp32 route the position kernels take to cos θ and sin θ for 16-bit
tables, emulated on the CPU, against the definition of the tables from
positions ("ANE实战RoPE位置编码在MIL中的纯ANE实现", section 第一步: θ = p /
base^(2i/h); cos θ and sin θ rounded once to the table type from their
double values, as oracle.round_double rounds). The route: θ = k π/2 + r in
double with π/2 split into three doubles (one fused multiply-add per part;
r = θ when k = 0),
the Taylor series of sin r (to r^9, as r + r z p(z)) and cos r (to r^10) in
fp32, the quadrant's swap and signs, then Ziv's test: a value v is kept
when the ends of an interval around it (half-width |v| 2^-21 + 2^-50 from
the sine, without the 2^-50 when k = 0 and the reduction is exact; 2^-21
from the cosine; each end moved out by |v| 2^-23) round to one value of
the table type.

Checked here, over angles of the workloads' kinds and of every edge: the
series' errors stay within the bounds the half-widths rest on (the sine
within 2.4 units of 2^-24 of |sin r|, the cosine within 1.1e-7), and every
value that passes the test rounds as the double value does. The GPU tests
check the kernels bit for bit; this checks the argument, on many more
angles. The reduction is done exactly (fractions) as fused multiply-adds
round it; the fp32 steps are numpy fp32 operations, a fused multiply-add
being the exact double product and sum rounded to fp32."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

getcontext().prec = 120
# pi to 110 digits
PI = Fraction(Decimal("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899862803482534211706798214808651"))
PIO2 = PI / 2
P1 = float(PIO2)
P2 = float(PIO2 - Fraction(P1))
P3 = float(PIO2 - Fraction(P1) - Fraction(P2))
TWO_OVER_PI = float(1 / PIO2)
F32 = np.float32


def _fma_round(a, b, c):
    """round(a*b + c) to double, exactly (one rounding)."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _reduce(theta: float):
    k = float(np.rint(theta * TWO_OVER_PI))
    if k == 0.0:
        return k, float(theta), Fraction(float(theta))   # exact; -0 keeps its sign
    r = _fma_round(-k, P1, theta)
    r = _fma_round(-k, P2, r)
    r = _fma_round(-k, P3, r)
    return k, r, Fraction(float(theta)) - PIO2 * Fraction(k)   # also the exact reduced argument


def _fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def _series(r: np.ndarray):
    x = r.astype(F32)
    z = x * x
    sp = np.full_like(x, F32(1 / 362880))
    for c in (-1 / 5040, 1 / 120, -1 / 6):
        sp = _fma32(sp, z, F32(c))
    sr = np.where(x == 0, x, _fma32(sp * z, x, x))   # sin(±0) = ±0 exactly
    cp = np.full_like(x, F32(-1 / 3628800))
    for c in (1 / 40320, -1 / 720, 1 / 24, -0.5):
        cp = _fma32(cp, z, F32(c))
    cr = _fma32(cp, z, F32(1.0))
    return sr, cr


def _angles():
    rng = np.random.default_rng(7)
    parts = []
    # long-context shard: positions with per-batch offsets, base 5e5, 32 pairs
    p = rng.integers(7000, 71000, 4000)
    i = rng.integers(0, 32, 4000)
    parts.append(p * 500000.0 ** (-2.0 * i / 64))
    # MLA-style: positions 0..4095, base 1e4
    p = rng.integers(0, 4096, 4000)
    i = rng.integers(0, 32, 4000)
    parts.append(p * 10000.0 ** (-2.0 * i / 64))
    # tiny angles, angles near multiples of pi/2 in every quadrant, large angles up to 2^30
    parts.append(10.0 ** rng.uniform(-14, 0, 3000) * rng.choice([-1.0, 1.0], 3000))
    k = rng.integers(-200000, 200000, 3000)
    parts.append(k * P1 + 10.0 ** rng.uniform(-12, -2, 3000))
    parts.append(rng.uniform(-2.0 ** 30, 2.0 ** 30, 3000))
    return np.concatenate(parts + [np.array([0.0, -0.0, P1, -P1, 2 * P1, 2.0 ** 30])])


@pytest.fixture(scope="module")
def route():
    th = _angles()
    ks, rs, exact = [], [], []
    for t in th:
        k, r, e = _reduce(float(t))
        ks.append(k), rs.append(r), exact.append(e)
    k = np.array(ks)
    r = np.array(rs)
    sr, cr = _series(r)
    return th, k, r, exact, sr, cr


def test_reduction_is_within_3e16(route):
    th, k, r, exact, _, _ = route
    err = max(abs(Fraction(float(a)) - b) for a, b in zip(r, exact))
    assert float(err) <= 3e-16


def test_series_within_the_bounds_the_test_uses(route):
    th, k, r, exact, sr, cr = route
    s_true, c_true = np.sin(r), np.cos(r)           # double sin and cos of the reduced argument
    rel_s = np.abs(sr.astype(np.float64) - s_true) / np.maximum(np.abs(s_true), 1e-300)
    assert rel_s.max() <= 2.4 * 2.0 ** -24
    assert np.abs(cr.astype(np.float64) - c_true).max() <= 1.1e-7


@pytest.mark.parametrize("tt", ["bf16", "f16"])
def test_values_passing_the_test_round_as_the_double_values(route, tt):
    th, k, r, exact, sr, cr = route
    q = k.astype(np.int64) & 3
    sv = np.where(q & 1, cr, sr)
    cv = np.where(q & 1, sr, cr)
    sn = np.where(q & 2, -sv, sv)
    cn = np.where((q + 1) & 2, -cv, cv)
    es = np.abs(sr) * F32(2.0 ** -21 + 2.0 ** -23) + np.where(k != 0, F32(2.0 ** -50), F32(0.0))
    ec = np.abs(cr) * F32(2.0 ** -23) + F32(2.0 ** -21)
    e_sn = np.where(q & 1, ec, es)
    e_cn = np.where(q & 1, es, ec)

    def rnd(v):   # fp32 values rounded once to tt (the value, as fp32)
        return oracle.round_double(np.asarray(v, np.float32).astype(np.float64), tt)

    for v, e, ref in ((cn, e_cn, np.cos(th)), (sn, e_sn, np.sin(th))):
        lo = (v - e).astype(F32)
        hi = (v + e).astype(F32)
        rv = rnd(v)
        ok = (rnd(lo).view(np.uint32) == rv.view(np.uint32)) & (rnd(hi).view(np.uint32) == rv.view(np.uint32))
        want = oracle.round_double(ref, tt)
        bad = ok & (rv.view(np.uint32) != want.view(np.uint32))
        assert not bad.any(), (th[bad][:5], v[bad][:5], want[bad][:5])
        # the route is taken for most values of the workloads' kinds (the
        # first 8000 angles); the edge sets are there for soundness
        assert ok[:8000].mean() > (0.995 if tt == "bf16" else 0.98)
