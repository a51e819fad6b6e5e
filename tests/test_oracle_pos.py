"""Pins of the oracle's cos/sin tables from positions (rope_oracle_pos_tables)
and of its one-step rounding from double to a table type. The table recipe is
that of "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 第一步 (θ = p /
base^(2i/h) per position p and pair i, each value written to both lanes of
its pair), with the per-pair frequencies given; rotate_half repeats pair i at
lanes i and i + L/2 (section 先搞懂RoPE)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# ---------------------------------------------------------------- one-step rounding


def _all_finite_values(dtype):
    """(values, patterns): every finite non-negative value of the 16-bit type,
    ascending, as float64, with its bit pattern; then +inf."""
    pats = np.arange(0, 0x8000, dtype=np.uint16)
    if dtype == "f16":
        vals = pats.view(np.float16).astype(np.float64)
    else:
        vals = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    keep = np.isfinite(vals)
    return vals[keep], pats[keep]


_TABLES = {}


def nearest_even(x: float, dtype: str) -> float:
    """The value of the 16-bit type nearest to x, ties to the even bit
    pattern; past the largest finite value by half a unit or more, infinity.
    Found among all values of the type, distances compared exactly."""
    if dtype not in _TABLES:
        _TABLES[dtype] = _all_finite_values(dtype)
    vals, pats = _TABLES[dtype]
    if x != x:
        return x
    if x < 0:
        return -nearest_even(-x, dtype)
    top = vals[-1]
    emax = math.frexp(top)[1] - 1
    p = 11 if dtype == "f16" else 8
    beyond = Fraction(2) ** (emax + 1)                 # where infinity sits in the rounding
    i = int(np.searchsorted(vals, x))
    if i < len(vals) and vals[i] == x:
        return x
    lo, lo_pat = (vals[i - 1], int(pats[i - 1]))
    if i < len(vals):
        hi, hi_pat = Fraction(vals[i]), int(pats[i])
    else:
        hi, hi_pat = beyond, 0x7f80 if dtype == "bf16" else 0x7c00   # infinity's pattern is even
    fx = Fraction(x)
    dlo, dhi = fx - Fraction(lo), hi - fx
    if dlo < dhi or (dlo == dhi and lo_pat % 2 == 0):
        return float(lo)
    return math.inf if hi == beyond else float(hi)


def _doubles(rng, n):
    """Random doubles across the 16-bit types' ranges, plus ties and
    near-ties of both types (midpoints, and a hair either side)."""
    mags = np.exp2(rng.uniform(-30, 18, n))
    v = mags * rng.choice([-1.0, 1.0], n)
    extra = []
    for dtype in ("f16", "bf16"):
        vals, _ = _all_finite_values(dtype)
        pick = rng.choice(len(vals) - 1, 300)
        mids = (vals[pick] + vals[pick + 1]) / 2      # exact in double
        for m in mids:
            extra += [m, np.nextafter(m, 0), np.nextafter(m, np.inf), -m]
    return np.concatenate([v, np.array(extra), [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-45, 3.4e38, 3.4e39]])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_round_double_is_nearest_even(dtype):
    rng = np.random.default_rng(7)
    v = _doubles(rng, 4000)
    got = oracle.round_double(v, dtype).astype(np.float64)
    with np.errstate(over="ignore"):
        want = np.array([nearest_even(float(t), dtype) for t in v])
    bad = [(t, g, w) for t, g, w in zip(v, got, want) if not (g == w and math.copysign(1, g) == math.copysign(1, w))]
    assert not bad, bad[:5]


def test_round_double_f16_matches_numpy_on_many_values():
    """numpy converts float64 to float16 in one rounding (pinned above on
    ties): a larger random sweep against it."""
    rng = np.random.default_rng(8)
    v = np.exp2(rng.uniform(-26, 17, 400000)) * rng.choice([-1.0, 1.0], 400000)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.round_double(v, "f16").astype(np.float64), want)


def test_round_double_f32_is_the_float_cast():
    rng = np.random.default_rng(9)
    v = np.exp2(rng.uniform(-140, 120, 200000)) * rng.choice([-1.0, 1.0], 200000)
    assert np.array_equal(oracle.round_double(v, "f32"), v.astype(np.float32))


def test_round_double_differs_from_rounding_through_fp32():
    """The case that separates one rounding from two: 1 + 2^-8 + 2^-30 is
    above the bf16 midpoint 1 + 2^-8, but rounds to it in fp32 first."""
    x = 1 + 2 ** -8 + 2 ** -30
    assert oracle.round_double(np.array([x]), "bf16")[0] == 1 + 2 ** -7
    assert torch.tensor([x], dtype=torch.float64).float().to(torch.bfloat16).item() == 1.0


# ---------------------------------------------------------------- tables from positions

def _storage_to_f64(a, dtype):
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()


def _freqs(L, base):
    return base ** (-2.0 * np.arange(L // 2) / L)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_pos_tables_match_libm_cos_sin(dtype, mode):
    """Small tables against math.cos / math.sin of the double product p*f,
    rounded by the definition above (f32: the float cast)."""
    L = 16
    pos = np.array([[0, 1, 7, 4095], [65535, 70000, 123, 9]], dtype=np.int64)
    f = _freqs(L, 500000.0)
    c, s = oracle.pos_tables(pos, f, L, mode, dtype)
    cv, sv = _storage_to_f64(c, dtype), _storage_to_f64(s, dtype)
    for b in range(2):
        for t in range(4):
            for i in range(L // 2):
                th = float(pos[b, t]) * float(f[i])
                if dtype == "f32":
                    wc, ws = float(np.float32(math.cos(th))), float(np.float32(math.sin(th)))
                else:
                    wc, ws = nearest_even(math.cos(th), dtype), nearest_even(math.sin(th), dtype)
                lanes = (2 * i, 2 * i + 1) if mode == "interleave" else (i, i + L // 2)
                for j in lanes:
                    assert cv[b, t, 0, j] == wc and sv[b, t, 0, j] == ws, (b, t, i, j)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pos_tables_at_scale_against_numpy(dtype):
    """A long-context-like table (offsets up to 65535 + 4096 positions)
    against numpy's cos/sin and one-step rounding: 16-bit values agree bit
    for bit (an ulp of difference between two double cos/sin implementations
    changes a 16-bit rounding only for a value within a double ulp of a
    midpoint, a chance of about 2^-40 per value)."""
    rng = np.random.default_rng(3)
    L = 64
    pos = (rng.integers(0, 65536, size=(4, 1)) + np.arange(4096)[None, :]).astype(np.int64)
    f = _freqs(L, 500000.0)
    c, s = oracle.pos_tables(pos, f, L, "interleave", dtype)
    th = pos.astype(np.float64)[:, :, None] * f[None, None, :]
    wc = oracle.round_double(np.cos(th), dtype).astype(np.float64)
    ws = oracle.round_double(np.sin(th), dtype).astype(np.float64)
    assert np.array_equal(_storage_to_f64(c, dtype)[:, :, 0, 0::2], wc)
    assert np.array_equal(_storage_to_f64(s, dtype)[:, :, 0, 1::2], ws)


@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_pos_tables_position_zero_and_layout(mode):
    L = 12
    pos = np.zeros((1, 3), np.int64)
    pos[0, 1], pos[0, 2] = 5, 1000
    c, s = oracle.pos_tables(pos, _freqs(L, 10000.0), L, mode, "f32")
    assert np.all(c[0, 0] == 1.0) and np.all(s[0, 0] == 0.0)
    for t in (1, 2):
        if mode == "interleave":
            assert np.array_equal(c[0, t, 0, 0::2], c[0, t, 0, 1::2])
            assert np.array_equal(s[0, t, 0, 0::2], s[0, t, 0, 1::2])
        else:
            assert np.array_equal(c[0, t, 0, :L // 2], c[0, t, 0, L // 2:])
            assert np.array_equal(s[0, t, 0, :L // 2], s[0, t, 0, L // 2:])


def test_pos_tables_read_strided_positions():
    """A non-contiguous position view gives the tables of its contiguous copy."""
    base = np.arange(40, dtype=np.int64).reshape(4, 10) * 37
    view = base[::2, ::3]
    assert not view.flags.c_contiguous
    f = _freqs(8, 10000.0)
    a = oracle.pos_tables(view, f, 8, "rotate_half", "bf16")
    b = oracle.pos_tables(np.ascontiguousarray(view), f, 8, "rotate_half", "bf16")
    assert a[0].tobytes() == b[0].tobytes() and a[1].tobytes() == b[1].tobytes()


def test_pos_tables_reject_undefined_arguments():
    pos = np.zeros((1, 2), np.int64)
    with pytest.raises(ValueError):
        oracle.pos_tables(pos, np.ones(3), 6, "sideways", "f32")
    with pytest.raises(ValueError):
        oracle.pos_tables(pos, np.ones(2), 6, "interleave", "f32")     # L/2 = 3 frequencies needed
    with pytest.raises(TypeError):
        oracle.pos_tables(pos.astype(np.int32), np.ones(3), 6, "interleave", "f32")
