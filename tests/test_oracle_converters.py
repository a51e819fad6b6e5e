"""Pins for the oracle's hand-written 16-bit float converters.

The oracle widens fp16/bf16 to fp32 and narrows its fp32 result with
round-to-nearest-even ("CANN ops-transformer 算子详解：inplace_partial_rotary_mul
原地部分旋转位置编码", mixed-precision paragraph of the tiling/kernel section:
results are written back with CAST_RINT). Its converters are checked here
against numpy's float16 and torch's bfloat16 casts, which are both RNE:
exhaustively in the widening direction, and on random patterns plus every tie
and boundary in the narrowing direction.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _same_f32(a: np.ndarray, b: np.ndarray) -> None:
    """Bit-identical, except that any NaN matches any NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))


def _same_u16(a: np.ndarray, b: np.ndarray, as_float) -> None:
    fa, fb = as_float(a), as_float(b)
    nan = np.isnan(fa)
    assert np.array_equal(nan, np.isnan(fb))
    bad = np.nonzero(a[~nan] != b[~nan])[0]
    assert bad.size == 0, f"{bad.size} mismatches, first input index {bad[:5]}"


ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _np_f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def _torch_bf16(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).copy()).view(torch.bfloat16).float().numpy()


def test_f16_to_f32_exhaustive():
    _same_f32(oracle.f16_bits_to_f32(ALL16), _np_f16(ALL16))


def test_bf16_to_f32_exhaustive():
    _same_f32(oracle.bf16_bits_to_f32(ALL16), _torch_bf16(ALL16))


RANDOM_CHUNK, RANDOM_CHUNKS = 1 << 22, 16   # 2^26 random fp32 patterns per narrowing direction


def _f32_cases(rng, n_random: int) -> np.ndarray:
    rnd = rng.integers(0, 2**32, size=n_random, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return rnd


def _ties_and_neighbours(grid_f32: np.ndarray) -> np.ndarray:
    """Midpoints between consecutive finite grid values, and the fp32 values
    one ulp either side of each midpoint and of each grid value."""
    g = np.sort(grid_f32[np.isfinite(grid_f32)].astype(np.float64))
    g = np.unique(g)
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)   # exact: one more bit than the grid
    pts = np.concatenate([mids, g.astype(np.float32)])
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    return np.concatenate([pts, up, dn]).astype(np.float32)


def test_f32_to_f16_random_and_ties():
    rng = np.random.default_rng(1234)
    grid = _np_f16(ALL16)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0,
                        65536.0, 1e9, -1e9, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-26,
                        2.0**-14, 2.0**-14 - 2.0**-25, 1e-30, -1e-30, 1.0e-45], np.float32)
    with np.errstate(over="ignore"):   # overflow to inf is part of what is checked
        for part in [np.concatenate([_ties_and_neighbours(grid), special])] + \
                [_f32_cases(rng, RANDOM_CHUNK) for _ in range(RANDOM_CHUNKS)]:
            _same_u16(oracle.f32_to_f16_bits(part), part.astype(np.float16).view(np.uint16), _np_f16)


def test_f32_to_bf16_random_and_ties():
    rng = np.random.default_rng(4321)
    grid = _torch_bf16(ALL16)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.3895314e38, 3.4028235e38,
                        1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1e-40, -1e-40, 1.0e-45], np.float32)
    for part in [np.concatenate([_ties_and_neighbours(grid), special])] + \
            [_f32_cases(rng, RANDOM_CHUNK) for _ in range(RANDOM_CHUNKS)]:
        want = torch.from_numpy(part).to(torch.bfloat16).view(torch.uint16).numpy()
        _same_u16(oracle.f32_to_bf16_bits(part), want, _torch_bf16)


def test_round_trip_16_bit_patterns():
    """Widening then narrowing returns every finite pattern unchanged."""
    for widen, narrow, as_float in (
        (oracle.f16_bits_to_f32, oracle.f32_to_f16_bits, _np_f16),
        (oracle.bf16_bits_to_f32, oracle.f32_to_bf16_bits, _torch_bf16),
    ):
        back = narrow(widen(ALL16))
        fin = ~np.isnan(as_float(ALL16))
        assert np.array_equal(back[fin], ALL16[fin])
        assert np.all(np.isnan(as_float(back[~fin])))


def test_f16_subnormals_kept():
    """Subnormal fp16 results are produced, not flushed to zero."""
    vals = np.array([2.0**-24, 5 * 2.0**-24, 2.0**-15, -(2.0**-20)], np.float32)
    bits = oracle.f32_to_f16_bits(vals)
    assert list(bits) == [0x0001, 0x0005, 0x0200, 0x8010]
