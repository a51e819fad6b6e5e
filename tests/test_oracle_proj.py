"""Pins of oracle.proj_rope, the projection followed by the rotation of each
head's slice ("ascend-transformer-boost 的 MlaPreprocessOperation：MLA 预处理
四阶段融合算子深度解析", section 3: the WUQ matmul, then RoPE on
Q[..., :qRopeDim] with cos/sin [tokenNum, 64] given from outside; section 2:
qRopeDim and the rotary coefficient).

Each pin states the operation another way: hand-derived cases that tell the
rounding order apart (tests/golden/proj/), the projection as exact integer
dot products, the rotation of each head as a dense matrix on that head's
fp32 projection, identity tables, and broadcast against expanded tables.
"""
import glob
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle_refs import round_to, widen

GOLDEN = sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "proj", "*.txt")))


def _load(path):
    case = {}
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        vals = rest.split()
        if key in ("dtype", "mode"):
            case[key] = vals[0]
        elif key in ("slice", "shape"):
            case[key] = tuple(int(v) for v in vals)
        else:
            case[key] = np.array([float(v) for v in vals], np.float64)
    return case


def _bits(a, dt):
    return round_to(np.asarray(a, np.float64), dt)


@pytest.mark.parametrize("path", GOLDEN, ids=[os.path.basename(p) for p in GOLDEN])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_golden_projection_then_rotation(path, out):
    c = _load(path)
    dt = c["dtype"]
    B, S, H, Dh = c["shape"]
    M, N = B * S, H * Dh
    K = c["x"].size // M
    x = _bits(c["x"], dt).reshape(M, K)
    w = _bits(c["w"], dt).reshape(N, K)
    assert np.array_equal(widen(x, dt).ravel(), c["x"]) and np.array_equal(widen(w, dt).ravel(), c["w"])
    L = c["slice"][1] - c["slice"][0]
    r1 = _bits(c["cos"], dt).reshape(1, 1, 1, L)
    r2 = _bits(c["sin"], dt).reshape(1, 1, 1, L)
    y = oracle.proj_rope(x, w, c["shape"], dt, r1, r2, c["mode"], c["slice"], out)
    assert widen(y, out).ravel().tolist() == c[f"expect_{out}"].tolist()


def test_golden_fixtures_present():
    assert len(GOLDEN) >= 2


def _rand_bits(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return round_to((torch.randn(shape, generator=g, dtype=torch.float64) * scale).numpy(), dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_projection_is_the_integer_dot_product(dt):
    """Small integers (exact in both 16-bit types): every output lane is the
    exact dot product of a token's inputs with that output lane's weight row
    (w is output lanes by inputs), checked with Python integers; non-square
    shapes so that a transposed operand cannot line up."""
    rng = np.random.default_rng(3)
    B, S, H, Dh, K = 2, 3, 3, 8, 20
    xi = rng.integers(-8, 9, size=(B * S, K))
    wi = rng.integers(-8, 9, size=(H * Dh, K))
    x, w = _bits(xi, dt), _bits(wi, dt)
    t = np.zeros((1, 1, 1, 0), np.uint16)
    y = oracle.proj_rope(x, w, (B, S, H, Dh), dt, t, t, "interleave", None, "f32")
    for m in range(B * S):
        b, s = divmod(m, S)
        for n in range(H * Dh):
            h, j = divmod(n, Dh)
            want = sum(int(xi[m, k]) * int(wi[n, k]) for k in range(K))
            assert y[b, s, h, j] == want
    # the 16-bit output is the library's rounding of those values
    y16 = oracle.proj_rope(x, w, (B, S, H, Dh), dt, t, t, "interleave", None, dt)
    ref = torch.from_numpy(y.astype(np.float32)).to({"bf16": torch.bfloat16, "f16": torch.float16}[dt])
    assert np.array_equal(y16, ref.view(torch.int16).numpy().view(np.uint16))


def _pair(L, mode):
    j = np.arange(L)
    if mode == "interleave":
        return j ^ 1, j % 2 == 0
    H = L // 2 if mode == "rotate_half" else L // int(mode)
    first = (j // H) % 2 == 0
    return np.where(first, j + H, j - H), first


@pytest.mark.parametrize("mode", ["interleave", "rotate_half", 4])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_each_head_is_a_dense_rotation_of_its_fp32_projection(mode, dt):
    """For every token and head: y[head] = fl32(J · p[head]) on the slice,
    with p the head's projection (exact products summed as fractions,
    rounded once to fp32) and J = diag(c) + diag(s)·P, P holding -1/+1 at
    (j, partner of j); lanes outside the slice are p itself. Random
    per-token tables (one row per (b,s), broadcast over heads)."""
    B, S, H, Dh, K, sl = 2, 3, 3, 12, 16, (2, 10)
    L = sl[1] - sl[0]
    x = _rand_bits((B * S, K), dt, 1)
    w = _rand_bits((H * Dh, K), dt, 2)
    r1 = _rand_bits((B, S, 1, L), dt, 3)
    r2 = _rand_bits((B, S, 1, L), dt, 4)
    y = oracle.proj_rope(x, w, (B, S, H, Dh), dt, r1, r2, mode, sl, "f32")
    xv, wv = widen(x, dt), widen(w, dt)
    cv, sv = widen(r1, dt), widen(r2, dt)
    partner, first = _pair(L, mode)
    for m in range(B * S):
        b, s = divmod(m, S)
        for h in range(H):
            p = np.array([float(np.float32(float(sum(Fraction(float(xv[m, k])) * Fraction(float(wv[h * Dh + j, k]))
                                                        for k in range(K)))))
                          for j in range(Dh)])
            J = np.diag(cv[b, s, 0].astype(np.float64))
            for j in range(L):
                J[j, partner[j]] += (-1.0 if first[j] else 1.0) * float(sv[b, s, 0, j])
            want = p.copy()
            want[sl[0]:sl[1]] = (J @ p[sl[0]:sl[1]]).astype(np.float32)
            assert np.array_equal(y[b, s, h], want.astype(np.float32)), (m, h)


def test_identity_tables_give_the_rounded_projection():
    """cos = 1, sin = 0 (position 0): the slice is the projection itself, and
    the 16-bit output is its rounding (torch's cast)."""
    B, S, H, Dh, K, sl = 1, 4, 2, 64, 32, (0, 64)
    x = _rand_bits((B * S, K), "bf16", 5)
    w = _rand_bits((H * Dh, K), "bf16", 6)
    one = _bits(np.ones((1, 1, 1, 64)), "bf16")
    zero = _bits(np.zeros((1, 1, 1, 64)), "bf16")
    y = oracle.proj_rope(x, w, (B, S, H, Dh), "bf16", one, zero, "rotate_half", sl, "bf16")
    p = (widen(x, "bf16") @ widen(w, "bf16").T).astype(np.float32)
    ref = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y.reshape(B * S, H * Dh), ref)


def test_broadcast_tables_equal_expanded_tables():
    """Tables (1, S, 1, L) broadcast over batch and heads give what the same
    values expanded to (B, S, H, L) give."""
    B, S, H, Dh, K, sl = 3, 2, 4, 16, 8, (4, 12)
    x = _rand_bits((B * S, K), "bf16", 7)
    w = _rand_bits((H * Dh, K), "bf16", 8)
    r1 = _rand_bits((1, S, 1, 8), "bf16", 9)
    r2 = _rand_bits((1, S, 1, 8), "bf16", 10)
    y = oracle.proj_rope(x, w, (B, S, H, Dh), "bf16", r1, r2, "interleave", sl, "bf16")
    e1 = np.ascontiguousarray(np.broadcast_to(r1, (B, S, H, 8)))
    e2 = np.ascontiguousarray(np.broadcast_to(r2, (B, S, H, 8)))
    y2 = oracle.proj_rope(x, w, (B, S, H, Dh), "bf16", e1, e2, "interleave", sl, "bf16")
    assert np.array_equal(y, y2)


def test_rejects_mismatched_operands():
    x = _rand_bits((6, 8), "bf16", 1)
    w = _rand_bits((8, 6), "bf16", 2)   # (K, N) instead of (N, K)
    t = np.zeros((1, 1, 1, 0), np.uint16)
    with pytest.raises(ValueError):
        oracle.proj_rope(x, w, (2, 3, 1, 6), "bf16", t, t, "interleave", None, "bf16")
