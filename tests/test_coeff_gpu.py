"""Rotary coefficients (mode value c >= 2: the slice in c parts of L/c lanes,
lane k of part 2g paired with lane k of part 2g+1; "ascend-transformer-boost
的 MlaPreprocessOperation", section 2, qRotaryCoeff / kRotaryCoeff) on the
GPU against the CPU oracle: the in-place, out-of-place, multi-tensor and
position entry points, on every kernel scheme a coefficient can take (own
vector with lane exchange, pair owner, own vector with the partner loaded,
row kernel). 16-bit results must match the oracle bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import TDT, announce, compare, expanded_tables, run_and_check, run_out_and_check

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _seed(*key):
    return zlib.crc32(repr(key).encode()) % 100000


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(DT[dtype])


def _pair_tables(B, S, L, coeff, dtype, seed, per_batch=False):
    """cos/sin of one angle per pair, pair i = g*H + k at lanes g*2H + k and
    g*2H + k + H; angles p * 1e4^(-2i/L) with p = offset + s."""
    g = torch.Generator().manual_seed(seed)
    Bt = B if per_batch else 1
    off = torch.randint(0, 60000, (Bt, 1), generator=g).double()
    pos = off + torch.arange(S, dtype=torch.float64)[None, :]
    th = pos[:, :, None] * 10000.0 ** (-2.0 * torch.arange(L // 2, dtype=torch.float64) / L)
    H = L // coeff
    first = torch.tensor([gg * 2 * H + k for gg in range(coeff // 2) for k in range(H)])
    lanes = torch.empty((Bt, S, L), dtype=torch.float64)
    cos, sin = lanes.clone(), lanes.clone()
    cos[..., first] = cos[..., first + H] = torch.cos(th)
    sin[..., first] = sin[..., first + H] = torch.sin(th)
    return cos.view(Bt, S, 1, L).to(DT[dtype]), sin.view(Bt, S, 1, L).to(DT[dtype])


def _plan_kernel(shape, dtype, r1, sl, coeff):
    x = torch.empty(shape, dtype=DT[dtype], device=DEV)
    r = r1.to(DEV)
    return rp.rope_partial_launch_info(x, r, r, coeff, sl)["kernel"]


# (shape, slice, coefficient, kernel for 16-bit x, kernel for fp32 x)
CASES = [
    ((2, 16, 8, 192), (0, 64), 4, "vector", "vector"),       # parts of 32 bytes: own vector, lane exchange
    ((2, 16, 8, 192), (0, 64), 8, "vector", "vector"),
    ((2, 16, 8, 128), (32, 96), 4, "vector", "vector"),      # half-line slice: whole-line coverage
    ((2, 8, 4, 1024), (0, 1024), 4, "vector", "vector"),     # rows wider than a wave: pair owner
    ((2, 8, 4, 1024), (0, 1024), 8, "vector", "vector"),
    ((3, 5, 7, 64), (0, 64), 16, "rows", "vector"),          # 16-bit parts of 8 bytes: the row kernel
    ((2, 6, 5, 96), (8, 56), 6, "vector", "vector"),         # six parts of 8 lanes
    ((2, 6, 5, 96), (2, 50), 4, "rows", "rows"),             # start off a vector boundary
]
IDS = [f"{c[0]}-{c[1]}-c{c[2]}" for c in CASES]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_coefficient_in_place(case, direction, dtype):
    shape, sl, coeff, k16, k32 = case
    L = sl[1] - sl[0]
    x = _rand(shape, dtype, _seed(case, dtype))
    r1, r2 = _pair_tables(shape[0], shape[1], L, coeff, dtype, _seed(case), per_batch=True)
    assert _plan_kernel(shape, dtype, r1, sl, coeff) == (k32 if dtype == "f32" else k16)
    info = run_and_check(x, r1, r2, coeff, sl, direction, f"c={coeff} {direction}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES[:4] + CASES[5:6], ids=IDS[:4] + IDS[5:6])
def test_coefficient_random_per_lane_tables(case, dtype):
    """Tables with no pair structure: the per-lane reading (sine at the
    lane itself forward, at the partner backward)."""
    shape, sl, coeff, _, _ = case
    L = sl[1] - sl[0]
    x = _rand(shape, dtype, _seed("r", case, dtype))
    r1 = _rand((1, shape[1], shape[2], L), dtype, _seed("r1", case))
    r2 = _rand((1, shape[1], shape[2], L), dtype, _seed("r2", case))
    for direction in ("fwd", "bwd"):
        info = run_and_check(x, r1, r2, coeff, sl, direction, f"c={coeff} random tables {direction}")
        if dtype != "f32":
            assert info["exact"] == info["n"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_coefficient_out_of_place(case, direction, dtype):
    """Out of place the threads cover whole rows: the lane exchange for rows
    of up to 64 vectors, the partner loaded from memory past that."""
    shape, sl, coeff, _, _ = case
    L = sl[1] - sl[0]
    x = _rand(shape, dtype, _seed("o", case, dtype))
    r1, r2 = _pair_tables(shape[0], shape[1], L, coeff, dtype, _seed("o", case))
    info = run_out_and_check(x, r1, r2, coeff, sl, direction, f"c={coeff} out of place {direction}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


def test_coefficient_two_and_L_equal_the_named_modes():
    shape, sl = (2, 32, 8, 128), (0, 128)
    x = _rand(shape, "bf16", 5).to(DEV)
    r1 = _rand((1, 32, 1, 128), "bf16", 6).to(DEV)
    r2 = _rand((1, 32, 1, 128), "bf16", 7).to(DEV)
    announce("coefficients 2 and L against the named modes")
    outs = {}
    for mode in ("rotate_half", 2, "interleave", 128):
        y = x.clone()
        rp.rope_partial_fwd_inplace(y, r1, r2, mode, sl)
        outs[mode] = y
    torch.cuda.synchronize()
    assert torch.equal(outs[2].view(torch.int16), outs["rotate_half"].view(torch.int16))
    assert torch.equal(outs[128].view(torch.int16), outs["interleave"].view(torch.int16))


def test_coefficient_multi_tensor():
    """Q (16 heads) and K (2 heads) with coefficient 4 in one call."""
    sl, coeff = (0, 64), 4
    q = _rand((2, 32, 16, 192), "bf16", 11)
    k = _rand((2, 32, 2, 192), "bf16", 12)
    r1, r2 = _pair_tables(2, 32, 64, coeff, "bf16", 13)
    announce("coefficient 4, multi-tensor")
    qd, kd = q.to(DEV), k.to(DEV)
    rp.rope_partial_fwd_inplace_multi([qd, kd], r1.to(DEV), r2.to(DEV), coeff, sl)
    torch.cuda.synchronize()
    for t, td in ((q, qd), (k, kd)):
        want = W.to_numpy_storage(t).copy()
        oracle.rope_rows(want, t.shape, "bf16", W.to_numpy_storage(r1), W.to_numpy_storage(r2), coeff, sl, "fwd")
        assert np.array_equal(W.to_numpy_storage(td.cpu()), want)


@pytest.mark.parametrize("dtype,tdtype", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[5], CASES[6]], ids=[IDS[0], IDS[3], IDS[5], IDS[6]])
def test_coefficient_positions(case, direction, dtype, tdtype):
    """The position entry points: pair i = g*H + k takes frequency i."""
    shape, sl, coeff, _, _ = case
    L = sl[1] - sl[0]
    x = _rand(shape, dtype, _seed("p", case, dtype))
    g = torch.Generator().manual_seed(_seed("pp", case))
    pos = torch.randint(0, 60000, (shape[0], 1), generator=g) + torch.arange(shape[1])[None, :]
    f = rp.rope_inv_freq(L, 500000.0)
    announce(f"positions c={coeff} shape={shape} {dtype} tables={tdtype} {direction}")
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), L, coeff, tdtype)
    xd = x.to(DEV)
    fn = rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos
    fn(xd, pos.to(DEV), f.to(DEV), coeff, sl, table_dtype=DT[tdtype])
    torch.cuda.synchronize()
    B, S, N, D = shape
    total = B * S * N
    rows = np.arange(total, dtype=np.int64)
    got = W.to_numpy_storage(xd.reshape(total, D).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x).reshape(total, D))
    want = x_rows.copy()
    oracle.rope_rows(want, shape, dtype, c, s, coeff, sl, direction, rows=rows, table_dtype=tdtype)
    r1, r2 = W.from_numpy_storage(c, tdtype), W.from_numpy_storage(s, tdtype)
    info = compare(got, want, x_rows, expanded_tables(r1, shape, rows, L), expanded_tables(r2, shape, rows, L),
                   dtype, coeff, direction, sl, f"positions c={coeff}")
    if dtype != "f32" and tdtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_coefficient_four_on_the_mla_shape(direction):
    """(4,4096,128,192) bf16, lanes [0,64) with coefficient 4 (MLA's rope
    part with the page's other coefficient); sampled rows."""
    w = W.WORKLOADS["c3_coeff4"]
    x = W.make_x(w)
    r1, r2 = W.make_tables(w)
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c3_coeff4 {direction}")
    assert info["rows"] == 4 * 4096 * 128
    assert info["exact"] == info["n"]
