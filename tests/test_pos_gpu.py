"""The position entry points (rope_partial_{fwd,bwd}_inplace_pos) against the
CPU oracle: the oracle builds the cos/sin tables from the same positions and
frequencies (rope_oracle_pos_tables: double angle, double cos/sin, one
rounding to the table type; "ANE实战RoPE位置编码在MIL中的纯ANE实现", section
第一步) and rotates with them; the GPU computes them in the kernel. Bit-exact
for 16-bit data with 16-bit tables; with fp32 tables, 16-bit data is held to
1 ulp (a last-bit difference between two double cos/sin implementations
moves an fp32 table value by one unit in about 2^-27 of the values, a
16-bit one in about 2^-40)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, compare, compare_all_rows, expanded_tables, oracle_all_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TDT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(DT[dtype])


def _positions(B, S, per_batch, seed, top=70000):
    g = torch.Generator().manual_seed(seed)
    Bp = B if per_batch else 1
    off = torch.randint(0, top, (Bp, 1), generator=g, dtype=torch.int64)
    return off + torch.arange(S, dtype=torch.int64)[None, :]


def run_pos_and_check(x, positions, inv_freq, mode, sl, direction, tdtype, what, sample=None, seed=0,
                      pos_dev=None, x_offset=0):
    """positions / inv_freq are CPU tensors; pos_dev optionally a device view
    with other strides (same values). Returns the comparison summary."""
    dtype = TDT[x.dtype]
    announce(f"{what} shape={tuple(x.shape)} {dtype} tables={tdtype} {mode} {direction} slice={sl}")
    L = sl[1] - sl[0]
    c, s = oracle.pos_tables(positions.numpy(), inv_freq.numpy(), L, mode, tdtype)
    r1, r2 = W.from_numpy_storage(c, tdtype), W.from_numpy_storage(s, tdtype)
    n = x.numel()
    buf = torch.zeros(n + x_offset, dtype=x.dtype, device=DEV)
    xd = buf[x_offset:].view(x.shape)
    xd.copy_(x.to(DEV))
    pd = positions.to(DEV) if pos_dev is None else pos_dev
    fn = rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos
    fn(xd, pd, inv_freq.to(DEV), mode, sl, table_dtype=DT[tdtype])
    torch.cuda.synchronize()
    B, S, N, D = x.shape
    total = B * S * N
    if sample is None:
        # every row; the oracle split over the host's cores
        got = W.to_numpy_storage(xd.cpu()).reshape(total, D)
        x_flat = W.to_numpy_storage(x).reshape(total, D)
        want = oracle_all_rows(x_flat, tuple(x.shape), dtype, r1, r2, mode, sl, direction)
        info = compare_all_rows(got, want, x_flat, r1, r2, tuple(x.shape), dtype, mode, direction, sl, what)
    else:
        rows = W.sample_rows(total, sample, seed)
        got = W.to_numpy_storage(xd.reshape(total, D)[torch.from_numpy(rows).to(DEV)].cpu())
        x_rows = np.ascontiguousarray(W.to_numpy_storage(x).reshape(total, D)[rows])
        want = x_rows.copy()
        oracle.rope_rows(want, x.shape, dtype, c, s, mode, sl, direction, rows=rows, table_dtype=tdtype)
        info = compare(got, want, x_rows, expanded_tables(r1, x.shape, rows, L),
                       expanded_tables(r2, x.shape, rows, L), dtype, mode, direction, sl, what)
    if dtype != "f32" and tdtype != "f32":
        assert info["exact"] == info["n"], f"{what}: {info['n'] - info['exact']} lanes differ from the oracle"
    return info, xd


CASES = [
    # (shape, slice, mode, positions per batch, kernel for 16-bit x, kernel for fp32 x)
    ((2, 16, 8, 128), (32, 96), "interleave", True, "vector", "vector"),     # half-line slice: whole lines
    ((2, 16, 8, 128), (0, 128), "rotate_half", False, "vector", "vector"),   # whole head, one row of positions
    ((3, 9, 13, 64), (0, 64), "interleave", True, "vector", "vector"),       # ragged heads (13 in chunks)
    ((1, 8, 40, 192), (0, 64), "interleave", False, "vector", "vector"),     # MLA-style slice
    ((2, 5, 3, 1024), (0, 1024), "rotate_half", True, "vector", "vector"),   # 512 pairs: the largest table
    ((2, 6, 5, 64), (3, 35), "interleave", True, "rows", "rows"),            # odd start
    ((2, 5, 3, 48), (4, 44), "rotate_half", False, "rows", "vector"),        # halves of 20 lanes
    ((2, 7, 1, 128), (0, 128), "rotate_half", True, "vector", "vector"),     # one head: 8 positions per block
    ((3, 5, 2, 64), (0, 64), "interleave", False, "vector", "vector"),       # two heads: the last block part-full
]


@pytest.mark.parametrize("dtype,tdtype", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("bf16", "f32"),
                                          ("f32", "bf16"), ("f16", "bf16")])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{'B' if c[3] else '1'}" for c in CASES])
def test_pos_against_oracle(case, direction, dtype, tdtype):
    shape, sl, mode, per_batch, k16, k32 = case
    seed = zlib.crc32(repr(("pos", case[:4], dtype, tdtype)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    pos = _positions(shape[0], shape[1], per_batch, seed + 1)
    # the kernel the case is meant to reach (plan of a 256-byte aligned x, as torch allocates)
    st, plan = rp.raw_launch_info_pos(1 << 20, shape, rp.DTYPE_CODES[dtype], 1 << 20, tuple(pos.shape),
                                      tuple(pos.stride()), 1 << 20, rp.DTYPE_CODES[tdtype], rp.MODES[mode], sl)
    assert st == rp.ROPE_OK and plan["kernel"] == (k32 if dtype == "f32" else k16), plan
    f = rp.rope_inv_freq(sl[1] - sl[0], 500000.0)
    run_pos_and_check(x, pos, f, mode, sl, direction, tdtype, f"{shape} {sl} {mode}")


def test_pos_strided_positions_and_unaligned_x():
    """positions as a strided device view (a column of a wider int64 tensor),
    x 2 bytes past alignment (the row kernel), and positions expanded over
    the batch (stride 0)."""
    shape, sl, mode = (2, 12, 4, 64), (0, 64), "interleave"
    x = _rand(shape, "bf16", 51)
    pos = _positions(2, 12, True, 52)
    wide = torch.zeros((2, 12, 3), dtype=torch.int64)
    wide[:, :, 1] = pos
    pdev = wide.to(DEV)[:, :, 1]
    assert pdev.stride() == (36, 3)
    f = rp.rope_inv_freq(64, 10000.0)
    run_pos_and_check(x, pos, f, mode, sl, "fwd", "bf16", "strided positions", pos_dev=pdev)
    run_pos_and_check(x, pos, f, mode, sl, "bwd", "bf16", "unaligned x", x_offset=1)
    # one row of positions expanded over the batch: batch stride 0
    shared = torch.arange(12, dtype=torch.int64).add_(40000).expand(2, 12)
    assert shared.stride() == (0, 1)
    run_pos_and_check(x, shared, f, mode, sl, "fwd", "bf16", "expanded positions", pos_dev=shared.to(DEV).expand(2, 12))


@pytest.mark.parametrize("tdtype", ["bf16", "f32"])
@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_pos_long_context_shard(direction, tdtype):
    """The long-context shard's x with its per-batch positions (offset + s)
    and base 5e5, bf16 or fp32 cos/sin computed in the kernel (the bench's
    c4:pos and c4_t32:pos launches); every row against the oracle."""
    w = W.WORKLOADS["c4"]
    x = W.make_x(w)
    pos = torch.from_numpy(W.positions(w))
    f = rp.rope_inv_freq(w.L, w.base)
    info, _ = run_pos_and_check(x, pos, f, w.mode, w.partial_slice, direction, tdtype,
                                f"c4 positions {direction} {tdtype}")
    assert info["rows"] == 16 * 8192 * 32


def test_pos_multi_gqa_q_and_k_full_size():
    """c2's Q (32,256,16,128) and K (32,256,8,128), rotate_half, in one
    position call (the bench's c2:posmulti launch); every row of both
    against the oracle."""
    w = W.WORKLOADS["c2"]
    q, k = W.make_x(w, 0), W.make_x(w, 1)
    pos = torch.from_numpy(W.positions(w))
    f = rp.rope_inv_freq(w.L, w.base)
    announce("positions multi c2 Q+K full size")
    qd, kd = q.to(DEV), k.to(DEV)
    rp.rope_partial_fwd_inplace_pos_multi([qd, kd], pos.to(DEV), f.to(DEV), w.mode, w.partial_slice)
    torch.cuda.synchronize()
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), w.L, w.mode, "bf16")
    for t, td in ((q, qd), (k, kd)):
        want = W.to_numpy_storage(t).copy()
        oracle.rope_rows(want, t.shape, "bf16", c, s, w.mode, w.partial_slice, "fwd", table_dtype="bf16")
        assert np.array_equal(W.to_numpy_storage(td.cpu()), want)


def test_pos_multi_tensor_parallel_q_and_k_full_size():
    """One tensor-parallel rank's Q (32,4096,4,128) and K (32,4096,1,128),
    rotate_half, positions shared by the batch, in one position call (the
    bench's tp_qk:posmulti launch: the batches are heads of one position per
    s); every row of both against the oracle."""
    w = W.WORKLOADS["tp_qk"]
    q, k = W.make_x(w, 0), W.make_x(w, 1)
    pos = torch.from_numpy(W.positions(w))
    assert pos.shape == (1, 4096)
    f = rp.rope_inv_freq(w.L, w.base)
    announce("positions multi tp_qk Q+K full size")
    qd, kd = q.to(DEV), k.to(DEV)
    rp.rope_partial_fwd_inplace_pos_multi([qd, kd], pos.to(DEV), f.to(DEV), w.mode, w.partial_slice)
    torch.cuda.synchronize()
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), w.L, w.mode, "bf16")
    for t, td in ((q, qd), (k, kd)):
        want = W.to_numpy_storage(t).copy()
        oracle.rope_rows(want, t.shape, "bf16", c, s, w.mode, w.partial_slice, "fwd", table_dtype="bf16")
        assert np.array_equal(W.to_numpy_storage(td.cpu()), want)


def test_pos_equals_the_table_call_with_the_oracle_tables():
    """The position call and the table call given the oracle's tables of the
    same positions write the same bytes."""
    shape, sl, mode = (4, 32, 8, 128), (0, 128), "rotate_half"
    x = _rand(shape, "bf16", 61)
    pos = _positions(4, 32, True, 62)
    f = rp.rope_inv_freq(128, 10000.0)
    announce("positions vs tables")
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), 128, mode, "bf16")
    r1 = W.from_numpy_storage(c, "bf16").to(DEV)
    r2 = W.from_numpy_storage(s, "bf16").to(DEV)
    a, b = x.to(DEV), x.to(DEV)
    rp.rope_partial_fwd_inplace_pos(a, pos.to(DEV), f.to(DEV), mode, sl)
    rp.rope_partial_fwd_inplace(b, r1, r2, mode, sl)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_pos_noops_and_errors():
    x = _rand((2, 4, 3, 64), "bf16", 71).to(DEV)
    before = x.clone()
    pos = torch.zeros((1, 4), dtype=torch.int64, device=DEV)
    f = rp.rope_inv_freq(32).to(DEV)
    announce("positions no-ops and errors")
    rp.rope_partial_fwd_inplace_pos(x, pos, f, "interleave", (8, 8))
    rp.rope_partial_fwd_inplace_pos(x, pos, f, "interleave", None)
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_inplace_pos(x, torch.zeros((1, 5), dtype=torch.int64, device=DEV), f, "interleave",
                                        (0, 32))
    assert e.value.status == rp.ROPE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), before.view(torch.int16))
    # position 0 everywhere: cos 1, sin 0, so the slice comes back as it was
    rp.rope_partial_bwd_inplace_pos(x, pos, f, "interleave", (0, 32))
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), before.view(torch.int16))


def test_pos_scalar_kernel_past_two_to_the_31_rows():
    """(1, 2^31 + 96, 1, 2) bf16 with positions s mod 65536 + 7: from 2^31
    rows the 64-bit scalar kernel runs with its position form. Sampled rows
    against the oracle's tables of their own positions."""
    shape, sl, mode = (1, 2 ** 31 + 96, 1, 2), (0, 2), "interleave"
    total = shape[1]
    announce(f"position scalar kernel shape={shape} bf16 fwd slice={sl}")
    x = W.make_x_device(shape, "bf16", seed=95)
    pos = torch.arange(total, dtype=torch.int64, device=DEV).remainder_(65536).add_(7).view(1, total)
    f = rp.rope_inv_freq(2, 10000.0)
    st, plan = rp.raw_launch_info_pos(x.data_ptr(), shape, rp.DTYPE_CODES["bf16"], pos.data_ptr(), tuple(pos.shape),
                                      tuple(pos.stride()), 1 << 20, rp.DTYPE_CODES["bf16"], rp.MODES[mode], sl)
    assert st == rp.ROPE_OK and plan["kernel"] == "scalar", plan
    xv = x.view(total, 2)
    rows = W.sample_rows(total, 4000, seed=95)
    rows_t = torch.from_numpy(rows).to(DEV)
    x_rows = np.ascontiguousarray(W.to_numpy_storage(xv.index_select(0, rows_t).cpu()))
    rp.rope_partial_fwd_inplace_pos(x, pos, f.to(DEV), mode, sl)
    torch.cuda.synchronize()
    got = W.to_numpy_storage(xv.index_select(0, rows_t).cpu())
    p_rows = (rows % 65536 + 7).astype(np.int64).reshape(1, -1)
    c, s = oracle.pos_tables(p_rows, f.numpy(), 2, mode, "bf16")
    want = x_rows.copy()
    oracle.rope_rows(want, (1, len(rows), 1, 2), "bf16", c, s, mode, sl, "fwd")
    cv = W.from_numpy_storage(c, "bf16").double().numpy().reshape(-1, 2)
    sv = W.from_numpy_storage(s, "bf16").double().numpy().reshape(-1, 2)
    info = compare(got, want, x_rows, cv, sv, "bf16", mode, "fwd", sl, "position scalar kernel")
    assert info["exact"] == info["n"]
    del x, xv, pos
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tdtype", ["bf16", "f32"])
def test_pos_large_and_negative_positions(tdtype):
    """Positions far beyond any context length and negative ones (the angle
    reaches 10^12 rad, so both sides reduce it over many periods), against
    the oracle's tables of the same positions."""
    shape, sl, mode = (2, 64, 4, 128), (0, 128), "rotate_half"
    x = _rand(shape, "bf16", 81)
    g = torch.Generator().manual_seed(82)
    mag = torch.randint(0, 2 ** 40, (2, 64), generator=g, dtype=torch.int64)
    sign = torch.where(torch.rand((2, 64), generator=g) < 0.5, -1, 1)
    pos = mag * sign
    pos[0, :4] = torch.tensor([0, -1, 2 ** 40, -(2 ** 40)])
    f = rp.rope_inv_freq(128, 10000.0)
    run_pos_and_check(x, pos, f, mode, sl, "fwd", tdtype, "large and negative positions")


@pytest.mark.parametrize("tdtype", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["interleave", "rotate_half"])
def test_pos_fast_evaluation_edges(mode, tdtype):
    """For 16-bit tables the kernels evaluate cos and sin in fp32 and keep a
    value only when its rounding to the table type is proven (Ziv's test),
    else they take the double evaluation. The frequencies and positions here
    reach every branch: a zero frequency (angle 0: the sine's interval
    straddles zero), tiny angles where the sine's relative bound decides
    (frequencies down to 1e-12), angles near multiples of pi/2 (small
    reduced arguments in every quadrant), negative positions (angle -0 with
    the zero frequency), angles past 2^30 (batch 1 starts at position
    2^31), and a dense spread of frequencies that puts many
    values near rounding midpoints. Every lane must equal the rotation with
    the oracle's tables bit for bit."""
    shape, sl = (2, 256, 4, 128), (0, 128)
    x = _rand(shape, "bf16", 91)
    g = torch.Generator().manual_seed(92)
    f = torch.empty(64, dtype=torch.float64)
    f[:8] = torch.tensor([0.0, 1e-12, 1e-9, 1e-6, 1e-4, 1e-2, 1.0, 1.5707963267948966], dtype=torch.float64)
    f[8:16] = torch.tensor([0.5 * np.pi, np.pi, 2 * np.pi, 0.25 * np.pi, 1e-3, 3e-7, 0.1, 0.7], dtype=torch.float64)
    f[16:] = 10.0 ** (torch.rand(48, generator=g, dtype=torch.float64) * 6 - 5)
    pos = torch.arange(256, dtype=torch.int64)[None, :].repeat(2, 1)
    pos[0, 200:216] = -torch.arange(1, 17)          # with the zero frequency: angle -0
    pos[1] += 2 ** 31
    run_pos_and_check(x, pos, f, mode, sl, "fwd", tdtype, f"fast evaluation edges {mode} {tdtype}")


# ---------------------------------------------------------------- several tensors

MULTI_CASES = [
    # (shapes, slice, mode): one launch when B, S and D agree
    (((2, 32, 16, 128), (2, 32, 2, 128)), (0, 128), "rotate_half"),       # GQA Q and K
    (((2, 32, 16, 128), (2, 32, 4, 128)), (32, 96), "interleave"),        # half-line slice
    (((1, 24, 8, 192), (1, 24, 1, 192), (1, 24, 3, 192), (1, 24, 5, 192)), (0, 64), 4),   # four, coefficient 4
    (((2, 16, 6, 192), (2, 16, 2, 64)), (0, 64), "interleave"),           # D differs: one launch each
    (((2, 12, 5, 64), (2, 12, 3, 64)), (3, 35), "interleave"),            # odd start: the row kernel each
    (((4, 20, 4, 128), (4, 20, 1, 128)), (0, 128), "rotate_half"),        # few heads: with shared positions,
    (((3, 17, 2, 64), (3, 17, 1, 64), (3, 17, 3, 64)), (0, 64), "interleave"),   # the batches become heads
]


@pytest.mark.parametrize("per_batch", [True, False], ids=["positions-per-batch", "positions-shared"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", MULTI_CASES, ids=[f"{len(c[0])}x-{c[1]}-{c[2]}" for c in MULTI_CASES])
def test_pos_multi_equals_single_calls_and_the_oracle(case, direction, per_batch):
    shapes, sl, mode = case
    L = sl[1] - sl[0]
    B, S = shapes[0][0], shapes[0][1]
    xs = [_rand(sh, "bf16", 300 + i) for i, sh in enumerate(shapes)]
    pos = _positions(B, S, per_batch, 310)
    f = rp.rope_inv_freq(L, 500000.0)
    announce(f"positions multi {[tuple(s) for s in shapes]} {sl} {mode} {direction}")
    multi = [x.to(DEV) for x in xs]
    single = [x.to(DEV) for x in xs]
    (rp.rope_partial_fwd_inplace_pos_multi if direction == "fwd" else rp.rope_partial_bwd_inplace_pos_multi)(
        multi, pos.to(DEV), f.to(DEV), mode, sl)
    fn = rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos
    for t in single:
        fn(t, pos.to(DEV), f.to(DEV), mode, sl)
    torch.cuda.synchronize()
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), L, mode, "bf16")
    for x, m, one in zip(xs, multi, single):
        assert torch.equal(m.view(torch.int16), one.view(torch.int16))
        want = W.to_numpy_storage(x).copy()
        oracle.rope_rows(want, x.shape, "bf16", c, s, mode, sl, direction, table_dtype="bf16")
        assert np.array_equal(W.to_numpy_storage(m.cpu()), want)


def test_pos_multi_error_touches_nothing():
    q = _rand((1, 8, 4, 64), "bf16", 320).to(DEV)
    k = _rand((1, 9, 2, 64), "bf16", 321).to(DEV)          # S differs from the positions'
    q0 = q.clone()
    pos = torch.arange(8, dtype=torch.int64, device=DEV).view(1, 8)
    f = rp.rope_inv_freq(64).to(DEV)
    announce("positions multi: an error touches nothing")
    with pytest.raises(rp.RopeError, match="tensor 1"):
        rp.rope_partial_fwd_inplace_pos_multi([q, k], pos, f, "interleave", (0, 64))
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16))


@pytest.mark.parametrize("out", [False, True])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_pos_mqa_k_positions_shared_by_the_batch(direction, out):
    """A single K head (32,4096,1,128) bf16, rotate_half, with one row of
    positions for all 32 batches: the kernels take the batches as heads of
    one position per s (each s's cos and sin evaluated once). Sampled rows
    against the oracle; out of place, x unchanged."""
    w = W.WORKLOADS["mqa_k"]
    x = W.make_x(w)
    pos = torch.from_numpy(W.positions(w))
    assert pos.shape == (1, 4096)
    f = rp.rope_inv_freq(w.L, w.base)
    st, plan = rp.raw_launch_info_pos(1 << 20, w.x_shapes[0], rp.DTYPE_CODES["bf16"], 1 << 20, (1, 4096), (4096, 1),
                                      1 << 20, rp.DTYPE_CODES["bf16"], rp.MODES[w.mode], w.partial_slice)
    # the batches as heads: 32 per s, in four chunks of 8 head lanes x 1 head (64-thread blocks)
    assert st == rp.ROPE_OK and plan["head_lanes"] == 8 and plan["threads"] == 64 and plan["blocks"] == 16384
    announce(f"positions mqa_k shared {direction} out={out}")
    xd = x.to(DEV)
    if out:
        y = torch.empty_like(xd)
        (rp.rope_partial_fwd_out_pos if direction == "fwd" else rp.rope_partial_bwd_out_pos)(
            y, xd, pos.to(DEV), f.to(DEV), w.mode, w.partial_slice)
    else:
        y = xd
        (rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos)(
            y, pos.to(DEV), f.to(DEV), w.mode, w.partial_slice)
    torch.cuda.synchronize()
    if out:
        assert torch.equal(xd.view(torch.int16), x.to(DEV).view(torch.int16))
    B, S, N, D = w.x_shapes[0]
    total = B * S * N
    rows = W.sample_rows(total, 4000, 23)
    got = W.to_numpy_storage(y.view(total, D).index_select(0, torch.from_numpy(rows).to(DEV)).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x).reshape(total, D)[rows])
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), w.L, w.mode, "bf16")
    want = x_rows.copy()
    oracle.rope_rows(want, x.shape, "bf16", c, s, w.mode, w.partial_slice, direction, rows=rows, table_dtype="bf16")
    assert np.array_equal(got, want)
