"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Every test calls the C ABI through the binding on an MI355X. Small cases are
compared on every row; the full-size workloads are compared on sampled rows
that the oracle computes one by one, while the lanes outside the slice are
checked bit-for-bit on the device for every row.
"""
import zlib

import numpy as np
import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, compare, run_and_check, oracle_rows, widen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload_inputs(name, k=0):
    w = W.WORKLOADS[name]
    x = W.make_x(w, k)
    r1, r2 = W.make_tables(w)
    return w, x, r1, r2


# ---------------------------------------------------------------- the five configurations

@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_c0_fp32_interleave(direction):
    w, x, r1, r2 = _workload_inputs("c0")
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c0 {direction}")
    assert info["n"] == 16 * 2 * 32


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_c0_noops(direction):
    w, x, r1, r2 = _workload_inputs("c0")
    announce(f"c0 no-op {direction}")
    xd = x.to(DEV)
    before = xd.clone()
    fn = rp.rope_partial_fwd_inplace if direction == "fwd" else rp.rope_partial_bwd_inplace
    fn(xd, r1.to(DEV), r2.to(DEV), "interleave", (8, 8))          # empty slice
    fn(xd, r1.to(DEV), r2.to(DEV), "interleave", None)            # None = [0, 0)
    empty = torch.empty((0, 16, 2, 64), device=DEV)
    fn(empty, r1.to(DEV), r2.to(DEV), "interleave", (0, 32))      # B = 0
    torch.cuda.synchronize()
    assert torch.equal(xd.view(torch.int32), before.view(torch.int32))


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_c1_fp16_mha(direction):
    w, x, r1, r2 = _workload_inputs("c1")
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c1 {direction}")
    assert info["exact"] == info["n"], "16-bit results should match the oracle bit for bit"


def test_c2_bf16_gqa_q_then_k():
    """Q then K rotated with the same tables on one stream."""
    w = W.WORKLOADS["c2"]
    r1, r2 = W.make_tables(w)
    q, k = W.make_x(w, 0), W.make_x(w, 1)
    announce("c2 Q and K, one stream")
    qd, kd = q.to(DEV), k.to(DEV)
    r1d, r2d = r1.to(DEV), r2.to(DEV)
    rp.rope_partial_fwd_inplace(qd, r1d, r2d, "rotate_half", (0, 128))
    rp.rope_partial_fwd_inplace(kd, r1d, r2d, "rotate_half", (0, 128))
    torch.cuda.synchronize()
    for name, src, dev in (("Q", q, qd), ("K", k, kd)):
        B, S, N, D = src.shape
        rows = np.arange(B * S * N, dtype=np.int64)
        x_rows = W.to_numpy_storage(src).reshape(-1, D)
        want = oracle_rows(x_rows, src.shape, "bf16", r1, r2, "rotate_half", (0, 128), "fwd", None)
        got = W.to_numpy_storage(dev.cpu()).reshape(-1, D)
        from gpu_support import expanded_tables
        c = expanded_tables(r1, src.shape, rows, 128)
        s = expanded_tables(r2, src.shape, rows, 128)
        info = compare(got, want.reshape(-1, D), x_rows, c, s, "bf16", "rotate_half", "fwd", (0, 128), name)
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_c3_bf16_mla_full_size(direction):
    w, x, r1, r2 = _workload_inputs("c3")
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c3 {direction}")
    assert info["rows"] == 4 * 4096 * 128
    assert info["exact"] == info["n"]


@pytest.mark.parametrize("name", ["c4", "c4_f32"])
@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_c4_long_context_full_size(name, direction):
    w, x, r1, r2 = _workload_inputs(name)
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"{name} {direction}")
    assert info["rows"] == 16 * 8192 * 32
    if w.dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("name", ["c2_s4096", "rh_64of128", "rh_32of128"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_rotate_half_layouts_full_size(name, direction):
    """rotate_half from HBM: a whole head (pair-owner scheme) and two partial
    slices with 64- and 32-byte halves (own-vector scheme, lane exchange)."""
    w, x, r1, r2 = _workload_inputs(name)
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"{name} {direction}")
    assert info["exact"] == info["n"]


# ---------------------------------------------------------------- more shapes and layouts

@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_single_op_example_random_tables(direction):
    """(2,32,8,128) fp16, slice [0,64), random BS1D tables: the per-lane reading."""
    w, x, r1, r2 = _workload_inputs("p1ex")
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"p1ex {direction}")
    assert info["exact"] == info["n"]


DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(DT[dtype])


CASES = [
    # (shape, slice, mode, table shape)     -- what it exercises
    ((2, 8, 4, 64), (0, 64), "interleave", (1, 8, 1, 64)),        # vector path, full slice
    ((2, 8, 4, 192), (64, 192), "interleave", (2, 8, 1, 128)),    # slice at the row end
    ((3, 5, 13, 96), (16, 80), "interleave", (1, 5, 1, 64)),      # ragged head count
    ((1, 4, 37, 128), (8, 104), "interleave", (1, 4, 1, 96)),     # 12 vectors per row (bf16)
    ((1, 3, 300, 64), (0, 64), "interleave", (1, 3, 1, 64)),      # many heads per block
    ((2, 6, 5, 64), (3, 35), "interleave", (1, 6, 1, 32)),        # odd start: general (row) kernel
    ((2, 6, 5, 40), (2, 14), "interleave", (1, 6, 1, 12)),        # L not a vector multiple
    ((2, 8, 4, 128), (0, 128), "rotate_half", (1, 8, 1, 128)),    # vector path
    ((2, 8, 4, 256), (64, 192), "rotate_half", (2, 8, 1, 128)),
    ((2, 5, 3, 48), (4, 44), "rotate_half", (1, 5, 1, 40)),       # half of 20 lanes: general (row) kernel
    ((2, 8, 4, 64), (0, 64), "interleave", (2, 8, 4, 64)),        # BSND tables (per head)
    ((2, 8, 4, 64), (0, 64), "interleave", (2, 1, 4, 64)),        # B1ND
    ((2, 8, 4, 64), (0, 64), "interleave", (2, 1, 1, 64)),        # B11D
    ((2, 8, 4, 64), (0, 64), "interleave", (1, 1, 1, 64)),        # 111D
    ((2, 8, 4, 128), (0, 128), "rotate_half", (2, 8, 4, 128)),    # per-head tables, rotate_half
    ((2, 8, 4, 128), (64, 128), "rotate_half", (1, 8, 1, 64)),    # 16-bit: own-vector rotate_half, one line
    ((2, 8, 4, 128), (32, 96), "rotate_half", (2, 8, 4, 64)),     # own vector over two lines, per-head tables
    ((3, 5, 13, 128), (0, 32), "rotate_half", (1, 5, 1, 32)),     # NeoX-style rotary_dim 32: own vector, whole line
    ((1, 3, 5, 1024), (8, 1000), "rotate_half", (1, 3, 1, 992)),  # rows wider than a wave: pair owner
    ((1, 3, 5, 1024), (8, 520), "rotate_half", (1, 3, 1, 512)),   # bf16: own vector over the slice, not its lines
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}" for c in CASES])
def test_shapes_layouts_dtypes(case, direction, dtype):
    shape, sl, mode, tshape = case
    seed = zlib.crc32(repr((shape, sl, mode, tshape)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    r1 = _rand(tshape, dtype, seed + 1)
    r2 = _rand(tshape, dtype, seed + 2)
    info = run_and_check(x, r1, r2, mode, sl, direction, f"{shape} {sl} {mode} {tshape}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_expanded_table_views(dtype):
    """Tables passed as expand() views (zero strides) and as strided slices
    of a wider buffer give the oracle's result."""
    shape, sl = (2, 16, 6, 128), (32, 96)
    x = _rand(shape, dtype, 21)
    base1 = _rand((1, 16, 1, 64), dtype, 22)
    base2 = _rand((1, 16, 1, 64), dtype, 23)
    e1 = base1.to(DEV).expand(2, 16, 6, 64)
    e2 = base2.to(DEV).expand(2, 16, 6, 64)
    run_and_check(x, base1, base2, "interleave", sl, "fwd", "expand() tables", r1_dev=e1, r2_dev=e2)
    wide1 = _rand((1, 16, 1, 192), dtype, 24)
    wide2 = _rand((1, 16, 1, 192), dtype, 25)
    s1, s2 = wide1[..., 64:128], wide2[..., 64:128]
    run_and_check(x, s1.contiguous(), s2.contiguous(), "interleave", sl, "bwd", "strided tables",
                  r1_dev=wide1.to(DEV)[..., 64:128], r2_dev=wide2.to(DEV)[..., 64:128])


def test_unaligned_x_uses_general_path():
    """x starting 2 bytes past a 16-byte boundary (a view into a buffer)."""
    shape, sl = (2, 4, 3, 64), (0, 32)
    x = _rand(shape, "bf16", 31)
    r1, r2 = _rand((1, 4, 1, 32), "bf16", 32), _rand((1, 4, 1, 32), "bf16", 33)
    announce("unaligned x")
    buf = torch.zeros(x.numel() + 1, dtype=torch.bfloat16, device=DEV)
    xd = buf[1:].view(shape)
    xd.copy_(x.to(DEV))
    assert xd.data_ptr() % 16 != 0
    rp.rope_partial_fwd_inplace(xd, r1.to(DEV), r2.to(DEV), "interleave", sl)
    torch.cuda.synchronize()
    want = oracle_rows(W.to_numpy_storage(x).reshape(-1, 64).copy(), shape, "bf16", r1, r2, "interleave", sl,
                       "fwd", None)
    assert W.to_numpy_storage(xd.cpu()).reshape(-1, 64).tobytes() == want.tobytes()
    assert buf[0].item() == 0


# ---------------------------------------------------------------- properties of the launch

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_untouched(dtype):
    """4 KiB guard bands before and after x stay bit-identical."""
    shape, sl = (2, 16, 6, 128), (32, 96)
    x = _rand(shape, dtype, 41)
    r1, r2 = _rand((1, 16, 1, 64), dtype, 42), _rand((1, 16, 1, 64), dtype, 43)
    announce(f"guard bands {dtype}")
    esz = torch.tensor([], dtype=DT[dtype]).element_size()
    guard = 4096 // esz
    buf = _rand((guard + x.numel() + guard,), dtype, 44).to(DEV)
    ref = buf.clone()
    xd = buf[guard: guard + x.numel()].view(shape)
    xd.copy_(x.to(DEV))
    for fn in (rp.rope_partial_fwd_inplace, rp.rope_partial_bwd_inplace):
        fn(xd, r1.to(DEV), r2.to(DEV), "interleave", sl)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int32)) if dtype == "f32" else (lambda t: t.view(torch.int16))
    assert torch.equal(bits(buf[:guard]), bits(ref[:guard]))
    assert torch.equal(bits(buf[guard + x.numel():]), bits(ref[guard + x.numel():]))


def test_deterministic_repeats():
    w, x, r1, r2 = _workload_inputs("c1")
    announce("determinism c1")
    outs = []
    for _ in range(3):
        xd = x.to(DEV)
        rp.rope_partial_fwd_inplace(xd, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))
        rp.rope_partial_bwd_inplace(xd, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))
        outs.append(xd.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_runs_on_a_side_stream():
    w, x, r1, r2 = _workload_inputs("c1")
    announce("side stream c1")
    xd, r1d, r2d = x.to(DEV), r1.to(DEV), r2.to(DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        rp.rope_partial_fwd_inplace(xd, r1d, r2d, "interleave", (0, 64))
    side.synchronize()
    D = 64
    want = oracle_rows(W.to_numpy_storage(x).reshape(-1, D).copy(), x.shape, "f16", r1, r2, "interleave",
                       (0, 64), "fwd", None)
    assert W.to_numpy_storage(xd.cpu()).reshape(-1, D).tobytes() == want.tobytes()


def test_errors_raise_before_touching_memory():
    x = _rand((2, 4, 3, 64), "bf16", 51).to(DEV)
    before = x.clone()
    r = _rand((1, 4, 1, 32), "bf16", 52).to(DEV)
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_inplace(x, r, r, "interleave", (0, 30))        # table last dim != L
    assert e.value.status == rp.ROPE_ERR_INVALID
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_inplace(x, r, r.float(), "interleave", (0, 32))    # r1 and r2 dtypes differ
    assert e.value.status == rp.ROPE_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), before.view(torch.int16))


def test_golden_cases_on_gpu():
    from golden_cases import all_cases
    for case in all_cases():
        dt = case["dtype"]
        D = case["x"].size
        L = case["slice"][1] - case["slice"][0]
        announce(f"golden {case['name']}")
        tt = case["table_dtype"]
        x = torch.tensor(case["x"], dtype=torch.float64).to(DT[dt]).view(1, 1, 1, D).to(DEV)
        c = torch.tensor(case["cos"], dtype=torch.float64).to(DT[tt]).view(1, 1, 1, L).to(DEV)
        s = torch.tensor(case["sin"], dtype=torch.float64).to(DT[tt]).view(1, 1, 1, L).to(DEV)
        fn = rp.rope_partial_fwd_inplace if case["direction"] == "fwd" else rp.rope_partial_bwd_inplace
        fn(x, c, s, case["mode"], case["slice"])
        torch.cuda.synchronize()
        assert x.double().cpu().view(-1).tolist() == case["expect"].tolist(), case["name"]


# ---------------------------------------------------------------- table dtypes other than x's

MIXED = [("bf16", "f32"), ("f16", "f32"), ("f32", "bf16"), ("f32", "f16"), ("f16", "bf16"), ("bf16", "f16")]
MIXED_CASES = [
    ((2, 8, 4, 128), (32, 96), "interleave", (2, 8, 1, 64)),     # vector path (whole lines for f32 tables)
    ((2, 8, 4, 128), (0, 128), "rotate_half", (1, 8, 1, 128)),   # vector path, rotate_half
    ((2, 8, 4, 64), (0, 64), "interleave", (2, 8, 4, 64)),       # per-head tables
    ((2, 6, 5, 64), (3, 35), "interleave", (1, 6, 1, 32)),       # odd start: general (row) kernel
]


@pytest.mark.parametrize("dtype,tdtype", MIXED, ids=[f"{a}-x-{b}-tables" for a, b in MIXED])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", MIXED_CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}" for c in MIXED_CASES])
def test_mixed_table_dtypes(case, direction, dtype, tdtype):
    shape, sl, mode, tshape = case
    seed = zlib.crc32(repr((shape, sl, mode, tshape, dtype, tdtype)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    r1 = _rand(tshape, tdtype, seed + 1)
    r2 = _rand(tshape, tdtype, seed + 2)
    info = run_and_check(x, r1, r2, mode, sl, direction, f"{dtype} x {tdtype} tables {shape} {sl} {mode}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_c4_bf16_with_fp32_tables_full_size(direction):
    """The page's mixed case at the long-context shape: bf16 dx, fp32 tables."""
    from dataclasses import replace
    w = replace(W.WORKLOADS["c4"], table_dtype="f32")
    x = W.make_x(w)
    r1, r2 = W.make_tables(w)
    assert r1.dtype == torch.float32
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c4 fp32 tables {direction}")
    assert info["rows"] == 16 * 8192 * 32
    assert info["exact"] == info["n"]


@pytest.mark.parametrize("tdtype", ["bf16", "f16"])
@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_c4_fp32_with_16bit_tables_full_size(tdtype, direction):
    """fp32 dx with 16-bit tables at the long-context shape: 8-byte table
    units in the vector kernel; within the fp32 bound of the oracle."""
    from dataclasses import replace
    w = replace(W.WORKLOADS["c4_f32"], table_dtype=tdtype)
    x = W.make_x(w)
    r1, r2 = W.make_tables(w)
    assert r1.dtype == W.TORCH_DTYPES[tdtype]
    assert rp.rope_partial_launch_info(x, r1, r2, w.mode, w.partial_slice)["kernel"] == "vector"
    info = run_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"c4 fp32 {tdtype} tables {direction}")
    assert info["rows"] == 16 * 8192 * 32


# ---------------------------------------------------------------- the largest head dimension

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,sl", [("interleave", (0, 1024)), ("rotate_half", (0, 1024)),
                                     ("interleave", (8, 1016)), ("interleave", (1000, 1024)),
                                     ("interleave", (1, 1023)), ("rotate_half", (2, 1022))])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_head_dim_limit(dtype, mode, sl, direction):
    """D = 1024, the constraint's limit: a full-width fp32 interleave slice
    needs 256 threads per row (the kernel's block limit); the misaligned
    slices of more than 512 lanes take the row kernel, whose 256 threads per
    row then loop over the pairs."""
    shape = (2, 3, 5, 1024)
    L = sl[1] - sl[0]
    seed = zlib.crc32(repr((dtype, mode, sl, direction)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    r1 = _rand((1, 3, 1, L), dtype, seed + 1)
    r2 = _rand((1, 3, 1, L), dtype, seed + 2)
    info = run_and_check(x, r1, r2, mode, sl, direction, f"D=1024 {dtype} {mode} {sl}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


def test_d_over_limit_is_rejected():
    x = torch.zeros((1, 1, 1, 1026), dtype=torch.bfloat16, device=DEV)
    r = torch.zeros((1, 1, 1, 2), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_inplace(x, r, r, "interleave", (0, 2))
    assert e.value.status == rp.ROPE_ERR_INVALID


# ---------------------------------------------------------------- a grid at the dispatch limit

def _lane_checksums(xv, lo, hi, rows_per_chunk=1 << 24):
    """(sum, sum of squares) of the 16-bit patterns of lanes [lo, hi) of
    every row, computed on the device chunk by chunk."""
    s = s2 = 0
    for r0 in range(0, xv.shape[0], rows_per_chunk):
        part = xv[r0:r0 + rows_per_chunk, lo:hi].contiguous().view(torch.int16).to(torch.int64)
        s += int(part.sum())
        s2 += int((part * part).sum())
        del part
    return s, s2


def test_grid_capped_at_the_dispatch_limit():
    """(1, 40e6, 5, 128) bf16, lanes [32,96): 5 heads in chunks of 4 make
    80e6 tile groups of 64 threads, past the 32-bit grid size of a dispatch.
    The grid is cut to fit and its blocks stride over the remaining groups;
    sampled rows against the oracle (the first and last among them), the
    lanes outside the slice checked on the device for every row."""
    shape, sl, mode = (1, 40_000_000, 5, 128), (32, 96), "interleave"
    B, S, N, D = shape
    total = B * S * N
    announce(f"grid cap shape={shape} bf16 {mode} bwd slice={sl}")
    x = W.make_x_device(shape, "bf16", seed=77, std=1e-2)
    r1 = _rand((1, 1, 1, 64), "bf16", 78)
    r2 = _rand((1, 1, 1, 64), "bf16", 79)
    r1d, r2d = r1.to(DEV), r2.to(DEV)
    plan = rp.rope_partial_launch_info(x, r1d, r2d, mode, sl)
    assert plan["kernel"] == "vector"
    assert plan["blocks"] * plan["threads"] <= 2 ** 32 - 1
    assert plan["blocks"] < B * S * 2          # the blocks stride over the tile groups
    xv = x.view(total, D)
    rows = W.sample_rows(total, 4000, seed=77)
    rows_t = torch.from_numpy(rows).to(DEV)
    x_rows = W.to_numpy_storage(xv.index_select(0, rows_t).cpu())
    head0, tail0 = _lane_checksums(xv, 0, sl[0]), _lane_checksums(xv, sl[1], D)
    rp.rope_partial_bwd_inplace(x, r1d, r2d, mode, sl)
    torch.cuda.synchronize()
    got = W.to_numpy_storage(xv.index_select(0, rows_t).cpu())
    want = oracle_rows(x_rows, shape, "bf16", r1, r2, mode, sl, "bwd", rows)
    L = sl[1] - sl[0]
    c = np.broadcast_to(r1.double().numpy().reshape(1, L), (len(rows), L))
    s = np.broadcast_to(r2.double().numpy().reshape(1, L), (len(rows), L))
    info = compare(got, want, x_rows, c, s, "bf16", mode, "bwd", sl, "grid cap")
    assert info["exact"] == info["n"]
    assert _lane_checksums(xv, 0, sl[0]) == head0
    assert _lane_checksums(xv, sl[1], D) == tail0
    del x, xv
    torch.cuda.empty_cache()


def test_scalar_kernel_past_two_to_the_31_rows():
    """(1, 2^31 + 96, 1, 2) bf16, the whole two-lane row as the slice: from
    2^31 rows the 64-bit scalar kernel runs. Sampled rows (the first and last
    among them) against the oracle."""
    shape, sl, mode = (1, 2 ** 31 + 96, 1, 2), (0, 2), "interleave"
    total = shape[1]
    announce(f"64-bit scalar kernel shape={shape} bf16 fwd slice={sl}")
    x = W.make_x_device(shape, "bf16", seed=91)
    r1 = _rand((1, 1, 1, 2), "bf16", 92)
    r2 = _rand((1, 1, 1, 2), "bf16", 93)
    r1d, r2d = r1.to(DEV), r2.to(DEV)
    assert rp.rope_partial_launch_info(x, r1d, r2d, mode, sl)["kernel"] == "scalar"
    xv = x.view(total, 2)
    rows = W.sample_rows(total, 4000, seed=91)
    rows_t = torch.from_numpy(rows).to(DEV)
    x_rows = W.to_numpy_storage(xv.index_select(0, rows_t).cpu())
    rp.rope_partial_fwd_inplace(x, r1d, r2d, mode, sl)
    torch.cuda.synchronize()
    got = W.to_numpy_storage(xv.index_select(0, rows_t).cpu())
    want = oracle_rows(x_rows, shape, "bf16", r1, r2, mode, sl, "fwd", rows)
    c = np.broadcast_to(r1.double().numpy().reshape(1, 2), (len(rows), 2))
    s = np.broadcast_to(r2.double().numpy().reshape(1, 2), (len(rows), 2))
    info = compare(got, want, x_rows, c, s, "bf16", mode, "fwd", sl, "64-bit scalar kernel")
    assert info["exact"] == info["n"]
    del x, xv
    torch.cuda.empty_cache()
