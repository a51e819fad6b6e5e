"""The position entry points out of place (rope_partial_{fwd,bwd}_out_pos)
and the autograd ops built on them (partial_rotary_mul_pos,
inplace_partial_rotary_mul_pos), against the CPU oracle: the oracle builds
the cos/sin tables of the same positions (rope_oracle_pos_tables; "ANE实战
RoPE位置编码在MIL中的纯ANE实现", section 第一步) and rotates with them. The
input is left unchanged; 16-bit results with 16-bit tables match bit for
bit."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, check_tensor, compare, expanded_tables

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TDT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _seed(*key):
    return zlib.crc32(repr(key).encode()) % 100000


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(DT[dtype])


def _positions(B, S, seed, per_batch=True):
    g = torch.Generator().manual_seed(seed)
    off = torch.randint(0, 70000, (B if per_batch else 1, 1), generator=g)
    return off + torch.arange(S)[None, :]


def _oracle(x_cpu, pos, f, mode, sl, direction, tdtype):
    """x rotated by the oracle with the tables of pos: a CPU tensor."""
    dtype = TDT[x_cpu.dtype]
    L = sl[1] - sl[0]
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), L, mode, tdtype)
    want = W.to_numpy_storage(x_cpu).copy()
    if L:
        oracle.rope_rows(want, x_cpu.shape, dtype, c, s, mode, sl, direction, table_dtype=tdtype)
    return W.from_numpy_storage(want, dtype), c, s


def _bits(t):
    t = t.contiguous()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


CASES = [
    # (shape, slice, mode)
    ((2, 16, 8, 128), (32, 96), "interleave"),     # half-line slice inside whole rows
    ((2, 16, 8, 128), (0, 128), "rotate_half"),    # whole head: partner in the other half
    ((2, 8, 6, 192), (0, 64), 4),                  # rotary coefficient 4 on an MLA-style row
    ((2, 7, 1, 128), (64, 128), "rotate_half"),    # one head: several positions per block
    ((1, 4, 3, 1024), (0, 1024), "rotate_half"),   # 512 pairs, rows of up to 256 vectors
    ((2, 6, 5, 64), (3, 35), "interleave"),        # odd start: copy, then the row kernel in place
]


@pytest.mark.parametrize("dtype,tdtype", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_out_of_place_positions(case, direction, dtype, tdtype):
    shape, sl, mode = case
    L = sl[1] - sl[0]
    seed = _seed(case, dtype, tdtype)
    x = _rand(shape, dtype, seed)
    pos = _positions(shape[0], shape[1], seed + 1)
    f = rp.rope_inv_freq(L, 500000.0)
    announce(f"out-of-place positions {shape} {sl} {mode} {dtype} tables={tdtype} {direction}")
    xd = x.to(DEV)
    y = torch.full_like(xd, float("nan"))
    fn = rp.rope_partial_fwd_out_pos if direction == "fwd" else rp.rope_partial_bwd_out_pos
    fn(y, xd, pos.to(DEV), f.to(DEV), mode, sl, DT[tdtype])
    torch.cuda.synchronize()
    assert torch.equal(_bits(xd), _bits(x.to(DEV))), "the input changed"
    want, c, s = _oracle(x, pos, f, mode, sl, direction, tdtype)
    B, S, N, D = shape
    rows = np.arange(B * S * N, dtype=np.int64)
    got = W.to_numpy_storage(y.cpu()).reshape(-1, D)
    info = compare(got, W.to_numpy_storage(want).reshape(-1, D), W.to_numpy_storage(x).reshape(-1, D),
                   expanded_tables(W.from_numpy_storage(c, tdtype), shape, rows, L),
                   expanded_tables(W.from_numpy_storage(s, tdtype), shape, rows, L), dtype, mode, direction, sl,
                   "out-of-place positions")
    if dtype != "f32" and tdtype != "f32":
        assert info["exact"] == info["n"]
    # 16-bit data: the same bytes as the in-place position call (fp32 data
    # may fuse its multiply-add, and the two schemes contract it differently)
    if dtype != "f32":
        xi = x.to(DEV)
        (rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos)(
            xi, pos.to(DEV), f.to(DEV), mode, sl, DT[tdtype])
        torch.cuda.synchronize()
        assert torch.equal(_bits(xi), _bits(y))


def test_out_of_place_positions_unaligned_and_empty_slice():
    """x 2 bytes past alignment (copy, then the in-place plan on y), and an
    empty slice (a plain copy)."""
    shape, sl, mode = (2, 12, 4, 64), (0, 64), "interleave"
    x = _rand(shape, "bf16", 91)
    pos = _positions(2, 12, 92)
    f = rp.rope_inv_freq(64, 10000.0)
    announce("out-of-place positions: unaligned x, empty slice")
    n = x.numel()
    buf = torch.zeros(n + 1, dtype=torch.bfloat16, device=DEV)
    xd = buf[1:].view(shape)
    xd.copy_(x.to(DEV))
    y = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    rp.rope_partial_fwd_out_pos(y, xd, pos.to(DEV), f.to(DEV), mode, sl)
    torch.cuda.synchronize()
    want, _, _ = _oracle(x, pos, f, mode, sl, "fwd", "bf16")
    assert torch.equal(_bits(y.cpu()), _bits(want))
    y2 = torch.zeros_like(y)
    rp.rope_partial_bwd_out_pos(y2, xd, pos.to(DEV), f.to(DEV), mode, (8, 8))
    torch.cuda.synchronize()
    assert torch.equal(_bits(y2), _bits(xd))


@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_out_of_place_positions_long_context_shard(direction):
    """The (16,8192,32,128) bf16 shard, lanes [32,96), per-batch positions:
    sampled rows against the oracle, and every row's lanes outside the
    slice equal to the input's."""
    w = W.WORKLOADS["c4"]
    x = W.make_x(w)
    pos = torch.from_numpy(W.positions(w))
    f = rp.rope_inv_freq(w.L, w.base)
    announce(f"out-of-place positions c4 {direction}")
    xd = x.to(DEV)
    y = torch.empty_like(xd)
    (rp.rope_partial_fwd_out_pos if direction == "fwd" else rp.rope_partial_bwd_out_pos)(
        y, xd, pos.to(DEV), f.to(DEV), w.mode, w.partial_slice)
    torch.cuda.synchronize()
    B, S, N, D = w.x_shapes[0]
    total = B * S * N
    rows = W.sample_rows(total, 4000, 17)
    rows_t = torch.from_numpy(rows).to(DEV)
    got = W.to_numpy_storage(y.view(total, D).index_select(0, rows_t).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x).reshape(total, D)[rows])
    c, s = oracle.pos_tables(pos.numpy(), f.numpy(), w.L, w.mode, "bf16")
    want = x_rows.copy()
    oracle.rope_rows(want, x.shape, "bf16", c, s, w.mode, w.partial_slice, direction, rows=rows, table_dtype="bf16")
    assert np.array_equal(got, want)
    lo, hi = w.partial_slice
    assert torch.equal(_bits(y[..., :lo]), _bits(xd[..., :lo])) and torch.equal(_bits(y[..., hi:]), _bits(xd[..., hi:]))


# ---------------------------------------------------------------- autograd

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode,sl", [("interleave", (32, 96)), ("rotate_half", (0, 128)), (4, (0, 64))])
@pytest.mark.parametrize("inplace", [False, True])
def test_position_autograd(inplace, mode, sl, dtype):
    """y = rope(x) from positions, loss = sum(y * w): y is the oracle's
    forward and x.grad the oracle's backward of w; positions and inv_freq
    get no gradient."""
    shape = (2, 16, 4, 128)
    L = sl[1] - sl[0]
    x = _rand(shape, dtype, _seed("ax", mode, dtype))
    w_ = _rand(shape, dtype, _seed("aw", mode, dtype))
    pos = _positions(2, 16, _seed("ap", mode))
    f = rp.rope_inv_freq(L, 10000.0)
    announce(f"position autograd inplace={inplace} {mode} {sl} {dtype}")
    xd = x.to(DEV).requires_grad_(True)
    fd = f.to(DEV).requires_grad_(True)
    if inplace:
        y = xd * 1.0
        rp.inplace_partial_rotary_mul_pos(y, pos.to(DEV), fd, mode, sl)
    else:
        y = rp.partial_rotary_mul_pos(xd, pos.to(DEV), fd, mode, sl)
    (y.float() * w_.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    want_y, c, s = _oracle(x, pos, f, mode, sl, "fwd", dtype)
    want_g, _, _ = _oracle(w_, pos, f, mode, sl, "bwd", dtype)
    got_y, got_g = y.detach().cpu(), xd.grad.cpu()
    # fp32: the normwise 1e-6 bound, with the oracle's tables of these
    # positions; 16-bit: bit for bit
    r1, r2 = W.from_numpy_storage(c, dtype), W.from_numpy_storage(s, dtype)
    info_y = check_tensor(got_y, x, want_y, r1, r2, mode, sl, "fwd", f"position autograd y {dtype}")
    info_g = check_tensor(got_g, w_, want_g, r1, r2, mode, sl, "bwd", f"position autograd x.grad {dtype}")
    if dtype != "f32":
        assert info_y["exact"] == info_y["n"] and info_g["exact"] == info_g["n"]
    assert fd.grad is None
    assert torch.equal(_bits(xd.detach().cpu()), _bits(x)), "x itself is not modified"


def test_position_autograd_leaf_rule_and_shared_gradient():
    x = _rand((1, 8, 2, 64), "bf16", 3).to(DEV).requires_grad_(True)
    pos = _positions(1, 8, 4).to(DEV)
    f = rp.rope_inv_freq(64).to(DEV)
    announce("position autograd: leaf rule, shared gradient")
    with pytest.raises(RuntimeError, match="leaf"):
        rp.inplace_partial_rotary_mul_pos(x, pos, f, "interleave", (0, 64))
    # y feeds two consumers through an add, whose backward hands both the
    # same gradient buffer: the rope backward must not modify it
    y = rp.partial_rotary_mul_pos(x, pos, f, "interleave", (0, 64))
    z = y * 1.0
    g = torch.randn_like(z)
    g0 = g.clone()
    out = z + y
    out.backward(g)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g), _bits(g0)), "the incoming gradient was modified"
    want, _, _ = _oracle(g.cpu(), pos.cpu(), f.cpu(), "interleave", (0, 64), "bwd", "bf16")
    # x.grad = bwd(g) (through y) + bwd(g) (through z = y * 1.0), each rounded to bf16, summed in bf16
    assert torch.equal(_bits(x.grad.cpu()), _bits(want + want))


SHARED = [
    # (shape, slice, mode, dtype, positions as one row (1,S) or expanded over the batch with stride 0)
    ((3, 37, 1, 128), (0, 128), "rotate_half", "bf16", "row"),      # one head: several positions per block
    ((4, 19, 2, 192), (0, 64), 4, "bf16", "expand"),                 # coefficient 4, two heads
    ((5, 23, 3, 64), (0, 64), "interleave", "f32", "row"),           # fp32, heads in a part-full chunk
    ((2, 9, 5, 128), (32, 96), "interleave", "f16", "expand"),       # half-line slice inside whole rows
]


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", SHARED, ids=[f"{c[0]}-{c[2]}-{c[3]}-{c[4]}" for c in SHARED])
def test_out_of_place_positions_shared_by_the_batch(case, direction):
    """Positions with batch stride 0 and few heads: the kernel takes the
    batches as heads of one position per s. Every row against the oracle;
    the input unchanged; 16-bit results equal to the in-place call's."""
    shape, sl, mode, dtype, layout = case
    B, S, N, D = shape
    L = sl[1] - sl[0]
    seed = _seed("shared", case)
    x = _rand(shape, dtype, seed)
    row = _positions(1, S, seed + 1)
    pos_dev = row.to(DEV) if layout == "row" else row.to(DEV).expand(B, S)
    assert layout == "row" or pos_dev.stride(0) == 0
    f = rp.rope_inv_freq(L, 10000.0)
    st, plan = rp.raw_launch_info_pos(1 << 20, shape, rp.DTYPE_CODES[dtype], 1 << 20, tuple(pos_dev.shape),
                                      tuple(pos_dev.stride()), 1 << 20, rp.DTYPE_CODES[dtype], rp.MODES.get(mode, mode),
                                      sl)
    assert st == rp.ROPE_OK and plan["kernel"] == "vector"
    # the in-place plan's blocks: ceil(S / positions per block) * head chunks of B*N heads
    heads = plan["head_lanes"] * plan["heads_per_thread"]
    assert plan["head_chunks"] == -(-(B * N) // heads)
    assert plan["blocks"] == -(-S // plan["positions_per_block"]) * plan["head_chunks"]
    announce(f"out-of-place positions shared by the batch {shape} {mode} {dtype} {layout} {direction}")
    xd = x.to(DEV)
    y = torch.full_like(xd, float("nan"))
    (rp.rope_partial_fwd_out_pos if direction == "fwd" else rp.rope_partial_bwd_out_pos)(
        y, xd, pos_dev, f.to(DEV), mode, sl)
    torch.cuda.synchronize()
    assert torch.equal(_bits(xd), _bits(x.to(DEV))), "the input changed"
    want, c, s = _oracle(x, row.expand(B, S), f, mode, sl, direction, dtype)
    rows = np.arange(B * S * N, dtype=np.int64)
    info = compare(W.to_numpy_storage(y.cpu()).reshape(-1, D), W.to_numpy_storage(want).reshape(-1, D),
                   W.to_numpy_storage(x).reshape(-1, D),
                   expanded_tables(W.from_numpy_storage(c, dtype), shape, rows, L),
                   expanded_tables(W.from_numpy_storage(s, dtype), shape, rows, L), dtype, mode, direction, sl,
                   "out-of-place positions shared by the batch")
    if dtype != "f32":
        assert info["exact"] == info["n"]
        xi = x.to(DEV)
        (rp.rope_partial_fwd_inplace_pos if direction == "fwd" else rp.rope_partial_bwd_inplace_pos)(
            xi, pos_dev, f.to(DEV), mode, sl)
        torch.cuda.synchronize()
        assert torch.equal(_bits(xi), _bits(y))
