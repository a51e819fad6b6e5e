"""The out-of-place entry points (rope_partial_fwd_out / rope_partial_bwd_out)
against the CPU oracle: y must equal the in-place result on a copy of x
(the oracle run on that copy), every lane outside the slice must be x's bytes,
and x must come back unchanged. Also the autograd ops that use them
("CANN ops-transformer 算子详解：inplace_partial_rotary_mul 原地部分旋转位置编码",
section 自动微分说明: the backward is the gradient with respect to x)."""
import zlib

import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, check_tensor, oracle_rows, run_out_and_check

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TDT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(DT[dtype])


def _bits(t):
    t = t.contiguous()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


CASES = [
    # (shape, slice, mode, table shape)     -- what it exercises
    ((2, 8, 4, 64), (0, 64), "interleave", (1, 8, 1, 64)),        # full slice
    ((2, 8, 4, 192), (64, 192), "interleave", (2, 8, 1, 128)),    # slice at the row end
    ((3, 5, 13, 96), (16, 80), "interleave", (1, 5, 1, 64)),      # ragged head count
    ((1, 4, 37, 128), (8, 104), "interleave", (1, 4, 1, 96)),     # slice inside 128-byte lines
    ((1, 3, 300, 64), (0, 64), "interleave", (1, 3, 1, 64)),      # many heads per block
    ((2, 6, 5, 64), (3, 35), "interleave", (1, 6, 1, 32)),        # odd start: copy, then the row kernel
    ((2, 8, 4, 128), (0, 128), "rotate_half", (1, 8, 1, 128)),
    ((2, 8, 4, 256), (64, 192), "rotate_half", (2, 8, 1, 128)),   # partial rotate_half: whole rows
    ((2, 5, 3, 48), (4, 44), "rotate_half", (1, 5, 1, 40)),       # general path
    ((2, 8, 4, 64), (0, 64), "interleave", (2, 8, 4, 64)),        # per-head tables
    ((2, 8, 4, 128), (32, 96), "rotate_half", (2, 8, 4, 64)),     # per-head tables, partial rotate_half
    ((2, 3, 5, 1024), (8, 1016), "interleave", (1, 3, 1, 1008)),  # D at its limit: 256 vectors per fp32 row
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}" for c in CASES])
def test_out_of_place_shapes(case, direction, dtype):
    shape, sl, mode, tshape = case
    seed = zlib.crc32(repr(("out", shape, sl, mode, tshape)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    r1 = _rand(tshape, dtype, seed + 1)
    r2 = _rand(tshape, dtype, seed + 2)
    info = run_out_and_check(x, r1, r2, mode, sl, direction, f"{shape} {sl} {mode} {tshape}")
    if dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("dtype,tdtype", [("bf16", "f32"), ("f32", "bf16"), ("f16", "bf16")])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_out_of_place_mixed_table_dtypes(dtype, tdtype, direction):
    shape, sl, mode, tshape = (2, 8, 4, 128), (32, 96), "interleave", (2, 8, 1, 64)
    seed = zlib.crc32(repr(("out-mixed", dtype, tdtype)).encode()) % 10000
    x = _rand(shape, dtype, seed)
    r1, r2 = _rand(tshape, tdtype, seed + 1), _rand(tshape, tdtype, seed + 2)
    info = run_out_and_check(x, r1, r2, mode, sl, direction, f"{dtype} x {tdtype} tables")
    if dtype != "f32":
        assert info["exact"] == info["n"]


@pytest.mark.parametrize("name", ["c4", "c3"])
@pytest.mark.parametrize("direction", ["bwd", "fwd"])
def test_out_of_place_full_size(name, direction):
    """The long-context shard and the MLA shape at full size, sampled rows;
    the lanes outside the slice are checked on the device for every row."""
    w = W.WORKLOADS[name]
    x = W.make_x(w)
    r1, r2 = W.make_tables(w)
    info = run_out_and_check(x, r1, r2, w.mode, w.partial_slice, direction, f"{name} {direction}")
    assert info["rows"] == w.x_shapes[0][0] * w.x_shapes[0][1] * w.x_shapes[0][2]
    assert info["exact"] == info["n"]


def test_out_of_place_equals_in_place_bitwise():
    """Both forms of the call give the same bytes (c1 workload, fp16)."""
    w = W.WORKLOADS["c1"]
    x = W.make_x(w)
    r1, r2 = (t.to(DEV) for t in W.make_tables(w))
    announce("out-of-place vs in-place c1")
    xd = x.to(DEV)
    y = torch.empty_like(xd)
    for direction in ("fwd", "bwd"):
        inplace = xd.clone()
        (rp.rope_partial_fwd_inplace if direction == "fwd" else rp.rope_partial_bwd_inplace)(
            inplace, r1, r2, w.mode, w.partial_slice)
        (rp.rope_partial_fwd_out if direction == "fwd" else rp.rope_partial_bwd_out)(
            y, xd, r1, r2, w.mode, w.partial_slice)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(inplace)), direction


def test_same_buffer_is_the_in_place_call():
    shape, sl = (2, 8, 4, 128), (32, 96)
    x = _rand(shape, "bf16", 61)
    r1, r2 = _rand((1, 8, 1, 64), "bf16", 62), _rand((1, 8, 1, 64), "bf16", 63)
    announce("out-of-place with y == x")
    xd = x.to(DEV)
    rp.rope_partial_bwd_out(xd, xd, r1.to(DEV), r2.to(DEV), "interleave", sl)
    torch.cuda.synchronize()
    want = oracle_rows(W.to_numpy_storage(x).reshape(-1, 128).copy(), shape, "bf16", r1, r2, "interleave", sl,
                       "bwd", None)
    assert W.to_numpy_storage(xd.cpu()).reshape(-1, 128).tobytes() == want.tobytes()


def test_overlap_is_rejected_before_touching_memory():
    shape, sl = (2, 4, 3, 64), (0, 32)
    announce("out-of-place overlap")
    buf = _rand((2 * 4 * 3 * 64 + 8,), "bf16", 71).to(DEV)
    before = buf.clone()
    r = _rand((1, 4, 1, 32), "bf16", 72).to(DEV)
    x = buf[:-8].view(shape)
    y = buf[8:].view(shape)
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_out(y, x, r, r, "interleave", sl)
    assert e.value.status == rp.ROPE_ERR_INVALID and "overlap" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(_bits(buf), _bits(before))


def test_empty_slice_copies_without_tables():
    """An empty slice makes y a copy of x; the tables are not looked at
    (NULL through the C ABI). An empty tensor touches nothing."""
    x = _rand((2, 4, 3, 64), "f16", 81)
    announce("out-of-place empty slice")
    xd = x.to(DEV)
    y = torch.full_like(xd, float("nan"))
    st = rp.raw_out_call("fwd", y.data_ptr(), xd.data_ptr(), tuple(xd.shape), 1, None, None, None, None, None,
                         None, 1, 1, (8, 8), torch.cuda.current_stream().cuda_stream)
    assert st == rp.ROPE_OK
    st = rp.raw_out_call("bwd", None, None, (0, 4, 3, 64), 1, None, None, None, None, None, None, 1, 1, (0, 32),
                         None)
    assert st == rp.ROPE_OK
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(xd))


@pytest.mark.parametrize("which", ["x", "y"])
def test_unaligned_buffers_take_the_general_path(which):
    """x or y 2 bytes past a 16-byte boundary: the library copies x into y and
    rotates y in place; guard elements around y stay untouched."""
    shape, sl = (2, 4, 3, 64), (16, 48)
    x = _rand(shape, "bf16", 91)
    r1, r2 = _rand((1, 4, 1, 32), "bf16", 92), _rand((1, 4, 1, 32), "bf16", 93)
    announce(f"out-of-place unaligned {which}")
    n = x.numel()
    xbuf = torch.zeros(n + 1, dtype=torch.bfloat16, device=DEV)
    ybuf = torch.full((n + 2,), 7.0, dtype=torch.bfloat16, device=DEV)
    xd = (xbuf[1:] if which == "x" else xbuf[:n]).view(shape)
    yd = (ybuf[1:n + 1] if which == "y" else ybuf[:n]).view(shape)
    xd.copy_(x.to(DEV))
    assert (xd.data_ptr() % 16 != 0) == (which == "x") and (yd.data_ptr() % 16 != 0) == (which == "y")
    run_out_and_check(x, r1, r2, "interleave", sl, "fwd", f"unaligned {which}", y_dev=yd, x_dev=xd)
    if which == "y":
        assert ybuf[0].item() == 7.0 and ybuf[-1].item() == 7.0
    else:
        assert ybuf[-1].item() == 7.0 and ybuf[-2].item() == 7.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_around_the_output(dtype):
    shape, sl = (2, 16, 6, 128), (32, 96)
    x = _rand(shape, dtype, 101)
    r1, r2 = _rand((1, 16, 1, 64), dtype, 102), _rand((1, 16, 1, 64), dtype, 103)
    announce(f"out-of-place guard bands {dtype}")
    esz = torch.tensor([], dtype=DT[dtype]).element_size()
    guard = 4096 // esz
    buf = _rand((guard + x.numel() + guard,), dtype, 104).to(DEV)
    ref = buf.clone()
    yd = buf[guard: guard + x.numel()].view(shape)
    xd = x.to(DEV)
    rp.rope_partial_fwd_out(yd, xd, r1.to(DEV), r2.to(DEV), "interleave", sl)
    rp.rope_partial_bwd_out(yd, xd, r1.to(DEV), r2.to(DEV), "rotate_half", (0, 64))
    torch.cuda.synchronize()
    assert torch.equal(_bits(buf[:guard]), _bits(ref[:guard]))
    assert torch.equal(_bits(buf[guard + x.numel():]), _bits(ref[guard + x.numel():]))


def test_graph_capture_of_out_of_place_calls():
    """Captured out-of-place calls (vector kernel, general path with its
    copy, empty-slice copy) replayed several times, with eager work between
    the replays, match the eager results bit for bit."""
    shape = (2, 8, 4, 128)
    x = _rand(shape, "bf16", 111).to(DEV)
    r1, r2 = _rand((1, 8, 1, 64), "bf16", 112).to(DEV), _rand((1, 8, 1, 64), "bf16", 113).to(DEV)
    r1o, r2o = _rand((1, 8, 1, 62), "bf16", 114).to(DEV), _rand((1, 8, 1, 62), "bf16", 115).to(DEV)
    announce("out-of-place graph capture")
    calls = [("fwd", (32, 96), r1, r2), ("bwd", (1, 63), r1o, r2o)]
    want = []
    for direction, sl, a, b in calls:
        y = torch.empty_like(x)
        (rp.rope_partial_fwd_out if direction == "fwd" else rp.rope_partial_bwd_out)(y, x, a, b, "interleave", sl)
        want.append(y)
    want.append(x.clone())
    torch.cuda.synchronize()
    outs = [torch.empty_like(x) for _ in range(3)]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for (direction, sl, a, b), y in zip(calls, outs):
            (rp.rope_partial_fwd_out if direction == "fwd" else rp.rope_partial_bwd_out)(
                y, x, a, b, "interleave", sl)
        rp.rope_partial_fwd_out(outs[2], x, r1, r2, "interleave", (4, 4))
    for rep in range(3):
        for y in outs:
            y.fill_(float(rep + 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outs, want):
            assert torch.equal(_bits(got), _bits(ref)), f"replay {rep}"


# ---------------------------------------------------------------- autograd

def _oracle(x, r1, r2, mode, sl, direction):
    D = x.shape[-1]
    dt = TDT[x.dtype]
    out = oracle_rows(W.to_numpy_storage(x).reshape(-1, D).copy(), x.shape, dt, r1, r2, mode, sl, direction, None)
    return W.from_numpy_storage(out.reshape(x.shape), dt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode,sl", [("interleave", (0, 64)), ("rotate_half", (32, 96))])
def test_out_of_place_op_on_a_leaf(dtype, mode, sl):
    """partial_rotary_mul on a leaf that requires grad: y from the forward,
    x unchanged, x.grad the oracle backward of dL/dy; no table gradients."""
    announce(f"partial_rotary_mul {dtype} {mode} {sl}")
    shape = (2, 32, 8, 128)
    x = _rand(shape, dtype, 121)
    r1, r2 = _rand((2, 32, 1, 64), dtype, 122), _rand((2, 32, 1, 64), dtype, 123)
    w = _rand(shape, dtype, 124)
    xd = x.to(DEV).requires_grad_(True)
    r1d, r2d = r1.to(DEV).requires_grad_(True), r2.to(DEV).requires_grad_(True)
    y = rp.partial_rotary_mul(xd, r1d, r2d, rotary_mode=mode, partial_slice=sl)
    (y.float() * w.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(_bits(xd.detach()), _bits(x.to(DEV)))
    want_y, want_g = _oracle(x, r1, r2, mode, sl, "fwd"), _oracle(w, r1, r2, mode, sl, "bwd")
    got_y, got_g = y.detach().cpu(), xd.grad.cpu()
    # fp32: the normwise 1e-6 bound; 16-bit: bit for bit
    info_y = check_tensor(got_y, x, want_y, r1, r2, mode, sl, "fwd", f"partial_rotary_mul y {dtype}")
    info_g = check_tensor(got_g, w, want_g, r1, r2, mode, sl, "bwd", f"partial_rotary_mul x.grad {dtype}")
    if dtype != "f32":
        assert info_y["exact"] == info_y["n"] and info_g["exact"] == info_g["n"]
    assert r1d.grad is None and r2d.grad is None


def test_backward_leaves_a_shared_gradient_alone():
    """y feeds two consumers whose gradient is one buffer (an add hands the
    same tensor to both inputs): the rope backward must not rotate that
    buffer in place, or the other branch's gradient would change."""
    announce("autograd shared gradient")
    shape, sl, mode = (2, 8, 4, 64), (0, 64), "interleave"
    x = _rand(shape, "bf16", 131)
    r1, r2 = _rand((1, 8, 1, 64), "bf16", 132), _rand((1, 8, 1, 64), "bf16", 133)
    w = _rand(shape, "bf16", 134)
    xd = x.to(DEV).requires_grad_(True)
    other = _rand(shape, "bf16", 135).to(DEV).requires_grad_(True)
    y = rp.partial_rotary_mul(xd, r1.to(DEV), r2.to(DEV), mode, sl)
    z = y + other
    z.backward(w.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(_bits(other.grad), _bits(w.to(DEV)))
    assert torch.equal(_bits(xd.grad.cpu()), _bits(_oracle(w, r1, r2, mode, sl, "bwd")))


def test_out_of_place_op_on_a_non_contiguous_input():
    """A transposed view: the op rotates a private contiguous copy, x is left
    alone, and the gradient reaches the view's base."""
    announce("partial_rotary_mul on a non-contiguous view")
    shape, sl, mode = (2, 8, 4, 64), (0, 64), "interleave"
    base = _rand((2, 4, 8, 64), "bf16", 141)
    r1, r2 = _rand((1, 8, 1, 64), "bf16", 142), _rand((1, 8, 1, 64), "bf16", 143)
    w = _rand(shape, "bf16", 144)
    bd = base.to(DEV).requires_grad_(True)
    xv = bd.transpose(1, 2)                     # (2, 8, 4, 64), not contiguous
    assert not xv.is_contiguous()
    y = rp.partial_rotary_mul(xv, r1.to(DEV), r2.to(DEV), mode, sl)
    y.backward(w.to(DEV))
    torch.cuda.synchronize()
    x = base.transpose(1, 2).contiguous()
    assert torch.equal(_bits(y.detach().cpu()), _bits(_oracle(x, r1, r2, mode, sl, "fwd")))
    assert torch.equal(_bits(bd.detach().cpu()), _bits(base))
    want_g = _oracle(w, r1, r2, mode, sl, "bwd").transpose(1, 2)
    assert torch.equal(_bits(bd.grad.cpu()), _bits(want_g))
