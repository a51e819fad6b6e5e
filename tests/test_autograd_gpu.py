"""The autograd op over the C ABI: forward in place with the tensor marked
dirty, backward through the backward entry point, no gradient for r1/r2
("CANN ops-transformer 算子详解：inplace_partial_rotary_mul 原地部分旋转位置编码",
section 自动微分说明 and the training example of section 调用说明). Checked
against the CPU oracle on the same inputs."""
import numpy as np
import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, check_tensor, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(dtype, seed, shape=(2, 32, 8, 128), L=64, tshape=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g).to(DT[dtype])
    tshape = tshape or (shape[0], shape[1], 1, L)
    r1 = torch.randn(tshape, generator=g).to(DT[dtype])
    r2 = torch.randn(tshape, generator=g).to(DT[dtype])
    w = torch.randn(shape, generator=g).to(DT[dtype])
    return x, r1, r2, w


def _oracle(x, r1, r2, mode, sl, direction):
    D = x.shape[-1]
    dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype]
    out = oracle_rows(W.to_numpy_storage(x).reshape(-1, D).copy(), x.shape, dt, r1, r2, mode, sl, direction, None)
    return W.from_numpy_storage(out.reshape(x.shape), dt)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mode,sl", [("interleave", (0, 64)), ("rotate_half", (32, 96))])
def test_training_step_gradients(dtype, mode, sl):
    """The page's training example: y = x * 1.0, rotate y in place, reduce,
    backward. x.grad equals the oracle backward of dL/dy."""
    announce(f"autograd {dtype} {mode} {sl}")
    x, r1, r2, w = _inputs(dtype, 7)
    xd = x.to(DEV).requires_grad_(True)
    r1d = r1.to(DEV).requires_grad_(True)
    r2d = r2.to(DEV).requires_grad_(True)
    y = xd * 1.0
    rp.inplace_partial_rotary_mul(y, r1d, r2d, rotary_mode=mode, partial_slice=sl)
    loss = (y.float() * w.to(DEV).float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    want_y = _oracle(x, r1, r2, mode, sl, "fwd")
    want_g = _oracle(w, r1, r2, mode, sl, "bwd")
    got_y, got_g = y.detach().cpu(), xd.grad.cpu()
    # fp32: the normwise 1e-6 bound; 16-bit: bit for bit
    info_y = check_tensor(got_y, x, want_y, r1, r2, mode, sl, "fwd", f"autograd y {dtype}")
    info_g = check_tensor(got_g, w, want_g, r1, r2, mode, sl, "bwd", f"autograd x.grad {dtype}")
    if dtype != "f32":
        assert info_y["exact"] == info_y["n"] and info_g["exact"] == info_g["n"]
    assert r1d.grad is None and r2d.grad is None


def test_expanded_incoming_gradient():
    """y.sum() hands backward a stride-0 gradient; the op copies it first."""
    announce("autograd expanded grad")
    x, r1, r2, _ = _inputs("bf16", 8)
    xd = x.to(DEV).requires_grad_(True)
    y = xd * 1.0
    rp.inplace_partial_rotary_mul(y, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))
    y.sum().backward()
    want = _oracle(torch.ones_like(x), r1, r2, "interleave", (0, 64), "bwd")
    assert torch.equal(xd.grad.cpu().view(torch.int16), want.view(torch.int16))


def test_leaf_requiring_grad_is_rejected():
    x, r1, r2, _ = _inputs("bf16", 9)
    xd = x.to(DEV).requires_grad_(True)
    with pytest.raises(RuntimeError, match="leaf"):
        rp.inplace_partial_rotary_mul(xd, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))


def test_no_grad_path_rotates_in_place():
    announce("autograd no-grad path")
    x, r1, r2, _ = _inputs("bf16", 10)
    xd = x.to(DEV)
    rp.inplace_partial_rotary_mul(xd, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))
    torch.cuda.synchronize()
    want = _oracle(x, r1, r2, "interleave", (0, 64), "fwd")
    assert torch.equal(xd.cpu().view(torch.int16), want.view(torch.int16))


def test_version_counter_bumps():
    """Autograd sees the in-place change: using the pre-rotation value of a
    tensor saved by another op raises."""
    x, r1, r2, _ = _inputs("f32", 11)
    xd = x.to(DEV).requires_grad_(True)
    y = xd * 1.0
    z = y * y      # saves y
    rp.inplace_partial_rotary_mul(y, r1.to(DEV), r2.to(DEV), "interleave", (0, 64))
    with pytest.raises(RuntimeError):
        z.sum().backward()
