"""Independent restatements of partial RoPE used to pin the oracle.

Nothing here is the oracle: each function states the operation in a different
form, so that a dropped term, a wrong sign, a wrong partner index or a
transposed backward in the oracle shows up as a mismatch.

* complex form: a pair (a, b) is the complex number a + i·b, and the forward
  rotation multiplies it by cos θ + i·sin θ (counter-clockwise); the backward
  multiplies by the conjugate.
* vector form: the formula of "CANN ops-transformer 算子详解：
  inplace_partial_rotary_mul 原地部分旋转位置编码", section 计算公式
  (x_out = x_slice·cos + x_rotate·sin with x_rotate built from the even and
  odd lanes), and for rotate_half the formula of "ANE实战RoPE位置编码在MIL中的
  纯ANE实现", section 先搞懂RoPE (q·cos + rotate_half(q)·sin, rotate_half
  swapping the halves and negating the first one); numpy array operations in
  fp64.
* gradient form: torch autograd (fp64, CPU) of the vector form gives the
  backward as the gradient with respect to x.

All take and return fp64 arrays; ``round_to`` applies the storage rounding
(fp32 arithmetic result, then RNE to the 16-bit type) with numpy/torch casts.
"""
from __future__ import annotations

import numpy as np
import torch


def expand_tables(r: np.ndarray, x_shape, L: int) -> np.ndarray:
    """A (possibly broadcast) 4-D table as a full fp64 (B,S,N,L) array."""
    B, S, N, _ = x_shape
    return np.broadcast_to(np.asarray(r, np.float64), (B, S, N, L)).copy()


def rotate_vector_form(x: np.ndarray, c: np.ndarray, s: np.ndarray, start: int, end: int,
                       mode: str) -> np.ndarray:
    """Forward on the lane range [start,end) of the last dim (fp64)."""
    y = np.array(x, np.float64, copy=True)
    xs = y[..., start:end].copy()
    L = end - start
    if mode == "interleave":
        x1 = xs[..., 0::2]
        x2 = xs[..., 1::2]
        # pairwise concatenation of (-x2, x1): lane 2i takes -x_{2i+1}, lane 2i+1 takes x_{2i}
        xr = np.stack([-x2, x1], axis=-1).reshape(xs.shape)
    else:
        h = L // 2
        xr = np.concatenate([-xs[..., h:], xs[..., :h]], axis=-1)
    y[..., start:end] = xs * c + xr * s
    return y


def rotate_complex_form(x: np.ndarray, c: np.ndarray, s: np.ndarray, start: int, end: int,
                        mode: str, inverse: bool = False) -> np.ndarray:
    """Forward (or inverse) rotation of each pair as a complex product.

    Needs tables that share one angle per pair (pair-duplicated for
    interleave, repeated halves for rotate_half); the first lane of each pair
    supplies cos and sin.
    """
    y = np.array(x, np.float64, copy=True)
    L = end - start
    xs = y[..., start:end]
    if mode == "interleave":
        a, b = xs[..., 0::2], xs[..., 1::2]
        cc, ss = c[..., 0::2], s[..., 0::2]
    else:
        h = L // 2
        a, b = xs[..., :h], xs[..., h:]
        cc, ss = c[..., :h], s[..., :h]
    rot = cc + 1j * ss
    if inverse:
        rot = np.conj(rot)
    z = (a + 1j * b) * rot
    out = np.empty_like(xs)
    if mode == "interleave":
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        h = L // 2
        out[..., :h], out[..., h:] = z.real, z.imag
    y[..., start:end] = out
    return y


def backward_by_autograd(g: np.ndarray, c: np.ndarray, s: np.ndarray, start: int, end: int,
                         mode: str) -> np.ndarray:
    """dL/dx of L = <g, forward(x)>: the Jacobian transpose applied to g."""
    xt = torch.zeros(g.shape, dtype=torch.float64, requires_grad=True)
    ct = torch.from_numpy(np.asarray(c, np.float64))
    st = torch.from_numpy(np.asarray(s, np.float64))
    xs = xt[..., start:end]
    if mode == "interleave":
        x1, x2 = xs[..., 0::2], xs[..., 1::2]
        xr = torch.stack([-x2, x1], dim=-1).reshape(xs.shape)
    else:
        h = (end - start) // 2
        xr = torch.cat([-xs[..., h:], xs[..., :h]], dim=-1)
    y = torch.cat([xt[..., :start], xs * ct + xr * st, xt[..., end:]], dim=-1)
    gt = torch.from_numpy(np.asarray(g, np.float64))
    (grad,) = torch.autograd.grad(y, xt, grad_outputs=gt)
    return grad.numpy()


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values -> storage form: fp32 result (RNE), then RNE to the 16-bit
    type for fp16/bf16. Returns float32 for f32, raw uint16 bits otherwise."""
    with np.errstate(over="ignore"):   # overflow to +-inf is the RNE result the pins expect
        f = np.asarray(v, np.float64).astype(np.float32)
        if dtype == "f32":
            return f
        if dtype == "f16":
            return f.astype(np.float16).view(np.uint16)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.uint16).numpy()


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> fp64 values, with numpy/torch casts."""
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16)).view(torch.bfloat16)
    return t.double().numpy()


def assert_storage_equal(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> None:
    """Bit-identical storage, except that any NaN matches any NaN."""
    gw, ww = widen(got, dtype), widen(want, dtype)
    nan = np.isnan(ww)
    assert np.array_equal(np.isnan(gw), nan), f"{what}: NaN pattern differs"
    key = np.uint32 if dtype == "f32" else np.uint16
    g = np.asarray(got).view(key)[~nan]
    w = np.asarray(want).view(key)[~nan]
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} elements differ; first: "
                           f"got {gw[~nan][bad[:4]]} want {ww[~nan][bad[:4]]}")
