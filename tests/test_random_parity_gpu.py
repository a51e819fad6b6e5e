"""Randomised parity sweep: the HIP path against the CPU oracle on seeded
random cases that mix every degree of freedom of the C ABI at once -- x and
table dtypes, mode, direction, head dimension (2..1024), slice position and
length, table broadcast shape (1 or the full size in B, S and N), table layout
(contiguous, expand() views with zero strides, slices of a wider buffer), x
alignment (16-byte aligned or 2-4 bytes past it), and the in-place,
out-of-place and multi-tensor entry points. Every row is compared. The
constraints are those of "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
原地部分旋转位置编码", section 约束说明; the rotate_half pairing is from
"ANE实战RoPE位置编码在MIL中的纯ANE实现", section 先搞懂RoPE."""
import random

import numpy as np
import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import TDT, announce, compare, expanded_tables, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
N_CASES = 160
MAX_ELEMS = 1 << 21


def make_case(i: int) -> dict:
    r = random.Random(1000 + i)
    dtype = r.choice(["f32", "f16", "bf16"])
    tdtype = dtype if r.random() < 0.7 else r.choice(["f32", "f16", "bf16"])
    mode = r.choice(["interleave", "rotate_half"])
    if r.random() < 0.6:
        D = r.choice([8, 16, 32, 48, 64, 96, 128, 192, 256, 320, 512, 1024])
    else:
        D = 2 * r.randint(1, 512)
    if r.random() < 0.5:   # starts and lengths on 16-byte boundaries (vector kernel), when D allows
        step = 16 // (4 if dtype == "f32" else 2)
        starts = list(range(0, D - 1, step)) or [0]
        start = r.choice(starts)
        lens = [v for v in range(2 * step, D - start + 1, 2 * step)] or [2]
        L = r.choice(lens) if start + 2 <= D else 2
    else:
        start = r.randint(0, D - 2)
        L = 2 * r.randint(1, (D - start) // 2)
    B, S = r.randint(1, 3), r.randint(1, 40)
    N = r.randint(1, 24)
    while B * S * N * D > MAX_ELEMS and N > 1:
        N //= 2
    while B * S * N * D > MAX_ELEMS and S > 1:
        S //= 2
    tshape = tuple(r.choice([1, v]) for v in (B, S, N)) + (L,)
    return dict(
        i=i, dtype=dtype, tdtype=tdtype, mode=mode, shape=(B, S, N, D), sl=(start, start + L), tshape=tshape,
        layout=r.choice(["contig", "contig", "expand", "wide"]), direction=r.choice(["fwd", "bwd"]),
        form=r.choice(["inplace", "inplace", "out", "multi"]), x_offset=r.choice([0, 0, 0, 1, 2]),
        tables=r.choice(["random", "rope"]), seed=r.randint(0, 2 ** 31 - 1))


def _rand(shape, dtype, g):
    return torch.randn(shape, generator=g).to(DT[dtype])


def make_tables(c, g):
    """(r1_cpu, r2_cpu, r1_dev, r2_dev): CPU tensors for the oracle (any
    strides) and the device tensors the call receives, in the case's layout."""
    B, S, N, D = c["shape"]
    L = c["sl"][1] - c["sl"][0]
    ts = c["tshape"]
    out = []
    for _ in range(2):
        if c["tables"] == "rope":
            # cos- or sin-like values in [-1, 1]
            base = torch.rand(ts, generator=g, dtype=torch.float64).mul(2).sub(1).to(DT[c["tdtype"]])
        else:
            base = _rand(ts, c["tdtype"], g)
        if c["layout"] == "expand":
            small = base[tuple(slice(0, 1) for _ in range(3))].contiguous()    # (1,1,1,L)
            cpu = small.expand(*ts)
            dev = small.to(DEV).expand(*ts)
        elif c["layout"] == "wide":
            extra = 5
            wide = _rand(ts[:3] + (L + extra,), c["tdtype"], g)
            cpu = wide[..., 3:3 + L]
            dev = wide.to(DEV)[..., 3:3 + L]
        else:
            cpu, dev = base, base.to(DEV)
        out.append((cpu, dev))
    return out[0][0], out[1][0], out[0][1], out[1][1]


def device_x(x_cpu, offset):
    """x on the device, `offset` elements past the start of its buffer."""
    n = x_cpu.numel()
    buf = torch.zeros(n + offset, dtype=x_cpu.dtype, device=DEV)
    xd = buf[offset:].view(x_cpu.shape)
    xd.copy_(x_cpu.to(DEV))
    return xd


def check(c, x_cpu, got_dev, r1, r2, what):
    B, S, N, D = x_cpu.shape
    rows = np.arange(B * S * N, dtype=np.int64)
    x_rows = W.to_numpy_storage(x_cpu).reshape(-1, D)
    want = oracle_rows(x_rows, x_cpu.shape, c["dtype"], r1.contiguous(), r2.contiguous(), c["mode"], c["sl"],
                       c["direction"], None)
    got = W.to_numpy_storage(got_dev.cpu()).reshape(-1, D)
    L = c["sl"][1] - c["sl"][0]
    info = compare(got, want, x_rows, expanded_tables(r1.contiguous(), x_cpu.shape, rows, L),
                   expanded_tables(r2.contiguous(), x_cpu.shape, rows, L), c["dtype"], c["mode"], c["direction"],
                   c["sl"], what)
    if c["dtype"] != "f32":
        assert info["exact"] == info["n"], f"{what}: {info['n'] - info['exact']} lanes differ from the oracle"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = make_case(i)
    what = (f"case {i}: {c['form']} {c['direction']} x={c['dtype']}{c['shape']}+{c['x_offset']} "
            f"tables={c['tdtype']}{c['tshape']} {c['layout']} {c['tables']} {c['mode']} slice={c['sl']}")
    announce(what)
    g = torch.Generator().manual_seed(c["seed"])
    x = _rand(c["shape"], c["dtype"], g)
    r1, r2, r1d, r2d = make_tables(c, g)
    if c["form"] == "inplace":
        xd = device_x(x, c["x_offset"])
        (rp.rope_partial_fwd_inplace if c["direction"] == "fwd" else rp.rope_partial_bwd_inplace)(
            xd, r1d, r2d, c["mode"], c["sl"])
        torch.cuda.synchronize()
        check(c, x, xd, r1, r2, what)
    elif c["form"] == "out":
        xd = device_x(x, c["x_offset"])
        y = torch.full_like(x, float("nan"), device=DEV)
        (rp.rope_partial_fwd_out if c["direction"] == "fwd" else rp.rope_partial_bwd_out)(
            y, xd, r1d, r2d, c["mode"], c["sl"])
        torch.cuda.synchronize()
        assert torch.equal(xd.cpu().view(-1).view(torch.uint8), x.view(-1).view(torch.uint8)), f"{what}: x changed"
        check(c, x, y, r1, r2, what)
    else:
        # a second tensor with another head count, when the tables broadcast over heads
        B, S, N, D = c["shape"]
        N2 = max(1, N // 2 + 1) if c["tshape"][2] == 1 else N
        x2 = _rand((B, S, N2, D), c["dtype"], g)
        xs = [device_x(x, c["x_offset"]), device_x(x2, 0)]
        (rp.rope_partial_fwd_inplace_multi if c["direction"] == "fwd" else rp.rope_partial_bwd_inplace_multi)(
            xs, r1d, r2d, c["mode"], c["sl"])
        torch.cuda.synchronize()
        check(c, x, xs[0], r1, r2, what + " [tensor 0]")
        check(c, x2, xs[1], r1, r2, what + " [tensor 1]")


def test_the_sweep_reaches_every_kernel():
    """The random cases cover the vector kernel, the row kernel, all three
    forms and both modes (checked on the launch plans, nothing launched)."""
    kinds, forms, modes = set(), set(), set()
    for i in range(N_CASES):
        c = make_case(i)
        forms.add(c["form"])
        modes.add(c["mode"])
        x = torch.empty(c["shape"], dtype=DT[c["dtype"]], device=DEV)
        r = torch.empty(c["tshape"], dtype=DT[c["tdtype"]], device=DEV)
        kinds.add(rp.rope_partial_launch_info(x, r, r, c["mode"], c["sl"])["kernel"])
    assert {"vector", "rows"} <= kinds and forms == {"inplace", "out", "multi"} and len(modes) == 2
