"""Randomised parity sweep of the position entry points and the rotary
coefficient: the HIP path against the CPU oracle on seeded random cases that
mix x and table dtypes, mode (interleave, rotate_half, or a rotary
coefficient c: the slice in c parts, part 2k paired with part 2k+1 lane by
lane), direction, head dimension (2..1024), slice position and length,
positions per batch or shared, their layout (contiguous, expanded over the
batch with stride 0, a strided column of a wider tensor), their values (far
offsets, negative), x alignment, and the in-place, out-of-place and
multi-tensor position calls -- plus table calls with a rotary coefficient.
Every row is compared; 16-bit results with 16-bit tables must match bit for
bit. The tables of a position call are the oracle's (rope_oracle_pos_tables:
"ANE实战RoPE位置编码在MIL中的纯ANE实现", section 第一步); the coefficient is
"ascend-transformer-boost 的 MlaPreprocessOperation", section 2."""
import random

import numpy as np
import pytest
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, compare, expanded_tables

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
N_CASES = 120
MAX_ELEMS = 1 << 21


def make_case(i: int) -> dict:
    r = random.Random(5000 + i)
    dtype = r.choice(["f32", "f16", "bf16"])
    tdtype = dtype if r.random() < 0.7 else r.choice(["f32", "f16", "bf16"])
    if r.random() < 0.6:
        D = r.choice([8, 16, 32, 48, 64, 96, 128, 192, 256, 320, 512, 1024])
    else:
        D = 2 * r.randint(1, 512)
    if r.random() < 0.5:   # 16-byte aligned starts and lengths (vector kernels), when D allows
        step = 16 // (4 if dtype == "f32" else 2)
        starts = list(range(0, D - 1, step)) or [0]
        start = r.choice(starts)
        lens = [v for v in range(2 * step, D - start + 1, 2 * step)] or [2]
        L = r.choice(lens) if start + 2 <= D else 2
    else:
        start = r.randint(0, D - 2)
        L = 2 * r.randint(1, (D - start) // 2)
    coeffs = [c for c in range(2, L + 1, 2) if L % c == 0]
    mode = r.choice(["interleave", "rotate_half", "coeff", "coeff"])
    if mode == "coeff":
        mode = r.choice(coeffs)
    B, S = r.randint(1, 3), r.randint(1, 40)
    N = r.randint(1, 24)
    while B * S * N * D > MAX_ELEMS and N > 1:
        N //= 2
    while B * S * N * D > MAX_ELEMS and S > 1:
        S //= 2
    return dict(
        i=i, dtype=dtype, tdtype=tdtype, mode=mode, shape=(B, S, N, D), sl=(start, start + L),
        direction=r.choice(["fwd", "bwd"]), form=r.choice(["inplace", "inplace", "out", "multi", "table"]),
        per_batch=r.random() < 0.6, playout=r.choice(["contig", "contig", "expand", "column"]),
        far=r.random() < 0.3, x_offset=r.choice([0, 0, 0, 1, 2]), seed=r.randint(0, 2 ** 31 - 1))


def _rand(shape, dtype, g):
    return torch.randn(shape, generator=g).to(DT[dtype])


def device_x(x_cpu, offset):
    n = x_cpu.numel()
    buf = torch.zeros(n + offset, dtype=x_cpu.dtype, device=DEV)
    xd = buf[offset:].view(x_cpu.shape)
    xd.copy_(x_cpu.to(DEV))
    return xd


def make_positions(c, g):
    """(positions_cpu, positions_dev): the same values, in the case's layout
    on the device (the oracle reads the CPU tensor's own strides)."""
    B, S = c["shape"][0], c["shape"][1]
    Bp = B if c["per_batch"] else 1
    top = 2 ** 40 if c["far"] else 70000
    off = torch.randint(0, top, (Bp, 1), generator=g, dtype=torch.int64)
    if c["far"]:
        off = off * torch.where(torch.rand((Bp, 1), generator=g) < 0.5, -1, 1)
    pos = off + torch.arange(S, dtype=torch.int64)[None, :]
    if c["playout"] == "expand" and Bp == B and B > 1:
        row = pos[:1].clone()
        return row.expand(B, S), row.to(DEV).expand(B, S)
    if c["playout"] == "column":
        wide = torch.zeros((Bp, S, 3), dtype=torch.int64)
        wide[:, :, 2] = pos
        return pos, wide.to(DEV)[:, :, 2]
    return pos, pos.to(DEV)


def check(c, x_cpu, got_dev, cos, sin, what):
    B, S, N, D = x_cpu.shape
    L = c["sl"][1] - c["sl"][0]
    rows = np.arange(B * S * N, dtype=np.int64)
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x_cpu).reshape(-1, D))
    want = x_rows.copy()
    oracle.rope_rows(want, x_cpu.shape, c["dtype"], cos, sin, c["mode"], c["sl"], c["direction"], rows=rows,
                     table_dtype=c["tdtype"])
    got = W.to_numpy_storage(got_dev.cpu()).reshape(-1, D)
    r1 = W.from_numpy_storage(np.ascontiguousarray(cos), c["tdtype"])
    r2 = W.from_numpy_storage(np.ascontiguousarray(sin), c["tdtype"])
    info = compare(got, want, x_rows, expanded_tables(r1, x_cpu.shape, rows, L),
                   expanded_tables(r2, x_cpu.shape, rows, L), c["dtype"], c["mode"], c["direction"], c["sl"], what)
    if c["dtype"] != "f32" and c["tdtype"] != "f32":
        assert info["exact"] == info["n"], f"{what}: {info['n'] - info['exact']} lanes differ from the oracle"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_position_case(i):
    c = make_case(i)
    what = (f"case {i}: {c['form']} {c['direction']} x={c['dtype']}{c['shape']}+{c['x_offset']} "
            f"tables={c['tdtype']} mode={c['mode']} slice={c['sl']} positions={'B' if c['per_batch'] else '1'} "
            f"{c['playout']}{' far' if c['far'] else ''}")
    announce(what)
    g = torch.Generator().manual_seed(c["seed"])
    x = _rand(c["shape"], c["dtype"], g)
    pos, pos_dev = make_positions(c, g)
    L = c["sl"][1] - c["sl"][0]
    f = rp.rope_inv_freq(L, random.Random(c["seed"]).choice([10000.0, 500000.0]))
    cos, sin = oracle.pos_tables(pos.numpy(), f.numpy(), L, c["mode"], c["tdtype"])
    tdt = DT[c["tdtype"]]
    fwd = c["direction"] == "fwd"
    if c["form"] == "inplace":
        xd = device_x(x, c["x_offset"])
        (rp.rope_partial_fwd_inplace_pos if fwd else rp.rope_partial_bwd_inplace_pos)(
            xd, pos_dev, f.to(DEV), c["mode"], c["sl"], tdt)
        torch.cuda.synchronize()
        check(c, x, xd, cos, sin, what)
    elif c["form"] == "out":
        xd = device_x(x, c["x_offset"])
        y = torch.full_like(x, float("nan"), device=DEV)
        (rp.rope_partial_fwd_out_pos if fwd else rp.rope_partial_bwd_out_pos)(
            y, xd, pos_dev, f.to(DEV), c["mode"], c["sl"], tdt)
        torch.cuda.synchronize()
        assert torch.equal(xd.cpu().view(-1).view(torch.uint8), x.view(-1).view(torch.uint8)), f"{what}: x changed"
        check(c, x, y, cos, sin, what)
    elif c["form"] == "multi":
        B, S, N, D = c["shape"]
        x2 = _rand((B, S, max(1, N // 2 + 1), D), c["dtype"], g)
        xs = [device_x(x, c["x_offset"]), device_x(x2, 0)]
        (rp.rope_partial_fwd_inplace_pos_multi if fwd else rp.rope_partial_bwd_inplace_pos_multi)(
            xs, pos_dev, f.to(DEV), c["mode"], c["sl"], tdt)
        torch.cuda.synchronize()
        check(c, x, xs[0], cos, sin, what + " [tensor 0]")
        check(c, x2, xs[1], cos, sin, what + " [tensor 1]")
    else:
        # the table call with the oracle's tables of the same positions
        xd = device_x(x, c["x_offset"])
        r1 = W.from_numpy_storage(cos, c["tdtype"]).to(DEV)
        r2 = W.from_numpy_storage(sin, c["tdtype"]).to(DEV)
        (rp.rope_partial_fwd_inplace if fwd else rp.rope_partial_bwd_inplace)(xd, r1, r2, c["mode"], c["sl"])
        torch.cuda.synchronize()
        check(c, x, xd, cos, sin, what)


def test_the_sweep_reaches_every_kernel_and_mode():
    """The cases cover the position vector kernel and the row kernel, every
    form, and interleave, rotate_half and coefficients other than 2 and L
    (launch plans only; nothing is launched)."""
    kinds, forms, modes = set(), set(), set()
    for i in range(N_CASES):
        c = make_case(i)
        forms.add(c["form"])
        L = c["sl"][1] - c["sl"][0]
        modes.add(c["mode"] if isinstance(c["mode"], str) else ("coeff" if 2 < c["mode"] < L else "coeff-named"))
        B, S = c["shape"][0], c["shape"][1]
        st, plan = rp.raw_launch_info_pos(1 << 20, c["shape"], rp.DTYPE_CODES[c["dtype"]], 1 << 20, (B, S), (S, 1),
                                          1 << 20, rp.DTYPE_CODES[c["tdtype"]],
                                          rp.MODES.get(c["mode"], c["mode"]), c["sl"])
        assert st == rp.ROPE_OK
        kinds.add(plan["kernel"])
    assert {"vector", "rows"} <= kinds
    assert forms == {"inplace", "out", "multi", "table"}
    assert {"interleave", "rotate_half", "coeff"} <= modes
