"""The entry points captured in a HIP graph (torch.cuda.graph) and replayed.

The library allocates nothing, records no memset and takes its stream from
the caller, so a captured call is a plain kernel node. Each replay is
compared bit for bit with the same calls made eagerly on a second buffer,
with eager work and synchronisations between the replays, and the first
replay also with the oracle (16-bit data, where the two agree bit for
bit)."""
import numpy as np
import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _oracle(x_cpu, r1, r2, mode, sl, direction):
    dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x_cpu.dtype]
    D = x_cpu.shape[-1]
    out = oracle_rows(W.to_numpy_storage(x_cpu).reshape(-1, D).copy(), x_cpu.shape, dt, r1, r2, mode, sl,
                      direction, None)
    return W.from_numpy_storage(out.reshape(x_cpu.shape), dt)


CASES = [
    # (workload, directions captured in order)
    ("c1", ("fwd",)),
    ("c1", ("bwd", "fwd")),
    ("c0", ("fwd", "bwd")),
]


@pytest.mark.parametrize("name,dirs", CASES, ids=[f"{n}-{'+'.join(d)}" for n, d in CASES])
def test_single_tensor_calls_replay_like_eager(name, dirs):
    w = W.WORKLOADS[name]
    x0 = W.make_x(w)
    r1, r2 = W.make_tables(w)
    r1d, r2d = r1.to(DEV), r2.to(DEV)
    announce(f"graph {name} {dirs}")

    def calls(x):
        for d in dirs:
            fn = rp.rope_partial_fwd_inplace if d == "fwd" else rp.rope_partial_bwd_inplace
            fn(x, r1d, r2d, w.mode, w.partial_slice)

    warm = x0.to(DEV)
    calls(warm)                      # first calls outside the capture (device queries cached)
    torch.cuda.synchronize()
    xg, xe = x0.to(DEV), x0.to(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(xg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(xg), _bits(x0.to(DEV))), "capture must not run the kernels"
    other = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        g.replay()
        calls(xe)
        other.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(xg), _bits(xe)), f"replay {rep} differs from the eager calls"
        if rep == 0 and x0.dtype != torch.float32:   # 16-bit data is bit-exact against the oracle
            want = x0
            for d in dirs:
                want = _oracle(want, r1, r2, w.mode, w.partial_slice, d)
            assert torch.equal(_bits(xg.cpu()), _bits(want)), "first replay differs from the oracle"


def test_multi_tensor_call_replays_like_eager():
    w = W.WORKLOADS["c2"]
    r1, r2 = W.make_tables(w)
    r1d, r2d = r1.to(DEV), r2.to(DEV)
    q0, k0 = W.make_x(w, 0), W.make_x(w, 1)
    announce("graph c2 multi fwd")
    warm = [q0.to(DEV), k0.to(DEV)]
    rp.rope_partial_fwd_inplace_multi(warm, r1d, r2d, w.mode, w.partial_slice)
    torch.cuda.synchronize()
    qg, kg, qe, ke = q0.to(DEV), k0.to(DEV), q0.to(DEV), k0.to(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rp.rope_partial_fwd_inplace_multi([qg, kg], r1d, r2d, w.mode, w.partial_slice)
    for rep in range(3):
        g.replay()
        rp.rope_partial_fwd_inplace(qe, r1d, r2d, w.mode, w.partial_slice)
        rp.rope_partial_fwd_inplace(ke, r1d, r2d, w.mode, w.partial_slice)
        torch.cuda.synchronize()
        assert torch.equal(_bits(qg), _bits(qe)) and torch.equal(_bits(kg), _bits(ke)), f"replay {rep}"


@pytest.mark.parametrize("mode,sl,shape", [("interleave", (32, 96), (4, 64, 8, 128)), (4, (0, 64), (2, 64, 16, 192)),
                                           ("rotate_half", (4, 44), (2, 16, 3, 48))],
                         ids=["interleave-vector", "coeff4-vector", "rotate_half-rows"])
def test_position_calls_replay_like_eager(mode, sl, shape):
    """The position entry points (cos and sin computed in the kernel) and a
    rotary coefficient, captured and replayed: the vector kernel and the row
    kernel's position form."""
    B, S = shape[0], shape[1]
    g0 = torch.Generator().manual_seed(41)
    x0 = torch.randn(shape, generator=g0).to(torch.bfloat16)
    pos = (torch.randint(0, 60000, (B, 1), generator=g0) + torch.arange(S)[None, :]).to(DEV)
    f = rp.rope_inv_freq(sl[1] - sl[0], 500000.0, DEV)
    announce(f"graph positions {mode} {shape} {sl}")

    def calls(x):
        rp.rope_partial_bwd_inplace_pos(x, pos, f, mode, sl)
        rp.rope_partial_fwd_inplace_pos(x, pos, f, mode, sl, table_dtype=torch.float32)

    warm = x0.to(DEV)
    calls(warm)
    torch.cuda.synchronize()
    xg, xe = x0.to(DEV), x0.to(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(xg)
    torch.cuda.synchronize()
    assert torch.equal(_bits(xg), _bits(x0.to(DEV))), "capture must not run the kernels"
    other = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        g.replay()
        calls(xe)
        other.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        assert torch.equal(_bits(xg), _bits(xe)), f"replay {rep} differs from the eager calls"
        assert not torch.equal(_bits(xg), _bits(x0.to(DEV))), "the calls must change x"


@pytest.mark.parametrize("mode,sl", [("interleave", (0, 64)), ("rotate_half", (0, 64)), ("interleave", None)])
def test_projection_call_replays_like_eager(mode, sl):
    """The projection with a rotary epilogue into a given output, captured
    and replayed (square tiles: the vector epilogue with the table rows
    staged in LDS, or the plain projection). x changes between the replays
    (eager work), and each replay writes the same bytes as an eager call on
    the same x."""
    g0 = torch.Generator().manual_seed(43)
    M, K, H, Dh = 300, 256, 4, 192
    x = torch.randn((1, M, K), generator=g0).to(torch.bfloat16).to(DEV)
    w = (torch.randn((H * Dh, K), generator=g0) / 16).to(torch.bfloat16).to(DEV)
    th = torch.randn((1, M, 1, 64), generator=g0, dtype=torch.float64)
    c = torch.cos(th).to(torch.bfloat16).to(DEV)
    s = torch.sin(th).to(torch.bfloat16).to(DEV)
    if sl is None:
        c = s = torch.zeros((1, 1, 1, 0), dtype=torch.bfloat16, device=DEV)
    announce(f"graph projection {mode} {sl}")
    yg = torch.empty((1, M, H, Dh), dtype=torch.bfloat16, device=DEV)
    ye = torch.empty_like(yg)
    rp.rope_proj_fwd(x, w, c, s, H, mode, sl, out=yg)      # first call outside the capture
    torch.cuda.synchronize()
    yg.fill_(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rp.rope_proj_fwd(x, w, c, s, H, mode, sl, out=yg)
    torch.cuda.synchronize()
    assert not bool(yg.view(torch.int16).any()), "capture must not run the kernel"
    for rep in range(4):
        x.mul_(-1.0).add_(0.25)                              # eager work: another x for each replay
        g.replay()
        rp.rope_proj_fwd(x, w, c, s, H, mode, sl, out=ye)
        torch.cuda.synchronize()
        assert torch.equal(yg.view(torch.int16), ye.view(torch.int16)), f"replay {rep} differs from the eager call"
