"""Several tensors with shared tables in one call (Q and K of a GQA layer):
the result equals the single-tensor entry point on each tensor in order, and
the oracle."""
import numpy as np
import pytest
import torch

import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce, check_tensor, compare, expanded_tables, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _oracle(x, r1, r2, mode, sl, direction):
    D = x.shape[-1]
    dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype]
    out = oracle_rows(W.to_numpy_storage(x).reshape(-1, D).copy(), x.shape, dt, r1, r2, mode, sl, direction, None)
    return W.from_numpy_storage(out.reshape(x.shape), dt)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _same(a, b):
    return torch.equal(_bits(a.contiguous()), _bits(b.contiguous()))


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_gqa_q_and_k_one_call(direction):
    w = W.WORKLOADS["c2"]
    r1, r2 = W.make_tables(w)
    q, k = W.make_x(w, 0), W.make_x(w, 1)
    announce(f"multi c2 {direction}")
    qd, kd = q.to(DEV), k.to(DEV)
    fn = rp.rope_partial_fwd_inplace_multi if direction == "fwd" else rp.rope_partial_bwd_inplace_multi
    fn([qd, kd], r1.to(DEV), r2.to(DEV), "rotate_half", (0, 128))
    torch.cuda.synchronize()
    assert _same(qd.cpu(), _oracle(q, r1, r2, "rotate_half", (0, 128), direction))
    assert _same(kd.cpu(), _oracle(k, r1, r2, "rotate_half", (0, 128), direction))


@pytest.mark.parametrize("dtype,tdtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f16", "f32")])
@pytest.mark.parametrize("mode,sl", [("interleave", (32, 96)), ("interleave", (0, 64)), ("rotate_half", (0, 128))])
def test_four_tensors_match_single_calls(dtype, tdtype, mode, sl):
    """Head counts 16, 8, 3, 1 and two row widths, one call; equal to four
    single calls and to the oracle. 16-bit x with fp32 tables takes two
    heads per thread in place, in the multi-tensor kernel as well."""
    announce(f"multi 4 tensors {dtype} tables={tdtype} {mode} {sl}")
    g = torch.Generator().manual_seed(5)
    shapes = [(2, 64, 16, 128), (2, 64, 8, 128), (2, 64, 3, 192), (1, 64, 1, 128)]
    xs = [torch.randn(s, generator=g).to(DT[dtype]) for s in shapes]
    L = sl[1] - sl[0]
    r1 = torch.randn((1, 64, 1, L), generator=g).to(DT[tdtype])
    r2 = torch.randn((1, 64, 1, L), generator=g).to(DT[tdtype])
    multi = [x.to(DEV) for x in xs]
    single = [x.to(DEV) for x in xs]
    rp.rope_partial_fwd_inplace_multi(multi, r1.to(DEV), r2.to(DEV), mode, sl)
    for x in single:
        rp.rope_partial_fwd_inplace(x, r1.to(DEV), r2.to(DEV), mode, sl)
    torch.cuda.synchronize()
    for x, m, s in zip(xs, multi, single):
        assert _same(m, s)
        want = _oracle(x, r1, r2, mode, sl, "fwd")
        if dtype == "f32":
            check_tensor(m.cpu(), x, want, r1, r2, mode, sl, "fwd", f"multi {dtype}/{tdtype}")
        elif tdtype == "f32":
            D = x.shape[-1]
            rows = np.arange(x.numel() // D, dtype=np.int64)
            compare(W.to_numpy_storage(m.cpu()).reshape(-1, D), W.to_numpy_storage(want).reshape(-1, D),
                    W.to_numpy_storage(x).reshape(-1, D), expanded_tables(r1, x.shape, rows, L),
                    expanded_tables(r2, x.shape, rows, L), dtype, mode, "fwd", sl, f"multi {dtype}/{tdtype}")
        else:
            assert _same(m.cpu(), want)


def test_mixed_kernels_fall_back_to_separate_launches():
    """One tensor 16-byte aligned, one not (general kernel): still one call."""
    announce("multi mixed kernels")
    g = torch.Generator().manual_seed(6)
    a = torch.randn((2, 8, 4, 64), generator=g).to(torch.bfloat16)
    b = torch.randn((2, 8, 2, 64), generator=g).to(torch.bfloat16)
    r1 = torch.randn((1, 8, 1, 32), generator=g).to(torch.bfloat16)
    r2 = torch.randn((1, 8, 1, 32), generator=g).to(torch.bfloat16)
    ad = a.to(DEV)
    buf = torch.zeros(b.numel() + 1, dtype=torch.bfloat16, device=DEV)
    bd = buf[1:].view(b.shape)
    bd.copy_(b.to(DEV))
    rp.rope_partial_fwd_inplace_multi([ad, bd], r1.to(DEV), r2.to(DEV), "interleave", (16, 48))
    torch.cuda.synchronize()
    assert _same(ad.cpu(), _oracle(a, r1, r2, "interleave", (16, 48), "fwd"))
    assert _same(bd.cpu(), _oracle(b, r1, r2, "interleave", (16, 48), "fwd"))


def test_error_in_one_tensor_touches_none():
    g = torch.Generator().manual_seed(7)
    a = torch.randn((2, 8, 4, 64), generator=g).to(torch.bfloat16).to(DEV)
    b = torch.randn((2, 9, 2, 64), generator=g).to(torch.bfloat16).to(DEV)   # S does not match the tables
    r = torch.randn((1, 8, 1, 32), generator=g).to(torch.bfloat16).to(DEV)
    a0 = a.clone()
    with pytest.raises(rp.RopeError) as e:
        rp.rope_partial_fwd_inplace_multi([a, b], r, r, "interleave", (0, 32))
    assert e.value.status == rp.ROPE_ERR_INVALID and "tensor 1" in str(e.value)
    torch.cuda.synchronize()
    assert _same(a, a0)
