"""Special values through the HIP kernels against the oracle: NaN, +-inf,
+-0, the largest finite values and subnormals, in every dtype, both modes
and both directions, on the vector kernel and on the row kernel (an odd
slice start). NaN must land on the same lanes; every other lane is held to
the usual bar (16-bit data within 1 ulp, fp32 within the normwise bound).
fp32 inputs stay below 1e30 so that no fp32 product overflows: near the
overflow threshold a fused fp32 evaluation and the fp64 oracle may disagree
about whether a cancelling sum is finite."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_support import run_and_check

pytestmark = pytest.mark.gpu
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BIG = {"f32": 1e30, "f16": 65504.0, "bf16": 3.3895e38}
TINY = {"f32": 1e-45, "f16": 6e-8, "bf16": 9.2e-41}     # smallest subnormals (rounded to the type)


def _special_x(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float64)
    flat = x.view(-1)
    n = flat.numel()
    idx = torch.randperm(n, generator=g)
    specials = [float("nan"), float("inf"), -float("inf"), 0.0, -0.0, BIG[dtype], -BIG[dtype],
                TINY[dtype], -TINY[dtype], 3 * TINY[dtype], BIG[dtype] / 3]
    per = n // 40
    for k, v in enumerate(specials):
        flat[idx[k * per:(k + 1) * per]] = v
    return x.to(TD[dtype])


def _tables(tshape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    theta = torch.rand(tshape, generator=g, dtype=torch.float64) * 6.3
    c, s = torch.cos(theta), torch.sin(theta)
    c.view(-1)[::7] = 0.0                        # exact zeros and a negative zero in the tables
    s.view(-1)[::11] = -0.0
    return c.to(TD[dtype]), s.to(TD[dtype])


CASES = [
    # (x shape, slice, mode, table shape)   -- kernel
    ((2, 8, 4, 128), (0, 64), "interleave", (1, 8, 1, 64)),     # vector
    ((2, 8, 4, 128), (32, 96), "interleave", (2, 8, 1, 64)),    # vector, whole-line coverage
    ((2, 8, 4, 128), (0, 128), "rotate_half", (1, 8, 1, 128)),  # vector, rotate_half
    ((2, 8, 4, 128), (1, 65), "interleave", (1, 8, 1, 64)),     # row kernel (odd start)
    ((2, 8, 4, 128), (2, 42), "rotate_half", (1, 8, 1, 40)),    # row kernel
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[2]}-{c[1]}" for c in CASES])
def test_special_values(case, direction, dtype):
    shape, sl, mode, tshape = case
    seed = 500 + CASES.index(case) * 10 + ("f32", "f16", "bf16").index(dtype)
    x = _special_x(shape, dtype, seed)
    r1, r2 = _tables(tshape, dtype, seed + 1)
    run_and_check(x, r1, r2, mode, sl, direction, f"special values {dtype} {mode} {sl} {direction}")
