"""Randomised parity sweep of the projection with a rotary epilogue
(rope_proj_fwd) against the oracle (oracle.proj_rope; "ascend-transformer-
boost 的 MlaPreprocessOperation：MLA 预处理四阶段融合算子深度解析", section 3,
with the rotary coefficient of section 2) on seeded random geometries that
mix its degrees of freedom at once: input dtype, output dtype (the inputs'
or fp32), table dtype, K, head width (32 to 576 lanes), head count, ragged
token counts, slice position and length (on and off the 8-lane grid, empty),
mode (interleave, rotate_half, coefficient 4) and table layout (one row per
token shared by the batch, per batch, per head). A case that
rope_proj_launch_info reports unsupported (a rotation group that no tile of
either kernel holds) must fail with that status; every other case is
compared on every output lane within check_proj's bound."""
import random

import pytest
import torch

import transformer_positional_encoding_amd as rp
from gpu_support import announce
from test_proj_gpu import TORCH, _rand, _tables, check_proj

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 160


def make_case(i: int) -> dict:
    r = random.Random(7000 + i)
    dt = r.choice(["bf16", "f16"])
    out = r.choice([dt, dt, "f32"])
    tdt = r.choice([dt, dt, "f32"])
    K = r.choice([64, 128, 192, 256, 384, 512])
    Dh = r.choice([32, 64, 96, 128, 192, 256, 384, 576])
    H = r.randint(1, max(1, 1536 // Dh))
    B, S = r.randint(1, 3), r.randint(1, 200)
    mode = r.choice(["interleave", "rotate_half", 4])
    if r.random() < 0.1:
        sl = None
    elif r.random() < 0.7:   # whole 8-lane vectors (the vector epilogues)
        start = 8 * r.randint(0, (Dh - 16) // 8)
        L = 16 * r.randint(1, (Dh - start) // 16)
        sl = (start, start + L)
    else:
        start = r.randint(0, Dh - 4)
        step = 4 if mode == 4 else 2
        L = step * r.randint(1, (Dh - start) // step)
        sl = (start, start + L)
    layout = r.choice(["token", "batch", "head"])
    return dict(dt=dt, out=out, tdt=tdt, K=K, Dh=Dh, H=H, B=B, S=S, mode=mode, sl=sl, layout=layout,
                seed=r.randint(0, 2 ** 20))


CASES = [make_case(i) for i in range(N_CASES)]


@pytest.mark.parametrize("case", CASES, ids=[f"{i}" for i in range(N_CASES)])
def test_random_projection_case(case):
    c = case
    B, S, K, H, Dh = c["B"], c["S"], c["K"], c["H"], c["Dh"]
    x = _rand((B, S, K), c["dt"], c["seed"], 0.5)
    w = _rand((H * Dh, K), c["dt"], c["seed"] + 1, 0.05)
    L = 0 if c["sl"] is None else c["sl"][1] - c["sl"][0]
    if L:
        r1, r2 = _tables(B, S, H, L, c["tdt"], c["seed"] + 2, per_batch=c["layout"] == "batch",
                         per_head=c["layout"] == "head", mode=c["mode"])
        if c["layout"] == "head":
            r1, r2 = r1.expand(-1, -1, H, -1).contiguous(), r2.expand(-1, -1, H, -1).contiguous()
    else:
        r1 = r2 = torch.zeros((1, 1, 1, 0), dtype=TORCH[c["tdt"]])
    code = rp.MODES[c["mode"]] if isinstance(c["mode"], str) else int(c["mode"])
    st, plan = rp.raw_proj_launch_info(rp._dtype_code(torch.empty(0, dtype=TORCH[c["out"]])), rp._dtype_code(x),
                                       (B, S, H, Dh), K, r1.data_ptr() or None, tuple(r1.shape), tuple(r1.stride()),
                                       r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                                       rp._dtype_code(r1) if r1.numel() else rp._dtype_code(x), code, c["sl"])
    what = f"random proj {c}"
    if st != rp.ROPE_OK:
        announce(f"{what}: unsupported ({rp.last_error()})")
        assert st == rp.ROPE_ERR_UNSUPPORTED, (what, st, rp.last_error())
        with pytest.raises(rp.RopeError) as e:
            rp.rope_proj_fwd(x.to(DEV), w.to(DEV), r1.to(DEV), r2.to(DEV), H, c["mode"], c["sl"],
                             out_dtype=TORCH[c["out"]])
        assert e.value.status == st
        return
    announce(f"{what}: {plan['kernel']} {plan['epilogue']} tables_in_lds={plan['tables_in_lds']}")
    check_proj(x, w, r1, r2, H, c["mode"], c["sl"], c["out"], what)


def test_random_cases_cover_both_kernels_and_epilogues():
    """The sweep above reaches both kernels and every square-tile epilogue
    (the plans only: rope_proj_launch_info launches nothing)."""
    seen = set()
    for c in CASES:
        B, S, H, Dh = c["B"], c["S"], c["H"], c["Dh"]
        L = 0 if c["sl"] is None else c["sl"][1] - c["sl"][0]
        shape = (B if c["layout"] == "batch" or c["layout"] == "head" else 1, S,
                 H if c["layout"] == "head" else 1, L) if L else (1, 1, 1, 0)
        t = torch.empty(shape, dtype=TORCH[c["tdt"]])
        code = rp.MODES[c["mode"]] if isinstance(c["mode"], str) else int(c["mode"])
        st, plan = rp.raw_proj_launch_info(rp._dtype_code(torch.empty(0, dtype=TORCH[c["out"]])),
                                           rp._dtype_code(torch.empty(0, dtype=TORCH[c["dt"]])), (B, S, H, Dh),
                                           c["K"], t.data_ptr() or None, tuple(t.shape), tuple(t.stride()),
                                           t.data_ptr() or None, tuple(t.shape), tuple(t.stride()),
                                           rp._dtype_code(t), code, c["sl"])
        if st == rp.ROPE_OK:
            seen.add((plan["kernel"], plan["epilogue"]))
    want = {("heads", None), ("square", "general"), ("square", "vector"), ("square", "vector_partner")}
    assert want <= seen, sorted(want - seen)
