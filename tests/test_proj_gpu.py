"""The projection with a rotary epilogue (rope_proj_fwd) against the oracle
(oracle.proj_rope: exact dot products rounded to fp32, each head's slice
rotated as fp32 data, one rounding to the output type; "ascend-transformer-
boost 的 MlaPreprocessOperation：MLA 预处理四阶段融合算子深度解析", section 3).

The GPU accumulates in fp32 in its own order, so its projection may differ
from the oracle's by the fp32 summation bound |dp| <= K * 2^-23 * sum_k
|x_k w_k| (any order of K fp32 additions, rounding or truncating). Every
output lane is held to that bound carried through the rotation
(|c_j| dp_j + |s_j| dp_p(j)) plus the fp32 rotation bound of the table call
(1e-6 (|p_j c_j| + |p_p s_j|) + 2^-126); a 16-bit output may in addition
differ by one unit in its last place (a rounding boundary between the two
fp32 values). Every token and lane is compared.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W
from gpu_support import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
CODE = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


def _widen(bits, dt):
    return W.from_numpy_storage(np.ascontiguousarray(bits), dt).double().numpy()


def _pair(L, mode):
    j = np.arange(L)
    if mode == "interleave":
        return j ^ 1
    H = L // 2 if mode == "rotate_half" else L // int(mode)
    return np.where((j // H) % 2 == 0, j + H, j - H)


def check_proj(x, w, r1, r2, heads, mode, sl, out_dtype, what, y_gpu=None, r1_dev=None, r2_dev=None):
    """Run rope_proj_fwd on CPU tensors x (B,S,K) / w (N,K) / tables (or the
    device tables r1_dev/r2_dev, same values, any strides) and compare every
    output lane with the oracle within the bound above."""
    dt = CODE[x.dtype]
    B, S, K = x.shape
    N = w.shape[0]
    Dh = N // heads
    announce(f"{what}: x {tuple(x.shape)} w {tuple(w.shape)} {dt} heads={heads} {mode} slice={sl} out={out_dtype}")
    if y_gpu is None:
        y_gpu = rp.rope_proj_fwd(x.to(DEV), w.to(DEV), r1.to(DEV) if r1_dev is None else r1_dev,
                                 r2.to(DEV) if r2_dev is None else r2_dev, heads, mode, sl,
                                 out_dtype=TORCH[out_dtype])
        torch.cuda.synchronize()
    got = W.to_numpy_storage(y_gpu.cpu())
    xs = W.to_numpy_storage(x).reshape(B * S, K)
    ws = W.to_numpy_storage(w)
    t1, t2 = W.to_numpy_storage(r1), W.to_numpy_storage(r2)
    tdt = CODE[r1.dtype]
    y_shape = (B, S, heads, Dh)
    want = oracle.proj_rope(xs, ws, y_shape, dt, t1, t2, mode, sl, out_dtype, table_dtype=tdt)
    # the oracle's fp32 projection (empty slice, fp32 out) and sum |x w|
    none = np.zeros((1, 1, 1, 0), t1.dtype)
    p = oracle.proj_rope(xs, ws, y_shape, dt, none, none, mode, None, "f32").astype(np.float64)
    a = np.abs(_widen(xs, dt)) @ np.abs(_widen(ws, dt)).T
    dp = (K * 2.0 ** -23) * a.reshape(y_shape)
    bound = dp + 2.0 ** -126
    start, end = (0, 0) if sl is None else sl
    L = end - start
    if L:
        c = np.broadcast_to(_widen(t1, tdt), (B, S, heads, L))
        s = np.broadcast_to(_widen(t2, tdt), (B, S, heads, L))
        pj = _pair(L, mode)
        ps = p[..., start:end]
        dps = dp[..., start:end]
        bound[..., start:end] = (np.abs(c) * dps + np.abs(s) * dps[..., pj]
                                 + 1e-6 * (np.abs(ps * c) + np.abs(ps[..., pj] * s)) + 2.0 ** -126)
    gv, wv = _widen(got, out_dtype), _widen(want, out_dtype)
    if out_dtype != "f32":
        bound = bound + _spacing(np.abs(wv), out_dtype)
    assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
    err = np.abs(gv - wv)
    bad = err > bound
    exact = float(np.mean(got == want))
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} lanes beyond the bound; "
                           f"max err/bound {float(np.max(err / bound)):.3g}; first at {np.argwhere(bad)[0].tolist()}")
    return {"n": int(got.size), "exact_fraction": exact, "max_err_over_bound": float(np.max(err / bound))}


def _spacing(v, dt):
    """The gap between consecutive values of the 16-bit type at |v|: 2^(e-7)
    for bf16 (2^-133 below the normal range), numpy's spacing for fp16."""
    if dt == "bf16":
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
        return 2.0 ** (e - 7)
    return np.spacing(v.astype(np.float16)).astype(np.float64)


def _rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(TORCH[dt])


def _tables(B, S, H, L, dt, seed, per_batch=False, per_head=False, base=10000.0, mode="interleave"):
    """cos/sin of theta = p * base^(-2i/L) for position p = s (+ an offset
    per batch), pairs laid out for the mode; random per-head scaling when
    per_head (so that the head index of the table matters)."""
    g = torch.Generator().manual_seed(seed)
    Bt = B if per_batch else 1
    off = torch.randint(0, 60000, (Bt, 1), generator=g).double() if per_batch else torch.zeros(1, 1).double()
    pos = off + torch.arange(S).double()[None, :]
    i = torch.arange(L // 2).double()
    f = base ** (-2 * i / L)
    th = pos[..., None] * f                      # (Bt, S, L/2)
    j = np.arange(L)
    if mode == "interleave":
        lane_pair = j // 2
    elif mode == "rotate_half":
        lane_pair = j % (L // 2)
    else:
        Hc = L // int(mode)
        lane_pair = (j // (2 * Hc)) * Hc + j % Hc
    th = th[..., torch.from_numpy(lane_pair)]   # (Bt, S, L)
    c, s = torch.cos(th)[:, :, None, :], torch.sin(th)[:, :, None, :]
    if per_head:
        sc = 0.5 + torch.rand((1, 1, H, 1), generator=g, dtype=torch.float64)
        c, s = c * sc, s * sc
    return c.to(TORCH[dt]), s.to(TORCH[dt])


# (B, S, K, heads, Dh, slice, mode, dtype, out, table dtype, table layout)
CASES = [
    # the page's MLA Q projection: 128 heads of 192 lanes, qRopeDim 64 at the head's start, coefficient 2
    (1, 1024, 1536, 128, 192, (0, 64), "rotate_half", "bf16", "bf16", "bf16", "token"),
    (1, 1024, 1536, 128, 192, (0, 64), "interleave", "bf16", "bf16", "bf16", "token"),
    # the rope lanes at the end of the head (the other common MLA split)
    (2, 160, 512, 16, 192, (128, 192), "interleave", "bf16", "bf16", "bf16", "batch"),
    # fp32 output: the accumulator rotated and stored without a 16-bit rounding
    (2, 160, 512, 16, 192, (0, 64), "rotate_half", "bf16", "f32", "bf16", "batch"),
    # fp16 inputs, fp32 tables, coefficient 4
    (1, 300, 256, 8, 128, (0, 64), 4, "f16", "f16", "f32", "token"),
    # ragged M (300 tokens: a part-full block tile), heads of 64 with an odd head count (part-full N tile)
    (3, 100, 128, 3, 64, (16, 48), "interleave", "bf16", "bf16", "bf16", "batch"),
    # heads of 32 and of 96, per-head tables
    (1, 257, 192, 12, 32, (0, 32), "rotate_half", "bf16", "bf16", "f32", "head"),
    (2, 64, 320, 5, 96, (32, 96), "interleave", "f16", "f32", "f16", "head"),
    # whole head rotated (rotate_half over 128 lanes), one token
    (1, 1, 64, 4, 128, (0, 128), "rotate_half", "bf16", "bf16", "bf16", "token"),
    # odd start (pairs straddle 8-lane vectors), and a start off the 8-lane grid with a
    # rotate_half distance of 16 (partners lane by lane)
    (2, 33, 128, 4, 64, (3, 35), "interleave", "bf16", "bf16", "bf16", "batch"),
    (2, 33, 128, 4, 64, (4, 36), "rotate_half", "bf16", "f32", "bf16", "token"),
    (1, 70, 64, 2, 128, (20, 116), 6, "f16", "f16", "f16", "head"),
    # tables as views one element into wider buffers: rows off the 16-byte grid
    (2, 90, 192, 6, 64, (0, 64), "interleave", "bf16", "bf16", "bf16", "offset"),
    (1, 70, 128, 4, 96, (32, 96), "rotate_half", "f16", "f16", "f32", "offset"),
    # the plain projection (empty slice)
    (1, 512, 1536, 32, 192, None, "interleave", "bf16", "bf16", "bf16", "token"),
    # heads wider than a tile: MLA's compressed KV (512 lanes) with its K rope lanes (64) at the
    # end, one 576-lane head over three 192-lane tiles ([P4] section 3, kRopeDim), both modes
    (1, 300, 512, 1, 576, (512, 576), "rotate_half", "bf16", "bf16", "bf16", "token"),
    (2, 100, 256, 1, 576, (512, 576), "interleave", "bf16", "f32", "f32", "batch"),
    # a 256-lane head over two 128-lane tiles, per-head tables; a coefficient inside a
    # 384-lane head's second tile; an odd start in a wide head (lane by lane)
    (1, 130, 128, 3, 256, (0, 64), "rotate_half", "f16", "f16", "f16", "head"),
    (1, 90, 192, 2, 384, (192, 320), 4, "bf16", "bf16", "bf16", "token"),
    (2, 33, 64, 1, 512, (3, 35), "interleave", "bf16", "bf16", "bf16", "batch"),
    # square tiles, fp32 tables too wide to stage in LDS (64 lanes x 4 bytes): read per vector
    (2, 96, 256, 4, 128, (0, 64), "interleave", "bf16", "bf16", "f32", "token"),
    # square tiles' general epilogue: 256-lane rotate_half groups fit the tile but not a wave's 128 lanes
    (1, 40, 128, 2, 256, (0, 256), "rotate_half", "f16", "f16", "f16", "token"),
    # whole 192-lane heads rotated: groups straddle 256-lane tiles, so tiles of whole heads
    (1, 64, 256, 4, 192, (0, 192), "rotate_half", "bf16", "bf16", "bf16", "token"),
    # a group across lane 192 of a 384-lane head (no 192-lane tile holds it) inside the 256-lane square tile
    (1, 50, 128, 1, 384, (160, 224), "rotate_half", "bf16", "bf16", "bf16", "token"),
    # table rows staged in LDS at every row width (16 to 128 bytes) and batch layout: a wave's
    # loads step 64/2^crl tokens at a time, carrying into the next batch when s passes S
    # (13, 50, 300 tokens per batch), or one division per load when S is shorter than a step
    # (5, 6 and 20 tokens per batch); ragged M
    (40, 5, 128, 2, 128, (0, 64), "interleave", "bf16", "bf16", "bf16", "batch"),
    (50, 6, 128, 2, 64, (0, 64), "rotate_half", "bf16", "bf16", "bf16", "token"),
    (23, 13, 256, 3, 128, (64, 128), "rotate_half", "f16", "f16", "f16", "batch"),
    (3, 50, 128, 4, 64, (0, 32), "interleave", "bf16", "bf16", "f32", "batch"),
    (2, 300, 128, 2, 128, (0, 16), "interleave", "bf16", "bf16", "bf16", "batch"),
    (30, 20, 128, 2, 128, (0, 16), "interleave", "bf16", "bf16", "bf16", "batch"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}xK{c[2]}-h{c[3]}x{c[4]}-{c[5]}-{c[6]}-{c[7]}-{c[8]}-{c[9]}-{c[10]}"
                                            for c in CASES])
def test_projection_with_rotary_epilogue(case):
    B, S, K, H, Dh, sl, mode, dt, out, tdt, layout = case
    x, w, r1, r2, r1_dev, r2_dev = _case_inputs(case)
    info = check_proj(x, w, r1, r2, H, mode, sl, out, f"proj {case}", r1_dev=r1_dev, r2_dev=r2_dev)
    announce(f"  exact {info['exact_fraction']:.4f}, max err/bound {info['max_err_over_bound']:.3g}")
    # the bound is loose (first-order, worst case); most 16-bit lanes match
    # the oracle exactly (fp32 lanes differ in the last bits with the order)
    if out != "f32":
        assert info["exact_fraction"] > 0.9


def test_projection_cases_cover_every_kernel_and_epilogue():
    """The cases above run every projection kernel and epilogue: tiles of
    whole heads, and square tiles with the general epilogue, the vector
    epilogue (partners in the vector, or whole vectors away) with the table
    rows staged in LDS and read from the tables (rope_proj_launch_info)."""
    seen = set()
    for case in CASES:
        B, S, K, H, Dh, sl, mode, dt, out, tdt, layout = case
        x, w, r1, r2, r1_dev, r2_dev = _case_inputs(case)
        t1 = r1 if r1_dev is None else r1_dev
        t2 = r2 if r2_dev is None else r2_dev
        code = rp.MODES[mode] if isinstance(mode, str) else int(mode)
        tcode = rp._dtype_code(t1) if t1.numel() else 2
        st, plan = rp.raw_proj_launch_info(rp._dtype_code(torch.empty(0, dtype=TORCH[out])), rp._dtype_code(x),
                                           (B, S, H, Dh), K, t1.data_ptr() or None, tuple(t1.shape),
                                           tuple(t1.stride()), t2.data_ptr() or None, tuple(t2.shape),
                                           tuple(t2.stride()), tcode, code, sl)
        assert st == rp.ROPE_OK, (case, rp.last_error())
        seen.add((plan["kernel"], plan["epilogue"], plan["tables_in_lds"]))
    want = {("heads", None, False), ("square", "general", False), ("square", "vector", True),
            ("square", "vector", False), ("square", "vector_partner", True), ("square", "vector_partner", False)}
    assert want <= seen, sorted(want - seen)


def _case_inputs(case):
    """x, w, the CPU tables and (for the "offset" layout) device views of
    them, for one entry of CASES."""
    B, S, K, H, Dh, sl, mode, dt, out, tdt, layout = case
    x = _rand((B, S, K), dt, 11, 0.5)
    w = _rand((H * Dh, K), dt, 12, 0.05)
    L = 0 if sl is None else sl[1] - sl[0]
    r1_dev = r2_dev = None
    if L:
        r1, r2 = _tables(B, S, H, L, tdt, 13, per_batch=layout == "batch", per_head=layout == "head", mode=mode)
        if layout == "head":
            r1, r2 = r1.expand(-1, -1, H, -1).contiguous(), r2.expand(-1, -1, H, -1).contiguous()
        if layout == "offset":
            # device views one element into wider buffers: rows off the 16-byte grid
            def widen_by_one(t):
                wide = torch.zeros(t.shape[:-1] + (t.shape[-1] + 1,), dtype=t.dtype, device=DEV)
                wide[..., 1:] = t.to(DEV)
                return wide[..., 1:]
            r1_dev, r2_dev = widen_by_one(r1), widen_by_one(r2)
            assert r1_dev.data_ptr() % 16 != 0
    else:
        r1 = r2 = torch.zeros((1, 1, 1, 0), dtype=TORCH[tdt])
    return x, w, r1, r2, r1_dev, r2_dev


def test_plain_projection_matches_torch_matmul_closely():
    """With an empty slice the call is a plain projection; compared with
    torch's fp32 matmul of the same bf16 values (another accumulation order),
    the bf16 outputs agree within one unit in the last place."""
    announce("plain projection vs torch matmul")
    x = _rand((1, 512, 1536), "bf16", 21, 0.5)
    w = _rand((4096, 1536), "bf16", 22, 0.05)
    z = torch.zeros((1, 1, 1, 0), dtype=torch.bfloat16, device=DEV)
    y = rp.rope_proj_fwd(x.to(DEV), w.to(DEV), z, z, 32, "interleave", None)
    ref = (x.to(DEV).float().reshape(512, 1536) @ w.to(DEV).float().contiguous().T).to(torch.bfloat16)
    torch.cuda.synchronize()
    d = (y.reshape(512, 4096).float() - ref.float()).abs()
    tol = ref.float().abs() * 2.0 ** -7 + 1e-3
    assert bool((d <= tol).all()), float((d - tol).max())


def test_projection_is_deterministic_and_leaves_inputs_alone():
    announce("proj determinism")
    x = _rand((1, 300, 256), "bf16", 31).to(DEV)
    w = _rand((8 * 192, 256), "bf16", 32).to(DEV)
    r1, r2 = (t.to(DEV) for t in _tables(1, 300, 8, 64, "bf16", 33))
    x0, w0 = x.clone(), w.clone()
    a = rp.rope_proj_fwd(x, w, r1, r2, 8, "interleave", (0, 64))
    b = rp.rope_proj_fwd(x, w, r1, r2, 8, "interleave", (0, 64))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(x.view(torch.int16), x0.view(torch.int16)) and torch.equal(w.view(torch.int16), w0.view(torch.int16))


def test_projection_guard_bands():
    """The output written into the middle of a larger buffer: nothing
    outside its range changes (ragged M and a part-full N tile)."""
    announce("proj guard bands")
    B, S, K, H, Dh = 1, 77, 128, 3, 64
    x = _rand((B, S, K), "bf16", 41).to(DEV)
    w = _rand((H * Dh, K), "bf16", 42).to(DEV)
    r1, r2 = (t.to(DEV) for t in _tables(B, S, H, 32, "bf16", 43))
    n = B * S * H * Dh
    guard = 2048
    buf = torch.full((n + 2 * guard,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[guard:guard + n].view(B, S, H, Dh)
    rp.rope_proj_fwd(x, w, r1, r2, H, "interleave", (0, 32), out=out)
    torch.cuda.synchronize()
    assert bool((buf[:guard] == -7.0).all()) and bool((buf[guard + n:] == -7.0).all())
    check_proj(x.cpu(), w.cpu(), r1.cpu(), r2.cpu(), H, "interleave", (0, 32), "bf16", "guard", y_gpu=out)


def test_projection_errors():
    x = _rand((1, 8, 96), "bf16", 1).to(DEV)                  # K = 96: not a multiple of 64
    w = _rand((128, 96), "bf16", 2).to(DEV)
    r = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rp.RopeError, match="multiple of 64"):
        rp.rope_proj_fwd(x, w, r, r, 1, "interleave", (0, 64))
    x = _rand((1, 8, 64), "bf16", 1).to(DEV)
    w = _rand((2 * 100, 64), "bf16", 2).to(DEV)                # Dh = 100
    with pytest.raises(rp.RopeError, match="head dimension"):
        rp.rope_proj_fwd(x, w, r, r, 2, "interleave", (0, 64))
    w = _rand((128, 64), "bf16", 2).to(DEV)
    with pytest.raises(rp.RopeError, match="last dimension"):  # tables of the wrong length
        rp.rope_proj_fwd(x, w, r[..., :32], r[..., :32], 1, "interleave", (0, 64))
    empty = rp.rope_proj_fwd(x[:, :0], w, r, r, 1, "interleave", (0, 64))   # no tokens: a no-op
    assert empty.shape == (1, 0, 1, 128)


def test_projection_at_the_bench_shape():
    """The bench's workload: the MLA Q projection (K 1536 -> 128 heads x 192)
    over 4 x 4096 tokens with c3's rotation ([0,64), interleave, tables
    (1,4096,1,64)), every output lane against the oracle."""
    pw = W.PROJ_WORKLOADS["c3_proj"]
    wr = W.WORKLOADS[pw.rope]
    x, w = W.make_proj_inputs(pw)
    r1, r2 = W.make_tables(wr)
    B, S, H, Dh = pw.y_shape
    info = check_proj(x, w, r1, r2, H, wr.mode, wr.partial_slice, "bf16", "c3_proj")
    announce(f"  exact {info['exact_fraction']:.4f}, max err/bound {info['max_err_over_bound']:.3g}")
    assert info["n"] == B * S * H * Dh and info["exact_fraction"] > 0.9
