"""Seeded synthetic inputs for in-place partial RoPE.

This module is shared by the tests, the bench and the smoke check. It holds
the shapes, value distributions and cos/sin table recipes of the workloads and
nothing of the rotation itself: it never applies r1/r2 to x. The HIP path and
the CPU oracle each receive the tensors built here as plain inputs.

Table recipe (the cos/sin tables are inputs of the operation, not part of it):
"ANE实战RoPE位置编码在MIL中的纯ANE实现", section 第一步 (the cos/sin table
is precomputed on the host, θ = p / base^(2i/h) for position p and pair i,
and each value is written to both lanes of its pair). For rotate_half the
value of pair i goes to lanes i and i + L/2 instead. Angles, cos and sin are
evaluated in fp64 and converted to the table's storage type by torch, which
rounds to nearest even through fp32 (so a 16-bit table value is rounded
twice).

Random tables with no structure (the single-op example of "CANN ops-transformer
算子详解：inplace_partial_rotary_mul 原地部分旋转位置编码", section 调用说明,
draws r1/r2 from a normal distribution) exercise the per-lane reading of the
formula.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    """One synthetic partial-RoPE case.

    x_shapes: one or more (B,S,N,D) tensors rotated with the same tables, in
    order, on one stream (the GQA Q and K of one attention layer, for example).
    """
    name: str
    x_shapes: tuple
    dtype: str
    partial_slice: tuple
    mode: object                    # "interleave", "rotate_half" or an int rotary coefficient
    table_shape: tuple
    seed: int
    std: float = 1.0
    base: float = 10000.0
    directions: tuple = ("fwd",)
    position_offsets: bool = False  # per-batch position offsets in [0, 65536)
    table_kind: str = "rope"        # "rope" (cos/sin recipe) or "random"
    table_dtype: str | None = None  # defaults to dtype
    note: str = field(default="", compare=False)

    @property
    def L(self) -> int:
        return int(self.partial_slice[1]) - int(self.partial_slice[0])

    @property
    def tdtype(self) -> str:
        return self.table_dtype or self.dtype

    def rows(self, k: int = 0) -> int:
        B, S, N, _ = self.x_shapes[k]
        return B * S * N

    def rotated_elements(self) -> int:
        return sum(B * S * N * self.L for (B, S, N, _) in self.x_shapes)

    def table_bytes(self) -> int:
        n = 1
        for v in self.table_shape:
            n *= int(v)
        return 2 * n * ESIZE[self.tdtype]

    def algorithmic_bytes(self, k: int | None = None) -> int:
        """Slice read once + slice written once + r1 and r2 read once, per launch
        (for tensor k), or summed over the tensors when k is None."""
        ks = range(len(self.x_shapes)) if k is None else [k]
        total = 0
        for i in ks:
            B, S, N, _ = self.x_shapes[i]
            total += 2 * B * S * N * self.L * ESIZE[self.dtype] + self.table_bytes()
        return total


W = Workload
WORKLOADS: dict[str, Workload] = {
    # Forward and backward, interleave, fp32; the empty-slice and B=0 cases are
    # derived from it in the tests.
    "c0": W("c0", ((1, 16, 2, 64),), "f32", (0, 32), "interleave", (1, 16, 1, 32),
            seed=0, directions=("fwd", "bwd"),
            note="small fp32 interleave case (1,16,2,64), slice [0,32)"),
    # MHA 12 heads, head dim 64 (the attention shape of a 12-layer 109M model).
    "c1": W("c1", ((8, 256, 12, 64),), "f16", (0, 64), "interleave", (1, 256, 1, 64),
            seed=1, directions=("fwd", "bwd"),
            note="MHA 12 heads HD 64, fp16, full slice"),
    # GQA Q (16 heads) and K (8 heads), head dim 128, rotate_half.
    "c2": W("c2", ((32, 256, 16, 128), (32, 256, 8, 128)), "bf16", (0, 128), "rotate_half",
            (1, 256, 1, 128), seed=2, directions=("fwd",),
            note="GQA Q/K 16/8 heads HD 128, bf16, rotate_half"),
    # MLA-style partial rope: first 64 of 192 lanes.
    "c3": W("c3", ((4, 4096, 128, 192),), "bf16", (0, 64), "interleave", (1, 4096, 1, 64),
            seed=3, directions=("fwd", "bwd"),
            note="MLA-style rope on lanes [0,64) of 192, bf16"),
    # Backward of a long-context shard: per-batch position offsets, base 5e5.
    "c4": W("c4", ((16, 8192, 32, 128),), "bf16", (32, 96), "interleave", (16, 8192, 1, 64),
            seed=4, std=1e-2, base=500000.0, directions=("bwd", "fwd"), position_offsets=True,
            note="long-context shard, per-batch offsets, slice [32,96), bf16"),
    # Single-op example shape with random (non-unit, non-duplicated) tables.
    "p1ex": W("p1ex", ((2, 32, 8, 128),), "f16", (0, 64), "interleave", (2, 32, 1, 64),
              seed=11, directions=("fwd", "bwd"), table_kind="random",
              note="single-op example shape, random BS1D tables"),
}
# A single K head (multi-query attention) at 4096 positions shared by the
# batch: each position's 64 pairs of cos/sin serve 512 bytes of x.
WORKLOADS["mqa_k"] = W("mqa_k", ((32, 4096, 1, 128),), "bf16", (0, 128), "rotate_half", (1, 4096, 1, 128),
                       seed=16, directions=("fwd", "bwd"),
                       note="MQA K (one head, HD 128) at 4096 positions, rotate_half, bf16")
# The GQA Q and K of one tensor-parallel rank (a 32/8-head layer split over
# 8 GPUs: 4 Q heads and 1 K head) at 4096 positions shared by the batch.
WORKLOADS["tp_qk"] = W("tp_qk", ((32, 4096, 4, 128), (32, 4096, 1, 128)), "bf16", (0, 128), "rotate_half",
                       (1, 4096, 1, 128), seed=17, directions=("fwd",),
                       note="GQA Q/K of one of 8 tensor-parallel ranks (4 + 1 heads, HD 128) at 4096 positions, "
                            "rotate_half, bf16")
# MLA's rope part with the page's coefficient 4 (two groups of two 16-lane parts).
WORKLOADS["c3_coeff4"] = replace(WORKLOADS["c3"], name="c3_coeff4", mode=4, seed=15,
                                 note="MLA-style rope on lanes [0,64) of 192, rotary coefficient 4, bf16")
WORKLOADS["c4_f32"] = replace(WORKLOADS["c4"], name="c4_f32", dtype="f32",
                              note="long-context shard, fp32 rerun")
# The page's mixed-precision case at the long-context shape: bf16 dx, fp32 tables.
WORKLOADS["c4_t32"] = replace(WORKLOADS["c4"], name="c4_t32", table_dtype="f32",
                              note="long-context shard, bf16 dx with fp32 tables")
# rotate_half layouts measured from HBM (c2 itself fits the 256 MB cache):
# the GQA Q layout of c2 at 4096 positions (whole head, halves of whole
# 128-byte lines), and partial slices whose halves are 64 and 32 bytes.
WORKLOADS["c2_s4096"] = W("c2_s4096", ((32, 4096, 16, 128),), "bf16", (0, 128), "rotate_half",
                          (1, 4096, 1, 128), seed=12, directions=("fwd", "bwd"),
                          note="GQA Q layout (16 heads, HD 128) at 4096 positions, rotate_half, bf16")
WORKLOADS["rh_64of128"] = W("rh_64of128", ((16, 4096, 32, 128),), "bf16", (64, 128), "rotate_half",
                            (1, 4096, 1, 64), seed=13, directions=("fwd", "bwd"),
                            note="rotate_half on lanes [64,128) of 128, bf16")
WORKLOADS["rh_32of128"] = W("rh_32of128", ((16, 4096, 40, 128),), "bf16", (0, 32), "rotate_half",
                            (1, 4096, 1, 32), seed=14, directions=("fwd", "bwd"),
                            note="rotate_half on lanes [0,32) of 128, 40 heads, bf16")


@dataclass(frozen=True)
class ProjWorkload:
    """A head projection whose result is rotated (the Q projection and RoPE
    stages of "ascend-transformer-boost 的 MlaPreprocessOperation：MLA 预处理
    四阶段融合算子深度解析", section 3): x (B*S, K) ~ N(0, 1) (the normalised
    latent the page's projection takes), w (H*Dh, K) ~ N(0, 1/K) (so each
    output lane is ~N(0, 1)), both rounded to `dtype`; the slice, mode and
    tables of the rotation workload `rope` (whose x shape is (B, S, H, Dh))."""
    name: str
    rope: str
    K: int
    seed: int
    note: str = field(default="", compare=False)

    @property
    def y_shape(self):
        return WORKLOADS[self.rope].x_shapes[0]

    def flops(self) -> int:
        B, S, H, Dh = self.y_shape
        return 2 * B * S * H * Dh * self.K


PROJ_WORKLOADS: dict[str, ProjWorkload] = {
    "c3_proj": ProjWorkload("c3_proj", "c3", 1536, 18,
                            note="MLA Q projection, K 1536 -> 128 heads x 192, over c3's 4 x 4096 tokens, "
                                 "rope lanes [0,64) interleave"),
}


def make_proj_inputs(p: ProjWorkload) -> tuple[torch.Tensor, torch.Tensor]:
    """x (B, S, K) and w (H*Dh, K) CPU tensors in the rotation workload's dtype."""
    w0 = WORKLOADS[p.rope]
    B, S, H, Dh = p.y_shape
    g = generator(p.seed)
    x = torch.randn((B, S, p.K), generator=g).to(TORCH_DTYPES[w0.dtype])
    w = (torch.randn((H * Dh, p.K), generator=g) * (1.0 / np.sqrt(p.K))).to(TORCH_DTYPES[w0.dtype])
    return x, w


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_x(w: Workload, k: int = 0, shape=None, seed=None) -> torch.Tensor:
    """x (or dx) ~ N(0, std^2), drawn in fp32 and rounded (RNE) to the
    storage type; a CPU tensor. Tensor k of the workload uses seed + 1000*k."""
    shape = tuple(w.x_shapes[k] if shape is None else shape)
    seed = w.seed + 1000 * k if seed is None else seed
    g = generator(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.std != 1.0:
        x.mul_(w.std)
    return x.to(TORCH_DTYPES[w.dtype])


def make_x_device(shape, dtype: str, seed: int, std: float = 1.0, device="cuda",
                  chunk: int = 1 << 28) -> torch.Tensor:
    """A large x ~ N(0, std^2) drawn on the device, chunk by chunk, from a
    seeded device generator (for tensors too large to draw on the host); the
    values are rounded (RNE) to the storage type like make_x's. Both sides of
    a comparison read their inputs back from this tensor."""
    x = torch.empty(tuple(shape), dtype=TORCH_DTYPES[dtype], device=device)
    flat = x.view(-1)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        v = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        flat[i:i + n].copy_(v)
        del v
    return x


def positions(w: Workload) -> np.ndarray:
    """Positions p for every (table-batch, s): shape (Bt, S) int64.
    With position_offsets, batch b uses p = offset_b + s, offset_b ~ U{0..65535}."""
    Bt, S = int(w.table_shape[0]), int(w.table_shape[1])
    s = np.arange(S, dtype=np.int64)[None, :]
    if w.position_offsets:
        g = generator(w.seed + 7)
        off = torch.randint(0, 65536, (Bt,), generator=g, dtype=torch.int64).numpy()
    else:
        off = np.zeros(Bt, dtype=np.int64)
    return off[:, None] + s


def rope_angles(w: Workload) -> np.ndarray:
    """θ for every (table-batch, s, lane j): shape (Bt, S, L) fp64, laid out
    for the workload's pairing (pair-duplicated or repeated halves)."""
    L = w.L
    half = L // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(w.base), -2.0 * i / float(L))          # base^(-2i/L)
    theta = positions(w).astype(np.float64)[:, :, None] * inv_freq[None, None, :]
    if w.mode == "interleave":
        return np.repeat(theta, 2, axis=-1)        # lanes 2i and 2i+1 share θ_i
    if w.mode == "rotate_half":
        return np.concatenate([theta, theta], axis=-1)  # lanes i and i+L/2 share θ_i
    # rotary coefficient c: pair i = g*H + k (H = L/c) at lanes g*2H + k and g*2H + k + H
    H = L // int(w.mode)
    out = np.empty(theta.shape[:2] + (L,))
    for i in range(half):
        g, k = divmod(i, H)
        out[..., g * 2 * H + k] = out[..., g * 2 * H + k + H] = theta[..., i]
    return out


def make_tables(w: Workload) -> tuple[torch.Tensor, torch.Tensor]:
    """(r1, r2) = (cos, sin) CPU tensors of w.table_shape in the table type."""
    tshape = tuple(int(v) for v in w.table_shape)
    tt = TORCH_DTYPES[w.tdtype]
    if w.table_kind == "random":
        g = generator(w.seed + 31)
        r1 = torch.randn(tshape, generator=g, dtype=torch.float32).to(tt)
        r2 = torch.randn(tshape, generator=g, dtype=torch.float32).to(tt)
        return r1, r2
    theta = rope_angles(w)                          # (Bt, S, L)
    Bt, S, _, L = tshape
    assert theta.shape == (Bt, S, L), (theta.shape, tshape)
    cos = torch.from_numpy(np.cos(theta)).reshape(tshape).to(tt)
    sin = torch.from_numpy(np.sin(theta)).reshape(tshape).to(tt)
    return cos.contiguous(), sin.contiguous()


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor as a numpy array in storage form: float32 for fp32 data,
    raw uint16 bit patterns for fp16/bf16 (shares memory where it can)."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.uint16).numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def from_numpy_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "f32":
        return t
    return t.view(TORCH_DTYPES[dtype])


def sample_rows(total_rows: int, n: int, seed: int) -> np.ndarray:
    """n sorted distinct flat row indices including the first and last rows
    (fewer only if 3n random draws repeat too often), drawn uniformly
    without replacement. Up to 2^24 rows from a seeded permutation; above,
    the first distinct values of seeded uniform draws, so that no
    permutation of billions of rows is built on the host."""
    if total_rows <= n:
        return np.arange(total_rows, dtype=np.int64)
    g = generator(seed + 99)
    k = max(n - 2, 0)
    if total_rows <= 1 << 24:
        pick = torch.randperm(total_rows, generator=g)[:k].numpy().astype(np.int64)
    else:
        draws = torch.randint(0, total_rows, (3 * max(k, 1),), generator=g, dtype=torch.int64).numpy()
        uniq, first = np.unique(draws, return_index=True)
        pick = uniq[np.argsort(first)][:k]
    return np.unique(np.concatenate([pick, [0, total_rows - 1]]).astype(np.int64))
