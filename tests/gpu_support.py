"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same seeded inputs, and compare them.

The bars: 16-bit data within 1 ulp of the oracle (the kernels are designed to
match it bit for bit, and the tests report any difference); fp32 data within
1e-6 of the size of the two terms, |x_j c| + |x_p s| (normwise, so that
cancellation between the terms does not make the bound meaningless), plus
2^-126; NaN on the same lanes and infinities equal; lanes outside the slice
bit-identical.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import transformer_positional_encoding_amd as rp
import workloads as W


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Distance in units in the last place between two storage arrays,
    through the ordered-integer map of their bit patterns."""
    if dtype == "f32":
        ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
        ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
        top = 1 << 31
    else:
        ia = np.asarray(a, np.uint16).astype(np.int64)
        ib = np.asarray(b, np.uint16).astype(np.int64)
        ia = np.where(ia >= 1 << 15, ia - (1 << 16), ia)
        ib = np.where(ib >= 1 << 15, ib - (1 << 16), ib)
        top = 1 << 15

    def ordered(i):
        return np.where(i < 0, -top - i, i)

    return np.abs(ordered(ia) - ordered(ib))


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    return W.from_numpy_storage(np.ascontiguousarray(a), dtype).double().numpy()


def term_scale(x: np.ndarray, c: np.ndarray, s: np.ndarray, mode: str, direction: str) -> np.ndarray:
    """|x_j c_j| + |x_p(j) s_k| for the slice lanes (fp64), where k = j
    forward and k = p(j) backward; x, c, s are fp64 arrays (..., L)."""
    L = x.shape[-1]
    if mode == "interleave":
        perm = np.arange(L) ^ 1
    elif mode == "rotate_half":
        perm = np.concatenate([np.arange(L // 2) + L // 2, np.arange(L // 2)])
    else:   # rotary coefficient c: parts of H = L/c lanes, part 2k paired with 2k+1
        H = L // int(mode)
        j = np.arange(L)
        perm = np.where((j // H) % 2 == 0, j + H, j - H)
    sk = s if direction == "fwd" else s[..., perm]
    return np.abs(x * c) + np.abs(x[..., perm] * sk)


def compare(got: np.ndarray, want: np.ndarray, x_in: np.ndarray, c: np.ndarray, s: np.ndarray,
            dtype: str, mode: str, direction: str, sl, what: str) -> dict:
    """Compare storage arrays of rows (..., D); c/s are the fp64 tables
    expanded to (..., L). Raises AssertionError with a summary on failure."""
    start, end = sl
    got = np.asarray(got)
    want = np.asarray(want)
    x_in = np.asarray(x_in)
    # outside the slice: the input bytes, untouched
    for part in (np.s_[..., :start], np.s_[..., end:]):
        assert got[part].tobytes() == x_in[part].tobytes(), f"{what}: lanes outside the slice changed"
    g, w = got[..., start:end], want[..., start:end]
    gv, wv = widen(g, dtype), widen(w, dtype)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan), f"{what}: NaN pattern differs"
    inf = np.isinf(wv)   # an infinite result must match exactly (1 ulp from the largest finite is not inf)
    assert np.array_equal(gv[inf], wv[inf]), f"{what}: infinite lanes differ"
    info = {"n": int(g.size), "exact": int(np.sum(g.view(np.uint32 if dtype == 'f32' else np.uint16)
                                                 == w.view(np.uint32 if dtype == 'f32' else np.uint16)))}
    if dtype == "f32":
        xv = widen(x_in[..., start:end], dtype)
        with np.errstate(invalid="ignore", over="ignore"):   # NaN/inf lanes are excluded below
            bound = 1e-6 * term_scale(xv, c, s, mode, direction) + 2.0 ** -126
            err = np.abs(gv - wv)
        fin = ~nan & np.isfinite(wv)
        bad = np.nonzero(fin & (err > bound))
        info["max_ulp"] = int(ulp_distance(g[fin], w[fin], dtype).max(initial=0))
        assert bad[0].size == 0, (f"{what}: {bad[0].size} fp32 lanes beyond the 1e-6 normwise bound; "
                                  f"max err/bound {np.max(err[fin] / bound[fin]):.3g}")
    else:
        d = ulp_distance(g[~nan], w[~nan], dtype)
        info["max_ulp"] = int(d.max(initial=0))
        assert info["max_ulp"] <= 1, f"{what}: {int(np.sum(d > 1))} lanes more than 1 ulp from the oracle"
    return info


TDT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def oracle_rows(x_rows: np.ndarray, x_shape, dtype: str, r1: torch.Tensor, r2: torch.Tensor, mode: str,
                sl, direction: str, rows) -> np.ndarray:
    out = np.array(x_rows, copy=True)
    oracle.rope_rows(out, x_shape, dtype, W.to_numpy_storage(r1), W.to_numpy_storage(r2), mode, sl,
                     direction, rows=rows, table_dtype=TDT[r1.dtype])
    return out


def expanded_tables(r: torch.Tensor, x_shape, rows: np.ndarray, L: int) -> np.ndarray:
    """fp64 table values for the listed flat rows: (len(rows), L)."""
    B, S, N, _ = x_shape
    n = rows % N
    s = (rows // N) % S
    b = rows // (N * S)
    rv = r.double().numpy()
    idx = tuple(np.zeros_like(rows) if r.shape[k] == 1 else v for k, v in enumerate((b, s, n)))
    return rv[idx[0], idx[1], idx[2], :]


def run_and_check(x_cpu: torch.Tensor, r1: torch.Tensor, r2: torch.Tensor, mode: str, sl, direction: str,
                  what: str, sample: int | None = None, seed: int = 0, device="cuda",
                  r1_dev: torch.Tensor | None = None, r2_dev: torch.Tensor | None = None) -> dict:
    """Copy inputs to the GPU, run the entry point, compare with the oracle
    (on every row, or on `sample` rows drawn with `seed`)."""
    dtype = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x_cpu.dtype]
    announce(f"{what} shape={tuple(x_cpu.shape)} {dtype} {mode} {direction} slice={sl}")
    x_dev = x_cpu.to(device)
    r1d = r1.to(device) if r1_dev is None else r1_dev
    r2d = r2.to(device) if r2_dev is None else r2_dev
    fn = rp.rope_partial_fwd_inplace if direction == "fwd" else rp.rope_partial_bwd_inplace
    fn(x_dev, r1d, r2d, mode, sl)
    torch.cuda.synchronize()
    B, S, N, D = x_cpu.shape
    total = B * S * N
    rows = np.arange(total, dtype=np.int64) if sample is None else W.sample_rows(total, sample, seed)
    rows_t = torch.from_numpy(rows).to(device)
    got = W.to_numpy_storage(x_dev.view(total, D).index_select(0, rows_t).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x_cpu).reshape(total, D)[rows])
    want = oracle_rows(x_rows, x_cpu.shape, dtype, r1, r2, mode, sl, direction, rows)
    L = sl[1] - sl[0]
    c = expanded_tables(r1, x_cpu.shape, rows, L)
    s = expanded_tables(r2, x_cpu.shape, rows, L)
    info = compare(got, want, x_rows, c, s, dtype, mode, direction, sl, what)
    if sample is not None:
        # every row's lanes outside the slice, checked on the device
        x0 = x_cpu.to(device)
        assert torch.equal(_bits(x_dev[..., : sl[0]]), _bits(x0[..., : sl[0]])), f"{what}: head lanes changed"
        assert torch.equal(_bits(x_dev[..., sl[1]:]), _bits(x0[..., sl[1]:])), f"{what}: tail lanes changed"
        del x0
    return info


def _bits(t: torch.Tensor) -> torch.Tensor:
    t = t.contiguous()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def run_out_and_check(x_cpu, r1, r2, mode, sl, direction, what, sample=None, seed=0, y_dev=None, x_dev=None,
                      device="cuda", r1_dev=None, r2_dev=None):
    """Run the out-of-place entry point from a fresh device copy of x into
    y_dev (default: a new tensor) and compare with the oracle on every row or
    on `sample` rows; x must be unchanged."""
    dtype = TDT[x_cpu.dtype]
    announce(f"{what} out-of-place shape={tuple(x_cpu.shape)} {dtype} {mode} {direction} slice={sl}")
    x_dev = x_cpu.to(device) if x_dev is None else x_dev
    y_dev = torch.full_like(x_dev, float("nan")) if y_dev is None else y_dev
    fn = rp.rope_partial_fwd_out if direction == "fwd" else rp.rope_partial_bwd_out
    fn(y_dev, x_dev, r1.to(device) if r1_dev is None else r1_dev, r2.to(device) if r2_dev is None else r2_dev,
       mode, sl)
    torch.cuda.synchronize()
    B, S, N, D = x_cpu.shape
    total = B * S * N
    assert torch.equal(_bits(x_dev), _bits(x_cpu.to(device))), f"{what}: the input changed"
    rows = np.arange(total, dtype=np.int64) if sample is None else W.sample_rows(total, sample, seed)
    rows_t = torch.from_numpy(rows).to(device)
    got = W.to_numpy_storage(y_dev.view(total, D).index_select(0, rows_t).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x_cpu).reshape(total, D)[rows])
    want = oracle_rows(x_rows, x_cpu.shape, dtype, r1, r2, mode, sl, direction, rows)
    L = sl[1] - sl[0]
    c = expanded_tables(r1, x_cpu.shape, rows, L)
    s = expanded_tables(r2, x_cpu.shape, rows, L)
    info = compare(got, want, x_rows, c, s, dtype, mode, direction, sl, what)
    if sample is not None:
        # every row's lanes outside the slice: x's bytes
        assert torch.equal(_bits(y_dev[..., : sl[0]]), _bits(x_dev[..., : sl[0]])), f"{what}: head lanes"
        assert torch.equal(_bits(y_dev[..., sl[1]:]), _bits(x_dev[..., sl[1]:])), f"{what}: tail lanes"
    return info
