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

import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def expanded_tables(r, x_shape, rows: np.ndarray, L: int) -> np.ndarray:
    """fp64 table values for the listed flat rows: (len(rows), L). `r` is a
    torch table or its fp64 numpy copy."""
    B, S, N, _ = x_shape
    n = rows % N
    s = (rows // N) % S
    b = rows // (N * S)
    rv = r if isinstance(r, np.ndarray) else r.double().numpy()
    idx = tuple(np.zeros_like(rows) if rv.shape[k] == 1 else v for k, v in enumerate((b, s, n)))
    return rv[idx[0], idx[1], idx[2], :]


def host_threads() -> int:
    """Threads for host-side checking: the cores this process may use, at
    most 16 (a GPU machine's CPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _row_chunks(total: int, per: int):
    return [(a, min(total, a + per)) for a in range(0, total, per)]


def oracle_all_rows(x_flat: np.ndarray, x_shape, dtype: str, r1: torch.Tensor, r2: torch.Tensor, mode, sl,
                    direction: str) -> np.ndarray:
    """The oracle on every row of a whole tensor (storage rows (B*S*N, D)),
    the rows split into contiguous blocks over the host's cores; each block
    is one call of the unchanged oracle (which releases the interpreter
    while it runs)."""
    want = np.array(x_flat, copy=True)
    t1, t2 = W.to_numpy_storage(r1), W.to_numpy_storage(r2)
    tdt = TDT[r1.dtype]

    def work(ab):
        a, b = ab
        oracle.rope_rows(want[a:b], x_shape, dtype, t1, t2, mode, sl, direction,
                         rows=np.arange(a, b, dtype=np.int64), table_dtype=tdt)

    total = want.shape[0]
    n = host_threads()
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(work, _row_chunks(total, max(1, -(-total // (4 * n))))))
    return want


def _pair_lane(L: int, mode) -> np.ndarray:
    """p(j) for the slice lanes j in [0, L)."""
    j = np.arange(L)
    if mode == "interleave":
        return j ^ 1
    if mode == "rotate_half":
        return np.where(j < L // 2, j + L // 2, j - L // 2)
    H = L // int(mode)
    return np.where((j // H) % 2 == 0, j + H, j - H)


def _f32_lanes(got, want, x_in, rows, rv1, rv2, x_shape, mode, direction, sl, what) -> dict:
    """compare()'s fp32 bar for a block of rows, evaluated only on the lanes
    whose bits differ from the oracle's (a lane with the oracle's bits is
    within any bound)."""
    start, end = sl
    L = end - start
    g, w = got[:, start:end], want[:, start:end]
    diff = g.view(np.uint32) != w.view(np.uint32)
    info = {"n": int(g.size), "exact": int(g.size - np.count_nonzero(diff)), "max_ulp": 0}
    ri, li = np.nonzero(diff)
    if ri.size == 0:
        return info
    gv, wv = g[ri, li].astype(np.float64), w[ri, li].astype(np.float64)
    nan = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), nan), f"{what}: NaN pattern differs"
    inf = np.isinf(wv)
    assert np.array_equal(gv[inf], wv[inf]), f"{what}: infinite lanes differ"
    B, S, N, _ = x_shape
    fr = rows[ri]
    n_, s_, b_ = fr % N, (fr // N) % S, fr // (N * S)

    def table(rv, lanes):
        idx = [np.zeros_like(fr) if rv.shape[k] == 1 else v for k, v in enumerate((b_, s_, n_))]
        return rv[idx[0], idx[1], idx[2], lanes]

    pj = _pair_lane(L, mode)[li]
    xj = x_in[ri, start + li].astype(np.float64)
    xp = x_in[ri, start + pj].astype(np.float64)
    c = table(rv1, li)
    sk = table(rv2, li if direction == "fwd" else pj)
    with np.errstate(invalid="ignore", over="ignore"):
        bound = 1e-6 * (np.abs(xj * c) + np.abs(xp * sk)) + 2.0 ** -126
        err = np.abs(gv - wv)
    fin = ~nan & np.isfinite(wv)
    bad = np.count_nonzero(fin & (err > bound))
    info["max_ulp"] = int(ulp_distance(g[ri, li][fin], w[ri, li][fin], "f32").max(initial=0))
    assert bad == 0, (f"{what}: {bad} fp32 lanes beyond the 1e-6 normwise bound; "
                      f"max err/bound {np.max(err[fin] / bound[fin]):.3g}")
    return info


def compare_all_rows(got: np.ndarray, want: np.ndarray, x_in: np.ndarray, r1, r2, x_shape, dtype: str, mode,
                     direction: str, sl, what: str, chunk_rows: int = 1 << 17) -> dict:
    """compare()'s bars over every row of a whole tensor (storage rows
    (B*S*N, D)), in blocks of rows checked in parallel. Lanes outside the
    slice must equal the input's bytes. 16-bit results equal to the
    oracle's bytes pass at once; otherwise a block goes through compare().
    fp32 lanes are held to the normwise bound wherever their bits differ
    from the oracle's."""
    start, end = sl
    total, D = got.shape
    bits = (lambda a: a.view(np.uint32)) if dtype == "f32" else (lambda a: a)
    for part in (np.s_[:, :start], np.s_[:, end:]):
        assert np.array_equal(bits(got)[part], bits(x_in)[part]), f"{what}: lanes outside the slice changed"
    n = total * (end - start)
    if dtype != "f32" and np.array_equal(got[:, start:end], want[:, start:end]):
        return {"n": n, "exact": n, "max_ulp": 0, "rows": total}
    rv1, rv2 = r1.double().numpy(), r2.double().numpy()
    L = end - start

    def one(ab):
        a, b = ab
        rows = np.arange(a, b, dtype=np.int64)
        tag = f"{what} rows [{a},{b})"
        if dtype == "f32":
            return _f32_lanes(got[a:b], want[a:b], x_in[a:b], rows, rv1, rv2, x_shape, mode, direction, sl, tag)
        if np.array_equal(got[a:b, start:end], want[a:b, start:end]):
            return {"n": (b - a) * L, "exact": (b - a) * L, "max_ulp": 0}
        return compare(got[a:b], want[a:b], x_in[a:b], expanded_tables(rv1, x_shape, rows, L),
                       expanded_tables(rv2, x_shape, rows, L), dtype, mode, direction, sl, tag)

    with ThreadPoolExecutor(min(8, host_threads())) as ex:
        infos = list(ex.map(one, _row_chunks(total, chunk_rows)))
    return {"n": sum(i["n"] for i in infos), "exact": sum(i["exact"] for i in infos),
            "max_ulp": max(i["max_ulp"] for i in infos), "rows": total}


def check_tensor(got: torch.Tensor, x_in: torch.Tensor, want: torch.Tensor, r1: torch.Tensor, r2: torch.Tensor,
                 mode, sl, direction: str, what: str) -> dict:
    """compare() for whole CPU tensors (B,S,N,D): the result, the input it
    was computed from and the oracle's result, with the tables that
    broadcast against them."""
    dtype = TDT[x_in.dtype]
    D = x_in.shape[-1]
    flat = lambda t: np.ascontiguousarray(W.to_numpy_storage(t.contiguous())).reshape(-1, D)
    return compare_all_rows(flat(got), flat(want), flat(x_in), r1, r2, tuple(x_in.shape), dtype, mode,
                            direction, sl, what)


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
    if sample is None:
        got = W.to_numpy_storage(x_dev.cpu()).reshape(total, D)
        x_flat = W.to_numpy_storage(x_cpu).reshape(total, D)
        want = oracle_all_rows(x_flat, tuple(x_cpu.shape), dtype, r1, r2, mode, sl, direction)
        return compare_all_rows(got, want, x_flat, r1, r2, tuple(x_cpu.shape), dtype, mode, direction, sl, what)
    rows = W.sample_rows(total, sample, seed)
    rows_t = torch.from_numpy(rows).to(device)
    got = W.to_numpy_storage(x_dev.view(total, D).index_select(0, rows_t).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x_cpu).reshape(total, D)[rows])
    want = oracle_rows(x_rows, x_cpu.shape, dtype, r1, r2, mode, sl, direction, rows)
    L = sl[1] - sl[0]
    c = expanded_tables(r1, x_cpu.shape, rows, L)
    s = expanded_tables(r2, x_cpu.shape, rows, L)
    info = compare(got, want, x_rows, c, s, dtype, mode, direction, sl, what)
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
    if sample is None:
        got = W.to_numpy_storage(y_dev.cpu()).reshape(total, D)
        x_flat = W.to_numpy_storage(x_cpu).reshape(total, D)
        want = oracle_all_rows(x_flat, tuple(x_cpu.shape), dtype, r1, r2, mode, sl, direction)
        return compare_all_rows(got, want, x_flat, r1, r2, tuple(x_cpu.shape), dtype, mode, direction, sl, what)
    rows = W.sample_rows(total, sample, seed)
    rows_t = torch.from_numpy(rows).to(device)
    got = W.to_numpy_storage(y_dev.view(total, D).index_select(0, rows_t).cpu())
    x_rows = np.ascontiguousarray(W.to_numpy_storage(x_cpu).reshape(total, D)[rows])
    want = oracle_rows(x_rows, x_cpu.shape, dtype, r1, r2, mode, sl, direction, rows)
    L = sl[1] - sl[0]
    c = expanded_tables(r1, x_cpu.shape, rows, L)
    s = expanded_tables(r2, x_cpu.shape, rows, L)
    info = compare(got, want, x_rows, c, s, dtype, mode, direction, sl, what)
    # every row's lanes outside the slice: x's bytes
    assert torch.equal(_bits(y_dev[..., : sl[0]]), _bits(x_dev[..., : sl[0]])), f"{what}: head lanes"
    assert torch.equal(_bits(y_dev[..., sl[1]:]), _bits(x_dev[..., sl[1]:])), f"{what}: tail lanes"
    return info
