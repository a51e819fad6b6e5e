"""CPU oracle for in-place partial RoPE (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path.

The arithmetic lives in ``rope_oracle.c`` (plain C, built with gcc and no
floating-point contraction); this module only marshals numpy arrays into it.
The operation follows two pages:

* "CANN ops-transformer 算子详解：inplace_partial_rotary_mul 原地部分旋转位置编码"
  -- section 计算公式 (the interleave formula), section 约束说明 (slice and
  broadcast rules), the mixed-precision paragraph of the tiling/kernel section
  (fp32 compute, round-to-nearest-even write-back), section 自动微分说明
  (backward = gradient of x only).
* "ANE实战RoPE位置编码在MIL中的纯ANE实现" -- section 先搞懂RoPE (the
  rotate_half pairing (i, i+h/2)) and the backward section (inverse rotation).

Storage convention: fp32 data is a ``numpy.float32`` array; fp16 and bf16
data are ``numpy.uint16`` arrays holding the raw 16-bit patterns.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force and library conversions. One reading is
parity unpinned: a rotary coefficient c other than 2 and L (the MLA
preprocess page, section 2, names qRotaryCoeff / kRotaryCoeff values 2, 4 and
headDim with no formula). The oracle's rule for it -- the slice in c parts,
part 2g paired lane by lane with part 2g+1 -- reduces to rotate_half at c = 2
and to interleave at c = L, which are pinned; for other c the pins check that
rule against restatements of itself, not against anything the pages fix.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rope_oracle.c")
_DEFAULT_LIB_PATH = os.path.join(_HERE, "librope_oracle.so")
# ROPE_ORACLE_LIB points the pins at another build of the oracle (the
# planted-mistake test runs them against deliberately broken copies).
_LIB_PATH = os.environ.get("ROPE_ORACLE_LIB") or _DEFAULT_LIB_PATH

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
MODES = {"rotate_half": 0, "interleave": 1}


def mode_code(mode) -> int:
    """A mode name, or an int: 0 / 1 (rotate_half / interleave) or a rotary
    coefficient c >= 2 (the slice in c parts of L/c lanes; part 2k pairs
    with part 2k+1 lane by lane)."""
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"unknown mode {mode!r}")
        return MODES[mode]
    return int(mode)
DIRECTIONS = {"fwd": 0, "bwd": 1}

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-fPIC", "-shared"]
GCC_CMD = ["gcc"] + GCC_FLAGS + [_SRC, "-o", _DEFAULT_LIB_PATH, "-lm"]


def build() -> str:
    """Compile the oracle library with gcc; returns its path."""
    subprocess.run(GCC_CMD, check=True)
    return _DEFAULT_LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            if _LIB_PATH != _DEFAULT_LIB_PATH:
                raise FileNotFoundError(_LIB_PATH)
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.rope_oracle_rows.restype = ctypes.c_int
        L.rope_oracle_rows.argtypes = [
            ctypes.c_void_p, i64p, ctypes.c_int,
            ctypes.c_void_p, i64p, i64p,
            ctypes.c_void_p, i64p, i64p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            i64p, ctypes.c_int64,
        ]
        for name in ("oracle_f16_to_f32_n", "oracle_bf16_to_f32_n"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        for name in ("oracle_f32_to_f16_n", "oracle_f32_to_bf16_n"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.rope_oracle_pos_tables.restype = ctypes.c_int
        L.rope_oracle_pos_tables.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ]
        L.oracle_round_double_n.restype = None
        L.oracle_round_double_n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        _lib = L
    return _lib


def _i64(seq) -> ctypes.Array:
    arr = (ctypes.c_int64 * len(seq))(*[int(v) for v in seq])
    return arr


def _check_storage(a: np.ndarray, dtype: str) -> None:
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be stored as {np.dtype(want).name}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("oracle buffers must be C-contiguous")


def _table_strides(t: np.ndarray) -> list[int]:
    item = t.itemsize
    return [s // item for s in t.strides]


def rope_rows(x: np.ndarray, x_shape, dtype: str, r1: np.ndarray, r2: np.ndarray,
              mode: str, partial_slice, direction: str, rows=None, table_dtype: str | None = None) -> None:
    """Rotate the slice of rows of ``x`` in place (see ``rope_oracle.c``).

    ``x`` holds either the whole (B,S,N,D) tensor (``rows=None``) or, in row
    order, the rows whose flat indices ``(b*S+s)*N+n`` are listed in ``rows``.
    ``r1``/``r2`` are 4-D numpy arrays (any strides, including the zero
    strides of ``np.broadcast_to``) whose size-1 dimensions broadcast.
    ``table_dtype`` defaults to ``dtype``. ``partial_slice=None`` means
    [0, 0), the empty slice.
    """
    _check_storage(x, dtype)
    table_dtype = dtype if table_dtype is None else table_dtype
    want = np.float32 if table_dtype == "f32" else np.uint16
    for t in (r1, r2):
        if t.dtype != want or t.ndim != 4:
            raise TypeError("tables must be 4-D arrays in the table storage type")
    start, end = (0, 0) if partial_slice is None else (int(partial_slice[0]), int(partial_slice[1]))
    B, S, N, D = (int(v) for v in x_shape)
    if rows is None:
        if x.size != B * S * N * D:
            raise ValueError("x does not hold the full tensor")
        rows_p = None
        nrows = B * S * N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if x.size != rows.size * D:
            raise ValueError("x must hold len(rows) rows of D elements")
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        nrows = rows.size
    rc = lib().rope_oracle_rows(
        x.ctypes.data, _i64(x_shape), DTYPES[dtype],
        r1.ctypes.data, _i64(r1.shape), _i64(_table_strides(r1)),
        r2.ctypes.data, _i64(r2.shape), _i64(_table_strides(r2)),
        DTYPES[table_dtype], mode_code(mode), start, end, DIRECTIONS[direction],
        rows_p, nrows)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


# Converters (oracle-private; exposed so that tests can pin them).

def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_f16_to_f32_n(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_bf16_to_f32_n(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def f32_to_f16_bits(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_f16_n(v.ctypes.data, out.ctypes.data, v.size)
    return out


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(v.ctypes.data, out.ctypes.data, v.size)
    return out


def pos_tables(positions: np.ndarray, inv_freq: np.ndarray, L: int, mode: str, table_dtype: str):
    """The (cos, sin) tables of shape (Bp, S, 1, L) in storage form that the
    position entry points compute in the kernel (see rope_oracle_pos_tables):
    θ = p * inv_freq[i] in double precision, cos and sin in double precision,
    rounded once to ``table_dtype``; pair i's values in lanes 2i and 2i+1
    (interleave), i and i + L/2 (rotate_half), or, for a rotary coefficient
    c with parts of H = L/c lanes, g*2H + k and g*2H + k + H (i = g*H + k).

    ``positions`` is a 2-D int64 array (Bp, S), any strides; ``inv_freq``
    holds L/2 doubles."""
    pos = np.asarray(positions)
    if pos.dtype != np.int64 or pos.ndim != 2:
        raise TypeError("positions must be a 2-D int64 array")
    if table_dtype not in DTYPES:
        raise ValueError("unknown table type")
    mode = mode_code(mode)
    f = np.ascontiguousarray(inv_freq, dtype=np.float64)
    if f.size != L // 2:
        raise ValueError("inv_freq must hold L/2 values")
    Bp, S = pos.shape
    sb, ss = (st // pos.itemsize for st in pos.strides)
    want = np.float32 if table_dtype == "f32" else np.uint16
    c = np.empty((Bp, S, 1, L), want)
    s_ = np.empty((Bp, S, 1, L), want)
    rc = lib().rope_oracle_pos_tables(pos.ctypes.data, Bp, S, sb, ss, f.ctypes.data, int(L), mode,
                                      DTYPES[table_dtype], c.ctypes.data, s_.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return c, s_


def proj_rope(x: np.ndarray, w: np.ndarray, y_shape, dtype: str, r1: np.ndarray, r2: np.ndarray, mode,
              partial_slice, out_dtype: str, table_dtype: str | None = None) -> np.ndarray:
    """A head projection followed by the rotation of each head's slice: the
    Q projection and RoPE stages of "ascend-transformer-boost 的
    MlaPreprocessOperation：MLA 预处理四阶段融合算子深度解析" (section 3, the
    four-stage pipeline: the WUQ matmul gives headNum x 192 lanes per token,
    then Q[..., :qRopeDim] is rotated with cos/sin of shape [tokenNum, 64]
    given from outside; section 2, qRopeDim and qRotaryCoeff).

    ``x`` holds M = B*S tokens of K inputs, (M, K); ``w`` the weights as a
    linear layer stores them, (N, K) with N = H*Dh (output lanes by inputs,
    the page's transposed-weight default). ``y_shape`` = (B, S, H, Dh).
    Storage as for rope_rows (fp32 as float32, 16-bit as uint16 bits).

    In the page's order, with the projection result in fp32 (a fused
    epilogue holds it in fp32 registers; nothing in between is rounded to
    the storage type):
      1. p = sum_k x[m,k] * w[n,k], in double precision (numpy matmul: the
         products of 16-bit inputs are exact, and a double sum of them is
         exact to far below fp32 resolution), rounded once to fp32;
      2. the slice [start, end) of each head of p rotated as fp32 data by
         rope_rows (fwd: double-precision evaluation, one rounding to fp32),
         tables (B or 1, S or 1, 1 or H, L) broadcasting as rope_rows takes
         them;
      3. rounded once more, to nearest even, to ``out_dtype`` (no rounding
         when it is fp32).
    Returns y, shape (B, S, H, Dh), in ``out_dtype`` storage."""
    B, S, H, Dh = (int(v) for v in y_shape)
    M, N = B * S, H * Dh
    for name, a in (("x", x), ("w", w)):
        _check_storage(a, dtype)
    if x.shape != (M, x.shape[-1]) or w.shape != (N, x.shape[-1]):
        raise ValueError("x must be (B*S, K) and w (H*Dh, K)")
    widen = {"f32": lambda a: a, "f16": f16_bits_to_f32, "bf16": bf16_bits_to_f32}[dtype]
    xd = widen(x).astype(np.float64)
    wd = widen(w).astype(np.float64)
    p = np.ascontiguousarray((xd @ wd.T).astype(np.float32)).reshape(B, S, H, Dh)
    start, end = (0, 0) if partial_slice is None else (int(partial_slice[0]), int(partial_slice[1]))
    if end > start:
        rope_rows(p, (B, S, H, Dh), "f32", r1, r2, mode, (start, end), "fwd",
                  table_dtype=table_dtype if table_dtype else dtype)
    if out_dtype == "f32":
        return p
    narrow = {"f16": f32_to_f16_bits, "bf16": f32_to_bf16_bits}[out_dtype]
    return narrow(p)


def round_double(values: np.ndarray, dtype: str) -> np.ndarray:
    """Doubles rounded once, to nearest even, to the values of ``dtype``
    (returned as float32, which holds every value of the three types)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.float32)
    lib().oracle_round_double_n(v.ctypes.data, out.ctypes.data, v.size, DTYPES[dtype])
    return out
