"""In-place partial rotary position embedding (RoPE) on MI355X (gfx950).

A thin ctypes binding over ``librope_partial.so``, whose C ABI is declared in
``include/rope_partial.h``. Every step of the operation runs in the library's
HIP kernels; this module only marshals torch tensors (device pointers, shapes,
strides, the current HIP stream) into the C calls and turns status codes into
exceptions. There is no CPU fallback: without the built library every call
raises.

The operation follows "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
原地部分旋转位置编码" (sections 功能与计算公式, 函数原型与参数说明, 约束说明,
自动微分说明) and, for the rotate_half pairing, "ANE实战RoPE位置编码在MIL中的纯
ANE实现" (section 先搞懂RoPE).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "rope_partial_fwd_inplace", "rope_partial_bwd_inplace", "rope_status_string", "inplace_partial_rotary_mul",
    "rope_partial_fwd_inplace_multi", "rope_partial_bwd_inplace_multi", "MULTI_MAX", "rope_partial_check",
    "rope_partial_launch_info", "rope_partial_fwd_out", "rope_partial_bwd_out", "partial_rotary_mul",
    "rope_partial_fwd_inplace_pos", "rope_partial_bwd_inplace_pos", "rope_inv_freq",
    "rope_partial_fwd_out_pos", "rope_partial_bwd_out_pos", "partial_rotary_mul_pos",
    "inplace_partial_rotary_mul_pos", "rope_partial_fwd_inplace_pos_multi", "rope_partial_bwd_inplace_pos_multi",
    "rope_proj_fwd", "RopeError", "library", "LIB_PATH", "ROPE_OK", "ROPE_ERR_NULLPTR", "ROPE_ERR_INVALID",
    "ROPE_ERR_UNSUPPORTED", "ROPE_ERR_RUNTIME", "MODES", "DTYPE_CODES",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "librope_partial.so")

ROPE_OK, ROPE_ERR_NULLPTR, ROPE_ERR_INVALID, ROPE_ERR_UNSUPPORTED, ROPE_ERR_RUNTIME = range(5)
MODES = {"rotate_half": 0, "interleave": 1}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
MULTI_MAX = 4

_I64x4 = ctypes.c_int64 * 4
_I64x2 = ctypes.c_int64 * 2
_ENTRY_ARGTYPES = [
    ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
    ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
    ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
    ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
    ctypes.c_void_p,
]


class RopeError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the code."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{rope_status_string(status)}: {detail}" if detail else rope_status_string(status))


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m transformer_positional_encoding_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name in ("rope_partial_fwd_inplace", "rope_partial_bwd_inplace"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = _ENTRY_ARGTYPES
        for name in ("rope_partial_fwd_out", "rope_partial_bwd_out"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] + _ENTRY_ARGTYPES
        pos_args = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_void_p,
                    ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p,
                    ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
        for name in ("rope_partial_fwd_inplace_pos", "rope_partial_bwd_inplace_pos"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = pos_args + [ctypes.c_void_p]
        for name in ("rope_partial_fwd_out_pos", "rope_partial_bwd_out_pos"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] + pos_args + [ctypes.c_void_p]
        for name in ("rope_partial_fwd_inplace_pos_multi", "rope_partial_bwd_inplace_pos_multi"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p] + pos_args[2:] + [ctypes.c_void_p]
        L.rope_partial_launch_info_pos.restype = ctypes.c_int
        L.rope_partial_launch_info_pos.argtypes = pos_args + [ctypes.POINTER(ctypes.c_int64)]
        for name in ("rope_partial_fwd_inplace_multi", "rope_partial_bwd_inplace_multi"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p] + _ENTRY_ARGTYPES[2:]
        L.rope_partial_check.restype = ctypes.c_int
        L.rope_partial_check.argtypes = _ENTRY_ARGTYPES[:-1]
        L.rope_partial_launch_info.restype = ctypes.c_int
        L.rope_partial_launch_info.argtypes = _ENTRY_ARGTYPES[:-1] + [ctypes.POINTER(ctypes.c_int64)]
        L.rope_proj_fwd.restype = ctypes.c_int
        L.rope_proj_fwd.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_int64), ctypes.c_int64] + _ENTRY_ARGTYPES[3:]
        L.rope_proj_launch_info.restype = ctypes.c_int
        L.rope_proj_launch_info.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                            ctypes.c_int64] + _ENTRY_ARGTYPES[3:-1] + [ctypes.POINTER(ctypes.c_int64)]
        L.rope_status_string.restype = ctypes.c_char_p
        L.rope_status_string.argtypes = [ctypes.c_int]
        L.rope_last_error.restype = ctypes.c_char_p
        L.rope_last_error.argtypes = []
        _lib = L
    return _lib


def rope_status_string(status: int) -> str:
    return library().rope_status_string(int(status)).decode()


def _arr4(v):
    if v is None:
        return None
    if len(v) != 4:
        raise ValueError(f"expected 4 values, got {len(v)}")
    try:
        return _I64x4(*v)                       # tuples of ints (torch sizes and strides)
    except TypeError:
        return _I64x4(*[int(t) for t in v])     # other integer types


def raw_call(direction: str, x_ptr, x_shape, dtype: int, r1_ptr, r1_shape, r1_strides,
             r2_ptr, r2_shape, r2_strides, table_dtype: int, mode: int, partial_slice,
             stream=None) -> int:
    """Call an entry point with plain integers and sequences (None = NULL);
    returns the status code without raising."""
    fn = library().rope_partial_fwd_inplace if direction == "fwd" else library().rope_partial_bwd_inplace
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    a1, s1 = _arr4(r1_shape), _arr4(r1_strides)
    # r2 usually has r1's geometry: the same arrays then serve both
    a2 = a1 if r2_shape == r1_shape else _arr4(r2_shape)
    s2 = s1 if r2_strides == r1_strides else _arr4(r2_strides)
    return fn(x_ptr, _arr4(x_shape), int(dtype), r1_ptr, a1, s1, r2_ptr, a2, s2, int(table_dtype), int(mode), sl,
              stream)


def raw_out_call(direction: str, y_ptr, x_ptr, x_shape, dtype: int, r1_ptr, r1_shape, r1_strides,
                 r2_ptr, r2_shape, r2_strides, table_dtype: int, mode: int, partial_slice,
                 stream=None) -> int:
    """Call rope_partial_{fwd,bwd}_out with plain integers and sequences
    (None = NULL); returns the status code without raising."""
    fn = library().rope_partial_fwd_out if direction == "fwd" else library().rope_partial_bwd_out
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    a1, s1 = _arr4(r1_shape), _arr4(r1_strides)
    a2 = a1 if r2_shape == r1_shape else _arr4(r2_shape)
    s2 = s1 if r2_strides == r1_strides else _arr4(r2_strides)
    return fn(y_ptr, x_ptr, _arr4(x_shape), int(dtype), r1_ptr, a1, s1, r2_ptr, a2, s2, int(table_dtype), int(mode),
              sl, stream)


def raw_pos_call(direction: str, x_ptr, x_shape, dtype: int, pos_ptr, pos_shape, pos_strides, inv_freq_ptr,
                 table_dtype: int, mode: int, partial_slice, stream=None) -> int:
    """Call rope_partial_{fwd,bwd}_inplace_pos with plain integers and
    sequences (None = NULL); returns the status code without raising."""
    L = library()
    fn = L.rope_partial_fwd_inplace_pos if direction == "fwd" else L.rope_partial_bwd_inplace_pos
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    ps = None if pos_shape is None else _I64x2(int(pos_shape[0]), int(pos_shape[1]))
    pt = None if pos_strides is None else _I64x2(int(pos_strides[0]), int(pos_strides[1]))
    return fn(x_ptr, _arr4(x_shape), int(dtype), pos_ptr, ps, pt, inv_freq_ptr, int(table_dtype), int(mode), sl,
              stream)


def raw_out_pos_call(direction: str, y_ptr, x_ptr, x_shape, dtype: int, pos_ptr, pos_shape, pos_strides,
                     inv_freq_ptr, table_dtype: int, mode: int, partial_slice, stream=None) -> int:
    """Call rope_partial_{fwd,bwd}_out_pos with plain integers and sequences
    (None = NULL); returns the status code without raising."""
    L = library()
    fn = L.rope_partial_fwd_out_pos if direction == "fwd" else L.rope_partial_bwd_out_pos
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    ps = None if pos_shape is None else _I64x2(int(pos_shape[0]), int(pos_shape[1]))
    pt = None if pos_strides is None else _I64x2(int(pos_strides[0]), int(pos_strides[1]))
    return fn(y_ptr, x_ptr, _arr4(x_shape), int(dtype), pos_ptr, ps, pt, inv_freq_ptr, int(table_dtype),
              int(mode), sl, stream)


def raw_check(x_ptr, x_shape, dtype: int, r1_ptr, r1_shape, r1_strides, r2_ptr, r2_shape, r2_strides,
              table_dtype: int, mode: int, partial_slice) -> int:
    """rope_partial_check with plain integers and sequences (None = NULL):
    the status the entry points would return, with nothing launched."""
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    return library().rope_partial_check(x_ptr, _arr4(x_shape), int(dtype), r1_ptr, _arr4(r1_shape),
                                        _arr4(r1_strides), r2_ptr, _arr4(r2_shape), _arr4(r2_strides),
                                        int(table_dtype), int(mode), sl)


LAUNCH_INFO_LEN = 8
KERNELS = {0: "none", 1: "vector", 2: "scalar", 3: "rows"}


def raw_launch_info(x_ptr, x_shape, dtype: int, r1_ptr, r1_shape, r1_strides, r2_ptr, r2_shape, r2_strides,
                    table_dtype: int, mode: int, partial_slice, info_out: bool = True):
    """rope_partial_launch_info with plain integers and sequences (None =
    NULL): (status, plan dict or None). The plan names the kernel and the
    launch shape; nothing is launched. info_out=False passes a NULL info."""
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    info = (ctypes.c_int64 * LAUNCH_INFO_LEN)() if info_out else None
    st = library().rope_partial_launch_info(x_ptr, _arr4(x_shape), int(dtype), r1_ptr, _arr4(r1_shape),
                                            _arr4(r1_strides), r2_ptr, _arr4(r2_shape), _arr4(r2_strides),
                                            int(table_dtype), int(mode), sl, info)
    if st != ROPE_OK or info is None:
        return st, None
    v = list(info)
    if v[0] == 3:
        return st, {"kernel": "rows", "blocks": v[1], "threads": v[2], "rows_per_block": v[4],
                    "threads_per_row": v[7]}
    return st, {"kernel": KERNELS.get(v[0], v[0]), "blocks": v[1], "threads": v[2], "heads_per_thread": v[3],
                "head_lanes": v[4], "tiles_per_block": v[5], "xcd_run": v[6], "row_vectors": v[7]}


def raw_launch_info_pos(x_ptr, x_shape, dtype: int, pos_ptr, pos_shape, pos_strides, inv_freq_ptr,
                        table_dtype: int, mode: int, partial_slice, info_out: bool = True):
    """rope_partial_launch_info_pos with plain integers and sequences (None =
    NULL): (status, plan dict or None); nothing is launched."""
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    ps = None if pos_shape is None else _I64x2(int(pos_shape[0]), int(pos_shape[1]))
    pt = None if pos_strides is None else _I64x2(int(pos_strides[0]), int(pos_strides[1]))
    info = (ctypes.c_int64 * LAUNCH_INFO_LEN)() if info_out else None
    st = library().rope_partial_launch_info_pos(x_ptr, _arr4(x_shape), int(dtype), pos_ptr, ps, pt, inv_freq_ptr,
                                                int(table_dtype), int(mode), sl, info)
    if st != ROPE_OK or info is None:
        return st, None
    v = list(info)
    if v[0] == 3:
        return st, {"kernel": "rows", "blocks": v[1], "threads": v[2], "rows_per_block": v[4],
                    "threads_per_row": v[7]}
    return st, {"kernel": KERNELS.get(v[0], v[0]), "blocks": v[1], "threads": v[2], "heads_per_thread": v[3],
                "head_lanes": v[4], "positions_per_block": v[5], "head_chunks": v[6], "row_vectors": v[7]}


def raw_multi_call(direction: str, x_ptrs, x_shapes, dtype: int, r1_ptr, r1_shape, r1_strides,
                   r2_ptr, r2_shape, r2_strides, table_dtype: int, mode: int, partial_slice,
                   stream=None, count=None) -> int:
    """Call a _multi entry point with plain integers and sequences (None =
    NULL); returns the status code without raising."""
    L = library()
    fn = L.rope_partial_fwd_inplace_multi if direction == "fwd" else L.rope_partial_bwd_inplace_multi
    n = len(x_ptrs) if x_ptrs is not None else 0
    count = n if count is None else count
    ptrs = None if x_ptrs is None else (ctypes.c_void_p * max(n, 1))(*x_ptrs)
    flat = [] if x_shapes is None else [int(v) for sh in x_shapes for v in sh]
    shapes = None if x_shapes is None else (ctypes.c_int64 * max(len(flat), 4))(*flat)
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    return fn(int(count), ptrs, shapes, int(dtype), r1_ptr, _arr4(r1_shape), _arr4(r1_strides),
              r2_ptr, _arr4(r2_shape), _arr4(r2_strides), int(table_dtype), int(mode), sl, stream)


def raw_pos_multi_call(direction: str, x_ptrs, x_shapes, dtype: int, pos_ptr, pos_shape, pos_strides,
                       inv_freq_ptr, table_dtype: int, mode: int, partial_slice, stream=None, count=None) -> int:
    """Call a _pos_multi entry point with plain integers and sequences
    (None = NULL); returns the status code without raising."""
    L = library()
    fn = L.rope_partial_fwd_inplace_pos_multi if direction == "fwd" else L.rope_partial_bwd_inplace_pos_multi
    n = len(x_ptrs) if x_ptrs is not None else 0
    count = n if count is None else count
    ptrs = None if x_ptrs is None else (ctypes.c_void_p * max(n, 1))(*x_ptrs)
    flat = [] if x_shapes is None else [int(v) for sh in x_shapes for v in sh]
    shapes = None if x_shapes is None else (ctypes.c_int64 * max(len(flat), 4))(*flat)
    sl = None if partial_slice is None else _I64x2(int(partial_slice[0]), int(partial_slice[1]))
    ps = None if pos_shape is None else _I64x2(int(pos_shape[0]), int(pos_shape[1]))
    pt = None if pos_strides is None else _I64x2(int(pos_strides[0]), int(pos_strides[1]))
    return fn(int(count), ptrs, shapes, int(dtype), pos_ptr, ps, pt, inv_freq_ptr, int(table_dtype), int(mode), sl,
              stream)


def raw_proj_call(y_ptr, y_dtype: int, x_ptr, w_ptr, dtype: int, y_shape, K: int, r1_ptr, r1_shape, r1_strides,
                  r2_ptr, r2_shape, r2_strides, table_dtype: int, mode: int, partial_slice, stream=None) -> int:
    """rope_proj_fwd with plain integers and sequences (None = NULL); returns
    the status code without raising."""
    sl = None if partial_slice is None else _I64x2(*partial_slice)
    return library().rope_proj_fwd(y_ptr, y_dtype, x_ptr, w_ptr, dtype, _arr4(y_shape), int(K),
                                   r1_ptr, _arr4(r1_shape), _arr4(r1_strides), r2_ptr, _arr4(r2_shape),
                                   _arr4(r2_strides), table_dtype, mode, sl, stream)


PROJ_KERNELS = {0: "none", 4: "heads", 5: "square"}
PROJ_EPILOGUES = {0: "general", 1: "vector", 2: "vector_partner"}


def raw_proj_launch_info(y_dtype: int, dtype: int, y_shape, K: int, r1_ptr, r1_shape, r1_strides, r2_ptr, r2_shape,
                         r2_strides, table_dtype: int, mode: int, partial_slice, info_out: bool = True):
    """rope_proj_launch_info with plain integers and sequences (None =
    NULL): (status, plan dict or None). The plan names the projection kernel,
    its tile and (square tiles) its epilogue; nothing is launched."""
    sl = None if partial_slice is None else _I64x2(*partial_slice)
    info = (ctypes.c_int64 * LAUNCH_INFO_LEN)() if info_out else None
    st = library().rope_proj_launch_info(int(y_dtype), int(dtype), _arr4(y_shape), int(K), r1_ptr, _arr4(r1_shape),
                                         _arr4(r1_strides), r2_ptr, _arr4(r2_shape), _arr4(r2_strides),
                                         int(table_dtype), int(mode), sl, info)
    if st != ROPE_OK or info is None:
        return st, None
    v = list(info)
    return st, {"kernel": PROJ_KERNELS.get(v[0], v[0]), "blocks": v[1], "threads": v[2], "tile_tokens": v[3],
                "tile_lanes": v[4], "epilogue": PROJ_EPILOGUES.get(v[5], v[5]) if v[0] == 5 else None,
                "tables_in_lds": bool(v[6])}


def last_error() -> str:
    return library().rope_last_error().decode()


_DTYPE_OF_TORCH = {}


def _dtype_code(t) -> int:
    if not _DTYPE_OF_TORCH:
        import torch
        _DTYPE_OF_TORCH.update({torch.float32: 0, torch.float16: 1, torch.bfloat16: 2})
    code = _DTYPE_OF_TORCH.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return code


def _call(direction: str, x, r1, r2, mode, partial_slice, stream) -> None:
    import torch
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        mode = MODES[mode]
    for name, t in (("x", x), ("r1", r1), ("r2", r2)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B,S,N,D layout), got {t.dim()}-D")
    if x.numel() and not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (BSND); non-contiguous tensors are not supported")
    dev = x.device
    for name, t in (("r1", r1), ("r2", r2)):
        if t.numel() and x.numel() and t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream if x.is_cuda else None
    else:
        handle = getattr(stream, "cuda_stream", stream)
    # the launch goes to the current device: switch only when x lives elsewhere
    switch = x.is_cuda and dev.index != torch.cuda.current_device()
    with torch.cuda.device(dev) if switch else _nullcontext():
        st = raw_call(direction, x.data_ptr() or None, tuple(x.shape), _dtype_code(x),
                      r1.data_ptr() or None, tuple(r1.shape), tuple(r1.stride()),
                      r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                      _dtype_code(r1) if r1.dtype == r2.dtype else -1, mode, partial_slice, handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


def _call_out(direction: str, y, x, r1, r2, mode, partial_slice, stream) -> None:
    import torch
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        mode = MODES[mode]
    for name, t in (("out", y), ("x", x), ("r1", r1), ("r2", r2)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B,S,N,D layout), got {t.dim()}-D")
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError(f"out must match x in shape and dtype: {tuple(y.shape)} {y.dtype} vs "
                         f"{tuple(x.shape)} {x.dtype}")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError("x and out must be contiguous (BSND)")
    if x.numel() and not (x.is_cuda and y.is_cuda and y.device == x.device):
        raise ValueError("x and out must be GPU tensors on one device")
    dev = x.device
    for name, t in (("r1", r1), ("r2", r2)):
        if t.numel() and x.numel() and t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream if x.is_cuda else None
    else:
        handle = getattr(stream, "cuda_stream", stream)
    switch = x.is_cuda and dev.index != torch.cuda.current_device()
    with torch.cuda.device(dev) if switch else _nullcontext():
        st = raw_out_call(direction, y.data_ptr() or None, x.data_ptr() or None, tuple(x.shape), _dtype_code(x),
                          r1.data_ptr() or None, tuple(r1.shape), tuple(r1.stride()),
                          r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                          _dtype_code(r1) if r1.dtype == r2.dtype else -1, mode, partial_slice, handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


def _call_multi(direction: str, xs, r1, r2, mode, partial_slice, stream) -> None:
    import torch
    xs = list(xs)
    if len(xs) > MULTI_MAX:
        raise ValueError(f"at most {MULTI_MAX} tensors per call")
    if not xs:
        return
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        mode = MODES[mode]
    for name, t in [(f"xs[{i}]", x) for i, x in enumerate(xs)] + [("r1", r1), ("r2", r2)]:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B,S,N,D layout), got {t.dim()}-D")
    dtypes = {x.dtype for x in xs}
    if len(dtypes) != 1:
        raise TypeError("all tensors of one call must share a dtype")
    devs = {x.device for x in xs if x.numel()}
    if len(devs) > 1:
        raise ValueError("all tensors of one call must be on one device")
    for i, x in enumerate(xs):
        if x.numel() and not x.is_cuda:
            raise ValueError(f"xs[{i}] must be a GPU tensor")
        if not x.is_contiguous():
            raise ValueError(f"xs[{i}] must be contiguous (BSND)")
    dev = next(iter(devs)) if devs else None
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream if dev is not None else None
    else:
        handle = getattr(stream, "cuda_stream", stream)
    with torch.cuda.device(dev) if dev is not None else _nullcontext():
        st = raw_multi_call(direction, [x.data_ptr() or None for x in xs], [tuple(x.shape) for x in xs],
                            _dtype_code(xs[0]), r1.data_ptr() or None, tuple(r1.shape), tuple(r1.stride()),
                            r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                            _dtype_code(r1) if r1.dtype == r2.dtype else -1, mode, partial_slice, handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


class _nullcontext:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


def rope_partial_check(x, r1, r2, rotary_mode="interleave", partial_slice=None) -> None:
    """Run the entry points' argument checks on tensors (on any device:
    nothing is launched or read); raises RopeError on the first failure."""
    if isinstance(rotary_mode, str):
        if rotary_mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        rotary_mode = MODES[rotary_mode]
    st = raw_check(x.data_ptr() or None, tuple(x.shape), _dtype_code(x), r1.data_ptr() or None, tuple(r1.shape),
                   tuple(r1.stride()), r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                   _dtype_code(r1) if r1.dtype == r2.dtype else -1, rotary_mode, partial_slice)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


def rope_partial_launch_info(x, r1, r2, rotary_mode="interleave", partial_slice=None) -> dict:
    """The kernel and launch shape a call with these tensors would use
    (nothing is launched or read); raises RopeError like the entry points."""
    if isinstance(rotary_mode, str):
        if rotary_mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        rotary_mode = MODES[rotary_mode]
    st, plan = raw_launch_info(x.data_ptr() or None, tuple(x.shape), _dtype_code(x), r1.data_ptr() or None,
                               tuple(r1.shape), tuple(r1.stride()), r2.data_ptr() or None, tuple(r2.shape),
                               tuple(r2.stride()), _dtype_code(r1) if r1.dtype == r2.dtype else -1,
                               rotary_mode, partial_slice)
    if st != ROPE_OK:
        raise RopeError(st, last_error())
    return plan


def rope_partial_fwd_inplace(x, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Rotate ``x[..., start:end)`` in place (forward).

    x: contiguous (B,S,N,D) GPU tensor, float32/float16/bfloat16.
    r1, r2: cos and sin tables, 4-D, last dim ``end-start``, other dims 1 or
    equal to x's (any strides, e.g. from ``expand``); one dtype for both,
    which may differ from x's (e.g. bf16 x with fp32 tables).
    rotary_mode: "interleave" (pairs 2i, 2i+1), "rotate_half" (i, i+L/2), or
    an int rotary coefficient c (even, dividing L): the slice in c parts,
    lane k of part 2g paired with lane k of part 2g+1 (2: rotate_half; L:
    interleave).
    partial_slice: (start, end) or None for the empty slice [0, 0).
    stream: a torch stream or raw hipStream_t; default torch's current stream.
    """
    _call("fwd", x, r1, r2, rotary_mode, partial_slice, stream)


def rope_partial_bwd_inplace(dx, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Backward of :func:`rope_partial_fwd_inplace`: ``dx`` (the incoming
    gradient) is replaced in place by the gradient with respect to x."""
    _call("bwd", dx, r1, r2, rotary_mode, partial_slice, stream)


def rope_partial_fwd_out(out, x, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Out-of-place forward: ``out`` receives ``x`` with ``x[..., start:end)``
    rotated and every other lane copied; ``x`` is left unchanged. ``out``
    must be a contiguous tensor of x's shape and dtype that does not overlap
    x (``out is x`` is the in-place call). Arguments as in
    :func:`rope_partial_fwd_inplace`."""
    _call_out("fwd", out, x, r1, r2, rotary_mode, partial_slice, stream)


def rope_partial_bwd_out(dx, dy, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Out-of-place backward: ``dx`` receives the gradient with respect to x
    for the incoming gradient ``dy``, which is left unchanged."""
    _call_out("bwd", dx, dy, r1, r2, rotary_mode, partial_slice, stream)


def rope_inv_freq(L: int, base: float = 10000.0, device=None):
    """The frequencies base^(-2i/L), i < L/2, of the page's recipe, as the
    float64 tensor the _pos entry points take (computed in double on the
    host)."""
    import torch
    i = torch.arange(L // 2, dtype=torch.float64)
    return torch.pow(torch.tensor(float(base), dtype=torch.float64), -2.0 * i / L).to(device)


def _call_pos(direction, x, positions, inv_freq, mode, partial_slice, table_dtype, stream, y=None):
    """The position entry points: in place on x, or (y given) out of place
    from x into y."""
    import torch
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        mode = MODES[mode]
    for name, t in (("x", x), ("positions", positions), ("inv_freq", inv_freq)) + ((("out", y),) if y is not None
                                                                                   else ()):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if x.dim() != 4:
        raise ValueError(f"x must be 4-D (B,S,N,D layout), got {x.dim()}-D")
    if positions.dim() != 2 or positions.dtype != torch.int64:
        raise ValueError("positions must be a 2-D int64 tensor (B or 1, S)")
    if inv_freq.dtype != torch.float64 or inv_freq.dim() != 1 or not inv_freq.is_contiguous():
        raise ValueError("inv_freq must be a contiguous 1-D float64 tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (BSND); non-contiguous tensors are not supported")
    if y is not None:
        if y.shape != x.shape or y.dtype != x.dtype:
            raise ValueError(f"out must match x in shape and dtype: {tuple(y.shape)} {y.dtype} vs "
                             f"{tuple(x.shape)} {x.dtype}")
        if not y.is_contiguous():
            raise ValueError("out must be contiguous (BSND)")
        if x.numel() and not (x.is_cuda and y.is_cuda and y.device == x.device):
            raise ValueError("x and out must be GPU tensors on one device")
    sl = (0, 0) if partial_slice is None else (int(partial_slice[0]), int(partial_slice[1]))
    if x.numel() and sl[1] > sl[0]:
        if inv_freq.numel() != (sl[1] - sl[0]) // 2:
            raise ValueError(f"inv_freq must hold (end - start) / 2 = {(sl[1] - sl[0]) // 2} frequencies")
        if not x.is_cuda:
            raise ValueError("x must be a GPU tensor")
        for name, t in (("positions", positions), ("inv_freq", inv_freq)):
            if t.device != x.device:
                raise ValueError(f"{name} must be on {x.device}")
    if table_dtype is None:
        tdt = _dtype_code(x)
    else:
        tdt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}.get(table_dtype, DTYPE_CODES.get(table_dtype))
        if tdt is None:
            raise TypeError(f"unsupported table dtype {table_dtype}")
    dev = x.device
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream if x.is_cuda else None
    else:
        handle = getattr(stream, "cuda_stream", stream)
    switch = x.is_cuda and dev.index != torch.cuda.current_device()
    with torch.cuda.device(dev) if switch else _nullcontext():
        if y is None:
            st = raw_pos_call(direction, x.data_ptr() or None, tuple(x.shape), _dtype_code(x),
                              positions.data_ptr() or None, tuple(positions.shape), tuple(positions.stride()),
                              inv_freq.data_ptr() or None, tdt, mode, partial_slice, handle)
        else:
            st = raw_out_pos_call(direction, y.data_ptr() or None, x.data_ptr() or None, tuple(x.shape),
                                  _dtype_code(x), positions.data_ptr() or None, tuple(positions.shape),
                                  tuple(positions.stride()), inv_freq.data_ptr() or None, tdt, mode,
                                  partial_slice, handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


def rope_partial_fwd_inplace_pos(x, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                                 table_dtype=None, stream=None) -> None:
    """Rotate ``x[..., start:end)`` in place with cos/sin computed in the
    kernel from positions: θ = positions[b, s] * inv_freq[i] (double), cos
    and sin in double precision rounded once to ``table_dtype`` (default:
    x's dtype) -- the values a table of that type built from the same angles
    would hold.

    positions: int64 GPU tensor (B or 1, S), any strides.
    inv_freq: contiguous float64 GPU tensor of (end - start) / 2 frequencies
    (``rope_inv_freq(L, base)`` gives base^(-2i/L)).
    """
    _call_pos("fwd", x, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream)


def rope_partial_bwd_inplace_pos(dx, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                                 table_dtype=None, stream=None) -> None:
    """Backward of :func:`rope_partial_fwd_inplace_pos`, in place on the
    incoming gradient."""
    _call_pos("bwd", dx, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream)


def rope_partial_fwd_out_pos(out, x, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                             table_dtype=None, stream=None) -> None:
    """Out-of-place :func:`rope_partial_fwd_inplace_pos`: ``out`` receives x
    with its slice rotated; x is left unchanged."""
    _call_pos("fwd", x, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream, y=out)


def rope_partial_bwd_out_pos(dx, dy, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                             table_dtype=None, stream=None) -> None:
    """Out-of-place backward of the position form: ``dx`` receives the
    gradient with respect to x for the incoming gradient ``dy``, which is
    left unchanged."""
    _call_pos("bwd", dy, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream, y=dx)


def rope_partial_fwd_inplace_multi(xs, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Forward on up to MULTI_MAX tensors that share r1/r2 (e.g. Q and K), in
    one kernel launch when they take the same kernel; same result as calling
    :func:`rope_partial_fwd_inplace` on each in order."""
    _call_multi("fwd", xs, r1, r2, rotary_mode, partial_slice, stream)


def rope_partial_bwd_inplace_multi(dxs, r1, r2, rotary_mode="interleave", partial_slice=None, stream=None) -> None:
    """Backward counterpart of :func:`rope_partial_fwd_inplace_multi`."""
    _call_multi("bwd", dxs, r1, r2, rotary_mode, partial_slice, stream)


# ---------------------------------------------------------------------------
# Autograd op over the C ABI ("CANN ops-transformer 算子详解：
# inplace_partial_rotary_mul 原地部分旋转位置编码", section 自动微分说明 and the
# training-mode example of section 调用说明): the forward rotates x in place
# and marks it dirty; the backward runs the in-place backward entry point on
# the incoming gradient; r1 and r2 receive no gradient.
# ---------------------------------------------------------------------------

def _autograd_function():
    import torch

    class InplacePartialRotaryMulFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, r1, r2, rotary_mode, partial_slice):
            rope_partial_fwd_inplace(x, r1, r2, rotary_mode, partial_slice)
            ctx.mark_dirty(x)
            ctx.save_for_backward(r1, r2)
            ctx.rotary_mode = rotary_mode
            ctx.partial_slice = None if partial_slice is None else tuple(int(v) for v in partial_slice)
            return x

        @staticmethod
        def backward(ctx, grad):
            r1, r2 = ctx.saved_tensors
            return _grad_x(grad, r1, r2, ctx.rotary_mode, ctx.partial_slice), None, None, None, None

    return InplacePartialRotaryMulFn


def _grad_x(grad, r1, r2, rotary_mode, partial_slice):
    """The gradient with respect to x for the incoming gradient ``grad``,
    in a new tensor. Autograd may hand the same gradient buffer to other
    consumers, so it is never modified: a contiguous gradient is read by
    the out-of-place backward (one pass), any other layout (e.g. the stride-0
    gradient of an expand) is first made into a private contiguous copy,
    which is then rotated in place."""
    import torch
    if grad.is_contiguous():
        dx = torch.empty_like(grad, memory_format=torch.contiguous_format)
        rope_partial_bwd_out(dx, grad, r1, r2, rotary_mode, partial_slice)
        return dx
    dx = grad.contiguous()
    rope_partial_bwd_inplace(dx, r1, r2, rotary_mode, partial_slice)
    return dx


def _rotated_copy(x, r1, r2, rotary_mode, partial_slice):
    """A new contiguous tensor holding x with its slice rotated. A
    non-contiguous x is first made into a private contiguous copy, which is
    then rotated in place (one pass less than copying it again)."""
    import torch
    xc = x.contiguous()
    if xc.numel() and xc.data_ptr() != x.data_ptr():
        rope_partial_fwd_inplace(xc, r1, r2, rotary_mode, partial_slice)
        return xc
    y = torch.empty_like(xc, memory_format=torch.contiguous_format)
    rope_partial_fwd_out(y, xc, r1, r2, rotary_mode, partial_slice)
    return y


def _out_of_place_function():
    import torch

    class PartialRotaryMulFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, r1, r2, rotary_mode, partial_slice):
            y = _rotated_copy(x, r1, r2, rotary_mode, partial_slice)
            ctx.save_for_backward(r1, r2)
            ctx.rotary_mode = rotary_mode
            ctx.partial_slice = None if partial_slice is None else tuple(int(v) for v in partial_slice)
            return y

        @staticmethod
        def backward(ctx, grad):
            r1, r2 = ctx.saved_tensors
            return _grad_x(grad, r1, r2, ctx.rotary_mode, ctx.partial_slice), None, None, None, None

    return PartialRotaryMulFn


_FN = None
_FN_OUT = None


def inplace_partial_rotary_mul(x, r1, r2, rotary_mode="interleave", partial_slice=None) -> None:
    """In-place partial RoPE that records itself for autograd when x needs a
    gradient, and calls the forward entry point directly otherwise.

    x must not be a leaf tensor that requires grad: in-place changes to such
    a tensor are illegal in autograd, so rotate a non-leaf copy (y = x * 1.0),
    as the training example on the page does. r1 and r2 never get gradients.
    """
    import torch
    global _FN
    if torch.is_grad_enabled() and x.requires_grad:
        if x.is_leaf:
            raise RuntimeError("inplace_partial_rotary_mul: x is a leaf tensor that requires grad; "
                               "rotate a non-leaf copy of it (e.g. y = x * 1.0)")
        if _FN is None:
            _FN = _autograd_function()
        _FN.apply(x, r1, r2, rotary_mode, partial_slice)
        return None
    rope_partial_fwd_inplace(x, r1, r2, rotary_mode, partial_slice)
    return None


def partial_rotary_mul(x, r1, r2, rotary_mode="interleave", partial_slice=None):
    """Out-of-place partial RoPE: returns a new contiguous tensor holding x
    with ``x[..., start:end)`` rotated; x is not modified. Records itself for
    autograd (the backward is the out-of-place backward entry point) and
    works on leaf tensors too, so a training step needs no ``x * 1.0`` copy
    before the in-place op. r1 and r2 never get gradients."""
    import torch
    global _FN_OUT
    if torch.is_grad_enabled() and x.requires_grad:
        if _FN_OUT is None:
            _FN_OUT = _out_of_place_function()
        return _FN_OUT.apply(x, r1, r2, rotary_mode, partial_slice)
    return _rotated_copy(x, r1, r2, rotary_mode, partial_slice)


# ---------------------------------------------------------------- autograd, cos/sin from positions

def _grad_x_pos(grad, positions, inv_freq, rotary_mode, partial_slice, table_dtype):
    """The gradient with respect to x for ``grad`` in a new tensor, cos and
    sin computed from the positions (see _grad_x: grad is never modified)."""
    import torch
    if grad.is_contiguous():
        dx = torch.empty_like(grad, memory_format=torch.contiguous_format)
        rope_partial_bwd_out_pos(dx, grad, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
        return dx
    dx = grad.contiguous()
    rope_partial_bwd_inplace_pos(dx, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
    return dx


def _pos_functions():
    import torch

    def _save(ctx, positions, inv_freq, rotary_mode, partial_slice, table_dtype):
        ctx.save_for_backward(positions, inv_freq)
        ctx.rotary_mode = rotary_mode
        ctx.partial_slice = None if partial_slice is None else tuple(int(v) for v in partial_slice)
        ctx.table_dtype = table_dtype

    def _backward(ctx, grad):
        positions, inv_freq = ctx.saved_tensors
        dx = _grad_x_pos(grad, positions, inv_freq, ctx.rotary_mode, ctx.partial_slice, ctx.table_dtype)
        return dx, None, None, None, None, None

    class InplacePartialRotaryMulPosFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, positions, inv_freq, rotary_mode, partial_slice, table_dtype):
            rope_partial_fwd_inplace_pos(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
            ctx.mark_dirty(x)
            _save(ctx, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
            return x

        backward = staticmethod(_backward)

    class PartialRotaryMulPosFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, positions, inv_freq, rotary_mode, partial_slice, table_dtype):
            y = _rotated_copy_pos(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
            _save(ctx, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
            return y

        backward = staticmethod(_backward)

    return InplacePartialRotaryMulPosFn, PartialRotaryMulPosFn


def _rotated_copy_pos(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype):
    import torch
    xc = x.contiguous()
    if xc.numel() and xc.data_ptr() != x.data_ptr():
        rope_partial_fwd_inplace_pos(xc, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
        return xc
    y = torch.empty_like(xc, memory_format=torch.contiguous_format)
    rope_partial_fwd_out_pos(y, xc, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
    return y


_POS_FNS = None


def inplace_partial_rotary_mul_pos(x, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                                   table_dtype=None) -> None:
    """:func:`inplace_partial_rotary_mul` with cos and sin computed in the
    kernel from positions (see :func:`rope_partial_fwd_inplace_pos`).
    positions and inv_freq never get gradients; x must not be a leaf tensor
    that requires grad."""
    import torch
    global _POS_FNS
    if torch.is_grad_enabled() and x.requires_grad:
        if x.is_leaf:
            raise RuntimeError("inplace_partial_rotary_mul_pos: x is a leaf tensor that requires grad; "
                               "rotate a non-leaf copy of it (e.g. y = x * 1.0)")
        if _POS_FNS is None:
            _POS_FNS = _pos_functions()
        _POS_FNS[0].apply(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
        return None
    rope_partial_fwd_inplace_pos(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
    return None


def partial_rotary_mul_pos(x, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                           table_dtype=None):
    """:func:`partial_rotary_mul` with cos and sin computed in the kernel from
    positions: returns a new tensor, x is not modified, and the backward is
    the out-of-place position backward. positions and inv_freq never get
    gradients."""
    import torch
    global _POS_FNS
    if torch.is_grad_enabled() and x.requires_grad:
        if _POS_FNS is None:
            _POS_FNS = _pos_functions()
        return _POS_FNS[1].apply(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)
    return _rotated_copy_pos(x, positions, inv_freq, rotary_mode, partial_slice, table_dtype)


def _call_pos_multi(direction, xs, positions, inv_freq, mode, partial_slice, table_dtype, stream):
    import torch
    xs = list(xs)
    if len(xs) > MULTI_MAX:
        raise ValueError(f"at most {MULTI_MAX} tensors per call")
    if not xs:
        return
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        mode = MODES[mode]
    for i, x in enumerate(xs):
        if not isinstance(x, torch.Tensor) or x.dim() != 4:
            raise ValueError(f"xs[{i}] must be a 4-D torch.Tensor (B,S,N,D layout)")
        if not x.is_contiguous():
            raise ValueError(f"xs[{i}] must be contiguous (BSND)")
        if x.numel() and not x.is_cuda:
            raise ValueError(f"xs[{i}] must be a GPU tensor")
    if len({x.dtype for x in xs}) != 1:
        raise TypeError("all tensors of one call must share a dtype")
    devs = {x.device for x in xs if x.numel()}
    if len(devs) > 1:
        raise ValueError("all tensors of one call must be on one device")
    if positions.dim() != 2 or positions.dtype != torch.int64:
        raise ValueError("positions must be a 2-D int64 tensor (B or 1, S)")
    if inv_freq.dtype != torch.float64 or inv_freq.dim() != 1 or not inv_freq.is_contiguous():
        raise ValueError("inv_freq must be a contiguous 1-D float64 tensor")
    dev = next(iter(devs)) if devs else None
    sl = (0, 0) if partial_slice is None else (int(partial_slice[0]), int(partial_slice[1]))
    if dev is not None and sl[1] > sl[0]:
        if inv_freq.numel() != (sl[1] - sl[0]) // 2:
            raise ValueError(f"inv_freq must hold (end - start) / 2 = {(sl[1] - sl[0]) // 2} frequencies")
        for name, t in (("positions", positions), ("inv_freq", inv_freq)):
            if t.device != dev:
                raise ValueError(f"{name} must be on {dev}")
    if table_dtype is None:
        tdt = _dtype_code(xs[0])
    else:
        tdt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}.get(table_dtype, DTYPE_CODES.get(table_dtype))
        if tdt is None:
            raise TypeError(f"unsupported table dtype {table_dtype}")
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream if dev is not None else None
    else:
        handle = getattr(stream, "cuda_stream", stream)
    with torch.cuda.device(dev) if dev is not None else _nullcontext():
        st = raw_pos_multi_call(direction, [x.data_ptr() or None for x in xs], [tuple(x.shape) for x in xs],
                                _dtype_code(xs[0]), positions.data_ptr() or None, tuple(positions.shape),
                                tuple(positions.stride()), inv_freq.data_ptr() or None, tdt, mode, partial_slice,
                                handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())


def rope_partial_fwd_inplace_pos_multi(xs, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                                       table_dtype=None, stream=None) -> None:
    """:func:`rope_partial_fwd_inplace_pos` on up to 4 tensors sharing the
    positions (e.g. Q and K of one layer), in one launch when they share B,
    S and D: each pair's cos and sin is then evaluated once per position."""
    _call_pos_multi("fwd", xs, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream)


def rope_partial_bwd_inplace_pos_multi(xs, positions, inv_freq, rotary_mode="interleave", partial_slice=None,
                                       table_dtype=None, stream=None) -> None:
    """Backward of :func:`rope_partial_fwd_inplace_pos_multi`."""
    _call_pos_multi("bwd", xs, positions, inv_freq, rotary_mode, partial_slice, table_dtype, stream)


def rope_proj_fwd(x, w, r1, r2, heads: int, rotary_mode="interleave", partial_slice=None, out=None,
                  out_dtype=None, stream=None):
    """Head projection with a rotary epilogue (the C ABI's rope_proj_fwd):
    ``y[b,s,h,:] = rotate(x[b,s,:] @ w[h*Dh:(h+1)*Dh, :].T)`` with each head's
    lanes ``[start, end)`` rotated by the tables, the projection accumulated
    in fp32 and rounded once, after the rotation, to ``out_dtype`` ("ascend-
    transformer-boost 的 MlaPreprocessOperation：MLA 预处理四阶段融合算子深度解析",
    section 3: the Q projection and RoPE stages, fused).

    x: (B, S, K) or (M, K) bf16/fp16; w: (H*Dh, K) of x's dtype (a linear
    layer's weight); r1/r2: 4-D tables broadcasting against (B, S, H, L).
    Returns ``out`` (allocated when None): (B, S, H, Dh) of ``out_dtype``
    (x's dtype by default, or torch.float32)."""
    import torch
    if isinstance(rotary_mode, str):
        if rotary_mode not in MODES:
            raise ValueError(f"rotary_mode must be one of {sorted(MODES)}")
        rotary_mode = MODES[rotary_mode]
    for name, t in (("x", x), ("w", w), ("r1", r1), ("r2", r2)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if x.dim() not in (2, 3) or w.dim() != 2:
        raise ValueError("x must be (B, S, K) or (M, K) and w (H*Dh, K)")
    B, S = (1, x.shape[0]) if x.dim() == 2 else (x.shape[0], x.shape[1])
    K = x.shape[-1]
    N = w.shape[0]
    if w.shape[1] != K or heads <= 0 or N % heads:
        raise ValueError(f"w must be (heads*Dh, K={K}), got {tuple(w.shape)} for {heads} heads")
    if w.dtype != x.dtype:
        raise ValueError("x and w must share a dtype")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    y_shape = (B, S, heads, N // heads)
    if out is None:
        out = torch.empty(y_shape, dtype=out_dtype or x.dtype, device=x.device)
    elif tuple(out.shape) != y_shape or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {y_shape} tensor")
    for name, t in (("x", x), ("w", w), ("out", out)):
        if t.numel() and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    dev = x.device
    handle = (torch.cuda.current_stream(dev).cuda_stream if x.is_cuda else None) if stream is None else \
        getattr(stream, "cuda_stream", stream)
    switch = x.is_cuda and dev.index != torch.cuda.current_device()
    with torch.cuda.device(dev) if switch else _nullcontext():
        st = raw_proj_call(out.data_ptr() or None, _dtype_code(out), x.data_ptr() or None, w.data_ptr() or None,
                           _dtype_code(x), y_shape, K, r1.data_ptr() or None, tuple(r1.shape), tuple(r1.stride()),
                           r2.data_ptr() or None, tuple(r2.shape), tuple(r2.stride()),
                           _dtype_code(r1) if r1.dtype == r2.dtype else -1, rotary_mode, partial_slice, handle)
    if st != ROPE_OK:
        raise RopeError(st, last_error())
    return out
