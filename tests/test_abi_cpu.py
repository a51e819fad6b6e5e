"""The C ABI on a machine without a GPU: the library loads, exports every
function the header declares, and rejects or no-ops arguments before any
HIP call, as the header documents (constraints from "CANN ops-transformer
算子详解：inplace_partial_rotary_mul 原地部分旋转位置编码", section 约束说明; no-op
rules from section 功能与计算公式)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import transformer_positional_encoding_amd as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULLPTR, INVALID, UNSUPPORTED = rp.ROPE_OK, rp.ROPE_ERR_NULLPTR, rp.ROPE_ERR_INVALID, rp.ROPE_ERR_UNSUPPORTED
F32, F16, BF16 = 0, 1, 2
IL, RH = 1, 0
FAKE = 0x10000  # never dereferenced: every call below returns before the launch


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:ROPE_API\s+)?(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("rope_partial_fwd_inplace", "rope_partial_bwd_inplace", "rope_status_string",
                 "rope_last_error", "rope_partial_fwd_inplace_multi", "rope_partial_bwd_inplace_multi",
                 "rope_partial_check", "rope_partial_launch_info", "rope_partial_fwd_out",
                 "rope_partial_bwd_out", "rope_partial_fwd_inplace_pos", "rope_partial_bwd_inplace_pos",
                 "rope_partial_launch_info_pos", "rope_partial_fwd_out_pos", "rope_partial_bwd_out_pos",
                 "rope_partial_fwd_inplace_pos_multi", "rope_partial_bwd_inplace_pos_multi"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = rp.library()
    out = subprocess.run(["nm", "-D", "--defined-only", rp.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings():
    for code in range(5):
        assert rp.rope_status_string(code).startswith("ROPE_")
    assert "unknown" in rp.rope_status_string(99)


SAME = object()  # r2 geometry defaults to r1's


def call(direction="check", x=FAKE, x_shape=(2, 4, 3, 64), dtype=BF16, r1=FAKE, r1_shape=(1, 4, 1, 32),
         r1_strides=(128, 32, 32, 1), r2=FAKE, r2_shape=SAME, r2_strides=SAME, table_dtype=None,
         mode=IL, sl=(0, 32)):
    """direction "check" runs rope_partial_check (never launches); "fwd"/"bwd"
    call the entry points and may only be used with arguments that fail
    validation or are no-ops, so that nothing is ever launched here."""
    args = (x, x_shape, dtype, r1, r1_shape, r1_strides, r2,
            r1_shape if r2_shape is SAME else r2_shape,
            r1_strides if r2_strides is SAME else r2_strides,
            dtype if table_dtype is None else table_dtype, mode, sl)
    if direction == "check":
        return rp.raw_check(*args)
    return rp.raw_call(direction, *args, None)


@pytest.mark.parametrize("dtype", [F32, F16, BF16])
@pytest.mark.parametrize("table_dtype", [F32, F16, BF16])
def test_valid_arguments_pass_the_checks(dtype, table_dtype):
    """Every x/table dtype pair is accepted (the page's mixed case is 16-bit x
    with fp32 tables)."""
    assert call(dtype=dtype, table_dtype=table_dtype) == OK
    assert call(dtype=dtype, table_dtype=table_dtype, mode=RH) == OK


@pytest.mark.parametrize("direction", ["check", "fwd", "bwd"])
@pytest.mark.parametrize("kwargs,code,text", [
    (dict(mode=3), INVALID, "mode"),                  # odd: neither a named mode nor a coefficient
    (dict(mode=-1), INVALID, "mode"),
    (dict(mode=6), INVALID, "divide"),                # a coefficient must divide L = 32
    (dict(mode=64), INVALID, "divide"),
    (dict(dtype=7), INVALID, "dtype"),
    (dict(x_shape=(2, -4, 3, 64)), INVALID, "negative"),
    (dict(x_shape=(2, 4, 3, 63), sl=(0, 32)), INVALID, "even"),
    (dict(x_shape=(1, 1, 1, 1026), sl=(0, 32)), INVALID, "1024"),
    (dict(sl=(-2, 30)), INVALID, ">= 0"),
    (dict(sl=(10, 8)), INVALID, "start"),
    (dict(sl=(40, 72)), INVALID, "<= D"),
    (dict(sl=(0, 31), r1_shape=(1, 4, 1, 31)), INVALID, "even"),
    (dict(x_shape=None), NULLPTR, "x_shape"),
])
def test_scalar_argument_errors(direction, kwargs, code, text):
    assert call(direction, **kwargs) == code
    assert text in rp.last_error()


@pytest.mark.parametrize("kwargs,code,text", [
    (dict(x=None), NULLPTR, "x is NULL"),
    (dict(r1=None), NULLPTR, "r1"),
    (dict(r2=None), NULLPTR, "r2"),
    (dict(r1_shape=None), NULLPTR, "r1"),
    (dict(r2_strides=None, r2_shape=(1, 4, 1, 32)), NULLPTR, "r2"),
    (dict(r1_shape=(1, 4, 1, 16)), INVALID, "last dimension"),
    (dict(r1_shape=(1, 3, 1, 32)), INVALID, "dimension S"),
    (dict(r1_shape=(2, 4, 2, 32)), INVALID, "dimension N"),
    (dict(r1_strides=(128, 32, 32, 2)), INVALID, "stride 1"),
    (dict(r1_strides=(128, -32, 32, 1)), INVALID, "negative"),
    (dict(r2_strides=(2**62, 2**62, 32, 1), r2_shape=(2, 4, 1, 32)), INVALID, "overflow"),
])
def test_pointer_and_table_errors(kwargs, code, text):
    for direction in ("check", "fwd", "bwd"):
        assert call(direction, **kwargs) == code
        assert text in rp.last_error()


@pytest.mark.parametrize("tshape,tstrides", [
    ((2, 4, 3, 32), (384, 96, 32, 1)),   # BSND
    ((2, 1, 3, 32), (96, 0, 32, 1)),     # B1ND
    ((2, 1, 1, 32), (32, 7, 99, 1)),     # B11D: strides of size-1 dims are ignored
    ((1, 1, 1, 32), (0, 0, 0, 1)),       # 111D
    ((2, 4, 1, 32), (128, 32, 0, 1)),    # BS1D
    ((1, 4, 1, 32), (0, 32, 0, 1)),      # expand()-style zero strides
])
def test_broadcast_layouts_accepted(tshape, tstrides):
    assert call(r1_shape=tshape, r1_strides=tstrides) == OK


@pytest.mark.parametrize("direction", ["check", "fwd", "bwd"])
@pytest.mark.parametrize("kwargs", [
    dict(sl=(8, 8)),                            # empty slice
    dict(sl=(64, 64)),
    dict(sl=None),                              # NULL partial_slice = [0, 0)
    dict(x_shape=(0, 4, 3, 64)),                # B = 0
    dict(x_shape=(2, 4, 0, 64)),                # N = 0
])
def test_noops_need_no_pointers(direction, kwargs):
    """No-ops return OK without reading x, the tables or their geometry."""
    assert call(direction, x=None, r1=None, r2=None, r1_shape=None, r1_strides=None,
                r2_shape=None, r2_strides=None, table_dtype=F32, **kwargs) == OK


def test_noop_still_checks_scalars():
    assert call(x=None, r1=None, r2=None, sl=(8, 8), mode=5) == INVALID
    assert call(x=None, r1=None, r2=None, x_shape=(0, 4, 3, 63), sl=(0, 0)) == INVALID


def test_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(2, 4, 3, 64)
    r = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        rp.rope_partial_fwd_inplace(x.view(8, 3, 64), r, r, "interleave", (0, 32))
    with pytest.raises(ValueError):
        rp.rope_partial_fwd_inplace(x, r, r, "sideways", (0, 32))
    with pytest.raises(ValueError):
        rp.rope_partial_fwd_inplace(x, r, r, "interleave", (0, 32))  # CPU tensor
    # an empty CPU tensor is a no-op that touches nothing
    rp.rope_partial_fwd_inplace(torch.zeros(0, 4, 3, 64), r, r, "interleave", (0, 32))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(rp, "_lib", None)
    monkeypatch.setattr(rp, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        rp.library()


def test_autograd_op_rejects_leaf_on_cpu():
    import torch
    x = torch.zeros(1, 2, 1, 8, requires_grad=True)
    r = torch.zeros(1, 2, 1, 8)
    with pytest.raises(RuntimeError, match="leaf"):
        rp.inplace_partial_rotary_mul(x, r, r, "interleave", (0, 8))


def mcall(direction="fwd", ptrs=(FAKE, FAKE), shapes=((2, 4, 3, 64), (2, 4, 1, 64)), table_dtype=None, **kw):
    r1_shape = kw.pop("r1_shape", (1, 4, 1, 32))
    r1_strides = kw.pop("r1_strides", (128, 32, 32, 1))
    return rp.raw_multi_call(direction, list(ptrs) if ptrs is not None else None,
                             list(shapes) if shapes is not None else None, kw.pop("dtype", BF16),
                             kw.pop("r1", FAKE), r1_shape, r1_strides, kw.pop("r2", FAKE), r1_shape, r1_strides,
                             BF16 if table_dtype is None else table_dtype, kw.pop("mode", IL), kw.pop("sl", (0, 32)),
                             None, count=kw.pop("count", None))


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_multi_checks_every_tensor_first(direction):
    # the second tensor's error is returned before anything runs, and named
    assert mcall(direction, shapes=((2, 4, 3, 64), (2, 5, 1, 64))) == INVALID
    assert "tensor 1" in rp.last_error()
    assert mcall(direction, ptrs=(FAKE, None)) == NULLPTR and "tensor 1" in rp.last_error()


def test_multi_count_rules():
    assert mcall(count=0, ptrs=None, shapes=None) == OK
    assert mcall(count=5, ptrs=[FAKE] * 5, shapes=[(2, 4, 3, 64)] * 5) == INVALID
    assert mcall(count=-1) == INVALID
    assert mcall(count=2, ptrs=None) == NULLPTR
    # every tensor a no-op: nothing launched, no pointer read
    assert mcall(ptrs=(None, None), sl=(8, 8), r1=None, r2=None) == OK


FAKE_Y = FAKE + 0x100000  # far from FAKE: no overlap with a small x


def ocall(direction="fwd", y=FAKE_Y, x=FAKE, x_shape=(2, 4, 3, 64), dtype=BF16, r1=FAKE, r1_shape=(1, 4, 1, 32),
          r1_strides=(128, 32, 32, 1), r2=FAKE, mode=IL, sl=(0, 32), table_dtype=None):
    """The out-of-place entry points, only with arguments that fail
    validation or are no-ops (nothing may be launched here)."""
    return rp.raw_out_call(direction, y, x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r1_shape, r1_strides,
                           dtype if table_dtype is None else table_dtype, mode, sl, None)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("kwargs,code,text", [
    (dict(mode=5), INVALID, "mode"),
    (dict(mode=12), INVALID, "divide"),
    (dict(x_shape=(2, 4, 3, 63)), INVALID, "even"),
    (dict(sl=(40, 72)), INVALID, "<= D"),
    (dict(x_shape=None), NULLPTR, "x_shape"),
    (dict(y=None), NULLPTR, "y is NULL"),
    (dict(x=None), NULLPTR, "x is NULL"),
    (dict(y=None, sl=(8, 8)), NULLPTR, "y is NULL"),      # an empty slice still copies x to y
    (dict(y=FAKE + 2), INVALID, "overlap"),               # 2 bytes past x: the buffers overlap
    (dict(x=FAKE_Y + 3070, y=FAKE_Y), INVALID, "overlap"),  # x starts 2 bytes before y's end
    (dict(r1=None), NULLPTR, "r1"),
    (dict(r1_shape=(1, 4, 1, 16)), INVALID, "last dimension"),
    (dict(r1_strides=(128, 32, 32, 2)), INVALID, "stride 1"),
])
def test_out_of_place_argument_errors(direction, kwargs, code, text):
    assert ocall(direction, **kwargs) == code
    assert text in rp.last_error()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_out_of_place_noops(direction):
    # empty tensor: no pointer is read
    assert ocall(direction, y=None, x=None, r1=None, r2=None, r1_shape=None, r1_strides=None,
                 x_shape=(0, 4, 3, 64)) == OK
    # empty slice on one buffer (y == x): nothing to do, tables not looked at
    assert ocall(direction, y=FAKE, x=FAKE, r1=None, r2=None, r1_shape=None, r1_strides=None, sl=(8, 8)) == OK
    # adjacent buffers do not overlap: the checks pass (then the launch would run)
    assert rp.raw_check(FAKE, (2, 4, 3, 64), BF16, FAKE, (1, 4, 1, 32), (128, 32, 32, 1), FAKE, (1, 4, 1, 32),
                        (128, 32, 32, 1), BF16, IL, (0, 32)) == OK


def test_out_of_place_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(2, 4, 3, 64)
    r = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError, match="shape and dtype"):
        rp.rope_partial_fwd_out(torch.zeros(2, 4, 3, 32), x, r, r, "interleave", (0, 32))
    with pytest.raises(ValueError, match="shape and dtype"):
        rp.rope_partial_fwd_out(x.half(), x, r, r, "interleave", (0, 32))
    with pytest.raises(ValueError, match="GPU"):
        rp.rope_partial_bwd_out(torch.zeros_like(x), x, r, r, "interleave", (0, 32))
    with pytest.raises(ValueError, match="contiguous"):
        rp.rope_partial_fwd_out(torch.zeros(2, 4, 64, 3).transpose(2, 3), torch.zeros(2, 4, 64, 3).transpose(2, 3),
                                r, r, "interleave", (0, 2))
    # an empty CPU tensor is a no-op that touches nothing
    e = torch.zeros(0, 4, 3, 64)
    rp.rope_partial_fwd_out(torch.zeros_like(e), e, r, r, "interleave", (0, 32))
    assert rp.partial_rotary_mul(e, r, r, "interleave", (0, 32)).shape == e.shape


def pcall(direction="fwd", x=FAKE, x_shape=(2, 4, 3, 64), dtype=BF16, pos=FAKE, pos_shape=(1, 4), pos_strides=(4, 1),
          inv_freq=FAKE, table_dtype=BF16, mode=IL, sl=(0, 32)):
    """The position entry points, only with arguments that fail validation
    or are no-ops."""
    return rp.raw_pos_call(direction, x, x_shape, dtype, pos, pos_shape, pos_strides, inv_freq, table_dtype, mode,
                           sl, None)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("kwargs,code,text", [
    (dict(mode=3), INVALID, "mode"),
    (dict(table_dtype=9), INVALID, "table dtype"),
    (dict(sl=(0, 31)), INVALID, "even"),
    (dict(x=None), NULLPTR, "x is NULL"),
    (dict(pos=None), NULLPTR, "positions is NULL"),
    (dict(inv_freq=None), NULLPTR, "inv_freq is NULL"),
    (dict(pos_shape=None), NULLPTR, "positions shape"),
    (dict(pos_strides=None), NULLPTR, "positions shape"),
    (dict(pos_shape=(3, 4)), INVALID, "dimension B"),
    (dict(pos_shape=(2, 5)), INVALID, "dimension S"),
    (dict(pos_shape=(2, 4), pos_strides=(-4, 1)), INVALID, "negative"),
    (dict(pos_shape=(2, 4), pos_strides=(2 ** 62, 2 ** 62)), INVALID, "overflow"),
])
def test_pos_argument_errors(direction, kwargs, code, text):
    assert pcall(direction, **kwargs) == code
    assert text in rp.last_error()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_pos_noops_need_no_pointers(direction):
    assert pcall(direction, x=None, pos=None, inv_freq=None, pos_shape=None, pos_strides=None, sl=(8, 8)) == OK
    assert pcall(direction, x=None, pos=None, inv_freq=None, x_shape=(0, 4, 3, 64)) == OK
    # a size-1 batch dimension's stride is ignored, however large
    assert pcall(direction, pos_shape=(1, 4), pos_strides=(2 ** 62, 1), x=None) == NULLPTR   # fails only on x


def test_pos_binding_checks():
    import torch
    x = torch.zeros(2, 4, 3, 64)
    f = rp.rope_inv_freq(32)
    with pytest.raises(ValueError, match="int64"):
        rp.rope_partial_fwd_inplace_pos(x, torch.zeros(1, 4), f, "interleave", (0, 32))
    with pytest.raises(ValueError, match="float64"):
        rp.rope_partial_fwd_inplace_pos(x, torch.zeros(1, 4, dtype=torch.int64), f.float(), "interleave", (0, 32))
    with pytest.raises(ValueError, match="frequencies"):
        rp.rope_partial_fwd_inplace_pos(x, torch.zeros(1, 4, dtype=torch.int64), rp.rope_inv_freq(16),
                                        "interleave", (0, 32))


@pytest.mark.parametrize("mode", [2, 4, 8, 16, 32])
def test_rotary_coefficients_that_divide_the_slice_pass_the_checks(mode):
    """A mode value c >= 2 is a rotary coefficient: the slice (L = 32) in c
    parts, part 2k paired with part 2k+1; any even c dividing L is valid."""
    assert call(mode=mode) == OK
    assert pcall("fwd", mode=mode, x=None) == NULLPTR          # past the mode checks, stops at x


def test_rotary_coefficient_with_an_empty_slice_is_a_noop():
    assert call("fwd", x=None, r1=None, r2=None, sl=(8, 8), mode=4) == OK


def opcall(direction="fwd", y=FAKE_Y, x=FAKE, x_shape=(2, 4, 3, 64), dtype=BF16, pos=FAKE, pos_shape=(1, 4),
           pos_strides=(4, 1), inv_freq=FAKE, mode=IL, sl=(0, 32)):
    """The out-of-place position entry points, only with arguments that
    fail validation or are no-ops."""
    return rp.raw_out_pos_call(direction, y, x, x_shape, dtype, pos, pos_shape, pos_strides, inv_freq, dtype,
                               mode, sl, None)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
@pytest.mark.parametrize("kwargs,code,text", [
    (dict(mode=3), INVALID, "mode"),
    (dict(y=None), NULLPTR, "y is NULL"),
    (dict(x=None), NULLPTR, "x is NULL"),
    (dict(x=FAKE_Y + 2), INVALID, "overlap"),
    (dict(pos=None), NULLPTR, "positions is NULL"),
    (dict(inv_freq=None), NULLPTR, "inv_freq is NULL"),
    (dict(pos_shape=(2, 5)), INVALID, "dimension S"),
    (dict(y=None, sl=(8, 8)), NULLPTR, "y is NULL"),      # an empty slice still copies x to y
])
def test_out_of_place_position_argument_errors(direction, kwargs, code, text):
    assert opcall(direction, **kwargs) == code
    assert text in rp.last_error()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_out_of_place_position_noops(direction):
    # an empty tensor: nothing is read, not even y or x
    assert opcall(direction, y=None, x=None, pos=None, inv_freq=None, x_shape=(0, 4, 3, 64)) == OK
    # y == x with an empty slice: nothing to do
    assert opcall(direction, y=FAKE, x=FAKE, pos=None, inv_freq=None, sl=(8, 8)) == OK


def pmcall(direction="fwd", ptrs=(FAKE, FAKE_Y), shapes=((2, 4, 3, 64), (2, 4, 1, 64)), pos=FAKE, pos_shape=(1, 4),
           pos_strides=(4, 1), inv_freq=FAKE, mode=IL, sl=(0, 32), count=None):
    """The multi-tensor position entry points, only with arguments that fail
    validation or are no-ops."""
    return rp.raw_pos_multi_call(direction, ptrs, shapes, BF16, pos, pos_shape, pos_strides, inv_freq, BF16, mode,
                                 sl, None, count=count)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_position_multi_argument_errors(direction):
    assert pmcall(direction, count=5) == INVALID and "count" in rp.last_error()
    assert pmcall(direction, count=-1) == INVALID
    assert pmcall(direction, ptrs=None, shapes=None, count=2) == NULLPTR
    assert pmcall(direction, shapes=((2, 4, 3, 64), (2, 5, 1, 64))) == INVALID
    assert "tensor 1" in rp.last_error() and "dimension S" in rp.last_error()
    assert pmcall(direction, ptrs=(FAKE, None)) == NULLPTR and "tensor 1" in rp.last_error()
    assert pmcall(direction, pos=None) == NULLPTR and "tensor 0" in rp.last_error()


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_position_multi_noops(direction):
    assert pmcall(direction, ptrs=None, shapes=None, count=0) == OK
    assert pmcall(direction, ptrs=(None, None), pos=None, inv_freq=None, sl=(8, 8)) == OK
    assert pmcall(direction, ptrs=(None, None), shapes=((0, 4, 3, 64), (2, 0, 1, 64)), pos=None, inv_freq=None) == OK


# ---------------------------------------------------------------- overlapping multi-tensor calls

@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_multi_rejects_overlapping_tensors(direction):
    """The same tensor twice, or two byte ranges that share bytes, are
    ROPE_ERR_INVALID before any launch (fake aligned addresses: nothing is
    dereferenced)."""
    shp = (2, 4, 3, 64)                      # bf16: 3072 bytes
    nbytes = 2 * 4 * 3 * 64 * 2
    tab = 0x200000
    args = dict(dtype=2, r1_ptr=tab, r1_shape=(1, 4, 1, 64), r1_strides=(0, 64, 0, 1), r2_ptr=tab,
                r2_shape=(1, 4, 1, 64), r2_strides=(0, 64, 0, 1), table_dtype=2, mode=1, partial_slice=(0, 64))
    for ptrs in ([0x100000, 0x100000], [0x100000, 0x100000 + nbytes - 16], [0x100000 + 16, 0x100000, 0x140000]):
        st = rp.raw_multi_call(direction, ptrs, [shp] * len(ptrs), **args)
        assert st == rp.ROPE_ERR_INVALID, ptrs
        assert "overlap" in rp.last_error()
    pos = dict(pos_ptr=0x300000, pos_shape=(1, 4), pos_strides=(4, 1), inv_freq_ptr=0x400000, table_dtype=2,
               mode=1, partial_slice=(0, 64))
    st = rp.raw_pos_multi_call(direction, [0x100000, 0x100000], [shp, shp], 2, **pos)
    assert st == rp.ROPE_ERR_INVALID and "overlap" in rp.last_error()


# ---------------------------------------------------------------- projection with a rotary epilogue

def _proj(**kw):
    base = dict(y_ptr=0x1000000, y_dtype=2, x_ptr=0x2000000, w_ptr=0x3000000, dtype=2, y_shape=(1, 8, 2, 192),
                K=128, r1_ptr=0x4000000, r1_shape=(1, 8, 1, 64), r1_strides=(0, 64, 0, 1), r2_ptr=0x5000000,
                r2_shape=(1, 8, 1, 64), r2_strides=(0, 64, 0, 1), table_dtype=2, mode=1, partial_slice=(0, 64))
    base.update(kw)
    return rp.raw_proj_call(*base.values())


@pytest.mark.parametrize("kwargs,code,text", [
    (dict(dtype=0, y_dtype=0), rp.ROPE_ERR_INVALID, "bf16 or fp16"),
    (dict(y_dtype=1), rp.ROPE_ERR_INVALID, "type of x and w"),
    (dict(K=-64), rp.ROPE_ERR_INVALID, "K is negative"),
    (dict(K=96), rp.ROPE_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(K=0), rp.ROPE_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(y_shape=(1, 8, 2, 160), r1_shape=(1, 8, 1, 64), r2_shape=(1, 8, 1, 64)), rp.ROPE_ERR_UNSUPPORTED,
     "head dimension"),
    # heads wider than a tile: 320 is neither a multiple of 192 nor of 128
    (dict(y_shape=(1, 8, 1, 320)), rp.ROPE_ERR_UNSUPPORTED, "head dimension"),
    # a 384-lane head over two 192-lane tiles: rotate_half over lanes [0, 384)
    # pairs lane j with j + 192, in the other tile (and wider than a 256-lane
    # square tile); [160, 224) straddles lane 192 too, and with K = 64 (not a
    # multiple of 128) there is no square tile to take it
    (dict(y_shape=(1, 8, 1, 384), r1_shape=(1, 8, 1, 384), r2_shape=(1, 8, 1, 384), r1_strides=(0, 384, 0, 1),
          r2_strides=(0, 384, 0, 1), mode=0, partial_slice=(0, 384)), rp.ROPE_ERR_UNSUPPORTED, "spans two column tiles"),
    (dict(y_shape=(1, 8, 1, 384), mode=0, partial_slice=(160, 224), K=64), rp.ROPE_ERR_UNSUPPORTED,
     "spans two column tiles"),
    # a coefficient's parts likewise: 4 parts of 32 over [160, 288) form groups [160, 224) and
    # [224, 288), the first across lane 192 (over [128, 256) the groups meet at 192 and are accepted)
    (dict(y_shape=(1, 8, 1, 384), r1_shape=(1, 8, 1, 128), r2_shape=(1, 8, 1, 128), r1_strides=(0, 128, 0, 1),
          r2_strides=(0, 128, 0, 1), mode=4, partial_slice=(160, 288)), rp.ROPE_ERR_UNSUPPORTED, "spans two column tiles"),
    (dict(y_ptr=None), rp.ROPE_ERR_NULLPTR, "y is NULL"),
    (dict(w_ptr=None), rp.ROPE_ERR_NULLPTR, "w is NULL"),
    (dict(x_ptr=0x2000008), rp.ROPE_ERR_INVALID, "16-byte aligned"),
    (dict(y_ptr=0x2000000 + 64), rp.ROPE_ERR_INVALID, "overlaps"),
    (dict(r1_shape=(1, 8, 1, 32)), rp.ROPE_ERR_INVALID, "last dimension"),
    (dict(r2_ptr=None), rp.ROPE_ERR_NULLPTR, "r2 is NULL"),
    (dict(partial_slice=(0, 200)), rp.ROPE_ERR_INVALID, "end must be <= D"),
    (dict(mode=3), rp.ROPE_ERR_INVALID, "mode"),
    (dict(y_shape=(1, 1 << 20, 2, 192), r1_shape=(1, 1 << 20, 1, 64), r2_shape=(1, 1 << 20, 1, 64), K=4096),
     rp.ROPE_ERR_UNSUPPORTED, "2^31"),
])
def test_projection_argument_errors(kwargs, code, text):
    assert _proj(**kwargs) == code
    assert text in rp.last_error()


def test_projection_wide_heads_pass_the_checks():
    """Heads wider than a tile pass every argument check when each rotation
    group stays in one tile: MLA's 576-lane compressed KV with rope on its
    last 64 lanes (interleave or rotate_half), a 256-lane head (two 128-lane
    tiles), and a coefficient's groups inside a 384-lane head's second tile.
    Without a GPU the call then fails at the launch, past every check."""
    for kw in (dict(y_shape=(1, 8, 1, 576), mode=1, partial_slice=(512, 576)),
               # [160, 224) crosses lane 192 of the head tiles but lies in the square tile [0, 256)
               dict(y_shape=(1, 8, 1, 384), mode=0, partial_slice=(160, 224)),
               dict(y_shape=(1, 8, 1, 576), mode=0, partial_slice=(512, 576)),
               dict(y_shape=(1, 8, 3, 256), mode=0, partial_slice=(0, 64)),
               dict(y_shape=(1, 8, 1, 384), r1_shape=(1, 8, 1, 128), r2_shape=(1, 8, 1, 128),
                    r1_strides=(0, 128, 0, 1), r2_strides=(0, 128, 0, 1), mode=4, partial_slice=(192, 320)),
               dict(y_shape=(1, 8, 1, 384), r1_shape=(1, 8, 1, 128), r2_shape=(1, 8, 1, 128),
                    r1_strides=(0, 128, 0, 1), r2_strides=(0, 128, 0, 1), mode=4, partial_slice=(128, 256))):
        st = _proj(**kw)
        assert st == rp.ROPE_ERR_RUNTIME, (kw, st, rp.last_error())


def test_projection_noops_need_no_pointers():
    """No tokens (or no heads): ROPE_OK without looking at any pointer."""
    none = dict(y_ptr=None, x_ptr=None, w_ptr=None, r1_ptr=None, r2_ptr=None)
    assert _proj(y_shape=(0, 8, 2, 192), **none) == rp.ROPE_OK
    assert _proj(y_shape=(1, 8, 0, 192), **none) == rp.ROPE_OK


def _proj_plan(**kw):
    base = dict(y_dtype=2, dtype=2, y_shape=(4, 4096, 128, 192), K=1536, r1_ptr=0x4000000, r1_shape=(1, 4096, 1, 64),
                r1_strides=(0, 64, 0, 1), r2_ptr=0x5000000, r2_shape=(1, 4096, 1, 64), r2_strides=(0, 64, 0, 1),
                table_dtype=2, mode=1, partial_slice=(0, 64))
    base.update(kw)
    st, plan = rp.raw_proj_launch_info(*base.values())
    assert st == rp.ROPE_OK, rp.last_error()
    return plan


def test_projection_plan_mla_q():
    """The MLA Q projection (4 x 4096 tokens, K 1536, 128 heads of 192, rope
    on lanes [0, 64) with one table row per token): 256 x 256 tiles (64 x 96
    of them), the vector epilogue with the table rows staged in LDS; with
    rotate_half the partners are 32 lanes (whole vectors) away."""
    plan = _proj_plan()
    assert plan == {"kernel": "square", "blocks": 64 * 96, "threads": 256, "tile_tokens": 256, "tile_lanes": 256,
                    "epilogue": "vector", "tables_in_lds": True}
    assert _proj_plan(mode=0)["epilogue"] == "vector_partner"
    assert _proj_plan(partial_slice=None)["epilogue"] == "vector"          # the plain projection


@pytest.mark.parametrize("kw,kernel,epilogue,lds", [
    # K = 192: three stages, not a whole number of stage pairs -> tiles of whole heads (384 x 192)
    (dict(K=192), "heads", None, False),
    # whole 192-lane heads under rotate_half: head 1's group [192, 384) crosses lane 256
    (dict(r1_shape=(1, 4096, 1, 192), r2_shape=(1, 4096, 1, 192), r1_strides=(0, 192, 0, 1),
          r2_strides=(0, 192, 0, 1), mode=0, partial_slice=(0, 192)), "heads", None, False),
    # heads of 128 with a 256-lane rotate_half group: inside the 256-lane tile, not inside a wave's 128
    (dict(y_shape=(1, 64, 8, 256), r1_shape=(1, 64, 1, 256), r2_shape=(1, 64, 1, 256), r1_strides=(0, 256, 0, 1),
          r2_strides=(0, 256, 0, 1), mode=0, partial_slice=(0, 256)), "square", "general", False),
    # an odd start: not whole vectors -> the general epilogue
    (dict(y_shape=(1, 64, 8, 64), r1_shape=(1, 64, 1, 32), r2_shape=(1, 64, 1, 32), r1_strides=(0, 32, 0, 1),
          r2_strides=(0, 32, 0, 1), partial_slice=(3, 35)), "square", "general", False),
    # tables per head (stride over heads): read per vector
    (dict(r1_shape=(1, 4096, 128, 64), r2_shape=(1, 4096, 128, 64), r1_strides=(0, 8192, 64, 1),
          r2_strides=(0, 8192, 64, 1)), "square", "vector", False),
    # fp32 tables: a row of 64 lanes is 256 bytes, too wide to stage
    (dict(table_dtype=0), "square", "vector", False),
    # fp32 tables of 32 lanes (128 bytes) are staged
    (dict(y_shape=(1, 64, 8, 64), r1_shape=(1, 64, 1, 32), r2_shape=(1, 64, 1, 32), r1_strides=(0, 32, 0, 1),
          r2_strides=(0, 32, 0, 1), partial_slice=(0, 32), table_dtype=0), "square", "vector", True),
    # per-batch rows (one per token) are staged too
    (dict(r1_shape=(4, 4096, 1, 64), r2_shape=(4, 4096, 1, 64), r1_strides=(4096 * 64, 64, 0, 1),
          r2_strides=(4096 * 64, 64, 0, 1)), "square", "vector", True),
    # MLA's compressed KV: one 576-lane head, rope on its last 64 lanes (tile 2 of 3)
    (dict(y_shape=(1, 4096, 1, 576), K=512, partial_slice=(512, 576)), "square", "vector", True),
    # fp32 output takes the vector epilogue as well
    (dict(y_dtype=0, mode=0), "square", "vector_partner", True),
])
def test_projection_plan_choices(kw, kernel, epilogue, lds):
    plan = _proj_plan(**kw)
    assert (plan["kernel"], plan["epilogue"], plan["tables_in_lds"]) == (kernel, epilogue, lds), plan


def test_projection_plan_shapes_and_errors():
    """Block counts follow the tile: 256 x 256 rounds both dimensions up;
    the 384 x 192 tiles of whole heads likewise. Errors are the call's own
    (same checks, same order); an empty y plans nothing; NULL info is an
    error."""
    p = _proj_plan(y_shape=(1, 300, 3, 128), r1_shape=(1, 300, 1, 64), r2_shape=(1, 300, 1, 64))
    assert (p["kernel"], p["blocks"]) == ("square", 2 * 2)
    p = _proj_plan(y_shape=(1, 300, 3, 192), r1_shape=(1, 300, 1, 64), r2_shape=(1, 300, 1, 64), K=64)
    assert (p["kernel"], p["blocks"], p["threads"], p["tile_tokens"], p["tile_lanes"]) == ("heads", 1 * 3, 768,
                                                                                           384, 192)
    st, plan = rp.raw_proj_launch_info(2, 2, (1, 8, 2, 192), 96, 0x4000000, (1, 8, 1, 64), (0, 64, 0, 1),
                                       0x5000000, (1, 8, 1, 64), (0, 64, 0, 1), 2, 1, (0, 64))
    assert st == rp.ROPE_ERR_UNSUPPORTED and "multiple of 64" in rp.last_error()
    st, plan = rp.raw_proj_launch_info(2, 2, (0, 8, 2, 192), 128, None, None, None, None, None, None, 2, 1, (0, 64))
    assert st == rp.ROPE_OK and plan["kernel"] == "none"
    st, plan = rp.raw_proj_launch_info(2, 2, (1, 8, 2, 192), 128, 0x4000000, (1, 8, 1, 64), (0, 64, 0, 1),
                                       0x5000000, (1, 8, 1, 64), (0, 64, 0, 1), 2, 1, (0, 64), info_out=False)
    assert st == rp.ROPE_ERR_NULLPTR
