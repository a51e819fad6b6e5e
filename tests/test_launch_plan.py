"""The launch plan on a machine without a GPU (rope_partial_launch_info):
which kernel a call takes and with what shape. Nothing is launched; the
pointers are fake, 128-byte aligned addresses that are never dereferenced."""
import pytest

import transformer_positional_encoding_amd as rp

OK, NULLPTR, INVALID = rp.ROPE_OK, rp.ROPE_ERR_NULLPTR, rp.ROPE_ERR_INVALID
F32, F16, BF16 = 0, 1, 2
IL, RH = 1, 0
FAKE = 0x10000
ESIZE = {F32: 4, F16: 2, BF16: 2}
MAX_GRID_ITEMS = 2 ** 32 - 1


def table_geometry(B, S, L, per_batch):
    shape = (B if per_batch else 1, S, 1, L)
    strides = (S * L, L, L, 1)
    return shape, strides


def plan(x_shape, dtype, sl, mode=IL, per_batch=False, table_dtype=None, x=FAKE, r=FAKE):
    B, S, N, D = x_shape
    L = sl[1] - sl[0]
    tshape, tstrides = table_geometry(B, S, L, per_batch)
    return rp.raw_launch_info(x, x_shape, dtype, r, tshape, tstrides, r, tshape, tstrides,
                              dtype if table_dtype is None else table_dtype, mode, sl)


def test_null_info_and_invalid_arguments():
    st, _ = rp.raw_launch_info(FAKE, (2, 4, 3, 64), BF16, FAKE, (1, 4, 1, 32), (128, 32, 32, 1),
                               FAKE, (1, 4, 1, 32), (128, 32, 32, 1), BF16, IL, (0, 32), info_out=False)
    assert st == NULLPTR
    st, info = plan((2, 4, 3, 64), BF16, (1, 33))          # odd start for interleave pairs is fine...
    assert st == OK
    st, info = plan((2, 4, 3, 64), BF16, (0, 31))          # ...an odd slice length is not
    assert st == INVALID and info is None


def test_noop_calls_launch_nothing():
    st, info = plan((0, 4, 3, 64), BF16, (0, 32))
    assert st == OK and info["kernel"] == "none" and info["blocks"] == 0
    st, info = plan((2, 4, 3, 64), BF16, (16, 16))
    assert st == OK and info["kernel"] == "none"


def test_long_context_shard_plan():
    """(16,8192,32,128) bf16, lanes [32,96), per-batch tables: the slice is
    half of each of two 128-byte lines, so each row's threads cover both
    lines (16 vectors); 4 heads per 64-thread block; runs of 384 KiB of x
    (48 positions of 8 blocks) per XCD."""
    st, info = plan((16, 8192, 32, 128), BF16, (32, 96), per_batch=True)
    assert st == OK
    assert info["kernel"] == "vector"
    assert info["row_vectors"] == 16 and info["threads"] == 64 and info["head_lanes"] == 4
    assert info["heads_per_thread"] == 1 and info["tiles_per_block"] == 1
    assert info["blocks"] == 16 * 8192 * 8
    assert info["xcd_run"] == 48 * 8


@pytest.mark.parametrize("dtype,tdtype,heads", [(BF16, F32, 2), (F16, F32, 2), (BF16, BF16, 1), (F32, F32, 1),
                                                (F32, BF16, 1)])
def test_in_place_heads_per_thread_follow_the_table_unit(dtype, tdtype, heads):
    """In place, a thread takes two heads when each 16-byte x vector needs
    two vectors each of cos and sin (16-bit x with fp32 tables), one head
    otherwise: the long-context shard's plan with per-batch tables."""
    st, info = plan((16, 8192, 32, 128), dtype, (32, 96), per_batch=True, table_dtype=tdtype)
    assert st == OK and info["kernel"] == "vector"
    assert info["heads_per_thread"] == heads and info["head_lanes"] == 4 and info["threads"] == 64
    assert info["blocks"] == 16 * 8192 * (32 // (4 * heads))


@pytest.mark.parametrize("x_shape,dtype,sl,mode,span", [
    ((4, 4096, 128, 192), BF16, (0, 64), IL, 8),       # whole line [0,128) bytes
    ((16, 8192, 32, 128), F32, (32, 96), IL, 16),      # bytes [128,384): two whole lines
    ((32, 256, 16, 128), BF16, (0, 128), RH, 8),       # rotate_half: one vector per half-pair unit
    ((8, 256, 12, 64), F16, (0, 64), IL, 8),
])
def test_vector_plans(x_shape, dtype, sl, mode, span):
    st, info = plan(x_shape, dtype, sl, mode)
    assert st == OK and info["kernel"] == "vector"
    assert info["row_vectors"] == span
    assert info["threads"] == span * info["head_lanes"] * info["tiles_per_block"] <= 64
    B, S, N, D = x_shape
    heads = info["head_lanes"] * info["heads_per_thread"]
    tiles = B * S * -(-N // heads)
    assert info["blocks"] == -(-tiles // info["tiles_per_block"])
    # XCD runs hold whole positions, so a table row is read by one XCD
    blocks_per_position = -(-N // heads) if info["tiles_per_block"] == 1 else 1
    assert info["xcd_run"] % blocks_per_position == 0


@pytest.mark.parametrize("case", ["misaligned_x", "misaligned_tables", "odd_start", "unaligned_length",
                                  "f16_x_bf16_tables", "bf16_x_f16_tables", "fp32_x_misaligned_16bit_tables"])
def test_scalar_plans(case):
    """Inputs the 16-byte vector kernel cannot take fall to the row kernel."""
    kw = {}
    x_shape, dtype, sl = (2, 4, 3, 64), BF16, (0, 32)
    if case == "misaligned_x":
        kw["x"] = FAKE + 2
    elif case == "misaligned_tables":
        kw["r"] = FAKE + 4
    elif case == "odd_start":
        sl = (1, 33)
    elif case == "unaligned_length":
        sl = (0, 12)                                    # 24 bytes: not a whole number of vectors
    elif case == "f16_x_bf16_tables":
        dtype, kw["table_dtype"] = F16, BF16
    elif case == "bf16_x_f16_tables":
        dtype, kw["table_dtype"] = BF16, F16
    else:                                               # 8-byte table units need 8-byte alignment
        dtype, kw["table_dtype"], kw["r"] = F32, BF16, FAKE + 4
    st, info = plan(x_shape, dtype, sl, **kw)
    assert st == OK and info["kernel"] == "rows"
    pairs = (sl[1] - sl[0]) // 2
    assert info["threads_per_row"] == min(pairs, 256)
    assert info["rows_per_block"] == 256 // info["threads_per_row"]
    assert info["threads"] == info["rows_per_block"] * info["threads_per_row"]
    assert info["blocks"] == -(-(2 * 4 * 3) // info["rows_per_block"])


@pytest.mark.parametrize("dtype,table_dtype", [(BF16, F32), (F16, F32), (F32, BF16), (F32, F16)])
@pytest.mark.parametrize("x_shape,sl,mode,per_batch", [
    ((16, 8192, 32, 128), (32, 96), IL, True),
    ((2, 8, 4, 128), (32, 96), IL, True),
    ((2, 8, 4, 128), (0, 128), RH, False),
])
def test_mixed_precision_vector_plans(dtype, table_dtype, x_shape, sl, mode, per_batch):
    """16-bit x with fp32 tables (two 16-byte table units per x vector) and
    fp32 x with 16-bit tables (one 8-byte unit) stay on the vector kernel."""
    st, info = plan(x_shape, dtype, sl, mode=mode, per_batch=per_batch, table_dtype=table_dtype)
    assert st == OK and info["kernel"] == "vector"


def test_grid_fits_the_dispatch_packet():
    """A ragged head count (5 heads in chunks of 4) pads the work-items past
    2^32 for a 6 GB tensor: the grid is cut so blocks x threads fits the
    32-bit grid size, and the blocks stride over the remaining tile groups."""
    x_shape = (1, 40_000_000, 5, 128)
    st, info = plan(x_shape, BF16, (32, 96))
    assert st == OK and info["kernel"] == "vector"
    assert info["head_lanes"] == 4 and info["threads"] == 64
    tiles = 40_000_000 * 2
    assert tiles * info["threads"] > MAX_GRID_ITEMS          # one block per tile group would not fit
    assert info["blocks"] * info["threads"] <= MAX_GRID_ITEMS
    assert info["blocks"] == MAX_GRID_ITEMS // info["threads"]


def test_plan_matches_direction_free_checks():
    """launch_info returns the status rope_partial_check returns."""
    for sl in [(0, 32), (0, 31), (-2, 30), (0, 66)]:
        args = (FAKE, (2, 4, 3, 64), BF16, FAKE, (1, 4, 1, sl[1] - sl[0]), (128, 32, 32, 1),
                FAKE, (1, 4, 1, sl[1] - sl[0]), (128, 32, 32, 1), BF16, IL, sl)
        assert rp.raw_launch_info(*args)[0] == rp.raw_check(*args)


def test_row_kernel_long_rows_loop():
    """A slice of more than 512 lanes: 256 threads per row, each taking
    several pairs."""
    st, info = plan((2, 3, 5, 1024), BF16, (1, 1023))
    assert st == OK and info["kernel"] == "rows"
    assert info["threads_per_row"] == 256 and info["rows_per_block"] == 1 and info["blocks"] == 30


def test_row_kernel_grid_fits_the_dispatch_packet():
    st, info = plan((1, 2 ** 30, 1, 4), BF16, (1, 3))       # 2^30 rows of one pair, odd start
    assert st == OK and info["kernel"] == "rows"
    assert info["blocks"] * info["threads"] <= MAX_GRID_ITEMS


def test_scalar_kernel_from_two_to_the_31_rows():
    """The row kernel's divisions hold below 2^31 rows; from there the
    64-bit scalar kernel runs."""
    st, info = plan((1, 2 ** 31, 1, 2), BF16, (0, 2))
    assert st == OK and info["kernel"] == "scalar"
    st, info = plan((1, 2 ** 31 - 1, 1, 2), BF16, (0, 2))
    assert st == OK and info["kernel"] == "rows"


@pytest.mark.parametrize("dtype,sl,span", [
    (BF16, (0, 128), 8),      # whole bf16 head: each half is one 128-byte line -> pair owner, first half only
    (F32, (0, 128), 16),      # fp32: halves of 256 bytes, on lines -> pair owner
    (BF16, (64, 128), 8),     # 64-byte halves -> own vector, the whole slice (one line)
    (BF16, (32, 96), 16),     # 64-byte halves off line boundaries -> own vector over both lines
    (BF16, (0, 32), 8),       # NeoX-style rotary_dim 32 of 128: own vector over the slice's whole line
    (F16, (0, 64), 8),        # 64-byte halves in one line -> own vector
])
def test_rotate_half_schemes(dtype, sl, span):
    """rotate_half in place: the pair-owner scheme (threads cover the first
    half) when each half is whole 128-byte lines, else the own-vector scheme
    (threads cover the slice's whole lines)."""
    st, info = plan((16, 4096, 32, 128), dtype, sl, mode=RH)
    assert st == OK and info["kernel"] == "vector"
    assert info["row_vectors"] == span
    assert info["threads"] <= 64


def test_rotate_half_own_vector_needs_single_wave_rows():
    """(1,3,5,1024) lanes [8,1000): the halves are off line boundaries, but a
    row of the own-vector scheme would need 124 threads (bf16) or 248 (fp32),
    more than one wave, so the pair owner runs (62 or 124 threads per row)."""
    for dtype, span in ((BF16, 62), (F32, 124)):
        st, info = plan((1, 3, 5, 1024), dtype, (8, 1000), mode=RH)
        assert st == OK and info["kernel"] == "vector" and info["row_vectors"] == span
    # lanes [8,520) bf16: the slice's whole lines would take 72 threads, the
    # slice itself 64, so the own-vector scheme runs over the slice alone
    st, info = plan((1, 3, 5, 1024), BF16, (8, 520), mode=RH)
    assert st == OK and info["row_vectors"] == 64 and info["threads"] == 64


# ---------------------------------------------------------------- position calls

POS_ESIZE = {"f32": 4, "f16": 2, "bf16": 2}


def pos_plan(x_shape, dtype, sl, mode=IL, per_batch=False, x=FAKE, table_dtype=None):
    B, S = x_shape[0], x_shape[1]
    pshape = (B if per_batch else 1, S)
    td = rp.DTYPE_CODES[table_dtype or dtype]
    return rp.raw_launch_info_pos(x, x_shape, rp.DTYPE_CODES[dtype], FAKE, pshape, (S, 1), FAKE, td,
                                  mode, sl)


def test_pos_plan_null_info_and_noops():
    assert rp.raw_launch_info_pos(FAKE, (2, 4, 3, 64), 2, FAKE, (1, 4), (4, 1), FAKE, 2, IL, (0, 32),
                                  info_out=False)[0] == rp.ROPE_ERR_NULLPTR
    assert pos_plan((2, 4, 3, 64), "bf16", (8, 8)) == (rp.ROPE_OK, {"kernel": "none", "blocks": 0, "threads": 0,
                                                                  "heads_per_thread": 0, "head_lanes": 0,
                                                                  "positions_per_block": 0, "head_chunks": 0,
                                                                  "row_vectors": 0})
    assert pos_plan((2, 4, 3, 64), "bf16", (0, 31))[0] == rp.ROPE_ERR_INVALID


def test_pos_plan_of_the_long_context_shard():
    st, p = pos_plan((16, 8192, 32, 128), "bf16", (32, 96), IL, per_batch=True)
    assert st == rp.ROPE_OK
    # whole 256-byte rows (the slice's lines), 8 head lanes x 2 heads, two chunks of 16 heads
    assert p == {"kernel": "vector", "blocks": 16 * 8192 * 2, "threads": 128, "heads_per_thread": 2,
                 "head_lanes": 8, "positions_per_block": 1, "head_chunks": 2, "row_vectors": 16}


@pytest.mark.parametrize("x_shape,dtype,sl,mode,per_batch,kernel,P", [
    ((2, 7, 1, 128), "bf16", (0, 128), RH, True, "vector", 8),   # one head: 8 positions of 8 threads per block
    ((3, 5, 2, 64), "bf16", (0, 64), IL, True, "vector", 8),
    ((2, 7, 1, 128), "bf16", (0, 128), RH, False, "vector", 4),  # shared positions: 2 batches x 1 head per s,
                                                                 # blocks of up to 64 threads
    ((3, 5, 2, 64), "bf16", (0, 64), IL, False, "vector", 1),    # 3 batches x 2 heads per s: 48 threads
    ((2, 5, 3, 1024), "f32", (0, 1024), RH, False, "vector", 1),  # 512 pairs: the whole LDS table
    ((2, 6, 5, 64), "bf16", (3, 35), IL, False, "rows", None),    # odd start
    ((2, 5, 3, 48), "bf16", (4, 44), RH, False, "rows", None),    # halves of 40 bytes
])
def test_pos_plan_kernels(x_shape, dtype, sl, mode, per_batch, kernel, P):
    st, p = pos_plan(x_shape, dtype, sl, mode, per_batch=per_batch)
    assert st == rp.ROPE_OK and p["kernel"] == kernel
    if P is not None:
        assert p["positions_per_block"] == P


def test_pos_plan_unaligned_x_takes_the_row_kernel():
    assert pos_plan((2, 4, 3, 64), "bf16", (0, 64), x=FAKE + 2)[1]["kernel"] == "rows"


def test_pos_plan_invariants_over_random_shapes():
    """Every vector plan: at most 256 threads, a multiple of the row's
    threads; the LDS table (positions per block x L/2 pairs) within 512
    entries; the head chunks cover N exactly; the rows' threads cover the
    slice; several positions per block only when a position's heads fill
    fewer than 128 threads; one block per chunk of positions. When the
    positions are shared by the batch, the positions are the S values and
    the heads the B*N (b, n) pairs."""
    import random
    rng = random.Random(5)
    seen = {"vector": 0, "rows": 0}
    for _ in range(3000):
        dtype = rng.choice(["f32", "f16", "bf16"])
        es = POS_ESIZE[dtype]
        D = rng.choice([8, 16, 24, 32, 48, 64, 96, 128, 192, 256, 512, 1024])
        start = rng.choice([0, 0, 0, 8, 16, 32, 3, 64]) % D
        start -= start % 2
        L = rng.randrange(0, D - start + 1, 2)
        if L == 0:
            continue
        mode = rng.choice([IL, RH])
        B, S, N = rng.randint(1, 4), rng.randint(1, 300), rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 64, 128])
        per_batch = rng.random() < 0.5
        shared_positions = not per_batch
        st, p = pos_plan((B, S, N, D), dtype, (start, start + L), mode, per_batch=per_batch)
        assert st == rp.ROPE_OK, (B, S, N, D, dtype, start, L, mode)
        seen[p["kernel"]] = seen.get(p["kernel"], 0) + 1
        aligned = (D * es) % 16 == 0 and (start * es) % 16 == 0
        unit = L * es if mode == IL else (L // 2) * es
        if not aligned or unit % 16:
            assert p["kernel"] != "vector"
            continue
        if p["kernel"] != "vector":
            continue
        span, HL, U, P, chunks = (p["row_vectors"], p["head_lanes"], p["heads_per_thread"],
                                  p["positions_per_block"], p["head_chunks"])
        # positions shared by the batch: the batches are heads of one position per s
        vheads = shared_positions and B > 1 and span * N < 128
        heads, positions = (B * N, S) if vheads else (N, B * S)
        assert p["threads"] == P * span * HL <= 256
        # with the batches as heads, blocks of up to 64 threads unless one row is wider
        if vheads:
            assert p["threads"] <= max(64, span)
        assert (chunks - 1) * HL * U < heads <= chunks * HL * U
        assert HL <= heads
        if mode == IL:
            assert span * 16 >= L * es and span * 16 <= D * es
        else:
            assert span * 16 == (L // 2) * es
        if P > 1:
            assert span * HL < (64 if vheads else 128)
        assert P * (L // 2) <= 512
        assert p["blocks"] == -(-positions // P) * chunks
    assert seen["vector"] > 500 and seen["rows"] > 100, seen


# ---------------------------------------------------------------- rotary coefficients

@pytest.mark.parametrize("x_shape,dtype,sl,coeff,kernel,span", [
    ((4, 4096, 128, 192), BF16, (0, 64), 4, "vector", 8),    # parts of 32 bytes: own vector, lane exchange
    ((4, 4096, 128, 192), BF16, (0, 64), 8, "vector", 8),    # parts of one vector
    ((4, 4096, 128, 192), BF16, (0, 64), 16, "rows", None),  # parts of 8 bytes: not whole vectors
    ((4, 4096, 128, 192), BF16, (0, 64), 64, "vector", 8),   # c = L: interleave
    ((2, 64, 4, 1024), F32, (0, 1024), 4, "vector", 128),    # rows wider than a wave: pair owner
])
def test_rotary_coefficient_plans(x_shape, dtype, sl, coeff, kernel, span):
    st, p = plan(x_shape, dtype, sl, mode=coeff)
    assert st == OK and p["kernel"] == kernel, p
    if span is not None:
        assert p["row_vectors"] == span


def test_rotary_coefficient_two_plans_as_rotate_half():
    for x_shape, dtype, sl in [((4, 4096, 16, 128), BF16, (0, 128)), ((16, 4096, 32, 128), BF16, (64, 128)),
                               ((2, 64, 4, 1024), F32, (0, 1024))]:
        assert plan(x_shape, dtype, sl, mode=2) == plan(x_shape, dtype, sl, mode=RH)
        L = sl[1] - sl[0]
        assert plan(x_shape, dtype, sl, mode=L) == plan(x_shape, dtype, sl, mode=IL)


@pytest.mark.parametrize("coeff,kernel", [(4, "vector"), (8, "vector"), (16, "rows")])
def test_rotary_coefficient_position_plans(coeff, kernel):
    st, p = pos_plan((4, 4096, 128, 192), "bf16", (0, 64), coeff)
    assert st == OK and p["kernel"] == kernel, p


def test_pos_plan_shares_positions_across_the_batch():
    """Positions the same for every batch (one row, or a batch stride of 0):
    the batches become heads of one position per s, in blocks of up to 64
    threads. For a single K head of 128 lanes (8 threads per row) and 32
    batches: 8 head lanes of 1 head (the rows' threads cover only the
    slice), four blocks per s."""
    st, p = pos_plan((32, 4096, 1, 128), "bf16", (0, 128), RH, per_batch=False)
    assert st == OK and p["head_lanes"] == 8 and p["head_chunks"] == 4 and p["positions_per_block"] == 1
    assert p["heads_per_thread"] == 1
    assert p["blocks"] == 4 * 4096 and p["threads"] == 64
    # per-batch positions: 16 consecutive (b, s) positions per block, LDS permitting (512 entries / 64 pairs)
    st, p = pos_plan((32, 4096, 1, 128), "bf16", (0, 128), RH, per_batch=True)
    assert st == OK and p["positions_per_block"] == 8 and p["blocks"] == 32 * 4096 // 8
