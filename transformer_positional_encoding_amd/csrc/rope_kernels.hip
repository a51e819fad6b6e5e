// Partial rotary position embedding for MI355X (gfx950, CDNA4), in place
// and out of place.
//
// Operation: "CANN ops-transformer 算子详解：inplace_partial_rotary_mul
// 原地部分旋转位置编码", section 功能与计算公式 (interleave pairs (2i,2i+1),
// out = x*cos + x_rotate*sin on the lanes [start,end), in place) and section
// 自动微分说明 (backward = gradient w.r.t. x); rotate_half pairs (i, i+L/2)
// from "ANE实战RoPE位置编码在MIL中的纯ANE实现", section 先搞懂RoPE.
// Precision: the mixed-precision paragraph of the first page's tiling/kernel
// section -- 16-bit data is computed in fp32 and written back with
// round-to-nearest-even.
//
// The page's AICore kernel builds an XOR-1 gather table, multiplies, gathers,
// negates the even lanes with a bit mask and adds, in separate vector passes.
// Here a thread instead loads whole rotation pairs with 16-byte loads (a pair
// of 16-bit lanes is one 32-bit word; a pair of fp32 lanes is 8 bytes), does
// the swap and sign in registers, computes in fp32 (one fp32 rounding, exact
// products for 16-bit data) and stores only the slice's 16-byte vectors, so
// lanes outside [start,end) are never written (in place). The path is
// HBM-bound (0.375-0.75 flop per byte), so there is no MFMA and nothing is
// staged in LDS (rotate_half partners may move between lanes through the LDS
// crossbar, ds_bpermute): a block takes a chunk of heads of one (b,s)
// position, the blocks of a position run on one XCD, and when the tables
// broadcast over heads its cos/sin rows are fetched from HBM once and served
// by that XCD's L2 to every head.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <string>

#include "rope_device.hpp"
#include "rope_general_kernels.hpp"
#include "rope_partial.h"
#include "rope_plan.hpp"
#include "rope_pos_kernels.hpp"
#include "rope_proj_kernels.hpp"
#include "rope_vec_kernels.hpp"

namespace rope {
namespace {

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
thread_local std::string g_last_error;

rope_status_t set_error(rope_status_t st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Heads per thread of the instantiated vector kernels. In place: one, or two
// for 16-bit x with fp32 tables, where each 16-byte x vector takes two
// vectors each of cos and sin. A wave lasts as long as its slowest load, so
// with one head per thread those four table loads come with one x load;
// with two heads they serve two. Measured on MI355X (cold data), the
// long-context shard (16,8192,32,128) bf16, lanes [32,96), per-batch fp32
// tables: 289 us with one head per thread, 260 us with two, 286 us with
// four. With tables of x's dtype two heads per thread are slower (that
// shard 255 -> 258 us, the (4,4096,128,192) MLA rope slice 94 -> 100 us).
// Out of place: two (see prepare_out).
constexpr int u_in_place(int dtype, int tdtype)
{
    return dtype != ROPE_DTYPE_F32 && tdtype == ROPE_DTYPE_F32 ? 2 : 1;
}
constexpr int kUOut = 2;

// Launch shape of the vector kernel.
struct VecConfig {
    int kmode = kModeIL;  // kernel scheme: kModeIL, kModeRH (pair owner) or kModeRHOwn
    int U = 1;          // heads per thread per tile (u_in_place or kUOut)
    uint32_t HL = 1;    // head lanes per tile
    uint32_t GL = 1;    // tiles per block iteration
    uint32_t grid = 0;  // blocks; 0 = one block per tile group
    uint32_t xcd_group = 1;  // P of the XCD renumbering (1: dispatch order)
    bool nt = true;     // nontemporal loads/stores of x (the library instantiates true)
};

// Can the 16-byte vector kernel run this plan? Fills the geometry of `a`.
// Table types: the same as x, fp32 with 16-bit x, or 16-bit with fp32 x;
// fp16 with bf16 (either way round) takes the general kernel.
bool vec_geometry(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize, ts = p.tesize;
    if (p.tdtype != p.dtype && p.tdtype != ROPE_DTYPE_F32 && p.dtype != ROPE_DTYPE_F32) return false;
    const int64_t tbytes = 16 * ts / es;                   // table bytes per x vector: 8, 16 or 32
    const int64_t unit = std::min<int64_t>(16, tbytes);    // table unit (TableLanes::Vec)
    const int64_t tv = tbytes / unit;                      // table units per x vector: 1 or 2
    const auto aligned = [](const void* q, int64_t n) { return (reinterpret_cast<uintptr_t>(q) % n) == 0; };
    if (!aligned16(p.x) || !aligned(p.r1, unit) || !aligned(p.r2, unit)) return false;
    if ((p.D * es) % 16 || (p.start * es) % 16) return false;
    const int64_t unit_bytes = p.mode == kModeIL ? p.L * es : (p.L / 2) * es;
    if (unit_bytes % 16) return false;
    if (p.mode == kModeRH && (p.half * es) % 16) return false;   // half-groups of whole vectors
    for (int k = 0; k < 3; ++k)
        if ((p.t1[k] * ts) % unit || (p.t2[k] * ts) % unit) return false;
    // 32-bit offsets: x must span fewer than 2^32 vectors and each table
    // fewer than 2^32 units; tile indices stay below 2^31 (finish_vec_args).
    const int64_t kMax = (1ll << 32) - 1;
    const int64_t x_vecs = p.B * p.S * p.N * (p.D * es / 16);
    if (x_vecs > kMax || p.N >= (1ll << 31) || p.S >= (1ll << 31) || p.B * p.S >= (1ll << 31)) return false;
    const int64_t dims[3] = {p.B, p.S, p.N};
    int64_t t1_span = p.L * ts / unit, t2_span = p.L * ts / unit;
    for (int k = 0; k < 3; ++k) {
        t1_span += (dims[k] - 1) * (p.t1[k] * ts / unit);
        t2_span += (dims[k] - 1) * (p.t2[k] * ts / unit);
    }
    if (t1_span > kMax || t2_span > kMax) return false;
    a->x = static_cast<v4u*>(p.x);
    a->src = nullptr;
    a->r1 = p.r1;
    a->r2 = p.r2;
    a->row_vecs = (uint32_t)(p.D * es / 16);
    a->start_vec = (uint32_t)(p.start * es / 16);
    a->lo_vec = a->start_vec;
    a->half_vecs = p.mode == kModeRH ? (uint32_t)(p.half * es / 16) : 0;
    a->gvec = 2 * a->half_vecs;
    a->thalf = (uint32_t)(a->half_vecs * tv);
    a->t1b = (uint32_t)(p.t1[0] * ts / unit); a->t1s = (uint32_t)(p.t1[1] * ts / unit);
    a->t1n = (uint32_t)(p.t1[2] * ts / unit);
    a->t2b = (uint32_t)(p.t2[0] * ts / unit); a->t2s = (uint32_t)(p.t2[1] * ts / unit);
    a->t2n = (uint32_t)(p.t2[2] * ts / unit);
    a->N = (uint32_t)p.N;
    a->s_div = make_fastdiv((uint32_t)p.S);
    a->nvec = (uint32_t)(unit_bytes / 16);
    a->span = a->nvec;
    return a->nvec >= 1 && a->nvec <= 256;
}

// Slices that cover only part of their first or last 128-byte line
// (interleave, and rotate_half in the own-vector scheme): let the threads of
// a row cover the whole lines around the slice (see the vector kernel).
// Needs rows that start on line boundaries so the lines stay inside the row. Measured on MI355X for bf16 lanes [32,96) of
// 128 (same HBM bytes either way): 3-4% faster in this kernel, and 15% in a
// bare read-modify-write of the same bytes.
void cover_whole_lines(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize;
    const int64_t lo = (p.start * es) / 128 * 128;
    const int64_t hi = ((p.start + p.L) * es + 127) / 128 * 128;
    if (lo == p.start * es && hi == (p.start + p.L) * es) return;   // whole lines already
    if ((p.D * es) % 128 || (reinterpret_cast<uintptr_t>(p.x) & 127u)) return;
    if ((hi - lo) / 16 > 256) return;
    a->lo_vec = (uint32_t)(lo / 16);
    a->span = (uint32_t)((hi - lo) / 16);
}

// Launch shape for U heads per thread and a target block size: head lanes
// cover the heads of a (b,s) position up to the block size, and the rest of
// the block takes further tiles.
VecConfig shape_for(const VecArgs& a, int U, uint32_t threads)
{
    VecConfig c;
    c.U = U;
    const uint32_t hl_max = std::max<uint32_t>(1, threads / a.span);
    c.HL = (uint32_t)std::min<uint64_t>(hl_max, (a.N + U - 1) / U);
    c.GL = std::max<uint32_t>(1, threads / (a.span * c.HL));
    return c;
}

// The launch shape. Measured on MI355X with every launch reading data that
// no cache holds (the slices of several shapes: 1/4, 1/3, 1/2 and all of the
// row, whole and half 128-byte lines, bf16 and fp32, tables shared or per
// batch), sweeping heads per thread (1-8), block size (64-256) and
// nontemporal x: one head per thread, 64-thread blocks and nontemporal x was
// within 3% of the best shape on every one. Streaming x past the caches
// leaves the L2 to the tables, and small blocks let the dispatcher keep
// every CU's load queues full.
//
// XCD runs (see xcd_grouped_block): each XCD takes about kXcdRunBytes of
// consecutive rows of x per window, in whole (b,s) positions. Swept from one
// block to an eighth of the grid on twelve shapes: the time depends on the
// run length in a way that follows the HBM address interleave rather than
// the shape (runs of 16-64 KiB were 10-25% slower than the best), and runs
// of 384 KiB were within 4% of the best run length on all but the fp32
// shapes whose slice is a third of the row (there an eighth of the grid per
// XCD was 4% faster), and 7% faster than an eighth per XCD for the bf16
// long-context shard (16,8192,32,128) with lanes [32,96).
constexpr uint64_t kXcdRunBytes = 384u << 10;

VecConfig choose_vec_config(const Plan& p, const VecArgs& a, int U, int kmode)
{
    VecConfig c = shape_for(a, U, 64);
    c.kmode = kmode;
    c.nt = true;
    const uint64_t heads_per_tile = (uint64_t)c.HL * c.U;
    const uint64_t blocks_per_position = c.GL == 1 ? (a.N + heads_per_tile - 1) / heads_per_tile : 1;
    const uint64_t block_bytes = heads_per_tile * c.GL * (uint64_t)p.D * (uint64_t)p.esize;
    const uint64_t position_bytes = block_bytes * blocks_per_position;
    const uint64_t positions = std::max<uint64_t>(1, (kXcdRunBytes + position_bytes / 2) / position_bytes);
    c.xcd_group = (uint32_t)std::min<uint64_t>(positions * blocks_per_position, 1u << 24);
    return c;
}

// The dispatch packet holds the grid size in work-items as a 32-bit number.
constexpr uint64_t kMaxGridItems = 0xFFFFFFFFull;

uint32_t vec_grid(const VecArgs& a, const VecConfig& cfg)
{
    // One block per tile group by default: measured faster on MI355X than a
    // persistent grid for these streaming shapes (the dispatcher keeps every
    // CU full and no loop-carried dependence serialises the loads). A grid
    // that would exceed kMaxGridItems work-items is cut to fit, and the
    // blocks stride over the remaining tile groups.
    const uint64_t threads = (uint64_t)a.span * a.HL * a.GL;
    uint64_t grid = cfg.grid ? cfg.grid : a.btiles;
    grid = std::min<uint64_t>(grid, kMaxGridItems / threads);
    return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(grid, a.btiles));
}

// Complete `a` for a launch shape: head chunks and tile counts. False if a
// tile index could come near 32-bit wrap-around (the grid-stride loop adds
// gridDim.x to it), in which case a general kernel runs instead.
bool finish_vec_args(const Plan& p, const VecConfig& cfg, VecArgs* a)
{
    // The library instantiates the chosen shapes only: u_in_place or kUOut
    // heads per thread, nontemporal x.
    if (cfg.U != (a->src ? kUOut : u_in_place(p.dtype, p.tdtype)) || !cfg.nt || cfg.HL < 1 || cfg.GL < 1 ||
        (uint64_t)cfg.HL * cfg.GL * a->span > 256)
        return false;
    a->HL = cfg.HL;
    a->GL = cfg.GL;
    const uint64_t heads_per_tile = (uint64_t)cfg.HL * cfg.U;
    const uint64_t nchunk = (a->N + heads_per_tile - 1) / heads_per_tile;
    const uint64_t tiles = (uint64_t)p.B * p.S * nchunk;
    if (tiles >= (1ull << 31) || nchunk * heads_per_tile >= (1ull << 31)) return false;
    a->nchunk = (uint32_t)nchunk;
    a->tiles = (uint32_t)tiles;
    a->btiles = (uint32_t)((tiles + cfg.GL - 1) / cfg.GL);
    a->span_div = make_fastdiv(a->span);
    a->hl_div = make_fastdiv(a->HL);
    a->nchunk_div = make_fastdiv(a->nchunk);
    const uint64_t G = vec_grid(*a, cfg);
    const uint64_t P = std::max<uint32_t>(1, cfg.xcd_group);
    a->xcd_group = (uint32_t)P;
    a->xcd_full = 0;
    a->xcd_div = make_fastdiv(8);
    if (P > 1 && 8 * P <= G) {
        a->xcd_full = (uint32_t)(G / (8 * P) * (8 * P));
        a->xcd_div = make_fastdiv((uint32_t)(8 * P));
    }
    return true;
}

// Which vector kernel: in place on one tensor, in place on several, or out
// of place.
enum VecKind { kVecOne = 0, kVecMulti = 1, kVecOut = 2 };

template <int DT, int TT, int DIR, int MODE, bool SHARE>
const void* vec_kernel_ptr(VecKind kind)
{
    switch (kind) {
    case kVecMulti:
        // in place: no memory partner loads
        if constexpr (MODE == kModeRHOwnLoad) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_multi_kernel<DT, TT, DIR, MODE, u_in_place(DT, TT), SHARE, true>);
    case kVecOut:
        // out of place, rotate_half always takes an own-vector scheme
        if constexpr (MODE == kModeRH) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_out_kernel<DT, TT, DIR, MODE, kUOut, SHARE, true>);
    default:
        if constexpr (MODE == kModeRHOwnLoad) return nullptr;
        else return reinterpret_cast<const void*>(&rope_vec_kernel<DT, TT, DIR, MODE, u_in_place(DT, TT), SHARE, true>);
    }
}

template <int DT, int TT, int DIR, int MODE>
const void* vec_kernel_s(bool share, VecKind kind)
{
    return share ? vec_kernel_ptr<DT, TT, DIR, MODE, true>(kind) : vec_kernel_ptr<DT, TT, DIR, MODE, false>(kind);
}

template <int DT, int TT, int DIR>
const void* vec_kernel_m(int kmode, bool share, VecKind kind)
{
    switch (kmode) {
    case kModeIL: return vec_kernel_s<DT, TT, DIR, kModeIL>(share, kind);
    case kModeRH: return vec_kernel_s<DT, TT, DIR, kModeRH>(share, kind);
    case kModeRHOwn: return vec_kernel_s<DT, TT, DIR, kModeRHOwn>(share, kind);
    default: return vec_kernel_s<DT, TT, DIR, kModeRHOwnLoad>(share, kind);
    }
}

template <int DT, int TT>
const void* vec_kernel_t(int dir, int kmode, bool share, VecKind kind)
{
    return dir == kFwd ? vec_kernel_m<DT, TT, kFwd>(kmode, share, kind) : vec_kernel_m<DT, TT, kBwd>(kmode, share, kind);
}

// The vector kernel instance for a plan that vec_geometry accepted, in the
// scheme `kmode` (VecConfig::kmode).
const void* vec_kernel(const Plan& p, int kmode, VecKind kind)
{
    const bool share = p.t1[2] == 0 && p.t2[2] == 0;
    const int tt = p.tdtype;
    switch (p.dtype) {
    case ROPE_DTYPE_F32:
        if (tt == ROPE_DTYPE_F16) return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_F16>(p.dir, kmode, share, kind);
        if (tt == ROPE_DTYPE_BF16) return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_BF16>(p.dir, kmode, share, kind);
        return vec_kernel_t<ROPE_DTYPE_F32, ROPE_DTYPE_F32>(p.dir, kmode, share, kind);
    case ROPE_DTYPE_F16:
        return tt == ROPE_DTYPE_F32 ? vec_kernel_t<ROPE_DTYPE_F16, ROPE_DTYPE_F32>(p.dir, kmode, share, kind)
                                    : vec_kernel_t<ROPE_DTYPE_F16, ROPE_DTYPE_F16>(p.dir, kmode, share, kind);
    default:
        return tt == ROPE_DTYPE_F32 ? vec_kernel_t<ROPE_DTYPE_BF16, ROPE_DTYPE_F32>(p.dir, kmode, share, kind)
                                    : vec_kernel_t<ROPE_DTYPE_BF16, ROPE_DTYPE_BF16>(p.dir, kmode, share, kind);
    }
}

// Launch the vector kernel; `a` is complete (vec_geometry + finish_vec_args).
// a.src set means out of place.
hipError_t launch_vec(const Plan& p, const VecArgs& a, const VecConfig& cfg, hipStream_t stream)
{
    const uint32_t threads = a.span * a.HL * a.GL;
    const void* fn = vec_kernel(p, cfg.kmode, a.src ? kVecOut : kVecOne);
    if (fn == nullptr) return hipErrorInvalidDeviceFunction;
    void* args[] = {const_cast<VecArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(vec_grid(a, cfg)), dim3(threads), args, 0, stream);
}

template <int DT, int TT, bool POS>
const void* scalar_kernel_t(int dir, int mode)
{
    if (dir == kFwd)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kFwd, kModeIL, POS>)
                               : reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kFwd, kModeRH, POS>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kBwd, kModeIL, POS>)
                           : reinterpret_cast<const void*>(&rope_scalar_kernel<DT, TT, kBwd, kModeRH, POS>);
}

template <int DT, int TT>
const void* scalar_kernel_p(bool pos, int dir, int mode)
{
    return pos ? scalar_kernel_t<DT, TT, true>(dir, mode) : scalar_kernel_t<DT, TT, false>(dir, mode);
}

template <int DT>
const void* scalar_kernel_dt(int tt, bool pos, int dir, int mode)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return scalar_kernel_p<DT, ROPE_DTYPE_F32>(pos, dir, mode);
    case ROPE_DTYPE_F16: return scalar_kernel_p<DT, ROPE_DTYPE_F16>(pos, dir, mode);
    default: return scalar_kernel_p<DT, ROPE_DTYPE_BF16>(pos, dir, mode);
    }
}

hipError_t launch_scalar(const Plan& p, int cus, hipStream_t stream)
{
    ScalarArgs a;
    a.x = p.x; a.r1 = p.r1; a.r2 = p.r2;
    a.pos = p.pos; a.inv_freq = p.inv_freq; a.pos_sb = p.pos_sb; a.pos_ss = p.pos_ss;
    a.S = p.S; a.N = p.N; a.D = p.D; a.start = p.start; a.L = p.L;
    a.half = p.half;
    a.pairs = p.L / 2;
    a.items = p.B * p.S * p.N * a.pairs;
    a.t1b = p.t1[0]; a.t1s = p.t1[1]; a.t1n = p.t1[2];
    a.t2b = p.t2[0]; a.t2s = p.t2[1]; a.t2n = p.t2[2];
    const uint32_t threads = 256;
    uint64_t grid = (uint64_t)cus * 8;
    grid = std::max<uint64_t>(1, std::min<uint64_t>(grid, (a.items + threads - 1) / threads));
    const void* fn;
    switch (p.dtype) {
    case ROPE_DTYPE_F32: fn = scalar_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    case ROPE_DTYPE_F16: fn = scalar_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    default: fn = scalar_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(threads), args, 0, stream);
}

template <int DT, int TT, bool POS>
const void* rows_kernel_t(int dir, int mode)
{
    if (dir == kFwd)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kFwd, kModeIL, POS>)
                               : reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kFwd, kModeRH, POS>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kBwd, kModeIL, POS>)
                           : reinterpret_cast<const void*>(&rope_rows_kernel<DT, TT, kBwd, kModeRH, POS>);
}

template <int DT, int TT>
const void* rows_kernel_p(bool pos, int dir, int mode)
{
    return pos ? rows_kernel_t<DT, TT, true>(dir, mode) : rows_kernel_t<DT, TT, false>(dir, mode);
}

template <int DT>
const void* rows_kernel_dt(int tt, bool pos, int dir, int mode)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return rows_kernel_p<DT, ROPE_DTYPE_F32>(pos, dir, mode);
    case ROPE_DTYPE_F16: return rows_kernel_p<DT, ROPE_DTYPE_F16>(pos, dir, mode);
    default: return rows_kernel_p<DT, ROPE_DTYPE_BF16>(pos, dir, mode);
    }
}

// Launch shape of the row kernel: up to 256 threads per row (longer rows
// loop), as many whole rows per block as fit in 256 threads, one block per
// row group while the grid fits the dispatch packet.
struct RowShape {
    uint32_t tpr = 1, rpb = 1, threads = 1, groups = 0, grid = 0;
};

bool rows_shape(const Plan& p, RowShape* r)
{
    const uint64_t rows = (uint64_t)p.B * p.S * p.N;
    if (rows >= (1ull << 31)) return false;
    const uint32_t pairs = (uint32_t)(p.L / 2);
    r->tpr = std::min<uint32_t>(pairs, 256);
    r->rpb = 256 / r->tpr;
    r->threads = r->tpr * r->rpb;
    r->groups = (uint32_t)((rows + r->rpb - 1) / r->rpb);
    r->grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(r->groups, kMaxGridItems / r->threads));
    return true;
}

hipError_t launch_rows(const Plan& p, const RowShape& r, hipStream_t stream)
{
    RowArgs a;
    a.x = p.x; a.r1 = p.r1; a.r2 = p.r2;
    a.pos = p.pos; a.inv_freq = p.inv_freq; a.pos_sb = p.pos_sb; a.pos_ss = p.pos_ss;
    a.D = p.D; a.start = p.start;
    a.t1b = p.t1[0]; a.t1s = p.t1[1]; a.t1n = p.t1[2];
    a.t2b = p.t2[0]; a.t2s = p.t2[1]; a.t2n = p.t2[2];
    a.L = (uint32_t)p.L;
    a.pairs = (uint32_t)(p.L / 2);
    a.half = (uint32_t)std::max<int64_t>(1, p.half);
    a.half_div = make_fastdiv(a.half);
    a.rows = (uint32_t)(p.B * p.S * p.N);
    a.N = (uint32_t)p.N;
    a.rpb = r.rpb;
    a.tpr = r.tpr;
    a.groups = r.groups;
    a.tpr_div = make_fastdiv(r.tpr);
    a.n_div = make_fastdiv((uint32_t)p.N);
    a.s_div = make_fastdiv((uint32_t)p.S);
    const void* fn;
    switch (p.dtype) {
    case ROPE_DTYPE_F32: fn = rows_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    case ROPE_DTYPE_F16: fn = rows_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    default: fn = rows_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.pos != nullptr, p.dir, p.mode); break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3(r.grid), dim3(r.threads), args, 0, stream);
}

// One tensor's launch, decided on the host.
struct Launch {
    Plan p;
    bool vec = false;
    VecArgs a{};
    VecConfig cfg;
    bool rows = false;  // row kernel (else the 64-bit scalar kernel) when not vec
    RowShape rs;
};

// In place, rotate_half: the pair-owner scheme requests each half with its
// own wave instruction, which covers whole 128-byte lines only when the
// halves start and end on line boundaries (e.g. a whole bf16 head of 128
// lanes). Otherwise take the own-vector scheme, whose threads cover the
// slice's whole lines -- when a row's threads fit one wave, as that scheme
// needs. Measured on MI355X, (16,4096,32,128) bf16 forward: lanes [64,128)
// 113 -> 86 us (the interleave slice of the same bytes takes 85 us), lanes
// [0,32) 95 -> 74 us. With the partner loaded from memory instead of taken
// from its lane, each line was requested twice: 100 and 76 us.
bool use_rh_own(const Plan& p, VecArgs* a)
{
    const int64_t es = p.esize;
    const int64_t half_bytes = p.half * es;
    if ((p.start * es) % 128 == 0 && half_bytes % 128 == 0) return false;   // halves on whole lines
    VecArgs own = *a;
    own.span = 2 * own.nvec;   // the whole slice
    cover_whole_lines(p, &own);
    if (own.span > 64) {       // the whole lines would not fit one wave: the slice alone may
        own.lo_vec = own.start_vec;
        own.span = 2 * own.nvec;
    }
    if (own.span > 64) return false;   // a row's threads would span waves
    *a = own;
    return true;
}

void prepare(Launch* L)
{
    L->vec = vec_geometry(L->p, &L->a);
    if (L->vec) {
        int kmode = L->p.mode;
        if (L->p.mode == kModeRH) {
            if (use_rh_own(L->p, &L->a)) kmode = kModeRHOwn;
        } else {
            cover_whole_lines(L->p, &L->a);
        }
        L->cfg = choose_vec_config(L->p, L->a, u_in_place(L->p.dtype, L->p.tdtype), kmode);
        L->vec = finish_vec_args(L->p, L->cfg, &L->a);
        // the own-vector scheme in place needs single-wave blocks
        if (L->vec && kmode == kModeRHOwn && L->a.span * L->a.HL * L->a.GL > 64) L->vec = false;
    }
    if (!L->vec) L->rows = rows_shape(L->p, &L->rs);
}

hipError_t launch_one(const Launch& L, int cus, hipStream_t s)
{
    if (L.vec) return launch_vec(L.p, L.a, L.cfg, s);
    return L.rows ? launch_rows(L.p, L.rs, s) : launch_scalar(L.p, cus, s);
}

// Out of place (p.src is the input, p.x the output; distinct buffers). The
// vector kernel reads src and writes x in one pass over whole rows: the
// slice rotated, the other vectors copied. Inputs it cannot take (alignment,
// sizes) get a device copy of src into x and then the in-place plan on x.
//
// Launch shape, measured on MI355X over six shapes (bf16 and fp32; slices
// of 1/3, 1/2 and all of the row; interleave and rotate_half; slices on and
// off 128-byte line boundaries), heads per thread 1-2, blocks of 64-256
// threads, and plain or nontemporal loads and stores chosen separately: two
// heads per thread, 64-thread blocks and nontemporal loads and stores was
// within 2% of the best on five shapes and 8% on the sixth (a rotate_half
// slice off line boundaries). One head per thread was 10-15% slower on the
// rotate_half shapes and the 192-lane rows. With every vector stored by one
// instruction (see the vector kernel) the long-context shard (16,8192,32,128)
// bf16 takes 322 us, 6.8 TB/s of read plus write, against 420 us for a
// plain device copy of the same tensor.
void prepare_out(Launch* L)
{
    L->vec = vec_geometry(L->p, &L->a) && aligned16(L->p.src);
    if (L->vec) {
        L->a.src = static_cast<const v4u*>(L->p.src);
        L->a.lo_vec = 0;
        L->a.span = L->a.row_vecs;
        // rotate_half: the partner vector from its lane when a row fits a wave
        const int kmode = L->p.mode == kModeIL ? kModeIL : L->a.span <= 64 ? kModeRHOwn : kModeRHOwnLoad;
        L->cfg = choose_vec_config(L->p, L->a, kUOut, kmode);
        L->vec = finish_vec_args(L->p, L->cfg, &L->a);
        // the lane exchange needs single-wave blocks
        if (L->vec && kmode == kModeRHOwn && L->a.span * L->a.HL * L->a.GL > 64) L->vec = false;
    }
    if (!L->vec) L->rows = rows_shape(L->p, &L->rs);
}

hipError_t launch_out(const Launch& L, int cus, hipStream_t s)
{
    if (L.vec) return launch_vec(L.p, L.a, L.cfg, s);
    hipError_t err = hipMemcpyAsync(L.p.x, L.p.src, (size_t)L.p.bytes, hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return err;
    return L.rows ? launch_rows(L.p, L.rs, s) : launch_scalar(L.p, cus, s);
}

rope_status_t device_cus(int* cus)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("hipGetDevice: ") + hipGetErrorString(err));
    *cus = cu_count(dev);
    return ROPE_OK;
}

rope_status_t run(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                  const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                  const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                  rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                  void* stream, Direction dir)
{
    Launch L;
    std::string why;
    rope_status_t st = make_plan(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                 table_dtype, mode, partial_slice, dir, &L.p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    prepare(&L);
    hipError_t err = launch_one(L, cus, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Launch plan of the position vector kernel; false if the plan needs a
// general kernel (alignment, sizes), as for the table vector kernel. A
// position's heads take up to kPosLanes threads (HL head lanes of span
// threads, U heads each, in chunks past U*HL heads); when they fill
// fewer threads, a block takes kPosLanes/lanes positions, as many as its
// LDS table holds.
// The vector geometry both position kernels share: alignment, sizes, the
// slice in vectors and the rotate_half groups. out: also src aligned.
static bool pos_vectors(const Plan& p, PosArgs* a, bool out)
{
    const int64_t es = p.esize;
    if (!aligned16(p.x) || (out && !aligned16(p.src)) || (p.D * es) % 16 || (p.start * es) % 16) return false;
    const int64_t unit_bytes = p.mode == kModeIL ? p.L * es : (p.L / 2) * es;
    if (unit_bytes % 16 || p.L / 2 > kPosLds) return false;
    if (p.mode == kModeRH && (p.half * es) % 16) return false;   // half-groups of whole vectors
    const int64_t kMax = (1ll << 32) - 1;
    if (p.B * p.S * p.N * (p.D * es / 16) > kMax || p.N >= (1ll << 31) || p.B * p.S >= (1ll << 31)) return false;
    a->x = static_cast<v4u*>(p.x);
    a->src = static_cast<const v4u*>(p.src);
    a->pos = p.pos;
    a->inv_freq = p.inv_freq;
    a->pos_sb = p.pos_sb;
    a->pos_ss = p.pos_ss;
    a->row_vecs = (uint32_t)(p.D * es / 16);
    a->start_vec = (uint32_t)(p.start * es / 16);
    a->half_vecs = p.mode == kModeRH ? (uint32_t)(p.half * es / 16) : 0;
    a->gvec = 2 * a->half_vecs;
    a->nvec = (uint32_t)(unit_bytes / 16);
    return true;
}

// Heads, positions per block and the grid, once the vectors a row's
// threads cover (lo_vec, span) are set: U heads per thread, a position's
// heads over up to `lanes_target` threads (`vheads_lanes` with the batches
// as heads).
static bool pos_launch_shape(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid, int U,
                             uint32_t lanes_target, uint32_t vheads_lanes)
{
    if (a->span < 1 || a->span > 256) return false;
    // positions shared by the batch (batch stride 0), and too few heads to
    // fill a block: the batches become heads of one position per s (see
    // PosArgs::vheads). With more heads the (b,s) order is kept, which
    // streams through x: the GQA Q layout (32,4096,16,128) took 197 us with
    // the batches as heads, where one (b,s) per block takes 167 us.
    a->vheads = p.pos_sb == 0 && p.B > 1 && (uint64_t)a->span * p.N < lanes_target;
    const uint64_t heads = a->vheads ? (uint64_t)p.B * p.N : (uint64_t)p.N;
    const uint64_t positions = a->vheads ? (uint64_t)p.S : (uint64_t)p.B * p.S;
    if (heads >= (1ull << 31) || positions >= (1ull << 31)) return false;
    a->N = (uint32_t)heads;
    a->pairs = (uint32_t)(p.L / 2);
    const uint32_t target = a->vheads ? vheads_lanes : lanes_target;   // threads a position's heads fill
    a->U = (uint32_t)U;
    a->HL = (uint32_t)std::min<uint64_t>(std::max<uint32_t>(1, target / a->span), heads);
    a->chunks = (uint32_t)((heads + (uint64_t)a->HL * U - 1) / ((uint64_t)a->HL * U));
    a->lanes = a->span * a->HL;
    a->P = a->lanes < target ? std::min<uint32_t>(target / a->lanes, kPosLds / a->pairs) : 1;
    a->entries = a->P * a->pairs;
    if (a->entries > (uint32_t)kPosLds) return false;
    a->bs = (uint32_t)positions;
    const uint64_t items = (((uint64_t)a->bs + a->P - 1) / a->P) * a->chunks;
    if (items >= (1ull << 31)) return false;
    a->items = (uint32_t)items;
    *threads = a->P * a->lanes;
    *grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(items, kMaxGridItems / *threads));
    // XCD runs of about kXcdRunBytes of x in whole position groups (all the
    // head chunks of P positions), as for the table kernels
    {
        const uint64_t group_bytes = (uint64_t)a->P * heads * (uint64_t)p.D * (uint64_t)p.esize;
        const uint64_t groups = std::max<uint64_t>(1, (kXcdRunBytes + group_bytes / 2) / group_bytes);
        const uint64_t P = std::min<uint64_t>(groups * a->chunks, 1u << 24);
        a->xcd_group = (uint32_t)P;
        a->xcd_full = 0;
        a->xcd_div = make_fastdiv(8);
        if (P > 1 && 8 * P <= *grid) {
            a->xcd_full = (uint32_t)(*grid / (8 * P) * (8 * P));
            a->xcd_div = make_fastdiv((uint32_t)(8 * P));
        }
    }
    a->span_div = make_fastdiv(a->span);
    a->lanes_div = make_fastdiv(a->lanes);
    a->pairs_div = make_fastdiv(a->pairs);
    a->chunk_div = make_fastdiv(a->chunks);
    a->s_div = make_fastdiv((uint32_t)p.S);
    a->nx_div = make_fastdiv((uint32_t)std::max<int64_t>(1, p.N));
    return true;
}

bool pos_geometry(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid)
{
    if (!pos_vectors(p, a, false)) return false;
    a->lo_vec = a->start_vec;
    a->span = a->nvec;
    if (p.mode == kModeIL) {
        VecArgs lines{};
        lines.lo_vec = a->lo_vec;
        lines.span = a->span;
        cover_whole_lines(p, &lines);
        a->lo_vec = lines.lo_vec;
        a->span = lines.span;
    }
    // more heads per thread when a row's threads also carry the dropped
    // vectors of whole-line coverage (see rope_pos_kernel)
    const int u = a->span > a->nvec ? kUPosLines : 1;
    return pos_launch_shape(p, a, threads, grid, u, kPosLanes, kPosVheadsLanes);
}

// Out of place: the threads of a row cover all of its vectors.
bool pos_geometry_out(const Plan& p, PosArgs* a, uint32_t* threads, uint32_t* grid)
{
    if (!pos_vectors(p, a, true)) return false;
    a->lo_vec = 0;
    a->span = a->row_vecs;
    return pos_launch_shape(p, a, threads, grid, pos_out_heads(p.mode), pos_out_lanes(p.mode),
                            pos_out_lanes(p.mode));
}

template <int DT, int TT, int DIR>
const void* pos_kernel_d(int mode, bool out, bool xchg, int u)
{
    if (out)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeIL, false>)
               : xchg          ? reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeRH, true>)
                               : reinterpret_cast<const void*>(&rope_pos_out_kernel<DT, TT, DIR, kModeRH, false>);
    if (u == 1)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, false, 1>)
                               : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, false, 1>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, false, kUPosLines>)
                           : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, false, kUPosLines>);
}

template <int DT, int TT, int DIR>
const void* pos_multi_kernel_d(int mode, int u)
{
    if (u == 1)
        return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, true, 1>)
                               : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, true, 1>);
    return mode == kModeIL ? reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeIL, true, kUPosLines>)
                           : reinterpret_cast<const void*>(&rope_pos_kernel<DT, TT, DIR, kModeRH, true, kUPosLines>);
}

template <int DT, int TT>
const void* pos_multi_kernel_t(int dir, int mode, int u)
{
    return dir == kFwd ? pos_multi_kernel_d<DT, TT, kFwd>(mode, u) : pos_multi_kernel_d<DT, TT, kBwd>(mode, u);
}

template <int DT>
const void* pos_multi_kernel_dt(int tt, int dir, int mode, int u)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return pos_multi_kernel_t<DT, ROPE_DTYPE_F32>(dir, mode, u);
    case ROPE_DTYPE_F16: return pos_multi_kernel_t<DT, ROPE_DTYPE_F16>(dir, mode, u);
    default: return pos_multi_kernel_t<DT, ROPE_DTYPE_BF16>(dir, mode, u);
    }
}

// the position kernel over several tensors at once
const void* pos_multi_kernel(const Plan& p, int u)
{
    switch (p.dtype) {
    case ROPE_DTYPE_F32: return pos_multi_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.dir, p.mode, u);
    case ROPE_DTYPE_F16: return pos_multi_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.dir, p.mode, u);
    default: return pos_multi_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.dir, p.mode, u);
    }
}

template <int DT, int TT>
const void* pos_kernel_t(int dir, int mode, bool out, bool xchg, int u)
{
    return dir == kFwd ? pos_kernel_d<DT, TT, kFwd>(mode, out, xchg, u) : pos_kernel_d<DT, TT, kBwd>(mode, out, xchg, u);
}

template <int DT>
const void* pos_kernel_dt(int tt, int dir, int mode, bool out, bool xchg, int u)
{
    switch (tt) {
    case ROPE_DTYPE_F32: return pos_kernel_t<DT, ROPE_DTYPE_F32>(dir, mode, out, xchg, u);
    case ROPE_DTYPE_F16: return pos_kernel_t<DT, ROPE_DTYPE_F16>(dir, mode, out, xchg, u);
    default: return pos_kernel_t<DT, ROPE_DTYPE_BF16>(dir, mode, out, xchg, u);
    }
}

// out: the out-of-place kernel; xchg: its lane exchange (a row's threads
// within one wave: rows of 64/k vectors)
const void* pos_kernel(const Plan& p, bool out, bool xchg = false, int u = kUPosLines)
{
    switch (p.dtype) {
    case ROPE_DTYPE_F32: return pos_kernel_dt<ROPE_DTYPE_F32>(p.tdtype, p.dir, p.mode, out, xchg, u);
    case ROPE_DTYPE_F16: return pos_kernel_dt<ROPE_DTYPE_F16>(p.tdtype, p.dir, p.mode, out, xchg, u);
    default: return pos_kernel_dt<ROPE_DTYPE_BF16>(p.tdtype, p.dir, p.mode, out, xchg, u);
    }
}

// Tables from positions, one planned tensor: the position vector kernel,
// else the row or scalar kernel with their POS form.
hipError_t launch_pos_plan(const Plan& p, int cus, hipStream_t s)
{
    PosArgs a{};
    uint32_t threads = 0, grid = 0;
    if (pos_geometry(p, &a, &threads, &grid)) {
        void* args[] = {&a};
        return hipLaunchKernel(pos_kernel(p, false, false, (int)a.U), dim3(grid), dim3(threads), args, 0, s);
    }
    RowShape rs;
    return rows_shape(p, &rs) ? launch_rows(p, rs, s) : launch_scalar(p, cus, s);
}

rope_status_t run_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype, const int64_t* positions,
                      const int64_t positions_shape[2], const int64_t positions_strides[2], const double* inv_freq,
                      rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2], void* stream,
                      Direction dir)
{
    Plan p;
    std::string why;
    rope_status_t st = make_plan_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                                     table_dtype, mode, partial_slice, dir, &p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (p.noop) return ROPE_OK;
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    const hipError_t err = launch_pos_plan(p, cus, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Several tensors with one set of positions (the Q and K of a layer): every
// tensor is checked first; when they share B, S, D and the vector geometry,
// one launch of the position kernel takes the heads of all of them, each
// pair's cos and sin evaluated once per position for every tensor;
// otherwise one launch per tensor.
rope_status_t run_pos_multi(int32_t count, void* const xs[], const int64_t (*x_shapes)[4], rope_dtype_t dtype,
                            const int64_t* positions, const int64_t positions_shape[2],
                            const int64_t positions_strides[2], const double* inv_freq, rope_dtype_t table_dtype,
                            int64_t mode, const int64_t partial_slice[2], void* stream, Direction dir)
{
    if (count < 0 || count > kMultiMax)
        return set_error(ROPE_ERR_INVALID, "count must be in [0, " + std::to_string(kMultiMax) + "]");
    if (count == 0) return ROPE_OK;
    if (xs == nullptr || x_shapes == nullptr) return set_error(ROPE_ERR_NULLPTR, "xs or x_shapes is NULL");
    Plan P[kMultiMax];
    int live = 0;
    for (int i = 0; i < count; ++i) {
        std::string why;
        rope_status_t st = make_plan_pos(xs[i], x_shapes[i], dtype, positions, positions_shape, positions_strides,
                                         inv_freq, table_dtype, mode, partial_slice, dir, &P[live], &why);
        if (st != ROPE_OK) return set_error(st, "tensor " + std::to_string(i) + ": " + why);
        if (!P[live].noop) ++live;
    }
    if (live == 0) return ROPE_OK;
    {
        std::string why;
        rope_status_t st = check_disjoint(P, live, &why);
        if (st != ROPE_OK) return set_error(st, why);
    }
    int cus = 0;
    rope_status_t st = device_cus(&cus);
    if (st != ROPE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool together = live > 1;
    PosArgs each[kMultiMax];
    uint64_t heads = 0;
    for (int i = 0; i < live && together; ++i) {
        uint32_t t = 0, g = 0;
        together = P[i].B == P[0].B && P[i].S == P[0].S && P[i].D == P[0].D &&
                   pos_geometry(P[i], &each[i], &t, &g) && each[i].lo_vec == each[0].lo_vec &&
                   each[i].span == each[0].span;
        heads += (uint64_t)P[i].N;
    }
    hipError_t err = hipSuccess;
    PosArgs m{};
    uint32_t threads = 0, grid = 0;
    if (together && heads < (1ull << 31)) {
        Plan q = P[0];
        q.N = (int64_t)heads;
        m = each[0];
        together = pos_launch_shape(q, &m, &threads, &grid, (int)m.U, kPosLanes, kPosVheadsLanes);
        uint32_t first = 0;
        for (int i = 0; i < kMultiMax; ++i) {
            m.xs[i] = i < live ? each[i].x : nullptr;
            m.nt[i] = i < live ? (uint32_t)P[i].N : 0;
            m.hoff[i] = i < live ? first : 0xFFFFFFFFu;
            if (i < live) first += (uint32_t)P[i].N;
        }
    } else {
        together = false;
    }
    if (together) {
        void* args[] = {&m};
        err = hipLaunchKernel(pos_multi_kernel(P[0], (int)m.U), dim3(grid), dim3(threads), args, 0, s);
    } else {
        for (int i = 0; i < live && err == hipSuccess; ++i) err = launch_pos_plan(P[i], cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Out of place from positions: the position out-of-place kernel, else a
// device copy of x into y and the in-place position plan on y.
rope_status_t run_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                          const int64_t* positions, const int64_t positions_shape[2],
                          const int64_t positions_strides[2], const double* inv_freq, rope_dtype_t table_dtype,
                          int64_t mode, const int64_t partial_slice[2], void* stream, Direction dir)
{
    Plan p;
    std::string why;
    rope_status_t st = make_plan_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides,
                                         inv_freq, table_dtype, mode, partial_slice, dir, &p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (p.noop) return ROPE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (p.copy_only) {
        err = hipMemcpyAsync(p.x, p.src, (size_t)p.bytes, hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("copy: ") + hipGetErrorString(err));
        return ROPE_OK;
    }
    if (p.src == nullptr)   // y == x: the in-place call
        return run_pos(p.x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                       mode, partial_slice, stream, dir);
    int cus = 0;
    if ((st = device_cus(&cus)) != ROPE_OK) return st;
    PosArgs a{};
    uint32_t threads = 0, grid = 0;
    if (pos_geometry_out(p, &a, &threads, &grid)) {
        void* args[] = {&a};
        const bool xchg = a.span <= 64 && 64 % a.span == 0;
        err = hipLaunchKernel(pos_kernel(p, true, xchg), dim3(grid), dim3(threads), args, 0, s);
    } else {
        err = hipMemcpyAsync(p.x, p.src, (size_t)p.bytes, hipMemcpyDeviceToDevice, s);
        if (err == hipSuccess) err = launch_pos_plan(p, cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Out of place: y = x with the slice rotated (y == x is the in-place call).
rope_status_t run_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                      const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                      const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                      rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                      void* stream, Direction dir)
{
    Launch L;
    std::string why;
    rope_status_t st = make_plan_out(y, x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                     table_dtype, mode, partial_slice, dir, &L.p, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (L.p.copy_only) {
        err = hipMemcpyAsync(L.p.x, L.p.src, (size_t)L.p.bytes, hipMemcpyDeviceToDevice, s);
    } else {
        int cus = 0;
        if ((st = device_cus(&cus)) != ROPE_OK) return st;
        if (L.p.src == nullptr) {
            prepare(&L);
            err = launch_one(L, cus, s);
        } else {
            prepare_out(&L);
            err = launch_out(L, cus, s);
        }
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Projection with a rotary epilogue: one launch of rope_proj_kernel.
template <int DT, int BN>
hipError_t launch_proj(const ProjArgs& a, int tdt, uint32_t grid, hipStream_t s)
{
    const dim3 block(ProjTile<BN>::THREADS);
    if (tdt == ROPE_DTYPE_BF16)
        hipLaunchKernelGGL((rope_proj_kernel<DT, BN, ROPE_DTYPE_BF16>), dim3(grid), block, 0, s, a);
    else if (tdt == ROPE_DTYPE_F16)
        hipLaunchKernelGGL((rope_proj_kernel<DT, BN, ROPE_DTYPE_F16>), dim3(grid), block, 0, s, a);
    else
        hipLaunchKernelGGL((rope_proj_kernel<DT, BN, ROPE_DTYPE_F32>), dim3(grid), block, 0, s, a);
    return hipGetLastError();
}

template <int DT, int EPI>
hipError_t launch_proj_sq(const ProjArgs& a, int tdt, uint32_t grid, hipStream_t s)
{
    const dim3 block(ProjSq::THREADS);
    if (tdt == ROPE_DTYPE_BF16)
        hipLaunchKernelGGL((rope_proj_sq_kernel<DT, ROPE_DTYPE_BF16, EPI>), dim3(grid), block, 0, s, a);
    else if (tdt == ROPE_DTYPE_F16)
        hipLaunchKernelGGL((rope_proj_sq_kernel<DT, ROPE_DTYPE_F16, EPI>), dim3(grid), block, 0, s, a);
    else
        hipLaunchKernelGGL((rope_proj_sq_kernel<DT, ROPE_DTYPE_F32, EPI>), dim3(grid), block, 0, s, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_proj_sq_epi(const ProjArgs& a, int tdt, uint32_t grid, hipStream_t s)
{
    switch (a.epi) {
    case 0: return launch_proj_sq<DT, 0>(a, tdt, grid, s);
    case 1: return launch_proj_sq<DT, 1>(a, tdt, grid, s);
    default: return launch_proj_sq<DT, -1>(a, tdt, grid, s);
    }
}

// A projection call's checked plan, kernel arguments and kernel choice.
struct ProjLaunch {
    ProjPlan q;
    ProjArgs a{};
    bool sq = false;            // square 256 x 256 tiles (else tiles of whole heads)
    int BM = 0, BN = 0, threads = 0;
    uint32_t grid = 0;
    int tdt = ROPE_DTYPE_BF16;  // table type the kernel is instantiated for
};

rope_status_t prepare_proj(void* y, rope_dtype_t y_dtype, const void* x, const void* w, rope_dtype_t dtype,
                           const int64_t y_shape[4], int64_t K,
                           const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                           const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2], ProjLaunch* P,
                           std::string* why)
{
    ProjPlan& q = P->q;
    rope_status_t st = make_proj_plan(y, y_dtype, x, w, dtype, y_shape, K, r1, r1_shape, r1_strides, r2, r2_shape,
                                      r2_strides, table_dtype, mode, partial_slice, &q, why);
    if (st != ROPE_OK || q.noop) return st;
    const Plan& p = q.rope;
    ProjArgs& a = P->a;
    a.x = static_cast<const uint16_t*>(q.x);
    a.w = static_cast<const uint16_t*>(q.w);
    a.y = q.y;
    a.ydt = q.out_dtype;
    a.r1 = p.r1;
    a.r2 = p.r2;
    a.t1b = p.t1[0]; a.t1s = p.t1[1]; a.t1n = p.t1[2];
    a.t2b = p.t2[0]; a.t2s = p.t2[1]; a.t2n = p.t2[2];
    // the plan bounds x and w below 2^31 elements, so M, N and K fit in 32 bits
    a.M = (int32_t)(p.B * p.S);
    a.N = (int32_t)(p.N * p.D);
    a.K = (int32_t)q.K;
    a.S = (int32_t)p.S;
    a.Dh = (int32_t)p.D;
    a.start = (int32_t)p.start;
    a.L = (int32_t)p.L;
    a.half = p.L > 0 ? (int32_t)p.half : 1;
    // Square 256 x 256 tiles when K is a whole number of stage pairs (128 k)
    // and every rotation group lies within one 256-lane column tile;
    // otherwise tiles of whole heads, or of part of one wider head: 192 lanes
    // (384 tokens) for heads of a multiple of 3 lanes, else 128 lanes (256
    // tokens).
    const bool sq = P->sq = a.K % (2 * kProjBK) == 0 &&
                    proj_groups_in_column_tiles(p.D, (int64_t)a.N, p.start, p.L, a.half, ProjSq::BN);
    const int BN = P->BN = sq ? ProjSq::BN : (int)proj_tile_lanes(p.D);
    const int BM = P->BM = sq ? ProjSq::BM : BN == 192 ? ProjTile<192>::BM : ProjTile<128>::BM;
    const int threads = P->threads = sq ? ProjSq::THREADS : BN == 192 ? ProjTile<192>::THREADS : ProjTile<128>::THREADS;
    const int64_t MB = (a.M + BM - 1) / BM, NB = (a.N + BN - 1) / BN;
    // the dispatch packet holds the grid in work-items as a 32-bit number
    if (MB * NB > (int64_t)(0xFFFFFFFFull / threads))
    {
        *why = "the projection's grid exceeds one launch";
        return ROPE_ERR_UNSUPPORTED;
    }
    a.MB = (int32_t)MB;
    a.NB = (int32_t)NB;
    // Measured on MI355X on the (4*4096 tokens, 1536) x (24576, 1536) MLA
    // projection: groups of 4 M-tiles with each XCD taking a contiguous run
    // of tiles.
    a.group_m = 4;
    a.xcd_chunk = (int32_t)(MB * NB / 8);
    a.s_div = make_fastdiv((uint32_t)p.S);
    a.dh_div = make_fastdiv((uint32_t)p.D);
    // The vector epilogue: whole 8-lane slice vectors whose partners are in
    // the vector or a whole vector away, and 16-byte aligned runs of 8 cos
    // and 8 sin values in every table row.
    {
        const int64_t per = 16 / p.tesize;                 // table lanes per 16 bytes
        bool f = p.L > 0 && p.start % 8 == 0 && p.L % 8 == 0 && (p.half == 1 || p.half % 8 == 0);
        f = f && aligned16(p.r1) && aligned16(p.r2);
        for (int k = 0; k < 3 && f; ++k) f = p.t1[k] % per == 0 && p.t2[k] % per == 0;
        a.fast = f ? 1 : 0;
    }
    // The square tiles' epilogue: the vector epilogue when the slice is
    // whole vectors (fast) whose partners are in the vector (interleave) or
    // whole vectors away within one wave's 128 lanes, with the tables' rows
    // staged in LDS when both tables are shared by all heads and a row's L
    // values take 16, 32, 64 or 128 bytes that 32-bit byte offsets reach;
    // otherwise the general one.
    a.epi = -1;
    a.tab_crl = -1;
    if (sq) {
        if (p.L == 0) {
            a.epi = 0;
        } else if (a.fast && (a.half == 1 || proj_groups_in_column_tiles(p.D, (int64_t)a.N, p.start, p.L, a.half,
                                                                          ProjSq::BN / 2))) {
            a.epi = a.half == 1 ? 0 : 1;
            if (p.t1[2] == 0 && p.t2[2] == 0) {
                const int64_t row = p.L * p.tesize;
                int crl = -1;
                for (int k = 0; k < 4; ++k)
                    if (row == (int64_t)16 << k) crl = k;
                const int64_t reach1 = ((p.B - 1) * p.t1[0] + (p.S - 1) * p.t1[1] + p.L) * p.tesize;
                const int64_t reach2 = ((p.B - 1) * p.t2[0] + (p.S - 1) * p.t2[1] + p.L) * p.tesize;
                if (crl >= 0 && reach1 <= (int64_t)UINT32_MAX && reach2 <= (int64_t)UINT32_MAX) a.tab_crl = crl;
            }
        }
    }
    P->grid = (uint32_t)(MB * NB);
    P->tdt = p.L > 0 ? p.tdtype : (int)ROPE_DTYPE_BF16;
    return ROPE_OK;
}

rope_status_t run_proj(void* y, rope_dtype_t y_dtype, const void* x, const void* w, rope_dtype_t dtype,
                       const int64_t y_shape[4], int64_t K,
                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2], void* stream)
{
    ProjLaunch P;
    std::string why;
    rope_status_t st = prepare_proj(y, y_dtype, x, w, dtype, y_shape, K, r1, r1_shape, r1_strides, r2, r2_shape,
                                    r2_strides, table_dtype, mode, partial_slice, &P, &why);
    if (st != ROPE_OK) return set_error(st, why);
    if (P.q.noop) return ROPE_OK;
    const ProjArgs& a = P.a;
    const uint32_t grid = P.grid;
    const int tdt = P.tdt;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (P.sq)
        err = P.q.in_dtype == ROPE_DTYPE_BF16 ? launch_proj_sq_epi<ROPE_DTYPE_BF16>(a, tdt, grid, s)
                                              : launch_proj_sq_epi<ROPE_DTYPE_F16>(a, tdt, grid, s);
    else if (P.q.in_dtype == ROPE_DTYPE_BF16)
        err = P.BN == 192 ? launch_proj<ROPE_DTYPE_BF16, 192>(a, tdt, grid, s)
                          : launch_proj<ROPE_DTYPE_BF16, 128>(a, tdt, grid, s);
    else
        err = P.BN == 192 ? launch_proj<ROPE_DTYPE_F16, 192>(a, tdt, grid, s)
                          : launch_proj<ROPE_DTYPE_F16, 128>(a, tdt, grid, s);
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

// Several tensors with shared tables: every tensor is checked before any
// launch; tensors that all take the same vector kernel and block size go in
// one launch, otherwise each is launched in turn (same result either way).
rope_status_t run_multi(int32_t count, void* const xs[], const int64_t (*x_shapes)[4], rope_dtype_t dtype,
                        const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                        const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                        rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                        void* stream, Direction dir)
{
    if (count < 0 || count > kMultiMax)
        return set_error(ROPE_ERR_INVALID, "count must be in [0, " + std::to_string(kMultiMax) + "]");
    if (count == 0) return ROPE_OK;
    if (xs == nullptr || x_shapes == nullptr) return set_error(ROPE_ERR_NULLPTR, "xs or x_shapes is NULL");
    Launch L[kMultiMax];
    int live = 0;
    for (int i = 0; i < count; ++i) {
        std::string why;
        rope_status_t st = make_plan(xs[i], x_shapes[i], dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                                     table_dtype, mode, partial_slice, dir, &L[live].p, &why);
        if (st != ROPE_OK) return set_error(st, "tensor " + std::to_string(i) + ": " + why);
        if (!L[live].p.noop) ++live;
    }
    if (live == 0) return ROPE_OK;
    {
        Plan ps[kMultiMax];
        for (int i = 0; i < live; ++i) ps[i] = L[i].p;
        std::string why;
        rope_status_t st = check_disjoint(ps, live, &why);
        if (st != ROPE_OK) return set_error(st, why);
    }
    int cus = 0;
    rope_status_t st = device_cus(&cus);
    if (st != ROPE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int i = 0; i < live; ++i) prepare(&L[i]);

    bool together = live > 1;
    const uint32_t threads = L[0].a.span * L[0].a.HL * L[0].a.GL;
    const void* fn = together && L[0].vec ? vec_kernel(L[0].p, L[0].cfg.kmode, kVecMulti) : nullptr;
    for (int i = 0; i < live && together; ++i) {
        together = L[i].vec && L[i].a.span * L[i].a.HL * L[i].a.GL == threads &&
                   vec_kernel(L[i].p, L[i].cfg.kmode, kVecMulti) == fn && L[i].cfg.grid == 0;
    }
    hipError_t err = hipSuccess;
    if (together) {
        MultiVecArgs m{};
        m.count = (uint32_t)live;
        uint64_t blocks = 0;
        for (int i = 0; i < live; ++i) {
            m.a[i] = L[i].a;
            m.first_block[i] = (uint32_t)blocks;
            blocks += vec_grid(L[i].a, L[i].cfg);
        }
        for (int i = live; i <= kMultiMax; ++i) m.first_block[i] = (uint32_t)blocks;
        if (blocks * threads > kMaxGridItems) together = false;
        if (together) {
            void* args[] = {&m};
            err = hipLaunchKernel(fn, dim3((uint32_t)blocks), dim3(threads), args, 0, s);
        }
    }
    if (!together) {
        for (int i = 0; i < live && err == hipSuccess; ++i) err = launch_one(L[i], cus, s);
    }
    if (err != hipSuccess) return set_error(ROPE_ERR_RUNTIME, std::string("kernel launch: ") + hipGetErrorString(err));
    return ROPE_OK;
}

}  // namespace
}  // namespace rope

extern "C" {

rope_status_t rope_partial_fwd_inplace(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype, mode,
                     partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run(x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype, mode,
                     partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_out(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                   const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                   const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                   rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                   void* stream)
{
    return rope::run_out(y, x, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype,
                         mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_out(void* dx, const void* dy, const int64_t x_shape[4], rope_dtype_t dtype,
                                   const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                   const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                   rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                   void* stream)
{
    return rope::run_out(dx, dy, x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides, table_dtype,
                         mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           void* stream)
{
    return rope::run_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                         mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_pos(void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           void* stream)
{
    return rope::run_pos(x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq, table_dtype,
                         mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_pos_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                                 rope_dtype_t dtype, const int64_t* positions,
                                                 const int64_t positions_shape[2], const int64_t positions_strides[2],
                                                 const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                                                 const int64_t partial_slice[2], void* stream)
{
    return rope::run_pos_multi(count, xs, x_shapes, dtype, positions, positions_shape, positions_strides, inv_freq,
                               table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_pos_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                                 rope_dtype_t dtype, const int64_t* positions,
                                                 const int64_t positions_shape[2], const int64_t positions_strides[2],
                                                 const double* inv_freq, rope_dtype_t table_dtype, int64_t mode,
                                                 const int64_t partial_slice[2], void* stream)
{
    return rope::run_pos_multi(count, xs, x_shapes, dtype, positions, positions_shape, positions_strides, inv_freq,
                               table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const int64_t* positions, const int64_t positions_shape[2],
                                       const int64_t positions_strides[2], const double* inv_freq,
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                             table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_out_pos(void* y, const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const int64_t* positions, const int64_t positions_shape[2],
                                       const int64_t positions_strides[2], const double* inv_freq,
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       void* stream)
{
    return rope::run_out_pos(y, x, x_shape, dtype, positions, positions_shape, positions_strides, inv_freq,
                             table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_fwd_inplace_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                             rope_dtype_t dtype, const void* r1, const int64_t r1_shape[4],
                                             const int64_t r1_strides[4], const void* r2, const int64_t r2_shape[4],
                                             const int64_t r2_strides[4], rope_dtype_t table_dtype, int64_t mode,
                                             const int64_t partial_slice[2], void* stream)
{
    return rope::run_multi(count, xs, x_shapes, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                           table_dtype, mode, partial_slice, stream, rope::kFwd);
}

rope_status_t rope_partial_bwd_inplace_multi(int32_t count, void* const xs[], const int64_t x_shapes[][4],
                                             rope_dtype_t dtype, const void* r1, const int64_t r1_shape[4],
                                             const int64_t r1_strides[4], const void* r2, const int64_t r2_shape[4],
                                             const int64_t r2_strides[4], rope_dtype_t table_dtype, int64_t mode,
                                             const int64_t partial_slice[2], void* stream)
{
    return rope::run_multi(count, xs, x_shapes, dtype, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                           table_dtype, mode, partial_slice, stream, rope::kBwd);
}

rope_status_t rope_partial_check(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                 const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                 const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                 rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2])
{
    rope::Plan p;
    std::string why;
    rope_status_t st = rope::make_plan(const_cast<void*>(x), x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape,
                                       r2_strides, table_dtype, mode, partial_slice, rope::kFwd, &p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    return ROPE_OK;
}

rope_status_t rope_partial_launch_info(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                       const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                       const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                       rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                       int64_t info[ROPE_LAUNCH_INFO_LEN])
{
    if (info == nullptr) return rope::set_error(ROPE_ERR_NULLPTR, "info is NULL");
    for (int i = 0; i < ROPE_LAUNCH_INFO_LEN; ++i) info[i] = 0;
    rope::Launch L;
    std::string why;
    rope_status_t st = rope::make_plan(const_cast<void*>(x), x_shape, dtype, r1, r1_shape, r1_strides, r2, r2_shape,
                                       r2_strides, table_dtype, mode, partial_slice, rope::kFwd, &L.p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    if (L.p.noop) return ROPE_OK;
    rope::prepare(&L);
    if (L.vec) {
        info[0] = ROPE_KERNEL_VECTOR;
        info[1] = rope::vec_grid(L.a, L.cfg);
        info[2] = (int64_t)L.a.span * L.a.HL * L.a.GL;
        info[3] = L.cfg.U;
        info[4] = L.a.HL;
        info[5] = L.a.GL;
        info[6] = L.a.xcd_group;
        info[7] = L.a.span;
    } else if (L.rows) {
        info[0] = ROPE_KERNEL_ROWS;
        info[1] = L.rs.grid;
        info[2] = L.rs.threads;
        info[4] = L.rs.rpb;
        info[7] = L.rs.tpr;
    } else {
        info[0] = ROPE_KERNEL_SCALAR;
        info[2] = 256;
    }
    return ROPE_OK;
}

rope_status_t rope_partial_launch_info_pos(const void* x, const int64_t x_shape[4], rope_dtype_t dtype,
                                           const int64_t* positions, const int64_t positions_shape[2],
                                           const int64_t positions_strides[2], const double* inv_freq,
                                           rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                           int64_t info[ROPE_LAUNCH_INFO_LEN])
{
    if (info == nullptr) return rope::set_error(ROPE_ERR_NULLPTR, "info is NULL");
    for (int i = 0; i < ROPE_LAUNCH_INFO_LEN; ++i) info[i] = 0;
    rope::Plan p;
    std::string why;
    rope_status_t st = rope::make_plan_pos(const_cast<void*>(x), x_shape, dtype, positions, positions_shape,
                                           positions_strides, inv_freq, table_dtype, mode, partial_slice, rope::kFwd,
                                           &p, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    if (p.noop) return ROPE_OK;
    rope::PosArgs a{};
    uint32_t threads = 0, grid = 0;
    rope::RowShape rs;
    if (rope::pos_geometry(p, &a, &threads, &grid)) {
        info[0] = ROPE_KERNEL_VECTOR;
        info[1] = grid;
        info[2] = threads;
        info[3] = a.U;
        info[4] = a.HL;
        info[5] = a.P;
        info[6] = a.chunks;
        info[7] = a.span;
    } else if (rope::rows_shape(p, &rs)) {
        info[0] = ROPE_KERNEL_ROWS;
        info[1] = rs.grid;
        info[2] = rs.threads;
        info[4] = rs.rpb;
        info[7] = rs.tpr;
    } else {
        info[0] = ROPE_KERNEL_SCALAR;
        info[2] = 256;
    }
    return ROPE_OK;
}

rope_status_t rope_proj_fwd(void* y, rope_dtype_t y_dtype, const void* x, const void* w, rope_dtype_t dtype,
                            const int64_t y_shape[4], int64_t K,
                            const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                            const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                            rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2], void* stream)
{
    return rope::run_proj(y, y_dtype, x, w, dtype, y_shape, K, r1, r1_shape, r1_strides, r2, r2_shape, r2_strides,
                          table_dtype, mode, partial_slice, stream);
}

rope_status_t rope_proj_launch_info(rope_dtype_t y_dtype, rope_dtype_t dtype, const int64_t y_shape[4], int64_t K,
                                    const void* r1, const int64_t r1_shape[4], const int64_t r1_strides[4],
                                    const void* r2, const int64_t r2_shape[4], const int64_t r2_strides[4],
                                    rope_dtype_t table_dtype, int64_t mode, const int64_t partial_slice[2],
                                    int64_t info[ROPE_LAUNCH_INFO_LEN])
{
    if (info == nullptr) return rope::set_error(ROPE_ERR_NULLPTR, "info is NULL");
    for (int i = 0; i < ROPE_LAUNCH_INFO_LEN; ++i) info[i] = 0;
    // distinct, 16-byte aligned stand-ins for y, x and w, never dereferenced:
    // the plan only compares them with NULL and checks alignment and overlap
    static const uint64_t kNowhere = uint64_t(1) << 62;
    void* y = reinterpret_cast<void*>(kNowhere);
    const void* x = reinterpret_cast<const void*>(kNowhere * 2);
    const void* w = reinterpret_cast<const void*>(kNowhere * 3);
    rope::ProjLaunch P;
    std::string why;
    rope_status_t st = rope::prepare_proj(y, y_dtype, x, w, dtype, y_shape, K, r1, r1_shape, r1_strides, r2, r2_shape,
                                          r2_strides, table_dtype, mode, partial_slice, &P, &why);
    if (st != ROPE_OK) return rope::set_error(st, why);
    if (P.q.noop) return ROPE_OK;
    info[0] = P.sq ? ROPE_KERNEL_PROJ_SQUARE : ROPE_KERNEL_PROJ_HEADS;
    info[1] = P.grid;
    info[2] = P.threads;
    info[3] = P.BM;
    info[4] = P.BN;
    info[5] = P.sq && P.a.epi >= 0 ? 1 + P.a.epi : 0;
    info[6] = P.sq && P.a.epi >= 0 && P.q.rope.L > 0 && P.a.tab_crl >= 0 ? 1 : 0;
    return ROPE_OK;
}

const char* rope_status_string(rope_status_t status)
{
    switch (status) {
    case ROPE_OK: return "ROPE_OK: success";
    case ROPE_ERR_NULLPTR: return "ROPE_ERR_NULLPTR: a required pointer is NULL";
    case ROPE_ERR_INVALID: return "ROPE_ERR_INVALID: an argument violates the operation's constraints";
    case ROPE_ERR_UNSUPPORTED: return "ROPE_ERR_UNSUPPORTED: valid arguments this library does not support";
    case ROPE_ERR_RUNTIME: return "ROPE_ERR_RUNTIME: the HIP runtime reported an error";
    default: return "unknown rope_status_t";
    }
}

const char* rope_last_error(void)
{
    return rope::g_last_error.c_str();
}

}  // extern "C"
