// hbm_probe.hip -- the bare access pattern of an in-place slice update, for
// measuring what HBM allows it: each launch reads a range of 16-byte vectors
// of every row of a buffer and writes a sub-range of them back unchanged. No
// tables and no arithmetic. Built as its own library (libhbm_probe.so); the
// rotation library does not use it. The benchmark times it beside the
// rotation kernels on the same shapes, so that each kernel's time can be set
// against the time of its bare access pattern on the same GPU.
//
// Launch shape as in the rotation library's vector kernel: 64-thread
// blocks, one vector per thread, the threads of a row covering the load
// range, and the blocks renumbered so that each of the 8 XCDs takes runs of
// consecutive blocks (xcd_run_blocks = 1 keeps dispatch order). Two further
// knobs: the cache-policy bits of the loads (sc0, sc1, nt; CDNA3/CDNA4
// global_load modifiers), and a row stride that gives a block the same row
// of several consecutive groups of `row_stride` rows (for example the same
// head of several consecutive positions) instead of consecutive rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace {

struct ProbeArgs {
    v4u* x;
    uint64_t rows;
    uint64_t blocks;
    uint64_t xcd_full;      // blocks [0, xcd_full) are renumbered (a multiple of 8P)
    uint32_t row_vecs;      // vectors per row
    uint32_t load_lo;       // first vector each row loads
    uint32_t span;          // vectors each row loads (threads per row)
    uint32_t store_lo;      // vectors [store_lo, store_hi) of the row are written back
    uint32_t store_hi;
    uint32_t rows_per_block;
    uint32_t xcd_group;     // P: runs of P consecutive blocks stay on one XCD
    uint32_t key;           // 0: the value written is the value read
    uint32_t row_stride;    // 1: a block takes consecutive rows
};

// One 16-byte load with the cache-policy bits POL (bit 0: sc0, bit 1: sc1,
// bit 2: nt), waited for before it returns.
template <int POL>
__device__ __forceinline__ v4u load_pol(const v4u* p)
{
    v4u v;
    if constexpr (POL == 0) asm volatile("global_load_dwordx4 %0, %1, off\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 1) asm volatile("global_load_dwordx4 %0, %1, off sc0\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 2) asm volatile("global_load_dwordx4 %0, %1, off sc1\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 3) asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 4) asm volatile("global_load_dwordx4 %0, %1, off nt\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 5) asm volatile("global_load_dwordx4 %0, %1, off sc0 nt\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 6) asm volatile("global_load_dwordx4 %0, %1, off sc1 nt\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    if constexpr (POL == 7) asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1 nt\n s_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    return v;
}

// POL < 0: the compiler's loads (nontemporal when NT); POL >= 0: load_pol.
template <bool NT, int POL>
__global__ void __launch_bounds__(64) hbm_probe_rmw_kernel(ProbeArgs a)
{
    const uint32_t t = threadIdx.x;
    const uint32_t r = t / a.span;
    const uint32_t v = a.load_lo + t % a.span;
    if (r >= a.rows_per_block) return;
    uint64_t bid = blockIdx.x;
    if (bid < a.xcd_full) {
        const uint64_t win = 8ull * a.xcd_group;
        const uint64_t w = bid / win, l = bid - w * win;
        bid = w * win + (l & 7u) * a.xcd_group + (l >> 3);
    }
    uint64_t row = bid * a.rows_per_block + r;
    if (a.row_stride > 1) {
        // block bid: row `inner` of the groups [outer*rpb, outer*rpb + rpb)
        const uint64_t inner = bid % a.row_stride, outer = bid / a.row_stride;
        row = (outer * a.rows_per_block + r) * a.row_stride + inner;
    }
    if (row >= a.rows) return;
    v4u* p = a.x + row * a.row_vecs + v;
    v4u val;
    if constexpr (POL >= 0) val = load_pol<POL>(p);
    else val = NT ? __builtin_nontemporal_load(p) : *p;
    // xor with a run-time zero, so the compiler cannot drop the store of a
    // value just loaded from the same address
    val ^= a.key;
    if (v >= a.store_lo && v < a.store_hi) {
        if (NT) __builtin_nontemporal_store(val, p);
        else *p = val;
    }
}

}  // namespace

// Read vectors [load_lo, load_hi) of each of `rows` rows of `row_vecs`
// 16-byte vectors at x (device memory, 16-byte aligned) and write
// [store_lo, store_hi) back unchanged, on `stream` (hipStream_t; NULL =
// default). nt != 0: nontemporal stores, and nontemporal loads when
// load_policy < 0. load_policy 0-7: the loads carry sc0 (bit 0), sc1 (bit 1)
// and nt (bit 2). xcd_run_blocks: P of the XCD renumbering. row_stride > 1:
// a block takes one row of each of rows_per_block consecutive groups of
// row_stride rows (rows must be a multiple of row_stride * rows_per_block).
// Returns 0, 1 for invalid arguments, 2 for a launch error.
extern "C" __attribute__((visibility("default"))) int hbm_probe_rmw(
    void* x, int64_t rows, int64_t row_vecs, int64_t load_lo, int64_t load_hi, int64_t store_lo,
    int64_t store_hi, int nt, int load_policy, int64_t xcd_run_blocks, int64_t row_stride, void* stream)
{
    if (!x || (reinterpret_cast<uintptr_t>(x) & 15u) || rows <= 0 || row_vecs <= 0) return 1;
    if (!(0 <= load_lo && load_lo <= store_lo && store_lo < store_hi && store_hi <= load_hi &&
          load_hi <= row_vecs))
        return 1;
    const int64_t span = load_hi - load_lo;
    if (span > 64 || xcd_run_blocks < 1 || xcd_run_blocks > (1 << 24)) return 1;
    if (load_policy < -1 || load_policy > 7 || row_stride < 1 || row_stride > (1 << 24)) return 1;
    if (rows > (INT64_MAX / 16) / row_vecs) return 1;
    ProbeArgs a;
    a.x = static_cast<v4u*>(x);
    a.rows = (uint64_t)rows;
    a.row_vecs = (uint32_t)row_vecs;
    a.load_lo = (uint32_t)load_lo;
    a.span = (uint32_t)span;
    a.store_lo = (uint32_t)store_lo;
    a.store_hi = (uint32_t)store_hi;
    a.rows_per_block = (uint32_t)(64 / span);
    a.blocks = (a.rows + a.rows_per_block - 1) / a.rows_per_block;
    if (a.blocks > 0xFFFFFFFFull / 64) return 1;   // grid size in work-items is 32-bit
    a.xcd_group = (uint32_t)xcd_run_blocks;
    a.xcd_full = a.blocks / (8ull * a.xcd_group) * (8ull * a.xcd_group);
    a.key = 0;
    a.row_stride = (uint32_t)row_stride;
    if (row_stride > 1 && rows % (row_stride * a.rows_per_block)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((uint32_t)a.blocks), block(64);
    switch (nt ? load_policy + 1 : load_policy + 10) {
    case 0: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, -1>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 0>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 1>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 3>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 4>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 5>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 6>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((hbm_probe_rmw_kernel<true, 7>), grid, block, 0, s, a); break;
    case 9: hipLaunchKernelGGL((hbm_probe_rmw_kernel<false, -1>), grid, block, 0, s, a); break;
    default: return 1;   // the load policies are probed with nontemporal stores only
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
