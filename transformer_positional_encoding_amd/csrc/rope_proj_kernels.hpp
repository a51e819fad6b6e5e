// rope_proj_kernels.hpp -- a head projection whose epilogue rotates each
// head's slice before the single store: y = rotate(x . w^T).
// Included once, by rope_kernels.hip (the one translation unit of the
// library): its kernels are instantiated there, next to the host code
// that selects and launches them.
//
// Operation: "ascend-transformer-boost 的 MlaPreprocessOperation：MLA 预处理
// 四阶段融合算子深度解析", section 3 (the WUQ matmul gives Q with headNum x 192
// lanes per token, then Q[..., :qRopeDim] is rotated with cos/sin of shape
// [tokenNum, 64] given from outside) and section 2 (qRopeDim, the rotary
// coefficient). The page fuses the stages so that the projection result
// never makes a round trip through memory before the rotation; here the
// rotation runs on the fp32 accumulator in the GEMM's epilogue.
//
// Layout: x (M, K) row-major, M = B*S tokens; w (N, K) row-major, N = H*Dh
// (output lanes by inputs, as a linear layer stores its weight); y (M, N)
// row-major = (B, S, H, Dh). Both operands are K-contiguous, which is what
// the MFMA fragments take: a lane of v_mfma_f32_32x32x16 holds 8 consecutive
// k of one row of A (x) and 8 consecutive k of one column of B (a row of w).
//
// Tiling (gfx950, 256 CUs, 160 KiB LDS per CU): a block of 4 waves computes a
// 256 x BN tile of y (BN = 128 or 192, a whole number of heads); wave (wm,
// wn) holds a 128 x BN/2 sub-tile as 4 x BN/64 accumulators of 32 x 32 fp32.
// The K loop runs over stages of 32 k: 256 x 32 of x and BN x 32 of w, 64
// bytes per row, in a ring of 4 LDS stages filled by the gfx950 direct
// global-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes go to
// the wave's LDS base + 16 * lane, no registers in between). A stage is
// loaded three stages ahead of its MFMAs. Within each 64-byte row the four
// 16-byte k-vectors are stored XOR-swizzled by bits 1-2 of the row, so the
// MFMA fragment reads (16 bytes of 8 consecutive rows at one k) fall in
// distinct LDS banks. The loads are issued from inline assembly and waited
// for with explicit vmcnt counts: the compiler, which does not see them,
// would otherwise wait for every outstanding load before each LDS read.
//
// Epilogue: the accumulators go to LDS in two halves of 128 rows (the ring
// is free by then), and each thread then takes 8 consecutive output lanes
// of a row (consecutive threads, consecutive lanes: the stores coalesce):
// lanes outside the slice are stored as they are; a slice lane j is rotated
// with its partner p(j) and the cos/sin of its token and head,
//   y_j = p_j c_j + sigma(j) p_p(j) s_j    (fp32, as the table call's fp32 rule),
// then rounded once to the output type. The next vector's table values are
// loaded (16 bytes at a time where aligned) while the current one is
// computed.
#pragma once

#include <type_traits>

#include "rope_device.hpp"

namespace rope {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProjBM = 256;      // tokens per block tile
constexpr int kProjBK = 32;       // k per LDS stage (64-byte rows)
constexpr int kProjStages = 4;    // LDS ring depth
constexpr int kProjThreads = 256;

__host__ __device__ constexpr int proj_stage_bytes(int BN) { return (kProjBM + BN) * kProjBK * 2; }
// epilogue: 64 rows of fp32 results, then cos and sin for those rows as fp32
// (at most 64 rows x BN lanes each: one table row per token and head)
__host__ __device__ constexpr int proj_epi_bytes(int BN) { return 64 * (BN + 4) * 4 + 2 * 64 * BN * 4; }
__host__ __device__ constexpr int proj_lds_bytes(int BN)
{
    return kProjStages * proj_stage_bytes(BN) > proj_epi_bytes(BN) ? kProjStages * proj_stage_bytes(BN)
                                                                    : proj_epi_bytes(BN);
}

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes go to
// LDS byte address lds_base + 16*l (lds_base is the same for the whole wave).
__device__ __forceinline__ void proj_dma16(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g) : "memory");
}

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt left free (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void proj_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct ProjArgs {
    const uint16_t* x;     // (M, K) 16-bit
    const uint16_t* w;     // (N, K) 16-bit
    void* y;               // (M, N), output type ydt
    int32_t ydt;           // rope_dtype_t of y: the inputs' type or fp32
    int32_t tdt;           // rope_dtype_t of r1 and r2
    const void* r1;        // cos, table type; element (b,s,h,j) at b*t1b + s*t1s + h*t1n + j
    const void* r2;        // sin
    int64_t t1b, t1s, t1n, t2b, t2s, t2n;
    int64_t M, N, K;
    int64_t S;             // tokens m = b*S + s
    int32_t Dh;            // lanes per head (BN is a multiple of Dh)
    int32_t start, L;      // the slice of each head, [start, start + L)
    int32_t half;          // pair distance: 1 (interleave), L/2 (rotate_half) or L/c
    int32_t MB, NB;        // block tiles along M and N
    int32_t group_m;       // raster: groups of group_m M-tiles walk all N-tiles
    int32_t xcd_chunk;     // blocks [0, 8*xcd_chunk) are dealt to the XCDs in contiguous chunks
    FastDiv s_div;         // division by S (tokens m < 2^31)
    FastDiv dh_div;        // division by Dh
    FastDiv l_div;         // division by L (L > 0)
    int32_t t1h, t2h;      // heads of the tile whose cos (sin) rows differ: BN/Dh, or 1 when broadcast over heads
    FastDiv lc_div;        // division by the 16-byte chunks of a table row (16-byte staging)
    // The 8-lane vectors of a head (Dh/8 of them) that meet the slice are
    // [rv_lo, rv_lo + nrv); the epilogue stores the others in a first pass
    // and rotates these in a second one.
    int32_t rv_lo, nrv;
    FastDiv rot_row_div;   // division by (BN/Dh) * nrv: rotated vectors per row of the tile
    FastDiv rot_head_div;  // division by nrv
    FastDiv cp_row_div;    // division by (BN/Dh) * (Dh/8 - nrv): other vectors per row
    FastDiv cp_head_div;   // division by Dh/8 - nrv
};

template <int DT>
__device__ __forceinline__ f32x16 proj_mfma(const v4u& a, const v4u& b, const f32x16& c)
{
    if constexpr (DT == ROPE_DTYPE_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
}

// The block's tile (mb, nb). Workgroup i runs on XCD i % 8; blocks are first
// dealt so that each XCD takes a contiguous run of tile numbers (tiles that
// share operands then share one L2), and tile numbers walk groups of
// group_m M-tiles across all N-tiles, M fastest, so that the blocks in
// flight on an XCD share a few x tiles and a few w tiles.
__device__ __forceinline__ void proj_tile(const ProjArgs& a, int32_t& mb, int32_t& nb)
{
    int32_t bid = (int32_t)blockIdx.x;
    if (bid < 8 * a.xcd_chunk) bid = (bid & 7) * a.xcd_chunk + (bid >> 3);
    const int32_t in_group = a.group_m * a.NB;
    const int32_t g = bid / in_group;
    const int32_t first = g * a.group_m;
    const int32_t gsize = min(a.MB - first, a.group_m);
    const int32_t r = bid - g * in_group;
    mb = first + r % gsize;
    nb = r / gsize;
}

// TV: the tables are staged in 16-byte chunks (every row aligned, L whole
// chunks); otherwise element by element.
template <int DT, int BN, bool TV>
__global__ void __launch_bounds__(kProjThreads) rope_proj_kernel(ProjArgs a)
{
    static_assert(BN == 128 || BN == 192, "block tile width");
    constexpr int NT = BN / 64;                        // 32-wide accumulator tiles per wave along N
    constexpr int MT = 4;                              // 32-high accumulator tiles per wave along M
    constexpr int LDC = BN + 4;                        // epilogue row pitch in floats
    static_assert(proj_epi_bytes(BN) <= proj_lds_bytes(BN), "epilogue staging fits the LDS");
    static_assert(proj_lds_bytes(BN) <= 160 * 1024, "LDS per block");
    __shared__ __attribute__((aligned(16))) uint16_t smem[proj_lds_bytes(BN) / 2];

    int32_t mb, nb;
    proj_tile(a, mb, nb);
    const int64_t m0 = (int64_t)mb * kProjBM;
    const int64_t n0 = (int64_t)nb * BN;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // A stage: rows 0..255 of x then rows 0..BN-1 of w, 64 bytes each; one
    // wave load instruction fills 16 consecutive rows (1 KiB). Wave `wave`
    // fills x rows [64*wave, +64) (4 loads) and w rows [BN/4*wave, +BN/4).
    // Lane l of a load writes row 16*i + l/4 at 16-byte slot l%4, which
    // holds k-vector (l%4) ^ ((row/2) % 4) of the stage. Rows past M or N
    // re-read the last row (always in bounds); their results are never
    // stored. Element offsets are 32-bit (x and w hold fewer than 2^31
    // elements).
    constexpr int A_LOADS = kProjBM / 16 / 4;          // 4 per wave
    constexpr int B_LOADS = BN / 16 / 4;               // 2 or 3 per wave
    constexpr int LOADS = A_LOADS + B_LOADS;           // per wave per stage
    uint32_t goff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const bool isA = i < A_LOADS;
        const int row = isA ? (wave * A_LOADS + i) * 16 + (lane >> 2)
                            : (wave * B_LOADS + (i - A_LOADS)) * 16 + (lane >> 2);
        const int kv = (lane & 3) ^ ((row >> 1) & 3);
        const int64_t g = isA ? min(m0 + row, a.M - 1) : min(n0 + row, a.N - 1);
        goff[i] = (uint32_t)(g * a.K + kv * 8);
    }
    const uint32_t smem_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // LDS byte address of load i of this wave in stage slot 0
    const uint32_t wave_a = __builtin_amdgcn_readfirstlane(smem_lds + wave * A_LOADS * 1024);
    const uint32_t wave_b = __builtin_amdgcn_readfirstlane(smem_lds + kProjBM * 64 + wave * B_LOADS * 1024);
    auto issue_stage = [&](int64_t k, int slot) {
        const uint32_t koff = (uint32_t)(k * kProjBK);
        const uint32_t sbase = (uint32_t)(slot * proj_stage_bytes(BN));
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) proj_dma16(a.x + (goff[i] + koff), wave_a + sbase + i * 1024);
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i)
            proj_dma16(a.w + (goff[A_LOADS + i] + koff), wave_b + sbase + i * 1024);
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

    // fragment reads: A row r = wm*128 + mt*32 + lane%32 (B row similarly),
    // k-vector kv = 2*kk + lane/32 at slot kv ^ ((r/2) % 4); lane%32 runs
    // over 32 consecutive rows, so (r/2) % 4 = ((lane%32)/2) % 4
    const int fr = lane & 31;
    const int sw = (fr >> 1) & 3;
    const int a_row = (wm * 128 + fr) * 32;            // in 16-bit elements
    const int b_row = kProjBM * 32 + (wn * (BN / 2) + fr) * 32;
    auto mma_stage = [&](int slot) {
        const uint16_t* S0 = smem + slot * (proj_stage_bytes(BN) / 2);
#pragma unroll
        for (int kk = 0; kk < kProjBK / 16; ++kk) {
            const int slot16 = ((2 * kk + (lane >> 5)) ^ sw) * 8;
            v4u fa[MT], fb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                fa[i] = *reinterpret_cast<const v4u*>(S0 + a_row + i * 32 * 32 + slot16);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                fb[j] = *reinterpret_cast<const v4u*>(S0 + b_row + j * 32 * 32 + slot16);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = proj_mfma<DT>(fa[i], fb[j], acc[i][j]);
        }
    };

    // Stage k lives in slot k % 4. Three stages are in flight ahead of the
    // one being computed; past the last stage the last one is loaded again
    // (into a free slot) so that every step waits for the same count.
    const int64_t KT = a.K / kProjBK;
#pragma unroll
    for (int k = 0; k < kProjStages - 1; ++k) issue_stage(min<int64_t>(k, KT - 1), k);
    for (int64_t kt = 0; kt < KT; ++kt) {
        proj_wait_vm<LOADS * (kProjStages - 2)>();     // this wave's loads of stage kt are in LDS
        // everyone's are, and everyone has consumed stage kt-1 (whose slot
        // is refilled next). A bare barrier: a fenced one would wait for
        // every outstanding load, the three stages in flight included.
        __builtin_amdgcn_s_barrier();
        issue_stage(min<int64_t>(kt + kProjStages - 1, KT - 1), (int)((kt + kProjStages - 1) % kProjStages));
        mma_stage((int)(kt % kProjStages));
    }
    proj_wait_vm<0>();
    __syncthreads();

    // ---------------------------------------------------------------- epilogue
    // Four quarters of 64 rows: accumulator row tile mt = qq of both wave
    // rows. For each quarter the block first stages, as fp32 in LDS, the cos
    // and sin values of its 64 tokens (and of each head of the tile when the
    // tables differ by head): independent loads spread over all threads, so
    // their latency is paid once per quarter. The accumulators follow into
    // LDS; then step `it` gives 8-lane vector v = 256*it + t of the quarter's
    // rows to thread t (consecutive threads, consecutive lanes of a row: the
    // stores coalesce).
    constexpr int RV = BN / 8;                         // 8-lane vectors per row of the tile
    float* Cs = reinterpret_cast<float*>(smem);        // [64][LDC]
    float* Tc = Cs + 64 * LDC;                         // [64][t1h][L]
    float* Tsn = Tc + 64 * a.t1h * a.L;                // [64][t2h][L]
    const int64_t N = a.N;
    const int64_t h0 = n0 / a.Dh;                      // the tile's first head
    auto token = [&](int qq, int lr) { return m0 + (lr >> 5) * 128 + qq * 32 + (lr & 31); };
    // Stage the table rows of quarter qq: row r = lr * th + head of the tile,
    // lanes [0, L). With 16-byte rows (TV), round `rd` gives thread t the
    // 16-byte chunks rd*R*256 + u*256 + t (u < R) of the quarter's rows;
    // otherwise single elements, R per round. A round's loads of both tables
    // go out together and land in registers; committing writes them to LDS.
    // Round 0 of the next quarter is loaded while this quarter's vectors are
    // computed, so for tables up to R*256 chunks per quarter (64 tokens x 64
    // lanes of 16-bit cos and sin, the MLA case) no load latency is exposed
    // after the first quarter.
    constexpr int es_chunk = 16;
    constexpr int R = 4;
    using TabVal = typename std::conditional<TV, v4u, float>::type;
    struct TabRound {
        TabVal c[R], s[R];
    };
    auto table_index = [&](int qq, int row, int th, int64_t tb, int64_t ts, int64_t tn) {
        const int lr = th == 1 ? row : row / th, hl = row - lr * th;
        const int64_t m = min(token(qq, lr), a.M - 1);
        const int64_t b = fast_div((uint32_t)m, a.s_div), sp = m - b * a.S;
        return b * tb + sp * ts + (h0 + hl) * tn;
    };
    const int tes = a.tdt == ROPE_DTYPE_F32 ? 4 : 2;
    const int per = es_chunk / tes;                       // lanes per 16-byte chunk (TV)
    // units (chunks or elements) per quarter of each table
    const int units1 = TV ? 64 * a.t1h * a.L / per : 64 * a.t1h * a.L;
    const int units2 = TV ? 64 * a.t2h * a.L / per : 64 * a.t2h * a.L;
    auto load_unit = [&](const void* tab, int qq, int th, int64_t tb, int64_t ts, int64_t tn, int units, int u,
                         TabVal& out) {
        u = min(u, units - 1);
        if constexpr (TV) {
            const int row = (int)fast_div((uint32_t)u, a.lc_div);
            const int lane0 = (u - row * (int)a.lc_div.d) * per;
            const int64_t i = table_index(qq, row, th, tb, ts, tn) + lane0;
            out = *reinterpret_cast<const v4u*>(static_cast<const char*>(tab) + i * tes);
        } else {
            const int row = (int)fast_div((uint32_t)u, a.l_div);
            const int64_t i = table_index(qq, row, th, tb, ts, tn) + (u - row * a.L);
            if (a.tdt == ROPE_DTYPE_BF16) out = Store<ROPE_DTYPE_BF16>::load1(tab, i);
            else if (a.tdt == ROPE_DTYPE_F16) out = Store<ROPE_DTYPE_F16>::load1(tab, i);
            else out = Store<ROPE_DTYPE_F32>::load1(tab, i);
        }
    };
    auto store_unit = [&](float* dst, int units, int u, const TabVal& v) {
        if (u >= units) return;
        if constexpr (TV) {
            float* d = dst + u * per;
            if (a.tdt == ROPE_DTYPE_F32) {
                *reinterpret_cast<v4u*>(d) = v;
            } else {
                float f[8];
                if (a.tdt == ROPE_DTYPE_BF16) {
                    Lanes<ROPE_DTYPE_BF16> T;
                    T.unpack(v);
#pragma unroll
                    for (int k = 0; k < 8; ++k) f[k] = T.v[k];
                } else {
                    Lanes<ROPE_DTYPE_F16> T;
                    T.unpack(v);
#pragma unroll
                    for (int k = 0; k < 8; ++k) f[k] = T.v[k];
                }
                reinterpret_cast<float4*>(d)[0] = float4{f[0], f[1], f[2], f[3]};
                reinterpret_cast<float4*>(d)[1] = float4{f[4], f[5], f[6], f[7]};
            }
        } else {
            dst[u] = v;
        }
    };
    auto load_round = [&](int qq, int rd, TabRound& r) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int u = (rd * R + k) * kProjThreads + t;
            load_unit(a.r1, qq, a.t1h, a.t1b, a.t1s, a.t1n, units1, u, r.c[k]);
            load_unit(a.r2, qq, a.t2h, a.t2b, a.t2s, a.t2n, units2, u, r.s[k]);
        }
    };
    auto store_round = [&](int rd, const TabRound& r) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int u = (rd * R + k) * kProjThreads + t;
            store_unit(Tc, units1, u, r.c[k]);
            store_unit(Tsn, units2, u, r.s[k]);
        }
    };
    const int rounds = (max(units1, units2) + R * kProjThreads - 1) / (R * kProjThreads);
    TabRound pre;                                          // round 0 of the next quarter
    if (a.L > 0) load_round(0, 0, pre);
    // The quarters run in a loop that is not unrolled (one copy of the
    // staging and vector code); only the write of the quarter's accumulators,
    // which must index them by constants to keep them in registers, is
    // replicated, behind a switch.
    auto write_acc = [&](const f32x16 (&accq)[NT]) {
        // accumulator (qq, nt), register r holds row 8*(r/4) + 4*(lane/32) + r%4
        // and column lane%32 of its 32 x 32 tile
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int col = wn * (BN / 2) + j * 32 + (lane & 31);
                Cs[row * LDC + col] = accq[j][r];
            }
    };
    static_assert(MT == 4, "four quarters");
#pragma unroll 1
    for (int qq = 0; qq < MT; ++qq) {
        if (a.L > 0) {
            store_round(0, pre);
            for (int rd = 1; rd < rounds; ++rd) {
                TabRound r;
                load_round(qq, rd, r);
                store_round(rd, r);
            }
        }
        switch (qq) {
        case 0: write_acc(acc[0]); break;
        case 1: write_acc(acc[1]); break;
        case 2: write_acc(acc[2]); break;
        default: write_acc(acc[3]); break;
        }
        __syncthreads();
        if (a.L > 0 && qq + 1 < MT) load_round(qq + 1, 0, pre);
        // One vector: row lr of the quarter, 8 lanes from column c0 of the
        // tile; rotated when `rot` (then it meets the slice).
        auto vector = [&](int lr, int c0, bool rot) {
            const int64_t m = token(qq, lr);
            const int64_t n = n0 + c0;
            if (m >= a.M || n >= N) return;
            const float* crow = Cs + lr * LDC;
            float val[8];
            {
                const float4 q0 = *reinterpret_cast<const float4*>(crow + c0);
                const float4 q1 = *reinterpret_cast<const float4*>(crow + c0 + 4);
                val[0] = q0.x; val[1] = q0.y; val[2] = q0.z; val[3] = q0.w;
                val[4] = q1.x; val[5] = q1.y; val[6] = q1.z; val[7] = q1.w;
            }
            if (rot) {
                const int hl = (int)fast_div((uint32_t)c0, a.dh_div);
                const int j0 = c0 - hl * a.Dh;
                const int rel0 = j0 - a.start;
                const float* crow_t = Tc + (lr * a.t1h + (a.t1h > 1 ? hl : 0)) * a.L;
                const float* srow_t = Tsn + (lr * a.t2h + (a.t2h > 1 ? hl : 0)) * a.L;
                const int g2 = 2 * a.half;
                // partners and pair roles: in the vector itself for interleave
                // with an even start (pairs never straddle a vector), a vector
                // `half` lanes away when the 8 lanes lie in one half-group
                // (half and the slice-relative start multiples of 8), else
                // lane by lane
                float xp[8];
                bool first[8];
                if (a.half == 1 && (a.start & 1) == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xp[e] = val[e ^ 1];
                        first[e] = (e & 1) == 0;
                    }
                } else if ((a.half & 7) == 0 && (rel0 & 7) == 0 && rel0 >= 0 && rel0 + 8 <= a.L) {
                    const bool f = rel0 % g2 < a.half;
                    const float* pp = crow + c0 + (f ? a.half : -a.half);
                    const float4 p0 = *reinterpret_cast<const float4*>(pp);
                    const float4 p1 = *reinterpret_cast<const float4*>(pp + 4);
                    xp[0] = p0.x; xp[1] = p0.y; xp[2] = p0.z; xp[3] = p0.w;
                    xp[4] = p1.x; xp[5] = p1.y; xp[6] = p1.z; xp[7] = p1.w;
#pragma unroll
                    for (int e = 0; e < 8; ++e) first[e] = f;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int rel = min(max(rel0 + e, 0), a.L - 1);
                        first[e] = rel % g2 < a.half;
                        xp[e] = crow[c0 + (rel - rel0) + (first[e] ? a.half : -a.half)];
                    }
                }
                // the 8 lanes' cos and sin from LDS, all read before any is
                // used (two 16-byte reads each when the lanes lie in the
                // slice on a 4-lane boundary, else clamped single reads)
                float cc[8], ss[8];
                if (rel0 >= 0 && rel0 + 8 <= a.L && (rel0 & 3) == 0 && (a.L & 3) == 0) {
                    const float4 c0v = *reinterpret_cast<const float4*>(crow_t + rel0);
                    const float4 c1v = *reinterpret_cast<const float4*>(crow_t + rel0 + 4);
                    const float4 s0v = *reinterpret_cast<const float4*>(srow_t + rel0);
                    const float4 s1v = *reinterpret_cast<const float4*>(srow_t + rel0 + 4);
                    cc[0] = c0v.x; cc[1] = c0v.y; cc[2] = c0v.z; cc[3] = c0v.w;
                    cc[4] = c1v.x; cc[5] = c1v.y; cc[6] = c1v.z; cc[7] = c1v.w;
                    ss[0] = s0v.x; ss[1] = s0v.y; ss[2] = s0v.z; ss[3] = s0v.w;
                    ss[4] = s1v.x; ss[5] = s1v.y; ss[6] = s1v.z; ss[7] = s1v.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int rc = min(max(rel0 + e, 0), a.L - 1);
                        cc[e] = crow_t[rc];
                        ss[e] = srow_t[rc];
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rel = rel0 + e;
                    const float yv = rotate_own<false>(val[e], xp[e], cc[e], ss[e], first[e]);
                    val[e] = rel >= 0 && rel < a.L ? yv : val[e];
                }
            }
            if (a.ydt == ROPE_DTYPE_F32) {
                float4* yp = reinterpret_cast<float4*>(static_cast<float*>(a.y) + m * N + n);
                yp[0] = float4{val[0], val[1], val[2], val[3]};
                yp[1] = float4{val[4], val[5], val[6], val[7]};
            } else {
                Lanes<DT> Y;   // the output is the inputs' 16-bit type
#pragma unroll
                for (int e = 0; e < 8; ++e) Y.v[e] = val[e];
                *reinterpret_cast<v4u*>(static_cast<uint16_t*>(a.y) + m * N + n) = Y.pack();
            }
        };
        const int vph = a.Dh / 8;                      // vectors per head
        const int heads_t = BN / a.Dh;                 // heads per tile
        // pass 1: the vectors outside the slice (stored as they are)
        {
            const int ncp = vph - a.nrv;
            const int total = 64 * heads_t * ncp;
#pragma unroll 1
            for (int k = t; k < total; k += kProjThreads) {
                const int lr = (int)fast_div((uint32_t)k, a.cp_row_div);
                const int idx = k - lr * (int)a.cp_row_div.d;
                const int hl = (int)fast_div((uint32_t)idx, a.cp_head_div);
                const int jv = idx - hl * ncp;
                vector(lr, (hl * vph + (jv < a.rv_lo ? jv : jv + a.nrv)) * 8, false);
            }
        }
        // pass 2: the vectors that meet the slice, rotated (every lane busy)
        if (a.nrv > 0) {
            const int total = 64 * heads_t * a.nrv;
#pragma unroll 1
            for (int k = t; k < total; k += kProjThreads) {
                const int lr = (int)fast_div((uint32_t)k, a.rot_row_div);
                const int idx = k - lr * (int)a.rot_row_div.d;
                const int hl = (int)fast_div((uint32_t)idx, a.rot_head_div);
                vector(lr, (hl * vph + a.rv_lo + (idx - hl * a.nrv)) * 8, true);
            }
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace rope
