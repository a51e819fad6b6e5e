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
// Tiling (gfx950: 256 CUs, 160 KiB LDS and 512 VGPRs per SIMD lane): a block
// computes a BM x BN tile of y (BN = 192 or 128 output lanes: a whole number
// of heads, or part of one head that spans whole tiles; BM = 384 or 256
// tokens) with BM/64 x 2 waves, each holding a
// 64 x BN/2 sub-tile as 2 x BN/64 accumulators of 32 x 32 fp32 (96 or 64
// registers), so that 3 (or 2) waves share each SIMD and one wave's LDS
// reads overlap another's MFMAs. The K loop runs over stages of 64 k: each
// row of x and w contributes one whole 128-byte line per stage (a stage of
// 32 k would fetch every line twice). Two stages of (BM + BN) x 128 bytes
// form the LDS ring, filled by the gfx950 direct global-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes go to the wave's LDS base +
// 16 * lane, no registers in between) one stage ahead of the MFMAs. They take
// the SGPR-base form (a uniform base per stage and operand plus a 32-bit byte
// offset per lane): the CU accepts these about a third faster than loads with
// a 64-bit address per lane, and a wave whose load cannot issue yet holds back
// the MFMAs behind it, so a stage's load issue is on the MFMAs' path. Within a
// 128-byte row the eight 16-byte k-vectors are stored XOR-swizzled by a
// function of the row modulo 32, chosen so that the 8, 16 or 32 lanes that
// one LDS cycle serves read distinct banks (the fragment reads take 16 bytes
// of 32 consecutive rows at one k). The loads are issued from inline
// assembly and waited for with explicit vmcnt counts: the compiler, which
// does not see them, would otherwise wait for every outstanding load before
// each LDS read.
//
// Epilogue, in two halves of BM/2 rows (the ring is free by then): every
// wave writes its accumulators for the half to LDS as fp32, then 8
// consecutive threads take the 8-lane vectors of one row (one 128-byte line
// of 16-bit output per 8 threads): lanes outside the slice are stored as
// they are; a slice lane j is rotated with its partner p(j) and the cos/sin
// of its token and head,
//   y_j = p_j c_j + sigma(j) p_p(j) s_j    (fp32, as the table call's fp32 rule),
// then rounded once to the output type. Each thread's cos and sin values
// for the half are loaded from the tables into registers before the half's
// accumulators are written to LDS, so their latency overlaps that write.
#pragma once

#include <type_traits>

#include "rope_device.hpp"

namespace rope {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProjBK = 64;       // k per LDS stage: one 128-byte line of each row
constexpr int kProjStages = 2;    // LDS ring depth

// The block tile for BN output lanes: BM tokens, (BM/64) x 2 waves of
// 64 x BN/2 each.
template <int BN>
struct ProjTile {
    static_assert(BN == 128 || BN == 192, "block tile width");
    static constexpr int BM = BN == 192 ? 384 : 256;
    static constexpr int WM = BM / 64;            // wave rows
    static constexpr int NW = 2 * WM;             // waves
    static constexpr int THREADS = 64 * NW;
    static constexpr int MT = 2;                  // 32-row accumulator tiles per wave
    static constexpr int NT = BN / 64;            // 32-column accumulator tiles per wave
    static constexpr int STAGE = (BM + BN) * kProjBK * 2;
    static constexpr int NLOAD = (BM + BN) / 8;   // 1 KiB wave loads (8 rows x 128 bytes) per stage
    static constexpr int LW = NLOAD / NW;         // per wave
    static_assert(NLOAD % NW == 0, "every wave issues the same number of loads");
    static_assert(BM % 8 == 0, "no wave load straddles x and w");
    static constexpr int LDC = BN + 4;            // epilogue row pitch in floats
    static constexpr int RH = BM / 2;             // rows per epilogue half
    static constexpr int EPI = RH * LDC * 4;
    static constexpr int LDS = kProjStages * STAGE > EPI ? kProjStages * STAGE : EPI;
    static_assert(LDS <= 160 * 1024, "LDS per block");
    static constexpr int RPP = THREADS / 8;       // rows per epilogue pass: 8 threads per row
    static constexpr int PR = RH / RPP;           // passes per half
    static_assert(RH % RPP == 0, "whole passes");
    static constexpr int VI = BN / 64;            // vectors per thread and row: 8 threads x 8 lanes per step
};

// The k-vector slot of row r: bits 0-2 of the result are r0^r3, r1^r4 and
// r2. For rows r..r+31 read at one k (one fragment), the lanes that one LDS
// cycle serves (8 rows of 128 bytes over 32 banks, 16 over 64 banks or 32
// over 128 banks) then meet distinct 16-byte bank groups; the value depends
// only on r mod 32, so every 32-row fragment uses the same slots.
__device__ __forceinline__ int proj_swz(int r) { return ((r ^ (r >> 3)) & 3) | (r & 4); }

// One direct global-to-LDS load of 16 bytes per lane from base + voff (base
// the same for the whole wave, voff lane l's byte offset): lane l's bytes go
// to LDS byte address lds_base + 16*l (lds_base the same for the whole wave).
__device__ __forceinline__ void proj_dma16(const void* base, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(base) : "memory");
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
    const void* r1;        // cos, table type; element (b,s,h,j) at b*t1b + s*t1s + h*t1n + j
    const void* r2;        // sin
    int64_t t1b, t1s, t1n, t2b, t2s, t2n;
    int32_t M, N, K;       // x and w hold fewer than 2^31 elements
    int32_t S;             // tokens m = b*S + s
    int32_t Dh;            // lanes per head (BN is a multiple of Dh)
    int32_t start, L;      // the slice of each head, [start, start + L)
    int32_t half;          // pair distance: 1 (interleave), L/2 (rotate_half) or L/c
    // every slice vector is whole (start and L multiples of 8), its partner
    // is in the vector (interleave) or a whole vector away (half a multiple
    // of 8), and its 8 cos and 8 sin values are 16-byte aligned in the tables
    int32_t fast;
    // square tiles' epilogue: -1 the general one (any geometry); 0 the
    // vector epilogue, partners in the vector (interleave, or no slice); 1
    // the vector epilogue, partners `half` lanes (whole vectors) away
    int32_t epi;
    // vector epilogue: >= 0 when the table rows of the tile's tokens go to
    // LDS during the last K stage, 2^tab_crl 16-byte chunks per row (the
    // slice's L lanes; the same row for every head); -1 reads them from the
    // tables
    int32_t tab_crl;
    int32_t MB, NB;        // block tiles along M and N
    int32_t group_m;       // raster: groups of group_m M-tiles walk all N-tiles
    int32_t xcd_chunk;     // blocks [0, 8*xcd_chunk) are dealt to the XCDs in contiguous chunks
    FastDiv s_div;         // division by S (tokens m < 2^31)
    FastDiv dh_div;        // division by Dh
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

// 8 table values as fp32 from an aligned 16-byte (16-bit table) or 32-byte
// (fp32 table) run.
template <int TT>
struct ProjTab8 {
    static constexpr int kVecs = TT == ROPE_DTYPE_F32 ? 2 : 1;
    v4u q[kVecs];
    __device__ void load(const void* tab, int64_t i)
    {
        const v4u* p = reinterpret_cast<const v4u*>(static_cast<const char*>(tab) + i * (TT == ROPE_DTYPE_F32 ? 4 : 2));
#pragma unroll
        for (int k = 0; k < kVecs; ++k) q[k] = p[k];
    }
    __device__ void widen(float (&f)[8]) const
    {
        if constexpr (TT == ROPE_DTYPE_F32) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f[k] = __uint_as_float(q[0][k]);
                f[4 + k] = __uint_as_float(q[1][k]);
            }
        } else {
            Lanes<TT> T;
            T.unpack(q[0]);
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] = T.v[k];
        }
    }
};

template <int DT, int BN, int TT>
__global__ void __launch_bounds__(ProjTile<BN>::THREADS)
    __attribute__((amdgpu_waves_per_eu(ProjTile<BN>::NW / 4, ProjTile<BN>::NW / 4))) rope_proj_kernel(ProjArgs a)
{
    using T_ = ProjTile<BN>;
    constexpr int BM = T_::BM, MT = T_::MT, NT = T_::NT, LW = T_::LW, LDC = T_::LDC;
    __shared__ __attribute__((aligned(16))) uint16_t smem[T_::LDS / 2];

    int32_t mb, nb;
    proj_tile(a, mb, nb);
    const int32_t m0 = mb * BM;
    const int32_t n0 = nb * BN;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave % T_::WM, wn = wave / T_::WM;

    // ---------------------------------------------------------------- main loop
    // A stage: rows 0..BM-1 of x then rows 0..BN-1 of w, 128 bytes each. Wave
    // load li (of NLOAD) fills stage rows 8*li .. 8*li+7; wave `wave` issues
    // loads [LW*wave, LW*wave + LW). Lane l of a load writes row 8*li + l/8
    // at 16-byte slot l%8, which holds k-vector (l%8) ^ proj_swz(row). Rows
    // past M or N re-read the last row (always in bounds); their results are
    // never stored. The SGPR-base loads take the per-lane byte offset as an
    // unsigned 32-bit number; x and w hold fewer than 2^31 elements, so every
    // offset is below 2^32.
    uint32_t goff[LW];
    bool from_x[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int li = wave * LW + i;
        const int srow = li * 8 + (lane >> 3);
        from_x[i] = li * 8 < BM;
        const int row = from_x[i] ? srow : srow - BM;
        const int kv = (lane & 7) ^ proj_swz(row & 31);
        const int32_t g = from_x[i] ? min(m0 + row, a.M - 1) : min(n0 + row, a.N - 1);
        goff[i] = ((uint32_t)g * (uint32_t)a.K + (uint32_t)(kv * 8)) * 2u;
    }
    const uint32_t smem_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(smem_lds + wave * LW * 1024);
    auto issue_stage = [&](int32_t k, int slot) {
        const uint16_t* xk = a.x + k * kProjBK;
        const uint16_t* wk = a.w + k * kProjBK;
        const uint32_t sbase = wave_lds + (uint32_t)(slot * T_::STAGE);
#pragma unroll
        for (int i = 0; i < LW; ++i) proj_dma16(from_x[i] ? xk : wk, goff[i], sbase + i * 1024);
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

    // fragment reads: A row r = wm*64 + mt*32 + lane%32 (B row similarly),
    // k-vector kv = 2*kk + lane/32 at slot kv ^ proj_swz(lane%32)
    const int fr = lane & 31;
    const int sw = proj_swz(fr);
    const int a_row = (wm * 64 + fr) * kProjBK;        // in 16-bit elements
    const int b_row = BM * kProjBK + (wn * (BN / 2) + fr) * kProjBK;
    auto mma_stage = [&](int slot) {
        const uint16_t* S0 = smem + slot * (T_::STAGE / 2);
        // interleave the LDS reads with the MFMAs of the stage
        __builtin_amdgcn_iglp_opt(1);
#pragma unroll
        for (int kk = 0; kk < kProjBK / 16; ++kk) {
            const int slot16 = ((2 * kk + (lane >> 5)) ^ sw) * 8;
            v4u fa[MT], fb[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                fa[i] = *reinterpret_cast<const v4u*>(S0 + a_row + i * 32 * kProjBK + slot16);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                fb[j] = *reinterpret_cast<const v4u*>(S0 + b_row + j * 32 * kProjBK + slot16);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = proj_mfma<DT>(fa[i], fb[j], acc[i][j]);
        }
    };

    // Stage k lives in slot k % 2 and is loaded while stage k-1 is computed.
    const int32_t KT = a.K / kProjBK;
    issue_stage(0, 0);
    for (int32_t kt = 0; kt < KT; ++kt) {
        proj_wait_vm<0>();                             // this wave's loads of stage kt are in LDS
        // everyone's are, and everyone has consumed stage kt-1, whose slot is
        // refilled next. A bare barrier (no fence); the empty asm keeps the
        // compiler from moving this stage's LDS reads above it.
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + 1 < KT) issue_stage(kt + 1, (int)((kt + 1) & 1));
        mma_stage((int)(kt & 1));
    }
    __syncthreads();                                   // every wave is done with the ring

    // ---------------------------------------------------------------- epilogue
    // Half h holds accumulator row tile mt = h of every wave: tile rows
    // wm*64 + h*32 + [0, 32), local row lr = wm*32 + [0, 32). Thread t takes
    // row lr = t/8 + p*RPP of the half (p < PR) and the 8-lane vectors
    // v = t%8 + 8*i (i < VI) of that row: consecutive threads take
    // consecutive vectors, so each 8 threads store one 128-byte line.
    float* Cs = reinterpret_cast<float*>(smem);        // [RH][LDC]
    const int tv = t & 7, tr = t >> 3;
    const int g2 = 2 * a.half;
    // per vector i: lanes [c0, c0+8) of the tile, in head hl (of y, from the
    // vector's column n0 + c0: a tile holds whole heads, or part of one head
    // wider than the tile), slice-relative first lane rel0
    int c0[T_::VI], hl[T_::VI], rel0[T_::VI];
    bool live_v[T_::VI], rot[T_::VI];
#pragma unroll
    for (int i = 0; i < T_::VI; ++i) {
        c0[i] = 8 * (tv + 8 * i);
        hl[i] = (int)fast_div((uint32_t)(n0 + c0[i]), a.dh_div);
        rel0[i] = n0 + c0[i] - hl[i] * a.Dh - a.start;
        live_v[i] = n0 + c0[i] < a.N;
        // rotated: meets the slice, in a head that exists (the last tile
        // along N may reach past N; its table rows must not be read)
        rot[i] = live_v[i] && a.L > 0 && rel0[i] < a.L && rel0[i] + 8 > 0;
    }
    auto write_acc = [&](const f32x16 (&accq)[NT]) {
        // accumulator (h, nt), register r holds row 8*(r/4) + 4*(lane/32) + r%4
        // and column lane%32 of its 32 x 32 tile
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int col = wn * (BN / 2) + j * 32 + (lane & 31);
                Cs[lr * LDC + col] = accq[j][r];
            }
    };
    // Table values prefetched for the first vector of each pass (lanes
    // [0, 64) of the tile: a 64-lane slice at the start of each head, as the
    // MLA rope dimension, is all prefetched); other vectors read theirs when
    // they come (more would not fit the registers of 3 waves per SIMD).
    constexpr int VP = 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int64_t m[T_::PR], o1[T_::PR], o2[T_::PR];
        ProjTab8<TT> pc[T_::PR][VP], ps[T_::PR][VP];
#pragma unroll
        for (int p = 0; p < T_::PR; ++p) {
            const int lr = tr + p * T_::RPP;
            m[p] = m0 + (lr >> 5) * 64 + h * 32 + (lr & 31);
            const int32_t mc = (int32_t)min<int64_t>(m[p], a.M - 1);
            const int32_t b = (int32_t)fast_div((uint32_t)mc, a.s_div), sp = mc - b * a.S;
            o1[p] = b * a.t1b + sp * a.t1s;
            o2[p] = b * a.t2b + sp * a.t2s;
            if (a.fast) {
#pragma unroll
                for (int i = 0; i < VP; ++i)
                    if (rot[i]) {
                        pc[p][i].load(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel0[i]);
                        ps[p][i].load(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel0[i]);
                    }
            }
        }
        if (h == 0) write_acc(acc[0]);
        else write_acc(acc[1]);
        __syncthreads();
#pragma unroll
        for (int p = 0; p < T_::PR; ++p) {
            if (m[p] >= a.M) continue;
            const float* crow = Cs + (tr + p * T_::RPP) * LDC;
#pragma unroll
            for (int i = 0; i < T_::VI; ++i) {
                if (!live_v[i]) continue;
                const int64_t yo = m[p] * a.N + n0 + c0[i];
                if (rot[i] && !a.fast) {
                    // any other geometry: lane by lane from the row in LDS
                    // (partners there too), cos and sin read one by one, one
                    // store per lane
#pragma unroll 1
                    for (int e = 0; e < 8; ++e) {
                        const int rel = rel0[i] + e;
                        float ye = crow[c0[i] + e];
                        if (rel >= 0 && rel < a.L) {
                            const bool f = rel % g2 < a.half;
                            const float xpe = crow[c0[i] + e + (f ? a.half : -a.half)];
                            const float ce = Store<TT>::load1(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel);
                            const float se = Store<TT>::load1(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel);
                            ye = rotate_own<false>(ye, xpe, ce, se, f);
                        }
                        if (a.ydt == ROPE_DTYPE_F32) Store<ROPE_DTYPE_F32>::store1(a.y, yo + e, ye);
                        else Store<DT>::store1(a.y, yo + e, ye);
                    }
                    continue;
                }
                float val[8];
                {
                    const float4 q0 = *reinterpret_cast<const float4*>(crow + c0[i]);
                    const float4 q1 = *reinterpret_cast<const float4*>(crow + c0[i] + 4);
                    val[0] = q0.x; val[1] = q0.y; val[2] = q0.z; val[3] = q0.w;
                    val[4] = q1.x; val[5] = q1.y; val[6] = q1.z; val[7] = q1.w;
                }
                if (rot[i]) {
                    // whole vector in the slice: partners in the vector
                    // (interleave) or the vector `half` lanes away
                    float cc[8], ss[8];
                    if (i < VP) {
                        pc[p][i < VP ? i : 0].widen(cc);
                        ps[p][i < VP ? i : 0].widen(ss);
                    } else {
                        ProjTab8<TT> c1, s1;
                        c1.load(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel0[i]);
                        s1.load(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel0[i]);
                        c1.widen(cc);
                        s1.widen(ss);
                    }
                    float xp[8];
                    bool first[8];
                    if (a.half == 1) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            xp[e] = val[e ^ 1];
                            first[e] = (e & 1) == 0;
                        }
                    } else {
                        const bool f = rel0[i] % g2 < a.half;
                        const float* pp = crow + c0[i] + (f ? a.half : -a.half);
                        const float4 p0 = *reinterpret_cast<const float4*>(pp);
                        const float4 p1 = *reinterpret_cast<const float4*>(pp + 4);
                        xp[0] = p0.x; xp[1] = p0.y; xp[2] = p0.z; xp[3] = p0.w;
                        xp[4] = p1.x; xp[5] = p1.y; xp[6] = p1.z; xp[7] = p1.w;
#pragma unroll
                        for (int e = 0; e < 8; ++e) first[e] = f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) val[e] = rotate_own<false>(val[e], xp[e], cc[e], ss[e], first[e]);
                }
                // nontemporal: y is not read again here, and the L2 is left to
                // the x and w tiles other blocks reuse (1.5-2% faster on the
                // MLA Q projection)
                if (a.ydt == ROPE_DTYPE_F32) {
                    v4u* yp = reinterpret_cast<v4u*>(static_cast<float*>(a.y) + yo);
                    __builtin_nontemporal_store(v4u{__float_as_uint(val[0]), __float_as_uint(val[1]),
                                                    __float_as_uint(val[2]), __float_as_uint(val[3])}, yp);
                    __builtin_nontemporal_store(v4u{__float_as_uint(val[4]), __float_as_uint(val[5]),
                                                    __float_as_uint(val[6]), __float_as_uint(val[7])}, yp + 1);
                } else {
                    Lanes<DT> Y;   // the output is the inputs' 16-bit type
#pragma unroll
                    for (int e = 0; e < 8; ++e) Y.v[e] = val[e];
                    __builtin_nontemporal_store(Y.pack(), reinterpret_cast<v4u*>(static_cast<uint16_t*>(a.y) + yo));
                }
            }
        }
        __syncthreads();                               // the half's rows are read before the next is written
    }
}

}  // namespace
}  // namespace rope

namespace rope {
namespace {

// ---------------------------------------------------------------------------
// Square tiles: 256 tokens x 256 output lanes per block, 4 waves (one per
// SIMD) of 128 x 128, each holding 4 x 4 accumulators of 32 x 32 fp32 (256
// registers, the accumulation registers of the wave). With one wave per SIMD
// nothing hides a stall, so the K loop is software-pipelined by hand: every
// MFMA of a 16-k step is paired with at most one LDS fragment read for the
// next step and one direct global-to-LDS load for the next stage, in a fixed
// order that the scheduler may not change. A stage's 16 loads per wave are
// spread over its first 32 MFMAs (one every 64 MFMA cycles per wave, about
// the rate at which the CU accepts them from its four waves), so no wave
// waits at the head of a stage for its loads to be accepted; they then have
// the rest of the stage to land. The accumulators are transposed (MFMA A =
// w fragment, B = x fragment): lane l holds token l%32 and 4 consecutive
// output lanes per register group, so each goes to the epilogue staging as
// one 16-byte LDS write.
// The tile is not aligned to heads: the epilogue finds each vector's head
// from its column, and the host takes this kernel only when no rotation
// group of the slice straddles two 256-lane tiles.
// ---------------------------------------------------------------------------
struct ProjSq {
    static constexpr int BM = 256, BN = 256;
    static constexpr int THREADS = 256;
    static constexpr int STAGE = (BM + BN) * kProjBK * 2;   // 64 KiB
    static constexpr int LW = (BM + BN) / 8 / 4;             // 16 wave loads per stage
    static constexpr int LDC = BN + 4;                        // staging pitch: rows 16 bytes apart mod 128
    static constexpr int RH = BM / 2;                         // rows per epilogue half
    static constexpr int EPI = RH * LDC * 4;
    static constexpr int LDS = 2 * STAGE > EPI ? 2 * STAGE : EPI;
    static_assert(LDS <= 160 * 1024, "LDS per block");
    static constexpr int RPP = THREADS / 8;                   // rows per epilogue pass
    static constexpr int PR = RH / RPP;                       // passes per half
    static constexpr int VI = BN / 64;                        // vectors per thread and row
    // the vector epilogue: table rows in stage slot 0, then each wave's 32 x
    // 128 fp32 staging rows of LDW floats (rows 16 bytes apart modulo 128)
    static constexpr int LDW = 132;
    static_assert(STAGE + 4 * 32 * LDW * 4 <= LDS, "vector epilogue staging");
    static_assert(2 * 256 * 128 <= STAGE, "table rows of up to 128 bytes in slot 0");
};

// The square tiles' vector epilogue, for slices of whole 8-lane vectors whose
// partners are in the vector (interleave, PV = false) or a whole number of
// vectors away (PV = true, any half that is a multiple of 8; the host keeps
// every group inside one wave's 128 lanes). Each wave works on its own
// 128 tokens x 128 output lanes, in four quarters of 32 tokens (token tile
// q), with no barrier: a wave's LDS operations complete in order, so its
// reads of a quarter see its writes and precede its next quarter's writes.
//  1. The wave writes its accumulators for the quarter to its own LDS
//     region as fp32, straight from the accumulation registers (16-byte
//     writes; lane l of acc[nt][q] holds 4 consecutive output lanes of token
//     l%32). Staging row l%32 of 132 floats (rows 16 bytes apart modulo 128,
//     so the 8 rows one write cycle serves meet distinct banks).
//  2. Lane l takes column vector 8*(l%8) + 64G of rows l/8 + 8k (k < 4), one
//     64-lane half G at a time (8 lanes of a row store one 128-byte line of
//     16-bit output). A vector in the slice is rotated with its partner (in
//     the vector, or `half` lanes away in the same staging row) and its 8
//     cos and 8 sin values, then rounded once. Whether a vector is rotated
//     depends only on its column, so for a slice of whole 64-lane groups
//     (MLA's rope lanes) it is the same for every lane of an instruction.
// The tables come from LDS when the host staged them there during the last
// K stage (tab_crl >= 0: [table][token][L lanes], 16-byte chunks of a row
// XOR-swizzled by the token's low bits), else from global memory.
template <int DT, int TT, bool PV>
__device__ __forceinline__ void proj_sq_epilogue_vec(const ProjArgs& a, const f32x16 (&acc)[4][4], uint16_t* smem,
                                                     int32_t m0, int32_t n0, int wm, int wn, int wave, int lane)
{
    constexpr int LDW = ProjSq::LDW;                    // staging row pitch in floats
    constexpr int TS = TT == ROPE_DTYPE_F32 ? 4 : 2;   // table element bytes
    const int fr = lane & 31, hw = lane >> 5;
    const uint8_t* tabs = reinterpret_cast<const uint8_t*>(smem);
    float* Cs = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + ProjSq::STAGE) + wave * 32 * LDW;
    const bool tab_lds = a.tab_crl >= 0;
    const int crl = tab_lds ? a.tab_crl : 0, crm = (1 << crl) - 1;
    // the lane's column vector in each 64-lane half G of the wave's 128
    // lanes, and its place in the slice
    const int vl = lane & 7, lr0 = lane >> 3;
    int32_t colg[2], rel0g[2];
    int64_t hn1g[2], hn2g[2];
    bool liveg[2], rotg[2], firstg[2];
#pragma unroll
    for (int G = 0; G < 2; ++G) {
        colg[G] = n0 + wn * 128 + 64 * G + 8 * vl;
        const int32_t hd = (int32_t)fast_div((uint32_t)colg[G], a.dh_div);
        rel0g[G] = colg[G] - hd * a.Dh - a.start;
        hn1g[G] = (int64_t)hd * a.t1n;
        hn2g[G] = (int64_t)hd * a.t2n;
        liveg[G] = colg[G] < a.N;
        rotg[G] = liveg[G] && a.L > 0 && rel0g[G] >= 0 && rel0g[G] < a.L;
        firstg[G] = !PV || rel0g[G] % (2 * a.half) < a.half;   // first half of its group: partner term negated
    }
    // 8 table values of token row tr (tile row) and absolute token m at
    // slice lane rel0 (head offsets hn1, hn2)
    auto tab8 = [&](int table, int tr, int32_t m, int32_t rel0, int64_t hn1, int64_t hn2, float (&f)[8]) {
        if (tab_lds) {
            const int byte = rel0 * TS;
            const uint8_t* row = tabs + (table << (12 + crl)) + (tr << (4 + crl));
            if constexpr (TT == ROPE_DTYPE_F32) {
                const v4u q0 = *reinterpret_cast<const v4u*>(row + (((byte >> 4) ^ (tr & crm)) << 4));
                const v4u q1 = *reinterpret_cast<const v4u*>(row + ((((byte >> 4) + 1) ^ (tr & crm)) << 4));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    f[k] = __uint_as_float(q0[k]);
                    f[4 + k] = __uint_as_float(q1[k]);
                }
            } else {
                const v4u q0 = *reinterpret_cast<const v4u*>(row + (((byte >> 4) ^ (tr & crm)) << 4));
                Lanes<TT> T;
                T.unpack(q0);
#pragma unroll
                for (int k = 0; k < 8; ++k) f[k] = T.v[k];
            }
        } else {
            const int32_t mc = min(m, a.M - 1);
            const int32_t b = (int32_t)fast_div((uint32_t)mc, a.s_div), sp = mc - b * a.S;
            ProjTab8<TT> q;
            q.load(table ? a.r2 : a.r1,
                   table ? b * a.t2b + sp * a.t2s + hn2 + rel0 : b * a.t1b + sp * a.t1s + hn1 + rel0);
            q.widen(f);
        }
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // 1. the quarter's accumulators to LDS, straight from the
        //    accumulation registers (q is a constant here: a loop over q
        //    kept as a loop reads every accumulator into VGPRs each time)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& c = acc[nt][q];
                *reinterpret_cast<float4*>(Cs + fr * LDW + nt * 32 + 8 * g + 4 * hw) =
                    float4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
            }
        // 2. the quarter's 32 rows of the wave's 128 lanes, one 64-lane half
        //    G at a time: all four rows' LDS reads (values, partners, cos and
        //    sin) go out before any arithmetic, inside one branch on
        //    "rotated" (the same for every lane when the slice is whole
        //    64-lane groups)
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            const int c8 = 64 * G + 8 * vl;                              // first float of the vector
            float val[4][8];
            auto read8 = [&](const float* p, float (&v)[8]) {
                const float4 q0 = *reinterpret_cast<const float4*>(p);
                const float4 q1 = *reinterpret_cast<const float4*>(p + 4);
                v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
                v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
            };
#pragma unroll
            for (int k = 0; k < 4; ++k) read8(Cs + (lr0 + 8 * k) * LDW + c8, val[k]);
            if (rotg[G]) {
                float cc[4][8], ss[4][8], xp[4][8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int tr = wm * 128 + q * 32 + lr0 + 8 * k;     // tile row
                    tab8(0, tr, m0 + tr, rel0g[G], hn1g[G], hn2g[G], cc[k]);
                    tab8(1, tr, m0 + tr, rel0g[G], hn1g[G], hn2g[G], ss[k]);
                    if constexpr (PV)
                        read8(Cs + (lr0 + 8 * k) * LDW + c8 + (firstg[G] ? a.half : -a.half), xp[k]);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (PV) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            val[k][e] = rotate_own<false>(val[k][e], xp[k][e], cc[k][e], ss[k][e], firstg[G]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) xp[k][e] = val[k][e ^ 1];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            val[k][e] = rotate_own<false>(val[k][e], xp[k][e], cc[k][e], ss[k][e], (e & 1) == 0);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int32_t m = m0 + wm * 128 + q * 32 + lr0 + 8 * k;
                if (m < a.M && liveg[G]) {
                    const int64_t yo = (int64_t)m * a.N + colg[G];
                    if (a.ydt == ROPE_DTYPE_F32) {
                        v4u* yp = reinterpret_cast<v4u*>(static_cast<float*>(a.y) + yo);
                        __builtin_nontemporal_store(v4u{__float_as_uint(val[k][0]), __float_as_uint(val[k][1]),
                                                        __float_as_uint(val[k][2]), __float_as_uint(val[k][3])}, yp);
                        __builtin_nontemporal_store(v4u{__float_as_uint(val[k][4]), __float_as_uint(val[k][5]),
                                                        __float_as_uint(val[k][6]), __float_as_uint(val[k][7])},
                                                    yp + 1);
                    } else {
                        Lanes<DT> Y;
#pragma unroll
                        for (int e = 0; e < 8; ++e) Y.v[e] = val[k][e];
                        __builtin_nontemporal_store(Y.pack(),
                                                    reinterpret_cast<v4u*>(static_cast<uint16_t*>(a.y) + yo));
                    }
                }
            }
        }
    }
}

// EPI: the epilogue (ProjArgs::epi): -1 the general one (any geometry), 0
// the vector epilogue with partners in the vector, 1 with partners whole
// vectors away (a kernel of its own each: one kernel holding several
// epilogues spills the accumulators)
template <int DT, int TT, int EPI>
__global__ void __launch_bounds__(ProjSq::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
    rope_proj_sq_kernel(ProjArgs a)
{
    using T_ = ProjSq;
    constexpr int BM = T_::BM, BN = T_::BN, LW = T_::LW, LDC = T_::LDC;
    __shared__ __attribute__((aligned(16))) uint16_t smem[T_::LDS / 2];

    int32_t mb, nb;
    proj_tile(a, mb, nb);
    const int32_t m0 = mb * BM;
    const int32_t n0 = nb * BN;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // ---------------------------------------------------------------- loads
    // A stage: rows 0..255 of x then rows 0..255 of w, 128 bytes each; waves
    // 0 and 1 load x rows [128*wave, +128), waves 2 and 3 w rows [128*(wave-2),
    // +128). Load i of a wave fills its rows 8i..8i+7; lane l writes row
    // 8i + l/8 at 16-byte slot l%8, which holds k-vector (l%8) ^ proj_swz(row).
    // Rows past M or N re-read the last row (in bounds); their results are
    // never stored. Offsets are unsigned 32-bit bytes (operands below 2^31
    // elements).
    const bool wx = wave < 2;
    const uint16_t* src = wx ? a.x : a.w;
    uint32_t goff[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int row = (wave & 1) * 128 + 8 * i + (lane >> 3);
        const int kv = (lane & 7) ^ proj_swz(row & 31);
        const int32_t g = wx ? min(m0 + row, a.M - 1) : min(n0 + row, a.N - 1);
        goff[i] = ((uint32_t)g * (uint32_t)a.K + (uint32_t)(kv * 8)) * 2u;
    }
    const uint32_t smem_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(smem_lds + wave * LW * 1024);
    auto load1 = [&](int32_t kt, int slot, int i) {
        proj_dma16(src + kt * kProjBK, goff[i], wave_lds + (uint32_t)(slot * T_::STAGE) + i * 1024);
    };

    // ---------------------------------------------------------------- fragments
    // x row r = wm*128 + mt*32 + lane%32, w row BM + wn*128 + nt*32 + lane%32;
    // k-vector kv = 2*kk + lane/32 at slot kv ^ proj_swz(lane%32)
    const int fr = lane & 31;
    const int sw = proj_swz(fr);
    const int a_row = (wm * 128 + fr) * kProjBK;
    const int b_row = (BM + wn * 128 + fr) * kProjBK;
    v4u fa[2][4], fb[2][4];
    // fragment read q of step kk (q < 8, in the order the MFMAs use them:
    // w fragment 0, x fragments 0..3, w fragments 1..3)
    auto read1 = [&](int slot, int kk, int buf, int q) {
        const uint16_t* S0 = smem + slot * (T_::STAGE / 2);
        const int s16 = ((2 * kk + (lane >> 5)) ^ sw) * 8;
        if (q == 0) fb[buf][0] = *reinterpret_cast<const v4u*>(S0 + b_row + s16);
        else if (q <= 4) fa[buf][q - 1] = *reinterpret_cast<const v4u*>(S0 + a_row + (q - 1) * 32 * kProjBK + s16);
        else fb[buf][q - 4] = *reinterpret_cast<const v4u*>(S0 + b_row + (q - 4) * 32 * kProjBK + s16);
    };

    // [nt][mt]: rows are output lanes, columns tokens; the first step of the
    // first stage starts them from an inline zero (no per-tile clearing)
    f32x16 acc[4][4];

    // One stage: 4 steps of 16 k, 16 MFMAs each (nt-major). Step kk reads the
    // fragments of step kk+1 (buffer (kk+1)&1); steps 0 and 1 issue the next
    // stage's loads, one per even MFMA; step 3 waits for those loads and for
    // its own fragment reads, meets the other waves at the barrier halfway
    // through, and reads the next stage's first fragments after it.
    // The vector epilogue's table rows (slice lanes [0, L) of the cos and
    // sin rows of the tile's 256 tokens, 2^tab_crl chunks each) go to ring
    // slot 0 during the last stage, whose slot 0 is free: wave load i of
    // wave w fills chunk positions p = (2^(crl+1)*w + i)*64 + lane of
    // [table][token][chunk slot]; slot cs of token tr holds chunk
    // cs ^ (tr % 2^crl). Rows past M re-read the last token's row.
    // Waves 0 and 1 load the cos rows, 2 and 3 the sin rows (2^(crl+2)
    // loads per table). The byte offsets are computed while the first
    // stage loads: between the last stage's MFMAs they would hold back the
    // MFMA issue (and wait for reloaded kernel arguments, a wait that also
    // waits out the fragment reads). Load i of a wave covers tokens
    // tr0 + i * (64 >> crl) at one chunk slot, so the offsets step by whole
    // rows, carrying into the next batch when s passes S (at most once per
    // step when S >= 64 >> crl; shorter sequences take one division per
    // load). 32-bit arithmetic: the host bounds every row's byte offset
    // below 2^32, so sums modulo 2^32 are exact.
    const int ntab = EPI >= 0 && a.L > 0 && a.tab_crl >= 0 ? 2 << a.tab_crl : 0;   // loads per wave
    const int tcrl = a.tab_crl < 0 ? 0 : a.tab_crl;
    const void* tab_base = wave >> 1 ? a.r2 : a.r1;
    const uint32_t tab_lds = __builtin_amdgcn_readfirstlane(smem_lds + (uint32_t)(wave * (2 << tcrl) * 1024));
    uint32_t toff[LW];
    auto tab_offsets = [&]() {
        const uint32_t tb = (uint32_t)(wave >> 1 ? a.t2b : a.t1b), ts = (uint32_t)(wave >> 1 ? a.t2s : a.t1s);
        constexpr uint32_t TS = TT == ROPE_DTYPE_F32 ? 4 : 2;
        const int tstep = 64 >> tcrl;
        const int pos = ((wave * (2 << tcrl)) * 64 + lane) & ((256 << tcrl) - 1);
        const int tr0 = pos >> tcrl;
        const uint32_t cb = (uint32_t)(((pos & ((1 << tcrl) - 1)) ^ (tr0 & ((1 << tcrl) - 1))) * 16);
        auto row = [&](int32_t m) {                    // element offset of token m's row
            const uint32_t b = fast_div((uint32_t)m, a.s_div);
            return b * tb + ((uint32_t)m - b * (uint32_t)a.S) * ts;
        };
        const uint32_t last = row(a.M - 1);            // rows past M re-read the last token's row
        int32_t m = m0 + tr0;
        if (a.S >= tstep) {
            const int32_t mc = min(m, a.M - 1);
            const uint32_t b = fast_div((uint32_t)mc, a.s_div);
            uint32_t sp = (uint32_t)mc - b * (uint32_t)a.S;
            uint32_t off = b * tb + sp * ts;
            const uint32_t rstep = (uint32_t)tstep * ts, carry = tb - (uint32_t)a.S * ts;
#pragma unroll
            for (int i = 0; i < LW; ++i) {
                toff[i] = (m < a.M ? off : last) * TS + cb;
                m += tstep;
                sp += tstep;
                off += rstep;
                if (sp >= (uint32_t)a.S) {
                    sp -= (uint32_t)a.S;
                    off += carry;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < LW; ++i) toff[i] = row(min(m + i * tstep, a.M - 1)) * TS + cb;
        }
#pragma unroll
        for (int i = 0; i < LW; ++i) asm volatile("" : "+v"(toff[i]));   // kept here, not sunk to the uses
    };
    auto tab_dma = [&](int i) { proj_dma16(tab_base, toff[i], tab_lds + (uint32_t)(i * 1024)); };
    auto stage = [&](auto slot_c, auto more_c, auto first_c, int32_t kt) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr bool more = decltype(more_c)::value;
        constexpr bool first = decltype(first_c)::value;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (kk == 3 && j == 8 && more) {
                    proj_wait_vm<0>();
                    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), vmcnt and expcnt free
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
                const int nt = j >> 2, mt = j & 3;
                acc[nt][mt] = proj_mfma<DT>(fb[cur][nt], fa[cur][mt], first && kk == 0 ? f32x16{} : acc[nt][mt]);
                if (more && kk < 2 && (j & 1) == 0) load1(kt + 1, slot ^ 1, kk * 8 + (j >> 1));
                if constexpr (!more && EPI >= 0)
                    if (kk < 2 && (j & 1) == 0 && kk * 8 + (j >> 1) < ntab) tab_dma(kk * 8 + (j >> 1));
                if (kk < 3 && (j & 1)) read1(slot, kk + 1, nxt, j >> 1);
                if (kk == 3 && j >= 8 && more) read1(slot ^ 1, 0, nxt, j - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // K is a whole number of stage pairs (the host checks): the last pair
    // ends the loop without a branch on the stage count
    const int32_t KT = a.K / kProjBK;
#pragma unroll
    for (int i = 0; i < LW; ++i) load1(0, 0, i);
    if constexpr (EPI >= 0)
        if (ntab) tab_offsets();
    proj_wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < 8; ++q) read1(0, 0, 0, q);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using More = std::true_type;
    using Last = std::false_type;
    using First = std::true_type;
    using Later = std::false_type;
    // stage kt in slot kt % 2: the first stage peeled (zero accumulators),
    // then pairs, then the last stage (KT even)
    stage(S0{}, More{}, First{}, 0);
    int32_t kt = 1;
    for (; kt + 2 < KT; kt += 2) {
        stage(S1{}, More{}, Later{}, kt);
        stage(S0{}, More{}, Later{}, kt + 1);
    }
    stage(S1{}, Last{}, Later{}, kt);
    proj_wait_vm<0>();                                 // this wave's table rows are in LDS
    __syncthreads();                                   // every wave is done with the ring

    if constexpr (EPI >= 0) {
        proj_sq_epilogue_vec<DT, TT, EPI == 1>(a, acc, smem, m0, n0, wm, wn, wave, lane);
        return;
    }

    // ---------------------------------------------------------------- epilogue
    // Half h stages accumulator columns mt = 2h, 2h+1 of every wave: tile
    // rows wm*128 + h*64 + [0, 64) at staging row lr = wm*64 + [0, 64).
    float* Cs = reinterpret_cast<float*>(smem);        // [RH][LDC]
    const int tv = t & 7, tr = t >> 3;
    const int g2 = 2 * a.half;
    int c0[T_::VI], hl[T_::VI], rel0[T_::VI];
    bool live_v[T_::VI], rot[T_::VI];
#pragma unroll
    for (int i = 0; i < T_::VI; ++i) {
        c0[i] = 8 * (tv + 8 * i);
        hl[i] = (int)fast_div((uint32_t)(n0 + c0[i]), a.dh_div);
        rel0[i] = n0 + c0[i] - hl[i] * a.Dh - a.start;
        live_v[i] = n0 + c0[i] < a.N;
        rot[i] = live_v[i] && a.L > 0 && rel0[i] < a.L && rel0[i] + 8 > 0;
    }
    // table values prefetched, before the half's accumulators go to LDS, for
    // every vector of a thread's rows (16-bit tables) or the first two (fp32
    // tables, which would not fit the registers); the rest read on demand
    constexpr int VP = TT == ROPE_DTYPE_F32 ? 2 : T_::VI;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int64_t m[T_::PR], o1[T_::PR], o2[T_::PR];
        ProjTab8<TT> pc[T_::PR][VP], ps[T_::PR][VP];
#pragma unroll
        for (int p = 0; p < T_::PR; ++p) {
            const int lr = tr + p * T_::RPP;
            m[p] = m0 + (lr >> 6) * 128 + h * 64 + (lr & 63);
            const int32_t mc = (int32_t)min<int64_t>(m[p], a.M - 1);
            const int32_t b = (int32_t)fast_div((uint32_t)mc, a.s_div), sp = mc - b * a.S;
            o1[p] = b * a.t1b + sp * a.t1s;
            o2[p] = b * a.t2b + sp * a.t2s;
            if (a.fast) {
#pragma unroll
                for (int i = 0; i < VP; ++i)
                    if (rot[i]) {
                        pc[p][i].load(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel0[i]);
                        ps[p][i].load(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel0[i]);
                    }
            }
        }
        // accumulator (nt, mt), register 4g + e of lane l: output lane
        // nt*32 + 8g + 4*(l/32) + e, token mt*32 + l%32
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int ml = 0; ml < 2; ++ml)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16& c = acc[nt][2 * h + ml];
                    const int lr = wm * 64 + ml * 32 + fr;
                    const int col = wn * 128 + nt * 32 + 8 * g + 4 * (lane >> 5);
                    *reinterpret_cast<float4*>(Cs + lr * LDC + col) =
                        float4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]};
                }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < T_::PR; ++p) {
            if (m[p] >= a.M) continue;
            const float* crow = Cs + (tr + p * T_::RPP) * LDC;
#pragma unroll
            for (int i = 0; i < T_::VI; ++i) {
                if (!live_v[i]) continue;
                const int64_t yo = m[p] * a.N + n0 + c0[i];
                if (rot[i] && !a.fast) {
#pragma unroll 1
                    for (int e = 0; e < 8; ++e) {
                        const int rel = rel0[i] + e;
                        float ye = crow[c0[i] + e];
                        if (rel >= 0 && rel < a.L) {
                            const bool f = rel % g2 < a.half;
                            const float xpe = crow[c0[i] + e + (f ? a.half : -a.half)];
                            const float ce = Store<TT>::load1(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel);
                            const float se = Store<TT>::load1(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel);
                            ye = rotate_own<false>(ye, xpe, ce, se, f);
                        }
                        if (a.ydt == ROPE_DTYPE_F32) Store<ROPE_DTYPE_F32>::store1(a.y, yo + e, ye);
                        else Store<DT>::store1(a.y, yo + e, ye);
                    }
                    continue;
                }
                float val[8];
                {
                    const float4 q0 = *reinterpret_cast<const float4*>(crow + c0[i]);
                    const float4 q1 = *reinterpret_cast<const float4*>(crow + c0[i] + 4);
                    val[0] = q0.x; val[1] = q0.y; val[2] = q0.z; val[3] = q0.w;
                    val[4] = q1.x; val[5] = q1.y; val[6] = q1.z; val[7] = q1.w;
                }
                if (rot[i]) {
                    float cc[8], ss[8];
                    if (i < VP) {
                        pc[p][i < VP ? i : 0].widen(cc);
                        ps[p][i < VP ? i : 0].widen(ss);
                    } else {
                        ProjTab8<TT> c1, s1;
                        c1.load(a.r1, o1[p] + (int64_t)hl[i] * a.t1n + rel0[i]);
                        s1.load(a.r2, o2[p] + (int64_t)hl[i] * a.t2n + rel0[i]);
                        c1.widen(cc);
                        s1.widen(ss);
                    }
                    float xp[8];
                    bool first[8];
                    if (a.half == 1) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            xp[e] = val[e ^ 1];
                            first[e] = (e & 1) == 0;
                        }
                    } else {
                        const bool f = rel0[i] % g2 < a.half;
                        const float* pp = crow + c0[i] + (f ? a.half : -a.half);
                        const float4 p0 = *reinterpret_cast<const float4*>(pp);
                        const float4 p1 = *reinterpret_cast<const float4*>(pp + 4);
                        xp[0] = p0.x; xp[1] = p0.y; xp[2] = p0.z; xp[3] = p0.w;
                        xp[4] = p1.x; xp[5] = p1.y; xp[6] = p1.z; xp[7] = p1.w;
#pragma unroll
                        for (int e = 0; e < 8; ++e) first[e] = f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) val[e] = rotate_own<false>(val[e], xp[e], cc[e], ss[e], first[e]);
                }
                if (a.ydt == ROPE_DTYPE_F32) {
                    v4u* yp = reinterpret_cast<v4u*>(static_cast<float*>(a.y) + yo);
                    __builtin_nontemporal_store(v4u{__float_as_uint(val[0]), __float_as_uint(val[1]),
                                                    __float_as_uint(val[2]), __float_as_uint(val[3])}, yp);
                    __builtin_nontemporal_store(v4u{__float_as_uint(val[4]), __float_as_uint(val[5]),
                                                    __float_as_uint(val[6]), __float_as_uint(val[7])}, yp + 1);
                } else {
                    Lanes<DT> Y;
#pragma unroll
                    for (int e = 0; e < 8; ++e) Y.v[e] = val[e];
                    __builtin_nontemporal_store(Y.pack(), reinterpret_cast<v4u*>(static_cast<uint16_t*>(a.y) + yo));
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace rope
