// Randomised check of the C ABI's argument validation (rope_plan.cpp), built
// with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by the CPU
// test suite. Arguments mix small, boundary and extreme 64-bit values; every
// accepted call must describe a launch whose offsets fit in 64 bits.
#include <stdint.h>
#include <stdio.h>

#include <limits>
#include <string>

#include "rope_plan.hpp"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next()  // splitmix64
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int64_t pick()
{
    static const int64_t edge[] = {0, 1, 2, 3, 7, 8, 63, 64, 1024, 1025, (1ll << 31) - 1, 1ll << 31, 1ll << 32,
                                   (1ll << 62), std::numeric_limits<int64_t>::max(), -1, -2,
                                   std::numeric_limits<int64_t>::min()};
    switch (next() % 4) {
    case 0: return edge[next() % (sizeof(edge) / sizeof(edge[0]))];
    case 1: return (int64_t)(next() % 16);
    case 2: return (int64_t)(next() % 4096);
    default: return (int64_t)next();
    }
}

typedef __int128 i128;

}  // namespace

int main()
{
    const long iters = 3000000;
    long ok = 0, noop = 0, bad = 0;
    void* const fake = reinterpret_cast<void*>(0x10000);
    for (long it = 0; it < iters; ++it) {
        int64_t xs[4], s1[4], st1[4], s2[4], st2[4], sl[2];
        for (int k = 0; k < 4; ++k) xs[k] = (next() % 3) ? (int64_t)(next() % 9) : pick();
        if (next() % 2) xs[3] = 2 * (int64_t)(next() % 520);
        sl[0] = (next() % 3) ? (int64_t)(next() % (xs[3] > 0 ? (uint64_t)xs[3] + 1 : 2)) : pick();
        // the driver's own arithmetic wraps (unsigned) so that extreme values stay defined
        sl[1] = (next() % 3) ? (int64_t)((uint64_t)sl[0] + 2 * (next() % 40)) : pick();
        const int64_t L = (int64_t)((uint64_t)sl[1] - (uint64_t)sl[0]);
        for (int k = 0; k < 4; ++k) {
            s1[k] = (next() % 4) ? ((next() % 2) ? 1 : xs[k]) : pick();
            s2[k] = (next() % 4) ? ((next() % 2) ? 1 : xs[k]) : pick();
            st1[k] = (next() % 4) ? (int64_t)(next() % 100000) : pick();
            st2[k] = (next() % 4) ? (int64_t)(next() % 100000) : pick();
        }
        if (next() % 2) { s1[3] = L; s2[3] = L; st1[3] = 1; st2[3] = 1; }
        if (next() % 2) {
            // a valid call with at most one field disturbed below
            for (int k = 0; k < 4; ++k) xs[k] = 1 + (int64_t)(next() % 9);
            xs[3] = 2 * (1 + (int64_t)(next() % 512));
            sl[0] = (int64_t)(next() % (uint64_t)(xs[3] + 1));
            sl[1] = sl[0] + 2 * (int64_t)(next() % ((uint64_t)(xs[3] - sl[0]) / 2 + 1));
            const int64_t l = sl[1] - sl[0];
            for (int k = 0; k < 3; ++k) {
                s1[k] = (next() % 2) ? 1 : xs[k];
                s2[k] = (next() % 2) ? 1 : xs[k];
            }
            s1[3] = s2[3] = l;
            st1[3] = st2[3] = 1;
            st1[2] = st2[2] = l;
            st1[1] = st1[2] * s1[2]; st2[1] = st2[2] * s2[2];
            st1[0] = st1[1] * s1[1]; st2[0] = st2[1] * s2[1];
            switch (next() % 12) {   // one disturbance, or none
            case 0: xs[next() % 4] = pick(); break;
            case 1: st1[next() % 4] = pick(); break;
            case 2: s2[next() % 4] = pick(); break;
            case 3: sl[next() % 2] = pick(); break;
            case 4: for (int k = 0; k < 3; ++k) st1[k] = (int64_t)(next() >> 2); break;   // huge strides
            default: break;
            }
        }
        const int dtype = (int)(next() % 4) - (next() % 8 == 0);       // mostly valid, sometimes -1 or 3
        const int tdtype = (int)(next() % 4) - (next() % 8 == 0);
        // mostly the named modes, sometimes a small even coefficient, sometimes anything
        const uint64_t mk = next() % 16;
        const int64_t mode = mk < 12 ? (int64_t)(next() % 2) : mk < 15 ? 2 * (int64_t)(1 + next() % 40) : pick();
        const bool null_x = next() % 16 == 0, null_shape = next() % 64 == 0, null_slice = next() % 32 == 0;
        rope::Plan p;
        std::string why;
        const rope_status_t st = rope::make_plan(null_x ? nullptr : fake, null_shape ? nullptr : xs,
                                                 (rope_dtype_t)dtype, fake, s1, st1, fake, s2, st2,
                                                 (rope_dtype_t)tdtype, mode, null_slice ? nullptr : sl,
                                                 rope::kFwd, &p, &why);
        if (st != ROPE_OK && st != ROPE_ERR_NULLPTR && st != ROPE_ERR_INVALID) { ++bad; continue; }
        if (st != ROPE_OK) {
            if (why.empty()) ++bad;
            continue;
        }
        if (p.noop) {
            ++noop;
            // a no-op is exactly an empty tensor or an empty slice
            if (!(p.L == 0 || p.B == 0 || p.S == 0 || p.N == 0 || p.D == 0)) ++bad;
            continue;
        }
        if (p.L == 0 || p.B == 0 || p.S == 0 || p.N == 0 || p.D == 0) ++bad;   // should have been a no-op
        ++ok;
        // an accepted launch: bounds, parity and 64-bit offsets
        bool good = p.start >= 0 && p.L > 0 && p.L % 2 == 0 && p.start + p.L <= p.D && p.D <= 1024 &&
                    p.D % 2 == 0 && p.x == fake && p.B > 0 && p.S > 0 && p.N > 0;
        i128 numel = (i128)p.B * p.S * p.N * p.D;
        good = good && numel * p.esize <= (i128)std::numeric_limits<int64_t>::max();
        const int64_t dims[3] = {p.B, p.S, p.N};
        for (const int64_t* t : {p.t1, p.t2}) {
            i128 span = p.L - 1;
            for (int k = 0; k < 3; ++k) {
                good = good && t[k] >= 0;
                span += (i128)t[k] * (dims[k] - 1);
            }
            good = good && span <= (i128)std::numeric_limits<int64_t>::max();
        }
        // the mode: a named mode, or an even coefficient dividing L, kept as
        // the pair distance of the interleave or rotate_half scheme
        if (mode == ROPE_MODE_INTERLEAVE) good = good && p.mode == ROPE_MODE_INTERLEAVE && p.half == 1;
        else if (mode == ROPE_MODE_ROTATE_HALF) good = good && p.mode == ROPE_MODE_ROTATE_HALF && p.half == p.L / 2;
        else good = good && mode >= 2 && mode % 2 == 0 && p.L % mode == 0 && p.half == p.L / mode &&
                    p.mode == (p.half == 1 ? ROPE_MODE_INTERLEAVE : ROPE_MODE_ROTATE_HALF);
        if (!good) ++bad;
    }
    // The out-of-place form: the same arguments with an input pointer that is
    // the output, overlaps it, lies elsewhere or is NULL. Pointers stay below
    // 2^47, as device addresses do, so that [p, p + bytes) never wraps.
    long out_ok = 0, out_copy = 0, out_overlap = 0;
    for (long it = 0; it < iters / 3; ++it) {
        int64_t xs[4], t[4] = {0, 0, 0, 1}, ts[4], sl[2];
        for (int k = 0; k < 3; ++k) xs[k] = (next() % 4) ? (int64_t)(next() % 9) : pick();
        xs[3] = (next() % 8) ? 2 * (int64_t)(next() % 520) : pick();
        sl[0] = (int64_t)(next() % 64);
        sl[1] = (next() % 4) ? sl[0] : sl[0] + 2 * (int64_t)(next() % 32);
        if (next() % 8 == 0) sl[1] = pick();
        const int64_t L = (int64_t)((uint64_t)sl[1] - (uint64_t)sl[0]);
        for (int k = 0; k < 3; ++k) { t[k] = 1; ts[k] = 0; }
        t[3] = L; ts[3] = 1;
        const int dtype = (int)(next() % 3);
        const uint64_t y = 0x10000 + (next() % (1ull << 40)) * 16;
        uint64_t x;
        switch (next() % 6) {
        case 0: x = y; break;
        case 1: x = 0; break;
        case 2: x = y + (next() % 8192); break;                                  // often inside y
        case 3: x = y > (next() % 8192) ? y - (next() % 8192) : y; break;        // often overlapping from below
        default: x = 0x10000 + (next() % (1ull << 46)); break;
        }
        const bool null_y = next() % 16 == 0;
        void* yp = null_y ? nullptr : reinterpret_cast<void*>(y);
        const void* xp = reinterpret_cast<const void*>(x);
        rope::Plan p;
        std::string why;
        const rope_status_t st = rope::make_plan_out(yp, xp, xs, (rope_dtype_t)dtype, fake, t, ts, fake, t, ts,
                                                     (rope_dtype_t)dtype, 1, sl, rope::kBwd, &p, &why);
        if (st != ROPE_OK && st != ROPE_ERR_NULLPTR && st != ROPE_ERR_INVALID) { ++bad; continue; }
        // the reference: every dimension and the slice valid, element count and bytes in 128 bits
        bool scalars = sl[0] >= 0 && sl[1] >= sl[0] && sl[1] <= xs[3] && L % 2 == 0 && xs[3] % 2 == 0 &&
                       xs[3] <= 1024;
        i128 numel = 1;
        for (int k = 0; k < 4; ++k) {
            scalars = scalars && xs[k] >= 0;
            if (xs[k] >= 0) numel *= xs[k];
            // saturate just past the 64-bit range (the exact size no longer matters)
            if (numel > (i128)std::numeric_limits<int64_t>::max()) numel = (i128)std::numeric_limits<int64_t>::max() + 1;
        }
        const i128 nbytes = numel * (dtype == 0 ? 4 : 2);
        scalars = scalars && nbytes <= (i128)std::numeric_limits<int64_t>::max();
        const bool empty = numel == 0;
        const bool overlap = !empty && !null_y && x != 0 && x != y && (i128)x < (i128)y + nbytes &&
                             (i128)y < (i128)x + nbytes;
        if (st != ROPE_OK) {
            if (why.empty()) ++bad;
            if (why.find("overlap") != std::string::npos) {
                ++out_overlap;
                if (!overlap) ++bad;
            }
            if (scalars && !empty && !null_y && x != 0 && !overlap) ++bad;   // nothing wrong with these arguments
            continue;
        }
        if (!scalars || overlap) { ++bad; continue; }
        if (empty) {
            if (!p.noop) ++bad;
            continue;
        }
        if (null_y || x == 0) { ++bad; continue; }
        if (p.bytes != (int64_t)nbytes || p.x != yp) ++bad;
        if (L == 0) {
            if (x == y ? !(p.noop && !p.copy_only) : !(p.copy_only && !p.noop && p.src == xp)) ++bad;
            out_copy += x != y;
            continue;
        }
        if (p.noop || p.copy_only || p.src != (x == y ? nullptr : xp)) ++bad;
        ++out_ok;
    }
    // The projection with a rotary epilogue: random shapes, K, types and
    // pointers (y, x, w below 2^47, sometimes overlapping). Accepted calls
    // must be within what the kernel tiles: K a positive multiple of 64, a
    // head dimension the kernel takes, x and w under 2^31 elements, 16-byte
    // aligned, disjoint buffers, and tables whose offsets fit in 64 bits.
    long proj_ok = 0;
    for (long it = 0; it < iters / 3; ++it) {
        int64_t ys[4], sl[2], ts[4], tst[4];
        static const int64_t dhs[] = {32, 64, 96, 128, 192, 100, 256, 2};
        for (int k = 0; k < 3; ++k) ys[k] = (next() % 4) ? (int64_t)(next() % 9) : pick();
        ys[3] = (next() % 4) ? dhs[next() % 8] : pick();
        const int64_t K = (next() % 4) ? 64 * (int64_t)(next() % 40) : pick();
        sl[0] = (int64_t)(next() % 64);
        sl[1] = sl[0] + 2 * (int64_t)(next() % 40);
        const int64_t L = sl[1] - sl[0];
        for (int k = 0; k < 4; ++k) {
            ts[k] = (next() % 4) ? ((next() % 2) ? 1 : ys[k]) : pick();
            tst[k] = (next() % 4) ? (int64_t)(next() % 100000) : pick();
        }
        ts[3] = (next() % 8) ? L : pick();
        tst[3] = (next() % 8) ? 1 : pick();
        uintptr_t base[3];
        for (int k = 0; k < 3; ++k) base[k] = (uintptr_t)((next() % (1ull << 40)) & ~(uintptr_t)((next() % 8) ? 15 : 0));
        if (next() % 4 == 0) base[0] = base[1] + (uintptr_t)(next() % 4096);   // y near x
        const int dt = (int)(next() % 3), yt = (next() % 2) ? dt : (int)(next() % 3), tt = (int)(next() % 3);
        const int64_t mode = (next() % 4) ? (int64_t)(next() % 2) : 2 * (int64_t)(1 + next() % 4);
        rope::ProjPlan q;
        std::string why;
        const rope_status_t st = rope::make_proj_plan(
            reinterpret_cast<void*>(base[0]), (rope_dtype_t)yt, reinterpret_cast<void*>(base[1]),
            reinterpret_cast<void*>(base[2]), (rope_dtype_t)dt, ys, K, fake, ts, tst, fake, ts, tst,
            (rope_dtype_t)tt, mode, sl, &q, &why);
        if (st != ROPE_OK) {
            if (why.empty() || (st != ROPE_ERR_NULLPTR && st != ROPE_ERR_INVALID && st != ROPE_ERR_UNSUPPORTED)) ++bad;
            continue;
        }
        if (q.noop) {
            if (!(ys[0] == 0 || ys[1] == 0 || ys[2] == 0 || ys[3] == 0)) ++bad;
            continue;
        }
        ++proj_ok;
        const i128 M = (i128)ys[0] * ys[1], N = (i128)ys[2] * ys[3];
        bool good = K > 0 && K % 64 == 0 && rope::proj_head_dim_supported(ys[3]) && M * K < ((i128)1 << 31) &&
                    N * K < ((i128)1 << 31) && (dt == ROPE_DTYPE_BF16 || dt == ROPE_DTYPE_F16) &&
                    (yt == dt || yt == ROPE_DTYPE_F32) && (base[0] & 15) == 0 && (base[1] & 15) == 0 &&
                    (base[2] & 15) == 0;
        const i128 yb = M * N * (yt == ROPE_DTYPE_F32 ? 4 : 2), xb = M * K * 2, wb = N * K * 2;
        const auto apart = [](i128 a, i128 na, i128 b, i128 nb) { return a + na <= b || b + nb <= a; };
        good = good && apart(base[0], yb, base[1], xb) && apart(base[0], yb, base[2], wb);
        if (!good) ++bad;
    }
    // Multi-tensor calls: tensors that share a byte are rejected, others pass.
    long disjoint_ok = 0, disjoint_bad = 0;
    for (long it = 0; it < iters / 30; ++it) {
        rope::Plan ps[4];
        const int n = 1 + (int)(next() % 4);
        for (int i = 0; i < n; ++i) {
            ps[i].x = reinterpret_cast<void*>((uintptr_t)(next() % (1ull << 16)));
            ps[i].bytes = (int64_t)(1 + next() % 4096);
        }
        std::string why;
        const bool rejected = rope::check_disjoint(ps, n, &why) != ROPE_OK;
        bool overlap = false;
        for (int i = 0; i < n; ++i)
            for (int j = i + 1; j < n; ++j) {
                const i128 a = (i128)reinterpret_cast<uintptr_t>(ps[i].x), b = (i128)reinterpret_cast<uintptr_t>(ps[j].x);
                if (!(a + ps[i].bytes <= b || b + ps[j].bytes <= a)) overlap = true;
            }
        if (rejected != overlap) ++bad;
        (rejected ? disjoint_bad : disjoint_ok)++;
    }
    printf("projection accepted %ld, multi disjoint %ld overlapping %ld\n", proj_ok, disjoint_ok, disjoint_bad);
    printf("iters %ld accepted %ld noop %ld out-of-place accepted %ld copies %ld overlaps %ld bad %ld\n", iters, ok,
           noop, out_ok, out_copy, out_overlap, bad);
    return bad == 0 && ok > 1000 && noop > 1000 && out_ok > 1000 && out_copy > 1000 && out_overlap > 1000 &&
                   proj_ok > 1000 && disjoint_ok > 1000 && disjoint_bad > 1000
               ? 0
               : 1;
}
