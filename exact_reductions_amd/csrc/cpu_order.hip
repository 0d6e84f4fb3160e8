// The CPU's own rounding past 2^53: the value of the CPU extractors' running
// double sums, bit for bit, on every frame.
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
//   [HVS]    "ADR-1397: GPU psnr_hvs twins reproduce the CPU's running float
//            sum bit for bit"
//
// The CPU adds its terms one by one, in raster order, into a double; below
// 2^53 units every add is exact, past it each add rounds to the sum's last
// place [PSNR, Consequences; MOMENT, Decision].  The float_moment page
// defers reproducing that sequence of roundings, and the psnr_hvs page
// sketches an order-preserving device reduction without giving it (MOMENT,
// Alternatives; HVS, Alternatives).  This file computes it.
//
// In integer units (the terms are integers below 2^32, the sum an integer
// below 2^58) one CPU step is S <- RN53(S + t): the exact sum rounded to 53
// significant bits, ties to even.  While S stays inside one binade
// [2^e, 2^(e+1)) with e >= 53, S = m * u with u = 2^(e-52), and adding t =
// q*u + r moves m to m + q + d, where d depends only on r against u/2 and,
// on a tie, on the parity of m + q.  So a run of terms acts on S, inside a
// binade, as a two-state machine: from the parity of m it gives the total
// increase of m and the parity after the run.  Such maps compose in order.
//
//  1. stage 1 + stage 2 (plane_stats.hip) give each chunk's exact totals;
//  2. cpu_order_prefix scans them per frame (the exact running sum at each
//     chunk start, which predicts the binade the CPU's sum is in there);
//  3. cpu_order_maps computes, for every chunk past 2^53, the chunk's map
//     in the predicted binade (lanes map contiguous runs; the runs' maps
//     are composed in order);
//  4. cpu_order_walk, one wave per frame and sum, walks the chunks in order
//     with the exact running value S: a chunk that stays below 2^53 adds
//     exactly; a chunk whose map is for S's binade and keeps S inside it is
//     applied; any other chunk (the one crossing 2^53 or a binade edge, or a
//     wrong prediction) is walked in 64 sub-runs with maps for S's binade
//     and the next, and a sub-run that still does not fit is walked term by
//     term.  Every step is checked against S itself, so a prediction only
//     decides how fast the walk is, never what it returns.

#include "plane_stats.h"
#include "terms.h"

namespace vqx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr uint64_t kTwo53 = 1ull << 53;

// record field of square sum kk (noise, ref^2, dist^2)
__device__ __forceinline__ int record_field(int kk) { return kk == kSqNoise ? kNoise : kk == kSqRef ? kRef2 : kDist2; }

__device__ __forceinline__ int binade(uint64_t x) { return 63 - __clzll(static_cast<long long>(x)); }

// One CPU add in integer units: the exact S + t rounded to 53 significant
// bits, ties to even (IEEE 754 binary64 addition of two integers).
__device__ __forceinline__ uint64_t cpu_add(uint64_t S, uint32_t t)
{
    const uint64_t x = S + t;
    if (x < kTwo53)
        return x;
    const int k = binade(x) - 52;
    const uint64_t u = 1ull << k;
    uint64_t q = x >> k;
    const uint64_t r = x & (u - 1);
    const uint64_t half = u >> 1;
    if (r > half || (r == half && (q & 1)))
        ++q;
    return q << k;
}

// The two-state map of a run of adds inside binade e (k = e - 52 >= 1):
// starting from parity x of m, the run adds dm[x] to m and leaves parity p[x].
struct Map2 {
    uint64_t dm0 = 0, dm1 = 0;
    uint32_t p0 = 0, p1 = 1;
};

__device__ __forceinline__ void map_add(Map2 &m, uint32_t t, int k)
{
    const uint32_t q = t >> k;
    const uint32_t r = t & ((1u << k) - 1);
    const uint32_t half = 1u << (k - 1);
    const uint32_t up = r > half ? 1u : 0u;
    const uint32_t tie = r == half ? 1u : 0u;
    // on a tie, round up exactly when m + q is odd
    const uint32_t d0 = up | (tie & ((m.p0 + q) & 1u));
    const uint32_t d1 = up | (tie & ((m.p1 + q) & 1u));
    m.dm0 += q + d0;
    m.dm1 += q + d1;
    m.p0 = (m.p0 + q + d0) & 1u;
    m.p1 = (m.p1 + q + d1) & 1u;
}

// a then b
__device__ __forceinline__ Map2 map_then(const Map2 &a, const Map2 &b)
{
    Map2 c;
    c.dm0 = a.dm0 + (a.p0 ? b.dm1 : b.dm0);
    c.p0 = a.p0 ? b.p1 : b.p0;
    c.dm1 = a.dm1 + (a.p1 ? b.dm1 : b.dm0);
    c.p1 = a.p1 ? b.p1 : b.p0;
    return c;
}

// Applies map `m` (made for binade e) to S if S is in binade e and stays
// there; returns false otherwise (S unchanged).
__device__ __forceinline__ bool map_apply(uint64_t &S, const Map2 &m, int e)
{
    if (S < kTwo53 || binade(S) != e)
        return false;
    const int k = e - 52;
    const uint64_t mm = S >> k;
    const uint64_t m2 = mm + ((mm & 1) ? m.dm1 : m.dm0);
    if (m2 >= kTwo53)  // would leave the binade: the map does not hold
        return false;
    S = m2 << k;
    return true;
}

template <int kBytes>
__device__ __forceinline__ uint32_t sample(const void *plane, int64_t i)
{
    if constexpr (kBytes == 1)
        return static_cast<const uint8_t *>(plane)[i];
    else
        return static_cast<const uint16_t *>(plane)[i];
}

// The samples of one 32-bit word of a 16-byte vector, lowest first.
template <int kBytes>
__device__ __forceinline__ uint32_t word_sample(uint32_t w, int j)
{
    if constexpr (kBytes == 1)
        return (w >> (8 * j)) & 0xffu;
    else
        return (w >> (16 * j)) & 0xffffu;
}

// Adds the terms of vectors [v0, v1) of the batch, in order, to the maps of
// the square sums selected by `want` (one map per sum, binade e[kk]).
template <int kBytes>
__device__ __forceinline__ void map_vectors(Map2 (&m)[kSquares], const bool (&want)[kSquares],
                                            const int (&k)[kSquares], const u32x4 *R,
                                            const u32x4 *D, int64_t v0, int64_t v1)
{
    constexpr int per_word = 4 / kBytes;
    const bool needR = want[kSqNoise] || want[kSqRef];
    const bool needD = want[kSqNoise] || want[kSqDist];
    for (int64_t v = v0; v < v1; ++v) {
        const u32x4 a = needR ? __builtin_nontemporal_load(R + v) : u32x4{0, 0, 0, 0};
        const u32x4 b = needD ? __builtin_nontemporal_load(D + v) : u32x4{0, 0, 0, 0};
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
            for (int j = 0; j < per_word; ++j) {
                const uint32_t r = word_sample<kBytes>(aw[wd], j);
                const uint32_t d = word_sample<kBytes>(bw[wd], j);
#pragma unroll
                for (int kk = 0; kk < kSquares; ++kk)
                    if (want[kk])
                        map_add(m[kk], square_term<kBytes>(kk, r, d), k[kk]);
            }
        }
    }
}

// One pass over vectors [v0, v1) for square sum kk: the exact total of its
// terms and their maps in binades eA and eA + 1.
template <int kBytes>
__device__ __forceinline__ void run_maps(int kk, int eA, const u32x4 *R, const u32x4 *D, int64_t v0,
                                         int64_t v1, uint64_t &total, Map2 &mA, Map2 &mB)
{
    constexpr int per_word = 4 / kBytes;
    const int kA = eA - 52, kB = eA - 51;
    uint64_t s = 0;
    for (int64_t v = v0; v < v1; ++v) {
        const u32x4 a = __builtin_nontemporal_load(R + v);
        const u32x4 b = __builtin_nontemporal_load(D + v);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
            for (int j = 0; j < per_word; ++j) {
                const uint32_t t = square_term<kBytes>(kk, word_sample<kBytes>(aw[wd], j),
                                                       word_sample<kBytes>(bw[wd], j));
                s += t;
                map_add(mA, t, kA);
                map_add(mB, t, kB);
            }
        }
    }
    total = s;
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v)
{
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

// ------------------------------------------------------------ 2. prefix scan
// One workgroup per frame.  prefix[(f*chunks + c)*3 + kk] = exact sum of
// square kk over chunks 0..c-1 (chunk 0's record also holds the frame's few
// samples outside whole vectors); totals[f*3 + kk] = the frame's exact sum.
// The first moments never reach 2^53 (below 2^25 * 2^16 = 2^41): the CPU's
// values are the exact sums, written here.
__global__ __launch_bounds__(kThreads) void cpu_order_prefix(const uint64_t *rec, int chunks,
                                                             uint64_t *prefix, uint64_t *totals,
                                                             uint64_t *out_cpu_moments)
{
    __shared__ uint64_t lds[kThreads];
    const int64_t f = blockIdx.x;
    const int t = threadIdx.x;
    const int per = (chunks + kThreads - 1) / kThreads;
    const int c0 = t * per;
    const int c1 = c0 + per < chunks ? c0 + per : chunks;
    for (int kk = 0; kk < kSquares + 2; ++kk) {
        const int field = kk < kSquares ? record_field(kk) : (kk == kSquares ? kRef1 : kDist1);
        uint64_t local = 0;
        for (int c = c0; c < c1; ++c)
            local += rec[(f * chunks + c) * kRecordStride + field];
        // inclusive scan of the per-thread sums (Hillis-Steele)
        lds[t] = local;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const uint64_t add = t >= off ? lds[t - off] : 0;
            __syncthreads();
            lds[t] += add;
            __syncthreads();
        }
        const uint64_t total = lds[kThreads - 1];
        if (kk < kSquares) {
            uint64_t run = lds[t] - local;  // exclusive
            for (int c = c0; c < c1; ++c) {
                prefix[(f * chunks + c) * kSquares + kk] = run;
                run += rec[(f * chunks + c) * kRecordStride + field];
            }
            if (t == 0)
                totals[f * kSquares + kk] = total;
        } else if (t == 0) {
            out_cpu_moments[4 * f + (kk - kSquares)] = total;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ 3. chunk maps
// Map entry of chunk wg, square kk: {dm0, dm1, flags}; flags bit 0 = valid,
// bits 8..15 = binade e, bit 16 = p0, bit 17 = p1.  Written for every chunk
// on every call (invalid where not computed), so nothing stale is read.
constexpr int kMapStride = 4;  // uint64 per entry

template <int kBytes>
__global__ __launch_bounds__(kThreads) void cpu_order_maps(const void *ref, const void *dist,
                                                           int64_t pixels, int chunks,
                                                           const uint64_t *rec,
                                                           const uint64_t *prefix,
                                                           const uint64_t *totals, uint64_t *maps)
{
    constexpr int V = 16 / kBytes;
    const int64_t wg = blockIdx.x;
    const int64_t frame = wg / chunks;
    const int chunk = static_cast<int>(wg - frame * chunks);
    const int64_t e0 = frame * pixels, e1 = e0 + pixels;
    const int64_t vb = (e0 + V - 1) / V, ve = e1 / V;
    const int64_t cb = vb + static_cast<int64_t>(chunk) * kChunkVectors;
    const int64_t ce = cb + kChunkVectors < ve ? cb + kChunkVectors : ve;

    bool want[kSquares];
    int k[kSquares];
    bool any = false;
#pragma unroll
    for (int kk = 0; kk < kSquares; ++kk) {
        const uint64_t p = prefix[wg * kSquares + kk];
        const uint64_t r = rec[wg * kRecordStride + record_field(kk)];
        want[kk] = vb < ve && totals[frame * kSquares + kk] >= kTwo53 && p + r >= kTwo53;
        const int e = binade(p > kTwo53 ? p : kTwo53);
        k[kk] = e - 52;
        any = any || want[kk];
    }
    __shared__ uint64_t s_dm0[kSquares][kThreads], s_dm1[kSquares][kThreads];
    __shared__ uint32_t s_p[kSquares][kThreads];
    const int t = threadIdx.x;
    if (any) {
        Map2 m[kSquares];
        const int64_t v0 = cb + static_cast<int64_t>(t) * (kChunkVectors / kThreads);
        int64_t v1 = v0 + kChunkVectors / kThreads;
        v1 = v1 < ce ? v1 : ce;
        map_vectors<kBytes>(m, want, k, static_cast<const u32x4 *>(ref), static_cast<const u32x4 *>(dist),
                            v0, v0 < v1 ? v1 : v0);
#pragma unroll
        for (int kk = 0; kk < kSquares; ++kk) {
            s_dm0[kk][t] = m[kk].dm0;
            s_dm1[kk][t] = m[kk].dm1;
            s_p[kk][t] = m[kk].p0 | (m[kk].p1 << 1);
        }
        // compose the 256 run maps in order (lane 0's run comes first)
        for (int s = 1; s < kThreads; s <<= 1) {
            __syncthreads();
            if ((t & (2 * s - 1)) == 0) {
#pragma unroll
                for (int kk = 0; kk < kSquares; ++kk) {
                    Map2 a, b;
                    a.dm0 = s_dm0[kk][t]; a.dm1 = s_dm1[kk][t];
                    a.p0 = s_p[kk][t] & 1u; a.p1 = s_p[kk][t] >> 1;
                    b.dm0 = s_dm0[kk][t + s]; b.dm1 = s_dm1[kk][t + s];
                    b.p0 = s_p[kk][t + s] & 1u; b.p1 = s_p[kk][t + s] >> 1;
                    const Map2 c = map_then(a, b);
                    s_dm0[kk][t] = c.dm0;
                    s_dm1[kk][t] = c.dm1;
                    s_p[kk][t] = c.p0 | (c.p1 << 1);
                }
            }
        }
        __syncthreads();
    }
    if (t == 0) {
#pragma unroll
        for (int kk = 0; kk < kSquares; ++kk) {
            uint64_t *e = maps + (wg * kSquares + kk) * kMapStride;
            if (any && want[kk]) {
                e[0] = s_dm0[kk][0];
                e[1] = s_dm1[kk][0];
                e[2] = 1u | (static_cast<uint64_t>(k[kk] + 52) << 8) |
                       (static_cast<uint64_t>(s_p[kk][0] & 1u) << 16) |
                       (static_cast<uint64_t>(s_p[kk][0] >> 1) << 17);
            } else {
                e[0] = 0;
                e[1] = 0;
                e[2] = 0;
            }
        }
    }
}

// ------------------------------------------------------------------ 4. walk
// Walks sub-run by sub-run through vectors [cb, ce) of one chunk from the
// exact running value S.  All 64 lanes hold the same S throughout.
template <int kBytes>
__device__ uint64_t walk_chunk(uint64_t S, int kk, const u32x4 *R, const u32x4 *D, int64_t cb,
                               int64_t ce, const void *ref, const void *dist)
{
    constexpr int V = 16 / kBytes;
    constexpr int kSub = kChunkVectors / 64;  // vectors per lane's sub-run
    constexpr int kPer = kSub * V / 64;           // samples per lane in a sub-run walk
    const int lane = threadIdx.x;
    const int eA = S >= kTwo53 ? binade(S) : 53;
    Map2 mA, mB;
    uint64_t tot = 0;
    const int64_t v0 = cb + static_cast<int64_t>(lane) * kSub;
    int64_t v1 = v0 + kSub;
    v1 = v1 < ce ? v1 : ce;
    run_maps<kBytes>(kk, eA, R, D, v0, v0 < v1 ? v1 : v0, tot, mA, mB);
    for (int j = 0; j < 64; ++j) {
        const uint64_t tj = __shfl(tot, j, 64);
        if (S + tj < kTwo53) {
            S += tj;
            continue;
        }
        Map2 a, b;
        a.dm0 = __shfl(mA.dm0, j, 64); a.dm1 = __shfl(mA.dm1, j, 64);
        a.p0 = __shfl(mA.p0, j, 64); a.p1 = __shfl(mA.p1, j, 64);
        if (map_apply(S, a, eA))
            continue;
        b.dm0 = __shfl(mB.dm0, j, 64); b.dm1 = __shfl(mB.dm1, j, 64);
        b.p0 = __shfl(mB.p0, j, 64); b.p1 = __shfl(mB.p1, j, 64);
        if (map_apply(S, b, eA + 1))
            continue;
        // term by term through sub-run j: lane i holds its kPer samples
        const int64_t sv0 = cb + static_cast<int64_t>(j) * kSub;
        const int64_t nsamp = ((sv0 + kSub < ce ? sv0 + kSub : ce) - sv0) * V;
        uint32_t term[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int64_t idx = static_cast<int64_t>(lane) * kPer + q;
            term[q] = idx < nsamp ? square_term<kBytes>(kk, sample<kBytes>(ref, sv0 * V + idx),
                                                        sample<kBytes>(dist, sv0 * V + idx))
                                  : 0u;
        }
        for (int src = 0; src < 64; ++src) {
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const uint32_t tq = __shfl(term[q], src, 64);
                if (static_cast<int64_t>(src) * kPer + q < nsamp)
                    S = cpu_add(S, tq);
            }
        }
    }
    return S;
}

// One wave per (frame, square sum).
template <int kBytes>
__global__ __launch_bounds__(64) void cpu_order_walk(const void *ref, const void *dist, int64_t pixels,
                                                     int chunks, const uint64_t *rec,
                                                     const uint64_t *totals, const uint64_t *maps,
                                                     uint64_t *out_cpu_noise, uint64_t *out_cpu_moments)
{
    constexpr int V = 16 / kBytes;
    const int64_t frame = blockIdx.x / kSquares;
    const int kk = static_cast<int>(blockIdx.x - frame * kSquares);
    const int lane = threadIdx.x;
    uint64_t *dst = kk == kSqNoise ? &out_cpu_noise[frame] : &out_cpu_moments[4 * frame + 1 + kk];
    const uint64_t total = totals[frame * kSquares + kk];
    if (total < kTwo53) {  // every add of the CPU is exact: its sum is the exact one
        if (lane == 0)
            *dst = total;
        return;
    }
    const int64_t e0 = frame * pixels, e1 = e0 + pixels;
    const int64_t vb = (e0 + V - 1) / V, ve = e1 / V;
    const int64_t head_end = vb < ve ? vb * V : e1;
    const int64_t tail_begin = vb < ve ? ve * V : e1;
    const int head = static_cast<int>(head_end - e0), tail = static_cast<int>(e1 - tail_begin);
    const uint32_t hterm = lane < head ? square_term<kBytes>(kk, sample<kBytes>(ref, e0 + lane),
                                                             sample<kBytes>(dist, e0 + lane))
                                       : 0u;
    const uint32_t tterm = lane < tail ? square_term<kBytes>(kk, sample<kBytes>(ref, tail_begin + lane),
                                                             sample<kBytes>(dist, tail_begin + lane))
                                       : 0u;
    const uint64_t hsum = wave_sum64(hterm), tsum = wave_sum64(tterm);
    // the head comes first in raster order; it is far below 2^53, so exact
    uint64_t S = hsum;
    const u32x4 *R = static_cast<const u32x4 *>(ref);
    const u32x4 *D = static_cast<const u32x4 *>(dist);
    const int field = record_field(kk);
    for (int base = 0; base < chunks; base += 64) {
        // one chunk per lane: its exact total and its map entry
        const int c = base + lane;
        const int64_t wg = frame * chunks + c;
        uint64_t T = 0, dm0 = 0, dm1 = 0, flags = 0;
        if (c < chunks) {
            T = rec[wg * kRecordStride + field];
            if (c == 0)
                T -= hsum + tsum;  // chunk 0's record also holds the head and tail
            dm0 = maps[(wg * kSquares + kk) * kMapStride + 0];
            dm1 = maps[(wg * kSquares + kk) * kMapStride + 1];
            flags = maps[(wg * kSquares + kk) * kMapStride + 2];
        }
        const int n = chunks - base < 64 ? chunks - base : 64;
        for (int j = 0; j < n; ++j) {
            const uint64_t Tj = __shfl(T, j, 64);
            if (S + Tj < kTwo53) {
                S += Tj;
                continue;
            }
            const uint64_t fl = __shfl(flags, j, 64);
            if (fl & 1u) {
                Map2 m;
                m.dm0 = __shfl(dm0, j, 64);
                m.dm1 = __shfl(dm1, j, 64);
                m.p0 = static_cast<uint32_t>((fl >> 16) & 1u);
                m.p1 = static_cast<uint32_t>((fl >> 17) & 1u);
                if (map_apply(S, m, static_cast<int>((fl >> 8) & 0xffu)))
                    continue;
            }
            const int64_t cb = vb + static_cast<int64_t>(base + j) * kChunkVectors;
            const int64_t ce = cb + kChunkVectors < ve ? cb + kChunkVectors : ve;
            if (cb < ce)
                S = walk_chunk<kBytes>(S, kk, R, D, cb, ce, ref, dist);
        }
    }
    // the tail comes last
    for (int j = 0; j < tail; ++j)
        S = cpu_add(S, __shfl(tterm, j, 64));
    if (lane == 0)
        *dst = S;
}

}  // namespace

CpuOrderLayout cpu_order_layout(const Geometry &g)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    CpuOrderLayout l{};
    const size_t wgs = static_cast<size_t>(g.workgroups);
    l.records = 0;
    l.prefix = up(l.records + g.workspace_bytes);
    l.totals = up(l.prefix + wgs * kSquares * sizeof(uint64_t));
    l.maps = up(l.totals + static_cast<size_t>(g.nframes) * kSquares * sizeof(uint64_t));
    l.bytes = up(l.maps + wgs * kSquares * kMapStride * sizeof(uint64_t));
    return l;
}

hipError_t launch_plane_stats_cpu_order(const Geometry &g, const void *ref, const void *dist,
                                        uint64_t *out_noise, uint64_t *out_moments,
                                        uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                        void *workspace, hipStream_t stream)
{
    const CpuOrderLayout l = cpu_order_layout(g);
    char *ws = static_cast<char *>(workspace);
    uint64_t *rec = reinterpret_cast<uint64_t *>(ws + l.records);
    uint64_t *prefix = reinterpret_cast<uint64_t *>(ws + l.prefix);
    uint64_t *totals = reinterpret_cast<uint64_t *>(ws + l.totals);
    uint64_t *maps = reinterpret_cast<uint64_t *>(ws + l.maps);
    hipError_t err = launch_plane_stats(g, ref, dist, out_noise, out_moments, rec, stream);
    if (err != hipSuccess)
        return err;
    const unsigned nf = static_cast<unsigned>(g.nframes);
    cpu_order_prefix<<<dim3(nf), kThreads, 0, stream>>>(rec, g.chunks, prefix, totals, out_cpu_moments);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const dim3 grid(static_cast<unsigned>(g.workgroups));
    if (g.sample_bytes == 1) {
        cpu_order_maps<1><<<grid, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, rec, prefix, totals, maps);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        cpu_order_walk<1><<<dim3(nf * kSquares), 64, 0, stream>>>(ref, dist, g.pixels, g.chunks, rec, totals,
                                                                  maps, out_cpu_noise, out_cpu_moments);
    } else {
        cpu_order_maps<2><<<grid, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, rec, prefix, totals, maps);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        cpu_order_walk<2><<<dim3(nf * kSquares), 64, 0, stream>>>(ref, dist, g.pixels, g.chunks, rec, totals,
                                                                  maps, out_cpu_noise, out_cpu_moments);
    }
    return hipGetLastError();
}

}  // namespace vqx
