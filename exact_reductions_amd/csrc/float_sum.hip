// The psnr_hvs CPU extractor's running float sum, reproduced on the device
// bit for bit: for each buffer of float terms, the value a binary32
// accumulator holds after the terms were added one by one, in order, from
// zero.
//
// Sources (web pages, cited by title and section):
//   [HVS]    "ADR-1397: GPU psnr_hvs twins reproduce the CPU's running float
//            sum bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
//
// calc_psnrhvs() accumulates all of a plane's masked coefficient errors in
// a single float, one at a time, so the rounding of each add depends on
// the value accumulated before it [HVS, Context].  The page stores the
// terms on the device (64 per 8x8 block, row-major, blocks in raster
// order) and sums them on the host [HVS, Decision]; an order-preserving
// reduction on the device is its deferred alternative [HVS,
// Alternatives].  This file is that reduction.
//
// The terms are nonnegative (squares), so the sum S never decreases.  While
// S stays in one binade [2^E, 2^(E+1)), S = m * u with u = 2^(E-23) and
// 2^23 <= m < 2^24 (zero and the subnormals share the unit 2^-149 with the
// lowest normal binade, so there E = -126 and 0 <= m < 2^24).  A term t
// moves m by h = t/u rounded half up, except on a tie (t/u exactly halfway
// between two integers), where the result is whichever of m + h - 1 and
// m + h is even.  So a run of terms acts on m as a two-state machine on m's
// parity: the increase is the run's sum of h less the ties rounded down,
// whose count depends only on the parity at the start -- the same algebra
// as the CPU's double sums past 2^53 (cpu_order.hip), here with a unit that
// is a power of two of any sign.  Such maps compose in order.
//
//  1. fsum_tile_totals: per tile of 4096 terms, the total in binary64 (a
//     prediction only) and whether any term is negative or not finite;
//  2. fsum_plan, per buffer: the running total at each tile start, which
//     predicts the binade the float sum is in there, with a margin;
//  3. fsum_tile_maps: each tile's map in the predicted binade (and the
//     next, where the tile may cross into it), tiles handed out across the
//     buffers so that all buffers' maps appear at one pace; from binary32
//     sums of h, or term by term in order where the tile holds a tie or a
//     large term;
//  4. fsum_walk: one workgroup per buffer walks it -- with the running
//     value S, scans up to 1024 tile maps at once for S's binade and
//     applies all of them up to the first tile that has no map for that
//     binade or whose map leaves it; that tile is taken as 256 runs of 16
//     terms, scanned the same way, and the run where S leaves its binade is
//     added term by term in binary32.  Every step is checked against S
//     itself, so a prediction decides only how fast the walk is, never what
//     it returns.
//
// Step 4 runs on a second stream while step 3 still makes the maps: each
// map is published in 64-bit words that carry their own "ready" bit,
// written and read with relaxed device-scope atomics (single-copy atomic
// and coherent across the XCDs' L2s, so no fence is needed: a word is
// either seen whole or seen as not ready).  A walk waits at a tile whose
// map is not out yet; its waits are bounded, and a walk that reaches the
// bound leaves its buffer to step 4 again, run after step 3 on the
// caller's stream.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include "plane_stats.h"

#pragma clang fp contract(off)

namespace vqx {
namespace {

constexpr int kThreads = kFsThreads;               // four wave64s
constexpr int kRun = kFsRunTerms;                  // terms per thread in a tile
constexpr int kTile = kFsTileTerms;                // terms per tile
constexpr int kPad = kTile + kTile / kRun;         // LDS words of a tile, one pad per run
constexpr uint32_t kTop = 1u << 24;                // m at the top of a binade
constexpr uint32_t kSat = 1u << 25;                // an increase this large leaves any binade
constexpr uint32_t kNaN = 0x7fc00000u;
constexpr uint32_t kInf = 0x7f800000u;
static_assert(kThreads * kRun == kTile, "a tile is one run per thread");

// The effect of a run of terms on m inside one binade: m grows by H less
// the ties rounded down, td0 from an even start and td1 from an odd one.
// H saturates at kSat (the run then certainly leaves the binade).
struct Map {
    uint32_t H, td0, td1;
};

// A tile's record: its plan (binades predicted) and its maps, published.
//   w0: bit 63 ready, bits 61..60 the count of planned binades (0..2),
//       bits 59..52 the first binade's unit exponent + 149, bits 51..0 the
//       map in the first binade;
//   w1: bit 63 ready, bits 51..0 the map in the second binade.
// A map is H (bits 25..0, at most kSat), td0 (38..26) and td1 (51..39);
// td0, td1 count ties, at most a tile's 4096 terms.
struct alignas(32) Rec {
    uint64_t w0, w1;
    uint32_t plan;  // (unit exponent of the first binade + 256) | (count << 16), count 0..2
    uint32_t unused[3];
};
static_assert(sizeof(Rec) == 32, "records stay 32 bytes");

constexpr uint64_t kReady = 1ull << 63;

__device__ __forceinline__ uint64_t pack_map(const Map &m)
{
    return static_cast<uint64_t>(m.H) | (static_cast<uint64_t>(m.td0) << 26) | (static_cast<uint64_t>(m.td1) << 39);
}

__device__ __forceinline__ Map unpack_map(uint64_t w)
{
    return {static_cast<uint32_t>(w) & 0x3ffffffu, static_cast<uint32_t>(w >> 26) & 0x1fffu,
            static_cast<uint32_t>(w >> 39) & 0x1fffu};
}

// w0's fields other than the map
__device__ __forceinline__ uint64_t rec_head(int count, int uexp)
{
    return (static_cast<uint64_t>(count) << 60) | (static_cast<uint64_t>(uexp + 149) << 52);
}

// Publication and observation of a record word (relaxed, device scope).
__device__ __forceinline__ void publish(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t observe(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t observe(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A buffer's done word, per call: open (cleared by fsum_plan), walked by
// the walk beside the map kernel (which then writes the result), given up
// by it, or claimed by the walk after the map kernel (which then writes
// the result).  The two walks change it by compare-and-swap from open, so
// exactly one of them writes each result.
enum : uint32_t { kOpen = 0, kWalked = 1, kGivenUp = 2, kClaimed = 3 };


__device__ __forceinline__ Map identity_map() { return {0u, 0u, 0u}; }
__device__ __forceinline__ Map leaving_map() { return {kSat, 0u, 0u}; }

// a, then b
__device__ __forceinline__ Map compose(const Map &a, const Map &b)
{
    // m's parity after a, from each start parity
    const uint32_t q0 = (a.H - a.td0) & 1u;
    const uint32_t q1 = (1u + a.H - a.td1) & 1u;
    Map c;
    const uint32_t h = a.H + b.H;  // both <= kSat: no wrap
    c.H = h > kSat ? kSat : h;
    c.td0 = a.td0 + (q0 ? b.td1 : b.td0);
    c.td1 = a.td1 + (q1 ? b.td1 : b.td0);
    return c;
}

// One term (a binary32 bit pattern, nonnegative) in the binade whose unit is
// 2^uexp.  t = M * 2^texp; h = M / 2^k rounded half up with k = uexp - texp.
__device__ __forceinline__ Map term_map(uint32_t t, int uexp)
{
    const uint32_t ef = (t >> 23) & 0xffu;
    const uint32_t M = ef ? ((t & 0x7fffffu) | 0x800000u) : (t & 0x7fffffu);
    const int texp = ef ? static_cast<int>(ef) - 150 : -149;
    const int k = uexp - texp;
    uint32_t h = 0;
    bool tie = false;
    if (k <= 0) {
        // t is a whole number of units
        h = M == 0 ? 0u : (k <= -2 ? kSat : (M << -k));
        h = h > kSat ? kSat : h;
    } else if (k < 26) {
        const uint32_t half = 1u << (k - 1);
        h = (M + half) >> k;
        tie = (M & ((1u << k) - 1u)) == half;
    }  // else t < u/4: h = 0, no tie
    // on a tie from parity p, m + h is rounded down when it is odd
    return {h, tie ? (h & 1u) : 0u, tie ? ((h & 1u) ^ 1u) : 0u};
}

// S's binade: the unit's exponent and m.
__device__ __forceinline__ void split(uint32_t S, int &uexp, uint32_t &m)
{
    const uint32_t ef = S >> 23;
    if (ef <= 1) {  // zero, subnormal, or the lowest normal binade
        uexp = -149;
        m = S;
    } else {
        uexp = static_cast<int>(ef) - 150;
        m = (S & 0x7fffffu) | 0x800000u;
    }
}

// S from its binade and m (m <= 2^24; m == 2^24 is the next power of two,
// or infinity above the largest binade).
__device__ __forceinline__ uint32_t join(int uexp, uint32_t m)
{
    return (static_cast<uint32_t>(uexp + 149) << 23) + m;
}

__device__ __forceinline__ bool bad_term(uint32_t t)
{
    return (t > 0x80000000u) || ((t & 0x7f800000u) == 0x7f800000u);
}

// ------------------------------------------------------- workgroup scans
// Ordered scan of the threads' maps (thread order = term order): returns
// the inclusive prefix, and the exclusive one in `excl`.  All threads must
// call it.
// The map of the lane CTRL (a DPP row shift or row broadcast) selects
// below this one, or the identity where there is none (ROWS: the rows that
// receive one).
// (Each move stays a move of its own: folded into the arithmetic that
// follows, a move with a row mask leaves the masked rows' destination as it
// was rather than the identity's, which compose does not tolerate.)
template <int CTRL, int ROWS>
__device__ __forceinline__ Map map_below(const Map &x)
{
    Map y;
    y.H = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.H), CTRL, ROWS, 0xf, false));
    y.td0 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.td0), CTRL, ROWS, 0xf, false));
    y.td1 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x.td1), CTRL, ROWS, 0xf, false));
    asm volatile("" : "+v"(y.H), "+v"(y.td0), "+v"(y.td1));
    return y;
}

__device__ __forceinline__ Map scan_maps(Map x, Map &excl)
{
    __shared__ Map wave_total[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // inclusive, in lane order: row_shr 1, 2, 4, 8 inside each row of 16,
    // then row_bcast 15 (into rows 1 and 3) and 31 (into rows 2 and 3)
    x = compose(map_below<0x111, 0xf>(x), x);
    x = compose(map_below<0x112, 0xf>(x), x);
    x = compose(map_below<0x114, 0xf>(x), x);
    x = compose(map_below<0x118, 0xf>(x), x);
    x = compose(map_below<0x142, 0xa>(x), x);
    x = compose(map_below<0x143, 0xc>(x), x);
    Map prev;
    prev.H = __shfl_up(x.H, 1, 64);
    prev.td0 = __shfl_up(x.td0, 1, 64);
    prev.td1 = __shfl_up(x.td1, 1, 64);
    if (lane == 0)
        prev = identity_map();
    if (lane == 63)
        wave_total[wave] = x;
    __syncthreads();
    Map before = identity_map();
    for (int w = 0; w < wave; ++w)
        before = compose(before, wave_total[w]);
    __syncthreads();
    excl = compose(before, prev);
    return compose(before, x);
}

__device__ __forceinline__ Map scan_maps(Map x)
{
    Map excl;
    return scan_maps(x, excl);
}

// Ordered composition of all the threads' maps; every thread gets it.
__device__ __forceinline__ Map reduce_maps(Map x)
{
    __shared__ Map last;
    x = scan_maps(x);
    if (threadIdx.x == kThreads - 1)
        last = x;
    __syncthreads();
    const Map r = last;
    __syncthreads();
    return r;
}

// The first thread whose flag is set, or kThreads.  All threads must call it.
__device__ __forceinline__ int first_set(bool flag)
{
    __shared__ int first[kThreads / 64];
    const uint64_t b = __ballot(flag);
    if ((threadIdx.x & 63) == 0)
        first[threadIdx.x >> 6] = b ? static_cast<int>(__builtin_ctzll(b)) + (threadIdx.x & ~63) : kThreads;
    __syncthreads();
    int f = kThreads;
    for (int w = 0; w < kThreads / 64; ++w)
        f = first[w] < f ? first[w] : f;
    __syncthreads();
    return f;
}

// A tile's terms into LDS, term i at i + i/kRun (a pad word per run keeps
// each thread's run on its own banks); missing terms past the buffer's end
// are zeros, which add nothing.
__device__ __forceinline__ void load_tile(const float *tile_base, int64_t count, uint32_t *lds)
{
    const uint32_t *src = reinterpret_cast<const uint32_t *>(tile_base);
    // every lane loads (past the end, the tile's first term, dropped after),
    // so that no branch stands between the 16 loads and their waits: they
    // are all in flight at once
    uint32_t v[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
        const int i = threadIdx.x + j * kThreads;
        v[j] = __builtin_nontemporal_load(src + (i < count ? i : 0));
    }
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
        const int i = threadIdx.x + j * kThreads;
        lds[i + i / kRun] = i < count ? v[j] : 0u;
    }
    __syncthreads();
}

__device__ __forceinline__ float pow2(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }

// This thread's run of the tile in LDS, in the binade of unit 2^uexp.  Where
// the unit scales to in binary32 and the run holds no tie and no term of
// 2^22 units or more, h = floor(t/u + 1/2) read off binary32 (exact, as in
// fsum_tile_maps) and summed in binary32 (exact below 2^24; a run that
// reaches 2^24 leaves any binade, and saturates); otherwise term by term
// in integers.
__device__ __forceinline__ Map run_map(const uint32_t *lds, int uexp)
{
    const uint32_t *r = lds + threadIdx.x * (kRun + 1);
    uint32_t v[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j)
        v[j] = r[j];
    if (uexp >= -126) {
        const float scale = pow2(-uexp);
        float H = 0.0f, lo = 1.0f, top = 0.0f;
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            const float x = __uint_as_float(v[j]) * scale;
            const float y = x + 0.5f;
            const float f = floorf(y);
            lo = fminf(lo, y - f);
            top = fmaxf(top, x);
            H += f;
        }
        if (lo != 0.0f && top < 0x1p22f)
            return H < 0x1p24f ? Map{static_cast<uint32_t>(H), 0u, 0u} : leaving_map();
    }
    Map x = identity_map();
#pragma unroll
    for (int j = 0; j < kRun; ++j)
        x = compose(x, term_map(v[j], uexp));
    return x;
}

// ------------------------------------------------------------- kernel 1
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// This thread's 16 terms of a tile, loaded: with 16-byte loads where the
// tile is whole and 16-byte aligned (thread t takes vectors t, t+256, t+512
// and t+768), else term by term (thread t takes terms t, t+256, ...); zeros
// stand in past the buffer's end.  The order of a thread's terms does not
// matter to the users (sums, ORs, counts).
struct TileTerms {
    u32x4 x[kRun / 4];
};

__device__ __forceinline__ TileTerms load_tile_terms(const float *tile_base, int64_t count)
{
    const uint32_t *src = reinterpret_cast<const uint32_t *>(tile_base);
    TileTerms t;
    if (count >= kTile && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        const u32x4 *v = reinterpret_cast<const u32x4 *>(src);
#pragma unroll
        for (int j = 0; j < kRun / 4; ++j)
            t.x[j] = __builtin_nontemporal_load(v + threadIdx.x + j * kThreads);
    } else {
        // branch-free loads, as in load_tile
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            const int i = threadIdx.x + j * kThreads;
            t.x[j / 4][j % 4] = __builtin_nontemporal_load(src + (i < count ? i : 0));
        }
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            const int i = threadIdx.x + j * kThreads;
            t.x[j / 4][j % 4] = i < count ? t.x[j / 4][j % 4] : 0u;
        }
    }
    return t;
}

template <class F>
__device__ __forceinline__ void for_terms(const TileTerms &t, F &&f)
{
#pragma unroll
    for (int j = 0; j < kRun / 4; ++j) {
        const uint32_t t0 = t.x[j].x, t1 = t.x[j].y, t2 = t.x[j].z, t3 = t.x[j].w;
        f(t0);
        f(t1);
        f(t2);
        f(t3);
    }
}

template <class F>
__device__ __forceinline__ void for_tile_terms(const float *tile_base, int64_t count, F &&f)
{
    for_terms(load_tile_terms(tile_base, count), f);
}

// Sum and OR over the workgroup; every thread gets both.  All threads must
// call it.
// Wave64 sums and ORs by DPP, at VALU speed (lane shuffles go through the
// LDS crossbar): quad swaps and row rotates total each row of 16 lanes in
// all its lanes, then row broadcasts carry rows 0..2 into the rows above,
// so lane 63 ends with the wave's total.  (+ and | are commutative, so the
// rows a broadcast leaves out keep their value either way.)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_from(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xf, false));
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op)
{
    v = op(v, dpp_from<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_from<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_from<0x124, 0xf>(v));  // row_ror:4
    v = op(v, dpp_from<0x128, 0xf>(v));  // row_ror:8
    v = op(v, dpp_from<0x142, 0xa>(v));  // row_bcast:15 into rows 1, 3
    v = op(v, dpp_from<0x143, 0xc>(v));  // row_bcast:31 into rows 2, 3
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a | b; });
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ float wave_sum_f32(float v)
{
    return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

__device__ __forceinline__ void workgroup_sum_or(float &s, uint32_t &o)
{
    __shared__ float ls[kThreads / 64];
    __shared__ uint32_t lo[kThreads / 64];
    s = wave_sum_f32(s);
    o = wave_or_u32(o);
    if ((threadIdx.x & 63) == 0) {
        ls[threadIdx.x >> 6] = s;
        lo[threadIdx.x >> 6] = o;
    }
    __syncthreads();
    s = 0.0f;
    o = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        s += ls[w];
        o |= lo[w];
    }
    __syncthreads();
}

// grid (tiles, buffers): each tile's total (binary32 adds in any order: a
// prediction only) and whether any term is negative or not finite.
__global__ __launch_bounds__(kThreads) void fsum_tile_totals(const float *terms, int64_t nterms, int ntiles,
                                                             double *totals, uint32_t *bad)
{
    const int tile = blockIdx.x, buf = blockIdx.y;
    const int64_t first = static_cast<int64_t>(tile) * kTile;
    float s = 0.0f;
    uint32_t b = 0;
    for_tile_terms(terms + static_cast<int64_t>(buf) * nterms + first, nterms - first, [&](uint32_t t) {
        b |= bad_term(t) ? 1u : 0u;
        s += __uint_as_float(t & 0x7fffffffu);
    });
    workgroup_sum_or(s, b);
    if (threadIdx.x == 0) {
        totals[static_cast<int64_t>(buf) * ntiles + tile] = static_cast<double>(s);
        bad[static_cast<int64_t>(buf) * ntiles + tile] = b;
    }
}

// ------------------------------------------------------------- kernel 2
// The binade (as the unit's exponent) a value v >= 0 lies in, clamped to
// the float range.
__device__ __forceinline__ int unit_exponent_of(double v)
{
    if (!(v >= 0x1p-125))
        return -149;
    if (v >= 0x1p127)
        return 127 - 23;
    int e;
    (void)frexp(v, &e);  // v = f * 2^e, 0.5 <= f < 1: binade e - 1
    return (e - 1) - 23;
}

// One workgroup per buffer: the running total at each tile start and the
// binades the float sum may be in over each tile.  plan = (unit exponent of
// the first + 256) | (count << 16), count 0 (no maps), 1 or 2.  The totals
// pass through LDS kPlanChunk at a time: read coalesced (every load of a
// chunk in flight at once), summed in order by thread runs of kPlanPer, the
// runs' sums scanned, the plans made along each run, and the records
// written coalesced.
constexpr int kPlanPer = 16;
constexpr int kPlanChunk = kThreads * kPlanPer;

__global__ __launch_bounds__(kThreads) void fsum_plan(const double *totals, const uint32_t *bad, int ntiles,
                                                      Rec *recs, uint32_t *buffer_bad, uint32_t *done)
{
    const int buf = blockIdx.x;
    const int me = static_cast<int>(threadIdx.x);
    if (me == 0)
        done[buf] = kOpen;
    const double *tot = totals + static_cast<int64_t>(buf) * ntiles;
    const uint32_t *bd = bad + static_cast<int64_t>(buf) * ntiles;
    Rec *rc = recs + static_cast<int64_t>(buf) * ntiles;
    // chunk entry i at i + i/kPlanPer: a pad per run keeps a run's serial
    // reads (and the plans' writes) spread over the banks
    __shared__ double tl[kPlanChunk + kThreads];
    __shared__ uint32_t pl[kPlanChunk + kThreads];
    __shared__ double ex[kThreads];
    constexpr double kMargin = 1.0 / 128;  // the float sum's drift from the exact one, allowed
    double base = 0.0;  // the running total before the chunk (a prediction: any order of adds will do)
    uint32_t b = 0;
    for (int c0 = 0; c0 < ntiles; c0 += kPlanChunk) {
        const int cn = ntiles - c0 < kPlanChunk ? ntiles - c0 : kPlanChunk;
        double v[kPlanPer];
        uint32_t f[kPlanPer];
#pragma unroll
        for (int j = 0; j < kPlanPer; ++j) {
            const int i = me + j * kThreads;
            const int64_t at = c0 + (i < cn ? i : 0);
            v[j] = tot[at];
            f[j] = bd[at];
        }
#pragma unroll
        for (int j = 0; j < kPlanPer; ++j) {
            const int i = me + j * kThreads;
            tl[i + i / kPlanPer] = i < cn ? v[j] : 0.0;
            b |= i < cn ? f[j] : 0u;
        }
        __syncthreads();
        const double *run = tl + me * (kPlanPer + 1);
        double mine = 0.0;
#pragma unroll
        for (int j = 0; j < kPlanPer; ++j)
            mine += run[j];
        ex[me] = mine;
        __syncthreads();
        for (int d = 1; d < kThreads; d <<= 1) {
            const double y = me >= d ? ex[me - d] : 0.0;
            __syncthreads();
            ex[me] += y;
            __syncthreads();
        }
        double p = base + (ex[me] - mine);
        const double chunk_total = ex[kThreads - 1];
        uint32_t *mine_pl = pl + me * (kPlanPer + 1);
#pragma unroll
        for (int j = 0; j < kPlanPer; ++j) {
            const double t = run[j];
            const int e_lo = unit_exponent_of(p * (1.0 - kMargin));
            const int e_hi = unit_exponent_of((p + t) * (1.0 + kMargin));
            const int n = e_hi - e_lo + 1;
            const int count = n <= 2 ? n : 0;
            mine_pl[j] = static_cast<uint32_t>(e_lo + 256) | (static_cast<uint32_t>(count) << 16);
            p += t;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPlanPer; ++j) {
            const int i = me + j * kThreads;
            if (i < cn) {
                const uint32_t plan = pl[i + i / kPlanPer];
                Rec &r = rc[c0 + i];
                r.plan = plan;
                // a tile without maps is ready now; the others once their maps are
                r.w0 = (plan >> 16) == 0 ? kReady | rec_head(0, static_cast<int>(plan & 0xffffu) - 256) : 0;
                r.w1 = 0;
            }
        }
        base += chunk_total;
        __syncthreads();  // before the next chunk overwrites the LDS
    }
    __shared__ uint32_t anybad;
    if (me == 0)
        anybad = 0;
    __syncthreads();
    if (b)
        atomicOr(&anybad, 1u);
    __syncthreads();
    if (me == 0)
        buffer_bad[buf] = anybad;
}

// A tile's maps in its planned binades, in order, term by term (where it
// holds a tie, a large term, or its unit is too small to scale to),
// published.  All threads must call it.
__device__ void ordered_maps(const float *terms, int64_t nterms, int ntiles, Rec *recs, uint32_t at, uint32_t *lds)
{
    const int buf = static_cast<int>(at / static_cast<uint32_t>(ntiles));
    const int tile = static_cast<int>(at - static_cast<uint32_t>(buf) * static_cast<uint32_t>(ntiles));
    const uint32_t pl = recs[at].plan;
    const int n = static_cast<int>(pl >> 16);
    const int uexp = static_cast<int>(pl & 0xffffu) - 256;
    const int64_t first = static_cast<int64_t>(tile) * kTile;
    load_tile(terms + static_cast<int64_t>(buf) * nterms + first, nterms - first, lds);
    Map m[2];
    for (int k = 0; k < n; ++k) {
        // this thread's run, term by term (one term in registers at a time)
        const uint32_t *r = lds + threadIdx.x * (kRun + 1);
        Map x = identity_map();
#pragma unroll 1
        for (int j = 0; j < kRun; ++j)
            x = compose(x, term_map(r[j], uexp + k));
        m[k] = reduce_maps(x);
    }
    if (threadIdx.x == 0) {
        if (n == 2)
            publish(&recs[at].w1, kReady | pack_map(m[1]));
        publish(&recs[at].w0, kReady | rec_head(n, uexp) | pack_map(m[0]));
    }
}

// ------------------------------------------------------------- kernel 3
// A tile's map in the binade of unit 2^uexp, from the terms as loaded, where
// no term is a tie and none is 2^22 units or more.  Then the map is the sum
// of h = floor(t/u + 1/2) and no tie is rounded down.  In binary32, x = t/u
// is exact (a power-of-two scale; where it falls below the normal range it
// is far below 1/2, and h = 0 either way), x + 1/2 is exact below 2^22, and
// the floor is exact: so h is read off floor(x + 1/2), and the term is a tie
// exactly where x + 1/2 is an integer.  Where that does not hold (a tie, a
// large term, or a unit too small to scale to) the map comes from the
// ordered path.  A sum of h that reaches 2^24 marks the tile as leaving the
// binade: with a large term that mark may be early, which only sends the
// walk through the tile run by run.

// One workgroup per tile, handed out tile by tile across the buffers (tile
// 0 of every buffer, then tile 1, ...): each planned tile's map in its one
// or two binades, published.
__global__ __launch_bounds__(kThreads) void fsum_tile_maps(const float *terms, int64_t nterms, int ntiles,
                                                           int nbuffers, Rec *recs)
{
    const uint32_t cell = blockIdx.x;
    const int tile = static_cast<int>(cell / static_cast<uint32_t>(nbuffers));
    const int buf = static_cast<int>(cell - static_cast<uint32_t>(tile) * static_cast<uint32_t>(nbuffers));
    const int64_t at = static_cast<int64_t>(buf) * ntiles + tile;
    const int64_t first = static_cast<int64_t>(tile) * kTile;
    const float *tb = terms + static_cast<int64_t>(buf) * nterms + first;
    // the terms are read before the plan arrives (only a sum's first tiles
    // have none), so the two reads are in flight together
    const TileTerms terms_in = load_tile_terms(tb, nterms - first);
    const uint32_t pl = recs[at].plan;
    const int n = static_cast<int>(pl >> 16);
    if (n == 0)
        return;
    const int uexp = static_cast<int>(pl & 0xffffu) - 256;
    // unscaled to units of the lower binade; the upper's units are twice as large
    const bool scalable = uexp >= -126;
    const float scale = pow2(scalable ? -uexp : 0);
    // per binade: the sum of h (in binary32: exact while below 2^24, and
    // at least 2^24 once the exact sum is), the smallest fraction of t/u +
    // 1/2 (0 where a term ties) and the largest t/u.  A buffer holding a
    // negative or non-finite term gets NaN whatever its maps say.
    float Hf0 = 0.0f, Hf1 = 0.0f, lo0 = 1.0f, lo1 = 1.0f, top = 0.0f;
    for_terms(terms_in, [&](uint32_t t) {
        const float x0 = __uint_as_float(t) * scale;
        const float y0 = x0 + 0.5f;
        const float f0 = floorf(y0);
        lo0 = fminf(lo0, y0 - f0);
        top = fmaxf(top, x0);
        Hf0 += f0;
        if (n == 2) {
            const float x1 = x0 * 0.5f;
            const float y1 = x1 + 0.5f;
            const float f1 = floorf(y1);
            lo1 = fminf(lo1, y1 - f1);
            Hf1 += f1;
        }
    });
    // odd: bit 0 a tie or a large term in the lower binade, bit 1 in the upper
    const uint32_t odd = ((lo0 == 0.0f || !(top < 0x1p22f)) ? 1u : 0u) |
                         ((n == 2 && (lo1 == 0.0f || !(top < 0x1p23f))) ? 2u : 0u);
    // a thread whose sum reaches 2^24 leaves any binade; the others' sums
    // are exact integers below 2^24
    const uint32_t leaves = (Hf0 >= 0x1p24f ? 1u : 0u) | (Hf1 >= 0x1p24f ? 2u : 0u);
    uint32_t H0 = static_cast<uint32_t>(Hf0 < 0x1p24f ? Hf0 : 0.0f);
    uint32_t H1 = static_cast<uint32_t>(Hf1 < 0x1p24f ? Hf1 : 0.0f);
    // the workgroup's flags and sums of h (each thread's below 2^24, so
    // the 256 add up below 2^32), one barrier for all three
    __shared__ uint32_t lh[3][kThreads / 64];
    {
        const uint32_t wf = wave_or_u32(odd | (leaves << 2) | (scalable ? 0u : 3u));
        const uint32_t w0 = wave_sum_u32(H0), w1 = wave_sum_u32(H1);
        if ((threadIdx.x & 63) == 0) {
            lh[0][threadIdx.x >> 6] = w0;
            lh[1][threadIdx.x >> 6] = w1;
            lh[2][threadIdx.x >> 6] = wf;
        }
    }
    __syncthreads();
    uint32_t flags = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w)
        flags |= lh[2][w];
    // a tile that needs the ordered path in any of its binades (a tie, a
    // large term, or a unit too small to scale to) has all its maps made
    // term by term, in order, from the tile staged in LDS (read again: such
    // tiles are few)
    if (flags & 3u) {
        __shared__ uint32_t lds[kPad];
        ordered_maps(terms, nterms, ntiles, recs, static_cast<uint32_t>(at), lds);
        return;
    }
    if (threadIdx.x == 0) {
        Map m[2];
        for (int k = 0; k < n; ++k) {
            if (flags & (4u << k)) {
                m[k] = leaving_map();
            } else {
                uint32_t h = 0;
#pragma unroll
                for (int w = 0; w < kThreads / 64; ++w)
                    h += lh[k][w];
                m[k] = {h > kSat ? kSat : h, 0u, 0u};
            }
        }
        if (n == 2)
            publish(&recs[at].w1, kReady | pack_map(m[1]));
        publish(&recs[at].w0, kReady | rec_head(n, uexp) | pack_map(m[0]));
    }
}

// ------------------------------------------------------------- kernel 4
// Applies a scanned map to (uexp, m): the new m, or kSat+ when it leaves.
__device__ __forceinline__ uint32_t apply(const Map &x, uint32_t m)
{
    if (x.H >= kSat)
        return kSat + kTop;
    return m + x.H - ((m & 1u) ? x.td1 : x.td0);
}

// Exclusive prefix sum of the threads' counts, in thread order; `total`
// gets the workgroup's.  All threads must call it.
__device__ __forceinline__ uint32_t scan_counts(uint32_t c, uint32_t &total)
{
    __shared__ uint32_t wave_total[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        x += lane >= d ? y : 0u;
    }
    if (lane == 63)
        wave_total[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        before += w < wave ? wave_total[w] : 0u;
        total += wave_total[w];
    }
    __syncthreads();
    return before + x - c;
}

// The tile in LDS, with S (bit pattern) at its start: S after it.  A tile
// over which the sum may cross more than two binades (the start of a sum)
// is added term by term by one thread, its zero terms left out (adding a
// zero leaves the sum as it was [HVS, Consequences]; -0 too, to a sum that
// is +0 or positive); any other tile run by run.  All threads must call it.
__device__ uint32_t walk_tile(const uint32_t *lds, uint32_t S, bool one_by_one)
{
    __shared__ uint32_t shared_S;
    if (one_by_one) {
        __shared__ uint32_t nonzero[kTile];
        // the tile's nonzero terms, in order, packed
        const uint32_t *mine = lds + threadIdx.x * (kRun + 1);
        uint32_t count = 0;
#pragma unroll
        for (int j = 0; j < kRun; ++j)
            count += (mine[j] & 0x7fffffffu) ? 1u : 0u;
        uint32_t total;
        uint32_t at = scan_counts(count, total);
#pragma unroll
        for (int j = 0; j < kRun; ++j)
            if (mine[j] & 0x7fffffffu)
                nonzero[at++] = mine[j];
        __syncthreads();
        if (threadIdx.x == 0) {
            float f = __uint_as_float(S);
            uint32_t i = 0;
            for (; i + kRun <= total; i += kRun) {
                // 16 reads issued together, then their 16 adds
                float v[kRun];
#pragma unroll
                for (int j = 0; j < kRun; ++j)
                    v[j] = __uint_as_float(nonzero[i + j]);
#pragma unroll
                for (int j = 0; j < kRun; ++j)
                    f = f + v[j];
            }
            for (; i < total; ++i)
                f = f + __uint_as_float(nonzero[i]);
            shared_S = __float_as_uint(f);
        }
        __syncthreads();
        S = shared_S;
        __syncthreads();
        return S;
    }
    int r0 = 0;  // runs before r0 are added
    while (r0 < kThreads && S != kInf) {
        int uexp;
        uint32_t m;
        split(S, uexp, m);
        const int me = static_cast<int>(threadIdx.x);
        const Map x = me >= r0 ? run_map(lds, uexp) : identity_map();
        const uint32_t after = apply(scan_maps(x), m);  // m after this thread's run
        const int stop = first_set(me >= r0 && after >= kTop);
        // S before run `stop` (after the whole tile if none stops)
        if (me == 0)
            shared_S = S;
        __syncthreads();
        if (me == stop - 1 && me >= r0)
            shared_S = join(uexp, after);
        __syncthreads();
        S = shared_S;
        __syncthreads();
        if (stop == kThreads)
            break;
        // run `stop` reaches the binade's top exactly -- applied whole: the
        // terms after the top add nothing in either binade -- or crosses
        // it, and is added term by term in binary32
        if (me == stop) {
            if (after == kTop) {
                shared_S = join(uexp, kTop);
            } else {
                float f = __uint_as_float(S);
                const uint32_t *r = lds + stop * (kRun + 1);
                float v[kRun];
#pragma unroll
                for (int j = 0; j < kRun; ++j)
                    v[j] = __uint_as_float(r[j]);
#pragma unroll
                for (int j = 0; j < kRun; ++j)
                    f = f + v[j];
                shared_S = __float_as_uint(f);
            }
        }
        __syncthreads();
        S = shared_S;
        __syncthreads();
        r0 = stop + 1;
    }
    return S;
}


// One workgroup per buffer.  A window is kWindow tiles, kPerThread
// consecutive ones per thread.
constexpr int kPerThread = 4;
constexpr int kWindow = kThreads * kPerThread;

// The walk waits where a map is not out yet.  While it waits one lane
// looks at the tile's record and at one kAhead tiles on (the map kernel
// hands tiles out in order, so most of the tiles between are out by then),
// every kNap (s_sleep units of 64 clocks).  Beside the map kernel a wait
// gets new maps within microseconds; one that lasts the bound (kWaitBound
// wall clock ticks of 10 ns, unless set otherwise) means the map kernel is
// not running beside it (a tool or a graph that runs the two streams'
// kernels one after the other): the walk gives up its buffer.  The walk
// after the map kernel waits up to the same bound for the buffer's done
// word to leave kOpen, and walks the buffer where it was given up or where
// it claims it; it never waits for a map: every map is out by then.
constexpr int kAhead = 128;
constexpr int kNap = 16;
constexpr uint64_t kWaitBound = 100000;  // 1 ms

// One workgroup per buffer: the buffer's running sum into out[buf].
// live: beside fsum_tile_maps, on the second stream.  Otherwise after it,
// on the caller's stream: the buffers the walk beside gave up or did not
// finish in time (all of them where done is null).
__global__ __launch_bounds__(kThreads) void fsum_walk(const float *terms, int64_t nterms, int ntiles,
                                                      const Rec *recs, const uint32_t *buffer_bad, uint32_t *done,
                                                      float *out, int live, uint64_t wait_bound)
{
    __shared__ uint32_t lds[kPad];
    const int buf = blockIdx.x;
    if (!live && done) {
        __shared__ uint32_t shared_state;
        if (threadIdx.x == 0) {
            const uint64_t start = wall_clock64();
            uint32_t state = observe(&done[buf]);
            while (state == kOpen && wall_clock64() - start <= wait_bound) {
                __builtin_amdgcn_s_sleep(kNap);
                state = observe(&done[buf]);
            }
            if (state == kOpen)
                state = atomicCAS(&done[buf], kOpen, kClaimed);  // kOpen: claimed here
            shared_state = state;
        }
        __syncthreads();
        if (shared_state == kWalked)
            return;  // walked beside the map kernel
    }
    // beside the map kernel, this workgroup's few waves share each SIMD
    // with its: it issues first, since the buffer's result waits on it
    __builtin_amdgcn_s_setprio(3);
    __shared__ uint32_t shared_S, shared_how, shared_late;
    const float *tb = terms + static_cast<int64_t>(buf) * nterms;
    const Rec *rb = recs + static_cast<int64_t>(buf) * ntiles;
    const int me = static_cast<int>(threadIdx.x);
    uint32_t S = 0;  // +0, the accumulator's start (and the sum of no terms)
    if (ntiles > 0 && buffer_bad[buf])
        S = kNaN;
    int t0 = 0;
    bool patient = live != 0;  // waits allowed (beside the map kernel, within the bound)
    bool gave_up = false;  // beside it: a wait reached the bound
    while (t0 < ntiles && S != kInf && S != kNaN) {
        // the window's records, read once: this thread's tiles are
        // t0 + me*kPerThread + c (a tile past the buffer's last reads the
        // last one's record and drops it)
        uint64_t w0[kPerThread], w1[kPerThread];
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const int tile = t0 + me * kPerThread + c;
            const Rec &r = rb[tile < ntiles ? tile : ntiles - 1];
            w0[c] = observe(&r.w0);
            w1[c] = observe(&r.w1);
        }
        const int wend = ntiles - t0 < kWindow ? ntiles : t0 + kWindow;
        int lo = t0;          // the window's tiles before lo are added
        int wait_at = -1;     // a tile whose map is not out yet: wait, then read again from there
        while (lo < wend && S != kInf) {
            int uexp;
            uint32_t m0;
            split(S, uexp, m0);
            Map x[kPerThread];
            int count[kPerThread];
            uint32_t late = 0;  // tiles whose map is not out yet
            Map mine = identity_map();
#pragma unroll
            for (int c = 0; c < kPerThread; ++c) {
                const int tile = t0 + me * kPerThread + c;
                const bool in = tile >= lo && tile < wend;
                const uint64_t a = w0[c];
                const bool ready = (a & kReady) != 0;
                const int cnt = static_cast<int>((a >> 60) & 3u);
                const int e0 = static_cast<int>((a >> 52) & 0xffu) - 149;
                // no map for S's binade: the tile stops the scan and is
                // added from its terms
                Map y = leaving_map();
                bool wait = !ready;
                if (ready) {
                    if (cnt >= 1 && uexp == e0) {
                        y = unpack_map(a);
                    } else if (cnt == 2 && uexp == e0 + 1) {
                        if (w1[c] & kReady)
                            y = unpack_map(w1[c]);
                        else
                            wait = true;
                    }
                }
                wait = wait && patient;
                late |= (in && wait) ? (1u << c) : 0u;
                count[c] = in ? (ready ? cnt : 1) : -1;  // -1: not in this pass
                x[c] = in ? y : identity_map();
                mine = compose(mine, x[c]);
            }
            Map before;
            (void)scan_maps(mine, before);
            // walk this thread's tiles from m at its first one
            uint32_t m = apply(before, m0);
            int local = kPerThread;  // this thread's first tile that stops (none)
            uint32_t after = 0;
            if (m < kTop) {
#pragma unroll
                for (int c = 0; c < kPerThread; ++c) {
                    if (local == kPerThread && count[c] >= 0) {
                        const uint32_t a = apply(x[c], m);
                        if (a >= kTop) {
                            local = c;
                            after = a;
                        } else {
                            m = a;
                        }
                    }
                }
            }
            const int stop = first_set(local < kPerThread);
            if (stop == kThreads) {
                // no tile of the pass stops: S after the window's last tile
                if (me == (wend - 1 - t0) / kPerThread)
                    shared_S = join(uexp, m);
                __syncthreads();
                S = shared_S;
                __syncthreads();
                lo = wend;
                break;
            }
            // S before the stopping tile; that tile has no map out yet (wait
            // for it), reaches the binade's top exactly (applied whole), or
            // has no map for S's binade or leaves it (walked run by run, or
            // term by term where the plan found it may cross more than two
            // binades)
            if (me == stop) {
                shared_S = join(uexp, m);
                shared_how = static_cast<uint32_t>(local) | (after == kTop ? 0x100u : 0u) |
                             (count[local] == 0 ? 0x200u : 0u) | (((late >> local) & 1u) ? 0x400u : 0u);
            }
            __syncthreads();
            S = shared_S;
            const uint32_t how = shared_how;
            __syncthreads();
            const int tile = t0 + stop * kPerThread + static_cast<int>(how & 0xffu);
            lo = tile;
            if (how & 0x400u) {
                wait_at = tile;
                break;
            }
            if (how & 0x100u) {
                S = join(uexp, kTop);
            } else {
                const int64_t first = static_cast<int64_t>(tile) * kTile;
                load_tile(tb + first, nterms - first, lds);
                S = walk_tile(lds, S, (how & 0x200u) != 0);
            }
            lo = tile + 1;
        }
        if (wait_at >= 0) {
            // one lane waits, within the bound, until the tile's maps are
            // out and the record kAhead tiles on (or the last) is written;
            // the workgroup then reads the window again
            if (me == 0) {
                const int probe = wait_at + kAhead < ntiles ? wait_at + kAhead : ntiles - 1;
                auto maps_out = [&]() {
                    const uint64_t a = observe(&rb[wait_at].w0);
                    if (!(a & kReady))
                        return false;
                    if (((a >> 60) & 3u) == 2u && !(observe(&rb[wait_at].w1) & kReady))
                        return false;
                    return (observe(&rb[probe].w0) & kReady) != 0;
                };
                const uint64_t start = wall_clock64();
                bool out_yet = maps_out();
                while (!out_yet && wall_clock64() - start <= wait_bound) {
                    __builtin_amdgcn_s_sleep(kNap);
                    out_yet = maps_out();
                }
                shared_late = out_yet ? 0u : 1u;
            }
            __syncthreads();
            const bool bound = shared_late != 0;
            __syncthreads();
            if (bound) {
                if (live) {
                    gave_up = true;
                    break;
                }
                patient = false;  // from here on, tiles without maps are added from their terms
            }
        }
        t0 = lo;
    }
    if (threadIdx.x == 0) {
        if (!live)
            out[buf] = __uint_as_float(S);
        else if (atomicCAS(&done[buf], kOpen, gave_up ? kGivenUp : kWalked) == kOpen && !gave_up)
            out[buf] = __uint_as_float(S);  // not claimed by the walk after the map kernel
    }
}

}  // namespace

FloatSumLayout float_sum_layout(int64_t nterms, int nbuffers)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    FloatSumLayout l{};
    l.ntiles = static_cast<int>((nterms + kTile - 1) / kTile);
    const size_t cells = static_cast<size_t>(l.ntiles) * nbuffers;
    l.totals = 0;
    l.bad = up(l.totals + cells * sizeof(double));
    l.recs = up(l.bad + cells * sizeof(uint32_t));
    l.buffer_bad = up(l.recs + cells * sizeof(Rec));
    l.done = up(l.buffer_bad + static_cast<size_t>(nbuffers) * sizeof(uint32_t));
    l.bytes = up(l.done + static_cast<size_t>(nbuffers) * sizeof(uint32_t));
    return l;
}

hipError_t launch_float_sums(const float *terms, int64_t nterms, int nbuffers, float *out, void *workspace,
                             hipStream_t stream, const SideStream *side)
{
    const FloatSumLayout l = float_sum_layout(nterms, nbuffers);
    char *ws = static_cast<char *>(workspace);
    double *totals = reinterpret_cast<double *>(ws + l.totals);
    uint32_t *bad = reinterpret_cast<uint32_t *>(ws + l.bad);
    Rec *recs = reinterpret_cast<Rec *>(ws + l.recs);
    uint32_t *buffer_bad = reinterpret_cast<uint32_t *>(ws + l.buffer_bad);
    uint32_t *done = reinterpret_cast<uint32_t *>(ws + l.done);
    // the map grid's workgroups are counted in 32 bits
    // (terms resident in device memory keep the tile count far below 2^32)
    const int64_t cells = static_cast<int64_t>(l.ntiles) * nbuffers;
    if (cells >= (int64_t{1} << 32))
        return hipErrorInvalidValue;
    // the bound of one wait of the walk (wall clock ticks of 10 ns); 0 makes
    // the walk beside the map kernel give every buffer to the walk after it
    uint64_t bound = kWaitBound;
    if (const char *e = std::getenv("VQX_FLOAT_SUM_WAIT_TICKS")) {
        char *end = nullptr;
        const unsigned long long v = std::strtoull(e, &end, 10);
        if (end != e && *end == '\0' && v <= 100000000ull)  // at most one second
            bound = v;
    }
    if (l.ntiles > 0) {
        const dim3 grid(static_cast<unsigned>(l.ntiles), static_cast<unsigned>(nbuffers));
        fsum_tile_totals<<<grid, kThreads, 0, stream>>>(terms, nterms, l.ntiles, totals, bad);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        // the fork: the walk beside the maps starts once the plan is out.
        // The event is the plan kernel's own completion, which puts no
        // marker between it and the map kernel -- except while the stream
        // is captured into a graph, which follows recorded events only.
        bool capturing = false;
        if (side) {
            hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
            err = hipStreamIsCapturing(stream, &st);
            if (err != hipSuccess)
                return err;
            capturing = st != hipStreamCaptureStatusNone;
        }
        {
            int nt = l.ntiles;
            void *args[] = {&totals, &bad, &nt, &recs, &buffer_bad, &done};
            err = hipExtLaunchKernel(reinterpret_cast<const void *>(&fsum_plan), dim3(static_cast<unsigned>(nbuffers)),
                                     dim3(kThreads), args, 0, stream, nullptr,
                                     side && !capturing ? side->fork : nullptr, 0);
            if (err == hipSuccess && side && capturing)
                err = hipEventRecord(side->fork, stream);
            if (err != hipSuccess)
                return err;
        }
        fsum_tile_maps<<<dim3(static_cast<unsigned>(cells)), kThreads, 0, stream>>>(terms, nterms, l.ntiles,
                                                                                    nbuffers, recs);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        // enqueued after the map kernel, so that where the two streams
        // share one hardware queue the walk simply follows it
        if (side) {
            err = hipStreamWaitEvent(side->stream, side->fork, 0);
            if (err != hipSuccess)
                return err;
            int nt = l.ntiles, live = 1;
            const Rec *rc = recs;
            const uint32_t *bb = buffer_bad;
            void *args[] = {const_cast<float **>(&terms), &nterms, &nt, &rc, &bb, &done, &out, &live, &bound};
            err = hipExtLaunchKernel(reinterpret_cast<const void *>(&fsum_walk), dim3(static_cast<unsigned>(nbuffers)),
                                     dim3(kThreads), args, 0, side->stream, nullptr,
                                     capturing ? nullptr : side->join, 0);
            if (err == hipSuccess && capturing)
                err = hipEventRecord(side->join, side->stream);
            if (err != hipSuccess)
                return err;
        }
    }
    // after the map kernel on the caller's stream: the buffers the walk
    // beside it gave up or did not finish within the bound, or all (each
    // writes +0 where there are no tiles); then the join, which also keeps
    // the stream from passing the call before the walk beside has ended
    const bool beside = l.ntiles > 0 && side;
    fsum_walk<<<dim3(static_cast<unsigned>(nbuffers)), kThreads, 0, stream>>>(
        terms, nterms, l.ntiles, recs, buffer_bad, beside ? done : nullptr, out, 0, bound);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess && beside)
        err = hipStreamWaitEvent(stream, side->join, 0);
    return err;
}

}  // namespace vqx
