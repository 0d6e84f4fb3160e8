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
// below 2^57) one CPU step is S <- RN53(S + t): the exact sum rounded to 53
// significant bits, ties to even.  While S stays inside one binade
// [2^e, 2^(e+1)) with e >= 53, S = m * u with u = 2^k, k = e - 52.  Write
// t + u/2 = h * u + rr.  Then adding t moves m to m + h, except on a tie
// (rr = 0, i.e. t's remainder is exactly u/2), where it moves to m + h - 1
// if m + h is odd and to m + h if it is even; after a tie m is always even.
// So a run of terms acts on S, inside a binade, as a two-state machine on
// the parity of m: the increase of m is the run's sum of h less the ties
// rounded down, both of which, and the parity after the run, depend only
// on the parity before it.  Such maps compose in order.
//
//  1. stage 1 (plane_stats.hip) gives each chunk's exact totals;
//  2. a prefix scan per frame (the exact running sum at each chunk start,
//     which predicts the binade the CPU's sum is in there) writes every
//     sum in which no add of the CPU's can round (those below 2^53, and
//     those whose terms share enough trailing zero bits to stay exact past
//     it), maps the chunks past 2^53 inside which nothing can round, and
//     queues the other chunks past 2^53;
//  3. in the same launch (cpu_order_maps: a group of workgroups per frame,
//     each running the frame's scan for itself), every slab of 256 vectors
//     of a queued chunk gets its exact total and maps in the predicted
//     binade (and the next one where the chunk may cross into it).  Most slabs need no
//     ordered work: if every term is a multiple of the binade's unit nothing
//     rounds, and without ties the map follows from two plain sums; only
//     slabs with ties chain their terms and compose the lanes' maps in
//     order.  The frame's waves share out its queued slabs, each wave
//     reading its next slab while mapping the current one;
//  4. cpu_order_walk, one workgroup per frame and sum past 2^53: its waves
//     first write a compact record per chunk (its map, its own or composed
//     from its slab maps, and its total) and per block of 64 chunks (their
//     composed map and total); then wave 0 walks the frame in order with
//     the running value S: a block that stays below 2^53 adds exactly; a
//     block whose map is for S's binade is applied if S stays in the binade;
//     otherwise chunk by chunk, then slab by slab, then 64 groups of 32
//     consecutive terms with maps made on the spot for S's binade and the
//     next, and within the group where S crosses, term by term.  Every step
//     is checked against S itself, so a prediction only decides how fast
//     the walk is, never what it returns.
//
// One-byte samples (8 bits per component) never get there: their squares
// are below 2^16 and a frame has at most 2^25 samples, so every sum stays
// below 2^41 and step 2 already gives the CPU's values.

#include <atomic>
#include <type_traits>

#include "plane_stats.h"
#include "terms.h"

namespace vqx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
static_assert(kThreads == kChunkThreads, "dispatch-size check");
constexpr uint64_t kTwo53 = 1ull << 53;
constexpr int kTerms = 8;  // terms of one 16-byte vector of two-byte samples

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

// ------------------------------------------------------------- wave helpers
// lane i receives lane i + s of its row of 16 (row_shl:s); a lane whose
// source lies outside the row receives 0
template <int S>
__device__ __forceinline__ uint32_t from_next(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x100 + S, 0xf, 0xf, false));
}

template <int S>
__device__ __forceinline__ uint64_t from_next64(uint64_t v)
{
    return static_cast<uint64_t>(from_next<S>(static_cast<uint32_t>(v))) |
           (static_cast<uint64_t>(from_next<S>(static_cast<uint32_t>(v >> 32))) << 32);
}

// lane l's value (l wave-uniform): the result is wave-uniform
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l)
{
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}

__device__ __forceinline__ uint64_t lane_value64(uint64_t v, int l)
{
    return static_cast<uint64_t>(lane_value(static_cast<uint32_t>(v), l)) |
           (static_cast<uint64_t>(lane_value(static_cast<uint32_t>(v >> 32), l)) << 32);
}

__device__ __forceinline__ uint32_t wave_total32(uint32_t v)
{
    v += from_next<1>(v);
    v += from_next<2>(v);
    v += from_next<4>(v);
    v += from_next<8>(v);
    return lane_value(v, 0) + lane_value(v, 16) + lane_value(v, 32) + lane_value(v, 48);
}

__device__ __forceinline__ uint64_t wave_total64(uint64_t v)
{
    v += from_next64<1>(v);
    v += from_next64<2>(v);
    v += from_next64<4>(v);
    v += from_next64<8>(v);
    return lane_value64(v, 0) + lane_value64(v, 16) + lane_value64(v, 32) + lane_value64(v, 48);
}

// ---------------------------------------------------------- run maps (u32)
// The map of a run of terms inside binade 2^(k+52), for both parities s of
// m before the run: C holds, per s, the number of ties rounded down (low 16
// bits s = 0, high 16 bits s = 1), P the parity of m after the run (bit 0
// s = 0, bit 16 s = 1).  The run's sum of h is kept apart: it is the same
// for both parities, and is recovered from the run's exact total and the
// sum of its rr.  Counts stay below 2^16 for runs of at most 8192 terms.
struct RunMap {
    uint32_t C = 0;
    uint32_t P = 0x10000u;
};

// Appends a term given as t2 = t + 2^(k-1) (terms are below 2^32 - 2^17,
// so t2 does not wrap).
__device__ __forceinline__ void run_step(RunMap &m, uint32_t t2, int k)
{
    const uint32_t hb = __builtin_amdgcn_ubfe(t2, static_cast<uint32_t>(k), 1u);
    const uint32_t x = m.P ^ (hb | (hb << 16));  // parity of m + h, per s
    const bool tie = (t2 & ((1u << k) - 1)) == 0;
    m.C += tie ? x : 0u;  // a tie rounds down from m + h exactly when m + h is odd
    m.P = tie ? 0u : x;
}

// Appends term t, also adding its rr to rr_sum.
__device__ __forceinline__ void run_add(RunMap &m, uint32_t &rr_sum, uint32_t t, int k)
{
    const uint32_t t2 = t + (1u << (k - 1));
    rr_sum += t2 & ((1u << k) - 1);
    run_step(m, t2, k);
}

__device__ __forceinline__ uint32_t swap_halves(uint32_t x) { return __builtin_amdgcn_alignbit(x, x, 16); }

// a then b
__device__ __forceinline__ RunMap run_then(const RunMap &a, const RunMap &b)
{
    // per half: where b is entered from the other parity than the half's own
    const uint32_t other = (a.P * 0xffffu) ^ 0xffff0000u;
    RunMap c;
    c.C = a.C + ((swap_halves(b.C) & other) | (b.C & ~other));
    c.P = (swap_halves(b.P) & other) | (b.P & ~other);
    return c;
}

template <int S>
__device__ __forceinline__ RunMap run_from_next(const RunMap &m)
{
    RunMap o;
    o.C = from_next<S>(m.C);
    o.P = from_next<S>(m.P);
    return o;
}

// The wave's lane maps composed in lane order (lane 0's first); uniform.
__device__ __forceinline__ RunMap wave_run(RunMap m)
{
    m = run_then(m, run_from_next<1>(m));
    m = run_then(m, run_from_next<2>(m));
    m = run_then(m, run_from_next<4>(m));
    m = run_then(m, run_from_next<8>(m));
    RunMap w;
    w.C = lane_value(m.C, 0);
    w.P = lane_value(m.P, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row) {
        RunMap r;
        r.C = lane_value(m.C, 16 * row);
        r.P = lane_value(m.P, 16 * row);
        w = run_then(w, r);
    }
    return w;
}

// ------------------------------------------------------------ wave scans
// Inclusive scans in lane order: row_shr steps within each row of 16, then
// row_bcast:15 (rows 1 and 3) and row_bcast:31 (rows 2 and 3) carry the
// rows below in.  A lane without a source takes `identity`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t from_below(uint32_t identity, uint32_t v)
{
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(v), CTRL, ROWS, 0xf, false));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t scan_step64(uint64_t v)
{
    return v + (static_cast<uint64_t>(from_below<CTRL, ROWS>(0u, static_cast<uint32_t>(v))) |
                (static_cast<uint64_t>(from_below<CTRL, ROWS>(0u, static_cast<uint32_t>(v >> 32))) << 32));
}

__device__ __forceinline__ uint64_t wave_scan64(uint64_t v)
{
    v = scan_step64<0x111, 0xf>(v);
    v = scan_step64<0x112, 0xf>(v);
    v = scan_step64<0x114, 0xf>(v);
    v = scan_step64<0x118, 0xf>(v);
    v = scan_step64<0x142, 0xa>(v);
    return scan_step64<0x143, 0xc>(v);
}

// ---------------------------------------------------------- maps (64-bit)
// The same two-state map with its increases of m written out: from parity
// s, m grows by dm_s and ends with parity p_s.
struct Map2 {
    uint64_t dm0 = 0, dm1 = 0;
    uint32_t p0 = 0, p1 = 1;
};

// A run of n terms with exact total `total` and sum of rr `rr_sum` in
// binade 2^(k+52): its sum of h is (total + n * 2^(k-1) - rr_sum) / 2^k.
__device__ __forceinline__ Map2 run_map(const RunMap &m, uint64_t total, uint64_t n, uint64_t rr_sum, int k)
{
    const uint64_t h = (total + (n << (k - 1)) - rr_sum) >> k;
    Map2 r;
    r.dm0 = h - (m.C & 0xffffu);
    r.dm1 = h - (m.C >> 16);
    r.p0 = m.P & 1u;
    r.p1 = m.P >> 16;
    return r;
}

// x if bit 0 of s is clear, y if it is set.  (Written with a mask: a plain
// ?: between two fields of one struct can become an indexed load from a
// stack copy of it.)
__device__ __forceinline__ uint64_t pick(uint64_t s, uint64_t x, uint64_t y)
{
    const uint64_t mask = 0 - (s & 1u);
    return (x & ~mask) | (y & mask);
}

// The map of a run without ties whose sum of h is h: m grows by h from
// either parity, and the parity flips with h's.
__device__ __forceinline__ Map2 untied_map(uint64_t h)
{
    Map2 m;
    m.dm0 = m.dm1 = h;
    m.p0 = static_cast<uint32_t>(h) & 1u;
    m.p1 = m.p0 ^ 1u;
    return m;
}

// a then b
__device__ __forceinline__ Map2 map_then(const Map2 &a, const Map2 &b)
{
    Map2 c;
    c.dm0 = a.dm0 + pick(a.p0, b.dm0, b.dm1);
    c.p0 = static_cast<uint32_t>(pick(a.p0, b.p0, b.p1));
    c.dm1 = a.dm1 + pick(a.p1, b.dm0, b.dm1);
    c.p1 = static_cast<uint32_t>(pick(a.p1, b.p0, b.p1));
    return c;
}

template <int S>
__device__ __forceinline__ Map2 map_from_next(const Map2 &m)
{
    Map2 o;
    o.dm0 = from_next64<S>(m.dm0);
    o.dm1 = from_next64<S>(m.dm1);
    o.p0 = from_next<S>(m.p0);
    o.p1 = from_next<S>(m.p1);
    return o;
}

__device__ __forceinline__ Map2 map_lane(const Map2 &m, int l)
{
    Map2 o;
    o.dm0 = lane_value64(m.dm0, l);
    o.dm1 = lane_value64(m.dm1, l);
    o.p0 = lane_value(m.p0, l);
    o.p1 = lane_value(m.p1, l);
    return o;
}

// The wave's maps composed in lane order; uniform.
__device__ __forceinline__ Map2 wave_map(Map2 m)
{
    m = map_then(m, map_from_next<1>(m));
    m = map_then(m, map_from_next<2>(m));
    m = map_then(m, map_from_next<4>(m));
    m = map_then(m, map_from_next<8>(m));
    Map2 w = map_lane(m, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row)
        w = map_then(w, map_lane(m, 16 * row));
    return w;
}

// Applies map `m` (made for binade e) to S if S is in binade e and stays
// there; returns false otherwise (S unchanged).  m only grows, so if it
// ends inside the binade every step of the run stayed inside it.
__device__ __forceinline__ bool map_apply(uint64_t &S, const Map2 &m, int e)
{
    if (S < kTwo53 || binade(S) != e)
        return false;
    const int k = e - 52;
    const uint64_t mm = S >> k;
    const uint64_t m2 = mm + pick(mm, m.dm0, m.dm1);
    if (m2 >= kTwo53)
        return false;
    S = m2 << k;
    return true;
}

// Stored maps: {dm0, dm1, flags}; flags bit 0 valid, bits 8..15 the
// binade, bit 16 p0, bit 17 p1.
__device__ __forceinline__ uint64_t map_flags(const Map2 &m, int e)
{
    return 1u | (static_cast<uint64_t>(e) << 8) | (static_cast<uint64_t>(m.p0 & 1u) << 16) |
           (static_cast<uint64_t>(m.p1 & 1u) << 17);
}

__device__ __forceinline__ Map2 map_from(uint64_t dm0, uint64_t dm1, uint64_t flags)
{
    Map2 m;
    m.dm0 = dm0;
    m.dm1 = dm1;
    m.p0 = static_cast<uint32_t>((flags >> 16) & 1u);
    m.p1 = static_cast<uint32_t>((flags >> 17) & 1u);
    return m;
}

__device__ __forceinline__ int flags_binade(uint64_t flags) { return static_cast<int>((flags >> 8) & 0xffu); }

// ------------------------------------------------------------------ terms
// Term i (raster order) of square sum KK in one 16-byte vector of each plane.
template <int KK>
__device__ __forceinline__ uint32_t vector_term(const u32x4 &a, const u32x4 &b, int i)
{
    const uint32_t wa = a[i >> 1], wb = b[i >> 1];
    const uint32_t r = (i & 1) ? wa >> 16 : wa & 0xffffu;
    const uint32_t d = (i & 1) ? wb >> 16 : wb & 0xffffu;
    return square_term<2>(KK, r, d);
}

// Vector v of the planes square sum KK reads; a lane with !ok reads vector
// `safe` (one known to exist) instead, for the caller to drop (keep_if).
// Every lane loads, so no branch separates the loads from the waits for
// them and the next vectors can be in flight while these are used.
// kSh: the map is general (R and D the bases rounded down to 16 bytes;
// each vector cut from the blocks that hold it).
template <int KK, bool kSh>
__device__ __forceinline__ void load_vector(const u32x4 *R, const u32x4 *D, const VecMap &M, int64_t frame,
                                            int64_t v, bool ok, int64_t safe, u32x4 &a, u32x4 &b)
{
    const u32x4 zero = {0, 0, 0, 0};
    int64_t ar, ad;
    if constexpr (kSh)
        map_vec_bytes(M, frame, ok ? v : safe, ar, ad);
    else
        map_vec(M, frame, ok ? v : safe, ar, ad);
    if constexpr (KK != kSqDist)
        a = kSh ? load_vec16_at(R, ar) : __builtin_nontemporal_load(R + ar);
    else
        a = zero;
    if constexpr (KK != kSqRef)
        b = kSh ? load_vec16_at(D, ad) : __builtin_nontemporal_load(D + ad);
    else
        b = zero;
}

// Zeros a loaded vector that lies past the end (zero terms change neither
// a map nor a total).
template <int KK>
__device__ __forceinline__ void keep_if(bool ok, u32x4 &a, u32x4 &b)
{
    const u32x4 zero = {0, 0, 0, 0};
    if constexpr (KK != kSqDist)
        a = ok ? a : zero;
    if constexpr (KK != kSqRef)
        b = ok ? b : zero;
}

// ------------------------------------------------------------ 3. slab maps
// Entry of chunk wg, square kk (kEntry uint64): the maps {dm0, dm1, flags}
// of its kSlabs slabs in the predicted binade e, their maps in binade e + 1
// (made only where the chunk's exact range reaches 2^(e+1), i.e. where the
// CPU's sum probably changes binade inside it; flags 0 otherwise), the
// slabs' exact totals, and a chunk map (flags 0 unless kChunkOnly).  Only
// chunks past 2^53 get an entry; the walk uses no other (below 2^53 it adds
// chunk totals exactly).
constexpr int kSlabVectors = 256;
constexpr int kSlabs = kChunkVectors / kSlabVectors;
constexpr int kLaneVectors = kSlabVectors / 64;  // vectors of a slab per lane
constexpr int kSlabMapsA = 0;
constexpr int kSlabMapsB = kSlabMapsA + 3 * kSlabs;
constexpr int kSlabTotals = kSlabMapsB + 3 * kSlabs;
constexpr int kChunkMap = kSlabTotals + kSlabs;  // {dm0, dm1, flags}: see kChunkOnly
constexpr int kEntry = kChunkMap + 3;
// Set in the chunk map's flags of a chunk whose entry holds only that map:
// every term of the chunk's sum is a multiple of its predicted binade's unit
// (from stage 1's low bits), so nothing rounds inside the chunk, and no
// crossing is predicted in it.  Its slabs are not mapped.
constexpr uint64_t kChunkOnly = 1ull << 20;
// The chunk-map flags of a queued chunk: its slabs are mapped.  A chunk
// that ends below 2^53 (or holds no vector) has flags 0.
constexpr uint64_t kQueued = 1ull << 21;

// Queues of chunks to map, one per square sum, each of capacity
// nframes * chunks, frame f's items in its own segment [f * chunks,
// (f + 1) * chunks): an item is (frame * chunks + chunk) | e << 32 |
// dual << 40, e the binade predicted at the chunk's start, dual set where
// the chunk's exact range reaches 2^(e+1).

// ------------------------------------------------------------ 2. prefix scan
// One workgroup scans a frame; thread t takes chunks [t * per, (t + 1) * per).
//  * The exact sum of each square over the chunks before chunk c (chunk 0's
//    record also holds the frame's few samples outside whole vectors)
//    predicts the CPU's sum there; totals[f*3 + kk] = the frame's exact sum.
//  * It writes the frame's five exact sums (so the CPU-order form needs no
//    stage 2), and the CPU's values of the sums in which no add can round,
//    which are the exact sums: those that stay below 2^53 (the first
//    moments always do: below 2^25 * 2^16 = 2^41), and those whose terms are
//    all multiples of 2^j (the OR of the frame's low bits, j <= 4) and that
//    stay below 2^(53+j) -- every partial sum is then a multiple of 2^j
//    below 2^(53+j), which a double holds exactly (bright 16-bit content:
//    every float square of a sample above 46340 is a multiple of 2^8).
//    totals[f*3 + kk] is the frame's exact sum where the walk has to find
//    the CPU's value, else 0.
//  * With `maps` (two-byte samples), each chunk of such a sum whose exact
//    range ends past 2^53 gets its case: a chunk that starts past 2^53, is
//    not predicted to change binade and whose terms are all multiples of
//    2^k (stage 1's low bits; k <= 4 since sums stay below 2^57) gets its
//    map from its total alone, since nothing inside it rounds; every other
//    such chunk goes on its sum's queue to have its slabs mapped.
__device__ __forceinline__ uint64_t wave_inclusive_then_total(uint64_t v, uint64_t *lds_totals, uint64_t &total)
{
    // inclusive scan inside the wave, then the totals of the waves below
    const int wave = threadIdx.x / 64;
    const uint64_t inc = wave_scan64(v);
    if ((threadIdx.x & 63) == 63)
        lds_totals[wave] = inc;
    __syncthreads();
    uint64_t below = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const uint64_t x = lds_totals[w];
        below += w < wave ? x : 0;
        total += x;
    }
    __syncthreads();
    return inc + below;
}

// wave_inclusive_then_total for N values at once, with one barrier between
// the waves' totals and their use (each value has its own LDS row).
template <int N>
__device__ __forceinline__ void wave_inclusive_then_total_n(const uint64_t (&v)[N], uint64_t (*lds_totals)[kThreads / 64],
                                                            uint64_t (&incl)[N], uint64_t (&total)[N])
{
    const int wave = threadIdx.x / 64;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        incl[j] = wave_scan64(v[j]);
        if ((threadIdx.x & 63) == 63)
            lds_totals[j][wave] = incl[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        uint64_t below = 0;
        total[j] = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            const uint64_t x = lds_totals[j][w];
            below += w < wave ? x : 0;
            total[j] += x;
        }
        incl[j] += below;
    }
}

struct ChunkCase {
    bool queued, chunk_only;
    int e;
    bool dual;
};

__device__ __forceinline__ ChunkCase chunk_case(uint64_t p, uint64_t r, uint32_t low, bool exists)
{
    ChunkCase x;
    const bool want = exists && p + r >= kTwo53;
    x.e = binade(p > kTwo53 ? p : kTwo53);
    x.dual = x.e < 56 && p + r >= (1ull << (x.e + 1));
    const uint32_t unit_bits = (1u << (x.e - 52)) - 1;
    x.chunk_only = want && !x.dual && p >= kTwo53 && (low & unit_bits) == 0;
    x.queued = want && !x.chunk_only;
    return x;
}

// Chunks of one frame at most: 2^25 two-byte samples hold at most 2^22
// whole vectors, 2048 chunks.
constexpr int kMaxFrameChunks = 2048;

// Records staged per round of frame_prefix: 256 records of 64 bytes, the
// maps kernel's transpose buffers (idle during the scan).
constexpr int kStageRecords = 256;

// The LDS of frame_prefix.
struct PrefixLds {
    uint64_t scan[kSums + 1][kThreads / 64];
    uint32_t nq[kSquares];  // the frame's queue length, per square sum
    uint32_t frame_low;     // the OR of the frame's low bits
};

// The prefix scan of frame f, by one workgroup (all threads call it).  Each
// workgroup that maps the frame's slabs runs it for itself (a frame's
// records are a few tens of KB, read from L2 after the first); `writer`
// (one workgroup per frame) also writes the sums, the totals and the chunk
// maps.  Every such workgroup writes the frame's queue items (the same
// values), into the frame's own segment of each queue (capacity `chunks`,
// in chunk order), and leaves their numbers in L.nq.
__device__ __forceinline__ void frame_prefix(PrefixLds &L, u32x4 *stage, int64_t f, int nframes, const uint64_t *rec,
                                             int64_t pixels, int chunks, bool writer, uint64_t *totals,
                                             uint64_t *out_noise, uint64_t *out_moments, uint64_t *out_cpu_noise,
                                             uint64_t *out_cpu_moments, uint64_t *maps, uint64_t *queue)
{
    constexpr int V = 8;
    const int t = threadIdx.x;
    if (t == 0)
        L.frame_low = 0;
    __syncthreads();
    const int per = (chunks + kThreads - 1) / kThreads;
    const int c0 = t * per < chunks ? t * per : chunks;
    const int c1 = c0 + per < chunks ? c0 + per : chunks;
    const uint64_t *frec = rec + f * chunks * kRecordStride;
    // the thread's sums of each record field, then their exclusive prefixes
    // over the frame and the frame's totals.  The thread's first kKept
    // chunks (all of them up to kKept * kThreads chunks a frame) keep what
    // the passes below need in registers, read once.
    constexpr int kKept = 2;
    uint64_t local[kSums], run[kSums], total[kSums];
    uint64_t kept_t[kKept][kSquares];
    uint32_t kept_low[kKept];
#pragma unroll
    for (int j = 0; j < kSums; ++j)
        local[j] = 0;
    uint32_t low_or = 0;
    {
        static_assert(kLowBits == kSums, "the low bits follow the sums in a record");
        static_assert(kRecordStride == 8, "a record is four 16-byte vectors");
        uint64_t v[kKept][kSums + 1];
        if (per <= kKept) {
            // the frame's records pass through `stage` (kStageRecords at a
            // time) read as consecutive 16-byte vectors, 1 KB per load
            // instruction, rather than one record per lane (64 lines per
            // instruction); each thread then takes its chunks' six words
            const u32x4 *src = reinterpret_cast<const u32x4 *>(frec);
#pragma unroll
            for (int i = 0; i < kKept; ++i)
#pragma unroll
                for (int j = 0; j <= kSums; ++j)
                    v[i][j] = 0;
            for (int r0 = 0; r0 < chunks; r0 += kStageRecords) {
                const int n = chunks - r0 < kStageRecords ? chunks - r0 : kStageRecords;
                u32x4 w[kStageRecords * 4 / kThreads];
#pragma unroll
                for (int k = 0; k < kStageRecords * 4 / kThreads; ++k) {
                    const int idx = t + k * kThreads;  // vector idx of the round's records
                    w[k] = src[static_cast<int64_t>(r0) * 4 + (idx < 4 * n ? idx : 0)];
                }
#pragma unroll
                for (int k = 0; k < kStageRecords * 4 / kThreads; ++k)
                    stage[t + k * kThreads] = w[k];
                __syncthreads();
#pragma unroll
                for (int i = 0; i < kKept; ++i) {
                    const int c = c0 + i;
                    if (c < c1 && c >= r0 && c < r0 + n) {
                        const u32x4 *x = stage + (c - r0) * 4;
#pragma unroll
                        for (int q = 0; q < 3; ++q) {
                            const u32x4 y = x[q];
                            v[i][2 * q] = y.x | (static_cast<uint64_t>(y.y) << 32);
                            v[i][2 * q + 1] = y.z | (static_cast<uint64_t>(y.w) << 32);
                        }
                    }
                }
                __syncthreads();  // before the next round overwrites the stage
            }
        } else {
            // all loads in flight together (a chunk the thread lacks reads
            // chunk 0 and drops it)
#pragma unroll
            for (int i = 0; i < kKept; ++i) {
                const int c = c0 + i < c1 ? c0 + i : 0;
#pragma unroll
                for (int j = 0; j <= kSums; ++j)
                    v[i][j] = frec[c * kRecordStride + j];  // kLowBits follows the sums
            }
        }
#pragma unroll
        for (int i = 0; i < kKept; ++i) {
            const bool mine = c0 + i < c1;
#pragma unroll
            for (int j = 0; j < kSums; ++j)
                local[j] += mine ? v[i][j] : 0;
            kept_low[i] = mine ? static_cast<uint32_t>(v[i][kSums]) : 0u;
            low_or |= kept_low[i];
#pragma unroll
            for (int kk = 0; kk < kSquares; ++kk)
                kept_t[i][kk] = mine ? v[i][record_field(kk)] : 0;
        }
    }
    for (int c = c0 + kKept; c < c1; ++c) {
#pragma unroll
        for (int j = 0; j < kSums; ++j)
            local[j] += frec[c * kRecordStride + j];
        low_or |= static_cast<uint32_t>(frec[c * kRecordStride + kLowBits]);
    }
    if (maps) {
        // the wave's OR first: an LDS atomic from every lane on one word
        // serializes (~3 us a workgroup), one per wave does not
#pragma unroll
        for (int d = 1; d < 64; d <<= 1)
            low_or |= __shfl_xor(low_or, d, 64);
        if ((t & 63) == 0 && low_or)
            atomicOr(&L.frame_low, low_or);  // complete after the scan's barrier
    }
    wave_inclusive_then_total_n<kSums>(local, L.scan, run, total);
    // the square sums whose every add is exact (one-byte samples: all)
    bool exact[kSquares];
#pragma unroll
    for (int kk = 0; kk < kSquares; ++kk) {
        const uint32_t nib = (L.frame_low >> (4 * kk)) & 15u;
        const int j = nib ? __builtin_ctz(nib) : 4;
        const uint64_t T = total[record_field(kk)];
        exact[kk] = !maps || T < kTwo53 || T < (kTwo53 << j);
    }
#pragma unroll
    for (int j = 0; j < kSums; ++j)
        run[j] -= local[j];
    if (writer && t == 0) {
        // the exact sums (stage 2's results), then the CPU's where they are
        // the exact ones
        out_noise[f] = total[kNoise];
        out_moments[4 * f + 0] = total[kRef1];
        out_moments[4 * f + 1] = total[kDist1];
        out_moments[4 * f + 2] = total[kRef2];
        out_moments[4 * f + 3] = total[kDist2];
#pragma unroll
        for (int kk = 0; kk < kSquares; ++kk)
            totals[f * kSquares + kk] = exact[kk] ? 0 : total[record_field(kk)];
        // otherwise the walk writes it
        if (exact[kSqNoise])
            out_cpu_noise[f] = total[kNoise];
        out_cpu_moments[4 * f + 0] = total[kRef1];
        out_cpu_moments[4 * f + 1] = total[kDist1];
        if (exact[kSqRef])
            out_cpu_moments[4 * f + 2] = total[kRef2];
        if (exact[kSqDist])
            out_cpu_moments[4 * f + 3] = total[kDist2];
    }
    if (t < kSquares)
        L.nq[t] = 0;
    const int64_t e0 = f * pixels;
    const int64_t nvec = (e0 + pixels) / V - (e0 + V - 1) / V;  // the frame's whole vectors
    // one-byte samples (every sum stays below 2^53), or no sum of the frame
    // that the walk takes: no chunk to map or queue
    if (!maps || (exact[kSqNoise] && exact[kSqRef] && exact[kSqDist])) {
        __syncthreads();
        return;
    }
    // f(c, T, low bits) for the thread's chunks of square sum kk, in order:
    // the kept ones from registers (each at a fixed index), then the rest
    auto each_chunk = [&](auto kkc, auto f) {
        constexpr int kk = decltype(kkc)::value;
#pragma unroll
        for (int i = 0; i < kKept; ++i)
            if (c0 + i < c1)
                f(c0 + i, kept_t[i][kk], kept_low[i]);
        for (int c = c0 + kKept; c < c1; ++c)
            f(c, frec[c * kRecordStride + record_field(kk)], static_cast<uint32_t>(frec[c * kRecordStride + kLowBits]));
    };
    // each square sum in turn, with its index known at compile time
    auto each_square = [&](auto body) {
        body(std::integral_constant<int, 0>{});
        body(std::integral_constant<int, 1>{});
        body(std::integral_constant<int, 2>{});
    };
    static_assert(kSquares == 3, "three square sums");
    // pass 1: chunk maps, and how many chunks the thread queues
    uint64_t nq = 0;  // 21 bits per square sum
    each_square([&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        if (exact[kk])
            return;
        uint64_t p = run[record_field(kk)];
        each_chunk(kkc, [&](int c, uint64_t T, uint32_t lows) {
            const uint32_t low = (lows >> (4 * kk)) & 15u;
            const ChunkCase x = chunk_case(p, T, low, static_cast<int64_t>(c) * kChunkVectors < nvec);
            uint64_t *entry = maps + ((f * chunks + c) * kSquares + kk) * kEntry;
            if (x.chunk_only) {
                if (writer) {
                    const Map2 m = untied_map(T >> (x.e - 52));
                    entry[kChunkMap + 0] = m.dm0;
                    entry[kChunkMap + 1] = m.dm1;
                    entry[kChunkMap + 2] = map_flags(m, x.e) | kChunkOnly;
                }
            } else {
                if (writer)
                    entry[kChunkMap + 2] = x.queued ? kQueued : 0;
                nq += x.queued ? 1ull << (21 * kk) : 0;
            }
            p += T;
        });
    });
    // each thread's first slot in the frame's segments, and their lengths
    uint64_t nq_total;
    const uint64_t at = wave_inclusive_then_total(nq, L.scan[kSums], nq_total) - nq;
    if (t < kSquares)
        L.nq[t] = static_cast<uint32_t>(nq_total >> (21 * t)) & 0x1fffffu;
    // pass 2: the queue items, in chunk order within the frame
    const int64_t cap = static_cast<int64_t>(nframes) * chunks;
    each_square([&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        if (exact[kk])
            return;
        uint64_t p = run[record_field(kk)];
        int64_t slot = f * chunks + ((at >> (21 * kk)) & 0x1fffffu);
        each_chunk(kkc, [&](int c, uint64_t T, uint32_t lows) {
            const uint32_t low = (lows >> (4 * kk)) & 15u;
            const ChunkCase x = chunk_case(p, T, low, static_cast<int64_t>(c) * kChunkVectors < nvec);
            if (x.queued)
                queue[kk * cap + slot++] = static_cast<uint64_t>(f * chunks + c) |
                                           (static_cast<uint64_t>(x.e) << 32) |
                                           (static_cast<uint64_t>(x.dual) << 40);
            p += T;
        });
    });
    __syncthreads();  // the segments and their lengths, for the workgroup
}

// The planes' vectors of one slab.  As loaded, lane l holds vectors l,
// 64 + l, 128 + l and 192 + l (each load instruction reads 1 KB in one
// piece), and bit j of ok is set where vector 64j + l lies inside the
// chunk; `consecutive` then gives lane l vectors 4l .. 4l + 3.
struct ItemData {
    u32x4 a[kLaneVectors], b[kLaneVectors];
    uint32_t ok;
    int all_ok;  // every vector of the slab inside the chunk (wave-uniform)
};

template <int KK, bool kSh>
__device__ __forceinline__ void load_item(ItemData &x, const u32x4 *R, const u32x4 *D, const VecMap &M,
                                          int64_t frame, int64_t cb, int64_t sb, int64_t ce)
{
    const int lane = threadIdx.x & 63;
    x.ok = 0;
    x.all_ok = sb + kSlabVectors <= ce;
#pragma unroll
    for (int j = 0; j < kLaneVectors; ++j) {
        const int64_t v = sb + 64 * j + lane;
        load_vector<KK, kSh>(R, D, M, frame, v, v < ce, cb, x.a[j], x.b[j]);
        x.ok |= (v < ce ? 1u : 0u) << j;
    }
}

// Orders the wave's LDS accesses on either side of it (the lanes of one
// wave exchange data through LDS; its accesses are carried out in order).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rearranges the slab through the wave's LDS (kSlabVectors vectors, one
// plane after the other) so that lane l holds vectors 4l .. 4l + 3: its 32
// terms are then consecutive in raster order.
template <int KK>
__device__ __forceinline__ void consecutive(u32x4 (&a)[kLaneVectors], u32x4 (&b)[kLaneVectors], u32x4 *lds)
{
    const int lane = threadIdx.x & 63;
    auto transpose = [&](u32x4 (&x)[kLaneVectors]) {
#pragma unroll
        for (int j = 0; j < kLaneVectors; ++j)
            lds[64 * j + lane] = x[j];
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < kLaneVectors; ++j)
            x[j] = lds[kLaneVectors * lane + j];
        wave_lds_sync();  // the next use may overwrite the buffer
    };
    if constexpr (KK != kSqDist)
        transpose(a);
    if constexpr (KK != kSqRef)
        transpose(b);
}

// The same with both planes' slabs in LDS at once (2 kSlabVectors vectors:
// plane a, then plane b), each left there in load order (vector v at v):
// the walk reads single terms from it afterwards.
template <int KK>
__device__ __forceinline__ void consecutive_kept(u32x4 (&a)[kLaneVectors], u32x4 (&b)[kLaneVectors], u32x4 *lds)
{
    const int lane = threadIdx.x & 63;
    u32x4 *la = lds, *lb = lds + kSlabVectors;
#pragma unroll
    for (int j = 0; j < kLaneVectors; ++j) {
        if constexpr (KK != kSqDist)
            la[64 * j + lane] = a[j];
        if constexpr (KK != kSqRef)
            lb[64 * j + lane] = b[j];
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < kLaneVectors; ++j) {
        if constexpr (KK != kSqDist)
            a[j] = la[kLaneVectors * lane + j];
        if constexpr (KK != kSqRef)
            b[j] = lb[kLaneVectors * lane + j];
    }
    wave_lds_sync();
}

// What one pass over the lane's 32 consecutive terms gathers for binade
// 2^(k+52), four terms at a time, one per byte of a register: only the low
// k + 1 <= 5 bits of t2 = t + 2^(k-1) matter here (rr, whether it is a
// tie, and h's parity), and they come from the terms' low k + 1 bits.
// Quad J holds terms J, J + 8, J + 16 and J + 24 (bytes 0..3), each masked
// to its low k + 1 bits, so that adding 2^(k-1) to every byte carries into
// no other byte.  Bit i of `untied` and `odd` is term i's (term order);
// rr4 holds the four bytes' sums of rr (at most 8 terms of rr < 2^k <= 16
// each: below 256).
struct SlabPass {
    uint32_t rr4 = 0;     // sum of rr, per byte
    uint32_t untied = 0;  // bit i: term i is no tie (rr > 0)
    uint32_t odd = 0;     // bit i: h_i is odd (bit k of t2)
};

template <int J>
__device__ __forceinline__ void pass_quad(SlabPass &p, uint32_t quad, int k)
{
    static_assert(J >= 0 && J < 8, "quad index");
    constexpr uint32_t kBytes = 0x01010101u;
    const uint32_t t2 = (quad & (((2u << k) - 1u) * kBytes)) + (1u << (k - 1)) * kBytes;
    const uint32_t rr = t2 & (((1u << k) - 1u) * kBytes);
    p.rr4 += rr;
    // bit 7 of each byte: rr > 0 (rr + 127 stays below 256); then bit 7
    // and bit k of byte b rotated to bit 8b + J
    const uint32_t nz = rr + 0x7f7f7f7fu;
    p.untied |= __builtin_amdgcn_alignbit(nz, nz, static_cast<uint32_t>(7 - J)) & (kBytes << J);
    p.odd |= __builtin_amdgcn_alignbit(t2, t2, static_cast<uint32_t>(k - J) & 31u) & (kBytes << J);
}

// The lane's run map from its pass (RunMap's packing: per start parity s,
// ties rounded down and the parity after).  From parity s, m + h_i has
// parity s ^ odd_0 ^ ... ^ odd_i up to the first tie; after a tie m is even,
// so from there on it is the XOR of odd over the terms since that tie --
// a prefix XOR in segments that start after each tie.  A tie rounds down
// where that parity is 1.
__device__ __forceinline__ RunMap lane_run_map(const SlabPass &p)
{
    const uint32_t tie = ~p.untied;
    RunMap m;
    if (tie == 0) {
        const uint32_t x = static_cast<uint32_t>(__builtin_popcount(p.odd)) & 1u;
        m.C = 0;
        m.P = x | ((x ^ 1u) << 16);
        return m;
    }
    uint32_t sx = p.odd, head = tie << 1;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
        sx ^= (sx << d) & ~head;
        head |= head << d;
    }
    const uint32_t first = tie & (0u - tie);
    const uint32_t upto_first = (first << 1) - 1u;  // bits 0 .. first tie (all of them if it is bit 31)
    const uint32_t rest = static_cast<uint32_t>(__builtin_popcount(tie & sx & ~upto_first));
    const uint32_t x1 = (sx & first) ? 1u : 0u;  // parity of m + h at the first tie, from s = 0
    m.C = (rest + x1) | ((rest + (x1 ^ 1u)) << 16);
    const uint32_t after = (tie >> 31) ? 0u : (sx >> 31);
    m.P = after | (after << 16);
    return m;
}

// The slab's map in binade 2^(k+52) from its exact total T, the OR of its
// terms (per lane) and the pass.  Three cases, decided for the whole wave:
// every term a multiple of 2^k (nothing rounds: m grows by T / 2^k); no
// ties (m grows by the sum of h, both parities flip with its parity);
// otherwise the lanes' run maps composed in lane order.
__device__ __forceinline__ Map2 slab_map(uint64_t T, uint32_t low_bits, const SlabPass &p, int k)
{
    constexpr uint64_t n = 64 * kLaneVectors * kTerms;
    if (__all((low_bits & ((1u << k) - 1)) == 0))
        return untied_map(T >> k);
    const uint32_t RR = wave_total32((p.rr4 & 0xffu) + ((p.rr4 >> 8) & 0xffu) + ((p.rr4 >> 16) & 0xffu) + (p.rr4 >> 24));
    if (__all(p.untied == ~0u))
        return untied_map((T + (n << (k - 1)) - RR) >> k);
    return run_map(wave_run(lane_run_map(p)), T, n, RR, k);
}

// The pass over the lane's 32 consecutive terms, quad by quad: quads[J]
// holds the low bytes of terms J, J + 8, J + 16 and J + 24.
__device__ __forceinline__ void pass_slab(SlabPass &p, const uint32_t (&quads)[8], int k)
{
    static_assert(kLaneVectors * kTerms == 32, "four quarters of 8 terms");
    pass_quad<0>(p, quads[0], k);
    pass_quad<1>(p, quads[1], k);
    pass_quad<2>(p, quads[2], k);
    pass_quad<3>(p, quads[3], k);
    pass_quad<4>(p, quads[4], k);
    pass_quad<5>(p, quads[5], k);
    pass_quad<6>(p, quads[6], k);
    pass_quad<7>(p, quads[7], k);
}

// Slab si of its chunk; lane 0 writes its part of the entry.  The terms
// are made once: their sum (the total), and the low bytes of each quad
// (J, J + 8, J + 16, J + 24), which are all the passes need (the low bits,
// and the pass for the predicted binade; a slab whose chunk may cross into
// the next binade gets a second pass for it).
template <int KK>
__device__ __forceinline__ void item_maps(ItemData &x, int si, int e, bool dual, uint64_t *entry, u32x4 *lds)
{
    const int k = e - 52;
    if (__builtin_amdgcn_readfirstlane(x.all_ok) == 0) {  // a slab past the frame's last vector
#pragma unroll
        for (int j = 0; j < kLaneVectors; ++j)
            keep_if<KK>((x.ok >> j) & 1u, x.a[j], x.b[j]);
    }
    consecutive<KK>(x.a, x.b, lds);
    // the lane's total (a 64-bit sum kept as two words and a carry add)
    uint32_t lo = 0, hi = 0, quad_or = 0;
    uint32_t quads[8];
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        uint32_t t[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            t[v] = vector_term<KK>(x.a[v], x.b[v], J);  // term J + 8v
            unsigned int carry;
            lo = __builtin_addc(lo, t[v], 0u, &carry);
            hi += carry;
        }
        // bytes 0..3: the low bytes of terms J, J + 8, J + 16, J + 24
        const uint32_t lo2 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);
        const uint32_t hi2 = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0400u);
        quads[J] = lo2 | (hi2 << 16);
        quad_or |= quads[J];
    }
    // the OR of the terms' low bytes (only bits below k <= 4 are asked)
    const uint32_t low_bits = (quad_or | (quad_or >> 8) | (quad_or >> 16) | (quad_or >> 24)) & 0xffu;
    const uint64_t T = wave_total64(lo | (static_cast<uint64_t>(hi) << 32));
    SlabPass p;
    pass_slab(p, quads, k);
    const Map2 slab = slab_map(T, low_bits, p, k);
    Map2 slab_b;
    if (dual) {
        SlabPass q;
        pass_slab(q, quads, k + 1);
        slab_b = slab_map(T, low_bits, q, k + 1);
    }
    if ((threadIdx.x & 63) == 0) {
        entry[kSlabMapsA + 3 * si + 0] = slab.dm0;
        entry[kSlabMapsA + 3 * si + 1] = slab.dm1;
        entry[kSlabMapsA + 3 * si + 2] = map_flags(slab, e);
        entry[kSlabMapsB + 3 * si + 0] = slab_b.dm0;
        entry[kSlabMapsB + 3 * si + 1] = slab_b.dm1;
        entry[kSlabMapsB + 3 * si + 2] = dual ? map_flags(slab_b, e + 1) : 0;
        entry[kSlabTotals + si] = T;
    }
}

// Where the slabs of the queues lie.  Slab item i of square sum KK's queue
// is slab i % kSlabs of the chunk queued at i / kSlabs.
struct Slabs {
    const u32x4 *R, *D;
    VecMap map;
    const uint64_t *queue;  // this square sum's queue segment of the frame
    uint64_t *maps;
    int64_t frame, vb, ve;  // the frame, its first whole vector and one past its last
    uint32_t first;         // frame * chunks: the frame's first queue index
};

struct SlabItem {
    int64_t frame, cb, sb, ce;
    uint64_t *entry;
    int si, e;
    bool dual;
};

// Slab item i (wave-uniform) of the frame's queue segment.
template <int KK>
__device__ __forceinline__ SlabItem slab_item(const Slabs &Q, int64_t i)
{
    const uint64_t q = Q.queue[i / kSlabs];
    const uint32_t idx = static_cast<uint32_t>(q);
    const uint32_t c = idx - Q.first;
    SlabItem x;
    x.frame = Q.frame;
    x.si = static_cast<int>(i % kSlabs);
    x.e = static_cast<int>((q >> 32) & 0xffu);
    x.dual = ((q >> 40) & 1u) != 0;
    x.cb = Q.vb + static_cast<int64_t>(c) * kChunkVectors;
    x.ce = x.cb + kChunkVectors < Q.ve ? x.cb + kChunkVectors : Q.ve;
    x.sb = x.cb + static_cast<int64_t>(x.si) * kSlabVectors;
    x.entry = Q.maps + (static_cast<uint64_t>(idx) * kSquares + KK) * kEntry;
    return x;
}

// Slab items below n of the frame's queue segment, handed out one at a time
// from the counter `ticket` to whichever wave of the frame's workgroups
// asks first.  The next item's vectors are read while the current one is
// mapped, except for the noise, which reads both planes.
template <int KK, bool kSh>
__device__ __forceinline__ void queue_maps(const Slabs &Q, uint32_t *ticket, int64_t n, u32x4 *lds)
{
    auto next = [&]() -> int64_t {
        uint32_t t = 0;
        if ((threadIdx.x & 63) == 0)
            t = atomicAdd(ticket, 1u);
        return static_cast<int64_t>(__builtin_amdgcn_readfirstlane(t));
    };
    ItemData x, y;
    auto map_item = [&](ItemData &d, const SlabItem &it) {
        item_maps<KK>(d, it.si, it.e, it.dual, it.entry, lds);
    };
    int64_t i = next();
    if (i >= n)
        return;
    SlabItem u = slab_item<KK>(Q, i);
    load_item<KK, kSh>(x, Q.R, Q.D, Q.map, u.frame, u.cb, u.sb, u.ce);
    if constexpr (KK == kSqNoise) {
        for (;;) {
            map_item(x, u);
            i = next();
            if (i >= n)
                return;
            u = slab_item<KK>(Q, i);
            load_item<KK, kSh>(x, Q.R, Q.D, Q.map, u.frame, u.cb, u.sb, u.ce);
        }
    } else {
        // Two buffers, taken in turn.  Each item mapped inside the loop
        // follows the loads of the next one, and the last item is mapped
        // apart, so that the waits before mapping an item never cover the
        // loads of the one after it.
        SlabItem v;
        for (;;) {
            i = next();
            if (i >= n) {
                map_item(x, u);
                return;
            }
            v = slab_item<KK>(Q, i);
            load_item<KK, kSh>(y, Q.R, Q.D, Q.map, v.frame, v.cb, v.sb, v.ce);
            map_item(x, u);
            i = next();
            if (i >= n) {
                map_item(y, v);
                return;
            }
            u = slab_item<KK>(Q, i);
            load_item<KK, kSh>(x, Q.R, Q.D, Q.map, u.frame, u.cb, u.sb, u.ce);
            map_item(y, v);
        }
    }
}

// Steps 2 and 3 in one launch: a group of workgroups per frame (the grid a
// multiple of nframes), each with the frame's prefix scan (frame_prefix),
// then the frame's queued slabs, which its waves take one at a time from
// the frame's counters (one per queue, in turn).  Workgroup 0 of each
// frame writes the prefix's results.
// Two-byte samples map slabs; one-byte ones only scan (one workgroup per
// frame).
// Five waves per SIMD fit its registers without spills (96 VGPRs), and its
// LDS (a 4 KB buffer per wave).
template <bool kSh>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) void cpu_order_maps(
    const void *ref, const void *dist, int64_t pixels, int chunks, int nframes, uint64_t *rec,
    uint64_t *totals, uint64_t *out_noise, uint64_t *out_moments, uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
    uint64_t *queue, uint64_t *maps, VecMap vmap)
{
    __shared__ PrefixLds pl;
    __shared__ u32x4 lds_all[kThreads / 64][kSlabVectors];
    // frame f's workgroups are f, f + nframes, ...: spread over the launch
    // order, so that each frame has workgroups of every age on the CUs
    // (older waves issue first) and the frames progress together
    const int64_t f = blockIdx.x % nframes;
    const int j = static_cast<int>(blockIdx.x / nframes);
    static_assert(sizeof(lds_all) >= kStageRecords * 64, "the stage fits the transpose buffers");
    // the scan at a raised issue priority: the SIMDs issue older waves
    // first, so a workgroup still scanning beside others already mapping
    // (a tight VALU loop) would otherwise wait behind them
    __builtin_amdgcn_s_setprio(2);
    frame_prefix(pl, &lds_all[0][0], f, nframes, rec, pixels, chunks, j == 0, totals, out_noise, out_moments, out_cpu_noise,
                 out_cpu_moments, maps, queue);
    __builtin_amdgcn_s_setprio(0);
    if (!maps)
        return;
    // the wave's index, made wave-uniform so that the items' bookkeeping
    // runs on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
    u32x4 *lds = lds_all[wave];
    uint32_t *tickets = reinterpret_cast<uint32_t *>(rec + f * chunks * kRecordStride + kTickets);
    const int64_t cap = static_cast<int64_t>(nframes) * chunks;
    constexpr int V = 8;
    Slabs Q;
    Q.R = static_cast<const u32x4 *>(ref);
    Q.D = static_cast<const u32x4 *>(dist);
    Q.map = vmap;
    Q.maps = maps;
    Q.frame = f;
    Q.vb = (f * pixels + V - 1) / V;
    Q.ve = (f * pixels + pixels) / V;
    Q.first = static_cast<uint32_t>(f * chunks);
    int64_t n = static_cast<int64_t>(pl.nq[kSqNoise]) * kSlabs;
    Q.queue = queue + kSqNoise * cap + f * chunks;
    if (n > 0)
        queue_maps<kSqNoise, kSh>(Q, tickets + kSqNoise, n, lds);
    n = static_cast<int64_t>(pl.nq[kSqRef]) * kSlabs;
    Q.queue = queue + kSqRef * cap + f * chunks;
    if (n > 0)
        queue_maps<kSqRef, kSh>(Q, tickets + kSqRef, n, lds);
    n = static_cast<int64_t>(pl.nq[kSqDist]) * kSlabs;
    Q.queue = queue + kSqDist * cap + f * chunks;
    if (n > 0)
        queue_maps<kSqDist, kSh>(Q, tickets + kSqDist, n, lds);
}

// ------------------------------------------------------------------ 4. walk
// All 64 lanes of the walking wave hold the same S throughout.  At every
// level (the chunks of a block, the slabs of a chunk, groups of 4 vectors of
// a slab, the terms of one group) the walk takes a row of up to 64 items,
// item j in lane j, each with its exact total and its maps for up to two
// binades, and moves S over them with wave scans.

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t from_below64(uint64_t identity, uint64_t v)
{
    return static_cast<uint64_t>(from_below<CTRL, ROWS>(static_cast<uint32_t>(identity), static_cast<uint32_t>(v))) |
           (static_cast<uint64_t>(
                from_below<CTRL, ROWS>(static_cast<uint32_t>(identity >> 32), static_cast<uint32_t>(v >> 32)))
            << 32);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ Map2 map_scan_step(const Map2 &m)
{
    Map2 o;  // the identity where there is no source
    o.dm0 = from_below64<CTRL, ROWS>(0, m.dm0);
    o.dm1 = from_below64<CTRL, ROWS>(0, m.dm1);
    o.p0 = from_below<CTRL, ROWS>(0u, m.p0);
    o.p1 = from_below<CTRL, ROWS>(1u, m.p1);
    return map_then(o, m);
}

// Lane j gets the composite of the maps of lanes 0..j, in lane order.
__device__ __forceinline__ Map2 wave_scan_map(Map2 m)
{
    m = map_scan_step<0x111, 0xf>(m);
    m = map_scan_step<0x112, 0xf>(m);
    m = map_scan_step<0x114, 0xf>(m);
    m = map_scan_step<0x118, 0xf>(m);
    m = map_scan_step<0x142, 0xa>(m);
    return map_scan_step<0x143, 0xc>(m);
}

// x if c, else y (field by field, so that nothing goes through a stack copy).
__device__ __forceinline__ Map2 select_map(bool c, const Map2 &x, const Map2 &y)
{
    Map2 m;
    m.dm0 = c ? x.dm0 : y.dm0;
    m.dm1 = c ? x.dm1 : y.dm1;
    m.p0 = c ? x.p0 : y.p0;
    m.p1 = c ? x.p1 : y.p1;
    return m;
}

// One item of a row: its exact total, and its maps for the binades in the
// flags fa and fb (flags 0: no map); `none`: an item that adds nothing
// (the identity in any binade).
struct Item {
    uint64_t T = 0;
    Map2 a, b;
    uint64_t fa = 0, fb = 0;
    bool none = false;
};

// Moves S over items 0..n-1 of the row (n <= 64).  Repeatedly: below 2^53,
// prefix sums of the totals find the item in which S gets there (every add
// before it is exact); past it, prefix compositions of each item's map for
// S's binade find the first item without one, or in which S leaves the
// binade (m only grows, so if it ends inside the binade it stayed there).
// S is moved to just before that item, which `one(S, j)` walks at a finer
// level.
template <class One>
__device__ __forceinline__ uint64_t walk_items(uint64_t S, const Item &it, int n, One one)
{
    const int lane = threadIdx.x & 63;
    int from = 0;  // items before `from` are done
    while (from < n) {
        const bool act = lane >= from && lane < n;
        int jx;
        if (S < kTwo53) {
            const uint64_t t = act ? it.T : 0;
            const uint64_t incl = wave_scan64(t);
            const uint64_t rest = lane_value64(incl, 63);
            if (S + rest < kTwo53)
                return S + rest;
            jx = __builtin_ctzll(__ballot(act && S + incl >= kTwo53));
            S += lane_value64(incl - t, jx);
        } else {
            const int e = binade(S);
            const int k = e - 52;
            const bool use_a = (it.fa & 1u) && flags_binade(it.fa) == e;
            const bool use_b = !use_a && (it.fb & 1u) && flags_binade(it.fb) == e;
            const bool ok = it.none || use_a || use_b;
            const Map2 pm = wave_scan_map(act && !it.none && ok ? select_map(use_a, it.a, it.b) : Map2{});
            const uint64_t mm = S >> k;
            const uint64_t m2 = mm + pick(mm, pm.dm0, pm.dm1);  // m after items from..lane
            const uint64_t bad = __ballot(act && (!ok || m2 >= kTwo53));
            if (!bad)
                return lane_value64(m2, 63) << k;
            jx = __builtin_ctzll(bad);
            if (jx > from)
                S = lane_value64(m2, jx - 1) << k;
        }
        S = one(S, jx);
        from = jx + 1;
    }
    return S;
}

// The map of one term t in binade 2^(k+52): m grows by h, less one on a tie
// (t + 2^(k-1) a multiple of 2^k) when m + h is odd; after a tie m is even.
__device__ __forceinline__ Map2 term_map(uint32_t t, int k)
{
    const uint32_t t2 = t + (1u << (k - 1));
    const uint64_t h = t2 >> k;
    const bool tie = (t2 & ((1u << k) - 1)) == 0;
    const uint32_t hb = static_cast<uint32_t>(h) & 1u;
    Map2 m;
    m.dm0 = h - (tie && hb ? 1 : 0);       // from parity 0, m + h has h's parity
    m.dm1 = h - (tie && !hb ? 1 : 0);      // from parity 1, the other one
    m.p0 = tie ? 0u : hb;
    m.p1 = tie ? 0u : hb ^ 1u;
    return m;
}

// Term i (raster order) of the 32 that lane group g holds in LDS after
// `consecutive` (vectors 4g .. 4g + 3).
template <int KK>
__device__ __forceinline__ uint32_t lds_term(const u32x4 *lds, int g, int i)
{
    const u32x4 zero = {0, 0, 0, 0};
    const u32x4 a = KK != kSqDist ? lds[kLaneVectors * g + (i >> 3)] : zero;
    const u32x4 b = KK != kSqRef ? lds[kSlabVectors + kLaneVectors * g + (i >> 3)] : zero;
    const int w = (i >> 1) & 3;
    const uint32_t wa = w == 0 ? a.x : w == 1 ? a.y : w == 2 ? a.z : a.w;
    const uint32_t wb = w == 0 ? b.x : w == 1 ? b.y : w == 2 ? b.z : b.w;
    const uint32_t r = (i & 1) ? wa >> 16 : wa & 0xffffu;
    const uint32_t d = (i & 1) ? wb >> 16 : wb & 0xffffu;
    return square_term<2>(KK, r, d);
}

// The planes as the walk reads them: their vectors through the map, of one
// frame.
struct Planes {
    const u32x4 *R, *D;
    VecMap map;
    int64_t frame;
};

// Vectors [sb, se) (at most 256) from S, with maps made here for S's binade
// and the next (a slab's total is far below S past 2^53, so S crosses at
// most one binade in it).  The slab goes through LDS so that lane g holds
// vectors 4g .. 4g + 3, 32 consecutive terms: one row of 64 groups, and
// inside the group where S crosses, one row of its 32 terms.
template <int KK, bool kSh>
__device__ __forceinline__ uint64_t walk_slab(uint64_t S, const Planes &P, int64_t sb, int64_t se, u32x4 *lds)
{
    const int lane = threadIdx.x & 63;
    const int eA = S >= kTwo53 ? binade(S) : 53;
    const int kA = eA - 52;
    u32x4 a[kLaneVectors], b[kLaneVectors];
#pragma unroll
    for (int j = 0; j < kLaneVectors; ++j) {
        const int64_t v = sb + 64 * j + lane;
        load_vector<KK, kSh>(P.R, P.D, P.map, P.frame, v, v < se, sb, a[j], b[j]);
        keep_if<KK>(v < se, a[j], b[j]);
    }
    consecutive_kept<KK>(a, b, lds);
    Item g;
    RunMap mA, mB;
    uint32_t rA = 0, rB = 0;
#pragma unroll
    for (int j = 0; j < kLaneVectors; ++j)
#pragma unroll
        for (int i = 0; i < kTerms; ++i) {
            const uint32_t t = vector_term<KK>(a[j], b[j], i);
            g.T += t;
            run_add(mA, rA, t, kA);
            run_add(mB, rB, t, kA + 1);
        }
    constexpr uint64_t n = kLaneVectors * kTerms;
    g.a = run_map(mA, g.T, n, rA, kA);
    g.b = run_map(mB, g.T, n, rB, kA + 1);
    g.fa = map_flags(g.a, eA);
    g.fb = map_flags(g.b, eA + 1);
    return walk_items(S, g, 64, [&](uint64_t S1, int grp) {
        // the 32 terms of group grp, term i in lane i
        const int e1 = S1 >= kTwo53 ? binade(S1) : 53;
        const uint32_t t = lane < kLaneVectors * kTerms ? lds_term<KK>(lds, grp, lane) : 0u;
        Item x;
        x.T = t;
        x.a = term_map(t, e1 - 52);
        x.b = term_map(t, e1 - 51);
        x.fa = map_flags(x.a, e1);
        x.fb = map_flags(x.b, e1 + 1);
        return walk_items(S1, x, kLaneVectors * kTerms,
                          [&](uint64_t S2, int i) { return cpu_add(S2, lane_value(t, i)); });
    });
}

// One chunk, from its slab maps; a slab where they do not apply is walked
// with maps made on the spot.
template <int KK, bool kSh>
__device__ __forceinline__ uint64_t walk_chunk(uint64_t S, const Planes &P, const uint64_t *entry, int64_t cb,
                                               int64_t ce, u32x4 *lds)
{
    const int lane = threadIdx.x & 63;
    if (entry[kChunkMap + 2] & kChunkOnly) {
        // no slab maps (S is not where the chunk map expects it): map each
        // slab on the spot
        for (int64_t sb = cb; sb < ce; sb += kSlabVectors)
            S = walk_slab<KK, kSh>(S, P, sb, sb + kSlabVectors < ce ? sb + kSlabVectors : ce, lds);
        return S;
    }
    const int n = static_cast<int>((ce - cb + kSlabVectors - 1) / kSlabVectors);  // slabs holding vectors
    Item it;
    if (lane < n) {
        it.T = entry[kSlabTotals + lane];
        it.fa = entry[kSlabMapsA + 3 * lane + 2];
        it.a = map_from(entry[kSlabMapsA + 3 * lane + 0], entry[kSlabMapsA + 3 * lane + 1], it.fa);
        it.fb = entry[kSlabMapsB + 3 * lane + 2];
        it.b = map_from(entry[kSlabMapsB + 3 * lane + 0], entry[kSlabMapsB + 3 * lane + 1], it.fb);
    }
    return walk_items(S, it, n, [&](uint64_t S1, int j) {
        const int64_t sb = cb + static_cast<int64_t>(j) * kSlabVectors;
        return walk_slab<KK, kSh>(S1, P, sb, sb + kSlabVectors < ce ? sb + kSlabVectors : ce, lds);
    });
}

// ---------------------------------------------------- 4a. chunk and block maps
// Compact maps for the walk, one record {T, dm0, dm1, flags} (kCompact
// uint64) per (frame, chunk, square sum) and per (frame, block of 64
// chunks, square sum):
//  * T: the exact total of the chunk's whole vectors (chunk 0's record
//    less the frame's head and tail samples), or of the block's chunks;
//  * the map composed from the chunk's slab maps (or its own map when it
//    cannot round), or from the block's chunk maps; flags 0 (no map) unless
//    every part holds a map for one binade.  Chunks without vectors count
//    as the identity.
// The walk kernel's waves write them (one wave per block) before its first
// wave walks the frame.
constexpr int kCompact = 4;
constexpr int kBlockChunks = 64;

__host__ __device__ __forceinline__ int frame_blocks(int chunks) { return (chunks + kBlockChunks - 1) / kBlockChunks; }

// Terms of the frame's samples before its first whole vector (lane < head)
// and after its last (lane < tail); both are fewer than 8.
struct FrameEdges {
    int64_t vb, ve, tail_begin;
    int head, tail;
    uint32_t hterm, tterm;
};

template <int KK>
__device__ __forceinline__ FrameEdges frame_edges(const void *ref, const void *dist, int64_t pixels, int64_t frame)
{
    constexpr int V = 8;
    const int lane = threadIdx.x & 63;
    const int64_t e0 = frame * pixels, e1 = e0 + pixels;
    FrameEdges x;
    x.vb = (e0 + V - 1) / V;
    x.ve = e1 / V;
    const int64_t head_end = x.vb < x.ve ? x.vb * V : e1;
    x.tail_begin = x.vb < x.ve ? x.ve * V : e1;
    x.head = static_cast<int>(head_end - e0);
    x.tail = static_cast<int>(e1 - x.tail_begin);
    const uint16_t *r16 = static_cast<const uint16_t *>(ref);
    const uint16_t *d16 = static_cast<const uint16_t *>(dist);
    x.hterm = lane < x.head ? square_term<2>(KK, r16[e0 + lane], d16[e0 + lane]) : 0u;
    x.tterm = lane < x.tail ? square_term<2>(KK, r16[x.tail_begin + lane], d16[x.tail_begin + lane]) : 0u;
    return x;
}

// The map of a chunk from its entry (flags 0 where it has none for one
// binade).
__device__ __forceinline__ Map2 entry_map(const uint64_t *entry, uint64_t &flags)
{
    const uint64_t cf = entry[kChunkMap + 2];
    if (cf & kChunkOnly) {
        flags = cf & ~kChunkOnly;
        return map_from(entry[kChunkMap + 0], entry[kChunkMap + 1], cf);
    }
    Map2 m;
    flags = 0;
    if (!(cf & kQueued))
        return m;
    const uint64_t key = entry[kSlabMapsA + 2] & 0xffffu;  // valid bit and binade of slab 0
    bool ok = (key & 1u) != 0;
#pragma unroll
    for (int j = 0; j < kSlabs; ++j) {
        const uint64_t fl = entry[kSlabMapsA + 3 * j + 2];
        m = map_then(m, map_from(entry[kSlabMapsA + 3 * j], entry[kSlabMapsA + 3 * j + 1], fl));
        ok = ok && (fl & 0xffffu) == key;
    }
    flags = ok ? map_flags(m, flags_binade(key)) : 0;
    return m;
}

template <int KK>
__device__ __forceinline__ void compose_block(const void *ref, const void *dist, int64_t pixels, int chunks,
                                              const uint64_t *rec, const uint64_t *maps, int64_t frame, int block,
                                              uint64_t *cmaps, uint64_t *bmaps)
{
    const int lane = threadIdx.x & 63;
    const FrameEdges fe = frame_edges<KK>(ref, dist, pixels, frame);
    const uint64_t edges = block == 0 ? wave_total64(fe.hterm) + wave_total64(fe.tterm) : 0;
    const int c = block * kBlockChunks + lane;
    const bool in = c < chunks;
    const bool empty = !in || fe.vb + static_cast<int64_t>(c) * kChunkVectors >= fe.ve;
    uint64_t T = 0, flags = 0;
    Map2 m;
    if (in) {
        const int64_t wg = frame * chunks + c;
        T = rec[wg * kRecordStride + record_field(KK)] - (c == 0 ? edges : 0);
        if (!empty)
            m = entry_map(maps + (wg * kSquares + KK) * kEntry, flags);
        uint64_t *out = cmaps + (wg * kSquares + KK) * kCompact;
        out[0] = T;
        out[1] = m.dm0;
        out[2] = m.dm1;
        out[3] = flags;
    }
    // the block: one binade for every chunk with vectors, else no map
    const uint64_t key = lane_value64(flags, 0) & 0xffffu;
    const bool ok = __all(empty || ((flags & 1u) && (flags & 0xffffu) == key));
    const Map2 bm = wave_map(m);
    const uint64_t BT = wave_total64(T);
    if (lane == 0) {
        uint64_t *out = bmaps + ((frame * frame_blocks(chunks) + block) * kSquares + KK) * kCompact;
        out[0] = BT;
        out[1] = bm.dm0;
        out[2] = bm.dm1;
        out[3] = ok && (key & 1u) ? map_flags(bm, flags_binade(key)) : 0;
    }
}

// ---------------------------------------------------------- 4b. the walk
// The 64 chunks of one block, chunk b*64 + j in lane j, from S, from their
// compact records; a chunk where they do not apply is walked slab by slab.
template <int KK, bool kSh>
__device__ __forceinline__ uint64_t walk_block(uint64_t S, const Planes &P, const uint64_t *cmaps,
                                               const uint64_t *entries, int64_t frame, int chunks, int block,
                                               const FrameEdges &fe, u32x4 *lds)
{
    const int lane = threadIdx.x & 63;
    const int c = block * kBlockChunks + lane;
    const int n = chunks - block * kBlockChunks < kBlockChunks ? chunks - block * kBlockChunks : kBlockChunks;
    Item it;
    it.none = lane >= n || fe.vb + static_cast<int64_t>(c) * kChunkVectors >= fe.ve;  // no vectors
    if (lane < n) {
        const uint64_t *x = cmaps + ((frame * chunks + c) * kSquares + KK) * kCompact;
        it.T = x[0];
        it.fa = x[3];
        it.a = map_from(x[1], x[2], it.fa);
    }
    return walk_items(S, it, n, [&](uint64_t S1, int j) {
        const int64_t cb = fe.vb + static_cast<int64_t>(block * kBlockChunks + j) * kChunkVectors;
        const int64_t ce = cb + kChunkVectors < fe.ve ? cb + kChunkVectors : fe.ve;
        return walk_chunk<KK, kSh>(S1, P, entries + static_cast<int64_t>(block * kBlockChunks + j) * kSquares * kEntry,
                              cb, ce, lds);
    });
}

template <int KK, bool kSh>
__device__ __forceinline__ void walk_frame(const void *ref, const void *dist, int64_t pixels, int chunks,
                                           const uint64_t *maps, const uint64_t *cmaps, const uint64_t *bmaps,
                                           int64_t frame, uint64_t *dst, u32x4 *lds, const VecMap &vmap)
{
    const int lane = threadIdx.x & 63;
    // (mapped planes hold whole vectors only: no head or tail samples)
    const FrameEdges fe = frame_edges<KK>(ref, dist, pixels, frame);
    // the head comes first in raster order; it is far below 2^53, so exact
    uint64_t S = wave_total64(fe.hterm);
    const Planes P{static_cast<const u32x4 *>(ref), static_cast<const u32x4 *>(dist), vmap, frame};
    const uint64_t *entries = maps + (frame * chunks * kSquares + KK) * kEntry;  // chunk c: + c * kSquares * kEntry
    // block b's record in lane b (a frame has at most 2^22 vectors: 32 blocks)
    const int blocks = frame_blocks(chunks);
    uint64_t BT = 0, bdm0 = 0, bdm1 = 0, bfl = 0;
    if (lane < blocks) {
        const uint64_t *x = bmaps + ((frame * blocks + lane) * kSquares + KK) * kCompact;
        BT = x[0];
        bdm0 = x[1];
        bdm1 = x[2];
        bfl = x[3];
    }
    for (int b = 0; b < blocks; ++b) {
        const uint64_t T = lane_value64(BT, b);
        if (S + T < kTwo53) {
            S += T;
            continue;
        }
        const uint64_t fl = lane_value64(bfl, b);
        if ((fl & 1u) && map_apply(S, map_from(lane_value64(bdm0, b), lane_value64(bdm1, b), fl), flags_binade(fl)))
            continue;
        S = walk_block<KK, kSh>(S, P, cmaps, entries, frame, chunks, b, fe, lds);
    }
    // the tail comes last
    for (int j = 0; j < fe.tail; ++j)
        S = cpu_add(S, lane_value(fe.tterm, j));
    if (lane == 0)
        *dst = S;
}

// One workgroup per (frame, square sum); two-byte samples only.  Sums in
// which no add rounds were written by the prefix scan.  The workgroup's waves
// first compose the frame's blocks (block b in wave b % kWalkWaves); after
// the barrier that makes their records visible, wave 0 walks the frame.
constexpr int kWalkWaves = 8;

template <int KK, bool kSh>
__device__ __forceinline__ void compose_then_walk(const void *ref, const void *dist, int64_t pixels, int chunks,
                                                  const uint64_t *rec, const uint64_t *maps, uint64_t *cmaps,
                                                  uint64_t *bmaps, int64_t frame, uint64_t *dst, u32x4 *lds,
                                                  const VecMap &vmap)
{
    const int wave = threadIdx.x / 64;
    for (int b = wave; b < frame_blocks(chunks); b += kWalkWaves)
        compose_block<KK>(ref, dist, pixels, chunks, rec, maps, frame, b, cmaps, bmaps);
    __syncthreads();
    if (wave == 0)
        walk_frame<KK, kSh>(ref, dist, pixels, chunks, maps, cmaps, bmaps, frame, dst, lds, vmap);
}

template <bool kSh>
__global__ __launch_bounds__(64 * kWalkWaves) void cpu_order_walk(const void *ref, const void *dist, int64_t pixels,
                                                                  int chunks, const uint64_t *rec,
                                                                  const uint64_t *totals, const uint64_t *maps,
                                                                  uint64_t *cmaps, uint64_t *bmaps,
                                                                  uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                                                  VecMap vmap)
{
    __shared__ u32x4 lds[2 * kSlabVectors];  // a slab of each plane, for `consecutive_kept`
    const int64_t frame = blockIdx.x / kSquares;
    const int kk = static_cast<int>(blockIdx.x - frame * kSquares);
    if (totals[frame * kSquares + kk] < kTwo53)  // the prefix wrote the CPU's value
        return;
    switch (kk) {
    case kSqNoise:
        compose_then_walk<kSqNoise, kSh>(ref, dist, pixels, chunks, rec, maps, cmaps, bmaps, frame, &out_cpu_noise[frame],
                                    lds, vmap);
        break;
    case kSqRef:
        compose_then_walk<kSqRef, kSh>(ref, dist, pixels, chunks, rec, maps, cmaps, bmaps, frame,
                                  &out_cpu_moments[4 * frame + 2], lds, vmap);
        break;
    default:
        compose_then_walk<kSqDist, kSh>(ref, dist, pixels, chunks, rec, maps, cmaps, bmaps, frame,
                                   &out_cpu_moments[4 * frame + 3], lds, vmap);
        break;
    }
}

// Workgroups of the maps kernel that the current device holds at once (its
// occupancy per CU, from its register and LDS use, times the CUs), asked
// once per device.
template <bool kSh>
hipError_t maps_resident_workgroups(int64_t &wgs)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int64_t> cache[kMaxDevices];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached && (wgs = cache[dev].load(std::memory_order_relaxed)) > 0)
        return hipSuccess;
    int per_cu = 0, cus = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cpu_order_maps<kSh>, kThreads, 0);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    wgs = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (cached)
        cache[dev].store(wgs, std::memory_order_relaxed);
    return hipSuccess;
}

}  // namespace

VecMap make_vec_map(int w, int h, const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                    const void *dist, int64_t dist_row_stride, int64_t dist_frame_stride)
{
    constexpr int V = 8;  // two-byte samples per vector
    VecMap M;
    M.vpr = static_cast<uint32_t>(w / V);
    M.frame_vecs = static_cast<int64_t>(h) * M.vpr;
    // floor(r / vpr) = (r * magic) >> shift for every r < 2^22: with
    // 2^(L-1) < vpr <= 2^L, shift = 22 + L and magic = ceil(2^shift / vpr),
    // the error r * (magic - 2^shift / vpr) / 2^shift < 2^-L <= 1 / vpr
    int L = 0;
    while ((1u << L) < M.vpr)
        ++L;
    M.shift = 22 + L;
    M.magic = ((1ull << M.shift) + M.vpr - 1) / M.vpr;
    M.pad_row_r = ref_row_stride / V - M.vpr;
    M.pad_row_d = dist_row_stride / V - M.vpr;
    M.pad_frame_r = ref_frame_stride / V - M.frame_vecs;
    M.pad_frame_d = dist_frame_stride / V - M.frame_vecs;
    M.phase_r = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ref) & 15u);
    M.phase_d = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dist) & 15u);
    M.row_bytes_r = 2 * ref_row_stride;
    M.frame_bytes_r = 2 * ref_frame_stride;
    M.row_bytes_d = 2 * dist_row_stride;
    M.frame_bytes_d = 2 * dist_frame_stride;
    const int64_t odd = (M.row_bytes_r | M.frame_bytes_r | M.row_bytes_d | M.frame_bytes_d) & 15;
    M.general = (M.phase_r | M.phase_d | static_cast<uint32_t>(odd)) != 0;
    return M;
}

CpuOrderLayout cpu_order_layout(const Geometry &g)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    CpuOrderLayout l{};
    const size_t wgs = static_cast<size_t>(g.workgroups);
    l.records = 0;
    l.queue = up(l.records + g.workspace_bytes);
    l.totals = up(l.queue + wgs * kSquares * sizeof(uint64_t));
    l.maps = up(l.totals + static_cast<size_t>(g.nframes) * kSquares * sizeof(uint64_t));
    l.cmaps = up(l.maps + wgs * kSquares * kEntry * sizeof(uint64_t));
    l.bmaps = up(l.cmaps + wgs * kSquares * kCompact * sizeof(uint64_t));
    l.bytes = up(l.bmaps + static_cast<size_t>(g.nframes) * frame_blocks(g.chunks) * kSquares * kCompact *
                               sizeof(uint64_t));
    return l;
}

hipError_t launch_plane_stats_cpu_order(const Geometry &g, const void *ref, const void *dist,
                                        uint64_t *out_noise, uint64_t *out_moments,
                                        uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                        void *workspace, hipStream_t stream, const VecMap &map)
{
    const CpuOrderLayout l = cpu_order_layout(g);
    char *ws = static_cast<char *>(workspace);
    uint64_t *rec = reinterpret_cast<uint64_t *>(ws + l.records);
    uint64_t *queue = reinterpret_cast<uint64_t *>(ws + l.queue);
    uint64_t *totals = reinterpret_cast<uint64_t *>(ws + l.totals);
    uint64_t *maps = reinterpret_cast<uint64_t *>(ws + l.maps);
    uint64_t *cmaps = reinterpret_cast<uint64_t *>(ws + l.cmaps);
    uint64_t *bmaps = reinterpret_cast<uint64_t *>(ws + l.bmaps);
    // stage 1 with the low bits of the terms, at two-byte samples
    if (map.vpr && g.sample_bytes != 2)
        return hipErrorInvalidValue;
    hipError_t err = map.vpr ? launch_stage1_mapped(g, ref, dist, rec, map, stream)
                             : launch_plane_stats(g, ref, dist, nullptr, nullptr, rec, stream, nullptr, nullptr,
                                                  g.sample_bytes == 2);
    if (err != hipSuccess)
        return err;
    const unsigned nf = static_cast<unsigned>(g.nframes);
    const bool two_byte = g.sample_bytes == 2;  // one-byte sums never reach 2^53
    if (g.chunks > kMaxFrameChunks)
        return hipErrorInvalidValue;
    const bool shifted = map.general != 0;
    // at two-byte samples, as many workgroups per frame as the device holds
    // at once over all frames (at least one), never more than the frame can
    // have slabs for, and with at most kScanChunks chunks scanned per frame:
    // each workgroup runs the frame's scan for itself, and past that more
    // of them cost more scans than they save (a 3840x2160x32 batch, 507
    // chunks a frame, with nothing to map: 166 us a step at 16 workgroups a
    // frame against 169 us at 32; a 2560x1440x64 one, 225 chunks, maps
    // 1.5 us faster at 20 than at 16)
    constexpr int64_t kScanChunks = 8192;
    int64_t per_frame = 1;
    if (two_byte) {
        int64_t resident = 0;
        err = shifted ? maps_resident_workgroups<true>(resident) : maps_resident_workgroups<false>(resident);
        if (err != hipSuccess)
            return err;
        const int64_t most = (static_cast<int64_t>(g.chunks) * kSquares * kSlabs + kThreads / 64 - 1) / (kThreads / 64);
        per_frame = resident / g.nframes;
        per_frame = per_frame < 1 ? 1 : per_frame > most ? most : per_frame;
        const int64_t scans = kScanChunks / g.chunks;
        per_frame = per_frame > scans ? (scans > 1 ? scans : 1) : per_frame;
    }
    const dim3 wgs(static_cast<unsigned>(g.nframes * per_frame));
    uint64_t *maps_arg = two_byte ? maps : nullptr;
    if (shifted)
        cpu_order_maps<true><<<wgs, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, g.nframes, rec, totals,
                                                           out_noise, out_moments, out_cpu_noise, out_cpu_moments,
                                                           queue, maps_arg, map);
    else
        cpu_order_maps<false><<<wgs, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, g.nframes, rec, totals,
                                                            out_noise, out_moments, out_cpu_noise, out_cpu_moments,
                                                            queue, maps_arg, map);
    err = hipGetLastError();
    if (err != hipSuccess || !two_byte)
        return err;
    if (shifted)
        cpu_order_walk<true><<<dim3(nf * kSquares), 64 * kWalkWaves, 0, stream>>>(
            ref, dist, g.pixels, g.chunks, rec, totals, maps, cmaps, bmaps, out_cpu_noise, out_cpu_moments, map);
    else
        cpu_order_walk<false><<<dim3(nf * kSquares), 64 * kWalkWaves, 0, stream>>>(
            ref, dist, g.pixels, g.chunks, rec, totals, maps, cmaps, bmaps, out_cpu_noise, out_cpu_moments, map);
    return hipGetLastError();
}

}  // namespace vqx
