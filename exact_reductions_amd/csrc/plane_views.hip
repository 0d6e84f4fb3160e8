// Stage 1 over plane views: planes read with a row stride and a frame stride
// (chroma planes, padded pitches, regions of interest, planar YUV frames),
// for the five sums and for the integer psnr noise.
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
//
// The terms are those of stage 1 (plane_stats.hip) for the five sums; the
// integer psnr twin keeps one integer per frame [PSNR, Alternatives], the
// sum of the exact squares of the sample differences (|r - d| < 2^16, so a
// square is below 2^32; at 8 bits it is stage 1's noise identity).  Only
// the addressing differs: a workgroup takes a tile of whole rows (or a
// segment of one long row) of one frame.  Where the tile's rows all start
// at the same offset within 16 bytes, and ref and dist at the same one,
// its 16-byte vectors are walked as one flat range across the rows (each
// row's few samples before its first and after its last whole vector are
// taken one by one); otherwise the tile is read sample by sample.  Integer
// sums make the tiling irrelevant to the result.

#include <type_traits>

#include "plane_stats.h"
#include "reduce.h"
#include "terms.h"

#pragma clang fp contract(off)

namespace vqx {
namespace {

constexpr int kTileVecs = 2048;  // 16-byte vectors of each plane per tile, at most

// ----------------------------------------------------------------- budgets
// A tile holds at most kTileVecs * 16 bytes of each plane (rows * cw <=
// kTileVecs * V samples, by the tiling), and whichever path reads it --
// whole vectors, rows at their own offsets (up to rows * slots vectors and
// one edge sample per row for a lane: up to 72 vectors and 64 samples when
// a row is 32 vectors wide), or sample by sample -- each of its samples is
// added by exactly one lane.  So a lane's, and a wave's, total is at most
// the tile's:
//  8 bits: sums of squares <= 32768 * 255^2 < 2^31, sample sums < 2^24;
// 16 bits: a lane's sum of squares <= 16384 * (2^32 - 1) < 2^46 (exact in
//          binary64 at every step), crossing the wave as its low 16 bits
//          (wave sum < 2^22) and the rest (wave sum <= 16384 * 2^16 = 2^30);
//          sample sums <= 16384 * 65535 < 2^30.
constexpr unsigned long long kTileSamples8 = kTileVecs * 16ull, kTileSamples16 = kTileVecs * 8ull;
static_assert(kTileSamples8 * 255ull * 255ull < (1ull << 32), "8-bit wave budget");
static_assert(kTileSamples8 * 255ull < (1ull << 32), "8-bit sample-sum budget");
static_assert((kTileSamples16 * 0xffffffffull >> 16) + 64ull * 0xffffull < (1ull << 32), "16-bit wave budget");
static_assert(kTileSamples16 * 65535ull < (1ull << 32), "16-bit sample-sum budget");
static_assert(kTileSamples16 * 0xffffffffull < (1ull << 53), "16-bit lane sums exact in binary64");

// ------------------------------------------------------- integer psnr terms
// 8 bits: sum (r-d)^2 = sum r^2 + sum d^2 - 2 sum r*d from dot products.
struct AccInt8 {
    uint32_t r2 = 0, d2 = 0, rd = 0;
};

__device__ __forceinline__ void add_dword(AccInt8 &a, uint32_t r, uint32_t d)
{
    a.r2 = __builtin_amdgcn_udot4(r, r, a.r2, false);
    a.d2 = __builtin_amdgcn_udot4(d, d, a.d2, false);
    a.rd = __builtin_amdgcn_udot4(r, d, a.rd, false);
}

// 9..16 bits: the absolute difference, below 2^16, squared in unsigned
// 32-bit arithmetic: the square is below 2^32, so the product is exact, and
// it is widened without sign.  (The 24-bit multiply builtin returns a signed
// int, which would sign-extend squares of 2^31 and above.)
struct AccInt16 {
    uint64_t noise = 0;
};

__device__ __forceinline__ uint32_t abs_diff(uint32_t a, uint32_t b) { return a > b ? a - b : b - a; }

__device__ __forceinline__ void add_dword(AccInt16 &a, uint32_t r, uint32_t d)
{
    const uint32_t e0 = abs_diff(r & 0xffffu, d & 0xffffu);
    const uint32_t e1 = abs_diff(r >> 16, d >> 16);
    a.noise += static_cast<uint64_t>(e0 * e0);
    a.noise += static_cast<uint64_t>(e1 * e1);
}

// ------------------------------------------------------------------ records
__device__ __forceinline__ void finish(const Acc8 &a, int64_t wg, uint64_t *part)
{
    const uint32_t v[5] = {a.r1, a.d1, a.r2, a.d2, a.rd};
    uint64_t s[5];
    workgroup_sums(v, s);
    const uint64_t rec[kSums] = {s[2] + s[3] - 2 * s[4], s[0], s[1], s[2], s[3]};
    write_record(part, wg, rec);
}

__device__ __forceinline__ void finish(const Acc16F64 &a, int64_t wg, uint64_t *part)
{
    const uint64_t n = lane_total(a.noise), r2 = lane_total(a.r2), d2 = lane_total(a.d2);
    const uint32_t v[8] = {static_cast<uint32_t>(n & 0xffffu), static_cast<uint32_t>(n >> 16), a.r1, a.d1,
                           static_cast<uint32_t>(r2 & 0xffffu), static_cast<uint32_t>(r2 >> 16),
                           static_cast<uint32_t>(d2 & 0xffffu), static_cast<uint32_t>(d2 >> 16)};
    uint64_t s[8];
    workgroup_sums(v, s);
    const uint64_t rec[kSums] = {s[0] + (s[1] << 16), s[2], s[3], s[4] + (s[5] << 16), s[6] + (s[7] << 16)};
    write_record(part, wg, rec);
}

__device__ __forceinline__ void finish(const AccInt8 &a, int64_t wg, uint64_t *part)
{
    const uint32_t v[3] = {a.r2, a.d2, a.rd};
    uint64_t s[3];
    workgroup_sums(v, s);
    const uint64_t rec[kSums] = {s[0] + s[1] - 2 * s[2], 0, 0, 0, 0};
    write_record(part, wg, rec);
}

__device__ __forceinline__ void finish(const AccInt16 &a, int64_t wg, uint64_t *part)
{
    const uint32_t v[2] = {static_cast<uint32_t>(a.noise & 0xffffu), static_cast<uint32_t>(a.noise >> 16)};
    uint64_t s[2];
    workgroup_sums(v, s);
    const uint64_t rec[kSums] = {s[0] + (s[1] << 16), 0, 0, 0, 0};
    write_record(part, wg, rec);
}

// ------------------------------------------------------------------- tiles
struct Tile {
    int y0, rows;  // rows [y0, y0 + rows)
    int x0, cw;    // columns [x0, x0 + cw)
};

__device__ __forceinline__ Tile tile_of(int t, int w, int h, int rows_per_tile, int seg, int segs)
{
    Tile T;
    if (rows_per_tile > 0) {
        T.y0 = t * rows_per_tile;
        T.rows = h - T.y0 < rows_per_tile ? h - T.y0 : rows_per_tile;
        T.x0 = 0;
        T.cw = w;
    } else {
        T.y0 = t / segs;
        T.rows = 1;
        T.x0 = (t - T.y0 * segs) * seg;
        T.cw = w - T.x0 < seg ? w - T.x0 : seg;
    }
    return T;
}

// Walks j = threadIdx.x, + kThreads, ... over a range laid out as rows of
// n items, keeping the item's column and, for each plane, the sample offset
// of its row from the tile's first row -- adds only, no multiply per step.
struct FlatWalk {
    int col, dcol, n;
    int64_t off_r, off_d, step_r, step_d, rs_r, rs_d;
    __device__ __forceinline__ FlatWalk(int start, int n_, int64_t rs_r_, int64_t rs_d_)
        : col(start % n_), dcol(kThreads % n_), n(n_), rs_r(rs_r_), rs_d(rs_d_)
    {
        const int row = start / n_, drow = kThreads / n_;
        off_r = row * rs_r;
        off_d = row * rs_d;
        step_r = drow * rs_r;
        step_d = drow * rs_d;
    }
    __device__ __forceinline__ void next()
    {
        off_r += step_r;
        off_d += step_d;
        col += dcol;
        if (col >= n) {
            col -= n;
            off_r += rs_r;
            off_d += rs_d;
        }
    }
};

template <int kBytes>
__device__ __forceinline__ const char *tile_base(const PlaneView &P, int64_t frame, int y, int x)
{
    return static_cast<const char *>(P.base) +
           (frame * P.frame_stride + static_cast<int64_t>(y) * P.row_stride + x) * kBytes;
}

template <int kBytes, class Acc>
__device__ __forceinline__ void add_samples(Acc &acc, const char *r, const char *d)
{
    add_dword(acc, load_sample<kBytes>(r, 0), load_sample<kBytes>(d, 0));
}

// The 16 bytes at byte offset 4Q + r (r in 0..3, 4Q + r in 1..15) of the 32
// bytes lo then hi.
template <int Q>
__device__ __forceinline__ u32x4 bytes_at(const u32x4 &lo, const u32x4 &hi, uint32_t r)
{
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u32x4 o;
    o.x = __builtin_amdgcn_alignbyte(d[Q + 1], d[Q + 0], r);
    o.y = __builtin_amdgcn_alignbyte(d[Q + 2], d[Q + 1], r);
    o.z = __builtin_amdgcn_alignbyte(d[Q + 3], d[Q + 2], r);
    o.w = __builtin_amdgcn_alignbyte(d[Q + 4], d[Q + 3], r);
    return o;
}

// A tile read row by row, for rows that start at different offsets within
// 16 bytes (an odd pitch) or ref and dist rows at different offsets, with
// dist's offset past ref's the same in every row.  In each row the samples
// before ref's first whole vector and after its last are read one by one,
// the whole vectors as vectors: ref's aligned, dist's the same (Q < 0) or
// cut from the two aligned blocks that hold them (bytes_at<Q>, shift rb;
// both blocks hold bytes of the row).  Work items (row, slot): the lane
// reads vector t + slot * kThreads of the row, for `slots` slots per row,
// four items at a time; a lane past the row's last vector reads its first
// and drops it.  Rows hold at least 32 vectors.
template <int kBytes, int Q, class Acc>
__device__ __forceinline__ void accumulate_rows(Acc &acc, const char *r0, const char *d0, int64_t rs_r, int64_t rs_d,
                                                const Tile &T, uint32_t rb)
{
    constexpr int V = 16 / kBytes;
    const int t = threadIdx.x;
    const int slots = (T.cw / V + kThreads - 1) / kThreads;
    // the row's first sample of whole ref vectors and its number of them
    auto row_vectors = [&](int y, int &head, int &nvec) {
        const int ph = static_cast<int>(reinterpret_cast<uintptr_t>(r0 + y * rs_r * kBytes) & 15);
        head = ((16 - ph) & 15) / kBytes;
        head = head < T.cw ? head : T.cw;
        nvec = (T.cw - head) / V;
    };
    for (int y = 0; y < T.rows; ++y) {
        int head, nvec;
        row_vectors(y, head, nvec);
        const int tail_begin = head + nvec * V;
        const int x = t < head ? t : tail_begin + (t - head);
        if (x < T.cw && (t < head || x >= tail_begin))
            add_samples<kBytes>(acc, r0 + (y * rs_r + x) * kBytes, d0 + (y * rs_d + x) * kBytes);
    }
    const int items = T.rows * slots;
    int y = 0, s = 0;
    for (int g = 0; g < items; g += 4) {
        u32x4 a[4], b[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int head, nvec;
            row_vectors(y, head, nvec);
            const int col = t + s * kThreads;
            ok[u] = g + u < items && col < nvec;
            const int64_t xr = y * rs_r + head + (ok[u] ? col : 0) * V;
            const int64_t xd = y * rs_d + head + (ok[u] ? col : 0) * V;
            a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(r0 + xr * kBytes));
            if constexpr (Q < 0) {
                b[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(d0 + xd * kBytes));
            } else {
                const u32x4 *db = reinterpret_cast<const u32x4 *>(reinterpret_cast<uintptr_t>(d0 + xd * kBytes) &
                                                                  ~static_cast<uintptr_t>(15));
                b[u] = bytes_at<Q>(__builtin_nontemporal_load(db), __builtin_nontemporal_load(db + 1), rb);
            }
            if (++s == slots) {
                s = 0;
                y = y + 1 < T.rows ? y + 1 : y;  // past the last item: stay on the last row
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 zero = {0, 0, 0, 0};
            add_vec(acc, ok[u] ? a[u] : zero, ok[u] ? b[u] : zero);
        }
    }
}

template <int kBytes, class Acc>
__device__ __forceinline__ void accumulate_tile(Acc &acc, const PlaneView &R, const PlaneView &D, int64_t frame,
                                                const Tile &T)
{
    constexpr int V = 16 / kBytes;
    const int t = threadIdx.x;
    const char *r0 = tile_base<kBytes>(R, frame, T.y0, T.x0);  // (x0, y0) of the tile
    const char *d0 = tile_base<kBytes>(D, frame, T.y0, T.x0);
    const int phase_r = static_cast<int>(reinterpret_cast<uintptr_t>(r0) & 15);
    const int phase_d = static_cast<int>(reinterpret_cast<uintptr_t>(d0) & 15);
    // every row of the tile starts at the same offset within 16 bytes
    const bool same_rows = T.rows == 1 || (((R.row_stride * kBytes) & 15) == 0 && ((D.row_stride * kBytes) & 15) == 0);
    if (same_rows && phase_r == phase_d) {
        int head = ((16 - phase_r) & 15) / kBytes;
        head = head < T.cw ? head : T.cw;
        const int nvec = (T.cw - head) / V;
        const int tail = T.cw - head - nvec * V;
        const int edges = head + tail;
        // the samples outside whole vectors, row by row
        if (edges > 0) {
            const int n = T.rows * edges;
            FlatWalk fw(t, edges, R.row_stride, D.row_stride);
            for (int s = t; s < n; s += kThreads, fw.next()) {
                const int x = fw.col < head ? fw.col : head + nvec * V + (fw.col - head);
                add_samples<kBytes>(acc, r0 + (fw.off_r + x) * kBytes, d0 + (fw.off_d + x) * kBytes);
            }
        }
        if (nvec == 0)
            return;
        // the whole vectors: one flat range across the rows, at most 8 per
        // lane, read in two groups of four; a lane past the end reads the
        // tile's first vector and drops it
        const char *rv = r0 + head * kBytes;
        const char *dv = d0 + head * kBytes;
        const int n = T.rows * nvec;
        FlatWalk fw(t, nvec, R.row_stride, D.row_stride);
#pragma unroll
        for (int g = 0; g < kTileVecs / kThreads; g += 4) {
            if (g * kThreads >= n)
                break;
            u32x4 a[4], b[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ok[u] = t + (g + u) * kThreads < n;
                const int64_t xr = ok[u] ? fw.off_r + fw.col * V : 0;
                const int64_t xd = ok[u] ? fw.off_d + fw.col * V : 0;
                a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rv + xr * kBytes));
                b[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(dv + xd * kBytes));
                fw.next();
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 zero = {0, 0, 0, 0};
                add_vec(acc, ok[u] ? a[u] : zero, ok[u] ? b[u] : zero);
            }
        }
    } else if ((((R.row_stride - D.row_stride) * kBytes) & 15) == 0 && T.cw >= 32 * V) {
        // rows at different offsets within 16 bytes, or ref and dist at
        // different ones (dist's past ref's the same in every row): row by row
        const uint32_t o = static_cast<uint32_t>(phase_d - phase_r) & 15u;
        const int64_t rs_r = R.row_stride, rs_d = D.row_stride;
        if (o == 0)
            accumulate_rows<kBytes, -1>(acc, r0, d0, rs_r, rs_d, T, 0u);
        else if (o < 4)
            accumulate_rows<kBytes, 0>(acc, r0, d0, rs_r, rs_d, T, o & 3u);
        else if (o < 8)
            accumulate_rows<kBytes, 1>(acc, r0, d0, rs_r, rs_d, T, o & 3u);
        else if (o < 12)
            accumulate_rows<kBytes, 2>(acc, r0, d0, rs_r, rs_d, T, o & 3u);
        else
            accumulate_rows<kBytes, 3>(acc, r0, d0, rs_r, rs_d, T, o & 3u);
    } else {
        // ref and dist rows drifting apart within 16 bytes, or narrow rows:
        // sample by sample
        const int n = T.rows * T.cw;
        FlatWalk fw(t, T.cw, R.row_stride, D.row_stride);
        for (int s = t; s < n; s += kThreads, fw.next())
            add_samples<kBytes>(acc, r0 + (fw.off_r + fw.col) * kBytes, d0 + (fw.off_d + fw.col) * kBytes);
    }
}

template <int kBytes, class Acc>
__global__ __launch_bounds__(kThreads) void view_stage1(PlaneView R, PlaneView D, int w, int h, int rows_per_tile,
                                                        int seg, int segs, int tiles, uint64_t *part)
{
    const int64_t wg = blockIdx.x;
    const int64_t frame = wg / tiles;
    const int t = static_cast<int>(wg - frame * tiles);
    Acc acc;
    accumulate_tile<kBytes>(acc, R, D, frame, tile_of(t, w, h, rows_per_tile, seg, segs));
    finish(acc, wg, part);
}

__global__ __launch_bounds__(kThreads) void view_combine(const uint64_t *part, int tiles, uint64_t *out_noise,
                                                         uint64_t *out_moments)
{
    combine_frame(part, tiles, blockIdx.x, out_noise, out_moments);
}

// ----------------------------------------------------------- several planes
// Up to kMaxViewPlanes planes of the same frames in one launch of each
// stage: the workgroups of plane p are [wg_begin[p], wg_begin[p+1]), frame
// by frame, tile by tile, as in the one-plane launch; the combine takes one
// workgroup per (plane, frame).  The descriptors travel as kernel
// arguments; a plane is picked by selects, never by indexing into them.
struct MultiViews {
    PlaneView R[kMaxViewPlanes], D[kMaxViewPlanes];
    int w[kMaxViewPlanes], h[kMaxViewPlanes];
    int rows_per_tile[kMaxViewPlanes], seg[kMaxViewPlanes], segs[kMaxViewPlanes], tiles[kMaxViewPlanes];
    int64_t wg_begin[kMaxViewPlanes + 1];
    int nplanes;
};

// Plane p's value among four, selected as values (a select of the array
// elements' addresses would make the compiler copy the descriptors to the
// stack).
template <class T>
__device__ __forceinline__ T pick4(T a, T b, T c, T d, int p)
{
    return p == 0 ? a : p == 1 ? b : p == 2 ? c : d;
}

__device__ __forceinline__ PlaneView pick_view(const PlaneView (&v)[kMaxViewPlanes], int p)
{
    static_assert(kMaxViewPlanes == 4, "one select per plane");
    PlaneView x;
    x.base = pick4(v[0].base, v[1].base, v[2].base, v[3].base, p);
    x.row_stride = pick4(v[0].row_stride, v[1].row_stride, v[2].row_stride, v[3].row_stride, p);
    x.frame_stride = pick4(v[0].frame_stride, v[1].frame_stride, v[2].frame_stride, v[3].frame_stride, p);
    return x;
}

#define VQX_PICK(arr, p) pick4((arr)[0], (arr)[1], (arr)[2], (arr)[3], (p))

template <int kBytes, class Acc>
__global__ __launch_bounds__(kThreads) void views_stage1(MultiViews M, uint64_t *part)
{
    const int64_t wg = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int q = 1; q < kMaxViewPlanes; ++q)
        p += q < M.nplanes && wg >= M.wg_begin[q] ? 1 : 0;
    const int64_t begin = VQX_PICK(M.wg_begin, p);
    const int tiles = VQX_PICK(M.tiles, p);
    const int64_t frame = (wg - begin) / tiles;
    const int t = static_cast<int>(wg - begin - frame * tiles);
    Acc acc;
    accumulate_tile<kBytes>(acc, pick_view(M.R, p), pick_view(M.D, p), frame,
                            tile_of(t, VQX_PICK(M.w, p), VQX_PICK(M.h, p), VQX_PICK(M.rows_per_tile, p),
                                    VQX_PICK(M.seg, p), VQX_PICK(M.segs, p)));
    finish(acc, wg, part);
}

__global__ __launch_bounds__(kThreads) void views_combine(MultiViews M, int nframes, const uint64_t *part,
                                                          uint64_t *out_noise, uint64_t *out_moments)
{
    const int p = static_cast<int>(blockIdx.x / nframes);
    const int64_t f = blockIdx.x - static_cast<int64_t>(p) * nframes;
    const int64_t begin = VQX_PICK(M.wg_begin, p);
    const int64_t at = static_cast<int64_t>(p) * nframes;
    combine_frame(part + begin * kRecordStride, VQX_PICK(M.tiles, p), f, out_noise + at,
                  out_moments ? out_moments + 4 * at : nullptr);
}

template <class Acc8T, class Acc16T>
hipError_t launch_multi(const ViewGeometry *g, const PlaneView *ref, const PlaneView *dist, int nplanes,
                        uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials, hipStream_t stream)
{
    MultiViews M{};
    M.nplanes = nplanes;
    int64_t at = 0;
    for (int p = 0; p < kMaxViewPlanes; ++p) {
        M.wg_begin[p] = at;
        if (p >= nplanes)
            continue;
        M.R[p] = ref[p];
        M.D[p] = dist[p];
        M.w[p] = g[p].w;
        M.h[p] = g[p].h;
        M.rows_per_tile[p] = g[p].rows_per_tile;
        M.seg[p] = g[p].seg_samples;
        M.segs[p] = g[p].segs_per_row;
        M.tiles[p] = g[p].tiles;
        at += g[p].workgroups;
    }
    M.wg_begin[kMaxViewPlanes] = at;
    const dim3 grid(static_cast<unsigned>(at));
    if (g[0].sample_bytes == 1)
        views_stage1<1, Acc8T><<<grid, kThreads, 0, stream>>>(M, partials);
    else
        views_stage1<2, Acc16T><<<grid, kThreads, 0, stream>>>(M, partials);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int nframes = g[0].nframes;
    views_combine<<<dim3(static_cast<unsigned>(nplanes * nframes)), kThreads, 0, stream>>>(M, nframes, partials,
                                                                                          out_noise, out_moments);
    return hipGetLastError();
}

// ------------------------------------------------------------------ gather
// Copies a view's samples into a contiguous [nframes][h][w] array: one
// workgroup per (frame, row) pair in turn, a grid of at most kGatherWgs
// workgroups.  Each row's whole 16-byte destination vectors are written
// whole (consecutive threads, consecutive vectors), the few samples before
// the first and after the last one by one.  The source bytes of a
// destination vector start at the same offset o within a 16-byte block for
// the whole row: where o is 0 the vector is copied as it is, otherwise it is
// cut from the two aligned blocks that hold it.  Those blocks each hold at
// least one byte of the row, so they lie in pages of the view.
constexpr int64_t kGatherWgs = 65536;

// Destination vectors 0..n-1 from the source blocks vs[0..n] at offset
// 4Q + r (> 0).
template <int Q>
__device__ __forceinline__ void copy_shifted(const u32x4 *vs, u32x4 *vd, int n, uint32_t r)
{
    for (int v = threadIdx.x; v < n; v += kThreads)
        vd[v] = bytes_at<Q>(vs[v], vs[v + 1], r);
}

template <int kBytes>
__global__ __launch_bounds__(kThreads) void gather_view(PlaneView P, int w, int h, int64_t rows, void *dst)
{
    using T = typename std::conditional<kBytes == 1, uint8_t, uint16_t>::type;
    const int t = threadIdx.x;
    for (int64_t fr = blockIdx.x; fr < rows; fr += gridDim.x) {
        const int64_t f = fr / h;
        const int64_t y = fr - f * h;
        const T *src = static_cast<const T *>(P.base) + f * P.frame_stride + y * P.row_stride;
        T *out = static_cast<T *>(dst) + fr * w;
        const uintptr_t sa = reinterpret_cast<uintptr_t>(src), oa = reinterpret_cast<uintptr_t>(out);
        const uintptr_t da = (oa + 15) & ~static_cast<uintptr_t>(15);
        const uintptr_t de = (oa + static_cast<uintptr_t>(w) * kBytes) & ~static_cast<uintptr_t>(15);
        if (da >= de) {  // no whole destination vector
            for (int x = t; x < w; x += kThreads)
                out[x] = src[x];
            continue;
        }
        const int head = static_cast<int>((da - oa) / kBytes);
        const int tail_begin = static_cast<int>((de - oa) / kBytes);
        if (t < head)
            out[t] = src[t];
        if (t < w - tail_begin)
            out[tail_begin + t] = src[tail_begin + t];
        const int n = static_cast<int>((de - da) / 16);
        const uintptr_t s0 = sa + (da - oa);  // source of the first destination vector
        const u32x4 *vs = reinterpret_cast<const u32x4 *>(s0 & ~static_cast<uintptr_t>(15));
        u32x4 *vd = reinterpret_cast<u32x4 *>(da);
        const uint32_t o = static_cast<uint32_t>(s0 & 15);
        switch (o >> 2) {
        case 0:
            if (o == 0) {
                for (int v = t; v < n; v += kThreads)
                    vd[v] = __builtin_nontemporal_load(vs + v);
            } else {
                copy_shifted<0>(vs, vd, n, o & 3);
            }
            break;
        case 1: copy_shifted<1>(vs, vd, n, o & 3); break;
        case 2: copy_shifted<2>(vs, vd, n, o & 3); break;
        default: copy_shifted<3>(vs, vd, n, o & 3); break;
        }
    }
}

template <class Acc8T, class Acc16T>
hipError_t launch_views(const ViewGeometry &g, const PlaneView &ref, const PlaneView &dist, uint64_t *out_noise,
                        uint64_t *out_moments, uint64_t *partials, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(g.workgroups));
    if (g.sample_bytes == 1)
        view_stage1<1, Acc8T><<<grid, kThreads, 0, stream>>>(ref, dist, g.w, g.h, g.rows_per_tile, g.seg_samples,
                                                             g.segs_per_row, g.tiles, partials);
    else
        view_stage1<2, Acc16T><<<grid, kThreads, 0, stream>>>(ref, dist, g.w, g.h, g.rows_per_tile, g.seg_samples,
                                                              g.segs_per_row, g.tiles, partials);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    view_combine<<<dim3(static_cast<unsigned>(g.nframes)), kThreads, 0, stream>>>(partials, g.tiles, out_noise,
                                                                                 out_moments);
    return hipGetLastError();
}

}  // namespace

ViewGeometry make_view_geometry(int w, int h, int bpc, int nframes)
{
    ViewGeometry g{};
    g.bpc = bpc;
    g.sample_bytes = bpc == 8 ? 1 : 2;
    g.w = w;
    g.h = h;
    g.nframes = nframes;
    const int tile_samples = kTileVecs * (16 / g.sample_bytes);
    if (w <= tile_samples) {
        g.rows_per_tile = tile_samples / w;
        g.seg_samples = w;
        g.segs_per_row = 1;
        g.tiles = (h + g.rows_per_tile - 1) / g.rows_per_tile;
    } else {
        g.rows_per_tile = 0;
        g.seg_samples = tile_samples;
        g.segs_per_row = (w + tile_samples - 1) / tile_samples;
        g.tiles = h * g.segs_per_row;
    }
    g.workgroups = static_cast<int64_t>(g.tiles) * nframes;
    g.workspace_bytes = static_cast<size_t>(g.workgroups) * kRecordStride * sizeof(uint64_t);
    return g;
}

hipError_t launch_view_stats(const ViewGeometry &g, const PlaneView &ref, const PlaneView &dist,
                             uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials, hipStream_t stream)
{
    return launch_views<Acc8, Acc16F64>(g, ref, dist, out_noise, out_moments, partials, stream);
}

hipError_t launch_view_psnr_int(const ViewGeometry &g, const PlaneView &ref, const PlaneView &dist,
                                uint64_t *out_noise, uint64_t *partials, hipStream_t stream)
{
    return launch_views<AccInt8, AccInt16>(g, ref, dist, out_noise, nullptr, partials, stream);
}

hipError_t launch_gather_view(const PlaneView &view, int w, int h, int bpc, int nframes, void *dst,
                              hipStream_t stream)
{
    const int64_t rows = static_cast<int64_t>(nframes) * h;
    const dim3 grid(static_cast<unsigned>(rows < kGatherWgs ? rows : kGatherWgs));
    if (bpc == 8)
        gather_view<1><<<grid, kThreads, 0, stream>>>(view, w, h, rows, dst);
    else
        gather_view<2><<<grid, kThreads, 0, stream>>>(view, w, h, rows, dst);
    return hipGetLastError();
}

hipError_t launch_planes_stats(const ViewGeometry *g, const PlaneView *ref, const PlaneView *dist, int nplanes,
                               uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials, hipStream_t stream)
{
    return launch_multi<Acc8, Acc16F64>(g, ref, dist, nplanes, out_noise, out_moments, partials, stream);
}

hipError_t launch_planes_psnr_int(const ViewGeometry *g, const PlaneView *ref, const PlaneView *dist, int nplanes,
                                  uint64_t *out_noise, uint64_t *partials, hipStream_t stream)
{
    return launch_multi<AccInt8, AccInt16>(g, ref, dist, nplanes, out_noise, nullptr, partials, stream);
}

}  // namespace vqx
