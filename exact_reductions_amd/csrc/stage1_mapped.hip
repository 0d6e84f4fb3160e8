// Stage 1 over plane views read in place, for gfx950: the exact sums, and
// the CPU-order form of them.
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
//
// The CPU adds a view's samples in raster order whatever its pitch [PSNR,
// Context; MOMENT, Context], so the chunks of a view are those of the same
// frames stored contiguously.  Where the view's rows are whole 16-byte
// vectors of two-byte samples (16-byte aligned, or for the CPU-order form
// all at one offset within 16 bytes), this kernel reads vector v of that
// contiguous order where the view keeps it (map_vec) and writes the records
// the contiguous stage 1 writes for the same samples -- with the low bits of
// the terms in the CPU-order form -- from the same terms in the same lane
// accumulators and workgroup sums.  Integer sums make the records, and so
// the frame sums, those of the contiguous planes.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "plane_stats.h"
#include "reduce.h"
#include "terms.h"

#pragma clang fp contract(off)

namespace vqx {
namespace {

constexpr int kLaneIters = kChunkVectors / kThreads;  // vectors per lane per plane
constexpr int kInFlight = 4;                          // vectors of each plane loaded before use
static_assert(kLaneIters % kInFlight == 0, "whole load groups");

// Stage 1 over plane views whose rows are whole 16-byte vectors
// (two-byte samples, so frames hold no partial vectors): the same chunks,
// terms and records as stage1_u16<kLowBitsOut>, each vector found through
// the VecMap; kLowBitsOut: also the low bits of the terms and zero item
// tickets, for the CPU-order form; kForm: where the planes' vectors start
// within 16-byte blocks -- all at 0 (kAligned: one 16-byte load per vector,
// found with the map's pads), at multiples of 4 bytes (kDword: ref and dist
// the bases rounded down to 16 bytes, each vector found with the map's byte
// strides and read with one dword-aligned 16-byte load), or anywhere (kCut:
// the same, each vector cut from dword-aligned loads).
enum : int { kAligned = 0, kCut = 1, kDword = 2 };

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// The 16 bytes at byte offset `at` (a multiple of 4) from P, in one load,
// non-temporal as every other read of the terms.
__device__ __forceinline__ u32x4 load_vec16_dword(const u32x4 *P, uint32_t at)
{
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_a4 *>(reinterpret_cast<const unsigned char *>(P) + at));
}

template <bool kLowBitsOut, int kForm>
__global__ __launch_bounds__(kThreads) void stage1_u16_mapped(const void *ref, const void *dist, int64_t pixels,
                                                              int chunks, uint64_t *part, VecMap M)
{
    const int64_t wg = blockIdx.x;
    const int64_t frame = wg / chunks;
    const int chunk = static_cast<int>(wg - frame * chunks);
    const u32x4 *R = static_cast<const u32x4 *>(ref);
    const u32x4 *D = static_cast<const u32x4 *>(dist);
    const int64_t vb = frame * (pixels / 8), ve = vb + pixels / 8;
    const int64_t cb = vb + static_cast<int64_t>(chunk) * kChunkVectors;
    const int64_t ce = cb + kChunkVectors < ve ? cb + kChunkVectors : ve;
    // map_vec written out for this frame: vector v of the frame's contiguous
    // order lies in row y = (r * magic) >> shift, r = v - vb < 2^22, and
    // magic < 2^24, so the product fits 64 bits from 32-bit factors
    const int64_t fr = frame * M.pad_frame_r, fd = frame * M.pad_frame_d;
    const uint32_t magic = static_cast<uint32_t>(M.magic);
    // general maps: each plane's frame from the 16-byte block that holds its
    // first byte (Rf, Df), and 32-bit byte offsets from there (a frame's
    // rows span less than 2^31 bytes on this path)
    const int64_t fbr = M.phase_r + frame * M.frame_bytes_r, fbd = M.phase_d + frame * M.frame_bytes_d;
    const u32x4 *Rf = R + (fbr >> 4), *Df = D + (fbd >> 4);
    const uint32_t lor = static_cast<uint32_t>(fbr & 15), lod = static_cast<uint32_t>(fbd & 15);
    const uint32_t rbr = static_cast<uint32_t>(M.row_bytes_r), rbd = static_cast<uint32_t>(M.row_bytes_d);
    typename std::conditional<kLowBitsOut, Acc16Low, Acc16F64>::type a;
    if (cb < ce) {
#pragma unroll 1
        for (int i = 0; i < kLaneIters; i += kInFlight) {
            u32x4 x[kInFlight], y[kInFlight];
            bool ok[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int64_t v0 = cb + threadIdx.x + static_cast<int64_t>(i + u) * kThreads;
                ok[u] = v0 < ce;
                const int64_t v = ok[u] ? v0 : cb;
                const uint32_t r = static_cast<uint32_t>(v - vb);
                const int64_t row = static_cast<int64_t>((static_cast<uint64_t>(r) * magic) >> M.shift);
                if constexpr (kForm == kAligned) {
                    const int64_t ar = v + fr + row * M.pad_row_r, ad = v + fd + row * M.pad_row_d;
                    x[u] = __builtin_nontemporal_load(R + ar);
                    y[u] = __builtin_nontemporal_load(D + ad);
                } else if constexpr (kForm == kDword) {
                    const uint32_t yr = static_cast<uint32_t>(row);
                    const uint32_t x16 = 16 * (r - yr * M.vpr);
                    x[u] = load_vec16_dword(Rf, lor + yr * rbr + x16);
                    y[u] = load_vec16_dword(Df, lod + yr * rbd + x16);
                } else {
                    const uint32_t yr = static_cast<uint32_t>(row);
                    const uint32_t x16 = 16 * (r - yr * M.vpr);
                    x[u] = load_vec16_at(Rf, lor + yr * rbr + x16);
                    y[u] = load_vec16_at(Df, lod + yr * rbd + x16);
                }
            }
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const u32x4 zero = {0, 0, 0, 0};
                add_vec(a, ok[u] ? x[u] : zero, ok[u] ? y[u] : zero);
            }
        }
    }
    const uint64_t n = lane_total(a.noise), r2 = lane_total(a.r2), d2 = lane_total(a.d2);
    const uint32_t v[8] = {static_cast<uint32_t>(n & 0xffffu), static_cast<uint32_t>(n >> 16), a.r1, a.d1,
                           static_cast<uint32_t>(r2 & 0xffffu), static_cast<uint32_t>(r2 >> 16),
                           static_cast<uint32_t>(d2 & 0xffffu), static_cast<uint32_t>(d2 >> 16)};
    uint64_t s[8];
    workgroup_sums(v, s);
    const uint64_t rec[kSums] = {s[0] + (s[1] << 16), s[2], s[3], s[4] + (s[5] << 16), s[6] + (s[7] << 16)};
    write_record(part, wg, rec);
    if constexpr (kLowBitsOut) {
        const uint32_t low = workgroup_or((a.or_noise & 15u) | ((a.or_r2 & 15u) << 4) | ((a.or_d2 & 15u) << 8));
        if (threadIdx.x == 0) {
            part[wg * kRecordStride + kLowBits] = low;
            if (chunk == 0) {
                part[wg * kRecordStride + kTickets] = 0;
                part[wg * kRecordStride + kTickets + 1] = 0;
            }
        }
    }
}

// One workgroup per frame adds the frame's records in uint64.
__global__ __launch_bounds__(kThreads) void mapped_combine(const uint64_t *part, int chunks, uint64_t *out_noise,
                                                           uint64_t *out_moments)
{
    combine_frame(part, chunks, blockIdx.x, out_noise, out_moments);
}

}  // namespace

hipError_t launch_stage1_mapped(const Geometry &g, const void *ref, const void *dist, uint64_t *partials,
                                const VecMap &map, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(g.workgroups));
    if (!map.general)
        stage1_u16_mapped<true, kAligned><<<grid, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, partials,
                                                                        map);
    else if (((map.phase_r | map.phase_d) & 3u) == 0 &&
             ((map.row_bytes_r | map.row_bytes_d | map.frame_bytes_r | map.frame_bytes_d) & 3) == 0)
        // every vector starts at a multiple of 4 bytes from its base
        stage1_u16_mapped<true, kDword><<<grid, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, partials, map);
    else
        stage1_u16_mapped<true, kCut><<<grid, kThreads, 0, stream>>>(ref, dist, g.pixels, g.chunks, partials, map);
    return hipGetLastError();
}

hipError_t launch_plane_stats_mapped(const Geometry &g, const void *ref, const void *dist, uint64_t *out_noise,
                                     uint64_t *out_moments, uint64_t *partials, const VecMap &map,
                                     hipStream_t stream)
{
    if (map.general)
        return hipErrorInvalidValue;  // whole aligned vectors only
    stage1_u16_mapped<false, kAligned><<<dim3(static_cast<unsigned>(g.workgroups)), kThreads, 0, stream>>>(
        ref, dist, g.pixels, g.chunks, partials, map);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    mapped_combine<<<dim3(static_cast<unsigned>(g.nframes)), kThreads, 0, stream>>>(partials, g.chunks, out_noise,
                                                                                   out_moments);
    return hipGetLastError();
}

}  // namespace vqx
