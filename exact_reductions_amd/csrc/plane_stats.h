// Launch geometry and launcher of the plane-stats kernels (internal to libvqx).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqx {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Number of 64-bit sums in one partial record, in this order.
enum : int { kNoise = 0, kRef1 = 1, kDist1 = 2, kRef2 = 3, kDist2 = 4, kSums = 5 };

// 16-byte vectors of each plane per chunk (one stage-1 workgroup each).
constexpr int kChunkVectors = 2048;

// A workgroup's partial record occupies its own 64-byte slot (8 uint64, 5
// used), so that no two workgroups write the same cache line.
constexpr int kRecordStride = 8;

// Slot kLowBits of a record, written by the stage 1 of the CPU-order form
// only (two-byte samples): the OR of the low 4 bits of the workgroup's
// terms of each square sum -- noise in bits 0..3, ref^2 in 4..7, dist^2 in
// 8..11.
constexpr int kLowBits = 5;

// Slots kTickets and kTickets + 1 of the record of each frame's chunk 0
// hold three uint32 counters (noise, ref^2, dist^2) from which the
// CPU-order form's maps kernel hands out slab items; its stage 1 zeroes
// them.
constexpr int kTickets = 6;


// Work split of one batch.  Each plane is read as 16-byte vectors; the
// vectors of a frame that lie wholly inside it are cut into chunks of
// chunk_vecs vectors, one workgroup per (frame, chunk).  The few samples of a
// frame before its first whole vector and after its last (frames need not
// start on a 16-byte boundary) are taken by chunk 0.
struct Geometry {
    int bpc;
    int sample_bytes;     // 1 (uint8, bpc 8) or 2 (uint16)
    int vec_elems;        // samples per 16-byte vector
    int64_t pixels;       // w*h
    int nframes;
    int chunk_vecs;       // 16-byte vectors per plane per workgroup
    int chunks;           // workgroups per frame
    int64_t workgroups;   // nframes * chunks
    size_t workspace_bytes;
};

Geometry make_geometry(int w, int h, int bpc, int nframes);

// Work-items per workgroup of the launches over (frame, chunk).
constexpr int kChunkThreads = 256;

// A dispatch counts its work-items in 32 bits.  The widest launch of every
// entry point is stage 1's (or its view form's), one workgroup per (frame,
// chunk).
inline bool fits_dispatch(const Geometry &g)
{
    return g.workgroups * kChunkThreads <= static_cast<int64_t>(0xffffffffu);
}

// Stage 1's grid and loads with no arithmetic (measurement only); the
// dispatch stamps `begin` and `end`, either of which may be null.
hipError_t launch_read_probe(const Geometry &g, const void *ref, const void *dist, uint64_t *partials,
                             hipStream_t stream, hipEvent_t begin, hipEvent_t end);

// Queues both stages on `stream`, recording `stage1_begin`/`stage1_end` (if
// not null) around stage 1; with both outputs null, stage 1 only (the
// caller combines the records).  Returns hipSuccess or the first error.
hipError_t launch_plane_stats(const Geometry &g, const void *ref, const void *dist,
                              uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials,
                              hipStream_t stream, hipEvent_t stage1_begin = nullptr,
                              hipEvent_t stage1_end = nullptr, bool low_bits = false);

// A plane of every frame of a batch, addressed sample by sample: sample
// (x, y) of frame f is at base + (f*frame_stride + y*row_stride + x) samples.
struct PlaneView {
    const void *base;
    int64_t row_stride;    // samples, >= w
    int64_t frame_stride;  // samples, >= 0
};

// Work split of the view kernels: one workgroup per (frame, tile).  A tile
// is rows_per_tile whole rows, or (rows_per_tile == 0, for rows longer than
// one tile) a segment of seg_samples samples of one row.
struct ViewGeometry {
    int bpc;
    int sample_bytes;
    int w, h, nframes;
    int rows_per_tile;
    int seg_samples, segs_per_row;
    int tiles;            // per frame
    int64_t workgroups;   // nframes * tiles
    size_t workspace_bytes;
};

ViewGeometry make_view_geometry(int w, int h, int bpc, int nframes);

// The five sums of every frame over plane views (stage 1 over tiles, then
// the per-frame combine); out_moments may be null for the noise only.
hipError_t launch_view_stats(const ViewGeometry &g, const PlaneView &ref, const PlaneView &dist,
                             uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials,
                             hipStream_t stream);

// The integer psnr noise, sum of (ref - dist)^2 in exact integers, of
// every frame over plane views.
hipError_t launch_view_psnr_int(const ViewGeometry &g, const PlaneView &ref, const PlaneView &dist,
                                uint64_t *out_noise, uint64_t *partials, hipStream_t stream);

// Copies a view's samples into a contiguous [nframes][h][w] array at `dst`
// (uint8 at 8 bits, else uint16).
hipError_t launch_gather_view(const PlaneView &view, int w, int h, int bpc, int nframes, void *dst,
                              hipStream_t stream);

// Several planes of the same frames (same bpc and nframes, each with its
// own geometry, made by make_view_geometry) in one launch of each stage:
// out_noise[p][f], out_moments[p][f][4]; the workspace holds every plane's
// records, plane after plane.
constexpr int kMaxViewPlanes = 4;
hipError_t launch_planes_stats(const ViewGeometry *g, const PlaneView *ref, const PlaneView *dist, int nplanes,
                               uint64_t *out_noise, uint64_t *out_moments, uint64_t *partials, hipStream_t stream);
hipError_t launch_planes_psnr_int(const ViewGeometry *g, const PlaneView *ref, const PlaneView *dist, int nplanes,
                                  uint64_t *out_noise, uint64_t *partials, hipStream_t stream);

// Workspace of the host-fed form: two staging slots (ref and dist planes of
// frames_per_upload frames each) and the stage-1 records of one sub-batch.
struct HostStreamLayout {
    size_t plane_bytes;  // one plane of frames_per_upload frames
    size_t ref[2], dist[2], partials, bytes;
};
HostStreamLayout host_stream_layout(int w, int h, int bpc, int frames_per_upload);

// Uploads the batch from host memory in sub-batches on `copy` while
// reducing earlier sub-batches on `compute`; returns when all is done.
hipError_t run_host_stream(int w, int h, int bpc, int nframes, int frames_per_upload, const void *ref_host,
                           const void *dist_host, uint64_t *out_noise, uint64_t *out_moments, void *workspace,
                           hipStream_t compute, hipStream_t copy);

// Workspace of the CPU-order form: byte offsets of its parts.
struct CpuOrderLayout {
    size_t records, queue, totals, maps, cmaps, bmaps, bytes;
};
CpuOrderLayout cpu_order_layout(const Geometry &g);

// Where the kernels that read plane views in place (the mapped stage 1, the
// CPU-order maps and walk) find a batch's 16-byte vectors.  They index them
// as if the batch were one contiguous [nframes][h][w] array (index v);
// a pair of plane views whose rows are whole 16-byte vectors maps v
// of frame f to v + f*pad_frame + y*pad_row (in vectors) for each plane, y
// the row of v in its frame.  vpr == 0: contiguous planes, v itself.
struct VecMap {
    uint32_t vpr = 0;        // vectors per row
    int64_t frame_vecs = 0;  // vectors per frame, h * vpr
    uint64_t magic = 0;      // y = (r * magic) >> shift for r < 2^22
    int shift = 0;
    int64_t pad_row_r = 0, pad_frame_r = 0, pad_row_d = 0, pad_frame_d = 0;
    // general != 0: some vector does not start on a 16-byte boundary.  The
    // kernels then take each plane's base rounded down to 16 bytes and find
    // vector (f, y, x) at byte phase + f*frame_bytes + y*row_bytes + 16*x
    // from there.
    uint32_t general = 0;
    uint32_t phase_r = 0, phase_d = 0;
    int64_t row_bytes_r = 0, frame_bytes_r = 0, row_bytes_d = 0, frame_bytes_d = 0;
};

// The 16 bytes at byte offset `at` (even, >= 0) from P, a 16-byte aligned
// base: the four dwords from the dword that holds the first byte (one
// dword-aligned load), then the dword after them where `at` is not a
// multiple of 4 (else the last of the four again), and each dword of the
// result cut from two neighbours with v_alignbyte.  Every dword read holds
// a byte of the vector, so no read leaves the 16-byte blocks that hold it.
__device__ __forceinline__ u32x4_t load_vec16_at(const u32x4_t *P, int64_t at)
{
    const uint32_t *d = reinterpret_cast<const uint32_t *>(P) + (at >> 2);
    const uint32_t r = static_cast<uint32_t>(at & 3);  // 0 or 2
    u32x4_t lo;
    __builtin_memcpy(&lo, d, sizeof(lo));
    const uint32_t hi = d[r ? 4 : 3];
    u32x4_t o;
    o.x = __builtin_amdgcn_alignbyte(lo.y, lo.x, r);
    o.y = __builtin_amdgcn_alignbyte(lo.z, lo.y, r);
    o.z = __builtin_amdgcn_alignbyte(lo.w, lo.z, r);
    o.w = __builtin_amdgcn_alignbyte(hi, lo.w, r);
    return o;
}

// Byte offset of vector v (index in the batch's contiguous order) of frame
// `frame` in each plane, from the bases rounded down (general maps, whose
// frames span less than 2^31 bytes, so offsets inside a frame are 32-bit).
__device__ __forceinline__ void map_vec_bytes(const VecMap &M, int64_t frame, int64_t v, int64_t &br, int64_t &bd)
{
    const uint32_t r = static_cast<uint32_t>(v - frame * M.frame_vecs);  // below 2^22
    const uint32_t y = static_cast<uint32_t>((static_cast<uint64_t>(r) * M.magic) >> M.shift);
    const uint32_t x16 = 16 * (r - y * M.vpr);
    br = M.phase_r + frame * M.frame_bytes_r + (y * static_cast<uint32_t>(M.row_bytes_r) + x16);
    bd = M.phase_d + frame * M.frame_bytes_d + (y * static_cast<uint32_t>(M.row_bytes_d) + x16);
}

// The VecMap of two views of w x h planes (two-byte samples) at `ref` and
// `dist` (two-byte aligned), strides in samples; the caller has checked
// that rows are whole vectors (w a multiple of 8).  Where `general` is set
// the kernels take the bases rounded down to 16 bytes (vec_base).
VecMap make_vec_map(int w, int h, const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                    const void *dist, int64_t dist_row_stride, int64_t dist_frame_stride);

inline const void *vec_base(const void *p)
{
    return reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(p) & ~static_cast<uintptr_t>(15));
}

__device__ __forceinline__ void map_vec(const VecMap &M, int64_t frame, int64_t v, int64_t &vr, int64_t &vd)
{
    vr = vd = v;
    if (M.vpr == 0)
        return;
    const uint64_t r = static_cast<uint64_t>(v - frame * M.frame_vecs);  // below 2^22
    const int64_t y = static_cast<int64_t>((r * M.magic) >> M.shift);
    vr += frame * M.pad_frame_r + y * M.pad_row_r;
    vd += frame * M.pad_frame_d + y * M.pad_row_d;
}

// Stage 1, then the kernels that reproduce the CPU's running double sums
// (cpu_order.hip): the exact sums, and out_cpu_noise[F] and
// out_cpu_moments[F][4] in the same units.  `map`: where the vectors lie
// (two-byte samples only; contiguous by default).
hipError_t launch_plane_stats_cpu_order(const Geometry &g, const void *ref, const void *dist,
                                        uint64_t *out_noise, uint64_t *out_moments,
                                        uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                        void *workspace, hipStream_t stream, const VecMap &map = VecMap{});

// The CPU-order form of stage 1 (two-byte samples, the low bits of the
// terms too) with its vectors found through `map`.
hipError_t launch_stage1_mapped(const Geometry &g, const void *ref, const void *dist, uint64_t *partials,
                                const VecMap &map, hipStream_t stream);

// The five exact sums of views whose rows are whole 16-byte aligned vectors
// of two-byte samples: stage 1 with its vectors found through `map`, then
// the per-frame combine; `partials` as for launch_plane_stats.
hipError_t launch_plane_stats_mapped(const Geometry &g, const void *ref, const void *dist, uint64_t *out_noise,
                                     uint64_t *out_moments, uint64_t *partials, const VecMap &map,
                                     hipStream_t stream);

// The running float sum (float_sum.hip): buffers of float32 terms, each
// summed in order into one binary32 accumulator.  Tiles of kFsTileTerms
// terms, one workgroup of kFsThreads threads each, kFsRunTerms per thread.
constexpr int kFsThreads = 256;
constexpr int kFsRunTerms = 16;
constexpr int kFsTileTerms = kFsThreads * kFsRunTerms;

// Workspace of the running float sums: byte offsets of its parts.
struct FloatSumLayout {
    int ntiles;  // per buffer
    size_t totals, bad, recs, buffer_bad, done, ordered, bytes;
};
FloatSumLayout float_sum_layout(int64_t nterms, int nbuffers);

// A second stream on the device, with two events, on which the walk runs
// while the tile maps are still being made (fork: after the plan; join:
// the caller's stream waits for the walk).  The caller keeps other users
// off it for the length of one launch_float_sums call.
struct SideStream {
    hipStream_t stream;
    hipEvent_t fork, join;
};

// nbuffers buffers of nterms float32 terms each, one after another at
// `terms`; out[k] gets buffer k's running sum (NaN if a term is negative or
// not finite).  side may be null: then the walk follows the maps on
// `stream` alone.
hipError_t launch_float_sums(const float *terms, int64_t nterms, int nbuffers, float *out, void *workspace,
                             hipStream_t stream, const SideStream *side);

}  // namespace vqx
