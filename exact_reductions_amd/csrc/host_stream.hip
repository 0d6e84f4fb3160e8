// Host-fed batches: the planes arrive in host memory and are uploaded in
// sub-batches while earlier sub-batches are reduced (host code only).
//
// Sources (web pages, cited by title and section):
//   [ADM] "ADR-1423: adm_hip takes its weights, shifts and score conclusion
//         from the CPU, folds the denominator once per row and clears its
//         accumulators after the upload" -- Decision: per frame the tool
//         uploads the luma planes, then queues the twin's work after the
//         upload on the same stream.
//
// Here the upload and the reduction run on two streams so that they
// overlap: two device staging slots alternate; sub-batch k's copies wait
// (on the copy stream) until the reduction of sub-batch k - 2, which used
// the same slot, is done, and its reduction waits (on the compute stream)
// for its copies.  Every stream keeps the default priority.  Nothing is
// cleared: stage 2 writes each frame's sums once, into the caller's output
// at the frame's place.

#include <hip/hip_runtime.h>

#include "plane_stats.h"

namespace vqx {

HostStreamLayout host_stream_layout(int w, int h, int bpc, int frames_per_upload)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const Geometry g = make_geometry(w, h, bpc, frames_per_upload);
    HostStreamLayout l{};
    l.plane_bytes = static_cast<size_t>(g.pixels) * g.sample_bytes * frames_per_upload;
    size_t at = 0;
    for (int s = 0; s < 2; ++s) {
        l.ref[s] = at;
        at = up(at + l.plane_bytes);
        l.dist[s] = at;
        at = up(at + l.plane_bytes);
    }
    l.partials = at;
    l.bytes = up(at + g.workspace_bytes);
    return l;
}

hipError_t run_host_stream(int w, int h, int bpc, int nframes, int frames_per_upload, const void *ref_host,
                           const void *dist_host, uint64_t *out_noise, uint64_t *out_moments, void *workspace,
                           hipStream_t compute, hipStream_t copy)
{
    const HostStreamLayout l = host_stream_layout(w, h, bpc, frames_per_upload);
    char *ws = static_cast<char *>(workspace);
    const size_t frame_bytes = l.plane_bytes / static_cast<size_t>(frames_per_upload);
    hipEvent_t uploaded[2] = {nullptr, nullptr}, reduced[2] = {nullptr, nullptr};
    hipError_t err = hipSuccess;
    for (int s = 0; s < 2 && err == hipSuccess; ++s) {
        err = hipEventCreateWithFlags(&uploaded[s], hipEventDisableTiming);
        if (err == hipSuccess)
            err = hipEventCreateWithFlags(&reduced[s], hipEventDisableTiming);
    }
    // the copy stream starts after what the caller queued on the compute
    // stream before this call (the outputs may be in use there)
    hipEvent_t start = nullptr;
    if (err == hipSuccess)
        err = hipEventCreateWithFlags(&start, hipEventDisableTiming);
    if (err == hipSuccess)
        err = hipEventRecord(start, compute);
    if (err == hipSuccess)
        err = hipStreamWaitEvent(copy, start, 0);
    const char *rh = static_cast<const char *>(ref_host);
    const char *dh = static_cast<const char *>(dist_host);
    for (int f0 = 0, k = 0; f0 < nframes && err == hipSuccess; f0 += frames_per_upload, ++k) {
        const int n = nframes - f0 < frames_per_upload ? nframes - f0 : frames_per_upload;
        const int s = k & 1;
        const size_t bytes = frame_bytes * static_cast<size_t>(n);
        // the slot is free once the reduction that last read it is done
        if (k >= 2)
            err = hipStreamWaitEvent(copy, reduced[s], 0);
        if (err == hipSuccess)
            err = hipMemcpyAsync(ws + l.ref[s], rh + frame_bytes * static_cast<size_t>(f0), bytes,
                                 hipMemcpyHostToDevice, copy);
        if (err == hipSuccess)
            err = hipMemcpyAsync(ws + l.dist[s], dh + frame_bytes * static_cast<size_t>(f0), bytes,
                                 hipMemcpyHostToDevice, copy);
        if (err == hipSuccess)
            err = hipEventRecord(uploaded[s], copy);
        if (err == hipSuccess)
            err = hipStreamWaitEvent(compute, uploaded[s], 0);
        if (err == hipSuccess)
            err = launch_plane_stats(make_geometry(w, h, bpc, n), ws + l.ref[s], ws + l.dist[s], out_noise + f0,
                                     out_moments + 4 * static_cast<size_t>(f0),
                                     reinterpret_cast<uint64_t *>(ws + l.partials), compute);
        if (err == hipSuccess)
            err = hipEventRecord(reduced[s], compute);
    }
    // the host buffers are the caller's again only when every copy is done,
    // and the sums are ready when the compute stream is
    const hipError_t sync_copy = hipStreamSynchronize(copy);
    const hipError_t sync_compute = hipStreamSynchronize(compute);
    if (err == hipSuccess)
        err = sync_copy != hipSuccess ? sync_copy : sync_compute;
    for (int s = 0; s < 2; ++s) {
        if (uploaded[s])
            (void)hipEventDestroy(uploaded[s]);
        if (reduced[s])
            (void)hipEventDestroy(reduced[s]);
    }
    if (start)
        (void)hipEventDestroy(start);
    return err;
}

}  // namespace vqx
