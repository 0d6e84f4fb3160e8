// C ABI of libvqx: argument checks, workspace, launches and the host-side
// conclusions.  Declarations and argument contracts are in include/vqx.h.
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "plane_stats.h"
#include "terms.h"
#include "vqx.h"

#pragma clang fp contract(off)

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by every entry point; no device call.
int check_shape(int w, int h, int bpc)
{
    if (w < 1 || h < 1 || static_cast<int64_t>(w) * h > VQX_MAX_PIXELS)
        return VQX_E_DIMS;
    if (bpc < 8 || bpc > 16)
        return VQX_E_BPC;
    return VQX_OK;
}

int check_batch(int w, int h, int bpc, int nframes)
{
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    if (nframes < 1)
        return VQX_E_NFRAMES;
    // every launch must fit one dispatch
    if (!vqx::fits_dispatch(vqx::make_geometry(w, h, bpc, nframes)))
        return VQX_E_NFRAMES;
    return VQX_OK;
}

// All argument checks of the plane-stats entry points, in a fixed order.
int check_stats_args(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                     const uint64_t *out_noise, const uint64_t *out_moments)
{
    if (!ref || !dist || !out_noise || !out_moments)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    if (!aligned(ref, 16) || !aligned(dist, 16) || !aligned(out_noise, 8) || !aligned(out_moments, 8))
        return VQX_E_ALIGN;
    return VQX_OK;
}

int device_ready()
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return VQX_E_NO_DEVICE;
    }
    return VQX_OK;
}

// (double)v rounds to nearest even, and only once v passes 2^53 [MOMENT,
// Decision]; the divisions by s^k are by powers of two and exact.
double unit_mean(uint64_t v, int power, int bpc, int64_t pixels)
{
    const double s = static_cast<double>(1 << (bpc - 8));
    const double scale = power == 2 ? s * s : s;
    return (static_cast<double>(v) / scale) / static_cast<double>(pixels);
}

// ------------------------------------------------------------ plane views
int check_view_batch(int w, int h, int bpc, int nframes)
{
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    if (nframes < 1)
        return VQX_E_NFRAMES;
    const vqx::ViewGeometry g = vqx::make_view_geometry(w, h, bpc, nframes);
    if (g.workgroups * vqx::kChunkThreads > static_cast<int64_t>(0xffffffffu))
        return VQX_E_NFRAMES;
    return VQX_OK;
}

// A view's last sample, (nframes-1)*frame_stride + (h-1)*row_stride + w - 1
// samples past its base, must lie within 2^62 bytes; each product is
// bounded before it is formed.
bool view_extent_ok(int64_t row_stride, int64_t frame_stride, int w, int h, int nframes, int bytes)
{
    if (row_stride < w || frame_stride < 0)
        return false;
    const int64_t limit = (static_cast<int64_t>(1) << 62) / bytes;  // in samples
    if (h > 1 && row_stride > limit / (h - 1))
        return false;
    if (nframes > 1 && frame_stride > limit / (nframes - 1))
        return false;
    const int64_t rows = static_cast<int64_t>(h - 1) * row_stride;
    const int64_t frames = static_cast<int64_t>(nframes - 1) * frame_stride;
    return rows <= limit - w && frames <= limit - w - rows;
}

int check_view_args(const void *ref, int64_t rrs, int64_t rfs, const void *dist, int64_t drs, int64_t dfs, int w,
                    int h, int bpc, int nframes, const uint64_t *out_noise, const uint64_t *out_moments,
                    bool need_moments)
{
    if (!ref || !dist || !out_noise || (need_moments && !out_moments))
        return VQX_E_NULL;
    int rc = check_view_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    const int bytes = bpc == 8 ? 1 : 2;
    if (!view_extent_ok(rrs, rfs, w, h, nframes, bytes) || !view_extent_ok(drs, dfs, w, h, nframes, bytes))
        return VQX_E_STRIDE;
    if (!aligned(ref, bytes) || !aligned(dist, bytes) || !aligned(out_noise, 8) ||
        (need_moments && !aligned(out_moments, 8)))
        return VQX_E_ALIGN;
    return VQX_OK;
}

double psnr_from_mse(double mse, int bpc, double psnr_max)
{
    if (mse == 0.0)
        return psnr_max > 0.0 ? psnr_max : HUGE_VAL;
    const double peak = static_cast<double>((1 << bpc) - 1) / static_cast<double>(1 << (bpc - 8));
    const double db = 10.0 * log10(peak * peak / mse);
    return (psnr_max > 0.0 && db > psnr_max) ? psnr_max : db;
}

static_assert(VQX_MAX_PLANES == vqx::kMaxViewPlanes, "one plane limit");

// Checks the planes and fills their geometries and views; `launch`: also
// the pointers, strides and outputs of a call that queues work.
int check_planes(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes, bool launch,
                 const uint64_t *out_noise, const uint64_t *out_moments, bool need_moments, vqx::ViewGeometry *g,
                 vqx::PlaneView *R, vqx::PlaneView *D, size_t *ws_bytes)
{
    if (!planes || (launch && (!out_noise || (need_moments && !out_moments))))
        return VQX_E_NULL;
    if (nplanes < 1 || nplanes > VQX_MAX_PLANES)
        return VQX_E_PLANES;
    int64_t wgs = 0;
    size_t bytes = 0;
    for (int p = 0; p < nplanes; ++p) {
        const vqx_plane_pair &P = planes[p];
        if (launch && (!P.ref || !P.dist))
            return VQX_E_NULL;
        int rc = check_view_batch(P.w, P.h, bpc, nframes);
        if (rc != VQX_OK)
            return rc;
        g[p] = vqx::make_view_geometry(P.w, P.h, bpc, nframes);
        wgs += g[p].workgroups;
        bytes += g[p].workspace_bytes;
    }
    if (wgs * vqx::kChunkThreads > static_cast<int64_t>(0xffffffffu))
        return VQX_E_NFRAMES;
    const int sb = bpc == 8 ? 1 : 2;
    if (launch) {
        for (int p = 0; p < nplanes; ++p) {
            const vqx_plane_pair &P = planes[p];
            if (!view_extent_ok(P.ref_row_stride, P.ref_frame_stride, P.w, P.h, nframes, sb) ||
                !view_extent_ok(P.dist_row_stride, P.dist_frame_stride, P.w, P.h, nframes, sb))
                return VQX_E_STRIDE;
        }
        for (int p = 0; p < nplanes; ++p)
            if (!aligned(planes[p].ref, sb) || !aligned(planes[p].dist, sb))
                return VQX_E_ALIGN;
        if (!aligned(out_noise, 8) || (need_moments && !aligned(out_moments, 8)))
            return VQX_E_ALIGN;
        for (int p = 0; p < nplanes; ++p) {
            R[p] = vqx::PlaneView{planes[p].ref, planes[p].ref_row_stride, planes[p].ref_frame_stride};
            D[p] = vqx::PlaneView{planes[p].dist, planes[p].dist_row_stride, planes[p].dist_frame_stride};
        }
    }
    *ws_bytes = bytes;
    return VQX_OK;
}

// Whether a view's rows are whole 16-byte aligned vectors of two-byte
// samples, which the CPU-order kernels read in place.
bool rows_of_vectors(const void *base, int64_t row_stride, int64_t frame_stride, int w, int bpc)
{
    return bpc > 8 && w % 8 == 0 && row_stride % 8 == 0 && frame_stride % 8 == 0 && aligned(base, 16);
}

// Rows of whole 16-byte vectors of two-byte samples, wherever they start,
// whose frames span less than 2^31 bytes from their first row's start to
// their last row's end (the mapped stage 1 keeps offsets inside a frame in
// 32 bits).
bool rows_of_any_vectors(const void *base, int64_t row_stride, int w, int h, int bpc)
{
    return bpc > 8 && w % 8 == 0 && aligned(base, 2) &&
           (static_cast<int64_t>(h) - 1) * row_stride + w + 16 < (static_cast<int64_t>(1) << 30);
}

// The CPU-order form over plane views that are not rows of vectors: both
// views gathered into contiguous planes after the contiguous form's
// workspace, then that form.
struct ViewCpuOrderLayout {
    size_t ref, dist, bytes;
};

ViewCpuOrderLayout view_cpu_order_layout(int w, int h, int bpc, int nframes)
{
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    const size_t plane = static_cast<size_t>(g.pixels) * g.sample_bytes * nframes;
    ViewCpuOrderLayout l{};
    l.ref = up(vqx::cpu_order_layout(g).bytes);
    l.dist = up(l.ref + plane);
    l.bytes = up(l.dist + plane);
    return l;
}

// The scratch of vqx_plane_stats_batch_noalloc: one array per GPU in the
// library's device image.  In host code its name stands for a host-side
// shadow, not a device address: only the address that hipGetSymbolAddress
// returns (looked up once per device, with that device current) is ever
// passed to a kernel.
static __device__ __align__(256) unsigned char scratch[VQX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_address[kMaxDevices];  // device address per device, null until looked up

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream).
int noalloc_scratch(hipStream_t stream, void **out)
{
    int current = 0, dev = 0;
    if (hipGetDevice(&current) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    dev = current;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return VQX_E_NO_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_address[dev]) {
        if (dev != current && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return VQX_E_HIP;
        }
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != current)
            (void)hipSetDevice(current);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return VQX_E_HIP;
        }
        scratch_address[dev] = p;
    }
    *out = scratch_address[dev];
    return VQX_OK;
}

// The host-fed form's copy stream when the caller brings none: one per
// device, created on first use (default priority, non-blocking) and kept
// until the process ends.  Calls on one device share it; each call orders
// its own copies and kernels with events, so shared use only serialises
// the copies.
std::mutex copy_stream_mutex;
hipStream_t copy_streams[kMaxDevices];

int cached_copy_stream(hipStream_t stream, hipStream_t *out)
{
    int current = 0, dev = 0;
    if (hipGetDevice(&current) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    dev = current;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return VQX_E_NO_DEVICE;
    std::lock_guard<std::mutex> lock(copy_stream_mutex);
    if (!copy_streams[dev]) {
        if (dev != current && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return VQX_E_HIP;
        }
        hipStream_t c = nullptr;
        const hipError_t e = hipStreamCreateWithFlags(&c, hipStreamNonBlocking);
        if (dev != current)
            (void)hipSetDevice(current);
        if (e != hipSuccess || !c) {
            (void)hipGetLastError();
            return VQX_E_HIP;
        }
        copy_streams[dev] = c;
    }
    *out = copy_streams[dev];
    return VQX_OK;
}

// The float sums' second stream and its two events: one set per device,
// made on first use (default priority, non-blocking) and kept until the
// process ends.  A call holds side_mutex while it enqueues its work, so
// that calls from several host threads do not interleave their records
// and waits on the shared events.
std::mutex side_mutex;
vqx::SideStream side_streams[kMaxDevices];
bool side_made[kMaxDevices];

// *out: the set of the device `stream` belongs to, or null where it cannot
// be made (the walk then follows the maps on the caller's stream).  Call
// with side_mutex held.
int float_sum_side(hipStream_t stream, const vqx::SideStream **out)
{
    *out = nullptr;
    int current = 0, dev = 0;
    if (hipGetDevice(&current) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    dev = current;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return VQX_E_NO_DEVICE;
    if (!side_made[dev]) {
        side_made[dev] = true;  // one attempt per device
        if (dev != current && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return VQX_OK;
        }
        vqx::SideStream s{};
        bool ok = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) == hipSuccess;
        // (events that a launch can record, so timing events)
        ok = ok && hipEventCreate(&s.fork) == hipSuccess;
        ok = ok && hipEventCreate(&s.join) == hipSuccess;
        if (dev != current)
            (void)hipSetDevice(current);
        if (!ok) {
            (void)hipGetLastError();
            return VQX_OK;
        }
        side_streams[dev] = s;
    }
    if (side_streams[dev].stream)
        *out = &side_streams[dev];
    return VQX_OK;
}

}  // namespace

extern "C" {

int vqx_abi_version(void) { return VQX_ABI_VERSION; }

const char *vqx_status_string(int status)
{
    switch (status) {
    case VQX_OK: return "ok";
    case VQX_E_NULL: return "a required pointer is NULL";
    case VQX_E_DIMS: return "w and h must be >= 1 with w*h <= 2^25";
    case VQX_E_BPC: return "bpc must be 8..16";
    case VQX_E_NFRAMES: return "nframes must be >= 1 (and the batch must fit one launch)";
    case VQX_E_ALIGN: return "ref/dist must be 16-byte aligned and outputs 8-byte aligned";
    case VQX_E_WORKSPACE: return "workspace missing, misaligned or smaller than vqx_plane_stats_workspace_bytes()";
    case VQX_E_HIP: return "the HIP runtime reported an error";
    case VQX_E_NO_DEVICE: return "no usable HIP device";
    case VQX_E_STRIDE: return "plane view: row stride below w, negative frame stride, or extent past 2^62 bytes";
    case VQX_E_PLANES: return "nplanes outside 1..VQX_MAX_PLANES";
    case VQX_E_SCRATCH: return "the batch needs more scratch than VQX_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
    }
}

int vqx_plane_stats_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    *bytes = vqx::make_geometry(w, h, bpc, nframes).workspace_bytes;
    return VQX_OK;
}

int vqx_plane_stats_batch_ws_timed(const void *ref, const void *dist, int w, int h, int bpc,
                                   int nframes, uint64_t *out_noise, uint64_t *out_moments,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   void *stage1_begin, void *stage1_end)
{
    int rc = check_stats_args(ref, dist, w, h, bpc, nframes, out_noise, out_moments);
    if (rc != VQX_OK)
        return rc;
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < g.workspace_bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    hipError_t err = vqx::launch_plane_stats(g, ref, dist, out_noise, out_moments,
                                             static_cast<uint64_t *>(workspace),
                                             static_cast<hipStream_t>(stream),
                                             static_cast<hipEvent_t>(stage1_begin),
                                             static_cast<hipEvent_t>(stage1_end));
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_read_probe_timed(const void *ref, const void *dist, int w, int h, int bpc, int nframes, void *workspace,
                         size_t workspace_bytes, void *stream, void *begin, void *end)
{
    if (!ref || !dist)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    if (!aligned(ref, 16) || !aligned(dist, 16))
        return VQX_E_ALIGN;
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < g.workspace_bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    if (vqx::launch_read_probe(g, ref, dist, static_cast<uint64_t *>(workspace), static_cast<hipStream_t>(stream),
                               static_cast<hipEvent_t>(begin), static_cast<hipEvent_t>(end)) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_batch_ws(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                             uint64_t *out_noise, uint64_t *out_moments, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    return vqx_plane_stats_batch_ws_timed(ref, dist, w, h, bpc, nframes, out_noise, out_moments,
                                          workspace, workspace_bytes, stream, nullptr, nullptr);
}

int vqx_float_sum_workspace_bytes(long long nterms, int nbuffers, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    if (nterms < 0 || nterms > (1ll << 36))
        return VQX_E_DIMS;
    if (nbuffers < 1 || nbuffers > 65535)
        return VQX_E_NFRAMES;
    *bytes = vqx::float_sum_layout(nterms, nbuffers).bytes;
    return VQX_OK;
}

int vqx_float_running_sums_ws(const float *terms, long long nterms, int nbuffers, float *out_sums,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    if (!out_sums || (!terms && nterms > 0))
        return VQX_E_NULL;
    size_t need = 0;
    int rc = vqx_float_sum_workspace_bytes(nterms, nbuffers, &need);
    if (rc != VQX_OK)
        return rc;
    if (!aligned(terms, 4) || !aligned(out_sums, 4))
        return VQX_E_ALIGN;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    std::lock_guard<std::mutex> lock(side_mutex);
    const vqx::SideStream *side = nullptr;
    rc = float_sum_side(static_cast<hipStream_t>(stream), &side);
    if (rc != VQX_OK)
        return rc;
    if (vqx::launch_float_sums(terms, nterms, nbuffers, out_sums, workspace, static_cast<hipStream_t>(stream),
                               side) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_batch_noalloc(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                                  uint64_t *out_noise, uint64_t *out_moments, void *stream)
{
    int rc = check_stats_args(ref, dist, w, h, bpc, nframes, out_noise, out_moments);
    if (rc != VQX_OK)
        return rc;
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    if (g.workspace_bytes > VQX_NOALLOC_SCRATCH_BYTES)
        return VQX_E_SCRATCH;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    rc = noalloc_scratch(s, &ws);
    if (rc != VQX_OK)
        return rc;
    if (vqx::launch_plane_stats(g, ref, dist, out_noise, out_moments, static_cast<uint64_t *>(ws), s) !=
        hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_batch(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                          uint64_t *out_noise, uint64_t *out_moments, void *stream)
{
    int rc = check_stats_args(ref, dist, w, h, bpc, nframes, out_noise, out_moments);
    if (rc != VQX_OK)
        return rc;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (hipMallocAsync(&ws, g.workspace_bytes, s) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    hipError_t err = vqx::launch_plane_stats(g, ref, dist, out_noise, out_moments,
                                             static_cast<uint64_t *>(ws), s);
    // freed in stream order, after the kernels that use it
    hipError_t ferr = hipFreeAsync(ws, s);
    if (err != hipSuccess || ferr != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_cpu_order_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    *bytes = vqx::cpu_order_layout(vqx::make_geometry(w, h, bpc, nframes)).bytes;
    return VQX_OK;
}

int vqx_plane_stats_batch_cpu_order_ws(const void *ref, const void *dist, int w, int h, int bpc,
                                       int nframes, uint64_t *out_noise, uint64_t *out_moments,
                                       uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = check_stats_args(ref, dist, w, h, bpc, nframes, out_noise, out_moments);
    if (rc != VQX_OK)
        return rc;
    if (!out_cpu_noise || !out_cpu_moments)
        return VQX_E_NULL;
    if (!aligned(out_cpu_noise, 8) || !aligned(out_cpu_moments, 8))
        return VQX_E_ALIGN;
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) ||
        workspace_bytes < vqx::cpu_order_layout(g).bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    hipError_t err = vqx::launch_plane_stats_cpu_order(g, ref, dist, out_noise, out_moments,
                                                       out_cpu_noise, out_cpu_moments, workspace,
                                                       static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_view_cpu_order_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    *bytes = view_cpu_order_layout(w, h, bpc, nframes).bytes;
    return VQX_OK;
}

int vqx_plane_stats_view_cpu_order_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                                      const void *dist, int64_t dist_row_stride, int64_t dist_frame_stride, int w,
                                      int h, int bpc, int nframes, uint64_t *out_noise, uint64_t *out_moments,
                                      uint64_t *out_cpu_noise, uint64_t *out_cpu_moments, void *workspace,
                                      size_t workspace_bytes, void *stream)
{
    int rc = check_view_args(ref, ref_row_stride, ref_frame_stride, dist, dist_row_stride, dist_frame_stride, w, h,
                             bpc, nframes, out_noise, out_moments, true);
    if (rc != VQX_OK)
        return rc;
    rc = check_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    if (!out_cpu_noise || !out_cpu_moments)
        return VQX_E_NULL;
    if (!aligned(out_cpu_noise, 8) || !aligned(out_cpu_moments, 8))
        return VQX_E_ALIGN;
    const ViewCpuOrderLayout l = view_cpu_order_layout(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < l.bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    char *ws = static_cast<char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const vqx::Geometry g = vqx::make_geometry(w, h, bpc, nframes);
    hipError_t err;
    if (rows_of_any_vectors(ref, ref_row_stride, w, h, bpc) && rows_of_any_vectors(dist, dist_row_stride, w, h, bpc)) {
        // read in place: each vector of the contiguous order found in the
        // views, at whatever offset within 16 bytes its row puts it
        const vqx::VecMap map = vqx::make_vec_map(w, h, ref, ref_row_stride, ref_frame_stride, dist,
                                                  dist_row_stride, dist_frame_stride);
        err = vqx::launch_plane_stats_cpu_order(g, vqx::vec_base(ref), vqx::vec_base(dist), out_noise, out_moments,
                                                out_cpu_noise, out_cpu_moments, workspace, s, map);
        if (err != hipSuccess) {
            (void)hipGetLastError();
            return VQX_E_HIP;
        }
        return VQX_OK;
    }
    err = vqx::launch_gather_view(vqx::PlaneView{ref, ref_row_stride, ref_frame_stride}, w, h, bpc,
                                             nframes, ws + l.ref, s);
    if (err == hipSuccess)
        err = vqx::launch_gather_view(vqx::PlaneView{dist, dist_row_stride, dist_frame_stride}, w, h, bpc, nframes,
                                      ws + l.dist, s);
    if (err == hipSuccess)
        err = vqx::launch_plane_stats_cpu_order(g, ws + l.ref, ws + l.dist, out_noise, out_moments, out_cpu_noise,
                                                out_cpu_moments, workspace, s);
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_plane_stats_host_workspace_bytes(int w, int h, int bpc, int frames_per_upload, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    int rc = check_batch(w, h, bpc, frames_per_upload);
    if (rc != VQX_OK)
        return rc;
    *bytes = vqx::host_stream_layout(w, h, bpc, frames_per_upload).bytes;
    return VQX_OK;
}

int vqx_plane_stats_host_ws(const void *ref_host, const void *dist_host, int w, int h, int bpc, int nframes,
                            int frames_per_upload, uint64_t *out_noise, uint64_t *out_moments, void *workspace,
                            size_t workspace_bytes, void *stream, void *copy_stream)
{
    if (!ref_host || !dist_host || !out_noise || !out_moments)
        return VQX_E_NULL;
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    if (nframes < 1)
        return VQX_E_NFRAMES;
    rc = check_batch(w, h, bpc, frames_per_upload);
    if (rc != VQX_OK)
        return rc;
    if (!aligned(out_noise, 8) || !aligned(out_moments, 8))
        return VQX_E_ALIGN;
    if (!workspace || !aligned(workspace, 16) ||
        workspace_bytes < vqx::host_stream_layout(w, h, bpc, frames_per_upload).bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    hipStream_t copy = static_cast<hipStream_t>(copy_stream);
    if (!copy) {
        rc = cached_copy_stream(static_cast<hipStream_t>(stream), &copy);
        if (rc != VQX_OK)
            return rc;
    }
    const hipError_t err = vqx::run_host_stream(w, h, bpc, nframes, frames_per_upload, ref_host, dist_host,
                                                out_noise, out_moments, workspace, static_cast<hipStream_t>(stream),
                                                copy);
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_conclude_psnr(uint64_t noise, int w, int h, int bpc, double psnr_max, double *mse,
                      double *psnr_db)
{
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    const double m = unit_mean(noise, 2, bpc, static_cast<int64_t>(w) * h);
    if (mse)
        *mse = m;
    if (psnr_db)
        *psnr_db = psnr_from_mse(m, bpc, psnr_max);
    return VQX_OK;
}

int vqx_conclude_moments(const uint64_t sums[4], int w, int h, int bpc, double out[4])
{
    if (!sums || !out)
        return VQX_E_NULL;
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    const int64_t pixels = static_cast<int64_t>(w) * h;
    const int power[4] = {1, 1, 2, 2};
    double tmp[4];
    for (int k = 0; k < 4; ++k)
        tmp[k] = unit_mean(sums[k], power[k], bpc, pixels);
    for (int k = 0; k < 4; ++k)
        out[k] = tmp[k];
    return VQX_OK;
}

int vqx_conclude_batch(const uint64_t *noise, const uint64_t *moments, int w, int h, int bpc,
                       int nframes, double psnr_max, double *out)
{
    if (!noise || !moments || !out)
        return VQX_E_NULL;
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    if (nframes < 1)
        return VQX_E_NFRAMES;
    for (int f = 0; f < nframes; ++f) {
        double *o = out + 6 * static_cast<size_t>(f);
        vqx_conclude_psnr(noise[f], w, h, bpc, psnr_max, &o[0], &o[1]);
        vqx_conclude_moments(moments + 4 * static_cast<size_t>(f), w, h, bpc, &o[2]);
    }
    return VQX_OK;
}

int vqx_plane_view_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    int rc = check_view_batch(w, h, bpc, nframes);
    if (rc != VQX_OK)
        return rc;
    *bytes = vqx::make_view_geometry(w, h, bpc, nframes).workspace_bytes;
    return VQX_OK;
}

int vqx_plane_stats_view_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride, const void *dist,
                            int64_t dist_row_stride, int64_t dist_frame_stride, int w, int h, int bpc, int nframes,
                            uint64_t *out_noise, uint64_t *out_moments, void *workspace, size_t workspace_bytes,
                            void *stream)
{
    int rc = check_view_args(ref, ref_row_stride, ref_frame_stride, dist, dist_row_stride, dist_frame_stride, w, h,
                             bpc, nframes, out_noise, out_moments, true);
    if (rc != VQX_OK)
        return rc;
    const vqx::ViewGeometry g = vqx::make_view_geometry(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < g.workspace_bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    const vqx::PlaneView R{ref, ref_row_stride, ref_frame_stride};
    const vqx::PlaneView D{dist, dist_row_stride, dist_frame_stride};
    hipError_t err;
    const vqx::Geometry cg = vqx::make_geometry(w, h, bpc, nframes);
    if (rows_of_vectors(ref, ref_row_stride, ref_frame_stride, w, bpc) &&
        rows_of_vectors(dist, dist_row_stride, dist_frame_stride, w, bpc) &&
        check_batch(w, h, bpc, nframes) == VQX_OK && workspace_bytes >= cg.workspace_bytes) {
        // rows of whole vectors: the contiguous chunks, each vector found in the views
        err = vqx::launch_plane_stats_mapped(cg, ref, dist, out_noise, out_moments,
                                             static_cast<uint64_t *>(workspace),
                                             vqx::make_vec_map(w, h, ref, ref_row_stride, ref_frame_stride,
                                                               dist, dist_row_stride, dist_frame_stride),
                                             static_cast<hipStream_t>(stream));
    } else {
        err = vqx::launch_view_stats(g, R, D, out_noise, out_moments, static_cast<uint64_t *>(workspace),
                                     static_cast<hipStream_t>(stream));
    }
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_psnr_int_view_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride, const void *dist,
                         int64_t dist_row_stride, int64_t dist_frame_stride, int w, int h, int bpc, int nframes,
                         uint64_t *out_noise, void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = check_view_args(ref, ref_row_stride, ref_frame_stride, dist, dist_row_stride, dist_frame_stride, w, h,
                             bpc, nframes, out_noise, nullptr, false);
    if (rc != VQX_OK)
        return rc;
    const vqx::ViewGeometry g = vqx::make_view_geometry(w, h, bpc, nframes);
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < g.workspace_bytes)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    const vqx::PlaneView R{ref, ref_row_stride, ref_frame_stride};
    const vqx::PlaneView D{dist, dist_row_stride, dist_frame_stride};
    if (vqx::launch_view_psnr_int(g, R, D, out_noise, static_cast<uint64_t *>(workspace),
                                  static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

// ---------------------------------------------------------- several planes
int vqx_planes_workspace_bytes(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes, size_t *bytes)
{
    if (!bytes)
        return VQX_E_NULL;
    vqx::ViewGeometry g[VQX_MAX_PLANES];
    return check_planes(planes, nplanes, bpc, nframes, false, nullptr, nullptr, false, g, nullptr, nullptr, bytes);
}

int vqx_plane_stats_planes_ws(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes, uint64_t *out_noise,
                              uint64_t *out_moments, void *workspace, size_t workspace_bytes, void *stream)
{
    vqx::ViewGeometry g[VQX_MAX_PLANES];
    vqx::PlaneView R[VQX_MAX_PLANES], D[VQX_MAX_PLANES];
    size_t need = 0;
    int rc = check_planes(planes, nplanes, bpc, nframes, true, out_noise, out_moments, true, g, R, D, &need);
    if (rc != VQX_OK)
        return rc;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    if (vqx::launch_planes_stats(g, R, D, nplanes, out_noise, out_moments, static_cast<uint64_t *>(workspace),
                                 static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_psnr_int_planes_ws(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes, uint64_t *out_noise,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    vqx::ViewGeometry g[VQX_MAX_PLANES];
    vqx::PlaneView R[VQX_MAX_PLANES], D[VQX_MAX_PLANES];
    size_t need = 0;
    int rc = check_planes(planes, nplanes, bpc, nframes, true, out_noise, nullptr, false, g, R, D, &need);
    if (rc != VQX_OK)
        return rc;
    if (!workspace || !aligned(workspace, 16) || workspace_bytes < need)
        return VQX_E_WORKSPACE;
    rc = device_ready();
    if (rc != VQX_OK)
        return rc;
    if (vqx::launch_planes_psnr_int(g, R, D, nplanes, out_noise, static_cast<uint64_t *>(workspace),
                                    static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return VQX_E_HIP;
    }
    return VQX_OK;
}

int vqx_conclude_psnr_int(uint64_t noise, int w, int h, int bpc, double psnr_max, double *mse, double *psnr_db)
{
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    const double m = static_cast<double>(noise) / static_cast<double>(static_cast<int64_t>(w) * h);
    if (mse)
        *mse = m;
    if (psnr_db) {
        if (m == 0.0) {
            *psnr_db = psnr_max > 0.0 ? psnr_max : HUGE_VAL;
        } else {
            const double peak = static_cast<double>((1 << bpc) - 1);
            const double db = 10.0 * log10(peak * peak / m);
            *psnr_db = (psnr_max > 0.0 && db > psnr_max) ? psnr_max : db;
        }
    }
    return VQX_OK;
}

int vqx_conclude_psnr_int_batch(const uint64_t *noise, int w, int h, int bpc, int nframes, double psnr_max,
                                double *out)
{
    if (!noise || !out)
        return VQX_E_NULL;
    int rc = check_shape(w, h, bpc);
    if (rc != VQX_OK)
        return rc;
    if (nframes < 1)
        return VQX_E_NFRAMES;
    for (int f = 0; f < nframes; ++f)
        vqx_conclude_psnr_int(noise[f], w, h, bpc, psnr_max, &out[2 * static_cast<size_t>(f)],
                              &out[2 * static_cast<size_t>(f) + 1]);
    return VQX_OK;
}

}  // extern "C"
