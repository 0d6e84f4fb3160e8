/*
 * vqx -- bit-exact luma-plane reductions for float_psnr and float_moment on
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * Sources (web pages, cited by title and section):
 *   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
 *            integers and returns the CPU's score bit for bit"
 *   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU
 *            adds, and is bit-identical while the CPU's own sum is exact"
 *   [ADM]    "ADR-1423: adm_hip takes its weights, shifts and score
 *            conclusion from the CPU, folds the denominator once per row and
 *            clears its accumulators after the upload"
 *
 * Terms and units.  For a frame of w*h samples at bpc bits per component,
 * scaler s = 2^(bpc-8) [PSNR, Context].  q(x) is the binary32 product x*x of
 * the sample value x (or sample difference) converted to float, rounded to
 * nearest even and read back as an integer; it is below 2^32 for every
 * 16-bit value [MOMENT, Decision].  Dividing a sample by s before squaring
 * does not change which bits that product drops, so q(x) is the CPU's float
 * term expressed in units of 1/s^2 [MOMENT, Decision; PSNR, Decision].
 *
 * Per frame the library returns five exact integer sums:
 *   noise = sum q(ref - dist)  (units 1/s^2; float_psnr's noise [PSNR, Decision])
 *   ref1  = sum ref,  dist1 = sum dist          (units 1/s)
 *   ref2  = sum q(ref), dist2 = sum q(dist)      (units 1/s^2)
 *   (float_moment's four sums [MOMENT, Context and Decision]).
 * No term is rounded after the float product and no sum is ever rounded, so
 * the sums are the exact integers whatever the summation order.  While a sum
 * is below 2^53 units it equals the CPU's running double times the unit, bit
 * for bit [PSNR, Context; MOMENT, Decision]; past 2^53 the CPU's own double
 * rounds and these sums stay exact [PSNR, Consequences; MOMENT, Decision].
 *
 * Status codes: every entry point returns VQX_OK (0) or a negative VQX_E_*.
 * An argument error is reported before anything is queued and leaves every
 * output untouched.
 */
#ifndef VQX_H
#define VQX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQX_ABI_VERSION 1

/* Largest frame accepted: 2^25 samples (an 8K frame, 7680x4320, has
 * 33 177 600).  Up to 12 bits the CPU's noise then needs at most 49 bits
 * [PSNR, Context]; every device sum stays below 2^57. */
#define VQX_MAX_PIXELS (1 << 25)

enum vqx_status {
    VQX_OK = 0,
    VQX_E_NULL = -1,      /* a required pointer is NULL */
    VQX_E_DIMS = -2,      /* w < 1, h < 1 or w*h > VQX_MAX_PIXELS */
    VQX_E_BPC = -3,       /* bpc outside 8..16 */
    VQX_E_NFRAMES = -4,   /* nframes < 1, or a batch too large for one dispatch: more
                             than (2^32-1)/256 chunks of 2048 16-byte vectors per plane
                             (frames round up to whole chunks) */
    VQX_E_ALIGN = -5,     /* ref/dist not 16-byte aligned, or an output not 8-byte aligned */
    VQX_E_WORKSPACE = -6, /* workspace smaller than vqx_plane_stats_workspace_bytes() */
    VQX_E_HIP = -7,       /* the HIP runtime reported an error (launch or allocation) */
    VQX_E_NO_DEVICE = -8, /* no usable HIP device */
    VQX_E_STRIDE = -9,    /* plane views: a row stride below w, a negative frame stride,
                             or a plane whose last sample lies past 2^62 bytes */
    VQX_E_PLANES = -10,   /* several planes: nplanes outside 1..VQX_MAX_PLANES */
    VQX_E_SCRATCH = -11   /* vqx_plane_stats_batch_noalloc: the batch needs more scratch than
                             VQX_NOALLOC_SCRATCH_BYTES */
};

/* VQX_ABI_VERSION of the loaded library. */
int vqx_abi_version(void);

/* Static English text for a status code; never NULL. */
const char *vqx_status_string(int status);

/*
 * Device scratch needed by vqx_plane_stats_batch_ws for this batch shape
 * (one partial record per workgroup).  Writes *bytes; host-only, no device
 * call.  Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES.
 */
int vqx_plane_stats_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes);

/*
 * The five exact sums of every frame of a batch, in one pass over each plane.
 *
 *   ref, dist    device pointers, 16-byte aligned, to [nframes][h][w] samples
 *                stored back to back (row stride w, frame stride w*h): uint8
 *                when bpc == 8, else uint16 holding the value in its low
 *                bits.  A stored value above 2^bpc - 1 is not an error: it is
 *                squared and summed like any other.  Frames inside the batch
 *                need not start on a 16-byte boundary.
 *   bpc          8..16.
 *   out_noise    uint64[nframes]: noise of frame f, units 1/s^2.
 *   out_moments  uint64[nframes][4]: {ref1, dist1, ref2, dist2} of frame f
 *                (units 1/s, 1/s, 1/s^2, 1/s^2).
 *                Both outputs must be addressable by the device: device
 *                memory, or pinned host memory mapped for the device (pass
 *                the address hipHostGetDevicePointer returns), into which
 *                the last kernel writes directly (40 bytes per frame).
 *   stream       a hipStream_t, or NULL for the null stream.
 *
 * Outputs are overwritten, never accumulated into, so they need no clearing
 * beforehand: a clear queued ahead of other work can be lost or reordered
 * [ADM, Context and Decision], and no clear is done here.  Every value is
 * below 2^58 and may be viewed as int64.
 *
 * The call only queues work on `stream` and never waits: results are valid
 * once the stream has passed this point.  The caller owns every buffer and
 * keeps it alive until then; the library keeps no pointer after returning.
 * This form takes its scratch from hipMallocAsync/hipFreeAsync on `stream`.
 *
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES, VQX_E_ALIGN
 * (before anything is queued); VQX_E_NO_DEVICE; VQX_E_HIP on a failed
 * allocation or launch (the HIP error is consumed).
 */
int vqx_plane_stats_batch(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                          uint64_t *out_noise, uint64_t *out_moments, void *stream);

/*
 * As vqx_plane_stats_batch, with caller-provided device scratch of at least
 * vqx_plane_stats_workspace_bytes() bytes (16-byte aligned).  The workspace
 * is written before it is read within the call, so its contents on entry do
 * not matter; two calls may not share one workspace concurrently.
 * Additional error: VQX_E_WORKSPACE (workspace NULL, too small or misaligned).
 */
int vqx_plane_stats_batch_ws(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                             uint64_t *out_noise, uint64_t *out_moments,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The five
 * sums of vqx_plane_stats_batch_ws, with the same arguments minus the
 * workspace, and no allocation of any kind: the scratch is one fixed array
 * per GPU in the library's device memory, VQX_NOALLOC_SCRATCH_BYTES long,
 * held by each GPU the library runs on until the process ends.  A batch
 * whose vqx_plane_stats_workspace_bytes() exceeds it is rejected with
 * VQX_E_SCRATCH (4 MiB holds, for example, 128 frames of 3840x2160 or 512
 * of 1920x1080 at 9..16 bits).
 *
 * Every call on one GPU uses that GPU's one array, and the array keeps the
 * last call's contents.  Each call writes every scratch byte it reads, so
 * nothing needs clearing; but calls that overlap on one GPU (on two streams,
 * or from two threads) race on the array, and the caller must order them.
 * The first call on a device looks up the array's device address (a symbol
 * lookup, no allocation) with that device current; the device is the one
 * of `stream` (the current device for the null stream).
 *
 * Errors: as vqx_plane_stats_batch, VQX_E_SCRATCH (before anything is
 * queued), and VQX_E_HIP if the address lookup fails.
 */
#define VQX_NOALLOC_SCRATCH_BYTES (4u << 20)
int vqx_plane_stats_batch_noalloc(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                                  uint64_t *out_noise, uint64_t *out_moments, void *stream);

/*
 * Device scratch needed by vqx_plane_stats_batch_cpu_order_ws.  Host-only.
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES.
 */
int vqx_plane_stats_cpu_order_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes);

/*
 * The exact sums, as vqx_plane_stats_batch_ws, and also the values the
 * CPU extractors' running double sums hold after their last add, bit for
 * bit, on every frame:
 *   out_cpu_noise    uint64[nframes], out_cpu_moments uint64[nframes][4],
 *                    in the units of the exact sums (every such double is an
 *                    integer in these units, below 2^58).
 * Below 2^53 units they equal the exact sums.  Past it the CPU rounds
 * every add to the sum's last place [PSNR, Consequences; MOMENT, Decision]
 * and these are its rounded values, reproduced by composing the
 * round-to-nearest-even steps of runs of adds (a two-state map per run
 * inside one binade) and walking the frame in the CPU's raster order --
 * the sequence of roundings that the float_moment page leaves to a later
 * change [MOMENT, Alternatives].  Concluding them with
 * vqx_conclude_batch gives the CPU's scores bit for bit on every frame.
 *
 * Frames whose sums stay below 2^53 cost only small kernels more than
 * vqx_plane_stats_batch_ws; a frame past 2^53 costs one more read of its
 * planes.  Arguments, layout, ownership and errors otherwise as
 * vqx_plane_stats_batch_ws, with the workspace sized by
 * vqx_plane_stats_cpu_order_workspace_bytes.
 */
int vqx_plane_stats_batch_cpu_order_ws(const void *ref, const void *dist, int w, int h, int bpc,
                                       int nframes, uint64_t *out_noise, uint64_t *out_moments,
                                       uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Device scratch of vqx_plane_stats_host_ws for this frame shape and upload
 * size: two staging slots of frames_per_upload frames of both planes, and
 * stage 1's records of one upload.  Host-only.
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES (frames_per_upload).
 */
int vqx_plane_stats_host_workspace_bytes(int w, int h, int bpc, int frames_per_upload, size_t *bytes);

/*
 * The five sums of vqx_plane_stats_batch_ws for a batch that lies in HOST
 * memory: the planes are uploaded frames_per_upload frames at a time into
 * the workspace's two staging slots, and each upload overlaps the reduction
 * of the one before (copies on copy_stream, kernels on stream, ordered by
 * events).  As in the tool, a frame's work is queued after its upload
 * [ADM, Decision].
 *   ref_host, dist_host  host [nframes][h][w] samples (uint8 at 8 bits,
 *                        uint16 otherwise), contiguous.  Page-locked memory
 *                        (hipHostMalloc, or a pinned tensor) is what lets
 *                        the copies run asynchronously and overlap; pageable
 *                        memory gives the same results, without overlap.
 *   frames_per_upload    frames per upload, >= 1 (a last, smaller upload
 *                        takes the rest)
 *   out_noise, out_moments  as vqx_plane_stats_batch_ws: device memory or
 *                        pinned host memory mapped for the device
 *   stream               where the kernels run (work queued on it before
 *                        the call comes first); copy_stream: where the
 *                        copies run, or NULL for the library's copy stream
 *                        of the device (created on the first such call,
 *                        default priority, kept until the process ends and
 *                        shared by such calls on that device).  One stream
 *                        for both is allowed: the results are the same,
 *                        nothing overlaps.
 * The call returns when every frame has been reduced and every copy is
 * done: the host buffers and the outputs are the caller's again.
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES (nframes or
 * frames_per_upload < 1, or an upload too large for one dispatch),
 * VQX_E_ALIGN (an output not 8-byte aligned), VQX_E_WORKSPACE (missing, not
 * 16-byte aligned or smaller than vqx_plane_stats_host_workspace_bytes()),
 * VQX_E_NO_DEVICE, VQX_E_HIP.
 */
int vqx_plane_stats_host_ws(const void *ref_host, const void *dist_host, int w, int h, int bpc,
                            int nframes, int frames_per_upload, uint64_t *out_noise,
                            uint64_t *out_moments, void *workspace, size_t workspace_bytes,
                            void *stream, void *copy_stream);

/*
 * float_psnr's conclusion from a frame's exact noise (host only).
 *   mse     = ((double)noise / s^2) / (w*h)    -- the 8-bit-scale mean
 *             squared error; (double) rounds once, to nearest even, and only
 *             at or past 2^53; the division by s^2 is exact [PSNR, Decision].
 *   psnr_db = 10*log10(peak^2 / mse), peak = (2^bpc - 1)/s, the largest
 *             sample on the 8-bit scale; min(psnr_db, psnr_max) when
 *             psnr_max > 0.  mse == 0 gives psnr_max, or +inf when
 *             psnr_max <= 0 (uncapped).
 * Either output pointer may be NULL.  Errors: VQX_E_DIMS, VQX_E_BPC.
 */
int vqx_conclude_psnr(uint64_t noise, int w, int h, int bpc, double psnr_max,
                      double *mse, double *psnr_db);

/*
 * float_moment's conclusion (host only): from {ref1, dist1, ref2, dist2} the
 * four means {ref1/s, dist1/s, ref2/s^2, dist2/s^2} each divided by w*h --
 * the conversion to double and the two divisions of [MOMENT, Decision].
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC.
 */
int vqx_conclude_moments(const uint64_t sums[4], int w, int h, int bpc, double out[4]);

/*
 * Both conclusions for a whole batch of host-side sums (host only).
 *   noise    host uint64[nframes], moments host uint64[nframes][4]
 *   out      host double[nframes][6]: {mse, psnr_db, ref_mean, dist_mean,
 *            ref_mean_sq, dist_mean_sq} per frame.
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES.
 */
int vqx_conclude_batch(const uint64_t *noise, const uint64_t *moments, int w, int h, int bpc,
                       int nframes, double psnr_max, double *out);

/*
 * ------------------------------------------------------------ plane views
 * The same reductions over planes that are not one contiguous [nframes][h][w]
 * array: chroma planes, planes with a padded row pitch, a region of interest
 * inside larger planes, or one plane of planar YUV frames stored one after
 * another.  A view addresses one plane of every frame of a batch: sample
 * (x, y) of frame f is at
 *     base + f*frame_stride + y*row_stride + x        (in samples)
 * with samples uint8 at 8 bits and uint16 otherwise.  row_stride >= w;
 * frame_stride >= 0 (0: the same plane for every frame); views may overlap
 * (they are only read).  The caller owns the memory and must make every
 * addressed sample readable.  ref and dist have views of their own, with the
 * same w, h and nframes.  The results are the same function of the selected
 * samples as the contiguous entry points' [PSNR, Context and Decision;
 * MOMENT, Decision]; the tiling never changes an integer sum.  Rows are
 * read as 16-byte vectors where dist starts each row the same distance past
 * ref within 16 bytes (row strides differing by a multiple of 16 bytes),
 * fastest where that distance is 0 and every row starts at one offset; rows
 * narrower than 32 vectors at varying offsets, and ref and dist rows that
 * drift apart from row to row, are read sample by sample, still exactly.
 *
 * Common errors, in this order: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC,
 * VQX_E_NFRAMES (also when the batch needs more than (2^32-1)/256 tiles of
 * 2048 16-byte vectors per plane), VQX_E_STRIDE, VQX_E_ALIGN (ref/dist not
 * aligned to one sample, an output not to 8 bytes), VQX_E_WORKSPACE
 * (missing, not 16-byte aligned or smaller than
 * vqx_plane_view_workspace_bytes()), VQX_E_NO_DEVICE, VQX_E_HIP.  Outputs
 * are written once each, never accumulated into; they may be pinned host
 * memory mapped for the device.  The calls queue work on `stream` and return.
 */

/* Device scratch of the plane-view entry points for this batch shape
 * (64 bytes per frame and tile).  Host-only. */
int vqx_plane_view_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes);

/* The five sums of vqx_plane_stats_batch_ws, over plane views.  Where both
 * views hold two-byte samples (bpc 9..16) in rows of whole 16-byte vectors
 * (w, both row strides and both frame strides multiples of 8 samples, both
 * bases 16-byte aligned) they are read with the contiguous form's chunks,
 * each vector found in place, at the contiguous form's speed; other views
 * are read in tiles of whole rows.  The sums are the same either way. */
int vqx_plane_stats_view_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                            const void *dist, int64_t dist_row_stride, int64_t dist_frame_stride,
                            int w, int h, int bpc, int nframes, uint64_t *out_noise,
                            uint64_t *out_moments, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * The integer psnr twin's noise over plane views: per frame one uint64,
 *   out_noise[f] = sum over the plane of (ref - dist)^2,
 * the squares exact integers of the stored samples (below 2^32), the sum
 * exact (below 2^57) -- the one integer per frame that the integer psnr twin
 * keeps [PSNR, Alternatives].  It equals the float noise of
 * vqx_plane_stats_* wherever |ref - dist| < 4096 (there the float square is
 * exact); above that the float square rounds and this one does not.
 */
int vqx_psnr_int_view_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                         const void *dist, int64_t dist_row_stride, int64_t dist_frame_stride,
                         int w, int h, int bpc, int nframes, uint64_t *out_noise,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The CPU-order form (vqx_plane_stats_batch_cpu_order_ws) over plane views:
 * the exact sums and the CPU's running double sums, bit for bit past 2^53
 * too, of views with any row and frame stride -- the CPU adds a view's
 * samples in raster order, row after row, whatever the pitch [PSNR,
 * Context; MOMENT, Context].  Where both views hold two-byte samples (bpc
 * 9..16) in rows of whole 16-byte vectors (w a multiple of 8 samples; any
 * strides; each base aligned to its samples; a frame's rows spanning less
 * than 2^31 bytes) they are read in place: at the contiguous form's speed
 * where both bases are 16-byte aligned and all strides multiples of 8
 * samples, else from the two aligned 16-byte blocks that hold each vector
 * (about 1.2 times the contiguous form's time).  Other views are
 * first copied into contiguous planes inside the workspace (about three
 * times the contiguous form's time), then reduced as the contiguous form
 * does; the results are the same either way.  Errors as for the views and the
 * contiguous CPU-order form; the workspace is
 * vqx_plane_stats_view_cpu_order_workspace_bytes() (the contiguous form's
 * and both planes of the batch, whichever way the call reads).
 */
int vqx_plane_stats_view_cpu_order_workspace_bytes(int w, int h, int bpc, int nframes, size_t *bytes);
int vqx_plane_stats_view_cpu_order_ws(const void *ref, int64_t ref_row_stride, int64_t ref_frame_stride,
                                      const void *dist, int64_t dist_row_stride,
                                      int64_t dist_frame_stride, int w, int h, int bpc, int nframes,
                                      uint64_t *out_noise, uint64_t *out_moments,
                                      uint64_t *out_cpu_noise, uint64_t *out_cpu_moments,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * ------------------------------------------------------------ several planes
 * Up to VQX_MAX_PLANES planes of the same frames at once -- Y, U and V of
 * planar frames, say -- each a pair of views as above with its own w and h;
 * bpc and nframes are common.  All planes go through one launch of each
 * stage, and the results are those of the one-plane entry points for each
 * plane, laid out plane after plane:
 *   out_noise    uint64[nplanes][nframes]
 *   out_moments  uint64[nplanes][nframes][4]  (vqx_plane_stats_planes_ws)
 * `planes` is a host array read during the call.  Errors as for the views,
 * and VQX_E_PLANES; VQX_E_NFRAMES also when all planes' tiles together
 * exceed (2^32-1)/256; the workspace is vqx_planes_workspace_bytes() (64
 * bytes per plane, frame and tile).
 */
#define VQX_MAX_PLANES 4

typedef struct vqx_plane_pair {
    const void *ref;            /* device pointer: sample (0, 0) of frame 0 */
    int64_t ref_row_stride;     /* samples */
    int64_t ref_frame_stride;   /* samples */
    const void *dist;
    int64_t dist_row_stride;
    int64_t dist_frame_stride;
    int w, h;                   /* the plane's size in samples */
} vqx_plane_pair;

/* Device scratch for these planes (only their w and h are read).  Host-only. */
int vqx_planes_workspace_bytes(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes,
                               size_t *bytes);

/* The five sums of every plane of every frame. */
int vqx_plane_stats_planes_ws(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes,
                              uint64_t *out_noise, uint64_t *out_moments, void *workspace,
                              size_t workspace_bytes, void *stream);

/* The integer psnr noise of every plane of every frame. */
int vqx_psnr_int_planes_ws(const vqx_plane_pair *planes, int nplanes, int bpc, int nframes,
                           uint64_t *out_noise, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The integer psnr conclusion (host only), on the stored scale:
 *   mse     = (double)noise / (w*h)   -- one rounding of the integer (only
 *             at or past 2^53), one division;
 *   psnr_db = 10*log10(peak^2 / mse), peak = 2^bpc - 1; min(psnr_db,
 *             psnr_max) when psnr_max > 0; mse == 0 gives psnr_max, or +inf
 *             when psnr_max <= 0.
 * The pages give no formula for it; this is float_psnr's ratio [PSNR,
 * Consequences] taken on the stored scale.  Either output pointer may be
 * NULL.  Errors: VQX_E_DIMS, VQX_E_BPC.
 */
int vqx_conclude_psnr_int(uint64_t noise, int w, int h, int bpc, double psnr_max, double *mse,
                          double *psnr_db);

/*
 * vqx_conclude_psnr_int for a batch (host only).
 *   noise  host uint64[nframes]
 *   out    host double[nframes][2]: {mse, psnr_db} per frame
 * Errors: VQX_E_NULL, VQX_E_DIMS, VQX_E_BPC, VQX_E_NFRAMES.
 */
int vqx_conclude_psnr_int_batch(const uint64_t *noise, int w, int h, int bpc, int nframes,
                                double psnr_max, double *out);

/* ------------------------------------------------------------------------
 * The psnr_hvs running float sum [HVS = "ADR-1397: GPU psnr_hvs twins
 * reproduce the CPU's running float sum bit for bit"].
 *
 * calc_psnrhvs() accumulates all of a plane's masked coefficient errors in
 * a single float, one at a time, so the rounding of each add depends on the
 * value accumulated before it [HVS, Context]; the page's twins store the terms (64 per 8x8 block, row-major,
 * blocks in raster order) and add them one by one into a float on the host
 * [HVS, Decision].  This call does that sum on the device, with an
 * order-preserving reduction [HVS, Alternatives]: for each of `nbuffers`
 * buffers of `nterms` float32 terms, stored one after another at `terms`
 * (device memory, 4-byte aligned), out_sums[k] (device, 4-byte aligned)
 * receives, bit for bit, the float S after S = 0.0f; S += term, in buffer
 * order, in IEEE binary32 round-to-nearest-even arithmetic.  The DCT, CSF
 * and masking that make the terms are not part of it.
 *
 * Terms must be nonnegative and finite (squares); -0.0 adds like +0.0.  A
 * buffer holding a negative, infinite or NaN term gets the quiet NaN
 * 0x7fc00000 as its sum (a rule of this library, not of the CPU).  A sum
 * that overflows is +infinity, as in the CPU's float.  nterms == 0 gives +0.
 *
 * Workspace: at least vqx_float_sum_workspace_bytes() bytes of device
 * memory, 16-byte aligned, written before it is read (contents on entry do
 * not matter); calls may not share one workspace concurrently.  The call
 * only queues work on `stream`; results are valid once the stream passes it.
 * Part of the work runs on a second stream of the device's own (made on the
 * first call, kept until the process ends), forked from `stream` and joined
 * back to it by events; a graph captured from `stream` takes it in.  The
 * environment variable VQX_FLOAT_SUM_WAIT_TICKS (0 to 100000000, in 10 ns
 * ticks, read on each call) bounds one wait of the part on that stream for
 * the maps made on `stream` (default 100000: past it the part after them
 * does the work); the results do not depend on it.
 *
 * Errors: VQX_E_NULL; VQX_E_DIMS (nterms < 0 or > 2^36); VQX_E_NFRAMES
 * (nbuffers outside 1..65535); VQX_E_ALIGN; VQX_E_WORKSPACE; VQX_E_NO_DEVICE;
 * VQX_E_HIP (launch failure, consumed).  Argument errors come before
 * anything is queued and leave the outputs untouched.
 */
int vqx_float_sum_workspace_bytes(long long nterms, int nbuffers, size_t *bytes);
int vqx_float_running_sums_ws(const float *terms, long long nterms, int nbuffers, float *out_sums,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Measurement entry points, outside the method's contract.
 *
 * These two exist to time the streaming kernel from inside a benchmark: one
 * runs the same computation as vqx_plane_stats_batch_ws with its first
 * kernel's dispatch stamping two events, the other reads the same bytes with
 * the same access pattern and computes nothing.  No application needs
 * them; they are kept in the library (rather than in a benchmark's own
 * code) because the kernels they launch are the library's.
 * ------------------------------------------------------------------------ */

/*
 * As vqx_plane_stats_batch_ws, and also stamps two caller-created
 * hipEvent_t with the start and the end of the streaming kernel (stage 1):
 * the kernel is launched with hipExtLaunchKernel, whose dispatch records the
 * events itself, so hipEventElapsedTime gives that kernel's duration and no
 * extra packet is queued.  Either event may be NULL.  Results and errors are
 * those of vqx_plane_stats_batch_ws.
 */
int vqx_plane_stats_batch_ws_timed(const void *ref, const void *dist, int w, int h, int bpc,
                                   int nframes, uint64_t *out_noise, uint64_t *out_moments,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   void *stage1_begin, void *stage1_end);

/*
 * Computes nothing of the method.  Reads both planes with exactly the grid,
 * chunks and 16-byte loads of vqx_plane_stats_batch_ws's first kernel, but
 * without its arithmetic (an
 * XOR of every word, written nowhere), so that its duration between the
 * events its dispatch stamps (either may be NULL) is the read time of that
 * access pattern: the practical ceiling to compare that kernel with.
 * Arguments, workspace and errors are those of vqx_plane_stats_batch_ws_timed
 * without the outputs; the workspace's contents are left unspecified.
 */
int vqx_read_probe_timed(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                         void *workspace, size_t workspace_bytes, void *stream, void *begin, void *end);

#ifdef __cplusplus
}
#endif

#endif /* VQX_H */
