"""ctypes binding of libvqx (include/vqx.h), same names without the prefix.

Argument marshalling only: every step of the reduction runs in libvqx's HIP
kernels, and the conclusions in libvqx's host code.  Torch supplies device
memory and the current stream.  There is no fallback: if libvqx.so is not
built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libvqx.so")

OK = 0
(E_NULL, E_DIMS, E_BPC, E_NFRAMES, E_ALIGN, E_WORKSPACE, E_HIP, E_NO_DEVICE, E_STRIDE, E_PLANES,
 E_SCRATCH) = range(-1, -12, -1)
MAX_PIXELS = 1 << 25
NOALLOC_SCRATCH_BYTES = 4 << 20

# Every symbol include/vqx.h declares.
SYMBOLS = (
    "vqx_abi_version",
    "vqx_status_string",
    "vqx_plane_stats_workspace_bytes",
    "vqx_plane_stats_batch",
    "vqx_plane_stats_batch_noalloc",
    "vqx_plane_stats_batch_ws",
    "vqx_plane_stats_batch_ws_timed",
    "vqx_read_probe_timed",
    "vqx_plane_stats_cpu_order_workspace_bytes",
    "vqx_plane_stats_batch_cpu_order_ws",
    "vqx_conclude_psnr",
    "vqx_conclude_moments",
    "vqx_conclude_batch",
    "vqx_plane_view_workspace_bytes",
    "vqx_plane_stats_view_ws",
    "vqx_psnr_int_view_ws",
    "vqx_conclude_psnr_int",
    "vqx_conclude_psnr_int_batch",
    "vqx_plane_stats_host_workspace_bytes",
    "vqx_plane_stats_host_ws",
    "vqx_plane_stats_view_cpu_order_workspace_bytes",
    "vqx_plane_stats_view_cpu_order_ws",
    "vqx_planes_workspace_bytes",
    "vqx_plane_stats_planes_ws",
    "vqx_psnr_int_planes_ws",
    "vqx_float_sum_workspace_bytes",
    "vqx_float_running_sums_ws",
)


class VqxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libvqx; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run __graft_entry__.build()")
        # torch ships its own HIP runtime; load it first so that libvqx binds
        # to that one (same soname) and stream handles mean the same thing.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIBRARY)
        vp, i, u64, sz, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_double
        i64 = ctypes.c_int64
        sigs = {
            "vqx_abi_version": (i, []),
            "vqx_status_string": (ctypes.c_char_p, [i]),
            "vqx_plane_stats_workspace_bytes": (i, [i, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_batch": (i, [vp, vp, i, i, i, i, vp, vp, vp]),
            "vqx_plane_stats_batch_noalloc": (i, [vp, vp, i, i, i, i, vp, vp, vp]),
            "vqx_plane_stats_batch_ws": (i, [vp, vp, i, i, i, i, vp, vp, vp, sz, vp]),
            "vqx_plane_stats_batch_ws_timed": (i, [vp, vp, i, i, i, i, vp, vp, vp, sz, vp, vp, vp]),
            "vqx_read_probe_timed": (i, [vp, vp, i, i, i, i, vp, sz, vp, vp, vp]),
            "vqx_plane_stats_cpu_order_workspace_bytes": (i, [i, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_batch_cpu_order_ws": (i, [vp, vp, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]),
            "vqx_conclude_psnr": (i, [u64, i, i, i, d, ctypes.POINTER(d), ctypes.POINTER(d)]),
            "vqx_conclude_moments": (i, [vp, i, i, i, vp]),
            "vqx_conclude_batch": (i, [vp, vp, i, i, i, i, d, vp]),
            "vqx_plane_view_workspace_bytes": (i, [i, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_view_ws": (i, [vp, i64, i64, vp, i64, i64, i, i, i, i, vp, vp, vp, sz, vp]),
            "vqx_psnr_int_view_ws": (i, [vp, i64, i64, vp, i64, i64, i, i, i, i, vp, vp, sz, vp]),
            "vqx_conclude_psnr_int": (i, [u64, i, i, i, d, ctypes.POINTER(d), ctypes.POINTER(d)]),
            "vqx_conclude_psnr_int_batch": (i, [vp, i, i, i, i, d, vp]),
            "vqx_plane_stats_host_workspace_bytes": (i, [i, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_host_ws": (i, [vp, vp, i, i, i, i, i, vp, vp, vp, sz, vp, vp]),
            "vqx_plane_stats_view_cpu_order_workspace_bytes": (i, [i, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_view_cpu_order_ws": (i, [vp, i64, i64, vp, i64, i64, i, i, i, i, vp, vp, vp, vp, vp,
                                                      sz, vp]),
            "vqx_planes_workspace_bytes": (i, [vp, i, i, i, ctypes.POINTER(sz)]),
            "vqx_plane_stats_planes_ws": (i, [vp, i, i, i, vp, vp, vp, sz, vp]),
            "vqx_psnr_int_planes_ws": (i, [vp, i, i, i, vp, vp, sz, vp]),
            "vqx_float_sum_workspace_bytes": (i, [ctypes.c_longlong, i, ctypes.POINTER(sz)]),
            "vqx_float_running_sums_ws": (i, [vp, ctypes.c_longlong, i, vp, vp, sz, vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime already mapped into this process (torch's), for the
    event calls of the bench; never a second copy."""
    lib()
    with open("/proc/self/maps") as f:
        paths = sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    if not paths:
        raise RuntimeError("no HIP runtime is loaded")
    return ctypes.CDLL(paths[0])


def abi_version() -> int:
    return lib().vqx_abi_version()


def status_string(status: int) -> str:
    return lib().vqx_status_string(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise VqxError(status, where)


def plane_stats_workspace_bytes(w: int, h: int, bpc: int, nframes: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().vqx_plane_stats_workspace_bytes(w, h, bpc, nframes, ctypes.byref(out)),
           "plane_stats_workspace_bytes")
    return out.value


def _planes(ref, dist, bpc):
    import torch
    if ref.dim() == 2:
        ref, dist = ref.unsqueeze(0), dist.unsqueeze(0)
    if ref.dim() != 3 or ref.shape != dist.shape:
        raise ValueError("ref and dist must both be [nframes][h][w] (or [h][w])")
    want = (torch.uint8,) if bpc == 8 else (torch.uint16, torch.int16)
    if ref.dtype not in want or dist.dtype not in want:
        raise TypeError(f"bpc {bpc} wants {'uint8' if bpc == 8 else 'uint16'} samples")
    if not (ref.is_cuda and dist.is_cuda and ref.device == dist.device):
        raise ValueError("ref and dist must be on one GPU")
    if not (ref.is_contiguous() and dist.is_contiguous()):
        raise ValueError("ref and dist must be contiguous")
    return ref, dist


def _stream_handle(device, stream):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def plane_stats_batch_ws(ref, dist, bpc: int, out_noise, out_moments, workspace, stream=None):
    """Queue the five sums of every frame into ``out_noise`` [F] and
    ``out_moments`` [F][4] (int64 device tensors), with a caller workspace
    (a device tensor of at least plane_stats_workspace_bytes bytes)."""
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    _check(lib().vqx_plane_stats_batch_ws(
        ref.data_ptr(), dist.data_ptr(), w, h, bpc, f, out_noise.data_ptr(), out_moments.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(ref.device, stream)), "plane_stats_batch_ws")
    return out_noise, out_moments


def plane_stats_batch_ws_timed(ref, dist, bpc: int, out_noise, out_moments, workspace,
                               stage1_begin, stage1_end, stream=None):
    """plane_stats_batch_ws that records two hipEvent_t handles (ints) around
    the streaming kernel on the stream."""
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    _check(lib().vqx_plane_stats_batch_ws_timed(
        ref.data_ptr(), dist.data_ptr(), w, h, bpc, f, out_noise.data_ptr(), out_moments.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(ref.device, stream), stage1_begin, stage1_end), "plane_stats_batch_ws_timed")
    return out_noise, out_moments


def plane_stats_batch(ref, dist, bpc: int, stream=None, out_noise=None, out_moments=None):
    """The five exact sums of every frame: ``(noise [F], moments [F][4])`` as
    int64 device tensors (the uint64 values, all below 2^58).  The workspace
    comes from torch's caching allocator; the call only queues work on the
    current (or given) stream."""
    import torch
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    dev = ref.device
    if out_noise is None:
        out_noise = torch.empty(f, dtype=torch.int64, device=dev)
    if out_moments is None:
        out_moments = torch.empty((f, 4), dtype=torch.int64, device=dev)
    ws = torch.empty(plane_stats_workspace_bytes(w, h, bpc, f), dtype=torch.uint8, device=dev)
    return plane_stats_batch_ws(ref, dist, bpc, out_noise, out_moments, ws, stream)


def plane_stats_cpu_order_workspace_bytes(w: int, h: int, bpc: int, nframes: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().vqx_plane_stats_cpu_order_workspace_bytes(w, h, bpc, nframes, ctypes.byref(out)),
           "plane_stats_cpu_order_workspace_bytes")
    return out.value


def plane_stats_batch_cpu_order(ref, dist, bpc: int, stream=None):
    """The exact sums and the CPU's running double sums of every frame:
    ``(noise [F], moments [F][4], cpu_noise [F], cpu_moments [F][4])`` as
    int64 device tensors.  The CPU's sums are the values its sequential
    double accumulators hold (times the unit), bit for bit, also past 2^53."""
    import torch
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    dev = ref.device
    out = torch.empty((2, 5 * f), dtype=torch.int64, device=dev)
    ws = torch.empty(plane_stats_cpu_order_workspace_bytes(w, h, bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_plane_stats_batch_cpu_order_ws(
        ref.data_ptr(), dist.data_ptr(), w, h, bpc, f, out[0, :f].data_ptr(), out[0, f:].data_ptr(),
        out[1, :f].data_ptr(), out[1, f:].data_ptr(), ws.data_ptr(), ws.numel(),
        _stream_handle(dev, stream)), "plane_stats_batch_cpu_order_ws")
    return out[0, :f], out[0, f:].view(f, 4), out[1, :f], out[1, f:].view(f, 4)


def plane_stats_batch_noalloc(ref, dist, bpc: int, out_noise, out_moments, stream=None):
    """vqx_plane_stats_batch_noalloc: the five sums into ``out_noise`` [F]
    and ``out_moments`` [F][4] (int64 device tensors), with the library's
    fixed per-GPU scratch and no allocation; calls that overlap on one GPU
    race on that scratch."""
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    _check(lib().vqx_plane_stats_batch_noalloc(
        ref.data_ptr(), dist.data_ptr(), w, h, bpc, f, out_noise.data_ptr(), out_moments.data_ptr(),
        _stream_handle(ref.device, stream)), "plane_stats_batch_noalloc")
    return out_noise, out_moments


def plane_stats_batch_selfalloc(ref, dist, bpc: int, out_noise, out_moments, stream=None):
    """vqx_plane_stats_batch itself: the library allocates its scratch with
    hipMallocAsync on the stream."""
    ref, dist = _planes(ref, dist, bpc)
    f, h, w = ref.shape
    _check(lib().vqx_plane_stats_batch(
        ref.data_ptr(), dist.data_ptr(), w, h, bpc, f, out_noise.data_ptr(), out_moments.data_ptr(),
        _stream_handle(ref.device, stream)), "plane_stats_batch")
    return out_noise, out_moments


def conclude_psnr(noise: int, w: int, h: int, bpc: int, psnr_max: float = 0.0):
    """(mse, psnr_db) of one frame from its exact noise (host)."""
    mse, db = ctypes.c_double(), ctypes.c_double()
    _check(lib().vqx_conclude_psnr(int(noise), w, h, bpc, float(psnr_max), ctypes.byref(mse),
                                   ctypes.byref(db)), "conclude_psnr")
    return mse.value, db.value


def conclude_moments(sums4, w: int, h: int, bpc: int) -> np.ndarray:
    """The four means of one frame from {ref1, dist1, ref2, dist2} (host)."""
    s = np.ascontiguousarray(np.asarray(sums4, dtype=np.uint64).reshape(4))
    out = np.zeros(4, dtype=np.float64)
    _check(lib().vqx_conclude_moments(s.ctypes.data, w, h, bpc, out.ctypes.data), "conclude_moments")
    return out


def conclude_batch(noise, moments, w: int, h: int, bpc: int, psnr_max: float = 0.0) -> np.ndarray:
    """[F][6] {mse, psnr_db, ref_mean, dist_mean, ref_mean_sq, dist_mean_sq}
    from host copies of the sums (numpy or CPU tensors)."""
    n = np.ascontiguousarray(np.asarray(noise).astype(np.uint64).reshape(-1))
    m = np.ascontiguousarray(np.asarray(moments).astype(np.uint64).reshape(-1, 4))
    f = n.shape[0]
    if m.shape[0] != f:
        raise ValueError("noise and moments disagree on nframes")
    out = np.zeros((f, 6), dtype=np.float64)
    _check(lib().vqx_conclude_batch(n.ctypes.data, m.ctypes.data, w, h, bpc, f, float(psnr_max),
                                    out.ctypes.data), "conclude_batch")
    return out


# ------------------------------------------------------------- plane views
def plane_view_workspace_bytes(w: int, h: int, bpc: int, nframes: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().vqx_plane_view_workspace_bytes(w, h, bpc, nframes, ctypes.byref(out)),
           "plane_view_workspace_bytes")
    return out.value


def _view(t, bpc):
    """(base pointer, row stride, frame stride) of a [F][h][w] (or [h][w])
    tensor view whose samples are adjacent along w: slices of larger planes,
    chroma planes of planar YUV frames, padded pitches."""
    import torch
    if t.dim() == 2:
        t = t.unsqueeze(0)
    if t.dim() != 3:
        raise ValueError("a plane view is [nframes][h][w] or [h][w]")
    want = (torch.uint8,) if bpc == 8 else (torch.uint16, torch.int16)
    if t.dtype not in want:
        raise TypeError(f"bpc {bpc} wants {'uint8' if bpc == 8 else 'uint16'} samples")
    if not t.is_cuda:
        raise ValueError("plane views must be on the GPU")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("samples of a row must be adjacent (stride 1 along w)")
    row = t.stride(1) if t.shape[1] > 1 else t.shape[2]
    frame = t.stride(0) if t.shape[0] > 1 else 0
    return t, t.data_ptr(), row, frame


def _views(ref, dist, bpc):
    ref, rp, rr, rf = _view(ref, bpc)
    dist, dp, dr, df = _view(dist, bpc)
    if ref.shape != dist.shape or ref.device != dist.device:
        raise ValueError("ref and dist views differ in shape or device")
    return ref, (rp, rr, rf, dp, dr, df)


def plane_stats_view(ref, dist, bpc: int, stream=None):
    """The five exact sums of every frame over plane views (tensor views of
    any row and frame stride): ``(noise [F], moments [F][4])`` as int64
    device tensors."""
    import torch
    ref, args = _views(ref, dist, bpc)
    f, h, w = ref.shape
    dev = ref.device
    out = torch.empty(5 * f, dtype=torch.int64, device=dev)
    ws = torch.empty(plane_view_workspace_bytes(w, h, bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_plane_stats_view_ws(*args, w, h, bpc, f, out[:f].data_ptr(), out[f:].data_ptr(),
                                         ws.data_ptr(), ws.numel(), _stream_handle(dev, stream)),
           "plane_stats_view_ws")
    return out[:f], out[f:].view(f, 4)


def psnr_int_view(ref, dist, bpc: int, stream=None):
    """The integer psnr noise of every frame over plane views: int64 [F]
    device tensor of exact sums of (ref - dist)^2."""
    import torch
    ref, args = _views(ref, dist, bpc)
    f, h, w = ref.shape
    dev = ref.device
    out = torch.empty(f, dtype=torch.int64, device=dev)
    ws = torch.empty(plane_view_workspace_bytes(w, h, bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_psnr_int_view_ws(*args, w, h, bpc, f, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                      _stream_handle(dev, stream)), "psnr_int_view_ws")
    return out


def plane_stats_view_cpu_order_workspace_bytes(w: int, h: int, bpc: int, nframes: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().vqx_plane_stats_view_cpu_order_workspace_bytes(w, h, bpc, nframes, ctypes.byref(out)),
           "plane_stats_view_cpu_order_workspace_bytes")
    return out.value


def plane_stats_view_cpu_order(ref, dist, bpc: int, stream=None):
    """plane_stats_batch_cpu_order over plane views (any row and frame
    stride): ``(noise [F], moments [F][4], cpu_noise [F], cpu_moments
    [F][4])`` as int64 device tensors."""
    import torch
    ref, args = _views(ref, dist, bpc)
    f, h, w = ref.shape
    dev = ref.device
    out = torch.empty((2, 5 * f), dtype=torch.int64, device=dev)
    ws = torch.empty(plane_stats_view_cpu_order_workspace_bytes(w, h, bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_plane_stats_view_cpu_order_ws(*args, w, h, bpc, f, out[0, :f].data_ptr(), out[0, f:].data_ptr(),
                                                   out[1, :f].data_ptr(), out[1, f:].data_ptr(), ws.data_ptr(),
                                                   ws.numel(), _stream_handle(dev, stream)),
           "plane_stats_view_cpu_order_ws")
    return out[0, :f], out[0, f:].view(f, 4), out[1, :f], out[1, f:].view(f, 4)


MAX_PLANES = 4


class PlanePair(ctypes.Structure):
    """vqx_plane_pair: a ref view and a dist view of one plane, and its size."""
    _fields_ = [("ref", ctypes.c_void_p), ("ref_row_stride", ctypes.c_int64), ("ref_frame_stride", ctypes.c_int64),
                ("dist", ctypes.c_void_p), ("dist_row_stride", ctypes.c_int64),
                ("dist_frame_stride", ctypes.c_int64), ("w", ctypes.c_int), ("h", ctypes.c_int)]


def plane_pairs(pairs, bpc: int):
    """A ctypes array of PlanePair from [(ref view, dist view), ...] tensor
    views (each [F][h][w] or [h][w], any row and frame stride), the views kept
    alive alongside; every plane must have the same number of frames."""
    arr = (PlanePair * max(1, len(pairs)))()
    keep, frames = [], set()
    for k, (ref, dist) in enumerate(pairs):
        ref, (rp, rr, rf, dp, dr, df) = _views(ref, dist, bpc)
        f, h, w = ref.shape
        frames.add(f)
        keep.append((ref, dist))
        arr[k] = PlanePair(rp, rr, rf, dp, dr, df, w, h)
    if len(frames) > 1:
        raise ValueError("every plane needs the same number of frames")
    return arr, keep, (frames.pop() if frames else 0)


def planes_workspace_bytes(sizes, bpc: int, nframes: int) -> int:
    """Device scratch of the several-planes entry points for planes of
    sizes [(w, h), ...]."""
    arr = (PlanePair * max(1, len(sizes)))()
    for k, (w, h) in enumerate(sizes):
        arr[k].w, arr[k].h = w, h
    out = ctypes.c_size_t(0)
    _check(lib().vqx_planes_workspace_bytes(arr, len(sizes), bpc, nframes, ctypes.byref(out)),
           "planes_workspace_bytes")
    return out.value


def plane_stats_planes(pairs, bpc: int, stream=None):
    """The five exact sums of every plane of every frame, all planes in one
    launch of each stage: ``(noise [P][F], moments [P][F][4])`` int64 device
    tensors."""
    import torch
    arr, keep, f = plane_pairs(pairs, bpc)
    n = len(pairs)
    dev = keep[0][0].device if keep else torch.device("cuda")
    out = torch.empty(5 * n * f, dtype=torch.int64, device=dev)
    ws = torch.empty(planes_workspace_bytes([(a.w, a.h) for a in arr[:n]], bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_plane_stats_planes_ws(arr, n, bpc, f, out[:n * f].data_ptr(), out[n * f:].data_ptr(),
                                           ws.data_ptr(), ws.numel(), _stream_handle(dev, stream)),
           "plane_stats_planes_ws")
    return out[:n * f].view(n, f), out[n * f:].view(n, f, 4)


def psnr_int_planes(pairs, bpc: int, stream=None):
    """The integer psnr noise of every plane of every frame, all planes in one
    launch of each stage: int64 [P][F] device tensor."""
    import torch
    arr, keep, f = plane_pairs(pairs, bpc)
    n = len(pairs)
    dev = keep[0][0].device if keep else torch.device("cuda")
    out = torch.empty(n * f, dtype=torch.int64, device=dev)
    ws = torch.empty(planes_workspace_bytes([(a.w, a.h) for a in arr[:n]], bpc, f), dtype=torch.uint8, device=dev)
    _check(lib().vqx_psnr_int_planes_ws(arr, n, bpc, f, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                        _stream_handle(dev, stream)), "psnr_int_planes_ws")
    return out.view(n, f)


def conclude_psnr_int(noise: int, w: int, h: int, bpc: int, psnr_max: float = 0.0):
    """(mse, psnr_db) of the integer psnr twin from one exact noise (host)."""
    mse, db = ctypes.c_double(), ctypes.c_double()
    _check(lib().vqx_conclude_psnr_int(int(noise), w, h, bpc, float(psnr_max), ctypes.byref(mse),
                                       ctypes.byref(db)), "conclude_psnr_int")
    return mse.value, db.value


def conclude_psnr_int_batch(noise, w: int, h: int, bpc: int, psnr_max: float = 0.0) -> np.ndarray:
    """[F][2] {mse, psnr_db} of the integer psnr twin from host noises."""
    n = np.ascontiguousarray(np.asarray(noise).astype(np.uint64).reshape(-1))
    out = np.zeros((n.shape[0], 2), dtype=np.float64)
    _check(lib().vqx_conclude_psnr_int_batch(n.ctypes.data, w, h, bpc, n.shape[0], float(psnr_max),
                                             out.ctypes.data), "conclude_psnr_int_batch")
    return out


# ---------------------------------------------------------- host-fed batches
def plane_stats_host_workspace_bytes(w: int, h: int, bpc: int, frames_per_upload: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().vqx_plane_stats_host_workspace_bytes(w, h, bpc, frames_per_upload, ctypes.byref(out)),
           "plane_stats_host_workspace_bytes")
    return out.value


def plane_stats_host(ref, dist, bpc: int, frames_per_upload: int = 4, device=0, stream=None, copy_stream=None):
    """The five exact sums of a batch held in host memory (CPU tensors,
    pinned for overlap, or numpy arrays), uploaded frames_per_upload frames
    at a time while earlier uploads are reduced.  Returns ``(noise [F],
    moments [F][4])`` as int64 device tensors; the call returns when all is
    done."""
    import torch
    r = torch.as_tensor(ref)
    d = torch.as_tensor(dist)
    if r.dim() == 2:
        r, d = r.unsqueeze(0), d.unsqueeze(0)
    if r.dim() != 3 or r.shape != d.shape:
        raise ValueError("ref and dist must both be [nframes][h][w] (or [h][w])")
    want = (torch.uint8,) if bpc == 8 else (torch.uint16, torch.int16)
    if r.dtype not in want or d.dtype not in want:
        raise TypeError(f"bpc {bpc} wants {'uint8' if bpc == 8 else 'uint16'} samples")
    if r.is_cuda or d.is_cuda or not (r.is_contiguous() and d.is_contiguous()):
        raise ValueError("ref and dist must be contiguous host tensors")
    f, h, w = r.shape
    dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
    out = torch.empty(5 * f, dtype=torch.int64, device=dev)
    ws = torch.empty(plane_stats_host_workspace_bytes(w, h, bpc, frames_per_upload), dtype=torch.uint8,
                     device=dev)
    cs = copy_stream.cuda_stream if copy_stream is not None else None
    _check(lib().vqx_plane_stats_host_ws(r.data_ptr(), d.data_ptr(), w, h, bpc, f, frames_per_upload,
                                         out[:f].data_ptr(), out[f:].data_ptr(), ws.data_ptr(), ws.numel(),
                                         _stream_handle(dev, stream), cs), "plane_stats_host_ws")
    return out[:f], out[f:].view(f, 4)


def float_sum_workspace_bytes(nterms: int, nbuffers: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().vqx_float_sum_workspace_bytes(nterms, nbuffers, ctypes.byref(out)), "float_sum_workspace_bytes")
    return out.value


def float_running_sums(terms, stream=None, out=None, workspace=None):
    """The psnr_hvs running float sums: for ``terms`` [nbuffers][nterms]
    float32 on the device, a [nbuffers] float32 device tensor with each
    buffer's terms added one by one, in order, into a float from zero
    (vqx_float_running_sums_ws).  The workspace comes from torch's caching
    allocator unless given."""
    import torch
    if terms.dtype != torch.float32 or not terms.is_cuda:
        raise TypeError("terms must be a float32 device tensor")
    if terms.dim() == 1:
        terms = terms.unsqueeze(0)
    if terms.dim() != 2 or not terms.is_contiguous():
        raise ValueError("terms must be a contiguous [nbuffers][nterms] tensor")
    nb, n = terms.shape
    if out is None:
        out = torch.empty(nb, dtype=torch.float32, device=terms.device)
    need = float_sum_workspace_bytes(n, nb)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=terms.device)
    _check(lib().vqx_float_running_sums_ws(terms.data_ptr(), n, nb, out.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(),
                                           _stream_handle(terms.device, stream)), "float_running_sums_ws")
    return out
