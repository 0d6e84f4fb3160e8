"""Bit-exact plane reductions (float_psnr and integer psnr noise, float_moment sums) on MI355X.

The product is libvqx.so (include/vqx.h): hand-written HIP kernels for
gfx950 behind a C ABI.  ``vqx`` is its thin ctypes binding over torch device
tensors and streams.
"""

from . import vqx  # noqa: F401
from .vqx import (  # noqa: F401
    VqxError,
    abi_version,
    conclude_batch,
    conclude_moments,
    conclude_psnr,
    conclude_psnr_int,
    conclude_psnr_int_batch,
    plane_stats_batch,
    plane_stats_batch_ws,
    plane_stats_host,
    plane_stats_host_workspace_bytes,
    plane_stats_planes,
    plane_stats_view,
    plane_stats_view_cpu_order,
    plane_stats_workspace_bytes,
    plane_view_workspace_bytes,
    planes_workspace_bytes,
    psnr_int_planes,
    psnr_int_view,
    status_string,
)
