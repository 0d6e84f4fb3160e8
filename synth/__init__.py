"""Seeded synthetic inputs shared by the tests, the bench and the oracle's checks.

Holds random-number draws only; none of the reductions is computed here.
"""

from .workloads import (  # noqa: F401
    CHROMA,
    HVS_4K_BLOCKS,
    WORKLOADS,
    Workload,
    constant_pair,
    float_terms,
    generate,
    hvs_like_terms,
    odd_dark_bright,
    past53_fullrange,
    past53_mixed,
    planar_yuv,
    sha256,
    uniform_planes,
)
