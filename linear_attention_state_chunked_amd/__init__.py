"""libhypic: linear-attention state composition for position-independent caching
on AMD MI355X (gfx950).

The computation lives in libhypic.so (C ABI, include/hypic.h; HIP kernels under
csrc/).  This package is its Python binding: the functions carry the C names
and only marshal arguments, with torch providing device memory and streams.
"""

from .api import (  # noqa: F401
    hypic_compose,
    hypic_compose_noalloc,
    hypic_compose_seam,
    hypic_conv_warmup,
    hypic_device_status,
    hypic_plan_schedule,
    hypic_seam_advance,
    hypic_seam_widths,
    hypic_segment_build,
    hypic_state_rerotate,
)
from ._abi import HypicError, LIB_PATH, lib  # noqa: F401
