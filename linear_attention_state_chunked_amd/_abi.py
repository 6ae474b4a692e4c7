"""ctypes mirror of include/hypic.h and the loader of libhypic.so.

Argument marshalling only: no arithmetic of the method lives here.  Loading
fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhypic.so")

# enums (values fixed by include/hypic.h)
OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_DEVICE = range(5)
F32, BF16 = 0, 1
DENSE, DIAG, SCALAR, KDA = 0, 1, 2, 3
SCHED = {"natural": 0, "lpt": 1, "rr": 2}
PREC = {"auto": 0, "f32": 1, "f16": 2, "f16_precise_t": 3}
COMPOSE = {"auto": 0, "fold": 1, "scan": 2, "naive_add": 3}
ACT = {"none": 0, "silu": 1}
KIND = {"dense": DENSE, "diag": DIAG, "scalar": SCALAR, "kda": KDA}
INLINE_SEGS = 160          # segment tables up to this size need no workspace
SEAM_SINK_DEFAULT = 8.0
COMPOSE_SEAM_MAX_W = 8
NOALLOC_SCRATCH_BYTES = 32 << 20   # fixed per-device scratch of hypic_compose_noalloc

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_enum = C.c_int


class BuildDesc(C.Structure):
    _fields_ = [
        ("kind", _enum), ("in_dtype", _enum), ("n_batch", _i32), ("n_tokens", _i64),
        ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32), ("chunk", _i32),
        ("n_seg", _i32), ("cu_seqlens", _p), ("skip_head", _i32), ("qk_l2norm", _i32),
        ("k", _p), ("v", _p), ("log_alpha", _p), ("beta", _p),
        ("T_hat", _p), ("T_exp", _p), ("S", _p),
        ("schedule", _enum), ("precision", _enum), ("workspace", _p), ("workspace_bytes", C.c_size_t),
        ("q", _p), ("o", _p), ("out_dtype", _enum),
    ]


class ComposeDesc(C.Structure):
    _fields_ = [
        ("kind", _enum), ("n_chain", _i32), ("d_k", _i32), ("d_v", _i32), ("n_elem", _i32),
        ("n_slot", _i32), ("slot", _p), ("T_hat", _p), ("T_exp", _p), ("S", _p), ("S0", _p),
        ("S_final", _p), ("S_prefix", _p), ("T_total", _p), ("T_total_exp", _p),
        ("mode", _enum), ("scan_block", _i32), ("workspace", _p), ("workspace_bytes", C.c_size_t),
    ]


class SeamDesc(C.Structure):
    _fields_ = [
        ("in_dtype", _enum), ("out_dtype", _enum), ("n_batch", _i32), ("n_tokens", _i64),
        ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32), ("n_seam", _i32),
        ("cu_seam", _p), ("qk_l2norm", _i32), ("q", _p), ("k", _p), ("v", _p),
        ("log_alpha", _p), ("beta", _p), ("S_in", _p), ("state_stride", _i64),
        ("o", _p), ("S_out", _p), ("T_hat", _p), ("T_exp", _p), ("S_seam", _p),
        ("precision", _enum), ("workspace", _p), ("workspace_bytes", C.c_size_t),
    ]


class ConvDesc(C.Structure):
    _fields_ = [
        ("in_dtype", _enum), ("out_dtype", _enum), ("n_batch", _i32), ("n_tokens", _i64),
        ("channels", _i32), ("width", _i32), ("n_seg", _i32), ("cu_seqlens", _p),
        ("x", _p), ("state_in", _p), ("n_state", _i32), ("state_index", _p),
        ("weight", _p), ("bias", _p), ("activation", _enum), ("y", _p), ("state_out", _p),
        ("workspace", _p), ("workspace_bytes", C.c_size_t),
    ]


class SeamComposeDesc(C.Structure):
    _fields_ = [
        ("n_batch", _i32), ("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32), ("n_elem", _i32),
        ("n_slot", _i32), ("slot", _p), ("T_hat", _p), ("T_exp", _p), ("S", _p), ("S0", _p), ("S_final", _p),
        ("S_prefix", _p), ("in_dtype", _enum), ("out_dtype", _enum), ("n_tokens", _i64), ("cu_seam", _p),
        ("qk_l2norm", _i32), ("q", _p), ("k", _p), ("v", _p), ("log_alpha", _p), ("beta", _p), ("o", _p),
        ("workspace", _p), ("workspace_bytes", C.c_size_t),
    ]


class RerotateDesc(C.Structure):
    _fields_ = [
        ("kind", _enum), ("n_elem", _i32), ("n_chain", _i32), ("d_k", _i32), ("d_v", _i32),
        ("rotary_dim", _i32), ("interleaved", _i32), ("rope_base", C.c_double), ("delta", _p),
        ("T_hat_in", _p), ("T_hat_out", _p), ("S_in", _p), ("S_out", _p),
    ]


EXPORTS = {
    "hypic_segment_build": ([C.POINTER(BuildDesc), _p], _enum),
    "hypic_segment_build_workspace_bytes": ([C.POINTER(BuildDesc)], C.c_size_t),
    "hypic_compose": ([C.POINTER(ComposeDesc), _p], _enum),
    "hypic_compose_workspace_bytes": ([C.POINTER(ComposeDesc)], C.c_size_t),
    "hypic_compose_noalloc": ([C.POINTER(ComposeDesc), _p], _enum),
    "hypic_seam_advance": ([C.POINTER(SeamDesc), _p], _enum),
    "hypic_compose_seam": ([C.POINTER(SeamComposeDesc), _p], _enum),
    "hypic_compose_seam_workspace_bytes": ([C.POINTER(SeamComposeDesc)], C.c_size_t),
    "hypic_seam_advance_workspace_bytes": ([C.POINTER(SeamDesc)], C.c_size_t),
    "hypic_conv_warmup": ([C.POINTER(ConvDesc), _p], _enum),
    "hypic_conv_warmup_workspace_bytes": ([C.POINTER(ConvDesc)], C.c_size_t),
    "hypic_plan_schedule": ([_p, _i32, _i32, _enum, _p, _p, _p], _enum),
    "hypic_state_rerotate": ([C.POINTER(RerotateDesc), _p], _enum),
    "hypic_seam_widths": ([_p, _i32, C.c_double, _p], _enum),
    "hypic_device_status": ([], _enum),
    "hypic_last_error": ([], C.c_char_p),
    "hypic_version": ([], C.c_int),
}

_lib = None


def lib() -> C.CDLL:
    """Load libhypic.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libhypic.so not found at {LIB_PATH}: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        for name, (argtypes, restype) in EXPORTS.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = L
    return _lib


class HypicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hypic status {status}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != OK:
        raise HypicError(status, lib().hypic_last_error().decode())
