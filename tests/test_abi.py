"""C-ABI checks that run without a GPU.

Every entry point validates its arguments on the host before any HIP call, so
invalid descriptors are rejected here with the documented status and message.
No test in this file makes a call that would reach the device.
"""

import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
from linear_attention_state_chunked_amd import _abi as A
from linear_attention_state_chunked_amd.api import hypic_plan_schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")


@pytest.fixture(scope="module")
def L():
    return A.lib()


def test_every_declared_symbol_is_exported(L):
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:hypic_status|size_t|const char\*|int)\s+(hypic_\w+)\s*\(", src, re.M))
    assert len(declared) == 17
    assert declared == set(A.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (hypic_\w+)", out))
    assert declared <= exported
    for name in declared:
        assert getattr(L, name) is not None


def test_probe_library_exports_its_declared_symbols():
    """libhypic_probe (the matrix-core rate probe the benchmark reports beside the build's rate) exports
    what include/hypic_probe.h declares; its flop count is the product count times 32 x 32 x 16 x 2."""
    src = open(os.path.join(ROOT, "include", "hypic_probe.h")).read()
    declared = set(re.findall(r"^\s*(?:int|double)\s+(hypic_probe_\w+)\s*\(", src, re.M))
    assert declared == {"hypic_probe_mfma_f16", "hypic_probe_mfma_f16_flops"}
    path = os.path.join(os.path.dirname(A.LIB_PATH), "libhypic_probe.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert declared <= set(re.findall(r"\bT (hypic_probe_\w+)", out))
    P = C.CDLL(path)
    P.hypic_probe_mfma_f16_flops.argtypes = [C.c_int, C.c_int]
    P.hypic_probe_mfma_f16_flops.restype = C.c_double
    assert P.hypic_probe_mfma_f16_flops(3, 5) == 3 * 8 * 5 * 4 * 32 * 32 * 16 * 2
    # invalid arguments are rejected on the host, before any HIP call
    P.hypic_probe_mfma_f16.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    P.hypic_probe_mfma_f16.restype = C.c_int
    assert P.hypic_probe_mfma_f16(0, 5, None, None, None) == -1
    assert P.hypic_probe_mfma_f16(4, 5, None, None, None) == -1


def test_struct_layouts_match_the_header(tmp_path):
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "hypic.h"', "int main(void) {"]
    structs = {"hypic_build_desc": A.BuildDesc, "hypic_compose_desc": A.ComposeDesc,
               "hypic_seam_desc": A.SeamDesc, "hypic_conv_desc": A.ConvDesc, "hypic_rerotate_desc": A.RerotateDesc,
               "hypic_seam_compose_desc": A.SeamComposeDesc}
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == C.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_version(L):
    assert L.hypic_version() == 1


def _build_desc(**kw):
    cu = kw.pop("_cu", np.array([0, 64, 128], np.int64))
    d = A.BuildDesc(kind=A.DENSE, in_dtype=A.BF16, n_batch=1, n_tokens=128, h_k=1, h_v=2, d_k=128, d_v=128,
                    chunk=64, n_seg=len(cu) - 1, cu_seqlens=cu.ctypes.data, skip_head=0, qk_l2norm=0,
                    k=0x1000, v=0x2000, log_alpha=0x3000, beta=0x4000, T_hat=0x5000, T_exp=0x6000, S=0x7000,
                    schedule=0, precision=0, workspace=0x10000, workspace_bytes=0)
    for key, val in kw.items():
        setattr(d, key, val)
    return d, cu


@pytest.mark.parametrize("field,value,status,msg", [
    ("chunk", 32, A.ERR_UNSUPPORTED, "chunk"),
    ("d_k", 96, A.ERR_UNSUPPORTED, "d_k"),
    ("d_v", 64, A.ERR_UNSUPPORTED, "d_k"),
    ("h_k", 3, A.ERR_INVALID_ARGUMENT, "multiple"),
    ("kind", 7, A.ERR_INVALID_ARGUMENT, "kind"),
    ("in_dtype", 5, A.ERR_INVALID_ARGUMENT, "in_dtype"),
    ("n_batch", 0, A.ERR_INVALID_ARGUMENT, "geometry"),
    ("skip_head", -1, A.ERR_INVALID_ARGUMENT, "skip_head"),
    ("beta", None, A.ERR_INVALID_ARGUMENT, "beta"),
    ("k", 0x1002, A.ERR_INVALID_ARGUMENT, "aligned"),
    ("T_exp", None, A.ERR_INVALID_ARGUMENT, "T_hat and T_exp"),
    ("S", None, A.ERR_INVALID_ARGUMENT, "S is NULL"),
    ("schedule", 9, A.ERR_INVALID_ARGUMENT, "schedule"),
    ("qk_l2norm", 2, A.ERR_INVALID_ARGUMENT, "qk_l2norm"),
])
def test_build_rejects_bad_descriptors(L, field, value, status, msg):
    d, cu = _build_desc(**{field: value})
    assert L.hypic_segment_build(C.byref(d), None) == status
    assert msg in L.hypic_last_error().decode()


def test_build_offsets_and_workspace(L):
    for cu, msg in ((np.array([1, 64], np.int64), "must be 0"), (np.array([0, 64, 32], np.int64), "decreasing"),
                    (np.array([0, 64, 200], np.int64), "exceeds n_tokens")):
        d, _ = _build_desc(_cu=cu)
        assert L.hypic_segment_build(C.byref(d), None) == A.ERR_INVALID_ARGUMENT
        assert msg in L.hypic_last_error().decode()
    # a table of at most INLINE_SEGS segments travels in the kernel arguments: no workspace
    d, cu = _build_desc()
    assert L.hypic_segment_build_workspace_bytes(C.byref(d)) == 0
    d, cu = _build_desc(schedule=A.SCHED["lpt"])
    assert L.hypic_segment_build_workspace_bytes(C.byref(d)) == 0
    # a larger one is uploaded into the workspace: starts, lengths and the segment order
    n = A.INLINE_SEGS + 1
    big = np.arange(0, 64 * (n + 1), 64, dtype=np.int64)
    d, cu = _build_desc(_cu=big, n_tokens=int(big[-1]))
    need = L.hypic_segment_build_workspace_bytes(C.byref(d))
    assert need >= n * (8 + 4 + 4) and need % 256 == 0
    d.workspace_bytes = need - 1
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_WORKSPACE_TOO_SMALL
    d.workspace = None
    d.workspace_bytes = need
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_WORKSPACE_TOO_SMALL
    d.workspace = 0x10010
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_INVALID_ARGUMENT
    assert "256-byte aligned" in L.hypic_last_error().decode()
    # the F32 operand plan needs d = 64; AUTO does not hand float32 inputs at d = 128 to f16
    d, cu = _build_desc(precision=A.PREC["f32"])
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_UNSUPPORTED
    d, cu = _build_desc(in_dtype=A.F32, precision=A.PREC["auto"])
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_UNSUPPORTED
    assert "HYPIC_PREC_F16" in L.hypic_last_error().decode()
    # diagonal kind: beta must be NULL, l2norm unsupported
    d, cu = _build_desc(kind=A.DIAG)
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_INVALID_ARGUMENT
    d, cu = _build_desc(kind=A.DIAG, beta=None, qk_l2norm=1)
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_UNSUPPORTED


def test_empty_build_is_a_no_op(L):
    cu = np.array([0], np.int64)
    d, _ = _build_desc(_cu=cu, n_seg=0, workspace=None)
    assert L.hypic_segment_build(C.byref(d), None) == A.OK


def _compose_desc(**kw):
    d = A.ComposeDesc(kind=A.DENSE, n_chain=4, d_k=128, d_v=128, n_elem=8, n_slot=8, slot=None, T_hat=0x1000,
                      T_exp=0x2000, S=0x3000, S0=None, S_final=0x4000, S_prefix=None, T_total=None,
                      T_total_exp=None, mode=A.COMPOSE["scan"], scan_block=0, workspace=None, workspace_bytes=0)
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def test_compose_validation(L):
    cases = [
        (dict(n_slot=4), A.ERR_INVALID_ARGUMENT, "n_slot"),
        (dict(S_final=None), A.ERR_INVALID_ARGUMENT, "S_final"),
        (dict(T_hat=None), A.ERR_INVALID_ARGUMENT, "T_hat and T_exp"),
        (dict(T_total=0x5000), A.ERR_INVALID_ARGUMENT, "T_total"),
        (dict(mode=A.COMPOSE["naive_add"], T_total=0x5000, T_total_exp=0x6000), A.ERR_INVALID_ARGUMENT, "NAIVE"),
        (dict(d_k=32, d_v=32), A.ERR_UNSUPPORTED, "d_k"),
        (dict(T_hat=0x1004), A.ERR_INVALID_ARGUMENT, "aligned"),
        (dict(), A.ERR_WORKSPACE_TOO_SMALL, "workspace"),
    ]
    for kw, status, msg in cases:
        d = _compose_desc(**kw)
        assert L.hypic_compose(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode(), kw
    d = _compose_desc()
    assert L.hypic_compose_workspace_bytes(C.byref(d)) > 0
    d = _compose_desc(mode=A.COMPOSE["fold"])
    assert L.hypic_compose_workspace_bytes(C.byref(d)) == 0


def test_seam_and_conv_validation(L):
    cu = np.array([0, 8, 16], np.int64)
    base = dict(in_dtype=A.BF16, out_dtype=A.BF16, n_batch=1, n_tokens=16, h_k=1, h_v=1, d_k=128, d_v=128,
                n_seam=2, cu_seam=cu.ctypes.data, qk_l2norm=0, q=0x1000, k=0x2000, v=0x3000, log_alpha=0x4000,
                beta=0x5000, S_in=None, state_stride=0, o=0x6000, S_out=None, T_hat=None, T_exp=None, S_seam=None,
                precision=0, workspace=None, workspace_bytes=0)
    n = A.INLINE_SEGS + 1
    big = np.arange(0, 8 * (n + 1), 8, dtype=np.int64)
    long_seam = np.array([0, 8, 40], np.int64)
    for kw, status, msg in ((dict(q=None), A.ERR_INVALID_ARGUMENT, "without q"),
                            (dict(state_stride=10), A.ERR_INVALID_ARGUMENT, "state_stride"),
                            (dict(n_seam=n, cu_seam=big.ctypes.data, n_tokens=int(big[-1])),
                             A.ERR_WORKSPACE_TOO_SMALL, "workspace"),
                            # float32 inputs, d = 128, a seam longer than 16 tokens: no float32 plan
                            (dict(in_dtype=A.F32, cu_seam=long_seam.ctypes.data, n_tokens=40),
                             A.ERR_UNSUPPORTED, "HYPIC_PREC_F16"),
                            (dict(in_dtype=A.F32, precision=A.PREC["f32"], cu_seam=long_seam.ctypes.data,
                                  n_tokens=40), A.ERR_UNSUPPORTED, "d = 64")):
        d = A.SeamDesc(**{**base, **kw})
        assert L.hypic_seam_advance(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode()
    d = A.SeamDesc(**base)
    assert L.hypic_seam_advance_workspace_bytes(C.byref(d)) == 0
    cb = dict(in_dtype=A.BF16, out_dtype=A.BF16, n_batch=1, n_tokens=16, channels=64, width=4, n_seg=2,
              cu_seqlens=cu.ctypes.data, x=0x1000, state_in=None, n_state=0, state_index=None, weight=0x2000,
              bias=None, activation=0, y=0x3000, state_out=None, workspace=None, workspace_bytes=0)
    for kw, status, msg in ((dict(width=3), A.ERR_UNSUPPORTED, "width"),
                            (dict(channels=12), A.ERR_UNSUPPORTED, "multiple of 8"),
                            (dict(state_in=0x4000, n_state=1), A.ERR_INVALID_ARGUMENT, "state_index"),
                            (dict(activation=5), A.ERR_INVALID_ARGUMENT, "activation"),
                            (dict(n_seg=n, cu_seqlens=big.ctypes.data, n_tokens=int(big[-1])),
                             A.ERR_WORKSPACE_TOO_SMALL, "workspace")):
        d = A.ConvDesc(**{**cb, **kw})
        assert L.hypic_conv_warmup(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode()
    assert L.hypic_conv_warmup_workspace_bytes(C.byref(A.ConvDesc(**cb))) == 0


def test_plan_schedule_matches_oracle_exactly():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(0, 40))
        m = int(rng.integers(1, 12))
        w = rng.integers(0, 130, size=n)
        order, assign, mk = hypic_plan_schedule(w, m, "lpt")
        o_order, o_assign, o_mk = O.lpt_schedule(w.tolist(), m)
        assert order.tolist() == o_order and assign.tolist() == o_assign and mk == o_mk
        _, rassign, rmk = hypic_plan_schedule(w, m, "rr")
        o_ra, o_rmk = O.rr_schedule(w.tolist(), m)
        assert rassign.tolist() == o_ra and rmk == o_rmk


def test_plan_schedule_rejects(L):
    w = np.array([1, -2], np.int64)
    assert L.hypic_plan_schedule(w.ctypes.data, 2, 2, 1, None, None, None) == A.ERR_INVALID_ARGUMENT
    assert L.hypic_plan_schedule(w.ctypes.data, 2, 0, 1, None, None, None) == A.ERR_INVALID_ARGUMENT


# ----------------------------------------------------------------------------------------
# seam-width knob (HYPIC project README, "PIC modes": 0 reuses the whole segment, a value in
# (0, 1] is a fraction of each segment, a value above 1 an absolute token count; default 8)


def test_seam_widths_knob_cases():
    from linear_attention_state_chunked_amd.api import hypic_seam_widths

    lens = [0, 1, 5, 8, 9, 700, 4096]
    assert hypic_seam_widths(lens).tolist() == [0, 1, 5, 8, 8, 8, 8]               # default 8
    assert hypic_seam_widths(lens, 0).tolist() == [0] * 7                          # whole segment reused
    assert hypic_seam_widths(lens, 1.0).tolist() == lens                           # the whole segment
    assert hypic_seam_widths(lens, 0.5).tolist() == [0, 1, 3, 4, 5, 350, 2048]     # ceil(len / 2)
    assert hypic_seam_widths(lens, 0.01).tolist() == [0, 1, 1, 1, 1, 7, 41]        # ceil(0.01 len)
    assert hypic_seam_widths(lens, 16).tolist() == [0, 1, 5, 8, 9, 16, 16]         # absolute count
    assert hypic_seam_widths(lens, 2.9).tolist() == [0, 1, 2, 2, 2, 2, 2]          # its integer part
    assert hypic_seam_widths([], 8).tolist() == []
    assert A.SEAM_SINK_DEFAULT == 8.0


def test_seam_widths_rejects(L):
    from linear_attention_state_chunked_amd.api import hypic_seam_widths

    for lens, sink in (([3], -1.0), ([3], float("inf")), ([-1], 8.0)):
        with pytest.raises(A.HypicError):
            hypic_seam_widths(lens, sink)
    with pytest.raises(ValueError):
        hypic_seam_widths([3], float("nan"))
    assert L.hypic_seam_widths(None, 2, 8.0, None) == A.ERR_INVALID_ARGUMENT


# ----------------------------------------------------------------------------------------
# the binding validates every tensor before calling the library (no GPU needed: the checks
# run before the device check, and a host tensor is itself rejected)


def _bt(*shape, dt=None):
    import torch
    return torch.zeros(shape, dtype=dt or torch.float32)


@pytest.mark.parametrize("case", ["v_dtype", "v_shape", "la_dtype", "la_numel", "beta_dtype", "beta_diag",
                                  "diag_la_last", "host"])
def test_binding_rejects_bad_build_tensors(case):
    import torch
    from linear_attention_state_chunked_amd import api as H

    B, N, hk, hv, d = 1, 64, 1, 2, 64
    k, v = _bt(B, N, hk, d, dt=torch.bfloat16), _bt(B, N, hv, d, dt=torch.bfloat16)
    la, beta = _bt(B, N, hv), _bt(B, N, hv)
    kw = dict(kind="dense")
    if case == "v_dtype":
        v = v.float()
    elif case == "v_shape":
        v = _bt(B, N + 1, hv, d, dt=torch.bfloat16)
    elif case == "la_dtype":
        la = la.bfloat16()
    elif case == "la_numel":
        la = _bt(B, N, hv + 1)
    elif case == "beta_dtype":
        beta = beta.double()
    elif case == "beta_diag":
        kw = dict(kind="diag")
        la = _bt(B, N, hv, d)
    elif case == "diag_la_last":
        kw = dict(kind="diag")
        la, beta = _bt(B, N, hv * d, 1), None
    with pytest.raises(ValueError):
        H.hypic_segment_build(k, v, la, [0, N], beta, **kw)


def test_binding_rejects_bad_compose_seam_conv_tensors():
    import torch
    from linear_attention_state_chunked_amd import api as H

    n, c, d = 3, 2, 64
    T, e, S = _bt(n, c, d, d), torch.zeros((n, c), dtype=torch.int32), _bt(n, c, d, d)
    bad = [dict(T_hat=T.double()), dict(T_exp=e.long()), dict(T_hat=_bt(n, c, d)),
           dict(S0=_bt(c, d, d + 1)), dict(slot=torch.zeros(n, dtype=torch.int64)), dict()]
    for b in bad:
        args = {"T_hat": T, "T_exp": e, "S": S, **b}
        kw = {k: args.pop(k) for k in ("S0", "slot") if k in args}
        with pytest.raises(ValueError):      # the last one: host tensors
            H.hypic_compose(args["T_hat"], args["T_exp"], args["S"], **kw)
    q = k = _bt(1, 16, 1, d)
    v = _bt(1, 16, 2, d)
    la = bt = _bt(1, 16, 2)
    for kw in (dict(q=q.bfloat16()), dict(v=_bt(1, 16, 2, d + 1)), dict(log_alpha=la.bfloat16()),
               dict(beta=_bt(1, 16, 3)), dict(S_in=_bt(1, 1, 2, d, d)), dict()):
        a = {"q": q, "k": k, "v": v, "log_alpha": la, "beta": bt, **kw}
        S_in = a.pop("S_in", None)
        with pytest.raises(ValueError):
            H.hypic_seam_advance(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], [0, 8, 16], S_in=S_in)
    x = _bt(1, 16, 64, dt=torch.bfloat16)
    for kw in (dict(weight=_bt(1, 64, 4).double()), dict(weight=_bt(1, 32, 4)), dict(bias=_bt(1, 63)),
               dict(state_in=_bt(2, 1, 3, 64)), dict(state_index=torch.zeros(2, dtype=torch.int64)), dict()):
        a = {"weight": _bt(1, 64, 4), **kw}
        w = a.pop("weight")
        with pytest.raises(ValueError):
            H.hypic_conv_warmup(x, w, [0, 8, 16], **a)


def test_rerotate_validation(L):
    dl = np.array([3, -5], np.int64)
    base = dict(kind=A.DENSE, n_elem=2, n_chain=3, d_k=64, d_v=64, rotary_dim=64, interleaved=0, rope_base=1e4,
                delta=dl.ctypes.data, T_hat_in=0x1000, T_hat_out=0x1000, S_in=0x2000, S_out=0x2000)
    for kw, status, msg in ((dict(kind=A.DIAG), A.ERR_UNSUPPORTED, "commute"),
                            (dict(rotary_dim=63), A.ERR_INVALID_ARGUMENT, "even"),
                            (dict(rotary_dim=66), A.ERR_INVALID_ARGUMENT, "rotary_dim"),
                            (dict(rope_base=0.0), A.ERR_INVALID_ARGUMENT, "rope_base"),
                            (dict(rope_base=float("nan")), A.ERR_INVALID_ARGUMENT, "rope_base"),
                            (dict(interleaved=2), A.ERR_INVALID_ARGUMENT, "interleaved"),
                            (dict(delta=None), A.ERR_INVALID_ARGUMENT, "delta"),
                            (dict(T_hat_in=None), A.ERR_INVALID_ARGUMENT, "T_hat_in"),
                            (dict(d_k=96, d_v=96), A.ERR_UNSUPPORTED, "d_k"),
                            (dict(n_chain=0), A.ERR_INVALID_ARGUMENT, "n_chain")):
        d = A.RerotateDesc(**{**base, **kw})
        assert L.hypic_state_rerotate(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode(), kw
    d = A.RerotateDesc(**{**base, "n_elem": 0})
    assert L.hypic_state_rerotate(C.byref(d), None) == A.OK      # nothing to do, nothing enqueued


def test_compose_seam_validation(L):
    cu = np.array([0, 8, 16], np.int64)
    long = np.array([0, 9, 16], np.int64)
    base = dict(n_batch=1, h_k=1, h_v=2, d_k=128, d_v=128, n_elem=2, n_slot=2, slot=None, T_hat=0x1000,
                T_exp=0x2000, S=0x3000, S0=None, S_final=0x4000, S_prefix=None, in_dtype=A.BF16, out_dtype=A.F32,
                n_tokens=16, cu_seam=cu.ctypes.data, qk_l2norm=0, q=0x5000, k=0x6000, v=0x7000,
                log_alpha=0x8000, beta=0x9000, o=None, workspace=None, workspace_bytes=0)
    for kw, status, msg in ((dict(cu_seam=long.ctypes.data), A.ERR_UNSUPPORTED, "at most 8"),
                            (dict(S_final=None), A.ERR_INVALID_ARGUMENT, "S_final"),
                            (dict(n_slot=1), A.ERR_INVALID_ARGUMENT, "n_slot"),
                            (dict(T_hat=None), A.ERR_INVALID_ARGUMENT, "T_hat"),
                            (dict(q=None), A.ERR_INVALID_ARGUMENT, "q, k, v"),
                            (dict(h_k=3), A.ERR_INVALID_ARGUMENT, "geometry"),
                            (dict(d_k=96, d_v=96), A.ERR_UNSUPPORTED, "d_k"),
                            (dict(out_dtype=7), A.ERR_INVALID_ARGUMENT, "dtype")):
        d = A.SeamComposeDesc(**{**base, **kw})
        assert L.hypic_compose_seam(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode(), kw
    assert L.hypic_compose_seam_workspace_bytes(C.byref(A.SeamComposeDesc(**base))) == 0
