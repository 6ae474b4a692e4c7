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
    assert len(declared) == 11
    assert declared == set(A.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (hypic_\w+)", out))
    assert declared <= exported
    for name in declared:
        assert getattr(L, name) is not None


def test_struct_layouts_match_the_header(tmp_path):
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "hypic.h"', "int main(void) {"]
    structs = {"hypic_build_desc": A.BuildDesc, "hypic_compose_desc": A.ComposeDesc,
               "hypic_seam_desc": A.SeamDesc, "hypic_conv_desc": A.ConvDesc}
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
    d, cu = _build_desc()
    need = L.hypic_segment_build_workspace_bytes(C.byref(d))
    assert need > 0 and need % 256 == 0
    d.workspace_bytes = 255          # below the segment table itself
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_WORKSPACE_TOO_SMALL
    d.workspace = None
    d.workspace_bytes = need
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_WORKSPACE_TOO_SMALL
    d, cu = _build_desc(schedule=A.SCHED["lpt"])
    assert L.hypic_segment_build_workspace_bytes(C.byref(d)) >= need + 2 * 4   # task order included
    # the F32 operand plan needs d = 64
    d, cu = _build_desc(precision=A.PREC["f32"])
    assert L.hypic_segment_build(C.byref(d), None) == A.ERR_UNSUPPORTED
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
    for kw, status, msg in ((dict(q=None), A.ERR_INVALID_ARGUMENT, "without q"),
                            (dict(state_stride=10), A.ERR_INVALID_ARGUMENT, "state_stride"),
                            (dict(), A.ERR_WORKSPACE_TOO_SMALL, "workspace")):
        d = A.SeamDesc(**{**base, **kw})
        assert L.hypic_seam_advance(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode()
    cb = dict(in_dtype=A.BF16, out_dtype=A.BF16, n_batch=1, n_tokens=16, channels=64, width=4, n_seg=2,
              cu_seqlens=cu.ctypes.data, x=0x1000, state_in=None, n_state=0, state_index=None, weight=0x2000,
              bias=None, activation=0, y=0x3000, state_out=None, workspace=None, workspace_bytes=0)
    for kw, status, msg in ((dict(width=3), A.ERR_UNSUPPORTED, "width"),
                            (dict(channels=12), A.ERR_UNSUPPORTED, "multiple of 8"),
                            (dict(state_in=0x4000, n_state=1), A.ERR_INVALID_ARGUMENT, "state_index"),
                            (dict(activation=5), A.ERR_INVALID_ARGUMENT, "activation"),
                            (dict(), A.ERR_WORKSPACE_TOO_SMALL, "workspace")):
        d = A.ConvDesc(**{**cb, **kw})
        assert L.hypic_conv_warmup(C.byref(d), None) == status, kw
        assert msg in L.hypic_last_error().decode()


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
