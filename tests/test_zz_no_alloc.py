"""hypic_compose_noalloc against hypic_compose, through the C ABI.

The allocation-free entry point keeps SCAN's scratch in a fixed per-device array
instead of a caller workspace; its outputs must equal hypic_compose's.  Two calls
in a row on the same array, the second with a smaller input (fewer elements,
chains and blocks), so stale contents of the first call would show.
"""

import ctypes as C

import numpy as np
import pytest
import torch

from linear_attention_state_chunked_amd import _abi as A
from synth import random_elements

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _desc(T, e, S, slot, S0, outs, mode, kind=A.DENSE, scan_block=0):
    n_slot, n_chain, d = S.shape[0], S.shape[1], S.shape[2]
    p = lambda t: None if t is None else t.data_ptr()
    return A.ComposeDesc(kind=kind, n_chain=n_chain, d_k=d, d_v=d, n_elem=slot.numel(), n_slot=n_slot,
                         slot=p(slot), T_hat=p(T), T_exp=p(e), S=p(S), S0=p(S0), S_final=p(outs["S_final"]),
                         S_prefix=p(outs["S_prefix"]), T_total=p(outs["T_total"]),
                         T_total_exp=p(outs["T_total_exp"]), mode=A.COMPOSE[mode], scan_block=scan_block,
                         workspace=None, workspace_bytes=0)


def _outs(n_elem, n_chain, d, want_T=True):
    f = lambda *sh: torch.full(sh, float("nan"), device=DEV)
    o = {"S_final": f(n_chain, d, d), "S_prefix": f(n_elem, n_chain, d, d), "T_total": None, "T_total_exp": None}
    if want_T:
        o["T_total"] = f(n_chain, d, d)
        o["T_total_exp"] = torch.full((n_chain,), -7, dtype=torch.int32, device=DEV)
    return o


def _case(seed, n_slot, n_elem, n_chain, d, mode, scan_block, want_T=True):
    L = A.lib()
    el = random_elements(seed, n_slot, n_chain, d)
    T = torch.from_numpy(el["T_hat"]).to(DEV)
    e = torch.from_numpy(el["T_exp"]).to(DEV)
    S = torch.from_numpy(el["S"]).to(DEV)
    slot = torch.from_numpy(np.random.default_rng(seed).integers(0, n_slot, n_elem).astype(np.int32)).to(DEV)
    S0 = torch.randn((n_chain, d, d), device=DEV, generator=torch.Generator(DEV).manual_seed(seed))
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the existing entry point with its own workspace
    ref = _outs(n_elem, n_chain, d, want_T)
    dr = _desc(T, e, S, slot, S0, ref, mode, scan_block=scan_block)
    need = L.hypic_compose_workspace_bytes(C.byref(dr))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    dr.workspace, dr.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_compose(C.byref(dr), stream))
    # the allocation-free one
    got = _outs(n_elem, n_chain, d, want_T)
    dn = _desc(T, e, S, slot, S0, got, mode, scan_block=scan_block)
    A.check(L.hypic_compose_noalloc(C.byref(dn), stream))
    torch.cuda.synchronize()
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(got[k], ref[k]), f"{k} differs (seed {seed}, {n_elem} elements x {n_chain} chains)"
    assert torch.isfinite(got["S_final"]).all() and torch.isfinite(got["S_prefix"]).all()
    return need


def test_compose_noalloc_matches_compose_twice(gpu):
    # first call: a SCAN of 48 elements x 6 chains in blocks of 5 (10 blocks of scratch)
    need1 = _case(101, 20, 48, 6, 128, "scan", 5)
    assert 0 < need1 <= A.NOALLOC_SCRATCH_BYTES
    # second call, smaller: 9 elements x 2 chains, blocks of 4 -- reads the same array
    need2 = _case(202, 7, 9, 2, 128, "scan", 4)
    assert need2 < need1
    # a FOLD needs no scratch at all
    _case(303, 5, 6, 3, 64, "fold", 0)
    # the running state alone: FOLD, and the SCAN's aggregate fold and re-fold, split each chain's
    # columns over several workgroups
    _case(404, 11, 40, 5, 128, "fold", 0, want_T=False)
    _case(505, 11, 40, 5, 128, "scan", 6, want_T=False)


def test_compose_noalloc_rejects_oversize(gpu):
    L = A.lib()
    n_elem, n_chain, d = 256, 960, 128
    T = torch.empty((1, 1, d, d), device=DEV)   # never read: rejected on the host
    dn = A.ComposeDesc(kind=A.DENSE, n_chain=n_chain, d_k=d, d_v=d, n_elem=n_elem, n_slot=n_elem, slot=None,
                       T_hat=T.data_ptr(), T_exp=T.data_ptr(), S=T.data_ptr(), S0=None, S_final=T.data_ptr(),
                       S_prefix=T.data_ptr(), T_total=None, T_total_exp=None, mode=A.COMPOSE["scan"],
                       scan_block=16, workspace=None, workspace_bytes=0)
    assert L.hypic_compose_workspace_bytes(C.byref(dn)) > A.NOALLOC_SCRATCH_BYTES
    assert L.hypic_compose_noalloc(C.byref(dn), None) == A.ERR_UNSUPPORTED
    assert "fixed per-device array" in L.hypic_last_error().decode()
