"""Python binding of libhypic with the C-ABI call names.

Argument marshalling only: torch supplies device memory (outputs and
workspaces are allocated with torch) and the current stream; every step of the
computation runs in libhypic's HIP kernels.  Layouts and semantics are those of
include/hypic.h.
"""

from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _abi as A


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return A.BF16
    if t.dtype == torch.float32:
        return A.F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _host_offsets(cu) -> np.ndarray:
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int64))


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _out(out, name, shape, dtype, device):
    """Caller-provided output tensor `out[name]` (checked), else a new one."""
    t = (out or {}).get(name)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"out[{name!r}] must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")
    return t


def _as4(x):
    return x if x.dim() == 4 else x.unsqueeze(0)


def hypic_segment_build(k, v, log_alpha, cu_seqlens, beta=None, *, kind="dense", with_T=True, skip_head=0,
                        qk_l2norm=False, schedule="natural", precision="auto", out=None, workspace_bytes=None,
                        workspace=None):
    """Per-segment (T_hat, T_exp, S) for every (segment, batch, value head).

    k [B,N,h_k,d] (or [N,h_k,d]), v [B,N,h_v,d]; log_alpha [B,N,h_v] (diag:
    [B,N,h_v,d]); beta [B,N,h_v] (dense).  Returns a dict with T_hat
    (dense [n_seg,B,h_v,d,d], diag [n_seg,B,h_v,d], scalar [n_seg,B,h_v]) or None,
    T_exp [n_seg,B,h_v] int32 or None, and S [n_seg,B,h_v,d,d] float32.
    `out` may hold preallocated "T_hat", "T_exp", "S" tensors of those shapes.
    workspace_bytes overrides the queried workspace size (a smaller one that still
    holds the segment table selects the single-launch engine); workspace passes a
    caller-owned uint8 device tensor instead.
    """
    k, v = _contig(_as4(k), "k"), _contig(_as4(v), "v")
    kd = A.KIND[kind]
    B, N, h_k, d = k.shape
    h_v = v.shape[2]
    la = _contig(log_alpha.reshape(B, N, h_v, -1) if kd == A.DIAG else log_alpha.reshape(B, N, h_v), "log_alpha")
    bt = _contig(beta.reshape(B, N, h_v), "beta") if beta is not None else None
    cu = _host_offsets(cu_seqlens)
    n_seg = len(cu) - 1
    dev = k.device
    S = _out(out, "S", (n_seg, B, h_v, d, d), torch.float32, dev)
    T_hat = T_exp = None
    if with_T:
        tshape = {A.DENSE: (n_seg, B, h_v, d, d), A.DIAG: (n_seg, B, h_v, d), A.SCALAR: (n_seg, B, h_v)}[kd]
        T_hat = _out(out, "T_hat", tshape, torch.float32, dev)
        T_exp = _out(out, "T_exp", (n_seg, B, h_v), torch.int32, dev)
    desc = A.BuildDesc(kind=kd, in_dtype=_dtype(k), n_batch=B, n_tokens=N, h_k=h_k, h_v=h_v, d_k=d, d_v=v.shape[3],
                       chunk=64, n_seg=n_seg, cu_seqlens=cu.ctypes.data, skip_head=skip_head,
                       qk_l2norm=int(bool(qk_l2norm)), k=_ptr(k), v=_ptr(v), log_alpha=_ptr(la), beta=_ptr(bt),
                       T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S=_ptr(S), schedule=A.SCHED[schedule],
                       precision=A.PREC[precision])
    L = A.lib()
    if workspace is not None:
        ws = _contig(workspace, "workspace")
    else:
        nbytes = L.hypic_segment_build_workspace_bytes(C.byref(desc)) if workspace_bytes is None else workspace_bytes
        ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_segment_build(C.byref(desc), _stream()))
    return {"T_hat": T_hat, "T_exp": T_exp, "S": S, "_workspace": ws}


def hypic_compose(T_hat, T_exp, S, *, kind="dense", slot=None, S0=None, mode="auto", want_prefix=False,
                  want_T=False, scan_block=0, n_elem=None):
    """Compose cached elements in request order.

    Element store: S [n_slot, C, d, d] float32, T_hat [n_slot, C, ...], T_exp
    [n_slot, C] int32 (the build outputs reshaped to [n_seg, B*h_v, ...]).  slot:
    device int32 [n_elem] (None = identity).  Returns S_final [C,d,d], S_prefix
    [n_elem,C,d,d] or None, T_total and T_total_exp or None.
    """
    kd = A.KIND[kind]
    n_slot, n_chain, d = S.shape[0], S.shape[1], S.shape[2]
    if n_elem is None:
        n_elem = slot.numel() if slot is not None else n_slot
    dev = S.device
    S_final = torch.empty((n_chain, d, d), dtype=torch.float32, device=dev)
    S_prefix = torch.empty((n_elem, n_chain, d, d), dtype=torch.float32, device=dev) if want_prefix else None
    T_total = T_total_exp = None
    if want_T:
        tshape = {A.DENSE: (n_chain, d, d), A.DIAG: (n_chain, d), A.SCALAR: (n_chain,)}[kd]
        T_total = torch.empty(tshape, dtype=torch.float32, device=dev)
        T_total_exp = torch.empty((n_chain,), dtype=torch.int32, device=dev)
    for t, nm in ((T_hat, "T_hat"), (T_exp, "T_exp"), (S, "S"), (S0, "S0"), (slot, "slot")):
        _contig(t, nm)
    desc = A.ComposeDesc(kind=kd, n_chain=n_chain, d_k=d, d_v=S.shape[3], n_elem=n_elem, n_slot=n_slot,
                         slot=_ptr(slot), T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S=_ptr(S), S0=_ptr(S0),
                         S_final=_ptr(S_final), S_prefix=_ptr(S_prefix), T_total=_ptr(T_total),
                         T_total_exp=_ptr(T_total_exp), mode=A.COMPOSE[mode], scan_block=scan_block)
    L = A.lib()
    nbytes = L.hypic_compose_workspace_bytes(C.byref(desc))
    ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_compose(C.byref(desc), _stream()))
    return {"S_final": S_final, "S_prefix": S_prefix, "T_total": T_total, "T_total_exp": T_total_exp,
            "_workspace": ws}


def hypic_seam_advance(q, k, v, log_alpha, beta, cu_seam, *, S_in=None, state_stride=0, want_o=True,
                       S_out="new", want_T=False, want_S_seam=False, out_dtype=None, qk_l2norm=False,
                       precision="auto", out=None):
    """Seam tokens through the running state.

    q, k [B,N,h_k,d]; v [B,N,h_v,d]; log_alpha, beta [B,N,h_v]; S_in float32
    with seam s at offset s*state_stride (0 = dense [n_seam,B,h_v,d,d]) or None.
    S_out: "new" (allocate), a tensor (may be S_in) or None.  Returns o
    [B,N,h_v,d], S_out, T_hat/T_exp [n_seam,B,h_v,d,d], S_seam.  `out` may hold
    preallocated "o", "T_hat", "T_exp", "S_seam" tensors of those shapes.
    """
    q, k, v = _contig(_as4(q), "q"), _contig(_as4(k), "k"), _contig(_as4(v), "v")
    B, N, h_k, d = k.shape
    h_v = v.shape[2]
    cu = _host_offsets(cu_seam)
    n_seam = len(cu) - 1
    dev = k.device
    la = _contig(log_alpha.reshape(B, N, h_v), "log_alpha")
    bt = _contig(beta.reshape(B, N, h_v), "beta")
    out_dtype = out_dtype or k.dtype
    o = _out(out, "o", (B, N, h_v, d), out_dtype, dev) if want_o else None
    if isinstance(S_out, str):
        S_out = torch.empty((n_seam, B, h_v, d, d), dtype=torch.float32, device=dev) if state_stride == 0 else None
    T_hat = _out(out, "T_hat", (n_seam, B, h_v, d, d), torch.float32, dev) if want_T else None
    T_exp = _out(out, "T_exp", (n_seam, B, h_v), torch.int32, dev) if want_T else None
    S_seam = _out(out, "S_seam", (n_seam, B, h_v, d, d), torch.float32, dev) if want_S_seam else None
    desc = A.SeamDesc(in_dtype=_dtype(k), out_dtype=_dtype(o) if o is not None else A.F32, n_batch=B, n_tokens=N,
                      h_k=h_k, h_v=h_v, d_k=d, d_v=v.shape[3], n_seam=n_seam, cu_seam=cu.ctypes.data,
                      qk_l2norm=int(bool(qk_l2norm)), q=_ptr(q), k=_ptr(k), v=_ptr(v), log_alpha=_ptr(la),
                      beta=_ptr(bt), S_in=_ptr(S_in), state_stride=state_stride, o=_ptr(o), S_out=_ptr(S_out),
                      T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S_seam=_ptr(S_seam), precision=A.PREC[precision])
    L = A.lib()
    nbytes = L.hypic_seam_advance_workspace_bytes(C.byref(desc))
    ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_seam_advance(C.byref(desc), _stream()))
    return {"o": o, "S_out": S_out, "T_hat": T_hat, "T_exp": T_exp, "S_seam": S_seam, "_workspace": ws}


def hypic_conv_warmup(x, weight, cu_seqlens, *, state_in=None, state_index=None, bias=None, activation="none",
                      out_dtype=None, want_state=True):
    """Depthwise causal conv (width 4) with carried state.

    x [B,N,C] (or [N,C]); weight [B,C,4] float32 ([C,4] when B = 1); bias [B,C]
    ([C] when B = 1) or None; state_in [n_state,B,3,C] (x's dtype) or None;
    state_index device int32 [n_seg] or None.  Returns y [B,N,C] and state_out
    [n_seg,B,3,C] (or None).
    """
    x = _contig(x if x.dim() == 3 else x.unsqueeze(0), "x")
    B, N, Cc = x.shape
    if weight.dim() == 2:
        weight = weight.unsqueeze(0)
    if bias is not None and bias.dim() == 1:
        bias = bias.unsqueeze(0)
    if weight.shape[0] != B or weight.shape[1] != Cc or (bias is not None and tuple(bias.shape) != (B, Cc)):
        raise ValueError("weight must be [B, C, W] and bias [B, C] (per batch entry)")
    cu = _host_offsets(cu_seqlens)
    n_seg = len(cu) - 1
    dev = x.device
    y = torch.empty((B, N, Cc), dtype=out_dtype or x.dtype, device=dev)
    st_out = torch.empty((n_seg, B, 3, Cc), dtype=x.dtype, device=dev) if want_state else None
    for t, nm in ((weight, "weight"), (state_in, "state_in"), (state_index, "state_index"), (bias, "bias")):
        _contig(t, nm)
    desc = A.ConvDesc(in_dtype=_dtype(x), out_dtype=_dtype(y), n_batch=B, n_tokens=N, channels=Cc, width=weight.shape[2],
                      n_seg=n_seg, cu_seqlens=cu.ctypes.data, x=_ptr(x), state_in=_ptr(state_in),
                      n_state=state_in.shape[0] if state_in is not None else 0, state_index=_ptr(state_index),
                      weight=_ptr(weight), bias=_ptr(bias), activation=A.ACT[activation], y=_ptr(y),
                      state_out=_ptr(st_out))
    L = A.lib()
    nbytes = L.hypic_conv_warmup_workspace_bytes(C.byref(desc))
    ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_conv_warmup(C.byref(desc), _stream()))
    return {"y": y, "state_out": st_out, "_workspace": ws}


def hypic_plan_schedule(weights, groups: int, schedule: str = "lpt"):
    """Host-only LPT / round-robin assignment of integer task weights to groups.

    Returns (order, assign, makespan) as numpy arrays and an int.
    """
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.int64))
    n = len(w)
    order = np.zeros(n, np.int32)
    assign = np.zeros(n, np.int32)
    mk = C.c_int64(0)
    A.check(A.lib().hypic_plan_schedule(w.ctypes.data if n else None, n, groups, A.SCHED[schedule],
                                        order.ctypes.data if n else None, assign.ctypes.data if n else None,
                                        C.byref(mk)))
    return order, assign, int(mk.value)
