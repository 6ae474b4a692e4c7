"""Python binding of libhypic with the C-ABI call names.

Argument marshalling only: torch supplies device memory (outputs and
workspaces are allocated with torch) and the current stream; every step of the
computation runs in libhypic's HIP kernels.  Layouts and semantics are those of
include/hypic.h.

Every tensor argument is checked before the library is called: dtype, shape (or
element count), contiguity, and that it lives on the same GPU as the call's
first input.  A kernel reads exactly the extents the header gives, so a tensor
of the wrong dtype or size would be read past its end; a host tensor would hand
a host address to the device.  Violations raise ValueError.
"""

from __future__ import annotations

import ctypes as C
import math

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
    raise ValueError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _host_offsets(cu) -> np.ndarray:
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int64))


def _check(t, name, *, dtype=None, shape=None, numel=None, device=None, optional=False):
    """Validate one tensor argument; returns it.  Checks run dtype, shape, contiguity,
    then device, so every rejection is reachable without a GPU."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _gpu_device(t, name):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the library runs on the device only), got {t.device}")
    return t.device


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _out(out, name, shape, dtype, device):
    """Caller-provided output tensor `out[name]` (checked), else a new one."""
    t = (out or {}).get(name)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _check(t, f"out[{name!r}]", dtype=dtype, shape=shape, device=device)


def _as4(x, name):
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if x.dim() == 3:
        return x.unsqueeze(0)
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B, N, heads, d] or [N, heads, d], got shape {tuple(x.shape)}")
    return x


_FLOAT_IN = (torch.bfloat16, torch.float32)


def hypic_segment_build(k, v, log_alpha, cu_seqlens, beta=None, *, kind="dense", with_T=True, skip_head=0,
                        qk_l2norm=False, schedule="natural", precision="auto", out=None, workspace_bytes=None,
                        workspace=None, q=None, want_o=False, out_dtype=None):
    """Per-segment (T_hat, T_exp, S) for every (segment, batch, value head).

    k [B,N,h_k,d] (or [N,h_k,d]), v [B,N,h_v,d] of k's dtype; log_alpha float32
    [B,N,h_v] (diag: [B,N,h_v,d]); beta float32 [B,N,h_v] (dense only).  Returns a
    dict with T_hat (dense [n_seg,B,h_v,d,d], diag [n_seg,B,h_v,d], scalar
    [n_seg,B,h_v]) or None, T_exp [n_seg,B,h_v] int32 or None, and S
    [n_seg,B,h_v,d,d] float32.  `out` may hold preallocated "T_hat", "T_exp", "S"
    tensors of those shapes.  workspace_bytes overrides the queried workspace size;
    workspace passes a caller-owned uint8 device tensor instead.  With want_o (dense
    kind, q [B,N,h_k,d] of k's dtype) the result also holds o [B,N,h_v,d] (out_dtype,
    default k's): each covered token's output from the segment's zero-start state.
    """
    if kind not in A.KIND:
        raise ValueError(f"unknown kind {kind!r}")
    kd = A.KIND[kind]
    k = _check(_as4(k, "k"), "k", dtype=_FLOAT_IN)
    B, N, h_k, d = k.shape
    v = _as4(v, "v")
    h_v = v.shape[2]
    v = _check(v, "v", dtype=k.dtype, shape=(B, N, h_v, v.shape[3]))
    per_channel = kd in (A.DIAG, A.KDA)
    la_numel = B * N * h_v * (d if per_channel else 1)
    _check(log_alpha, "log_alpha", dtype=torch.float32, numel=la_numel)
    if per_channel and log_alpha.shape[-1] != d:
        raise ValueError(f"{kind} log_alpha must have last dimension d = {d}, got shape {tuple(log_alpha.shape)}")
    if kd in (A.DENSE, A.KDA):
        _check(beta, "beta", dtype=torch.float32, numel=B * N * h_v)
    elif beta is not None:
        raise ValueError("beta is used by the dense and KDA kinds only")
    if want_o:
        if kd != A.DENSE:
            raise ValueError("per-token outputs are implemented for the dense kind only")
        q = _check(_as4(q, "q"), "q", dtype=k.dtype, shape=k.shape)
    elif q is not None:
        raise ValueError("q is given but want_o is False")
    out_dtype = out_dtype or k.dtype
    if out_dtype not in _FLOAT_IN:
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    dev = _gpu_device(k, "k")
    _check(v, "v", device=dev)
    _check(q, "q", device=dev, optional=True)
    la = _check(log_alpha.reshape(B, N, h_v, d) if per_channel else log_alpha.reshape(B, N, h_v), "log_alpha",
                device=dev)
    bt = _check(beta.reshape(B, N, h_v), "beta", device=dev) if beta is not None else None
    cu = _host_offsets(cu_seqlens)
    n_seg = len(cu) - 1
    S = _out(out, "S", (n_seg, B, h_v, d, d), torch.float32, dev)
    T_hat = T_exp = None
    if with_T:
        tshape = {A.DENSE: (n_seg, B, h_v, d, d), A.KDA: (n_seg, B, h_v, d, d), A.DIAG: (n_seg, B, h_v, d),
                  A.SCALAR: (n_seg, B, h_v)}[kd]
        T_hat = _out(out, "T_hat", tshape, torch.float32, dev)
        T_exp = _out(out, "T_exp", (n_seg, B, h_v), torch.int32, dev)
    o = _out(out, "o", (B, N, h_v, d), out_dtype, dev) if want_o else None
    desc = A.BuildDesc(kind=kd, in_dtype=_dtype(k), n_batch=B, n_tokens=N, h_k=h_k, h_v=h_v, d_k=d, d_v=v.shape[3],
                       chunk=64, n_seg=n_seg, cu_seqlens=cu.ctypes.data, skip_head=skip_head,
                       qk_l2norm=int(bool(qk_l2norm)), k=_ptr(k), v=_ptr(v), log_alpha=_ptr(la), beta=_ptr(bt),
                       T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S=_ptr(S), schedule=A.SCHED[schedule],
                       precision=A.PREC[precision], q=_ptr(q), o=_ptr(o),
                       out_dtype=A.BF16 if out_dtype == torch.bfloat16 else A.F32)
    L = A.lib()
    if workspace is not None:
        ws = _check(workspace, "workspace", dtype=torch.uint8, device=dev)
    else:
        nbytes = L.hypic_segment_build_workspace_bytes(C.byref(desc)) if workspace_bytes is None else workspace_bytes
        ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_segment_build(C.byref(desc), _stream()))
    return {"T_hat": T_hat, "T_exp": T_exp, "S": S, "o": o, "_workspace": ws}


def hypic_compose_noalloc(T_hat, T_exp, S, **kw):
    """hypic_compose through the allocation-free entry point: SCAN's scratch comes from
    the library's fixed per-device array instead of a workspace (outputs are still
    allocated here, by the caller's side).  Same arguments and results."""
    return hypic_compose(T_hat, T_exp, S, _noalloc=True, **kw)


def hypic_compose(T_hat, T_exp, S, *, kind="dense", slot=None, S0=None, mode="auto", want_prefix=False,
                  want_T=False, scan_block=0, n_elem=None, _noalloc=False):
    """Compose cached elements in request order.

    Element store: S [n_slot, C, d, d] float32, T_hat [n_slot, C, ...] float32,
    T_exp [n_slot, C] int32 (the build outputs reshaped to [n_seg, B*h_v, ...]).
    slot: device int32 [n_elem] (None = identity).  S0: float32 [C, d, d] or None.
    Returns S_final [C,d,d], S_prefix [n_elem,C,d,d] or None, T_total and
    T_total_exp or None.
    """
    if kind not in A.KIND:
        raise ValueError(f"unknown kind {kind!r}")
    kd = A.KIND[kind]
    if not isinstance(S, torch.Tensor) or S.dim() != 4:
        raise ValueError("S must be a [n_slot, n_chain, d, d] tensor")
    n_slot, n_chain, d = S.shape[0], S.shape[1], S.shape[2]
    _check(S, "S", dtype=torch.float32, shape=(n_slot, n_chain, d, d))
    naive = mode == "naive_add"
    tshape = {A.DENSE: (n_slot, n_chain, d, d), A.KDA: (n_slot, n_chain, d, d), A.DIAG: (n_slot, n_chain, d),
              A.SCALAR: (n_slot, n_chain)}[kd]
    _check(T_hat, "T_hat", dtype=torch.float32, shape=tshape, optional=naive)
    _check(T_exp, "T_exp", dtype=torch.int32, shape=(n_slot, n_chain), optional=naive)
    _check(S0, "S0", dtype=torch.float32, shape=(n_chain, d, d), optional=True)
    if slot is not None:
        _check(slot, "slot", dtype=torch.int32)
        if slot.dim() != 1:
            raise ValueError("slot must be a 1-D int32 tensor")
    if n_elem is None:
        n_elem = slot.numel() if slot is not None else n_slot
    if slot is not None and slot.numel() < n_elem:
        raise ValueError(f"slot holds {slot.numel()} entries, n_elem = {n_elem}")
    dev = _gpu_device(S, "S")
    for t, nm in ((T_hat, "T_hat"), (T_exp, "T_exp"), (S0, "S0"), (slot, "slot")):
        _check(t, nm, device=dev, optional=True)
    S_final = torch.empty((n_chain, d, d), dtype=torch.float32, device=dev)
    S_prefix = torch.empty((n_elem, n_chain, d, d), dtype=torch.float32, device=dev) if want_prefix else None
    T_total = T_total_exp = None
    if want_T:
        tout = {A.DENSE: (n_chain, d, d), A.KDA: (n_chain, d, d), A.DIAG: (n_chain, d), A.SCALAR: (n_chain,)}[kd]
        T_total = torch.empty(tout, dtype=torch.float32, device=dev)
        T_total_exp = torch.empty((n_chain,), dtype=torch.int32, device=dev)
    desc = A.ComposeDesc(kind=kd, n_chain=n_chain, d_k=d, d_v=S.shape[3], n_elem=n_elem, n_slot=n_slot,
                         slot=_ptr(slot), T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S=_ptr(S), S0=_ptr(S0),
                         S_final=_ptr(S_final), S_prefix=_ptr(S_prefix), T_total=_ptr(T_total),
                         T_total_exp=_ptr(T_total_exp), mode=A.COMPOSE[mode], scan_block=scan_block)
    L = A.lib()
    if _noalloc:
        A.check(L.hypic_compose_noalloc(C.byref(desc), _stream()))
        return {"S_final": S_final, "S_prefix": S_prefix, "T_total": T_total, "T_total_exp": T_total_exp}
    nbytes = L.hypic_compose_workspace_bytes(C.byref(desc))
    ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_compose(C.byref(desc), _stream()))
    return {"S_final": S_final, "S_prefix": S_prefix, "T_total": T_total, "T_total_exp": T_total_exp,
            "_workspace": ws}


def hypic_compose_seam(T_hat, T_exp, S, q, k, v, log_alpha, beta, cu_seam, *, slot=None, S0=None, want_o=True,
                       want_prefix=False, out_dtype=None, qk_l2norm=False):
    """The warm hit path in one pass: for each request position, the seam tokens run
    through the running state (outputs emitted), then the cached element is composed.

    Element store as hypic_compose (dense): S, T_hat [n_slot, C, d, d] float32, T_exp
    [n_slot, C] int32 with C = B * h_v; slot device int32 [n_elem] or None; S0 [C, d, d]
    or None.  Seam tokens packed over request positions (cu_seam host [n_elem + 1], each
    at most 8): q, k [B, N, h_k, d], v [B, N, h_v, d] of one dtype; log_alpha, beta float32
    [B, N, h_v].  Returns S_final [C, d, d], S_prefix [n_elem, C, d, d] or None (the state
    entering each position, before its seam), o [B, N, h_v, d] or None.
    """
    if not isinstance(S, torch.Tensor) or S.dim() != 4:
        raise ValueError("S must be a [n_slot, n_chain, d, d] tensor")
    n_slot, n_chain, d = S.shape[0], S.shape[1], S.shape[2]
    _check(S, "S", dtype=torch.float32, shape=(n_slot, n_chain, d, d))
    _check(T_hat, "T_hat", dtype=torch.float32, shape=(n_slot, n_chain, d, d))
    _check(T_exp, "T_exp", dtype=torch.int32, shape=(n_slot, n_chain))
    _check(S0, "S0", dtype=torch.float32, shape=(n_chain, d, d), optional=True)
    k = _check(_as4(k, "k"), "k", dtype=_FLOAT_IN)
    B, N, h_k, dk = k.shape
    q = _check(_as4(q, "q"), "q", dtype=k.dtype, shape=k.shape)
    v = _as4(v, "v")
    h_v = v.shape[2]
    v = _check(v, "v", dtype=k.dtype, shape=(B, N, h_v, d))
    if dk != d or B * h_v != n_chain:
        raise ValueError(f"seam tokens [B={B}, h_v={h_v}, d={dk}] do not match the {n_chain} chains of d = {d}")
    _check(log_alpha, "log_alpha", dtype=torch.float32, numel=B * N * h_v)
    _check(beta, "beta", dtype=torch.float32, numel=B * N * h_v)
    cu = _host_offsets(cu_seam)
    n_elem = len(cu) - 1
    if slot is not None:
        _check(slot, "slot", dtype=torch.int32, numel=n_elem)
    elif n_slot < n_elem:
        raise ValueError(f"{n_elem} request positions but only {n_slot} slots and no slot map")
    dev = _gpu_device(S, "S")
    for t, nm in ((T_hat, "T_hat"), (T_exp, "T_exp"), (S0, "S0"), (slot, "slot"), (q, "q"), (k, "k"), (v, "v"),
                  (log_alpha, "log_alpha"), (beta, "beta")):
        _check(t, nm, device=dev, optional=True)
    out_dtype = out_dtype or k.dtype
    if out_dtype not in _FLOAT_IN:
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    S_final = torch.empty((n_chain, d, d), dtype=torch.float32, device=dev)
    S_prefix = torch.empty((n_elem, n_chain, d, d), dtype=torch.float32, device=dev) if want_prefix else None
    o = torch.empty((B, N, h_v, d), dtype=out_dtype, device=dev) if want_o else None
    desc = A.SeamComposeDesc(n_batch=B, h_k=h_k, h_v=h_v, d_k=d, d_v=d, n_elem=n_elem, n_slot=n_slot,
                             slot=_ptr(slot), T_hat=_ptr(T_hat), T_exp=_ptr(T_exp), S=_ptr(S), S0=_ptr(S0),
                             S_final=_ptr(S_final), S_prefix=_ptr(S_prefix), in_dtype=_dtype(k),
                             out_dtype=A.BF16 if out_dtype == torch.bfloat16 else A.F32, n_tokens=N,
                             cu_seam=cu.ctypes.data, qk_l2norm=int(bool(qk_l2norm)), q=_ptr(q), k=_ptr(k),
                             v=_ptr(v), log_alpha=_ptr(log_alpha), beta=_ptr(beta), o=_ptr(o))
    L = A.lib()
    ws = _workspace(L.hypic_compose_seam_workspace_bytes(C.byref(desc)), dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_compose_seam(C.byref(desc), _stream()))
    return {"S_final": S_final, "S_prefix": S_prefix, "o": o, "_workspace": ws}


def _state_numel(n_seam, stride, block):
    """Floats a seam-state array must hold: seam s at s * stride (stride 0: dense blocks)."""
    if n_seam == 0:
        return 0
    return (n_seam - 1) * (stride or block) + block


def hypic_seam_advance(q, k, v, log_alpha, beta, cu_seam, *, S_in=None, state_stride=0, want_o=True,
                       S_out="new", want_T=False, want_S_seam=False, out_dtype=None, qk_l2norm=False,
                       precision="auto", out=None):
    """Seam tokens through the running state.

    q, k [B,N,h_k,d] of one dtype; v [B,N,h_v,d] of that dtype; log_alpha, beta
    float32 [B,N,h_v]; S_in float32 with seam s at offset s*state_stride (0 =
    dense [n_seam,B,h_v,d,d]) or None.  S_out: "new" (allocate), a tensor (may be
    S_in) or None.  Returns o [B,N,h_v,d], S_out, T_hat/T_exp [n_seam,B,h_v,d,d],
    S_seam.  `out` may hold preallocated "o", "T_hat", "T_exp", "S_seam" tensors.
    """
    k = _check(_as4(k, "k"), "k", dtype=_FLOAT_IN)
    B, N, h_k, d = k.shape
    q = _check(_as4(q, "q"), "q", dtype=k.dtype, shape=k.shape)
    v = _as4(v, "v")
    h_v = v.shape[2]
    v = _check(v, "v", dtype=k.dtype, shape=(B, N, h_v, d))
    _check(log_alpha, "log_alpha", dtype=torch.float32, numel=B * N * h_v)
    _check(beta, "beta", dtype=torch.float32, numel=B * N * h_v)
    cu = _host_offsets(cu_seam)
    n_seam = len(cu) - 1
    block = B * h_v * d * d
    need = _state_numel(n_seam, state_stride, block)
    _check(S_in, "S_in", dtype=torch.float32, optional=True)
    if S_in is not None and S_in.numel() < need:
        raise ValueError(f"S_in holds {S_in.numel()} floats, the seams address {need}")
    dev = _gpu_device(k, "k")
    for t, nm in ((q, "q"), (v, "v"), (log_alpha, "log_alpha"), (beta, "beta"), (S_in, "S_in")):
        _check(t, nm, device=dev, optional=nm == "S_in")
    la = log_alpha.reshape(B, N, h_v)
    bt = beta.reshape(B, N, h_v)
    out_dtype = out_dtype or k.dtype
    if out_dtype not in _FLOAT_IN:
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    o = _out(out, "o", (B, N, h_v, d), out_dtype, dev) if want_o else None
    if isinstance(S_out, str):
        if S_out != "new":
            raise ValueError('S_out must be "new", a tensor or None')
        S_out = torch.empty((n_seam, B, h_v, d, d), dtype=torch.float32, device=dev) if state_stride == 0 else None
    elif S_out is not None:
        _check(S_out, "S_out", dtype=torch.float32, device=dev)
        if S_out.numel() < need:
            raise ValueError(f"S_out holds {S_out.numel()} floats, the seams address {need}")
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

    x [B,N,C] (or [N,C]); weight float32 [B,C,4] ([C,4] when B = 1); bias float32
    [B,C] ([C] when B = 1) or None; state_in [n_state,B,3,C] of x's dtype or None;
    state_index device int32 [n_seg] or None.  Returns y [B,N,C] and state_out
    [n_seg,B,3,C] (or None).
    """
    if not isinstance(x, torch.Tensor) or x.dim() not in (2, 3):
        raise ValueError("x must be a [B, N, C] or [N, C] tensor")
    x = _check(x if x.dim() == 3 else x.unsqueeze(0), "x", dtype=_FLOAT_IN)
    B, N, Cc = x.shape
    if isinstance(weight, torch.Tensor) and weight.dim() == 2:
        weight = weight.unsqueeze(0)
    if isinstance(bias, torch.Tensor) and bias.dim() == 1:
        bias = bias.unsqueeze(0)
    _check(weight, "weight", dtype=torch.float32)
    if weight.dim() != 3 or weight.shape[0] != B or weight.shape[1] != Cc:
        raise ValueError(f"weight must be [B, C, W] = [{B}, {Cc}, W] (per batch entry), got {tuple(weight.shape)}")
    _check(bias, "bias", dtype=torch.float32, shape=(B, Cc), optional=True)
    cu = _host_offsets(cu_seqlens)
    n_seg = len(cu) - 1
    if state_in is not None:
        _check(state_in, "state_in", dtype=x.dtype)
        if state_in.dim() != 4 or tuple(state_in.shape[1:]) != (B, weight.shape[2] - 1, Cc):
            raise ValueError(f"state_in must be [n_state, {B}, W-1, {Cc}], got {tuple(state_in.shape)}")
    if state_index is not None:
        _check(state_index, "state_index", dtype=torch.int32, numel=n_seg)
    dev = _gpu_device(x, "x")
    for t, nm in ((weight, "weight"), (bias, "bias"), (state_in, "state_in"), (state_index, "state_index")):
        _check(t, nm, device=dev, optional=True)
    out_dtype = out_dtype or x.dtype
    if out_dtype not in _FLOAT_IN:
        raise ValueError(f"out_dtype must be bfloat16 or float32, got {out_dtype}")
    y = torch.empty((B, N, Cc), dtype=out_dtype, device=dev)
    st_out = torch.empty((n_seg, B, 3, Cc), dtype=x.dtype, device=dev) if want_state else None
    desc = A.ConvDesc(in_dtype=_dtype(x), out_dtype=_dtype(y), n_batch=B, n_tokens=N, channels=Cc,
                      width=weight.shape[2], n_seg=n_seg, cu_seqlens=cu.ctypes.data, x=_ptr(x),
                      state_in=_ptr(state_in), n_state=state_in.shape[0] if state_in is not None else 0,
                      state_index=_ptr(state_index), weight=_ptr(weight), bias=_ptr(bias),
                      activation=A.ACT[activation], y=_ptr(y), state_out=_ptr(st_out))
    L = A.lib()
    nbytes = L.hypic_conv_warmup_workspace_bytes(C.byref(desc))
    ws = _workspace(nbytes, dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    A.check(L.hypic_conv_warmup(C.byref(desc), _stream()))
    return {"y": y, "state_out": st_out, "_workspace": ws}


def hypic_state_rerotate(T_hat, S, delta, *, kind="dense", rotary_dim=None, rope_base=10000.0, interleaved=False,
                         inplace=False):
    """RoPE re-rotation of cached elements moved by delta[i] positions.

    S float32 [n_elem, C, d, d]; T_hat float32 [n_elem, C, d, d] (dense) or None
    (scalar: the transition is unchanged); delta: host int64 [n_elem].  rotary_dim
    defaults to d.  Returns {"T_hat", "S"}: new tensors, or the inputs updated in
    place with inplace=True.
    """
    if kind not in A.KIND:
        raise ValueError(f"unknown kind {kind!r}")
    kd = A.KIND[kind]
    if not isinstance(S, torch.Tensor) or S.dim() != 4:
        raise ValueError("S must be a [n_elem, n_chain, d, d] tensor")
    n_elem, n_chain, d = S.shape[0], S.shape[1], S.shape[2]
    _check(S, "S", dtype=torch.float32, shape=(n_elem, n_chain, d, d))
    if kd == A.DENSE:
        _check(T_hat, "T_hat", dtype=torch.float32, shape=(n_elem, n_chain, d, d))
    elif T_hat is not None and not isinstance(T_hat, torch.Tensor):
        raise ValueError("T_hat must be a tensor or None")
    dl = np.ascontiguousarray(np.asarray(delta, dtype=np.int64))
    if dl.shape != (n_elem,):
        raise ValueError(f"delta must hold {n_elem} shifts, got shape {dl.shape}")
    dev = _gpu_device(S, "S")
    if kd == A.DENSE:
        _check(T_hat, "T_hat", device=dev)
    S_out = S if inplace else torch.empty_like(S)
    T_in = T_hat if kd == A.DENSE else None
    T_out = (T_hat if inplace else torch.empty_like(T_hat)) if kd == A.DENSE else None
    desc = A.RerotateDesc(kind=kd, n_elem=n_elem, n_chain=n_chain, d_k=d, d_v=S.shape[3],
                          rotary_dim=d if rotary_dim is None else rotary_dim, interleaved=int(bool(interleaved)),
                          rope_base=float(rope_base), delta=dl.ctypes.data if n_elem else None, T_hat_in=_ptr(T_in),
                          T_hat_out=_ptr(T_out), S_in=_ptr(S), S_out=_ptr(S_out))
    A.check(A.lib().hypic_state_rerotate(C.byref(desc), _stream()))
    return {"T_hat": T_out if kd == A.DENSE else T_hat, "S": S_out}


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


def hypic_seam_widths(seg_lens, sink=A.SEAM_SINK_DEFAULT) -> np.ndarray:
    """Seam width of each segment from the seam-width knob (host only).

    0 -> no seam; 0 < sink <= 1 -> ceil(sink * len); sink > 1 -> floor(sink);
    capped at each segment's length.  Returns int32 widths.
    """
    lens = np.ascontiguousarray(np.asarray(seg_lens, dtype=np.int64))
    n = len(lens)
    w = np.zeros(n, np.int32)
    if isinstance(sink, float) and math.isnan(sink):
        raise ValueError("sink is NaN")
    A.check(A.lib().hypic_seam_widths(lens.ctypes.data if n else None, n, float(sink),
                                      w.ctypes.data if n else None))
    return w


def hypic_device_status() -> None:
    """Synchronise the device and raise HypicError if a kernel's bounded internal wait
    gave up since the last call (its outputs are then unreliable)."""
    A.check(A.lib().hypic_device_status())
