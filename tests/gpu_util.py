"""Helpers for the GPU parity tests: seeded inputs on the device, oracle runs."""

import numpy as np
import torch

import oracle as O


def dev_tensor(x, dtype=torch.float32, device="cuda:0"):
    """Upload a float32 numpy array (bf16-exact for bf16) without changing its values."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dtype)


def cu_of(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def oracle_segments(kind, k, v, la, beta, lens, skip=0):
    """Per-segment oracle (T_hat, T_exp, S) for one chain; k, v [N, d]."""
    out = []
    s0 = 0
    for n in lens:
        lo, hi = s0 + min(skip, n), s0 + n
        if kind == "dense":
            r = O.dense_recurrence(k[lo:hi], v[lo:hi], la[lo:hi], beta[lo:hi])
        elif kind == "diag":
            r = O.diag_recurrence(k[lo:hi], v[lo:hi], la[lo:hi])
        else:
            r = O.scalar_recurrence(k[lo:hi], v[lo:hi], la[lo:hi])
        out.append(r)
        s0 += n
    return out


def max_err(errs):
    a = np.asarray(errs, dtype=np.float64)
    return float(a.max()) if a.size else 0.0
