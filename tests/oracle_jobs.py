"""fp64 oracle jobs for sampled chains of the full-size workloads.

Each job regenerates one chain's inputs from its numpy streams and runs the
oracle on it, so a process pool can spread the sampled chains over the host
cores.  This module imports numpy, the oracle and the input generators only.
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle as O
from synth import WORKLOADS, chain_inputs, conv_chain_inputs, request_order, segment_lengths


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def dense_segments_job(args):
    """(workload, layer, head, segment ids or None = all, with_fold) ->
    {'seg': {s: (T_hat, T_exp, S)}, and with_fold (segments must be all):
    'S_final', 'T_hat', 'T_exp', 'S_prefix' of the fold over all segments}."""
    name, layer, head, segs, with_fold = args
    wl = WORKLOADS[name]
    lens = segment_lengths(wl)
    cu = _cu(lens)
    c = chain_inputs(wl, layer, head)
    todo = range(len(lens)) if segs is None else segs
    out = {"seg": {}}
    elems = []
    for s in todo:
        lo, hi = int(cu[s]), int(cu[s + 1])
        r = O.dense_recurrence(c["k"][lo:hi], c["v"][lo:hi], c["log_alpha"][lo:hi], c["beta"][lo:hi])
        out["seg"][s] = (r["T_hat"], r["T_exp"], r["S"])
        elems.append(r)
    if with_fold:
        f = O.compose_fold("dense", elems)
        out.update(S_final=f["S_final"], T_hat=f["T_hat"], T_exp=f["T_exp"], S_prefix=f["S_prefix"])
    return out


def warm_chain_job(args):
    """(layer, head) of the warm workload -> S_start [n_seg,d,d], o_seam [n_seg,w,d],
    S_final, all in request order."""
    layer, head = args
    wl = WORKLOADS["warm30_bf16"]
    lens = np.asarray(segment_lengths(wl))
    order = request_order(wl)
    cu = _cu(lens)
    x = conv_chain_inputs(wl, layer, head)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    r = O.warm_chain_reference(x["xq"][idx], x["xk"][idx], x["xv"][idx], x["wq"], x["wk"], x["wv"],
                               x["beta"][idx], x["log_alpha"][idx], lens[order], wl.seam)
    return {"S_start": r["S_start"], "o_seam": np.stack(r["o_seam"]), "S_final": r["S_final"]}


def run_pool(fn, jobs):
    """Run jobs on single-threaded worker processes (spawned: the parent may hold a GPU)."""
    n = max(1, min(len(jobs), 16, len(os.sched_getaffinity(0))))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(n) as pool:
            return pool.map(fn, jobs, chunksize=1)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def start_pool(fn, jobs):
    """Like run_pool, but returns (pool, AsyncResult) so GPU work can overlap."""
    n = max(1, min(len(jobs), 16, len(os.sched_getaffinity(0))))
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    pool = mp.get_context("spawn").Pool(n)
    return pool, pool.map_async(fn, jobs, chunksize=1)
