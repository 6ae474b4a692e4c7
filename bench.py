"""Benchmark of the state-composition hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input: the dense
gated-delta segment build of a 65,536-token prompt cut into 64 segments of 1,024
tokens (32 value heads on 16 key heads, d = 128, bf16 inputs; T_C and S(C|0) for
all 2,048 segment-heads in one launch), then the composition of the 64 cached
segments into one running state per head.  Inputs are resident in HBM before
the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "segment-build tokens/s for (T_C,S|0) + compose µs/segment, % MFMA/HBM peak"
PEAK_MFMA_F16 = 2.5e15        # MI355X dense f16/bf16 matrix peak, FLOP/s
PEAK_HBM = 8.0e12             # MI355X HBM3E, B/s
D, CHUNK = 128, 64


def build_flops_per_chunk(d=D, c=CHUNK, r=2):
    """Algorithmic flops of one 64-token chunk of one value head (dense build with T):
    gram K K^T shared by r value heads, UT solve, W' and U, and the [T | S] carry."""
    return 2 * c * c * d / r + c ** 3 / 3 + 4 * c * c * d + 4 * c * d * (d + d)


def make_inputs(dev):
    import torch

    from synth import WORKLOADS, layer_inputs, segment_lengths

    wl = WORKLOADS["gdn64k_bf16"]
    x = layer_inputs(wl, 0, with_q=False)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    inp = {
        "k": t(x["k"][None], torch.bfloat16),
        "v": t(x["v"][None], torch.bfloat16),
        "beta": t(x["beta"][None], torch.float32),
        "log_alpha": t(x["log_alpha"][None], torch.float32),
    }
    lens = segment_lengths(wl)
    return wl, inp, np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


class Path:
    """Pre-built C-ABI descriptors and buffers: each step is two library calls."""

    def __init__(self, wl, inp, cu, dev, compose_mode="auto"):
        import torch

        from linear_attention_state_chunked_amd import _abi as A

        self.A, self.L = A, A.lib()
        self.cu = cu
        n_seg = len(cu) - 1
        B, N, h_k, d = inp["k"].shape
        h_v = inp["v"].shape[2]
        self.n_seg, self.h_v, self.N = n_seg, h_v, N
        f32 = torch.float32
        self.T_hat = torch.empty((n_seg, B, h_v, d, d), dtype=f32, device=dev)
        self.T_exp = torch.empty((n_seg, B, h_v), dtype=torch.int32, device=dev)
        self.S = torch.empty((n_seg, B, h_v, d, d), dtype=f32, device=dev)
        self.S_final = torch.empty((B * h_v, d, d), dtype=f32, device=dev)
        self.inp = inp
        self.bd = A.BuildDesc(kind=A.DENSE, in_dtype=A.BF16, n_batch=B, n_tokens=N, h_k=h_k, h_v=h_v, d_k=d, d_v=d,
                              chunk=64, n_seg=n_seg, cu_seqlens=cu.ctypes.data, skip_head=0, qk_l2norm=0,
                              k=inp["k"].data_ptr(), v=inp["v"].data_ptr(), log_alpha=inp["log_alpha"].data_ptr(),
                              beta=inp["beta"].data_ptr(), T_hat=self.T_hat.data_ptr(), T_exp=self.T_exp.data_ptr(),
                              S=self.S.data_ptr(), schedule=A.SCHED["natural"], precision=A.PREC["auto"])
        nb = self.L.hypic_segment_build_workspace_bytes(C.byref(self.bd))
        self.ws_b = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        self.bd.workspace, self.bd.workspace_bytes = self.ws_b.data_ptr(), self.ws_b.numel()
        self.cd = A.ComposeDesc(kind=A.DENSE, n_chain=B * h_v, d_k=d, d_v=d, n_elem=n_seg, n_slot=n_seg, slot=None,
                                T_hat=self.T_hat.data_ptr(), T_exp=self.T_exp.data_ptr(), S=self.S.data_ptr(),
                                S0=None, S_final=self.S_final.data_ptr(), S_prefix=None, T_total=None,
                                T_total_exp=None, mode=A.COMPOSE[compose_mode], scan_block=0)
        nc = self.L.hypic_compose_workspace_bytes(C.byref(self.cd))
        self.ws_c = torch.empty(max(nc, 256), dtype=torch.uint8, device=dev)
        self.cd.workspace, self.cd.workspace_bytes = self.ws_c.data_ptr(), self.ws_c.numel()
        self.stream = torch.cuda.current_stream()
        self.sp = C.c_void_p(self.stream.cuda_stream)

    def build(self):
        self.A.check(self.L.hypic_segment_build(C.byref(self.bd), self.sp))

    def compose(self):
        self.A.check(self.L.hypic_compose(C.byref(self.cd), self.sp))

    def step(self):
        self.build()
        self.compose()


def time_events(fn, reps, stream):
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]


def _oracle_chain(args):
    """CPU-baseline worker: the fp64 oracle over one (head, segment) chain."""
    h, lo, hi = args
    import oracle as O
    from synth import WORKLOADS, chain_inputs

    wl = WORKLOADS["gdn64k_bf16"]
    c = chain_inputs(wl, 0, h, hi)
    t0 = time.perf_counter()
    O.dense_recurrence(c["k"][lo:hi], c["v"][lo:hi], c["log_alpha"][lo:hi], c["beta"][lo:hi])
    return hi - lo, time.perf_counter() - t0


def cpu_baseline(budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the same workload on the host cores."""
    import multiprocessing as mp

    cores = min(16, len(os.sched_getaffinity(0)))
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    tasks = [(h, s * 1024, (s + 1) * 1024) for s in range(64) for h in range(32)]
    rng = np.random.default_rng(0)
    rng.shuffle(tasks)
    done_tok, busy, t0 = 0, 0.0, time.perf_counter()
    n_chains = 0
    with mp.get_context("spawn").Pool(cores) as pool:
        it = pool.imap_unordered(_oracle_chain, tasks[: cores * 64])
        for ntok, dt in it:
            done_tok += ntok
            busy += dt
            n_chains += 1
            if time.perf_counter() - t0 > budget_s:
                pool.terminate()
                break
    wall = time.perf_counter() - t0
    # aggregate rate of `cores` concurrently busy single-threaded workers
    token_heads_per_s = done_tok / busy * cores
    return {"value": token_heads_per_s / 32.0, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_chains} (value head, 1024-token segment) chains of the same workload, fp64 token loop "
                      f"with T, {cores} single-threaded worker processes for {wall:.1f} s; "
                      f"token-heads/s divided by the workload's 32 heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    wl, inp, cu = make_inputs(dev)
    path = Path(wl, inp, cu, dev)
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        path.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = path.N * args.steps / wall

    # per-call device time of the dominant kernel (build) and of the compose, HIP events
    # on the launch stream
    reps = max(5, args.steps)
    t_build = float(np.median(time_events(path.build, reps, path.stream)))
    t_comp = float(np.median(time_events(path.compose, reps, path.stream)))
    n_chunks = sum((int(cu[i + 1] - cu[i]) + 63) // 64 for i in range(len(cu) - 1))
    flops = build_flops_per_chunk() * n_chunks * path.h_v
    achieved = flops / t_build
    comp_bytes = path.n_seg * path.h_v * (2 * D * D * 4)     # read T_hat and S per element
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gdn64k_bf16: dense gated-delta layer, 32 value heads on 16 key heads, d=128, "
                               "bf16 q/k/v, fp32 state and T, one 65,536-token prompt = 64 segments x 1,024 "
                               "tokens, chunk 64; build all segments then compose into one running state",
                   "tokens": int(path.N), "segments": int(path.n_seg), "value_heads": int(path.h_v)},
        "build_ms": t_build * 1e3,
        "build_tokens_per_s": path.N / t_build,
        "compose_us": t_comp * 1e6,
        "compose_us_per_segment": t_comp * 1e6 / path.n_seg,
        "compose_hbm_frac": comp_bytes / t_comp / PEAK_HBM,
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_MFMA_F16 / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_F16, "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
