"""Benchmark of the state-composition hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input: the dense
gated-delta segment build of a 65,536-token prompt cut into 64 segments of 1,024
tokens (32 value heads on 16 key heads, d = 128, bf16 inputs; T_C and S(C|0) for
all 2,048 segment-heads in one launch), then the composition of the 64 cached
segments into one running state per head.  Inputs are resident in HBM before
the timed region.  Prints one JSON line.

Beside the headline line's fields, "rows" times every other step of the path on
its own workload shape (inputs filled on the device; the timing does not depend on
the values): the diagonal/scalar build (16 x 512 tokens, 16 RetNet + 16 GLA
heads); the headline layer under the precise-T plan, as a plain state pass, as the
output-fused build with and without T (the T overhead on the segment forward) and
its re-rotation to new offsets; the per-channel gated delta (KDA) build; the warm
30-layer path (conv warm-up of the seam tokens, seam advance, compose of 128
segments x 960 chains with prefix states, and the same path fused into one pass);
and the cold 100k-token 30-layer build in LPT, round-robin and natural order, with
the precise-T plan and the single sequential pass beside it.  Each carries its
algorithmic bytes or flops and the fraction of the matching MI355X peak; each row's
launches are timed one by one after a 512 MiB cache flush, so they read from HBM.
The last row, "mfma_probe", measures the dense f16 matrix-core rate this GPU
sustains on back-to-back products alone (libhypic_probe), with its clock.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-rows]
  python bench.py --calibrate-copy      (a plain 1 GiB device copy, for HBM counters)
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
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
PEAK_ALU_F32 = 157.3e12       # MI355X fp32 vector peak (packed fp32), FLOP/s
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


def engine_source_sha256():
    path = os.path.join(ROOT, "linear_attention_state_chunked_amd", "csrc", "gdn_build.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per build launch from the committed rocprofv3 counter summary, if it
    was taken on the current build engine source; else None."""
    path = os.path.join(ROOT, "profiles", "gdn_build_gdn64k_hbm_counters.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("engine source sha256") != engine_source_sha256():
        return None
    try:
        return float(kv["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
    gives the scale of the counters."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def time_events(fn, reps, stream):
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]


_FLUSH = None


def _flush_caches():
    """Write a 512 MiB buffer: evicts the L2 caches and the 256 MB MALL, so the next launch
    reads its inputs from HBM."""
    import torch

    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    _FLUSH.fill_(1)


def _median_time(fn, reps=5, warm=2):
    """Median of `reps` launches, each timed with HIP events after a cache flush (outside the
    events), so every row reads its inputs from HBM."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        _flush_caches()
        ts += time_events(fn, 1, stream)
    return float(np.median(ts))


def _hbm(nbytes, t):
    return {"s": t, "bytes": nbytes, "TB_per_s": nbytes / t / 1e12, "hbm_frac": nbytes / t / PEAK_HBM}


def _mfma(flops, t):
    return {"s": t, "flops": flops, "TFLOP_per_s": flops / t / 1e12, "mfma_frac": flops / t / PEAK_MFMA_F16}


def row_mfma_probe(dev):
    """Achievable dense f16 matrix-core rate of this GPU (libhypic_probe): 4 workgroups per CU of 8 waves,
    each wave with 4 independent v_mfma_f32_32x32x16_f16 products in flight on register operands, 10
    launches of about 4 ms back to back after 3 warm-up launches.  The clock is read inside the kernel
    (core-clock cycles over 100 MHz real-time ticks), so the rate per cycle comes out as well."""
    import torch

    L = C.CDLL(os.path.join(ROOT, "linear_attention_state_chunked_amd", "libhypic_probe.so"))
    L.hypic_probe_mfma_f16.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    L.hypic_probe_mfma_f16.restype = C.c_int
    L.hypic_probe_mfma_f16_flops.argtypes = [C.c_int, C.c_int]
    L.hypic_probe_mfma_f16_flops.restype = C.c_double
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    groups, iters = 4 * cus, 10000
    sink = torch.empty(groups * 512, dtype=torch.float32, device=dev)
    clocks = torch.empty(groups * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    ts, ghz = [], []
    for i in range(13):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = L.hypic_probe_mfma_f16(groups, iters, C.c_void_p(sink.data_ptr()), C.c_void_p(clocks.data_ptr()),
                                    C.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"hypic_probe_mfma_f16 returned {rc}")
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(e0.elapsed_time(e1) * 1e-3)
            c = clocks.view(-1, 2).double().cpu().numpy()
            ghz.append(float(np.median(c[:, 0] / (c[:, 1] * 10e-9))) * 1e-9)
    flops = L.hypic_probe_mfma_f16_flops(groups, iters)
    t, clk = float(np.median(ts)), float(np.median(ghz))
    return {"flops": flops, "s": t, "TFLOP_per_s": flops / t / 1e12, "frac_of_spec_peak": flops / t / PEAK_MFMA_F16,
            "clock_GHz": clk, "flop_per_cycle_per_cu": flops / (t * clk * 1e9 * cus), "compute_units": cus}


def row_diag(dev):
    """Diagonal / scalar-decay build and compose: 16 x 512 tokens, 16 RetNet heads
    (scalar) and 16 GLA heads (per-channel), d = 128, bf16 k and v."""
    import torch
    import torch.nn.functional as F

    from linear_attention_state_chunked_amd import api as H

    g = torch.Generator(device=dev)
    g.manual_seed(1)
    N, h, d, n_seg = 8192, 16, 128, 16
    cu = np.arange(0, N + 1, N // n_seg, dtype=np.int64)
    k = F.normalize(torch.randn(1, N, h, d, device=dev, generator=g), dim=-1).bfloat16()
    v = torch.randn(1, N, h, d, device=dev, generator=g).bfloat16()
    gam = 1.0 - 2.0 ** -(5.0 + 4.0 * torch.arange(h, device=dev) / 15.0)
    la_s = torch.log(gam)[None, None, :].expand(1, N, h).contiguous().float()
    la_g = (-F.softplus(-(2.0 + torch.randn(1, N, h, d, device=dev, generator=g))) / 16.0).float()
    out = {}
    for kind, la in (("scalar", la_s), ("diag", la_g)):
        t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, kind=kind))
        b = H.hypic_segment_build(k, v, la, cu, kind=kind)
        tlen = d if kind == "diag" else 1
        nbytes = 2 * k.numel() * 2 + la.numel() * 4 + n_seg * h * (d * d + tlen + 1) * 4
        row = _hbm(nbytes, t)
        row["flops"] = 2 * N * h * d * d
        Tn = b["T_hat"].reshape((n_seg, h) + ((d,) if kind == "diag" else ()))
        tc = _median_time(lambda: H.hypic_compose(Tn, b["T_exp"].reshape(n_seg, h), b["S"].reshape(n_seg, h, d, d),
                                                  kind=kind, mode="fold"))
        row["compose"] = _hbm(n_seg * h * (d * d + tlen + 1) * 4, tc)
        out[kind] = row
    return out


def row_warm(dev):
    """Warm 30-layer path, 128 cached segments x 32 value heads (16 key heads), seam
    w = 8: conv warm-up of the 1,024 seam tokens per layer with the carried conv
    state, seam build (T, S from zero), compose of the 256 interleaved (seam, rest)
    elements per chain with prefix states, seam outputs from the composed states."""
    import torch

    from linear_attention_state_chunked_amd import api as H

    L, hk, hv, d, n_slot, w = 30, 16, 32, 128, 128, 8
    nw, nc = n_slot * w, L * hv
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    rnd = lambda *sh, dt=torch.float32: torch.randn(*sh, device=dev, generator=g).to(dt)
    xs = {"q": rnd(L, nw, hk * d, dt=torch.bfloat16), "k": rnd(L, nw, hk * d, dt=torch.bfloat16),
          "v": rnd(L, nw, hv * d, dt=torch.bfloat16)}
    ws = {n: 0.5 * rnd(L, x.shape[2], 4) for n, x in xs.items()}
    st = {n: rnd(n_slot, L, 3, x.shape[2], dt=torch.bfloat16) for n, x in xs.items()}
    sidx = torch.from_numpy(np.concatenate([[-1], np.random.default_rng(3).permutation(n_slot)[:-1]]).astype(np.int32)).to(dev)
    cu_seam = np.arange(0, nw + 1, w, dtype=np.int64)
    beta = torch.sigmoid(rnd(L, nw, hv))
    la = -0.05 * torch.nn.functional.softplus(rnd(L, nw, hv))
    y = {}

    def conv():
        for n in ("q", "k", "v"):
            y[n] = H.hypic_conv_warmup(xs[n], ws[n], cu_seam, state_in=st[n], state_index=sidx,
                                       out_dtype=torch.float32, want_state=False)["y"]

    t_conv = _median_time(conv)
    conv()
    conv_bytes = sum(x.numel() * 2 + x.numel() * 4 + n_slot * L * 3 * x.shape[2] * 2 for x in xs.values())
    sq, sk, sv = y["q"].view(L, nw, hk, d), y["k"].view(L, nw, hk, d), y["v"].view(L, nw, hv, d)
    E_T = torch.empty((2 * n_slot, nc, d, d), device=dev)
    E_e = torch.full((2 * n_slot, nc), -60, dtype=torch.int32, device=dev)
    E_S = torch.empty((2 * n_slot, nc, d, d), device=dev)
    E_T[:n_slot].normal_(generator=g).mul_(0.05)
    E_S[:n_slot].normal_(generator=g)
    seam_out = {"T_hat": E_T[n_slot:].view(n_slot, L, hv, d, d), "T_exp": E_e[n_slot:].view(n_slot, L, hv),
                "S_seam": E_S[n_slot:].view(n_slot, L, hv, d, d)}
    seam1 = lambda: H.hypic_seam_advance(sq, sk, sv, la, beta, cu_seam, want_o=False, S_out=None, want_T=True,
                                         want_S_seam=True, qk_l2norm=True, out=seam_out)
    t_seam1 = _median_time(seam1)
    seam1()
    slot = np.empty(2 * n_slot, np.int32)
    slot[0::2] = n_slot + np.arange(n_slot)
    slot[1::2] = np.random.default_rng(3).permutation(n_slot)
    slot_d = torch.from_numpy(slot).to(dev)
    res = {}

    def compose():
        res["c"] = H.hypic_compose(E_T, E_e, E_S, slot=slot_d, mode="auto", want_prefix=True)

    t_comp = _median_time(compose, reps=3)
    pre = res["c"]["S_prefix"]
    seam2 = lambda: H.hypic_seam_advance(sq, sk, sv, la, beta, cu_seam, S_in=pre, state_stride=2 * nc * d * d,
                                         S_out=None, qk_l2norm=True, out_dtype=torch.float32)
    t_seam2 = _median_time(seam2)
    order_d = slot_d[1::2].contiguous()
    fused = lambda: H.hypic_compose_seam(E_T[:n_slot], E_e[:n_slot], E_S[:n_slot], sq, sk, sv, la, beta, cu_seam,
                                         slot=order_d, out_dtype=torch.float32, qk_l2norm=True)
    t_fused = _median_time(fused, reps=3)
    tok_bytes = (2 * hk + hv) * d * 4 * L * nw + 2 * hv * 4 * L * nw
    seam1_bytes = tok_bytes + 2 * n_slot * nc * d * d * 4 + n_slot * nc * 4
    comp_bytes = 2 * n_slot * nc * (2 * d * d * 4 + 4) + 2 * n_slot * nc * d * d * 4
    seam2_bytes = tok_bytes + n_slot * nc * d * d * 4 + L * nw * hv * d * 4
    # fused: read each cached (T_hat, S) once, the seam tokens, write the outputs and the final state
    fused_bytes = n_slot * nc * (2 * d * d * 4 + 4) + tok_bytes + L * nw * hv * d * 4 + nc * d * d * 4
    return {"conv_warmup": _hbm(conv_bytes, t_conv),
            "seam_build": _hbm(seam1_bytes, t_seam1),
            "compose_fold_prefix": dict(_hbm(comp_bytes, t_comp), us_per_segment=t_comp * 1e6 / n_slot),
            "seam_outputs": _hbm(seam2_bytes, t_seam2),
            "total_ms": (t_conv + t_seam1 + t_comp + t_seam2) * 1e3,
            "fused_seam_compose": dict(_hbm(fused_bytes, t_fused), us_per_segment=t_fused * 1e6 / n_slot),
            "fused_total_ms": (t_conv + t_fused) * 1e3}


def row_cold(dev):
    """Cold 100,000-token request, 30 layers x 32 value heads (16 key heads), 20
    segments of uneven length: the build of all 19,200 segment-heads in LPT,
    round-robin and natural task order, and the single sequential pass (no T); then one
    layer alone (640 segment-heads), where the task order and segment parallelism matter."""
    import torch

    from linear_attention_state_chunked_amd import api as H
    from synth import WORKLOADS, segment_lengths
    from synth.device_fill import fill_dense_layer_

    wl = WORKLOADS["cold100k_bf16"]
    lens = segment_lengths(wl)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, L, hk, hv, d = int(cu[-1]), wl.n_layers, wl.h_k, wl.h_v, wl.d
    k = torch.empty((L, N, hk, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((L, N, hv, d), dtype=torch.bfloat16, device=dev)
    beta = torch.empty((L, N, hv), device=dev)
    la = torch.empty((L, N, hv), device=dev)
    for layer in range(L):
        fill_dense_layer_(wl, layer, k[layer], v[layer], beta[layer], la[layer])
    n_seg = len(lens)
    out = {"T_hat": torch.empty((n_seg, L, hv, d, d), device=dev),
           "T_exp": torch.empty((n_seg, L, hv), dtype=torch.int32, device=dev),
           "S": torch.empty((n_seg, L, hv, d, d), device=dev)}
    chunks = sum((n + CHUNK - 1) // CHUNK for n in lens)
    flops = build_flops_per_chunk() * chunks * L * hv
    res = {}
    for sched in ("lpt", "rr", "natural"):
        t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, beta, schedule=sched, out=out), reps=3)
        res[sched] = _mfma(flops, t)
    single_flops = (2 * CHUNK * CHUNK * d / 2 + CHUNK ** 3 / 3 + 4 * CHUNK * CHUNK * d + 4 * CHUNK * d * d) \
        * ((N + CHUNK - 1) // CHUNK) * L * hv
    t = _median_time(lambda: H.hypic_segment_build(k, v, la, [0, N], beta, with_T=False), reps=3)
    res["single_pass_no_T"] = _mfma(single_flops, t)
    t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, beta, schedule="lpt", out=out,
                                                    precision="f16_precise_t"), reps=3)
    res["lpt_precise_T"] = _mfma(flops, t)
    E = (out["T_hat"].view(n_seg, L * hv, d, d), out["T_exp"].view(n_seg, L * hv), out["S"].view(n_seg, L * hv, d, d))
    tc = _median_time(lambda: H.hypic_compose(*E, mode="scan"), reps=3)
    res["compose_scan"] = dict(_hbm(n_seg * L * hv * (2 * d * d * 4 + 4), tc), us_per_segment=tc * 1e6 / n_seg)
    # one layer of the same request: 640 segment-heads of 512..8192 tokens on 256 compute units,
    # where the task order decides the makespan, against the single pass over the whole prompt
    # (32 chains: a long sequence alone cannot fill the device)
    one = {key: torch.empty((n_seg, 1) + tuple(t.shape[2:]), dtype=t.dtype, device=dev) for key, t in out.items()}
    k1, v1, la1, b1 = k[:1], v[:1], la[:1], beta[:1]
    res1 = {}
    for sched in ("lpt", "rr", "natural"):
        t = _median_time(lambda: H.hypic_segment_build(k1, v1, la1, cu, b1, schedule=sched, out=one), reps=3)
        res1[sched] = _mfma(flops / L, t)
    # the same segment lengths in increasing order over the same tokens (the longest last): the
    # order LPT protects against; the natural order then starts the longest tasks last
    cu_asc = np.concatenate([[0], np.cumsum(sorted(lens))]).astype(np.int64)
    t = _median_time(lambda: H.hypic_segment_build(k1, v1, la1, cu_asc, b1, schedule="natural", out=one), reps=3)
    res1["natural_ascending"] = _mfma(flops / L, t)
    t = _median_time(lambda: H.hypic_segment_build(k1, v1, la1, cu_asc, b1, schedule="lpt", out=one), reps=3)
    res1["lpt_ascending"] = _mfma(flops / L, t)
    t = _median_time(lambda: H.hypic_segment_build(k1, v1, la1, [0, N], b1, with_T=False), reps=3)
    res1["single_pass_no_T"] = _mfma(single_flops / L, t)
    res["one_layer"] = res1
    return res


def row_build_plans(dev):
    """The 64k-token GDN layer of the headline step under the other build plans: the
    precise-T plan (transition-only pass with hi/lo operands, then the state pass), the
    output-fused build (per-token outputs from each segment's zero start, with and without
    T: the T overhead on the segment forward), the plain state pass, and the RoPE
    re-rotation of the layer's 2,048 cached (T, S) elements."""
    import torch
    import torch.nn.functional as F

    from linear_attention_state_chunked_amd import api as H

    wl, inp, cu = make_inputs(dev)
    k, v, la, bt = inp["k"], inp["v"], inp["log_alpha"], inp["beta"]
    N, h_v = k.shape[1], v.shape[2]
    n_chunks = sum((int(cu[i + 1] - cu[i]) + 63) // 64 for i in range(len(cu) - 1))
    flops = build_flops_per_chunk() * n_chunks * h_v
    out = {}
    t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, bt, precision="f16_precise_t"))
    out["precise_T"] = _mfma(flops, t)
    t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, bt, with_T=False))
    # without T the carry covers the d state columns only: 4 C d d instead of 4 C d 2d
    state_flops = flops - 4 * CHUNK * D * D * n_chunks * h_v
    out["state_only"] = _mfma(state_flops, t)
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    q = F.normalize(torch.randn(k.shape, device=dev, generator=g), dim=-1).to(k.dtype)
    t_to = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, bt, q=q, want_o=True))
    t_o = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, bt, q=q, want_o=True, with_T=False))
    # algorithmic flops of the outputs per chunk: Q K^T (r-shared) and the two output products
    out_flops = (2 * CHUNK * CHUNK * D / 2 + 2 * CHUNK * D * D + 2 * CHUNK * CHUNK * D) * n_chunks * h_v
    out["output_fused_with_T"] = _mfma(flops + out_flops, t_to)
    out["output_fused_no_T"] = _mfma(flops - 4 * CHUNK * D * D * n_chunks * h_v + out_flops, t_o)
    out["output_fused_T_overhead_pct"] = (t_to / t_o - 1.0) * 100.0
    b = H.hypic_segment_build(k, v, la, cu, bt)
    n_seg = len(cu) - 1
    Tn, Sn = b["T_hat"].reshape(n_seg, h_v, D, D), b["S"].reshape(n_seg, h_v, D, D)
    delta = np.arange(n_seg, dtype=np.int64) * 1000 - 31_000
    t = _median_time(lambda: H.hypic_state_rerotate(Tn, Sn, delta, inplace=True))
    out["rerotate_T_and_S"] = _hbm(2 * 2 * Tn.numel() * 4, t)     # read and write T and S
    return out


def row_kda(dev):
    """Per-channel gated delta rule (KDA) build: 32 value heads on 16 key heads, d = 128,
    16 segments x 512 tokens, bf16 inputs; token recurrence in float32 vector arithmetic
    (bound: the vector ALUs; 157.3 TFLOP/s is the chip's fp32 vector peak with packed
    fp32 math, which this build does not use)."""
    import torch

    from linear_attention_state_chunked_amd import api as H
    from synth import WORKLOADS, layer_inputs, segment_lengths

    wl = WORKLOADS["kda_bf16"]
    x = layer_inputs(wl, 0, with_q=False)
    t_ = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    k, v = t_(x["k"][None], torch.bfloat16), t_(x["v"][None], torch.bfloat16)
    la, bt = t_(x["log_alpha"][None], torch.float32), t_(x["beta"][None], torch.float32)
    lens = segment_lengths(wl)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = _median_time(lambda: H.hypic_segment_build(k, v, la, cu, bt, kind="kda"))
    n_tok = int(cu[-1]) * wl.h_v
    # per token and column of [T | S]: k^T X (2d), decay and rank-1 update (3d), write (2d for S)
    flops = n_tok * (2 * D * (2 * D) + 3 * D * (2 * D) + 2 * D * D)
    return {"s": t, "flops": flops, "TFLOP_per_s": flops / t / 1e12, "alu_frac": flops / t / PEAK_ALU_F32,
            "tokens_per_s": int(cu[-1]) / t}


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
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
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

    # timed region: exactly K steps; HIP events on the launch stream bracket every build
    # and compose launch inside it (recording them costs no device time)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(path.stream)
        path.build()
        e[1].record(path.stream)
        path.compose()
        e[2].record(path.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = path.N * args.steps / wall

    # average per-launch device time of the dominant kernel (build) and of the compose
    t_build = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    t_comp = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    n_chunks = sum((int(cu[i + 1] - cu[i]) + 63) // 64 for i in range(len(cu) - 1))
    flops = build_flops_per_chunk() * n_chunks * path.h_v
    achieved = flops / t_build
    comp_bytes = path.n_seg * path.h_v * (2 * D * D * 4)     # read T_hat and S per element
    traffic = measured_traffic()
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
                     "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_F16, "traffic": traffic},
    }
    if not args.no_rows:
        del path, inp
        torch.cuda.empty_cache()
        rows = {}
        for name, fn in (("diag_scalar_build_16x512", row_diag), ("gdn64k_build_plans", row_build_plans),
                         ("kda_build_16x512", row_kda), ("warm30_seam_compose", row_warm),
                         ("cold100k_build", row_cold), ("mfma_probe", row_mfma_probe)):
            rows[name] = fn(dev)
            torch.cuda.empty_cache()
        out["rows"] = rows
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
