"""GPU parity: libhypic (through the C ABI) against the fp64 oracle.

Tolerances: relative Frobenius error per output block (one T, S or o matrix per
segment or seam and chain), 1e-5 for float32 inputs and 2e-3 for bf16 inputs
with float32 state and T.  T is compared exponent-aligned; an exactly-zero
reference block must be exactly zero on the device.
"""

import numpy as np
import pytest
import torch

import linear_attention_state_chunked_amd as H
import oracle as O
from synth import WORKLOADS, chain_inputs, segment_lengths
from tests.gpu_util import cu_of, dev_tensor, max_err, oracle_segments

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-3


def _dense_inputs(wl, n, h_v, layer=0, raw_keys=False):
    """Device inputs [1, n, h, d] for value heads 0..h_v-1 of workload wl, plus the
    per-chain numpy arrays for the oracle."""
    h_k = max(1, (h_v * wl.h_k) // wl.h_v)
    chains = [chain_inputs(wl, layer, h, n) for h in range(h_v)]
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    kk = np.stack([chains[(kh * wl.h_v) // wl.h_k]["k"] for kh in range(h_k)], axis=1)
    qq = np.stack([chains[(kh * wl.h_v) // wl.h_k]["q"] for kh in range(h_k)], axis=1)
    if raw_keys:
        rng = np.random.default_rng(99)
        scale = rng.uniform(0.5, 3.0, size=kk.shape[:2] + (1,)).astype(np.float32)
        kk = kk * scale
        qq = qq * scale
        if wl.dtype == "bf16":
            from synth import rne_bf16
            kk, qq = rne_bf16(kk), rne_bf16(qq)
    dev = {
        "k": dev_tensor(kk[None], dt),
        "q": dev_tensor(qq[None], dt),
        "v": dev_tensor(np.stack([c["v"] for c in chains], axis=1)[None], dt),
        "log_alpha": dev_tensor(np.stack([c["log_alpha"] for c in chains], axis=1)[None]),
    }
    if wl.kind == "dense":
        dev["beta"] = dev_tensor(np.stack([c["beta"] for c in chains], axis=1)[None])
    for h, c in enumerate(chains):
        kh = (h * h_k) // h_v
        c["k"] = kk[:, kh].astype(np.float32)
        c["q"] = qq[:, kh].astype(np.float32)
    return dev, chains


def _check_build(out, chains, lens, kind, tol, skip=0, normalise=False):
    errs_T, errs_S = [], []
    for h, c in enumerate(chains):
        k = O.l2_normalise(c["k"]) if normalise else c["k"]
        ref = oracle_segments(kind, k, c["v"], c["log_alpha"], c.get("beta"), lens, skip=skip)
        for s, r in enumerate(ref):
            S = out["S"][s, 0, h].cpu().numpy()
            if np.all(r["S"] == 0):
                assert np.all(S == 0), (s, h)
            else:
                errs_S.append(float(O.rel_err(S, r["S"])))
            if out["T_hat"] is not None:
                Th = out["T_hat"][s, 0, h].cpu().numpy()
                errs_T.append(float(O.rel_err_T(kind, Th, int(out["T_exp"][s, 0, h]), r["T_hat"], r["T_exp"])))
    assert max_err(errs_S) < tol, max_err(errs_S)
    assert max_err(errs_T) < tol, max_err(errs_T)
    return max_err(errs_T), max_err(errs_S)


# ----------------------------------------------------------------------------------------
# tiny fp32 gated-delta head: 4 x 256 tokens, build + compose against the 1024-token run


@pytest.mark.parametrize("name", ["tiny_gdn_f32", "tiny_gdn_f32_slow"])
def test_tiny_fp32_build_and_compose(gpu, name):
    wl = WORKLOADS[name]
    lens = segment_lengths(wl)
    n = sum(lens)
    dev, chains = _dense_inputs(wl, n, 1)
    out = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens), beta=dev["beta"])
    torch.cuda.synchronize()
    _check_build(out, chains, lens, "dense", TOL_F32)
    c = chains[0]
    full = O.dense_recurrence(c["k"], c["v"], c["log_alpha"], c["beta"])
    cuts = cu_of(lens)
    n_seg = len(lens)
    for mode in ("fold", "scan"):
        comp = H.hypic_compose(out["T_hat"].reshape(n_seg, 1, 64, 64), out["T_exp"].reshape(n_seg, 1),
                               out["S"].reshape(n_seg, 1, 64, 64), mode=mode, want_T=True, want_prefix=True,
                               scan_block=2)
        torch.cuda.synchronize()
        assert O.rel_err(comp["S_final"][0].cpu().numpy(), full["S"]) < TOL_F32, mode
        assert O.rel_err_T("dense", comp["T_total"][0].cpu().numpy(), int(comp["T_total_exp"][0]),
                           full["T_hat"], full["T_exp"]) < TOL_F32, mode
        for i in range(1, n_seg):
            lo = cuts[i]
            pre = O.dense_recurrence(c["k"][:lo], c["v"][:lo], c["log_alpha"][:lo], c["beta"][:lo])["S"]
            assert O.rel_err(comp["S_prefix"][i, 0].cpu().numpy(), pre) < TOL_F32, (mode, i)
        assert torch.all(comp["S_prefix"][0] == 0)


# ----------------------------------------------------------------------------------------
# composition of synthetic elements: well-conditioned transitions, request order by slot


@pytest.mark.parametrize("d", [64, 128])
def test_compose_random_elements(gpu, d):
    from synth import random_elements

    n_slot, n_chain, n_elem = 23, 3, 37
    el = random_elements(11 + d, n_slot, n_chain, d)
    slot = np.random.default_rng([11, d]).integers(0, n_slot, size=n_elem).astype(np.int32)
    S0 = np.random.default_rng([12, d]).standard_normal((n_chain, d, d)).astype(np.float32)
    refs = []
    for c in range(n_chain):
        elems = [{"T_hat": el["T_hat"][s, c], "T_exp": el["T_exp"][s, c], "S": el["S"][s, c]} for s in slot]
        refs.append(O.compose_fold("dense", elems, S0=S0[c]))
    Td, ed, Sd = dev_tensor(el["T_hat"]), dev_tensor(el["T_exp"], torch.int32), dev_tensor(el["S"])
    sd, S0d = dev_tensor(slot, torch.int32), dev_tensor(S0)
    for mode, blk in (("fold", 0), ("scan", 0), ("scan", 5), ("auto", 0)):
        r = H.hypic_compose(Td, ed, Sd, slot=sd, S0=S0d, mode=mode, want_T=True, want_prefix=True, scan_block=blk)
        torch.cuda.synchronize()
        for c in range(n_chain):
            ref = refs[c]
            eS = float(O.rel_err(r["S_final"][c].cpu().numpy(), ref["S_final"]))
            eT = float(O.rel_err_T("dense", r["T_total"][c].cpu().numpy(), int(r["T_total_exp"][c]),
                                   ref["T_hat"], ref["T_exp"]))
            eP = float(np.max(O.rel_err(r["S_prefix"][:, c].cpu().numpy(), ref["S_prefix"])))
            assert max(eS, eT, eP) < TOL_F32, (mode, blk, c, eS, eT, eP)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_elem", [1, 2, 3, 70, 130])
def test_compose_state_only_column_scales(gpu, d, n_elem):
    """Running state alone (no composed transition), the path that splits each chain's columns
    over workgroups: 9 chains (not a whole group of 8), slots, an initial state, element counts
    on both sides of a 64-element batch, and S0 and every S_i scaled by powers of two in
    [2^-40, 2^40].  The composition is linear in S, so each column of the result carries its
    column's scale exactly and is compared on its own.  Every mode gets one scale per 32-column
    block (the block width of the transition-carrying kernels, which scale a block as a whole);
    FOLD, whose state-only form scales each column on its own, also gets one scale per column."""
    from synth import random_elements

    n_slot, n_chain = 23, 9
    el = random_elements(31 + d + n_elem, n_slot, n_chain, d)
    rng = np.random.default_rng([31, d, n_elem])
    S1 = el["S"]
    S01 = rng.standard_normal((n_chain, d, d)).astype(np.float32)
    slot = rng.integers(0, n_slot, size=n_elem).astype(np.int32)
    Td, ed, sd = dev_tensor(el["T_hat"]), dev_tensor(el["T_exp"], torch.int32), dev_tensor(slot, torch.int32)

    def col_err(x, ref):
        # relative error of every column on its own
        return float(np.max(O.rel_err(np.swapaxes(x, -1, -2), np.swapaxes(ref, -1, -2), nd=1)))

    blocks = np.repeat(rng.integers(-40, 41, size=d // 32), 32)
    cols = rng.integers(-40, 41, size=d)
    for ex, modes in ((blocks, (("fold", 0), ("scan", 0), ("scan", 5), ("auto", 0))), (cols, (("fold", 0),))):
        cs = np.ldexp(1.0, ex).astype(np.float32)
        S, S0 = S1 * cs, S01 * cs
        refs = []
        for c in range(n_chain):
            elems = [{"T_hat": el["T_hat"][s, c], "T_exp": el["T_exp"][s, c], "S": S[s, c]} for s in slot]
            refs.append(O.compose_fold("dense", elems, S0=S0[c]))
        Sd, S0d = dev_tensor(S), dev_tensor(S0)
        for mode, blk in modes:
            if mode == "scan" and n_elem < 2:
                continue
            for want_prefix in (False, True):
                r = H.hypic_compose(Td, ed, Sd, slot=sd, S0=S0d, mode=mode, want_prefix=want_prefix,
                                    scan_block=blk)
                torch.cuda.synchronize()
                H.hypic_device_status()   # raises if a bounded wait ran out
                for c in range(n_chain):
                    ref = refs[c]
                    eS = col_err(r["S_final"][c].cpu().numpy(), ref["S_final"])
                    eP = col_err(r["S_prefix"][:, c].cpu().numpy(), ref["S_prefix"]) if want_prefix else 0.0
                    assert max(eS, eP) < TOL_F32, (mode, blk, want_prefix, c, eS, eP)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["scalar", "diag"])
def test_compose_random_elements_diag_scalar(gpu, d, kind):
    """Diagonal / scalar compose of random elements with slots, an initial state, prefix states
    and the composed transition, in every mode, and naive addition; against the oracle's fold."""
    n_slot, n_chain, n_elem = 23, 3, 37
    rng = np.random.default_rng([13, d, len(kind)])
    tshape = (n_slot, n_chain, d) if kind == "diag" else (n_slot, n_chain)
    T_hat = rng.uniform(0.5, 1.0, size=tshape).astype(np.float32)
    T_exp = rng.integers(-3, 1, size=(n_slot, n_chain)).astype(np.int32)
    S = rng.standard_normal((n_slot, n_chain, d, d)).astype(np.float32)
    slot = rng.integers(0, n_slot, size=n_elem).astype(np.int32)
    S0 = rng.standard_normal((n_chain, d, d)).astype(np.float32)
    refs = []
    for c in range(n_chain):
        elems = [{"T_hat": T_hat[s, c], "T_exp": T_exp[s, c], "S": S[s, c]} for s in slot]
        refs.append((O.compose_fold(kind, elems, S0=S0[c]), O.naive_add(elems, S0=S0[c])))
    Td, ed, Sd = dev_tensor(T_hat), dev_tensor(T_exp, torch.int32), dev_tensor(S)
    sd, S0d = dev_tensor(slot, torch.int32), dev_tensor(S0)
    for mode, blk in (("fold", 0), ("scan", 0), ("scan", 5), ("auto", 0)):
        r = H.hypic_compose(Td, ed, Sd, kind=kind, slot=sd, S0=S0d, mode=mode, want_T=True, want_prefix=True,
                            scan_block=blk)
        torch.cuda.synchronize()
        for c in range(n_chain):
            ref = refs[c][0]
            eS = float(O.rel_err(r["S_final"][c].cpu().numpy(), ref["S_final"]))
            eT = float(O.rel_err_T(kind, r["T_total"][c].cpu().numpy(), int(r["T_total_exp"][c]),
                                   ref["T_hat"], ref["T_exp"]))
            eP = float(np.max(O.rel_err(r["S_prefix"][:, c].cpu().numpy(), ref["S_prefix"])))
            assert max(eS, eT, eP) < TOL_F32, (mode, blk, c, eS, eT, eP)
    r = H.hypic_compose(None, None, Sd, kind=kind, slot=sd, S0=S0d, mode="naive_add")
    torch.cuda.synchronize()
    for c in range(n_chain):
        assert float(O.rel_err(r["S_final"][c].cpu().numpy(), refs[c][1])) < TOL_F32


# ----------------------------------------------------------------------------------------
# bf16 dense build: ragged segments spanning several chunks, empty segments, GQA


RAGGED = [1, 63, 64, 65, 130, 0, 300, 700]


@pytest.fixture(scope="module")
def ragged_dense(gpu):
    wl = WORKLOADS["gdn64k_bf16"]
    return (wl,) + _dense_inputs(wl, sum(RAGGED), 4)


def test_dense_bf16_ragged_build(ragged_dense):
    wl, dev, chains = ragged_dense
    out = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(RAGGED), beta=dev["beta"])
    torch.cuda.synchronize()
    H.hypic_device_status()      # no bounded wait of the build gave up
    eT, eS = _check_build(out, chains, RAGGED, "dense", TOL_BF16)
    print(f"ragged dense bf16: max T err {eT:.2e}, max S err {eS:.2e}")
    # the empty segment is the identity element
    e = RAGGED.index(0)
    Te = torch.ldexp(out["T_hat"][e, 0], out["T_exp"][e, 0][:, None, None].float())
    assert torch.equal(Te, torch.eye(128, device=Te.device).expand_as(Te))


def test_dense_bf16_skip_head_and_no_T(ragged_dense):
    wl, dev, chains = ragged_dense
    out = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(RAGGED), beta=dev["beta"], skip_head=8)
    plain = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(RAGGED), beta=dev["beta"],
                                  skip_head=8, with_T=False)
    torch.cuda.synchronize()
    _check_build(out, chains, RAGGED, "dense", TOL_BF16, skip=8)
    # the T columns never feed the S columns: the plain state pass is bitwise the same
    assert torch.equal(plain["S"], out["S"])


# ----------------------------------------------------------------------------------------
# output-fused build: each covered token's output from the segment's zero-start state, with
# T and S(C|0) as side outputs (the segment's own prefill forward)


def _check_outputs(o, chains, lens, tol, skip=0, normalise=False):
    """o [1, N, h, d] against the oracle's per-token outputs of each segment from zero."""
    worst = 0.0
    s0 = 0
    for n in lens:
        lo, hi = s0 + min(skip, n), s0 + n
        for h, c in enumerate(chains):
            k, q = (O.l2_normalise(c["k"]), O.l2_normalise(c["q"])) if normalise else (c["k"], c["q"])
            if hi > lo:
                r = O.dense_recurrence(k[lo:hi], c["v"][lo:hi], c["log_alpha"][lo:hi], c["beta"][lo:hi], q=q[lo:hi])
                got = o[0, lo:hi, h].float().cpu().numpy()
                e = float(O.rel_err(got, r["o"]))     # the segment's outputs as one block
                assert e < tol, f"segment [{lo}, {hi}) head {h}: output err {e:.3e}"
                worst = max(worst, e)
        s0 += n
    return worst


@pytest.mark.parametrize("variant", ["bf16", "bf16_skip_l2norm_no_T", "f32_d64"])
def test_output_fused_build(gpu, variant):
    if variant == "f32_d64":
        wl, lens, tol, h_v = WORKLOADS["tiny_gdn_f32"], [1, 63, 64, 65, 130, 0, 300], TOL_F32, 1
    else:
        wl, lens, tol, h_v = WORKLOADS["gdn64k_bf16"], RAGGED, TOL_BF16, 4
    skip, l2, with_T = (8, True, False) if variant == "bf16_skip_l2norm_no_T" else (0, False, True)
    dev, chains = _dense_inputs(wl, sum(lens), h_v, raw_keys=l2)
    out = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens), beta=dev["beta"], q=dev["q"],
                                want_o=True, out_dtype=torch.float32, skip_head=skip, qk_l2norm=l2, with_T=with_T)
    torch.cuda.synchronize()
    eo = _check_outputs(out["o"], chains, lens, tol, skip=skip, normalise=l2)
    eT, eS = _check_build(out, chains, lens, "dense", tol, skip=skip, normalise=l2)
    print(f"output-fused build {variant}: max o err {eo:.2e}, T err {eT:.2e}, S err {eS:.2e}")


def test_dense_bf16_l2norm_on_load(gpu):
    wl = WORKLOADS["gdn64k_bf16"]
    lens = [100, 64, 37]
    dev, chains = _dense_inputs(wl, sum(lens), 2, raw_keys=True)
    out = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens), beta=dev["beta"], qk_l2norm=True)
    torch.cuda.synchronize()
    _check_build(out, chains, lens, "dense", TOL_BF16, normalise=True)


@pytest.mark.parametrize("shift", [-8, 10])
@pytest.mark.parametrize("kind", ["dense", "diag"])
def test_f16_plan_value_range(gpu, kind, shift):
    """bf16 values scaled by 2^shift (exact in bf16): at |v| ~ 2^-8 the f16 operands stay
    normal, at |v| ~ 2^10 (largest |v| and |S| near 2^13) they stay below the f16 maximum, and
    the build holds the bf16 tolerance at both ends of the documented range."""
    lens = [64, 130, 700]
    if kind == "dense":
        dev, chains = _dense_inputs(WORKLOADS["gdn64k_bf16"], sum(lens), 2)
        k, la, beta = dev["k"], dev["log_alpha"], dev["beta"]
        v = dev["v"] * (2.0 ** shift)
    else:
        wl = WORKLOADS["gla_bf16"]
        chains = [chain_inputs(wl, 0, i, sum(lens)) for i in range(2)]
        k = dev_tensor(np.stack([c["k"] for c in chains], 1)[None], torch.bfloat16)
        v = dev_tensor(np.stack([c["v"] for c in chains], 1)[None], torch.bfloat16) * (2.0 ** shift)
        la, beta = dev_tensor(np.stack([c["log_alpha"] for c in chains], 1)[None]), None
    assert v.dtype == torch.bfloat16
    for c in chains:
        c["v"] = np.ldexp(c["v"], shift)
    out = H.hypic_segment_build(k, v, la, cu_of(lens), beta=beta, kind=kind)
    torch.cuda.synchronize()
    H.hypic_device_status()
    s_max = float(out["S"].abs().max())
    assert 2.0 ** (shift - 6) < s_max < 2.0 ** 15, s_max
    eT, eS = _check_build(out, chains, lens, kind, TOL_BF16)
    print(f"{kind} v x 2^{shift}: max |S| {s_max:.3g}, T err {eT:.2e}, S err {eS:.2e}")


def test_schedules_are_bitwise_identical(ragged_dense):
    wl, dev, chains = ragged_dense
    outs = []
    for sched in ("natural", "lpt", "rr", "natural"):
        o = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(RAGGED), beta=dev["beta"],
                                  schedule=sched)
        torch.cuda.synchronize()
        outs.append(o)
    for o in outs[1:]:
        assert torch.equal(o["S"], outs[0]["S"])
        assert torch.equal(o["T_hat"], outs[0]["T_hat"])
        assert torch.equal(o["T_exp"], outs[0]["T_exp"])


@pytest.mark.parametrize("variant", ["fast", "no_T_skip_head", "precise_T", "outputs", "outputs_no_T_skip_head"])
def test_stream_build_matches_per_task_build(gpu, variant):
    """Equal segments take the stream path (one persistent workgroup per compute unit running
    the chunks of its tasks back to back); the same segments built with one workgroup per task
    (a ragged last segment turns the stream off) must agree bit for bit, and a block from a
    workgroup's second task must match the oracle.  Variants: the fast plan; the plain state
    pass (no T) with a skipped head; segments over 2,048 tokens (hi/lo T operands); the
    output-fused build (per-token outputs, with T from its own pass, and without T with a
    skipped head)."""
    wl = WORKLOADS["gdn64k_bf16"]
    h_v = wl.h_v
    seg = 2112 if variant == "precise_T" else 256
    skip = 8 if variant.endswith("skip_head") else 0
    with_T = "no_T" not in variant
    outputs = variant.startswith("outputs")
    lens_u = [seg] * 16                      # 512 tasks: two per workgroup on 256 compute units
    lens_r = [seg] * 15 + [seg - 1]
    dev, chains = _dense_inputs(wl, sum(lens_u), h_v)
    kw = dict(beta=dev["beta"], with_T=with_T, skip_head=skip)
    if outputs:
        kw.update(q=dev["q"], want_o=True, out_dtype=torch.float32)
    uni = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens_u), **kw)
    rag = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens_r), **kw)
    torch.cuda.synchronize()
    for key in ("S", "T_hat", "T_exp") if with_T else ("S",):
        assert torch.equal(uni[key][:15], rag[key][:15]), key
    if outputs:
        covered = np.concatenate([np.arange(i * seg + skip, (i + 1) * seg) for i in range(15)])
        cov = torch.from_numpy(covered).cuda()
        assert torch.equal(uni["o"][:, cov], rag["o"][:, cov]), "o"
    s, h = 12, 5
    lo, hi = s * seg + skip, (s + 1) * seg
    c = chains[h]
    r = O.dense_recurrence(c["k"][lo:hi], c["v"][lo:hi], c["log_alpha"][lo:hi], c["beta"][lo:hi],
                           q=c["q"][lo:hi] if outputs else None)
    e_S = float(O.rel_err(uni["S"][s, 0, h].cpu().numpy(), r["S"]))
    e_T = e_o = 0.0
    if with_T:
        e_T = float(O.rel_err_T("dense", uni["T_hat"][s, 0, h].cpu().numpy(), int(uni["T_exp"][s, 0, h]),
                                r["T_hat"], r["T_exp"]))
    if outputs:
        e_o = float(O.rel_err(uni["o"][0, lo:hi, h].cpu().numpy(), r["o"]))
    print(f"stream build ({variant}), segment {s} head {h}: S {e_S:.2e}, T {e_T:.2e}, o {e_o:.2e}")
    assert e_S < TOL_BF16 and e_T < TOL_BF16 and e_o < TOL_BF16


def test_stream_build_d64_bf16(gpu):
    """The stream path at d = 64 with 16-bit inputs: one head, 512 equal segments of 256 tokens
    (two tasks per workgroup), against the per-task build bit for bit and the oracle on the
    rounded inputs."""
    wl = WORKLOADS["tiny_gdn_f32"]
    seg, n_seg = 256, 512
    c = chain_inputs(wl, 0, 0, seg * n_seg)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    k16, v16 = bf(c["k"]), bf(c["v"])
    dev = {"k": k16[None, :, None, :].cuda(), "v": v16[None, :, None, :].cuda(),
           "log_alpha": dev_tensor(c["log_alpha"][None, :, None]), "beta": dev_tensor(c["beta"][None, :, None])}
    lens_u = [seg] * n_seg
    lens_r = [seg] * (n_seg - 1) + [seg - 1]
    uni = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens_u), beta=dev["beta"])
    rag = H.hypic_segment_build(dev["k"], dev["v"], dev["log_alpha"], cu_of(lens_r), beta=dev["beta"])
    torch.cuda.synchronize()
    for key in ("S", "T_hat", "T_exp"):
        assert torch.equal(uni[key][:n_seg - 1], rag[key][:n_seg - 1]), key
    s = 300
    lo, hi = s * seg, (s + 1) * seg
    kr, vr = k16.float().numpy(), v16.float().numpy()
    r = O.dense_recurrence(kr[lo:hi], vr[lo:hi], c["log_alpha"][lo:hi], c["beta"][lo:hi])
    e_S = float(O.rel_err(uni["S"][s, 0, 0].cpu().numpy(), r["S"]))
    e_T = float(O.rel_err_T("dense", uni["T_hat"][s, 0, 0].cpu().numpy(), int(uni["T_exp"][s, 0, 0]),
                            r["T_hat"], r["T_exp"]))
    print(f"stream build d=64 bf16, segment {s}: S {e_S:.2e}, T {e_T:.2e}")
    assert e_S < TOL_BF16 and e_T < TOL_BF16


# ----------------------------------------------------------------------------------------
# diagonal (GLA) and scalar (RetNet) decay families


@pytest.mark.parametrize("name,kind", [("retnet_bf16", "scalar"), ("gla_bf16", "diag")])
def test_diag_scalar_build_compose_and_naive(gpu, name, kind):
    wl = WORKLOADS[name]
    lens = list(segment_lengths(wl))
    n, h = sum(lens), wl.h_v
    chains = [chain_inputs(wl, 0, i, n) for i in range(h)]
    k = dev_tensor(np.stack([c["k"] for c in chains], 1)[None], torch.bfloat16)
    v = dev_tensor(np.stack([c["v"] for c in chains], 1)[None], torch.bfloat16)
    la = dev_tensor(np.stack([c["log_alpha"] for c in chains], 1)[None])
    out = H.hypic_segment_build(k, v, la, cu_of(lens), kind=kind)
    torch.cuda.synchronize()
    # per-segment parity on every head
    _check_build(out, chains, lens, kind, TOL_BF16)
    n_seg = len(lens)
    tshape = (n_seg, h, 128) if kind == "diag" else (n_seg, h)
    comp = H.hypic_compose(out["T_hat"].reshape(tshape), out["T_exp"].reshape(n_seg, h),
                           out["S"].reshape(n_seg, h, 128, 128), kind=kind, mode="fold")
    naive = H.hypic_compose(None, None, out["S"].reshape(n_seg, h, 128, 128), kind=kind, mode="naive_add")
    torch.cuda.synchronize()
    fn = O.diag_recurrence if kind == "diag" else O.scalar_recurrence
    # the whole prompt per head, all heads as one batch of independent chains
    full = fn(np.stack([c["k"] for c in chains]), np.stack([c["v"] for c in chains]),
              np.stack([c["log_alpha"] for c in chains]))["S"]
    errs = O.rel_err(comp["S_final"].cpu().numpy(), full)
    naive_errs = O.rel_err(naive["S_final"].cpu().numpy(), full)
    for i in range(h):
        print(f"{name} head {i}: transition-compose err {errs[i]:.2e}, naive-addition err {naive_errs[i]:.3f}")
    assert float(np.max(errs)) < TOL_BF16
    assert float(np.min(naive_errs)) > 10 * TOL_BF16   # decay makes naive addition structurally wrong


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["scalar", "diag"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_diag_scalar_build_shapes(gpu, d, kind, dtype):
    """Diagonal / scalar build at both head sizes with 32- and 16-bit inputs, on ragged segments:
    empty, one token, a partial chunk, exactly one chunk, one token past it, and odd and even
    chunk counts with ragged tails; against the oracle on the inputs as the kernel sees them."""
    rng = np.random.default_rng(101 + d)
    lens = [0, 1, 63, 64, 65, 200, 130, 256]
    n, h = sum(lens), 2
    k = rng.standard_normal((n, h, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n, h, d))
    if kind == "scalar":
        la = np.log1p(-(2.0 ** -rng.uniform(3.0, 8.0, size=(n, h))))
    else:
        la = -np.logaddexp(0.0, -(2.0 + rng.standard_normal((n, h, d)))) / 16.0   # log sigmoid / 16
    la = la.astype(np.float32).astype(np.float64)   # the gates as the kernel reads them
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kt, vt = torch.from_numpy(k).to(tdt), torch.from_numpy(v).to(tdt)
    out = H.hypic_segment_build(kt[None].cuda(), vt[None].cuda(), dev_tensor(la[None]), cu_of(lens), kind=kind)
    torch.cuda.synchronize()
    kr, vr = kt.double().numpy(), vt.double().numpy()
    chains = [{"k": kr[:, i], "v": vr[:, i], "log_alpha": la[:, i]} for i in range(h)]
    e_T, e_S = _check_build(out, chains, lens, kind, TOL_BF16 if dtype == "bf16" else TOL_F32)
    print(f"{kind} d={d} {dtype}: T {e_T:.2e}, S {e_S:.2e}")


# ----------------------------------------------------------------------------------------
# seam advance


SEAM_WIDTHS = {"tiny": [1, 8, 0, 5, 8, 3, 2],              # all <= 8: closed rank-w kernel, 8-token instance
               "short": [1, 8, 16, 0, 5, 12, 3],          # all <= 16: closed rank-w kernel
               "long": [1, 8, 8, 33, 64, 0, 70]}          # some > 16: chunked engine


@pytest.mark.parametrize("widths", ["tiny", "short", "long"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_seam_advance(gpu, dtype, widths):
    wl = WORKLOADS["gdn64k_bf16" if dtype == "bf16" else "tiny_gdn_f32"]
    d = wl.d
    ws = SEAM_WIDTHS[widths]
    n = sum(ws)
    h_v = 2 if dtype == "bf16" else 1
    dev, chains = _dense_inputs(wl, n, h_v)
    rng = np.random.default_rng(5)
    S_in = rng.standard_normal((len(ws), 1, h_v, d, d)).astype(np.float32)
    res = H.hypic_seam_advance(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], cu_of(ws),
                               S_in=dev_tensor(S_in), want_T=True, want_S_seam=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    cuts = cu_of(ws)
    errs = {"o": [], "S_out": [], "T": [], "S_seam": []}
    for h, c in enumerate(chains):
        for s in range(len(ws)):
            lo, hi = cuts[s], cuts[s + 1]
            r = O.seam_advance(c["q"][lo:hi], c["k"][lo:hi], c["v"][lo:hi], c["log_alpha"][lo:hi],
                               c["beta"][lo:hi], S_in[s, 0, h])
            if hi > lo:
                errs["o"].append(float(O.rel_err(res["o"][0, lo:hi, h].cpu().numpy(), r["o"])))
            errs["S_out"].append(float(O.rel_err(res["S_out"][s, 0, h].cpu().numpy(), r["S_out"])))
            errs["T"].append(float(O.rel_err_T("dense", res["T_hat"][s, 0, h].cpu().numpy(),
                                               int(res["T_exp"][s, 0, h]), r["T_hat"], r["T_exp"])))
            S_seam = res["S_seam"][s, 0, h].cpu().numpy()
            if hi == lo:
                assert np.all(S_seam == 0)
            else:
                errs["S_seam"].append(float(O.rel_err(S_seam, r["S_seam"])))
    for key, e in errs.items():
        print(f"seam {dtype} {widths} {key}: max err {max_err(e):.2e}")
        assert max_err(e) < tol, key


def test_seam_in_place_and_strided(gpu):
    wl = WORKLOADS["gdn64k_bf16"]
    ws = [8, 8, 8]
    dev, chains = _dense_inputs(wl, sum(ws), 2)
    rng = np.random.default_rng(6)
    # states of 3 seams interleaved with 3 other blocks (stride = 2 dense blocks)
    buf = dev_tensor(rng.standard_normal((6, 1, 2, 128, 128)).astype(np.float32))
    orig = buf.clone()
    ref_in = buf[0::2].clone()
    stride = 2 * 2 * 128 * 128
    a = H.hypic_seam_advance(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], cu_of(ws),
                             S_in=ref_in, want_o=False)
    b = H.hypic_seam_advance(dev["q"], dev["k"], dev["v"], dev["log_alpha"], dev["beta"], cu_of(ws),
                             S_in=buf, S_out=buf, state_stride=stride, want_o=False)
    torch.cuda.synchronize()
    assert torch.equal(buf[0::2], a["S_out"])
    assert torch.equal(buf[1::2], orig[1::2])   # blocks between the seams untouched


# ----------------------------------------------------------------------------------------
# conv warm-up


@pytest.mark.parametrize("act,out_dtype", [("none", torch.float32), ("silu", torch.float32), ("none", torch.bfloat16)])
def test_conv_warmup(gpu, act, out_dtype):
    from synth import rne_bf16
    rng = np.random.default_rng(7)
    lens = [1, 2, 3, 8, 50, 0]
    n, C = sum(lens), 256
    x = rne_bf16(rng.standard_normal((n, C)).astype(np.float32))
    w = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    bias = rng.standard_normal(C).astype(np.float32)
    states = rne_bf16(rng.standard_normal((4, 1, 3, C)).astype(np.float32))
    idx = np.array([-1, 0, 2, 1, 3, 0], np.int32)
    res = H.hypic_conv_warmup(dev_tensor(x[None], torch.bfloat16), dev_tensor(w), cu_of(lens),
                              state_in=dev_tensor(states, torch.bfloat16),
                              state_index=torch.from_numpy(idx).to(gpu), bias=dev_tensor(bias), activation=act,
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    cuts = cu_of(lens)
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    for s in range(len(lens)):
        lo, hi = cuts[s], cuts[s + 1]
        st = None if idx[s] < 0 else states[idx[s], 0]
        y, so = O.causal_conv(x[lo:hi], w, bias=bias, state=st, activation=act)
        if hi > lo:
            assert O.rel_err(res["y"][0, lo:hi].float().cpu().numpy(), y) < tol, s
        # the carried state is a copy: bit-exact
        assert np.array_equal(res["state_out"][s, 0].float().cpu().numpy(), so.astype(np.float32)), s


# ----------------------------------------------------------------------------------------
# RoPE state re-rotation of cached elements moved to a new offset


@pytest.mark.parametrize("d,rd,interleaved,kind,n_elem,inplace", [
    (128, 128, False, "dense", 5, False),
    (128, 96, True, "dense", 4, True),
    (64, 32, False, "scalar", 6, False),
    (64, 64, True, "dense", 170, False),      # more shifts than one launch carries
])
def test_rerotate_elements(gpu, d, rd, interleaved, kind, n_elem, inplace):
    rng = np.random.default_rng(500 + d + rd + n_elem)
    n_chain = 3 if n_elem < 100 else 2
    T = rng.standard_normal((n_elem, n_chain, d, d)).astype(np.float32)
    S = rng.standard_normal((n_elem, n_chain, d, d)).astype(np.float32)
    delta = rng.integers(-200_000, 200_000, size=n_elem).astype(np.int64)
    delta[0] = 0
    Td, Sd = dev_tensor(T), dev_tensor(S)
    r = H.hypic_state_rerotate(Td if kind == "dense" else None, Sd, delta, kind=kind, rotary_dim=rd,
                               rope_base=10000.0, interleaved=interleaved, inplace=inplace)
    torch.cuda.synchronize()
    if inplace:
        assert r["S"].data_ptr() == Sd.data_ptr()
    Sg = r["S"].cpu().numpy()
    Tg = r["T_hat"].cpu().numpy() if kind == "dense" else None
    worst = 0.0
    for e in range(n_elem):
        for c in range(n_chain):
            ref = O.rerotate(kind, T[e, c] if kind == "dense" else np.float64(1.0), 0, S[e, c], int(delta[e]), rd,
                             10000.0, interleaved)
            err = float(O.rel_err(Sg[e, c], ref["S"]))
            if kind == "dense":
                err = max(err, float(O.rel_err(Tg[e, c], ref["T_hat"])))
            worst = max(worst, err)
    print(f"rerotate d={d} rd={rd} interleaved={interleaved} {kind} x{n_elem}: max err {worst:.2e}")
    assert worst < TOL_F32
    assert np.array_equal(Sg[0], S[0])          # a zero shift is the identity, bit for bit


def test_rerotate_end_to_end_at_new_offset(gpu):
    """Cache two segments with keys rotated at their original offsets (fp32, d = 64, the F32
    plan), re-rotate both to the offsets of a different request and compose them: the state
    equals the recurrence over the keys rotated at the new positions."""
    wl = WORKLOADS["tiny_gdn_f32"]
    c = chain_inputs(wl, 0, 0, 512)
    rd, base = 48, 5000.0
    lens = [300, 212]
    p_old = [7000, 123]            # where each segment was first prefilled
    p_new = [40, 340]              # where the request places them (contiguous from 40)
    ks, vs, las, bts = [], [], [], []
    s0 = 0
    for n, p in zip(lens, p_old):
        ks.append(O.rope_rotate(c["k"][s0:s0 + n], p + np.arange(n), rd, base, False).astype(np.float32))
        vs.append(c["v"][s0:s0 + n]); las.append(c["log_alpha"][s0:s0 + n]); bts.append(c["beta"][s0:s0 + n])
        s0 += n
    k = dev_tensor(np.concatenate(ks)[None, :, None])
    v = dev_tensor(np.concatenate(vs)[None, :, None])
    la = dev_tensor(np.concatenate(las)[None, :, None])
    bt = dev_tensor(np.concatenate(bts)[None, :, None])
    b = H.hypic_segment_build(k, v, la, cu_of(lens), bt)
    delta = np.array([pn - po for pn, po in zip(p_new, p_old)], np.int64)
    r = H.hypic_state_rerotate(b["T_hat"].reshape(2, 1, 64, 64), b["S"].reshape(2, 1, 64, 64), delta,
                               rotary_dim=rd, rope_base=base)
    comp = H.hypic_compose(r["T_hat"], b["T_exp"].reshape(2, 1), r["S"], mode="fold", want_T=True)
    torch.cuda.synchronize()
    k_new = np.concatenate([O.rope_rotate(c["k"][a:a + n], p + np.arange(n), rd, base, False)
                            for a, n, p in ((0, lens[0], p_new[0]), (lens[0], lens[1], p_new[1]))])
    full = O.dense_recurrence(k_new, c["v"][:512], c["log_alpha"][:512], c["beta"][:512])
    eS = float(O.rel_err(comp["S_final"][0].cpu().numpy(), full["S"]))
    eT = float(O.rel_err_T("dense", comp["T_total"][0].cpu().numpy(), int(comp["T_total_exp"][0]),
                           full["T_hat"], full["T_exp"]))
    # without the re-rotation the composed state is wrong at the new offsets
    stale = H.hypic_compose(b["T_hat"].reshape(2, 1, 64, 64), b["T_exp"].reshape(2, 1), b["S"].reshape(2, 1, 64, 64),
                            mode="fold")
    e_stale = float(O.rel_err(stale["S_final"][0].cpu().numpy(), full["S"]))
    print(f"rerotated compose at the new offsets: S {eS:.2e}, T {eT:.2e} (without re-rotation {e_stale:.2e})")
    assert eS < TOL_F32 and eT < TOL_F32
    assert e_stale > 100 * TOL_F32


# ----------------------------------------------------------------------------------------
# per-channel gated delta rule (KDA): build, and composition through the dense law


def _kda_segments(c, lens):
    out, s0 = [], 0
    for n in lens:
        out.append(O.kda_recurrence(c["k"][s0:s0 + n], c["v"][s0:s0 + n], c["log_alpha"][s0:s0 + n],
                                    c["beta"][s0:s0 + n]))
        s0 += n
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kda_build_ragged_and_compose(gpu, dtype):
    wl = WORKLOADS["kda_bf16"]
    lens = [0, 1, 63, 64, 65, 200, 130, 300] if dtype == "bf16" else [1, 17, 129, 0, 90]
    n, h_v = sum(lens), 4 if dtype == "bf16" else 2
    dt, tol = (torch.bfloat16, TOL_BF16) if dtype == "bf16" else (torch.float32, TOL_F32)
    chains = [chain_inputs(wl, 0, h, n) for h in range(h_v)]
    h_k = h_v // 2
    kk = np.stack([chains[2 * kh]["k"] for kh in range(h_k)], axis=1)
    for h, c in enumerate(chains):
        c["k"] = kk[:, h // 2]
        if dtype == "f32":      # full-precision values (the workload's are bf16-exact)
            c["v"] = c["v"] + np.float32(1e-3) * np.sin(np.arange(c["v"].size, dtype=np.float32)).reshape(c["v"].shape)
    k = dev_tensor(kk[None], dt)
    v = dev_tensor(np.stack([c["v"] for c in chains], 1)[None], dt)
    la = dev_tensor(np.stack([c["log_alpha"] for c in chains], 1)[None])
    bt = dev_tensor(np.stack([c["beta"] for c in chains], 1)[None])
    out = H.hypic_segment_build(k, v, la, cu_of(lens), bt, kind="kda")
    plain = H.hypic_segment_build(k, v, la, cu_of(lens), bt, kind="kda", with_T=False)
    n_seg = len(lens)
    E = (out["T_hat"].reshape(n_seg, h_v, 128, 128), out["T_exp"].reshape(n_seg, h_v),
         out["S"].reshape(n_seg, h_v, 128, 128))
    fold = H.hypic_compose(*E, kind="kda", mode="fold", want_T=True, want_prefix=True)
    scan = H.hypic_compose(*E, kind="kda", mode="scan", want_T=True, scan_block=3)
    torch.cuda.synchronize()
    assert torch.equal(plain["S"], out["S"])       # the T columns never feed the state columns
    wT = wS = wF = 0.0
    for h, c in enumerate(chains):
        refs = _kda_segments(c, lens)
        for s, r in enumerate(refs):
            S = out["S"][s, 0, h].cpu().numpy()
            if lens[s] == 0:
                Te = torch.ldexp(out["T_hat"][s, 0, h], out["T_exp"][s, 0, h].float())
                assert torch.equal(Te, torch.eye(128, device=Te.device)) and not S.any()
                continue
            eT = float(O.rel_err_T("dense", out["T_hat"][s, 0, h].cpu().numpy(), int(out["T_exp"][s, 0, h]),
                                   r["T_hat"], r["T_exp"]))
            eS = float(O.rel_err(S, r["S"]))
            assert eT < tol and eS < tol, f"{dtype} head {h} segment {s}: T {eT:.3e}, S {eS:.3e}"
            wT, wS = max(wT, eT), max(wS, eS)
        full = O.kda_recurrence(c["k"], c["v"], c["log_alpha"], c["beta"])
        for lab, cc in (("fold", fold), ("scan", scan)):
            eF = float(O.rel_err(cc["S_final"][h].cpu().numpy(), full["S"]))
            eTT = float(O.rel_err_T("dense", cc["T_total"][h].cpu().numpy(), int(cc["T_total_exp"][h]),
                                    full["T_hat"], full["T_exp"]))
            assert eF < tol and eTT < tol, f"{dtype} {lab} head {h}: S_final {eF:.3e}, T_total {eTT:.3e}"
            wF = max(wF, eF, eTT)
    print(f"kda {dtype}: segment T {wT:.2e}, S {wS:.2e}; composed S_final / T_total {wF:.2e}")


# ----------------------------------------------------------------------------------------
# fused warm path: seam window + composition in one pass, state kept on chip


@pytest.mark.parametrize("dtype,l2", [("f32", False), ("bf16", True)])
def test_compose_seam_fused(gpu, dtype, l2):
    from synth import random_elements, rne_bf16

    rng = np.random.default_rng(77)
    d, B, h_k, h_v = 128, 2, 1, 2
    n_chain, n_slot = B * h_v, 6
    el = random_elements(78, n_slot, n_chain, d)     # well-conditioned T: every cross term counts
    slots = np.array([3, 0, 5, 0, 2, 4, 1], np.int32)
    widths = [8, 3, 0, 8, 1, 5, 8]
    cu = np.concatenate([[0], np.cumsum(widths)]).astype(np.int64)
    N = int(cu[-1])
    q = rng.standard_normal((B, N, h_k, d)).astype(np.float32)
    k = rng.standard_normal((B, N, h_k, d)).astype(np.float32)
    if not l2:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, N, h_v, d)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, N, h_v))))).astype(np.float32)
    la = (-0.05 * np.logaddexp(0.0, rng.standard_normal((B, N, h_v)))).astype(np.float32)
    if dtype == "bf16":
        q, k, v = rne_bf16(q), rne_bf16(k), rne_bf16(v)
    dt, tol = (torch.float32, TOL_F32) if dtype == "f32" else (torch.bfloat16, TOL_BF16)
    S0 = rng.standard_normal((n_chain, d, d)).astype(np.float32)
    r = H.hypic_compose_seam(dev_tensor(el["T_hat"]), torch.from_numpy(el["T_exp"]).to("cuda:0"),
                             dev_tensor(el["S"]), dev_tensor(q, dt), dev_tensor(k, dt), dev_tensor(v, dt),
                             dev_tensor(la), dev_tensor(beta), cu, slot=torch.from_numpy(slots).to("cuda:0"),
                             S0=dev_tensor(S0), want_prefix=True, out_dtype=torch.float32, qk_l2norm=l2)
    torch.cuda.synchronize()
    o, Sf, Sp = r["o"].cpu().numpy(), r["S_final"].cpu().numpy(), r["S_prefix"].cpu().numpy()
    worst = 0.0
    for c in range(n_chain):
        b, h = c // h_v, c % h_v
        kk = O.l2_normalise(k[b, :, 0]) if l2 else k[b, :, 0]
        qq = O.l2_normalise(q[b, :, 0]) if l2 else q[b, :, 0]
        S = S0[c].astype(np.float64)
        for i, s in enumerate(slots):
            e = float(O.rel_err(Sp[i, c], S))
            lo, hi = int(cu[i]), int(cu[i + 1])
            if hi > lo:
                run = O.dense_recurrence(kk[lo:hi], v[b, lo:hi, h], la[b, lo:hi, h], beta[b, lo:hi, h], S0=S,
                                         q=qq[lo:hi])
                e = max(e, float(O.rel_err(o[b, lo:hi, h], run["o"])))
                S = run["S"]
            S = O.apply_T("dense", el["T_hat"][s, c], el["T_exp"][s, c], S) + el["S"][s, c]
            assert e < tol, f"chain {c} position {i}: err {e:.3e}"
            worst = max(worst, e)
        e = float(O.rel_err(Sf[c], S))
        assert e < tol, f"chain {c}: final state err {e:.3e}"
        worst = max(worst, e)
    print(f"fused seam + compose {dtype}: max err {worst:.2e}")
