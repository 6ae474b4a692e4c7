"""The five synthetic workloads: shapes, value distributions and seeded streams.

Every tensor of every chain comes from its own stream
``numpy.random.default_rng([seed, layer, head, tensor_id])`` so that any single
(layer, head) chain can be regenerated on its own, bit for bit, for the CPU
reference while the device consumes the whole layer.

Distributions (the same for the device and the CPU reference):
  * keys and queries: i.i.d. N(0,1) rows, scaled to unit L2 norm;
  * values: i.i.d. N(0,1);
  * write strength beta = sigmoid(N(0,1)), float32;
  * gated-delta decay log(alpha) = -scale * softplus(N(0,1)), scale 0.05 (0.005 for
    the slow-decay workloads, 0 for the DeltaNet ones, alpha = 1), float32;
  * RetNet-style scalar decay gamma_h = 1 - 2**-(5 + 4h/15) for scalar head h;
  * GLA per-channel gates alpha = sigmoid(N(2,1)) ** (1/16), stored as log(alpha)
    (also the per-channel gates of the KDA workload, with beta as above);
  * pre-convolution activations N(0,1), depthwise conv taps N(0,1)/2.
bf16 workloads round k, v, q (and the pre-conv activations) to bfloat16 with
round-to-nearest-even; the rounded values are returned as float32 arrays that
hold them exactly, so the CPU reference sees exactly what the device sees.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids inside a stream key; never renumber (stored expectations depend on them)
TID = {
    "k": 0, "v": 1, "beta": 2, "alpha": 3, "q": 4,
    "xq": 5, "xk": 6, "xv": 7, "wq": 8, "wk": 9, "wv": 10,
    "gla": 11, "order": 12,
}


def stream(seed: int, layer: int, head: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng([seed, layer, head, TID[tensor]])


def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns float32 holding the rounded values exactly.  Finite inputs only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_layers: int
    h_k: int
    h_v: int
    d: int
    dtype: str                      # 'f32' or 'bf16' for q/k/v
    kind: str                       # 'dense', 'scalar', 'diag'
    alpha_scale: float = 0.05       # gated-delta decay scale
    seam: int = 0                   # seam window width w (0 = none)
    conv_width: int = 0             # depthwise conv width (0 = no conv)
    n_slots: int = 0                # cached segments (warm workload)
    fixed_lens: tuple = field(default=())

    def khead(self, vhead: int) -> int:
        """Grouped-query map: value head h reads key head floor(h*H_k/H_v)."""
        return (vhead * self.h_k) // self.h_v


def _lognormal_lens(seed: int, n: int, median: float, sigma: float, lo: int, hi: int):
    z = np.random.default_rng(seed).standard_normal(n)
    return tuple(int(v) for v in np.clip(np.exp(np.log(median) + sigma * z), lo, hi))


def _uniform_until(seed: int, lo: int, hi: int, total: int):
    rng = np.random.default_rng(seed)
    lens, acc = [], 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return tuple(lens)


WORKLOADS = {
    # tiny fp32 gated-delta head: 4 x 256 tokens
    "tiny_gdn_f32": Workload("tiny_gdn_f32", 0, 1, 1, 1, 64, "f32", "dense",
                             fixed_lens=(256,) * 4),
    # same, slow decay variant (weakly decaying transition keeps the
    # cross-segment term visible at fp32 tolerance)
    "tiny_gdn_f32_slow": Workload("tiny_gdn_f32_slow", 0, 1, 1, 1, 64, "f32", "dense",
                                  alpha_scale=0.005, fixed_lens=(256,) * 4),
    # scalar (RetNet) half of the diagonal/scalar workload: 16 heads x 16 x 512 tokens
    "retnet_bf16": Workload("retnet_bf16", 1, 1, 16, 16, 128, "bf16", "scalar",
                            fixed_lens=(512,) * 16),
    # GLA per-channel half of the same workload
    "gla_bf16": Workload("gla_bf16", 1, 1, 16, 16, 128, "bf16", "diag",
                         fixed_lens=(512,) * 16),
    # dense GDN layer: 32 v-heads on 16 k-heads, one 64k-token prompt = 64 x 1024
    "gdn64k_bf16": Workload("gdn64k_bf16", 2, 1, 16, 32, 128, "bf16", "dense",
                            fixed_lens=(1024,) * 64),
    # warm hit path: 30 layers x 32 heads, 128 cached segments, seam w=8, conv width 4
    "warm30_bf16": Workload("warm30_bf16", 3, 30, 16, 32, 128, "bf16", "dense",
                            seam=8, conv_width=4, n_slots=128),
    # long cold request: 100k tokens in uneven segments, 30 layers x 32 heads
    "cold100k_bf16": Workload("cold100k_bf16", 4, 30, 16, 32, 128, "bf16", "dense"),
    # composition checks where cross-segment terms stay large: slow decay (log alpha
    # scale 0.005) and no decay at all (alpha = 1, DeltaNet), 32 v-heads on 16 k-heads,
    # 16 x 1024 and 4 x 4096 tokens
    "gdn_slow16x1k_bf16": Workload("gdn_slow16x1k_bf16", 5, 1, 16, 32, 128, "bf16", "dense",
                                   alpha_scale=0.005, fixed_lens=(1024,) * 16),
    "gdn_slow4x4k_bf16": Workload("gdn_slow4x4k_bf16", 6, 1, 16, 32, 128, "bf16", "dense",
                                  alpha_scale=0.005, fixed_lens=(4096,) * 4),
    "delta16x1k_bf16": Workload("delta16x1k_bf16", 7, 1, 16, 32, 128, "bf16", "dense",
                                alpha_scale=0.0, fixed_lens=(1024,) * 16),
    "delta4x4k_bf16": Workload("delta4x4k_bf16", 8, 1, 16, 32, 128, "bf16", "dense",
                               alpha_scale=0.0, fixed_lens=(4096,) * 4),
    # per-channel gated delta rule (KDA): 32 v-heads on 16 k-heads, 16 x 512 tokens
    "kda_bf16": Workload("kda_bf16", 9, 1, 16, 32, 128, "bf16", "kda", fixed_lens=(512,) * 16),
}


def segment_lengths(wl: Workload) -> tuple:
    """Segment lengths in storage order (cached-slot order for the warm workload)."""
    if wl.fixed_lens:
        return wl.fixed_lens
    if wl.name.startswith("warm30"):
        # lognormal, median 700, sigma 0.5, clipped to [512, 4096]
        return _lognormal_lens(wl.seed, wl.n_slots, 700.0, 0.5, 512, 4096)
    if wl.name.startswith("cold100k"):
        # uniform 512..8192 (inclusive) until 100,000 tokens; the last one truncated
        return _uniform_until(wl.seed, 512, 8192, 100_000)
    raise KeyError(wl.name)


def request_order(wl: Workload) -> np.ndarray:
    """Order in which cached slots appear in the request (identity unless warm)."""
    n = len(segment_lengths(wl))
    if wl.n_slots:
        return stream(wl.seed, 0, 0, "order").permutation(n).astype(np.int64)
    return np.arange(n, dtype=np.int64)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(x.dtype)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return rne_bf16(x.astype(np.float32))


def _normal(rng, shape, dtype):
    if dtype == "f32":
        return rng.standard_normal(shape)              # float64, rounded once at the end
    return rng.standard_normal(shape, dtype=np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _key_like(wl, layer, khead, n, tensor):
    x = _normal(stream(wl.seed, layer, khead, tensor), (n, wl.d), wl.dtype)
    return _store(_unit_rows(x), wl.dtype)


def _value_side(wl: Workload, layer: int, vhead: int, n: int) -> dict:
    out = {"v": _store(_normal(stream(wl.seed, layer, vhead, "v"), (n, wl.d), wl.dtype), wl.dtype)}
    if wl.kind == "dense":
        b = stream(wl.seed, layer, vhead, "beta").standard_normal(n)
        a = stream(wl.seed, layer, vhead, "alpha").standard_normal(n)
        out["beta"] = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
        out["log_alpha"] = (-wl.alpha_scale * _softplus(a)).astype(np.float32)
    elif wl.kind == "scalar":
        g = 1.0 - 2.0 ** (-(5.0 + 4.0 * vhead / 15.0))
        out["log_alpha"] = np.full(n, np.log(g), dtype=np.float32)
    elif wl.kind == "diag":
        x = 2.0 + stream(wl.seed, layer, vhead, "gla").standard_normal((n, wl.d))
        out["log_alpha"] = (-_softplus(-x) / 16.0).astype(np.float32)
    elif wl.kind == "kda":
        # per-channel gates as the GLA heads', write strength as the gated delta rule's
        b = stream(wl.seed, layer, vhead, "beta").standard_normal(n)
        out["beta"] = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
        x = 2.0 + stream(wl.seed, layer, vhead, "gla").standard_normal((n, wl.d))
        out["log_alpha"] = (-_softplus(-x) / 16.0).astype(np.float32)
    else:
        raise ValueError(wl.kind)
    return out


def chain_inputs(wl: Workload, layer: int, vhead: int, n: int | None = None) -> dict:
    """Inputs of one (layer, value-head) chain over the whole storage-order stream.

    Returns float32 arrays: k, q [n, d] (of the mapped key head), v [n, d],
    beta [n] (dense only) and log_alpha ([n] dense/scalar, [n, d] diag).
    """
    if n is None:
        n = int(sum(segment_lengths(wl)))
    kh = wl.khead(vhead)
    out = {"k": _key_like(wl, layer, kh, n, "k"), "q": _key_like(wl, layer, kh, n, "q")}
    out.update(_value_side(wl, layer, vhead, n))
    return out


def layer_inputs(wl: Workload, layer: int, heads: range | None = None, with_q: bool = True) -> dict:
    """All chains of one layer in token-major layout.

    k, q: [N, H_k, d]; v: [N, H_v, d]; beta: [N, H_v]; log_alpha: [N, H_v]
    (diag: [N, H_v, d]).  Built head by head from the same streams as
    ``chain_inputs`` so both agree exactly.
    """
    n = int(sum(segment_lengths(wl)))
    hv = range(wl.h_v) if heads is None else heads
    khs = sorted({wl.khead(h) for h in hv})
    k = np.empty((n, wl.h_k, wl.d), np.float32)
    q = np.empty((n, wl.h_k, wl.d), np.float32) if with_q else None
    v = np.empty((n, wl.h_v, wl.d), np.float32)
    la_shape = (n, wl.h_v, wl.d) if wl.kind in ("diag", "kda") else (n, wl.h_v)
    la = np.zeros(la_shape, np.float32)
    beta = np.zeros((n, wl.h_v), np.float32)

    def key_job(kh):
        k[:, kh] = _key_like(wl, layer, kh, n, "k")
        if with_q:
            q[:, kh] = _key_like(wl, layer, kh, n, "q")

    def value_job(h):
        c = _value_side(wl, layer, h, n)
        v[:, h] = c["v"]
        la[:, h] = c["log_alpha"]
        if "beta" in c:
            beta[:, h] = c["beta"]

    # heads are independent streams: fill them concurrently (numpy releases the GIL)
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(key_job, khs))
        list(ex.map(value_job, hv))
    return {"k": k, "q": q, "v": v, "log_alpha": la, "beta": beta}


# ----------------------------------------------------------------------------------------
# warm workload: pre-convolution activations and conv taps (q || k || v channels)


def conv_chain_inputs(wl: Workload, layer: int, vhead: int) -> dict:
    """Pre-conv activations and taps feeding one (layer, value-head) chain.

    xq, xk [N, d] (mapped key head), xv [N, d]; taps wq, wk, wv [d, width]
    float32; beta [N]; log_alpha [N].  Storage (cached-slot) order.
    """
    n = int(sum(segment_lengths(wl)))
    kh = wl.khead(vhead)
    W = wl.conv_width
    out = {
        "xq": rne_bf16(stream(wl.seed, layer, kh, "xq").standard_normal((n, wl.d), dtype=np.float32)),
        "xk": rne_bf16(stream(wl.seed, layer, kh, "xk").standard_normal((n, wl.d), dtype=np.float32)),
        "xv": rne_bf16(stream(wl.seed, layer, vhead, "xv").standard_normal((n, wl.d), dtype=np.float32)),
        "wq": (0.5 * stream(wl.seed, layer, kh, "wq").standard_normal((wl.d, W))).astype(np.float32),
        "wk": (0.5 * stream(wl.seed, layer, kh, "wk").standard_normal((wl.d, W))).astype(np.float32),
        "wv": (0.5 * stream(wl.seed, layer, vhead, "wv").standard_normal((wl.d, W))).astype(np.float32),
    }
    b = stream(wl.seed, layer, vhead, "beta").standard_normal(n)
    a = stream(wl.seed, layer, vhead, "alpha").standard_normal(n)
    out["beta"] = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    out["log_alpha"] = (-wl.alpha_scale * _softplus(a)).astype(np.float32)
    return out


def layer_conv_inputs(wl: Workload, layer: int) -> dict:
    """One layer of the warm workload, token-major, storage order.

    x: [N, C] with C = (2*H_k + H_v)*d channels laid out q || k || v, each part
    head-major (channel = head*d + i); taps w: [C, width]; beta, log_alpha [N, H_v].
    """
    n = int(sum(segment_lengths(wl)))
    d, W = wl.d, wl.conv_width
    C = (2 * wl.h_k + wl.h_v) * d
    x = np.empty((n, C), np.float32)
    w = np.empty((C, W), np.float32)
    beta = np.empty((n, wl.h_v), np.float32)
    la = np.empty((n, wl.h_v), np.float32)
    qo, ko, vo = 0, wl.h_k * d, 2 * wl.h_k * d
    done_k = set()
    for h in range(wl.h_v):
        c = conv_chain_inputs(wl, layer, h)
        kh = wl.khead(h)
        if kh not in done_k:
            x[:, qo + kh * d: qo + (kh + 1) * d] = c["xq"]
            x[:, ko + kh * d: ko + (kh + 1) * d] = c["xk"]
            w[qo + kh * d: qo + (kh + 1) * d] = c["wq"]
            w[ko + kh * d: ko + (kh + 1) * d] = c["wk"]
            done_k.add(kh)
        x[:, vo + h * d: vo + (h + 1) * d] = c["xv"]
        w[vo + h * d: vo + (h + 1) * d] = c["wv"]
        beta[:, h] = c["beta"]
        la[:, h] = c["log_alpha"]
    return {"x": x, "w": w, "beta": beta, "log_alpha": la}


# ----------------------------------------------------------------------------------------
# synthetic element stores for the composition (well-conditioned transitions)


def random_elements(seed: int, n_slot: int, n_chain: int, d: int) -> dict:
    """A cache of n_slot elements for n_chain chains: T_hat = c Q (Q orthogonal from
    the QR factor of a Gaussian matrix, c ~ U[0.6, 1]), T_exp in {-1, 0}, S ~ N(0,1).
    Represented transitions have norm <= 1 and no preferred direction, so every
    product T_i X carries weight in the composed state.  float32 values."""
    rng = np.random.default_rng([seed, 0, 0, 13])
    T = np.empty((n_slot, n_chain, d, d), np.float32)
    for i in range(n_slot):
        for c in range(n_chain):
            q, r = np.linalg.qr(rng.standard_normal((d, d)))
            q = q * np.sign(np.diag(r))[None, :]
            T[i, c] = (rng.uniform(0.6, 1.0) * q).astype(np.float32)
    e = rng.integers(-1, 1, size=(n_slot, n_chain), endpoint=True).astype(np.int32)
    S = rng.standard_normal((n_slot, n_chain, d, d)).astype(np.float32)
    return {"T_hat": T, "T_exp": e, "S": S}
