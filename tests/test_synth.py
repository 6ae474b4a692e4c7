"""The seeded generators: stream independence and storage rounding."""

import numpy as np
import torch

from synth import WORKLOADS, chain_inputs, layer_inputs, rne_bf16, segment_lengths


def test_rne_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000), rng.standard_normal(1000) * 1e-30,
                        rng.standard_normal(1000) * 1e30]).astype(np.float32)
    assert np.array_equal(rne_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_layer_inputs_equal_chain_inputs():
    wl = WORKLOADS["gdn64k_bf16"]
    n = 256
    import dataclasses
    small = dataclasses.replace(wl, fixed_lens=(128, 128))
    x = layer_inputs(small, 0)
    for h in (0, 1, 7, 31):
        c = chain_inputs(small, 0, h, n)
        kh = small.khead(h)
        for key, ref in (("k", x["k"][:, kh]), ("q", x["q"][:, kh]), ("v", x["v"][:, h]),
                         ("beta", x["beta"][:, h]), ("log_alpha", x["log_alpha"][:, h])):
            assert np.array_equal(c[key], ref), (h, key)
    assert np.allclose(np.linalg.norm(x["k"], axis=-1), 1.0, atol=1e-2)   # unit rows, bf16-rounded
    assert np.array_equal(rne_bf16(x["v"]), x["v"])


def test_decay_ranges():
    wl = WORKLOADS["tiny_gdn_f32"]
    c = chain_inputs(wl, 0, 0)
    assert np.all(c["log_alpha"] < 0) and np.all((c["beta"] > 0) & (c["beta"] < 1))
    r = chain_inputs(WORKLOADS["retnet_bf16"], 0, 15, 64)
    assert np.allclose(np.exp(r["log_alpha"]), 1 - 2.0 ** -9)
    g = chain_inputs(WORKLOADS["gla_bf16"], 0, 3, 64)
    assert g["log_alpha"].shape == (64, 128) and np.all(g["log_alpha"] < 0)
    assert sum(segment_lengths(WORKLOADS["cold100k_bf16"])) == 100_000
