"""The chunked WY/UT form (the device algorithm, in fp64) equals the oracle."""

import numpy as np
import pytest

import oracle as O
from synth import WORKLOADS, chain_inputs
from tests.chunk_ref import chunk_outputs, chunked_build


@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 256])
def test_chunk_form_equals_token_recurrence(n):
    wl = WORKLOADS["tiny_gdn_f32"]
    c = chain_inputs(wl, 0, 0)
    k, v, la, b = c["k"][:n], c["v"][:n], c["log_alpha"][:n], c["beta"][:n]
    Th, e, S = chunked_build(k, v, la, b)
    r = O.dense_recurrence(k, v, la, b)
    assert O.rel_err_T("dense", Th, e, r["T_hat"], r["T_exp"]) < 1e-13
    assert O.rel_err(S, r["S"]) < 1e-13


def test_seam_form_equals_token_recurrence():
    rng = np.random.default_rng(3)
    wl = WORKLOADS["tiny_gdn_f32"]
    c = chain_inputs(wl, 0, 0)
    S0 = rng.standard_normal((64, 64))
    sl = slice(100, 108)
    O_, S_ = chunk_outputs(c["q"][sl], c["k"][sl], c["v"][sl], c["log_alpha"][sl], c["beta"][sl], S0)
    r = O.dense_recurrence(c["k"][sl], c["v"][sl], c["log_alpha"][sl], c["beta"][sl], S0=S0, q=c["q"][sl])
    assert np.max(O.rel_err(O_, r["o"])) < 1e-13
    assert O.rel_err(S_, r["S"]) < 1e-13
