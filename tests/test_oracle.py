"""Pins of the fp64 oracle against what the HYPIC pages and mathematics fix.

Nothing here compares the oracle with itself: each check uses an independent
formulation (explicit matrix products, closed forms, special cases, the pages'
printed figure, exhaustive search) chosen so that a dropped term, a wrong sign
or index, or a transposed operand in the oracle fails at least one of them.
"""

import itertools
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_chain(rng, n, dk, dv, unit=False):
    k = rng.standard_normal((n, dk))
    if unit:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    la = -0.3 * rng.random(n)
    b = rng.random(n)
    q = rng.standard_normal((n, dk))
    return k, v, la, b, q


def _A(k, la, b):
    """Explicit per-token transition alpha (I - beta k k^T)."""
    return np.exp(la) * (np.eye(len(k)) - b * np.outer(k, k))


def _brute(k, v, la, b, S0=None):
    """T = A_n ... A_1 and S = T S0 + sum_t (A_n ... A_{t+1}) beta_t k_t v_t^T,
    by explicit dense products (no rank-1 updates)."""
    n, dk = k.shape
    As = [_A(k[t], la[t], b[t]) for t in range(n)]
    T = np.eye(dk)
    for A in As:
        T = A @ T
    S = np.zeros((dk, v.shape[1])) if S0 is None else T @ S0
    for t in range(n):
        P = np.eye(dk)
        for A in As[t + 1:]:
            P = A @ P
        S = S + P @ (b[t] * np.outer(k[t], v[t]))
    return T, S


def _as_el(r):
    return {"T_hat": r["T_hat"], "T_exp": r["T_exp"], "S": r["S"]}


# ----------------------------------------------------------------------------------------
# token recurrence


@pytest.mark.parametrize("dk,dv", [(1, 1), (2, 3), (3, 2), (4, 4), (4, 1)])
@pytest.mark.parametrize("n", [1, 2, 3, 6])
def test_dense_brute_force(dk, dv, n):
    rng = np.random.default_rng(100 * dk + 10 * dv + n)
    k, v, la, b, q = _rand_chain(rng, n, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    r = O.dense_recurrence(k, v, la, b, S0=S0, q=q, renorm_every=2)
    T, S = _brute(k, v, la, b, S0)
    assert np.allclose(O.T_value("dense", r["T_hat"], r["T_exp"]), T, rtol=0, atol=1e-14)
    assert np.allclose(r["S"], S, rtol=0, atol=1e-13)
    # outputs: o_t = S_t^T q_t with S_t the state after token t
    for t in range(n):
        _, St = _brute(k[:t + 1], v[:t + 1], la[:t + 1], b[:t + 1], S0)
        assert np.allclose(r["o"][t], St.T @ q[t], rtol=0, atol=1e-13)


def test_single_token_closed_form():
    rng = np.random.default_rng(1)
    k, v, la, b, _ = _rand_chain(rng, 1, 5, 3)
    r = O.dense_recurrence(k, v, la, b)
    a = np.exp(la[0])
    assert np.allclose(O.T_value("dense", r["T_hat"], r["T_exp"]),
                       a * (np.eye(5) - b[0] * np.outer(k[0], k[0])), atol=1e-15)
    # the write is not decayed at its own step
    assert np.allclose(r["S"], b[0] * np.outer(k[0], v[0]), atol=1e-15)


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    k, v, la, _, _ = _rand_chain(rng, 40, 6, 4)
    r = O.dense_recurrence(k, v, la, np.zeros(40))
    assert np.allclose(O.T_value("dense", r["T_hat"], r["T_exp"]), np.exp(la.sum()) * np.eye(6),
                       atol=1e-15)
    assert np.all(r["S"] == 0)


def test_orthonormal_keys_undecayed():
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    k = Q.T[:5]                         # 5 orthonormal keys in R^8
    v = rng.standard_normal((5, 3))
    r = O.dense_recurrence(k, v, np.zeros(5), np.ones(5))
    assert np.allclose(O.T_value("dense", r["T_hat"], r["T_exp"]), np.eye(8) - k.T @ k, atol=1e-14)
    assert np.allclose(r["S"], k.T @ v, atol=1e-14)


def test_householder_orthogonal():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((30, 7))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    r = O.dense_recurrence(k, np.zeros((30, 2)), np.zeros(30), 2.0 * np.ones(30))
    T = O.T_value("dense", r["T_hat"], r["T_exp"])
    assert np.allclose(T.T @ T, np.eye(7), atol=1e-13)
    assert not np.allclose(T, np.eye(7))


def test_empty_segment_identity():
    r = O.dense_recurrence(np.zeros((0, 4)), np.zeros((0, 3)), np.zeros(0), np.zeros(0))
    assert np.array_equal(O.T_value("dense", r["T_hat"], r["T_exp"]), np.eye(4))
    assert np.all(r["S"] == 0)
    for kind, fn in (("diag", O.diag_recurrence), ("scalar", O.scalar_recurrence)):
        la = np.zeros((0, 4)) if kind == "diag" else np.zeros(0)
        r = fn(np.zeros((0, 4)), np.zeros((0, 3)), la)
        assert np.all(O.T_value(kind, r["T_hat"], r["T_exp"]) == 1) and np.all(r["S"] == 0)


def test_renormalised_T_never_underflows():
    # 8192 tokens of fast decay: T ~ exp(-0.5 * 8192) is far below float64's range
    n = 8192
    rng = np.random.default_rng(5)
    la = -0.5 * np.ones(n)
    r = O.dense_recurrence(rng.standard_normal((n, 2)), np.zeros((n, 1)), la, np.zeros(n))
    assert 0.5 <= np.abs(r["T_hat"]).max() < 1.0
    log_T = np.log(np.abs(r["T_hat"][0, 0])) + r["T_exp"] * np.log(2.0)
    assert abs(log_T - la.sum()) < 1e-9


def test_batched_chains_match_single():
    rng = np.random.default_rng(6)
    ks, vs, las, bs = [], [], [], []
    for _ in range(3):
        k, v, la, b, _ = _rand_chain(rng, 20, 4, 3)
        ks.append(k); vs.append(v); las.append(la); bs.append(b)
    rb = O.dense_recurrence(np.stack(ks), np.stack(vs), np.stack(las), np.stack(bs))
    for i in range(3):
        r = O.dense_recurrence(ks[i], vs[i], las[i], bs[i])
        assert np.array_equal(rb["S"][i], r["S"])
        assert np.array_equal(rb["T_hat"][i], r["T_hat"]) and rb["T_exp"][i] == r["T_exp"]


# ----------------------------------------------------------------------------------------
# composition


def _segment(k, v, la, b, lo, hi):
    return _as_el(O.dense_recurrence(k[lo:hi], v[lo:hi], la[lo:hi], b[lo:hi], renorm_every=3))


def test_every_segmentation_matches_sequential():
    rng = np.random.default_rng(7)
    n = 7
    k, v, la, b, _ = _rand_chain(rng, n, 3, 2)
    full = O.dense_recurrence(k, v, la, b)
    Tfull = O.T_value("dense", full["T_hat"], full["T_exp"])
    for mask in range(2 ** (n - 1)):
        cuts = [0] + [i + 1 for i in range(n - 1) if mask >> i & 1] + [n]
        els = [_segment(k, v, la, b, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
        f = O.compose_fold("dense", els)
        assert np.allclose(f["S_final"], full["S"], rtol=0, atol=1e-13)
        assert np.allclose(O.T_value("dense", f["T_hat"], f["T_exp"]), Tfull, rtol=0, atol=1e-14)
        # the state entering each element is the sequential state at that cut
        for i, lo in enumerate(cuts[:-1]):
            _, Sref = _brute(k[:lo], v[:lo], la[:lo], b[:lo]) if lo else (None, np.zeros((3, 2)))
            assert np.allclose(f["S_prefix"][i], Sref, rtol=0, atol=1e-13)


def test_random_splits_long_with_initial_state():
    rng = np.random.default_rng(8)
    n, d = 500, 16
    k, v, la, b, _ = _rand_chain(rng, n, d, d, unit=True)
    S0 = rng.standard_normal((d, d))
    full = O.dense_recurrence(k, v, la * 0.1, b, S0=S0)
    for _ in range(5):
        cuts = [0] + sorted(rng.choice(np.arange(1, n), 6, replace=False).tolist()) + [n]
        els = [_segment(k, v, la * 0.1, b, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
        f = O.compose_fold("dense", els, S0=S0)
        assert np.max(O.rel_err(f["S_final"], full["S"])) < 1e-12
        assert np.max(O.rel_err_T("dense", f["T_hat"], f["T_exp"], full["T_hat"], full["T_exp"])) < 1e-12


@pytest.mark.parametrize("kind", ["dense", "diag", "scalar"])
def test_associativity(kind):
    rng = np.random.default_rng(9)
    d = 5
    els = []
    for _ in range(3):
        if kind == "dense":
            Th = rng.standard_normal((d, d))
        elif kind == "diag":
            Th = rng.standard_normal(d)
        else:
            Th = np.array(rng.standard_normal())
        els.append({"T_hat": Th, "T_exp": np.array(int(rng.integers(-40, 3))),
                    "S": rng.standard_normal((d, 4))})
    a, b, c = els
    left = O.affine_compose(kind, O.affine_compose(kind, a, b), c)
    right = O.affine_compose(kind, a, O.affine_compose(kind, b, c))
    assert np.max(O.rel_err(left["S"], right["S"])) < 1e-13
    assert np.max(O.rel_err_T(kind, left["T_hat"], left["T_exp"], right["T_hat"], right["T_exp"])) < 1e-13
    # identity element (I, 0): composing with it changes nothing
    ident = {"T_hat": np.eye(d) if kind == "dense" else (np.ones(d) if kind == "diag" else np.array(1.0)),
             "T_exp": np.array(0), "S": np.zeros((d, 4))}
    for x in (O.affine_compose(kind, ident, a), O.affine_compose(kind, a, ident)):
        assert np.max(O.rel_err(x["S"], a["S"])) < 1e-15
        assert np.max(O.rel_err_T(kind, x["T_hat"], x["T_exp"], a["T_hat"], a["T_exp"])) < 1e-15


def test_compose_order_matters():
    # the law is T(C2) S(C1) + S(C2): swapping the operands must change the result
    rng = np.random.default_rng(10)
    k, v, la, b, _ = _rand_chain(rng, 12, 4, 4)
    a, c = _segment(k, v, la, b, 0, 6), _segment(k, v, la, b, 6, 12)
    ac = O.affine_compose("dense", a, c)
    ca = O.affine_compose("dense", c, a)
    full = O.dense_recurrence(k, v, la, b)
    assert np.max(O.rel_err(ac["S"], full["S"])) < 1e-13
    assert np.max(O.rel_err(ca["S"], full["S"])) > 1e-3


# ----------------------------------------------------------------------------------------
# naive addition


def test_naive_addition_exact_without_decay():
    rng = np.random.default_rng(11)
    k, v = rng.standard_normal((40, 6)), rng.standard_normal((40, 5))
    els = [_as_el(O.scalar_recurrence(k[i:i + 10], v[i:i + 10], np.zeros(10))) for i in range(0, 40, 10)]
    full = O.scalar_recurrence(k, v, np.zeros(40))
    assert np.max(np.abs(O.naive_add(els) - full["S"])) < 1e-13
    assert np.max(np.abs(O.compose_fold("scalar", els)["S_final"] - full["S"])) < 1e-13


def test_naive_addition_scalar_decay_closed_form():
    # one step: naive - true = (1 - gamma**n2) S(C1), exactly
    rng = np.random.default_rng(12)
    g = 1 - 2.0 ** -7
    n1, n2 = 50, 37
    k, v = rng.standard_normal((n1 + n2, 4)), rng.standard_normal((n1 + n2, 3))
    la = np.full(n1 + n2, np.log(g))
    c1 = _as_el(O.scalar_recurrence(k[:n1], v[:n1], la[:n1]))
    c2 = _as_el(O.scalar_recurrence(k[n1:], v[n1:], la[n1:]))
    true = O.compose_fold("scalar", [c1, c2])["S_final"]
    assert np.max(O.rel_err(true, O.scalar_recurrence(k, v, la)["S"])) < 1e-13
    naive = O.naive_add([c1, c2])
    assert np.allclose(naive - true, (1 - g ** n2) * c1["S"], rtol=0, atol=1e-12)


def test_naive_addition_22_percent_golden():
    with open(os.path.join(GOLDEN, "naive_addition_retnet.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    gap, n2, printed, rounding = int(rows[0][0]), int(rows[0][1]), float(rows[0][2]), float(rows[0][3])
    g = 1 - 2.0 ** -gap
    rng = np.random.default_rng(13)
    n1 = 256
    k = rng.standard_normal((n1 + n2, 32))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n1 + n2, 32))
    la = np.full(n1 + n2, np.log(g))
    c1 = _as_el(O.scalar_recurrence(k[:n1], v[:n1], la[:n1]))
    c2 = _as_el(O.scalar_recurrence(k[n1:], v[n1:], la[n1:]))
    true = O.compose_fold("scalar", [c1, c2])["S_final"]
    err = np.linalg.norm(O.naive_add([c1, c2]) - true) / np.linalg.norm(c1["S"])
    assert abs(err - printed) <= rounding          # the pages' ~22%
    assert abs(err - (1 - g ** n2)) < 1e-12        # and the exact closed form


def test_naive_addition_fails_under_gated_delta():
    rng = np.random.default_rng(14)
    k, v, _, b, _ = _rand_chain(rng, 512, 16, 16, unit=True)
    la = -0.05 * np.logaddexp(0, rng.standard_normal(512))
    els = [_segment(k, v, la, b, i, i + 128) for i in range(0, 512, 128)]
    full = O.dense_recurrence(k, v, la, b)["S"]
    assert np.max(O.rel_err(O.compose_fold("dense", els)["S_final"], full)) < 1e-12
    assert np.linalg.norm(O.naive_add(els) - full) / np.linalg.norm(full) > 0.3


# ----------------------------------------------------------------------------------------
# diagonal and scalar families: closed forms


def test_diag_closed_form():
    rng = np.random.default_rng(15)
    n, dk, dv = 90, 6, 4
    k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
    la = -0.2 * rng.random((n, dk))
    r = O.diag_recurrence(k, v, la)
    G = np.cumsum(la, axis=0)
    S = sum(np.exp(G[-1] - G[t])[:, None] * np.outer(k[t], v[t]) for t in range(n))
    assert np.allclose(O.T_value("diag", r["T_hat"], r["T_exp"]), np.exp(G[-1]), rtol=1e-13, atol=0)
    assert np.max(O.rel_err(r["S"], S)) < 1e-13


@pytest.mark.parametrize("kind", ["diag", "scalar"])
def test_diag_scalar_compose_equals_whole_chain(kind):
    # Composition law (HYPIC news article, linear-layer paragraph) for the decaying families,
    # with gates strong enough that every segment's T_hat carries an exponent <= -3: a sign or
    # index slip in how apply_T / compose_T use the exponent changes S and T by powers of two.
    rng = np.random.default_rng(31)
    n, dk, dv = 240, 6, 4
    k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
    if kind == "diag":
        la = -0.08 - 0.1 * rng.random((n, dk))
        rec = lambda lo, hi: O.diag_recurrence(k[lo:hi], v[lo:hi], la[lo:hi], renorm_every=7)
    else:
        la = np.log(0.9) * (1.0 + 0.5 * rng.random(n))
        rec = lambda lo, hi: O.scalar_recurrence(k[lo:hi], v[lo:hi], la[lo:hi], renorm_every=7)
    # G[t] = sum of log alpha over tokens 0..t-1, per channel (scalar: the same for all)
    G = np.zeros((n + 1, dk))
    G[1:] = np.cumsum(la if kind == "diag" else la[:, None] * np.ones(dk), axis=0)
    S0 = rng.standard_normal((dk, dv))

    def closed(hi):
        """State after tokens [0, hi) from S0: e^{G_hi} S0 + sum_t e^{G_hi - G_{t+1}} k_t v_t^T."""
        S = np.exp(G[hi])[:, None] * S0
        for t in range(hi):
            S = S + np.exp(G[hi] - G[t + 1])[:, None] * np.outer(k[t], v[t])
        return S

    cuts = [0, 37, 90, 130, 160, 240]
    els = [_as_el(rec(lo, hi)) for lo, hi in zip(cuts[:-1], cuts[1:])]
    assert all(int(e["T_exp"]) <= -3 for e in els)
    f = O.compose_fold(kind, els, S0=S0)
    assert np.max(O.rel_err(f["S_final"], closed(n))) < 1e-12
    Tf = O.T_value(kind, f["T_hat"], f["T_exp"])
    Tn = np.exp(G[n]) if kind == "diag" else np.exp(G[n, 0])
    assert np.max(np.abs(Tf - Tn)) < 1e-12 * np.max(np.abs(Tn))
    for i, lo in enumerate(cuts[:-1]):          # the state entering each element
        assert np.max(O.rel_err(f["S_prefix"][i], closed(lo))) < 1e-12
    # pairwise affine_compose in a tree gives the same element as the whole chain
    ab = O.affine_compose(kind, els[0], els[1])
    cde = O.affine_compose(kind, O.affine_compose(kind, els[2], els[3]), els[4])
    tot = O.affine_compose(kind, ab, cde)
    whole = rec(0, n)
    assert np.max(O.rel_err(tot["S"], whole["S"])) < 1e-12
    assert np.max(O.rel_err_T(kind, tot["T_hat"], tot["T_exp"], whole["T_hat"], whole["T_exp"])) < 1e-12
    assert np.max(O.rel_err(O.apply_T(kind, tot["T_hat"], tot["T_exp"], S0) + tot["S"], closed(n))) < 1e-12


def test_scalar_closed_form_and_diag_agreement():
    rng = np.random.default_rng(16)
    n, dk, dv, g = 70, 5, 3, 0.97
    k, v = rng.standard_normal((n, dk)), rng.standard_normal((n, dv))
    r = O.scalar_recurrence(k, v, np.full(n, np.log(g)))
    S = sum(g ** (n - 1 - t) * np.outer(k[t], v[t]) for t in range(n))
    assert abs(O.T_value("scalar", r["T_hat"], r["T_exp"]) - g ** n) < 1e-14
    assert np.max(O.rel_err(r["S"], S)) < 1e-13
    rd = O.diag_recurrence(k, v, np.full((n, dk), np.log(g)))
    assert np.max(O.rel_err(rd["S"], r["S"])) < 1e-14


# ----------------------------------------------------------------------------------------
# seam window


def test_seam_outputs_and_state():
    rng = np.random.default_rng(17)
    w, d = 8, 4
    k, v, la, b, q = _rand_chain(rng, w, d, 3, unit=True)
    S_in = rng.standard_normal((d, 3))
    r = O.seam_advance(q, k, v, la, b, S_in)
    T, S = _brute(k, v, la, b, S_in)
    assert np.allclose(r["S_out"], S, atol=1e-13)
    for t in range(w):
        _, St = _brute(k[:t + 1], v[:t + 1], la[:t + 1], b[:t + 1], S_in)
        assert np.allclose(r["o"][t], St.T @ q[t], atol=1e-13)
    # the seam's own pair composes with S_in to S_out
    own = O.apply_T("dense", r["T_hat"], r["T_exp"], S_in) + r["S_seam"]
    assert np.allclose(own, r["S_out"], atol=1e-13)


# ----------------------------------------------------------------------------------------
# depthwise causal convolution


def _conv_brute(x, w, state):
    n, C = x.shape
    W = w.shape[1]
    y = np.zeros((n, C))
    for t in range(n):
        for c in range(C):
            for j in range(W):
                src = t - (W - 1) + j          # absolute position of the tap
                val = x[src, c] if src >= 0 else (state[W - 1 + src, c] if state is not None else 0.0)
                y[t, c] += w[c, j] * val
    return y


def test_conv_definition_and_special_taps():
    rng = np.random.default_rng(18)
    x, st = rng.standard_normal((9, 5)), rng.standard_normal((3, 5))
    w = rng.standard_normal((5, 4))
    y, so = O.causal_conv(x, w, state=st)
    assert np.allclose(y, _conv_brute(x, w, st), atol=1e-14)
    assert np.array_equal(so, x[-3:])
    ident = np.zeros((5, 4)); ident[:, 3] = 1
    assert np.array_equal(O.causal_conv(x, ident, state=st)[0], x)
    shift = np.zeros((5, 4)); shift[:, 0] = 1
    assert np.array_equal(O.causal_conv(x, shift, state=st)[0], np.concatenate([st, x])[:9])
    # short input: the carried state keeps the older rows
    y2, so2 = O.causal_conv(x[:2], w, state=st)
    assert np.array_equal(so2, np.concatenate([st, x[:2]])[-3:])
    # bias and SiLU
    bias = rng.standard_normal(5)
    ys, _ = O.causal_conv(x, w, bias=bias, state=st, activation="silu")
    z = _conv_brute(x, w, st) + bias
    assert np.allclose(ys, z * (1 / (1 + np.exp(-z))), atol=1e-14)


def test_conv_carry_invariant():
    rng = np.random.default_rng(19)
    x, w = rng.standard_normal((50, 7)), rng.standard_normal((7, 4))
    whole, _ = O.causal_conv(x, w)
    st, parts = None, []
    for lo, hi in ((0, 2), (2, 20), (20, 21), (21, 50)):
        y, st = O.causal_conv(x[lo:hi], w, state=st)
        parts.append(y)
    assert np.array_equal(np.concatenate(parts), whole)


def test_warm_chain_reference_matches_whole_prompt():
    rng = np.random.default_rng(20)
    lens = [13, 9, 20]
    N, d = sum(lens), 4
    xq, xk, xv = (rng.standard_normal((N, d)) for _ in range(3))
    wq, wk, wv = (rng.standard_normal((d, 4)) for _ in range(3))
    b, la = rng.random(N), -0.1 * rng.random(N)
    r = O.warm_chain_reference(xq, xk, xv, wq, wk, wv, b, la, lens, seam=8)
    q = _conv_brute(xq, wq, None); k = _conv_brute(xk, wk, None); v = _conv_brute(xv, wv, None)
    q /= np.linalg.norm(q, axis=1, keepdims=True); k /= np.linalg.norm(k, axis=1, keepdims=True)
    _, Sfin = _brute(k, v, la, b)
    assert np.allclose(r["S_final"], Sfin, atol=1e-12)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for i, s0 in enumerate(starts):
        _, Ss = _brute(k[:s0], v[:s0], la[:s0], b[:s0]) if s0 else (None, np.zeros((d, d)))
        assert np.allclose(r["S_start"][i], Ss, atol=1e-12)
        for t in range(8):
            _, St = _brute(k[:s0 + t + 1], v[:s0 + t + 1], la[:s0 + t + 1], b[:s0 + t + 1])
            assert np.allclose(r["o_seam"][i][t], St.T @ q[s0 + t], atol=1e-12)


# ----------------------------------------------------------------------------------------
# schedules


def test_lpt_graham_bound_vs_bruteforce():
    rng = np.random.default_rng(21)
    for _ in range(60):
        m = int(rng.integers(2, 5))
        w = rng.integers(1, 20, size=int(rng.integers(m, 10))).tolist()
        _, assign, mk = O.lpt_schedule(w, m)
        loads = np.bincount(assign, weights=w, minlength=m)
        assert loads.max() == mk and loads.sum() == sum(w)
        opt = O.opt_makespan_bruteforce(w, m)
        assert opt <= mk <= (4 / 3 - 1 / (3 * m)) * opt + 1e-9


def test_lpt_tight_example_and_rr():
    # Graham's tight instance for m = 2: LPT gives 7, the optimum is 6
    order, assign, mk = O.lpt_schedule([3, 3, 2, 2, 2], 2)
    assert order == [0, 1, 2, 3, 4] and mk == 7
    assert O.opt_makespan_bruteforce([3, 3, 2, 2, 2], 2) == 6
    a, mk_rr = O.rr_schedule([5, 1, 5, 1], 2)
    assert a == [0, 1, 0, 1] and mk_rr == 10
    assert O.lpt_schedule([5, 1, 5, 1], 2)[2] == 6


# ----------------------------------------------------------------------------------------
# error metric


def test_error_metric_conventions():
    ref = np.zeros((2, 3, 3)); ref[0] = 1
    x = ref.copy()
    assert np.all(O.rel_err(x, ref) == 0)
    x[1, 0, 0] = 1e-30
    assert np.isinf(O.rel_err(x, ref)[1])
    Th = np.eye(3) * 0.5
    assert O.rel_err_T("dense", Th * 2, np.array(4), Th, np.array(5)) == 0
    assert abs(O.rel_err_T("dense", Th * 1.001, np.array(5), Th, np.array(5)) - 1e-3) < 1e-12


# ----------------------------------------------------------------------------------------
# RoPE state re-rotation (HYPIC news article, linear-layer paragraph; README, "PIC modes",
# transition_rope): a segment cached with keys rotated at positions p + t and reused at
# p + delta + t


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("kind", ["dense", "scalar"])
def test_rerotation_equals_recomputation_at_the_new_offset(kind, interleaved):
    # pinned against recomputing the recurrence on keys rotated at the new positions
    rng = np.random.default_rng(41)
    n, d, rd, base, p0, delta = 50, 8, 6, 100.0, 1000, -377
    k, v, la, b, _ = _rand_chain(rng, n, d, 3, unit=True)
    pos = p0 + np.arange(n)
    k0 = O.rope_rotate(k, pos, rd, base, interleaved)
    k1 = O.rope_rotate(k, pos + delta, rd, base, interleaved)
    if kind == "dense":
        r0 = O.dense_recurrence(k0, v, la, b)
        r1 = O.dense_recurrence(k1, v, la, b)
    else:
        r0 = O.scalar_recurrence(k0, v, la)
        r1 = O.scalar_recurrence(k1, v, la)
    m = O.rerotate(kind, r0["T_hat"], r0["T_exp"], r0["S"], delta, rd, base, interleaved)
    assert np.max(O.rel_err(m["S"], r1["S"])) < 1e-12
    assert np.max(O.rel_err_T(kind, m["T_hat"], m["T_exp"], r1["T_hat"], r1["T_exp"])) < 1e-12
    # without the correction the cached state is wrong at the new offset
    assert np.max(O.rel_err(r0["S"], r1["S"])) > 1e-2


def test_rope_rotation_closed_form_and_group_laws():
    # base 1, rotary_dim 4: every pair turns by exactly delta radians; a quarter turn maps
    # (x_a, x_b) to (-x_b, x_a) on each pair and leaves channels 4, 5 alone
    x = np.arange(1.0, 7.0)
    for inter, pairs in ((True, [(0, 1), (2, 3)]), (False, [(0, 2), (1, 3)])):
        y = O.rope_rotate(x[None], [np.pi / 2], 4, 1.0, inter)[0]
        want = x.copy()
        for a, b in pairs:
            want[a], want[b] = -x[b], x[a]
        assert np.allclose(y, want, atol=1e-15)
    R = lambda t: O.rope_matrix(10, t, 8, 500.0, False)
    assert np.allclose(R(0.0), np.eye(10))
    assert np.allclose(R(3.0) @ R(-11.0), R(-8.0), atol=1e-14)             # R(a) R(b) = R(a + b)
    assert np.allclose(R(7.5).T @ R(7.5), np.eye(10), atol=1e-14)          # orthogonal
    # the matrix and the row rotation agree (both used by the re-rotation pin above)
    rng = np.random.default_rng(43)
    z = rng.standard_normal((5, 10))
    assert np.allclose(O.rope_rotate(z, [12.0] * 5, 8, 500.0, True), z @ O.rope_matrix(10, 12.0, 8, 500.0, True).T)


def test_rope_outputs_are_relative():
    # rotating q and k by the same shift leaves every output o_t = S_t^T q_t unchanged: the
    # re-rotated state is what the shifted queries read
    rng = np.random.default_rng(44)
    n, d, rd = 30, 8, 8
    k, v, la, b, q = _rand_chain(rng, n, d, 4, unit=True)
    a = O.dense_recurrence(O.rope_rotate(k, np.arange(n), rd, 50.0, False), v, la, b,
                           q=O.rope_rotate(q, np.arange(n), rd, 50.0, False))
    c = O.dense_recurrence(O.rope_rotate(k, np.arange(n) + 999, rd, 50.0, False), v, la, b,
                           q=O.rope_rotate(q, np.arange(n) + 999, rd, 50.0, False))
    assert np.max(np.abs(a["o"] - c["o"])) < 1e-12
    m = O.rerotate("dense", a["T_hat"], a["T_exp"], a["S"], 999, rd, 50.0, False)
    assert np.max(O.rel_err(m["S"], c["S"])) < 1e-12


def test_rerotation_rejects_per_channel_gates():
    with pytest.raises(ValueError):
        O.rerotate("diag", np.ones(4), 0, np.zeros((4, 4)), 3, 4, 10.0, False)


# ----------------------------------------------------------------------------------------
# per-channel gated delta rule (KDA, named in the HYPIC news article's linear-layer paragraph):
# A_t = diag(alpha_t) (I - beta_t k_t k_t^T)


def _kda_brute(k, v, la, b, S0):
    n, dk = k.shape
    As = [np.diag(np.exp(la[t])) @ (np.eye(dk) - b[t] * np.outer(k[t], k[t])) for t in range(n)]
    T = np.eye(dk)
    for A in As:
        T = A @ T
    S = T @ S0
    for t in range(n):
        P = np.eye(dk)
        for A in As[t + 1:]:
            P = A @ P
        S = S + P @ (b[t] * np.outer(k[t], v[t]))
    return T, S


@pytest.mark.parametrize("dk,dv,n", [(1, 1, 3), (3, 2, 5), (4, 4, 6)])
def test_kda_brute_force(dk, dv, n):
    rng = np.random.default_rng(60 + dk + n)
    k, v, _, b, q = _rand_chain(rng, n, dk, dv)
    la = -0.4 * rng.random((n, dk))
    S0 = rng.standard_normal((dk, dv))
    r = O.kda_recurrence(k, v, la, b, S0=S0, q=q, renorm_every=2)
    T, S = _kda_brute(k, v, la, b, S0)
    assert np.allclose(O.T_value("dense", r["T_hat"], r["T_exp"]), T, rtol=0, atol=1e-14)
    assert np.allclose(r["S"], S, rtol=0, atol=1e-13)
    for t in range(n):
        _, St = _kda_brute(k[:t + 1], v[:t + 1], la[:t + 1], b[:t + 1], S0)
        assert np.allclose(r["o"][t], St.T @ q[t], rtol=0, atol=1e-13)


def test_kda_reductions():
    rng = np.random.default_rng(62)
    n, d = 90, 6
    k, v, la, b, q = _rand_chain(rng, n, d, 4, unit=True)
    # channel-uniform gates: the gated delta rule
    ku = O.kda_recurrence(k, v, np.repeat(la[:, None], d, 1), b, q=q)
    g = O.dense_recurrence(k, v, la, b, q=q)
    assert np.max(O.rel_err(ku["S"], g["S"])) < 1e-13
    assert np.max(O.rel_err_T("dense", ku["T_hat"], ku["T_exp"], g["T_hat"], g["T_exp"])) < 1e-13
    assert np.max(np.abs(ku["o"] - g["o"])) < 1e-12
    # no writes (beta = 0): pure per-channel decay, T = diag(e^{sum log alpha}), S = T S0
    lad = -0.2 * rng.random((n, d))
    S0 = rng.standard_normal((d, 4))
    z = O.kda_recurrence(k, v, lad, np.zeros(n), S0=S0)
    Tz = O.T_value("dense", z["T_hat"], z["T_exp"])
    assert np.allclose(Tz, np.diag(np.exp(lad.sum(0))), rtol=1e-12, atol=0)
    assert np.max(O.rel_err(z["S"], np.exp(lad.sum(0))[:, None] * S0)) < 1e-13


def test_kda_segments_compose_with_the_dense_law():
    rng = np.random.default_rng(63)
    n, d = 300, 8
    k, v, _, b, _ = _rand_chain(rng, n, d, 5, unit=True)
    la = -0.05 - 0.2 * rng.random((n, d))
    S0 = rng.standard_normal((d, 5))
    full = O.kda_recurrence(k, v, la, b, S0=S0)
    cuts = [0, 41, 42, 170, 300]
    els = [_as_el(O.kda_recurrence(k[a:c], v[a:c], la[a:c], b[a:c], renorm_every=5)) for a, c in zip(cuts[:-1], cuts[1:])]
    f = O.compose_fold("dense", els, S0=S0)
    assert np.max(O.rel_err(f["S_final"], full["S"])) < 1e-12
    assert np.max(O.rel_err_T("dense", f["T_hat"], f["T_exp"], full["T_hat"], full["T_exp"])) < 1e-12
