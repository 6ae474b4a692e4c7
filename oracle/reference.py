"""Plain fp64 token-by-token reference of the state-composition path.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests/, the
smoke check and the benchmark's CPU-baseline leg, never by the device path.

Conventions (readings of the HYPIC pages, each pinned in tests/test_oracle.py):
  * state S is d_k x d_v, a transition T is d_k x d_k and acts from the left,
    as in the composition law S(C1.C2) = T(C2) S(C1) + S(C2) of the HYPIC news
    article's linear-layer paragraph; per-token output o_t = S_t^T q_t;
  * dense (gated delta rule): S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T, the write not decayed at its own step;
  * diagonal (GLA): S_t = diag(alpha_t) S_{t-1} + k_t v_t^T;
    scalar (RetNet, Mamba2): S_t = alpha_t S_{t-1} + k_t v_t^T;
  * T is carried as T_hat * 2**T_exp (int exponent per chain), rescaled by an
    exact power of two every 64 tokens so that long, fast-decaying segments
    never underflow.  The pair is not unique; only its value is meaningful.
Leading dimensions of every array are independent chains (batch).
"""

from __future__ import annotations

import numpy as np

_TDIMS = {"dense": 2, "diag": 1, "scalar": 0}


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _renorm(T_hat, T_exp, nd):
    """Rescale each chain's T_hat by 2**-e so that max|T_hat| is in [0.5, 1)."""
    if nd:
        m = np.max(np.abs(T_hat), axis=tuple(range(T_hat.ndim - nd, T_hat.ndim)))
    else:
        m = np.abs(T_hat)
    _, e = np.frexp(m)
    e = np.where(m > 0, e, 0).astype(np.int64)
    T_hat = np.ldexp(T_hat, -e.reshape(e.shape + (1,) * nd))
    return T_hat, np.asarray(T_exp, np.int64) + e


def T_value(kind, T_hat, T_exp):
    """The represented transition T_hat * 2**T_exp in float64 (may underflow)."""
    nd = _TDIMS[kind]
    e = np.asarray(T_exp, np.int64)
    return np.ldexp(_f64(T_hat), e.reshape(e.shape + (1,) * nd))


def apply_T(kind, T_hat, T_exp, X):
    """T X for a d_k x d_v (or d_k x d_k) matrix X, in float64."""
    X = _f64(X)
    e = np.asarray(T_exp, np.int64)[..., None, None]
    T_hat = _f64(T_hat)
    if kind == "dense":
        return np.ldexp(T_hat @ X, e)
    if kind == "diag":
        return np.ldexp(T_hat[..., :, None] * X, e)
    if kind == "scalar":
        return np.ldexp(T_hat[..., None, None] * X, e)
    raise ValueError(kind)


def compose_T(kind, second, first):
    """(T2 T1) for transitions given as (T_hat, T_exp) pairs, renormalised."""
    (h2, e2), (h1, e1) = second, first
    h2, h1 = _f64(h2), _f64(h1)
    if kind == "dense":
        h = h2 @ h1
    else:
        h = h2 * h1
    return _renorm(h, np.asarray(e2, np.int64) + np.asarray(e1, np.int64), _TDIMS[kind])


# ----------------------------------------------------------------------------------------
# token recurrences


def dense_recurrence(k, v, log_alpha, beta, S0=None, q=None, renorm_every=64):
    """Gated delta rule over n tokens, starting from (T, S) = (I, S0).

    k [..., n, d_k], v [..., n, d_v], log_alpha [..., n], beta [..., n],
    S0 [..., d_k, d_v] or None (zero), q [..., n, d_k] or None.
    Returns T_hat [..., d_k, d_k], T_exp [...], S [..., d_k, d_v] and, with q,
    o [..., n, d_v] where o_t = S_t^T q_t uses the state after token t.
    """
    k, v, la, b = _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    batch = k.shape[:-2]
    n, dk = k.shape[-2:]
    dv = v.shape[-1]
    S = np.zeros(batch + (dk, dv)) if S0 is None else np.array(_f64(S0), copy=True)
    T = np.array(np.broadcast_to(np.eye(dk), batch + (dk, dk)), copy=True)
    e = np.zeros(batch, np.int64)
    o = np.zeros(batch + (n, dv)) if q is not None else None
    qf = _f64(q) if q is not None else None
    for t in range(n):
        a = np.exp(la[..., t])[..., None, None]
        bt = b[..., t][..., None, None]
        kt = k[..., t, :]
        kcol = kt[..., :, None]
        kS = (kt[..., None, :] @ S)                      # k^T S      [..., 1, d_v]
        S = a * (S - bt * (kcol @ kS)) + bt * (kcol @ v[..., t, None, :])
        kT = (kt[..., None, :] @ T)                      # k^T T      [..., 1, d_k]
        T = a * (T - bt * (kcol @ kT))
        if qf is not None:
            o[..., t, :] = (qf[..., t, None, :] @ S)[..., 0, :]   # (S^T q)^T = q^T S
        if (t + 1) % renorm_every == 0:
            T, e = _renorm(T, e, 2)
    T, e = _renorm(T, e, 2)
    return {"T_hat": T, "T_exp": e, "S": S, "o": o}


def kda_recurrence(k, v, log_alpha, beta, S0=None, q=None, renorm_every=64):
    """Per-channel gated delta rule (KDA-style): A_t = diag(alpha_t) (I - beta_t k_t k_t^T),
    S_t = A_t S_{t-1} + beta_t k_t v_t^T, the write not decayed at its own step.

    k [..., n, d_k], v [..., n, d_v], log_alpha [..., n, d_k] (per channel), beta [..., n].
    T is a dense d_k x d_k matrix, carried as (T_hat, T_exp) like the gated delta rule's,
    so cached KDA segments compose with the dense composition law.  With q, o_t = S_t^T q_t.
    """
    k, v, la, b = _f64(k), _f64(v), _f64(log_alpha), _f64(beta)
    batch = k.shape[:-2]
    n, dk = k.shape[-2:]
    dv = v.shape[-1]
    S = np.zeros(batch + (dk, dv)) if S0 is None else np.array(_f64(S0), copy=True)
    T = np.array(np.broadcast_to(np.eye(dk), batch + (dk, dk)), copy=True)
    e = np.zeros(batch, np.int64)
    o = np.zeros(batch + (n, dv)) if q is not None else None
    qf = _f64(q) if q is not None else None
    for t in range(n):
        a = np.exp(la[..., t, :])[..., :, None]          # per-channel decay, rows
        bt = b[..., t][..., None, None]
        kt = k[..., t, :]
        kcol = kt[..., :, None]
        kS = kt[..., None, :] @ S
        S = a * (S - bt * (kcol @ kS)) + bt * (kcol @ v[..., t, None, :])
        kT = kt[..., None, :] @ T
        T = a * (T - bt * (kcol @ kT))
        if qf is not None:
            o[..., t, :] = (qf[..., t, None, :] @ S)[..., 0, :]
        if (t + 1) % renorm_every == 0:
            T, e = _renorm(T, e, 2)
    T, e = _renorm(T, e, 2)
    return {"T_hat": T, "T_exp": e, "S": S, "o": o}


def diag_recurrence(k, v, log_alpha, S0=None, q=None, renorm_every=64):
    """GLA per-channel decay: S_t = diag(alpha_t) S_{t-1} + k_t v_t^T.

    log_alpha [..., n, d_k].  T is diagonal and returned as its diagonal
    T_hat [..., d_k] with exponent T_exp [...].
    """
    k, v, la = _f64(k), _f64(v), _f64(log_alpha)
    batch = k.shape[:-2]
    n, dk = k.shape[-2:]
    dv = v.shape[-1]
    S = np.zeros(batch + (dk, dv)) if S0 is None else np.array(_f64(S0), copy=True)
    T = np.ones(batch + (dk,))
    e = np.zeros(batch, np.int64)
    o = np.zeros(batch + (n, dv)) if q is not None else None
    for t in range(n):
        a = np.exp(la[..., t, :])
        S = a[..., :, None] * S + k[..., t, :, None] * v[..., t, None, :]
        T = a * T
        if q is not None:
            o[..., t, :] = np.einsum("...ij,...i->...j", S, _f64(q)[..., t, :])
        if (t + 1) % renorm_every == 0:
            T, e = _renorm(T, e, 1)
    T, e = _renorm(T, e, 1)
    return {"T_hat": T, "T_exp": e, "S": S, "o": o}


def scalar_recurrence(k, v, log_alpha, S0=None, q=None, renorm_every=64):
    """Scalar decay (RetNet gamma, Mamba2): S_t = alpha_t S_{t-1} + k_t v_t^T.

    log_alpha [..., n].  T = (prod alpha_t) I, returned as the scalar
    T_hat [...] with exponent T_exp [...].
    """
    k, v, la = _f64(k), _f64(v), _f64(log_alpha)
    batch = k.shape[:-2]
    n, dk = k.shape[-2:]
    dv = v.shape[-1]
    S = np.zeros(batch + (dk, dv)) if S0 is None else np.array(_f64(S0), copy=True)
    T = np.ones(batch)
    e = np.zeros(batch, np.int64)
    o = np.zeros(batch + (n, dv)) if q is not None else None
    for t in range(n):
        a = np.exp(la[..., t])
        S = a[..., None, None] * S + k[..., t, :, None] * v[..., t, None, :]
        T = a * T
        if q is not None:
            o[..., t, :] = np.einsum("...ij,...i->...j", S, _f64(q)[..., t, :])
        if (t + 1) % renorm_every == 0:
            T, e = _renorm(T, e, 0)
    T, e = _renorm(T, e, 0)
    return {"T_hat": T, "T_exp": e, "S": S, "o": o}


# ----------------------------------------------------------------------------------------
# composition


def affine_compose(kind, first, second):
    """Segment C1 (``first``) followed by C2 (``second``).

    Each is a dict with T_hat, T_exp, S.  Returns (T2 T1, T2 S1 + S2), the
    composition law of the HYPIC news article's linear-layer paragraph.
    """
    T_hat, T_exp = compose_T(kind, (second["T_hat"], second["T_exp"]),
                             (first["T_hat"], first["T_exp"]))
    S = apply_T(kind, second["T_hat"], second["T_exp"], first["S"]) + _f64(second["S"])
    return {"T_hat": T_hat, "T_exp": T_exp, "S": S}


def compose_fold(kind, elements, S0=None):
    """Sequential fold S <- T_i S + S_i over ``elements`` in request order.

    Returns S_final, S_prefix (the state entering each element, stacked on a
    new leading axis) and the total transition T_n ... T_1 as T_hat/T_exp.
    """
    first = elements[0]
    S = np.zeros_like(_f64(first["S"])) if S0 is None else _f64(S0)
    nd = _TDIMS[kind]
    Th = np.ones_like(_f64(first["T_hat"]))
    if kind == "dense":
        Th = np.array(np.broadcast_to(np.eye(Th.shape[-1]), Th.shape), copy=True)
    Te = np.zeros(np.shape(first["T_exp"]), np.int64)
    Th, Te = _renorm(Th, Te, nd)
    prefix = []
    for el in elements:
        prefix.append(S)
        S = apply_T(kind, el["T_hat"], el["T_exp"], S) + _f64(el["S"])
        Th, Te = compose_T(kind, (el["T_hat"], el["T_exp"]), (Th, Te))
    return {"S_final": S, "S_prefix": np.stack(prefix), "T_hat": Th, "T_exp": Te}


def naive_add(elements, S0=None):
    """The straw-man composition: plain sum of zero-start end states."""
    S = np.zeros_like(_f64(elements[0]["S"])) if S0 is None else _f64(S0)
    for el in elements:
        S = S + _f64(el["S"])
    return S


# ----------------------------------------------------------------------------------------
# seam window and convolution warm-up


def seam_advance(q, k, v, log_alpha, beta, S_in=None):
    """Run the w seam tokens through the gated delta rule from S_in.

    Returns o [..., w, d_v] (o_t = S_t^T q_t), S_out, and the seam's own
    zero-start pair (T_hat, T_exp, S_seam), which composes with S_in to S_out.
    """
    run = dense_recurrence(k, v, log_alpha, beta, S0=S_in, q=q)
    own = dense_recurrence(k, v, log_alpha, beta)
    return {"o": run["o"], "S_out": run["S"], "T_hat": own["T_hat"],
            "T_exp": own["T_exp"], "S_seam": own["S"]}


def causal_conv(x, weight, bias=None, state=None, activation="none"):
    """Depthwise causal convolution (cross-correlation) with carried state.

    x [n, C]; weight [C, W] where tap W-1 multiplies the current token;
    state [W-1, C] holds the W-1 inputs before x (zero if None).
    y_t[c] = sum_j weight[c, j] * xx[t + j, c] with xx = state ++ x, plus bias,
    then SiLU if requested.  Returns y [n, C] and state_out = the last W-1 rows
    of xx (the state the next segment needs).
    """
    x, w = _f64(x), _f64(weight)
    n, C = x.shape
    W = w.shape[1]
    st = np.zeros((W - 1, C)) if state is None else _f64(state)
    xx = np.concatenate([st, x], axis=0)
    y = np.zeros((n, C))
    for t in range(n):
        acc = np.zeros(C)
        for j in range(W):
            acc = acc + w[:, j] * xx[t + j]
        y[t] = acc
    if bias is not None:
        y = y + _f64(bias)[None, :]
    if activation == "silu":
        y = y / (1.0 + np.exp(-y))
    elif activation != "none":
        raise ValueError(activation)
    return y, xx[n:].copy()


def l2_normalise(x):
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def warm_chain_reference(xq, xk, xv, wq, wk, wv, beta, log_alpha, seg_lens, seam,
                         activation="none"):
    """Whole-prompt reference for one chain of the warm hit path.

    Inputs are in request order: pre-conv activations xq, xk, xv [N, d],
    taps w* [d, W], beta, log_alpha [N].  The prompt is convolved as one
    sequence (zero initial conv state), q and k are L2-normalised per token,
    and the gated delta rule runs over all N tokens from S = 0.
    Returns S_start [n_seg, d_k, d_v] (state entering each segment),
    o_seam [n_seg, w, d_v] (outputs of each segment's first w tokens), S_final,
    and the post-conv q, k, v.
    """
    q, _ = causal_conv(xq, wq, activation=activation)
    k, _ = causal_conv(xk, wk, activation=activation)
    v, _ = causal_conv(xv, wv, activation=activation)
    q, k = l2_normalise(q), l2_normalise(k)
    starts = np.concatenate([[0], np.cumsum(seg_lens)[:-1]]).astype(np.int64)
    dk, dv = k.shape[1], v.shape[1]
    S = np.zeros((dk, dv))
    S_start, o_seam = [], []
    for s0, n in zip(starts, seg_lens):
        S_start.append(S)
        w = min(seam, n)
        head = dense_recurrence(k[s0:s0 + w], v[s0:s0 + w], log_alpha[s0:s0 + w],
                                beta[s0:s0 + w], S0=S, q=q[s0:s0 + w])
        o_seam.append(head["o"])
        rest = dense_recurrence(k[s0 + w:s0 + n], v[s0 + w:s0 + n], log_alpha[s0 + w:s0 + n],
                                beta[s0 + w:s0 + n], S0=head["S"])
        S = rest["S"]
    return {"S_start": np.stack(S_start), "o_seam": o_seam, "S_final": S,
            "q": q, "k": k, "v": v}


# ----------------------------------------------------------------------------------------
# RoPE state re-rotation (HYPIC news article, linear-layer paragraph: the alignment patch
# for variants that rotate q and k by absolute position; HYPIC project README, "PIC
# modes": the transition_rope mode corrects the positions of segments reused elsewhere)


def rope_pairs(d, rotary_dim, interleaved):
    """Channel pairs (a, b) rotated together and the frequency index of each.

    interleaved: pairs (2i, 2i+1); otherwise (i, i + rotary_dim/2), i < rotary_dim/2.
    Channels >= rotary_dim are not rotated."""
    h = rotary_dim // 2
    if interleaved:
        return [(2 * i, 2 * i + 1, i) for i in range(h)]
    return [(i, i + h, i) for i in range(h)]


def rope_matrix(d, delta, rotary_dim, base, interleaved):
    """The d x d rotation R(delta): on each pair (a, b) with frequency
    theta_i = base^(-2i / rotary_dim) it maps (x_a, x_b) to
    (x_a cos(delta theta_i) - x_b sin(delta theta_i), x_a sin(delta theta_i) + x_b cos(delta theta_i));
    identity on the other channels.  A key rotated at position p is R(p) k."""
    R = np.eye(d)
    for a, b, i in rope_pairs(d, rotary_dim, interleaved):
        ang = float(delta) * float(base) ** (-2.0 * i / rotary_dim)
        c, s_ = np.cos(ang), np.sin(ang)
        R[a, a], R[a, b], R[b, a], R[b, b] = c, -s_, s_, c
    return R


def rope_rotate(x, positions, rotary_dim, base, interleaved):
    """Rotate rows x[..., n, d] by R(positions[t]) each, channel pair by channel pair."""
    x = np.array(_f64(x), copy=True)
    pos = np.asarray(positions, np.float64)
    out = x.copy()
    for a, b, i in rope_pairs(x.shape[-1], rotary_dim, interleaved):
        ang = pos * float(base) ** (-2.0 * i / rotary_dim)
        c, s_ = np.cos(ang), np.sin(ang)
        out[..., a] = x[..., a] * c - x[..., b] * s_
        out[..., b] = x[..., a] * s_ + x[..., b] * c
    return out


def rerotate(kind, T_hat, T_exp, S, delta, rotary_dim, base, interleaved):
    """A cached element whose keys were rotated at positions p + t, moved to p + delta + t.

    Rotated keys R k give per-token transitions R A_t R^T and writes R k v^T, so the
    segment's transition becomes R T R^T and its state R S (R = R(delta)).  A scalar
    transition commutes with R and is unchanged.  Per-channel (diagonal) gates do not
    commute with R unless tied on every rotated pair; that kind is not handled."""
    if kind not in ("dense", "scalar"):
        raise ValueError(f"re-rotation is defined here for the dense and scalar kinds, not {kind}")
    d = np.shape(S)[-2]
    R = rope_matrix(d, delta, rotary_dim, base, interleaved)
    S2 = R @ _f64(S)
    if kind == "dense":
        return {"T_hat": R @ _f64(T_hat) @ R.T, "T_exp": np.asarray(T_exp), "S": S2}
    return {"T_hat": _f64(T_hat), "T_exp": np.asarray(T_exp), "S": S2}


# ----------------------------------------------------------------------------------------
# schedules (integer)


def lpt_schedule(weights, m):
    """Longest-processing-time-first list scheduling onto m workers.

    Tasks are taken in order of decreasing weight (ties: lower index first)
    and each goes to the currently least-loaded worker (ties: lower worker).
    Returns (order, assignment, makespan).
    """
    w = [int(x) for x in weights]
    order = sorted(range(len(w)), key=lambda i: (-w[i], i))
    loads = [0] * m
    assign = [0] * len(w)
    for i in order:
        g = min(range(m), key=lambda j: (loads[j], j))
        assign[i] = g
        loads[g] += w[i]
    return order, assign, max(loads) if w else 0


def rr_schedule(weights, m):
    """Round-robin: task i goes to worker i mod m.  Returns (assignment, makespan)."""
    loads = [0] * m
    assign = []
    for i, x in enumerate(weights):
        assign.append(i % m)
        loads[i % m] += int(x)
    return assign, max(loads) if len(assign) else 0


def opt_makespan_bruteforce(weights, m):
    """Exact minimum makespan by exhaustive search (small inputs only)."""
    w = sorted((int(x) for x in weights), reverse=True)
    best = [sum(w)]

    def rec(i, loads):
        if max(loads) >= best[0]:
            return
        if i == len(w):
            best[0] = max(loads)
            return
        seen = set()
        for g in range(m):
            if loads[g] in seen:
                continue
            seen.add(loads[g])
            loads[g] += w[i]
            rec(i + 1, loads)
            loads[g] -= w[i]

    rec(0, [0] * m)
    return best[0]


# ----------------------------------------------------------------------------------------
# error metric


def rel_err(x, ref, nd=2):
    """Relative Frobenius error per output block (the last ``nd`` axes).

    Where the reference block is exactly zero the result is 0 if x is also
    exactly zero there and +inf otherwise.
    """
    x, ref = _f64(x), _f64(ref)
    axes = tuple(range(ref.ndim - nd, ref.ndim))
    num = np.sqrt(np.sum((x - ref) ** 2, axis=axes))
    den = np.sqrt(np.sum(ref ** 2, axis=axes))
    zero = den == 0
    out = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    return np.where(zero & (num != 0), np.inf, out)


def rel_err_T(kind, Tg_hat, Tg_exp, Tr_hat, Tr_exp):
    """Relative error of a represented transition, compared exponent-aligned:
    || 2**(eg - er) Tg_hat - Tr_hat ||_F / || Tr_hat ||_F per chain."""
    nd = _TDIMS[kind]
    de = np.asarray(Tg_exp, np.int64) - np.asarray(Tr_exp, np.int64)
    g = np.ldexp(_f64(Tg_hat), de.reshape(de.shape + (1,) * nd))
    return rel_err(g, Tr_hat, nd)
