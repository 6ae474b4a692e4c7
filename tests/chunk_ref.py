"""fp64 CPU model of the chunked WY/UT form the device kernels compute.

Not the oracle: this is the device algorithm written out in float64, used to
check that the chunk identities equal the token recurrence and to localise a
device mismatch stage by stage.  Chunk identities (derived from the gated delta
rule; WY/UT representation: Bischof & Van Loan 1987, Joffrain et al. 2006;
chunkwise delta rule: Yang et al., NeurIPS 2024):

  G_i = sum_{j<=i} log alpha_j, gamma_i = exp(G_i), Gamma = gamma_C
  L_ij = beta_i (gamma_i/gamma_j) k_i.k_j for i > j
  Tg = (I + L)^-1 diag(beta), U = Tg V, W' = Tg diag(gamma) K
  X = [T | S] <- Gamma X + K^T diag(Gamma/gamma) ([0 | U] - W' X)
  outputs from S0: O = diag(gamma) Q S0 + M (U - W' S0), M_ij = (gamma_i/gamma_j) q_i.k_j, j <= i
"""

import numpy as np


def chunk_stage(k, v, la, b):
    """Per-chunk quantities for one chunk (n <= C tokens)."""
    k, v, la, b = (np.asarray(a, np.float64) for a in (k, v, la, b))
    G = np.cumsum(la)
    gam = np.exp(G)
    n = len(la)
    Gij = np.exp(G[:, None] - G[None, :])
    L = np.tril(b[:, None] * Gij * (k @ k.T), -1)
    Tg = np.linalg.solve(np.eye(n) + L, np.diag(b))
    return {"G": G, "gamma": gam, "Gamma": gam[-1] if n else 1.0, "L": L, "Tg": Tg,
            "U": Tg @ v, "W": Tg @ (gam[:, None] * k)}


def chunked_build(k, v, la, b, C=64):
    """(T, S) of one segment by the chunk form; T as (T_hat, exponent)."""
    n, dk = k.shape
    dv = v.shape[1]
    X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
    e = 0
    for c0 in range(0, n, C):
        c1 = min(n, c0 + C)
        st = chunk_stage(k[c0:c1], v[c0:c1], la[c0:c1], b[c0:c1])
        kk = np.asarray(k[c0:c1], np.float64)
        Vn = np.concatenate([np.zeros((c1 - c0, dk)), st["U"]], axis=1) - st["W"] @ X
        Vn *= (st["Gamma"] / st["gamma"])[:, None]
        X = st["Gamma"] * X + kk.T @ Vn
        m = np.abs(X[:, :dk]).max()
        _, s = np.frexp(m)
        X[:, :dk] = np.ldexp(X[:, :dk], -s)
        e += int(s)
    return X[:, :dk], e, X[:, dk:]


def chunk_outputs(q, k, v, la, b, S0):
    """Outputs and end state of one chunk from S0 (the seam form)."""
    st = chunk_stage(k, v, la, b)
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    G = st["G"]
    M = np.tril(np.exp(G[:, None] - G[None, :]) * (q @ k.T))
    Qt = st["gamma"][:, None] * q - M @ st["W"]
    O = Qt @ S0 + M @ st["U"]
    S = st["Gamma"] * S0 + k.T @ ((st["Gamma"] / st["gamma"])[:, None] * (st["U"] - st["W"] @ S0))
    return O, S
