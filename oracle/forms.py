"""Two independent re-formulations of the gated delta rule, used only to pin the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy, float64.

* ``recurrence_dense``: the per-token update written as a full matrix product,
      S_t = e^{g_t} (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
  which is algebraically the definition (substitute d = beta (v - e^g S^T k) into
  S_t = e^g S + k d^T).

* ``recurrence_wy``: the chunked form of "#1372 DeltaNet recurrence:
  STRATA_GDN_CHUNKED=1", section "What it does": per chunk of C tokens, gamma is the
  inclusive running sum of the gate inside the chunk, A[t][i] = beta_t e^{gamma_t -
  gamma_i} k_t.k_i for i < t, D solves (I + A) D = beta (V - e^{gamma} K S0), the
  outputs are O = diag(e^{gamma}) Q S0 + P D with P[t][i] = e^{gamma_t - gamma_i} q_t.k_i
  for i <= t, and the state after the chunk is
  S' = e^{gamma_last} S0 + K^T diag(e^{gamma_last - gamma}) D.
  Here D comes from ``numpy.linalg.solve`` (a library solve, not a substitution loop).

Both take the library layout: q, k [T][Hk][dk]; v [T][Hv][dv]; g, beta [T][Hv];
S0 [Hv][dk][dv]; value head h reads key head h mod Hk.  They return (o [T][Hv][dv],
S_T [Hv][dk][dv]) in float64.
"""
from __future__ import annotations

import numpy as np


def _expand(q, k, Hv):
    Hk = q.shape[1]
    idx = np.arange(Hv) % Hk
    return q[:, idx, :].astype(np.float64), k[:, idx, :].astype(np.float64)


def recurrence_dense(q, k, v, g, beta, S0):
    T = q.shape[0]
    Hv, dk, dv = S0.shape
    qe, ke = _expand(q, k, Hv)
    v = v.astype(np.float64)
    g = g.astype(np.float64)
    beta = beta.astype(np.float64)
    S = S0.astype(np.float64).copy()
    o = np.zeros((T, Hv, dv))
    eye = np.eye(dk)
    for t in range(T):
        kt = ke[t]                                   # [Hv][dk]
        outer = kt[:, :, None] * kt[:, None, :]      # [Hv][dk][dk]
        trans = np.exp(g[t])[:, None, None] * (eye[None] - beta[t][:, None, None] * outer)
        S = np.matmul(trans, S) + beta[t][:, None, None] * kt[:, :, None] * v[t][:, None, :]
        o[t] = np.einsum("hij,hi->hj", S, qe[t])
    return o, S


def recurrence_wy(q, k, v, g, beta, S0, C=32):
    T = q.shape[0]
    Hv, dk, dv = S0.shape
    qe, ke = _expand(q, k, Hv)
    v = v.astype(np.float64)
    g = g.astype(np.float64)
    beta = beta.astype(np.float64)
    S = S0.astype(np.float64).copy()
    o = np.zeros((T, Hv, dv))
    for c0 in range(0, T, C):
        c1 = min(c0 + C, T)
        n = c1 - c0
        K = np.transpose(ke[c0:c1], (1, 0, 2))       # [Hv][n][dk]
        Q = np.transpose(qe[c0:c1], (1, 0, 2))
        V = np.transpose(v[c0:c1], (1, 0, 2))        # [Hv][n][dv]
        b = beta[c0:c1].T                            # [Hv][n]
        gam = np.cumsum(g[c0:c1].T, axis=1)          # inclusive running sum
        diff = gam[:, :, None] - gam[:, None, :]     # gamma_t - gamma_i
        lower_strict = np.tril(np.ones((n, n)), -1)
        lower_incl = np.tril(np.ones((n, n)))
        decay = np.exp(np.where(lower_incl > 0, diff, 0.0)) * lower_incl
        KK = np.matmul(K, np.transpose(K, (0, 2, 1)))
        QK = np.matmul(Q, np.transpose(K, (0, 2, 1)))
        A = b[:, :, None] * decay * KK * lower_strict
        P = decay * QK                               # includes the diagonal
        W = np.matmul(K, S)                          # rows: S0^T k_t
        rhs = b[:, :, None] * (V - np.exp(gam)[:, :, None] * W)
        D = np.linalg.solve(np.eye(n)[None] + A, rhs)
        O = np.exp(gam)[:, :, None] * np.matmul(Q, S) + np.matmul(P, D)
        o[c0:c1] = np.transpose(O, (1, 0, 2))
        last = gam[:, -1]
        scale = np.exp(last[:, None] - gam)          # e^{gamma_last - gamma_t}
        S = np.exp(last)[:, None, None] * S + np.matmul(np.transpose(K, (0, 2, 1)),
                                                        scale[:, :, None] * D)
    return o, S
