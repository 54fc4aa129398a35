"""Seeded synthetic inputs of the model's shape (no model, no dataset).

This module is the one piece shared by the HIP path's tests/bench and the oracle: it only
draws random numbers and holds none of the method's arithmetic.  The distributions follow
the synthetic workload of the pages' parity test ("#413 prefill: DeltaNet recurrence ...",
section "Exactness": synthetic inputs of the model's shape, from a non-zero state):

    q, k   ~ N(0, 1), L2-normalised over the key dim per (token, key head); q also * 1/sqrt(dk)
    v      ~ N(0, 1)
    g      = -exp(U(-4, 0))            (log-decay, so e^g lies in (0.368, 0.982])
    beta   = sigmoid(N(0, 1))
    S0     ~ N(0, 0.1)                 (standard deviation 0.1)
    w      ~ N(1, 0.1)  per value head and column  (output-norm weight)
    z      ~ N(0, 1)                   (output-norm gate input)

Draw order within one seed (numpy PCG64): q, k, v, g, beta, S0, then w, z when asked.
Every array is drawn in float64 and cast once to float32; the oracle widens those same
float32 values back to float64.
"""
from __future__ import annotations

import numpy as np

# Shapes of the layer the pages measure: 16 key heads, 3 value heads per key head,
# dk = dv = 128.
N_K_HEADS = 16
N_V_HEADS = 48
DK = 128
DV = 128


def make_inputs(T: int, seed: int = 0, n_k_heads: int = N_K_HEADS,
                n_v_heads: int = N_V_HEADS, dk: int = DK, dv: int = DV,
                with_norm: bool = False) -> dict:
    """Return a dict of contiguous float32 numpy arrays in the library layout:
    q, k [T][Hk][dk]; v [T][Hv][dv]; g, beta [T][Hv]; s0 [Hv][dk][dv];
    and, if ``with_norm``, w [Hv][dv] and z [T][Hv][dv]."""
    rng = np.random.default_rng(seed)
    out = {}
    q = rng.standard_normal((T, n_k_heads, dk))
    q /= np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-30)
    q *= 1.0 / np.sqrt(dk)
    out["q"] = q.astype(np.float32)
    del q
    k = rng.standard_normal((T, n_k_heads, dk))
    k /= np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-30)
    out["k"] = k.astype(np.float32)
    del k
    out["v"] = rng.standard_normal((T, n_v_heads, dv)).astype(np.float32)
    out["g"] = (-np.exp(rng.uniform(-4.0, 0.0, (T, n_v_heads)))).astype(np.float32)
    out["beta"] = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, n_v_heads))))).astype(np.float32)
    out["s0"] = (0.1 * rng.standard_normal((n_v_heads, dk, dv))).astype(np.float32)
    if with_norm:
        out["w"] = (1.0 + 0.1 * rng.standard_normal((n_v_heads, dv))).astype(np.float32)
        out["z"] = rng.standard_normal((T, n_v_heads, dv)).astype(np.float32)
    return out


# The edge-length sweep of the pages' parity test (from a non-zero state).
EDGE_LENGTHS = (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 257, 1000, 4099)


def make_pre_inputs(T: int, seed: int = 0, n_k_heads: int = N_K_HEADS,
                    n_v_heads: int = N_V_HEADS, dk: int = DK, dv: int = DV,
                    zero_history: bool = False) -> dict:
    """Seeded synthetic inputs of the step before the recurrence, in the library layout
    (float32, contiguous):

        x        [T][C]  ~ N(0, 1)      projection output, C = 2*Hk*dk + Hv*dv channels
                                        (q of each key head, then k, then v of each value head)
        conv_w   [C][4]  ~ N(0, 0.5)    4-tap conv weights (standard deviation 0.5)
        hist     [3][C]  ~ N(0, 1)      conv inputs of the 3 tokens before (zeros if
                                        ``zero_history``: the start of a prompt)
        a, b     [T][Hv] ~ N(0, 1)      raw gate and beta inputs
        A_log    [Hv]    = log(U(1, 16)) gate scale (log)
        dt_bias  [Hv]    ~ N(0, 0.5)    gate bias

    Draw order within one seed (numpy PCG64): x, conv_w, hist, a, b, A_log, dt_bias.  These
    are draws of the shape of the model's projections, no model."""
    rng = np.random.default_rng(seed)
    C = 2 * n_k_heads * dk + n_v_heads * dv
    out = {}
    out["x"] = rng.standard_normal((T, C)).astype(np.float32)
    out["conv_w"] = (0.5 * rng.standard_normal((C, 4))).astype(np.float32)
    hist = rng.standard_normal((3, C)).astype(np.float32)
    out["hist"] = np.zeros_like(hist) if zero_history else hist
    out["a"] = rng.standard_normal((T, n_v_heads)).astype(np.float32)
    out["b"] = rng.standard_normal((T, n_v_heads)).astype(np.float32)
    out["A_log"] = np.log(rng.uniform(1.0, 16.0, n_v_heads)).astype(np.float32)
    out["dt_bias"] = (0.5 * rng.standard_normal(n_v_heads)).astype(np.float32)
    return out
