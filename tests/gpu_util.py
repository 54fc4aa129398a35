"""Helpers of the GPU parity tests: move the seeded inputs to the device, run an entry point
through the C-ABI binding, compare with the oracle."""
import sys

import numpy as np

# Gates against the FP64 oracle, max|diff| / max|value| per tensor and call.
SEQ_TOL = 2e-6
CHUNKED_TOL = 5e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x, names=("q", "k", "v", "g", "beta", "s0", "w", "z")):
    import torch
    return {n: torch.from_numpy(x[n]).cuda() for n in names if n in x}


def run(kind, d, state_out=None, o=None, ws=None):
    from linear_attention_recurrence_gated_amd import gdn
    if kind == "seq":
        return gdn.recurrence_seq(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                  state_out=state_out, o=o)
    return gdn.recurrence_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"],
                                  state_out=state_out, o=o, ws=ws)


def f16_ulp_distance(a16, b16):
    """Distance in units in the last place between two float16 arrays (bit patterns mapped
    to a monotone integer scale, so +0 and -0 are 0 apart)."""
    ia = a16.view(np.uint16).astype(np.int32)
    ib = b16.view(np.uint16).astype(np.int32)
    ia = np.where(ia & 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib & 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def y_end_to_end_violations(y_gpu16, o_ref, z, w, eps, tol, y_ref16):
    """Elements of the GPU norm output outside the end-to-end bound; returns (count, worst)
    where worst describes the largest excess.

    Three errors compose.  (1) The recurrence gate allows |o_gpu - o_ref| <= tol * max|o_ref|
    per element; through y_j = o_j r w_j sigmoid(z_j) that becomes at most about
    tol * max|o_ref| * r * |w_j| * sigmoid(z_j) (doubled to cover the change of r).
    (2) The norm kernel's own result is within 1 ulp of the round-to-nearest-even of its
    exact value (the isolated check), i.e. within 1.5 ulp of the exact value.  (3) The
    reference is itself rounded, 0.5 ulp.  Bound: 2 ulp + (1)."""
    o_ref = np.asarray(o_ref, np.float64)
    r = 1.0 / np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    gate = 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))
    prop = 2.0 * tol * np.max(np.abs(o_ref)) * r * np.abs(np.asarray(w, np.float64)) * gate
    yr = y_ref16.astype(np.float64)
    ulp = np.abs(np.spacing(y_ref16)).astype(np.float64)
    diff = np.abs(y_gpu16.astype(np.float64) - yr)
    bound = 2.0 * ulp + prop
    bad = diff > bound
    worst = ""
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, diff / bound, 0)), diff.shape)
        worst = "at %s: gpu %r ref %r diff %.3e ulp %.3e prop %.3e" % (
            i, float(y_gpu16[i]), float(yr[i]), diff[i], ulp[i], prop[i])
    return int(np.count_nonzero(bad)), worst
