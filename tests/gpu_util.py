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
