"""Write ``oracle_small.json``: the FP64 oracle's outputs on three small seeded cases, kept
so that any later change of the oracle's arithmetic shows up as a failing comparison (the
pages print no worked example whose values could be stored instead).

Calls only the seeded input generators and ``oracle/``:

    python tests/golden/make_oracle_small.py

Values are stored as float.hex() strings (exact).  Cases (dk = dv = 8 so that the file
stays small; the oracle takes any head size):
  recurrence  T = 7, 1 key head, 2 value heads, seed 11: o [7][2][8], final state [2][8][8]
  out_norm    the recurrence's o with z, w of the same draw, eps = 1e-6: y bits [7][2][8]
  pre         T = 5, 1 key head, 2 value heads, seed 12, SiLU, eps = 1e-6: q, k [5][1][8],
              v [5][2][8], g, beta [5][2], hist [3][32]
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from linear_attention_recurrence_gated_amd.inputs import make_inputs, make_pre_inputs  # noqa: E402

D = 8


def cases():
    x = make_inputs(7, seed=11, n_k_heads=1, n_v_heads=2, dk=D, dv=D, with_norm=True)
    o, s = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"], threads=1)
    y = oracle.out_norm(o, x["z"], x["w"], 1e-6, threads=1)
    p = make_pre_inputs(5, seed=12, n_k_heads=1, n_v_heads=2, dk=D, dv=D)
    r = oracle.pre(p["x"], p["conv_w"], p["hist"], 1, 2, dk=D, dv=D, a=p["a"], b=p["b"],
                   A_log=p["A_log"], dt_bias=p["dt_bias"], activation=1, eps=1e-6)
    return {
        "recurrence": {"o": o, "state": s},
        "out_norm": {"y_bits": y.view(np.uint16)},
        "pre": {n: r[n] for n in ("q", "k", "v", "g", "beta", "hist")},
    }


def encode(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return {"shape": list(a.shape), "uint16": [int(v) for v in a.ravel()]}
    return {"shape": list(a.shape), "hex": [float(v).hex() for v in a.ravel()]}


def decode(e):
    if "uint16" in e:
        return np.array(e["uint16"], dtype=np.uint16).reshape(e["shape"])
    return np.array([float.fromhex(h) for h in e["hex"]], dtype=np.float64).reshape(e["shape"])


if __name__ == "__main__":
    out = {"note": "written by tests/golden/make_oracle_small.py from oracle/ only",
           "cases": {c: {n: encode(a) for n, a in d.items()} for c, d in cases().items()}}
    # one line per array, so that a change shows as a short diff
    lines = ["{", '"note": %s,' % json.dumps(out["note"]), '"cases": {']
    cs = list(out["cases"].items())
    for i, (c, d) in enumerate(cs):
        lines.append("%s: {" % json.dumps(c))
        items = list(d.items())
        for j, (n, e) in enumerate(items):
            lines.append("  %s: %s%s" % (json.dumps(n), json.dumps(e), "," if j + 1 < len(items) else ""))
        lines.append("}" + ("," if i + 1 < len(cs) else ""))
    lines += ["}", "}"]
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", os.path.join(HERE, "oracle_small.json"))
