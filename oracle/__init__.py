"""FP64 CPU oracle for the gated delta rule and the gated RMS output norm.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports it, and this package imports nothing from the
product path.  The two sides meet only through the seeded float32 input arrays.

What it computes (O1 recurrence, O2 output norm, O3 the step before the recurrence: the
4-tap causal conv with its history, the q/k normalisation and the gate/beta formation) is
documented, with citations of the pages, in ``gdn_oracle.c``; ``forms.py`` holds two
independent re-formulations used only to pin O1 (the dense per-token form and the chunked
WY form).

The C part is built with plain ``gcc -O2 -fopenmp`` (no fast-math) into
``oracle/libgdn_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# ORACLE_LIB_OVERRIDE points the loader at another build of this same source (used to
# check that the pins catch deliberately planted mistakes).
_LIB = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (plain gcc, FP64, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    lib.gdn_oracle_recurrence.argtypes = [P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                                          ctypes.c_int, P, P, ctypes.c_int]
    lib.gdn_oracle_recurrence.restype = ctypes.c_int
    lib.gdn_oracle_recurrence_f64.argtypes = [P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, P]
    lib.gdn_oracle_recurrence_f64.restype = ctypes.c_int
    lib.gdn_oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.gdn_oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.gdn_oracle_out_norm.argtypes = [P, P, P, P, ctypes.c_double, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
    lib.gdn_oracle_out_norm.restype = ctypes.c_int
    lib.gdn_oracle_pre.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, P, P, P, P, P, P]
    lib.gdn_oracle_pre.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.argtypes = []
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def recurrence(q, k, v, g, beta, state_in, heads=None, threads: int = 0):
    """O1 on float32 inputs in the library layout.

    q, k [T][Hk][dk]; v [T][Hv][dv]; g, beta [T][Hv]; state_in [Hv][dk][dv] (float32).
    ``heads`` selects value heads (default: all).  Returns float64 arrays
    ``o [T][n_sel][dv]`` and ``state [n_sel][dk][dv]`` for the selected heads, in order.
    """
    lib = _load()
    q = _c(q, np.float32); k = _c(k, np.float32); v = _c(v, np.float32)
    g = _c(g, np.float32); beta = _c(beta, np.float32); s0 = _c(state_in, np.float32)
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, Hv)
    assert beta.shape == (T, Hv) and s0.shape == (Hv, dk, dv)
    sel = np.arange(Hv, dtype=np.int32) if heads is None else _c(heads, np.int32)
    n = int(sel.size)
    o_sel = np.empty((n, T, dv), np.float64)
    s_sel = np.empty((n, dk, dv), np.float64)
    rc = lib.gdn_oracle_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                   T, Hk, Hv, dk, dv, _ptr(sel), n, _ptr(o_sel), _ptr(s_sel),
                                   int(threads))
    if rc != 0:
        raise ValueError("gdn_oracle_recurrence rejected its arguments")
    return np.ascontiguousarray(o_sel.transpose(1, 0, 2)), s_sel


def recurrence_f64(q, k, v, g, beta, state_in):
    """O1 for one head from float64 inputs: q, k [T][dk]; v [T][dv]; g, beta [T];
    state_in [dk][dv].  Returns (o [T][dv], state [dk][dv]) in float64."""
    lib = _load()
    q = _c(q, np.float64); k = _c(k, np.float64); v = _c(v, np.float64)
    g = _c(g, np.float64); beta = _c(beta, np.float64)
    st = np.array(state_in, dtype=np.float64, order="C", copy=True)
    T, dk = q.shape
    dv = v.shape[1]
    o = np.empty((T, dv), np.float64)
    rc = lib.gdn_oracle_recurrence_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(st), T, dk, dv, _ptr(o))
    if rc != 0:
        raise ValueError("gdn_oracle_recurrence_f64 rejected its arguments")
    return o, st


def f64_to_f16_bits(x: float) -> int:
    """The oracle's own double -> binary16 (round to nearest even) encoding."""
    return int(_load().gdn_oracle_f64_to_f16(float(x)))


def out_norm(o, z, w, eps: float, heads=None, threads: int = 0, return_prerounding=False):
    """O2.  o, z [..., Hv_sel, dv] (any float dtype, widened to float64);
    w [Hv][dv]; ``heads`` gives the value head of each position of axis -2 (default
    0..Hv-1).  Returns y as float16 with o's shape (and the float64 value before
    rounding if ``return_prerounding``)."""
    lib = _load()
    o = np.asarray(o)
    shape = o.shape
    dv = shape[-1]
    nh = shape[-2]
    w = _c(w, np.float64)
    hsel = np.arange(nh, dtype=np.int32) if heads is None else _c(heads, np.int32)
    assert hsel.size == nh
    o2 = _c(o.reshape(-1, dv), np.float64)
    z2 = _c(np.asarray(z).reshape(-1, dv), np.float64)
    assert z2.shape == o2.shape
    n_rows = o2.shape[0]
    w_idx = _c(np.tile(hsel, n_rows // nh), np.int32)
    y16 = np.empty((n_rows, dv), np.uint16)
    y64 = np.empty((n_rows, dv), np.float64) if return_prerounding else None
    rc = lib.gdn_oracle_out_norm(_ptr(o2), _ptr(z2), _ptr(w), _ptr(w_idx), float(eps),
                                 n_rows, w.shape[0], dv,
                                 _ptr(y64) if y64 is not None else None, _ptr(y16),
                                 int(threads))
    if rc != 0:
        raise ValueError("gdn_oracle_out_norm rejected its arguments")
    y = y16.view(np.float16).reshape(shape)
    if return_prerounding:
        return y, y64.reshape(shape)
    return y


def pre(x, conv_w, hist, n_k_heads, n_v_heads, dk=128, dv=128, a=None, b=None, A_log=None,
        dt_bias=None, activation=1, eps=1e-6):
    """O3, the step before the recurrence, on float32 inputs in the library layout:
    x [T][2*Hk*dk + Hv*dv] (q | k | v channels), conv_w [C][4], hist [3][C]; optionally
    a, b [T][Hv] and A_log, dt_bias [Hv] for the gate and beta.  Returns a dict of float64
    arrays: q, k [T][Hk][dk]; v [T][Hv][dv]; hist [3][C]; and g, beta [T][Hv] when the gate
    inputs are given."""
    lib = _load()
    x = _c(x, np.float32); w = _c(conv_w, np.float32); hs = _c(hist, np.float32)
    T, C = x.shape
    assert C == 2 * n_k_heads * dk + n_v_heads * dv
    assert w.shape == (C, 4) and hs.shape == (3, C)
    out = {"q": np.empty((T, n_k_heads, dk)), "k": np.empty((T, n_k_heads, dk)),
           "v": np.empty((T, n_v_heads, dv)), "hist": np.empty((3, C))}
    gates = a is not None
    if gates:
        a = _c(a, np.float32); b = _c(b, np.float32)
        A_log = _c(A_log, np.float32); dt_bias = _c(dt_bias, np.float32)
        assert a.shape == (T, n_v_heads) and b.shape == (T, n_v_heads)
        assert A_log.shape == (n_v_heads,) and dt_bias.shape == (n_v_heads,)
        out["g"] = np.empty((T, n_v_heads))
        out["beta"] = np.empty((T, n_v_heads))
    nul = ctypes.c_void_p(0)
    rc = lib.gdn_oracle_pre(_ptr(x), _ptr(w), _ptr(hs),
                            _ptr(a) if gates else nul, _ptr(b) if gates else nul,
                            _ptr(A_log) if gates else nul, _ptr(dt_bias) if gates else nul,
                            int(activation), float(eps), T, n_k_heads, n_v_heads, dk, dv,
                            _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]),
                            _ptr(out["g"]) if gates else nul,
                            _ptr(out["beta"]) if gates else nul, _ptr(out["hist"]))
    if rc != 0:
        raise ValueError("gdn_oracle_pre rejected its arguments")
    return out
