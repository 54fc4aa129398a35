"""Thin Python binding of libgdn.so (include/gdn.h) over torch tensors.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels; torch provides device memory and the current stream.  If the library has not
been built, every call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_BAD_SHAPE",
          3: "GDN_ERR_MISALIGNED", 4: "GDN_ERR_ALIASING", 5: "GDN_ERR_WORKSPACE",
          6: "GDN_ERR_HIP"}

# Names and C signatures of every exported entry point (mirrors include/gdn.h).
_P, _I, _I64, _SZ, _F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                         ctypes.c_float)
SIGNATURES = {
    "gdn_recurrence_seq": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _P]),
    "gdn_chunked_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "gdn_recurrence_chunked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _P,
                                    _SZ, _P]),
    "gdn_recurrence_chunked_timed": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I,
                                          _P, _SZ, _P, _I, _P]),
    "gdn_out_norm": (_I, [_P, _P, _P, _F, _P, _I64, _I, _I, _P]),
    "gdn_recurrence": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _P, _SZ, _P]),
    "gdn_layer_chunked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _P, _I64, _I, _I,
                               _I, _I, _P, _SZ, _P]),
    "gdn_layer_chunked_timed": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _P, _I64, _I,
                                     _I, _I, _I, _P, _SZ, _P, _I, _P]),
    "gdn_layer_chunked_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _P, _I64,
                                       _I, _I, _I, _I, _P]),
    "gdn_pre": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _P, _I64, _I, _I,
                     _I, _I, _P]),
    "gdn_status_string": (ctypes.c_char_p, [_I]),
    "gdn_last_hip_error": (_I, []),
    "gdn_abi_version": (_I, []),
}

_lib = None


class GdnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        name = STATUS.get(status, str(status))
        detail = lib().gdn_status_string(status).decode()
        if status == 6:
            detail += " (hipError_t %d)" % lib().gdn_last_hip_error()
        super().__init__("%s failed: %s (%s)" % (fn, name, detail))


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build() or "
                               "python -m linear_attention_recurrence_gated_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise GdnError(fn, status)


def _f32(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError("%s must be a contiguous float32 tensor" % name)
    return t


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _shapes(q, v):
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    return T, Hk, Hv, dk, dv


def check_shapes(q, k, v, g, beta, state_in, state_out=None, o=None, z=None, w=None, y=None):
    """Check every operand's shape against (T, n_k_heads, dk) from q and (n_v_heads, dv)
    from v; raise ValueError on the first mismatch.  Only ``.shape`` is read, so this runs
    on any array (the library receives bare pointers and sizes: a short operand would
    otherwise be read or written past its end).  Returns (T, Hk, Hv, dk, dv)."""
    if len(q.shape) != 3 or len(v.shape) != 3:
        raise ValueError("q must be [T][n_k_heads][dk] and v [T][n_v_heads][dv]; got q %s, v %s"
                         % (tuple(q.shape), tuple(v.shape)))
    T, Hk, Hv, dk, dv = _shapes(q, v)
    want = {"k": (k, (T, Hk, dk)), "v": (v, (T, Hv, dv)), "g": (g, (T, Hv)),
            "beta": (beta, (T, Hv)), "state_in": (state_in, (Hv, dk, dv)),
            "state_out": (state_out, (Hv, dk, dv)), "o": (o, (T, Hv, dv)),
            "z": (z, (T, Hv, dv)), "w": (w, (Hv, dv)), "y": (y, (T, Hv, dv))}
    for name, (t, shape) in want.items():
        if t is not None and tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s (T=%d, n_k_heads=%d, n_v_heads=%d, "
                             "dk=%d, dv=%d)" % (name, tuple(t.shape), shape, T, Hk, Hv, dk, dv))
    return T, Hk, Hv, dk, dv


def check_norm_shapes(o, z, w, y=None):
    """Shapes of the output norm's operands: o, z, y [T][n_v_heads][dv], w [n_v_heads][dv]."""
    if len(o.shape) != 3:
        raise ValueError("o must be [T][n_v_heads][dv]; got %s" % (tuple(o.shape),))
    T, Hv, dv = o.shape
    for name, t, shape in (("z", z, (T, Hv, dv)), ("w", w, (Hv, dv)), ("y", y, (T, Hv, dv))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
    return T, Hv, dv


def recurrence_seq(q, k, v, g, beta, state_in, state_out=None, o=None, stream=None):
    """Sequential kernel.  Returns (o, state_out); state_out may be state_in (in place)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state_in, "state_in")):
        _f32(t, n)
    check_shapes(q, k, v, g, beta, state_in, state_out, o)
    T, Hk, Hv, dk, dv = _shapes(q, v)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if o is None:
        o = torch.empty_like(v)
    _f32(state_out, "state_out"); _f32(o, "o")
    st = lib().gdn_recurrence_seq(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(state_in), _ptr(state_out), _ptr(o), T, Hk, Hv, dk, dv,
                                  _stream(stream, q.device))
    _check("gdn_recurrence_seq", st)
    return o, state_out


def chunked_workspace_bytes(n_k_heads, n_v_heads, dk=128, dv=128):
    return int(lib().gdn_chunked_workspace_bytes(n_k_heads, n_v_heads, dk, dv))


_workspaces = {}


def workspace(device, n_k_heads, n_v_heads, dk=128, dv=128, stream=None):
    """The chunked kernels' scratch, one per (device, stream): allocated on first use and
    kept.  Calls on one stream are ordered, so they can share it; calls on different
    streams may overlap, so each stream gets its own (calls that pass a workspace
    themselves must not share one across streams either)."""
    need = chunked_workspace_bytes(n_k_heads, n_v_heads, dk, dv)
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (dev.index, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        if ws is not None:
            s.synchronize()  # work already queued on this stream may still use the old one
        with torch.cuda.stream(s):  # the allocator ties the memory to the stream it serves
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def recurrence_chunked(q, k, v, g, beta, state_in, state_out=None, o=None, ws=None,
                       stream=None, scan_events=None):
    """Chunked WY kernels.  Returns (o, state_out).  ``scan_events`` (a sequence of raw
    hipEvent_t handles) selects the profiling entry point, which records them around each
    super-block's scan kernel."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state_in, "state_in")):
        _f32(t, n)
    check_shapes(q, k, v, g, beta, state_in, state_out, o)
    T, Hk, Hv, dk, dv = _shapes(q, v)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if o is None:
        o = torch.empty_like(v)
    _f32(state_out, "state_out"); _f32(o, "o")
    if ws is None:
        ws = workspace(q.device, Hk, Hv, dk, dv, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(state_out),
            _ptr(o), T, Hk, Hv, dk, dv, _ptr(ws), ws.numel() * ws.element_size())
    if scan_events is None:
        st = lib().gdn_recurrence_chunked(*args, _stream(stream, q.device))
        _check("gdn_recurrence_chunked", st)
    else:
        arr = (ctypes.c_void_p * max(1, len(scan_events)))(*scan_events)
        st = lib().gdn_recurrence_chunked_timed(*args, arr, len(scan_events),
                                                _stream(stream, q.device))
        _check("gdn_recurrence_chunked_timed", st)
    return o, state_out


CHUNKED_MIN_T = 56  # GDN_CHUNKED_MIN_T of gdn.h


def recurrence(q, k, v, g, beta, state_in, state_out=None, o=None, ws=None, stream=None):
    """The recurrence with the kernel chosen by T (sequential below CHUNKED_MIN_T tokens,
    chunked from there).  Returns (o, state_out)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state_in, "state_in")):
        _f32(t, n)
    check_shapes(q, k, v, g, beta, state_in, state_out, o)
    T, Hk, Hv, dk, dv = _shapes(q, v)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if o is None:
        o = torch.empty_like(v)
    _f32(state_out, "state_out"); _f32(o, "o")
    if ws is None and T >= CHUNKED_MIN_T:
        ws = workspace(q.device, Hk, Hv, dk, dv, stream)
    ws_ptr, ws_bytes = (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())
    st = lib().gdn_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                              _ptr(state_out), _ptr(o), T, Hk, Hv, dk, dv, ws_ptr, ws_bytes,
                              _stream(stream, q.device))
    _check("gdn_recurrence", st)
    return o, state_out


def layer_chunked(q, k, v, g, beta, state_in, z, w, eps=1e-6, state_out=None, o=None, y=None,
                  ws=None, stream=None, scan_events=None):
    """Chunked recurrence + gated RMS norm in one call.  Returns (y, o, state_out);
    ``scan_events`` selects the profiling entry point (events around each recurrence
    launch)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state_in, "state_in"),
                 (z, "z"), (w, "w")):
        _f32(t, n)
    check_shapes(q, k, v, g, beta, state_in, state_out, o, z, w, y)
    T, Hk, Hv, dk, dv = _shapes(q, v)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if o is None:
        o = torch.empty_like(v)
    if y is None:
        y = torch.empty(v.shape, dtype=torch.float16, device=v.device)
    _f32(state_out, "state_out"); _f32(o, "o")
    if y.dtype != torch.float16 or not y.is_contiguous() or not y.is_cuda:
        raise TypeError("y must be a contiguous float16 CUDA tensor")
    if ws is None:
        ws = workspace(q.device, Hk, Hv, dk, dv, stream)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(state_out),
            _ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(y), T, Hk, Hv, dk, dv, _ptr(ws),
            ws.numel() * ws.element_size())
    if scan_events is None:
        st = lib().gdn_layer_chunked(*args, _stream(stream, q.device))
        _check("gdn_layer_chunked", st)
    else:
        arr = (ctypes.c_void_p * max(1, len(scan_events)))(*scan_events)
        st = lib().gdn_layer_chunked_timed(*args, arr, len(scan_events), _stream(stream, q.device))
        _check("gdn_layer_chunked_timed", st)
    return y, o, state_out


def check_pre_shapes(x, conv_w, hist_in, n_k_heads, n_v_heads, dk=128, dv=128, hist_out=None,
                     a=None, b=None, A_log=None, dt_bias=None, q=None, k=None, v=None, g=None,
                     beta=None):
    """Shapes of gdn_pre's operands against T from x and the head counts (ValueError on the
    first mismatch; only ``.shape`` is read).  Returns (T, C)."""
    if len(x.shape) != 2:
        raise ValueError("x must be [T][C]; got %s" % (tuple(x.shape),))
    T, C = x.shape
    if C != (2 * n_k_heads) * dk + n_v_heads * dv:
        raise ValueError("x has %d channels, expected 2*%d*%d + %d*%d"
                         % (C, n_k_heads, dk, n_v_heads, dv))
    want = {"conv_w": (conv_w, (C, 4)), "hist_in": (hist_in, (3, C)),
            "hist_out": (hist_out, (3, C)), "a": (a, (T, n_v_heads)), "b": (b, (T, n_v_heads)),
            "A_log": (A_log, (n_v_heads,)), "dt_bias": (dt_bias, (n_v_heads,)),
            "q": (q, (T, n_k_heads, dk)), "k": (k, (T, n_k_heads, dk)),
            "v": (v, (T, n_v_heads, dv)), "g": (g, (T, n_v_heads)), "beta": (beta, (T, n_v_heads))}
    for name, (t, shape) in want.items():
        if t is not None and tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
    return T, C


def pre(x, conv_w, hist_in, n_k_heads, n_v_heads, a=None, b=None, A_log=None, dt_bias=None,
        activation=1, eps=1e-6, hist_out=None, q=None, k=None, v=None, g=None, beta=None,
        stream=None):
    """gdn_pre: the 4-tap causal conv with its history, the q/k normalisation and (when a,
    b, A_log, dt_bias are given) the gate and beta.  Returns a dict with q, k, v, hist_out
    and, with the gate inputs, g and beta."""
    for t, n in ((x, "x"), (conv_w, "conv_w"), (hist_in, "hist_in")):
        _f32(t, n)
    gates = a is not None
    if gates:
        for t, n in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias")):
            _f32(t, n)
    dk = dv = 128
    T, C = check_pre_shapes(x, conv_w, hist_in, n_k_heads, n_v_heads, dk, dv, hist_out, a, b,
                            A_log, dt_bias, q, k, v, g, beta)
    dev = x.device
    if hist_out is None:
        hist_out = torch.empty_like(hist_in)
    if q is None:
        q = torch.empty((T, n_k_heads, dk), dtype=torch.float32, device=dev)
    if k is None:
        k = torch.empty((T, n_k_heads, dk), dtype=torch.float32, device=dev)
    if v is None:
        v = torch.empty((T, n_v_heads, dv), dtype=torch.float32, device=dev)
    if gates and g is None:
        g = torch.empty((T, n_v_heads), dtype=torch.float32, device=dev)
    if gates and beta is None:
        beta = torch.empty((T, n_v_heads), dtype=torch.float32, device=dev)
    for t, n in ((hist_out, "hist_out"), (q, "q"), (k, "k"), (v, "v")):
        _f32(t, n)
    if gates:
        _f32(g, "g"); _f32(beta, "beta")
    st = lib().gdn_pre(_ptr(x), _ptr(conv_w), _ptr(hist_in), _ptr(hist_out),
                       _ptr(a if gates else None), _ptr(b if gates else None),
                       _ptr(A_log if gates else None), _ptr(dt_bias if gates else None),
                       int(activation), float(eps), _ptr(q), _ptr(k), _ptr(v),
                       _ptr(g if gates else None), _ptr(beta if gates else None), T, n_k_heads,
                       n_v_heads, dk, dv, _stream(stream, dev))
    _check("gdn_pre", st)
    out = {"q": q, "k": k, "v": v, "hist_out": hist_out}
    if gates:
        out["g"], out["beta"] = g, beta
    return out


NOALLOC_MAX_V_HEADS = 64  # the static workspace's head count (gdn.h)


def layer_chunked_noalloc(q, k, v, g, beta, state_in, z, w, state_out, o, y, eps=1e-6,
                          stream=None):
    """gdn_layer_chunked_noalloc: the one-call layer with the library's static workspace.
    Every output is the caller's (nothing is allocated here either).  Returns
    (y, o, state_out)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state_in, "state_in"),
                 (z, "z"), (w, "w"), (state_out, "state_out"), (o, "o")):
        _f32(t, n)
    check_shapes(q, k, v, g, beta, state_in, state_out, o, z, w, y)
    T, Hk, Hv, dk, dv = _shapes(q, v)
    if y.dtype != torch.float16 or not y.is_contiguous() or not y.is_cuda:
        raise TypeError("y must be a contiguous float16 CUDA tensor")
    st = lib().gdn_layer_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(o),
        _ptr(z), _ptr(w), float(eps), _ptr(y), T, Hk, Hv, dk, dv, _stream(stream, q.device))
    _check("gdn_layer_chunked_noalloc", st)
    return y, o, state_out


def out_norm(o, z, w, eps=1e-6, y=None, stream=None):
    """Gated RMS output norm.  Returns y as a float16 tensor [T][Hv][dv]."""
    _f32(o, "o"); _f32(z, "z"); _f32(w, "w")
    T, Hv, dv = check_norm_shapes(o, z, w, y)
    if y is None:
        y = torch.empty(o.shape, dtype=torch.float16, device=o.device)
    if y.dtype != torch.float16 or not y.is_contiguous() or not y.is_cuda:
        raise TypeError("y must be a contiguous float16 CUDA tensor")
    st = lib().gdn_out_norm(_ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(y), T, Hv, dv,
                            _stream(stream, o.device))
    _check("gdn_out_norm", st)
    return y
