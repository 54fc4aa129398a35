"""Parity of gdn_pre (the step before the recurrence) with the FP64 oracle, on the GPU.

Gate: max|diff| / max|value| per output tensor and call <= 1e-6 for q, k, v, g and beta.
Derivation: each output element is a short FP32 expression of its inputs (a 4-term FMA
chain for the conv; for SiLU a correctly rounded exp, add and divide; for q and k a
128-term sum of squares, a correctly rounded square root and divide, and for q the
rounded 1/sqrt(128); for g an exp, a log1p and a product), so every element is within
about 12 units of 2^-24 of its exact value relative to its own size, below 7.2e-7; the
history out is a copy and must match bit for bit.  Inputs are the seeded draws of
``make_pre_inputs`` (the shapes of the model's projections: 16 key heads, 48 value heads,
dk = dv = 128).
"""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import CHUNKED_TOL, log
from linear_attention_recurrence_gated_amd.inputs import make_pre_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PRE_TOL = 1e-6
HK, HV = 16, 48


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_gated_amd import gdn
    gdn.lib()  # raises if the library is not built: no fallback


def _dev(x):
    return {n: torch.from_numpy(a).cuda() for n, a in x.items()}


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _run_gpu(d, T, activation, eps, gates=True, hk=HK, hv=HV):
    from linear_attention_recurrence_gated_amd import gdn
    kw = dict(a=d["a"], b=d["b"], A_log=d["A_log"], dt_bias=d["dt_bias"]) if gates else {}
    out = dict(q=_nan((T, hk, 128)), k=_nan((T, hk, 128)), v=_nan((T, hv, 128)),
               hist_out=_nan(tuple(d["hist"].shape)))
    if gates:
        out.update(g=_nan((T, hv)), beta=_nan((T, hv)))
    return gdn.pre(d["x"], d["conv_w"], d["hist"], hk, hv, activation=activation, eps=eps,
                   **kw, **out)


def _compare(x, r, T, activation, eps, gates=True, hk=HK, hv=HV, tag=""):
    import oracle
    kw = dict(a=x["a"], b=x["b"], A_log=x["A_log"], dt_bias=x["dt_bias"]) if gates else {}
    ref = oracle.pre(x["x"], x["conv_w"], x["hist"], hk, hv, activation=activation, eps=eps,
                     **kw)
    torch.cuda.synchronize()
    errs = {}
    for n in ("q", "k", "v") + (("g", "beta") if gates else ()):
        got = r[n].cpu().numpy()
        assert np.isfinite(got).all(), (tag, n)
        errs[n] = rel_err(got, ref[n])
    log("pre %s T=%d act=%d eps=%g: %s" % (tag, T, activation, eps,
                                          " ".join("%s %.2e" % kv for kv in errs.items())))
    for n, e in errs.items():
        assert e <= PRE_TOL, (tag, n, e)
    assert np.array_equal(r["hist_out"].cpu().numpy().astype(np.float64), ref["hist"]), tag
    return ref


@pytest.mark.parametrize("activation", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 100,
                               2049])
def test_pre_against_oracle(T, activation):
    """Run lengths around the 32-token runs of a wave and its 16-token load batches, from a
    non-zero history, with and without the activation."""
    x = make_pre_inputs(T, seed=T + 7 * activation)
    r = _run_gpu(_dev(x), T, activation, 1e-6)
    _compare(x, r, T, activation, 1e-6)


def test_pre_zero_history_other_heads_eps_zero():
    """The start of a prompt (zero history), 4 key heads with 2 value heads each, eps = 0
    (no row is all zero), no gate inputs."""
    T, hk, hv = 300, 4, 8
    x = make_pre_inputs(T, seed=3, n_k_heads=hk, n_v_heads=hv, zero_history=True)
    r = _run_gpu(_dev(x), T, 1, 0.0, gates=False, hk=hk, hv=hv)
    _compare(x, r, T, 1, 0.0, gates=False, hk=hk, hv=hv, tag="zero-hist")
    assert "g" not in r


def test_pre_extreme_values():
    """Rows far from the workload: large inputs (SiLU saturates to the identity and to 0),
    a zero block (its q/k normalise to 0 through eps), gate inputs of +-60 (softplus and the
    sigmoid saturate)."""
    T = 70
    x = make_pre_inputs(T, seed=17)
    x["x"][5] *= 300.0
    x["x"][6, :HK * 128] = 0.0
    x["hist"][:] = 0.0
    x["a"][10] = 60.0
    x["a"][11] = -60.0
    x["b"][12] = 60.0
    x["b"][13] = -60.0
    r = _run_gpu(_dev(x), T, 1, 1e-6)
    _compare(x, r, T, 1, 1e-6, tag="extreme")


@pytest.mark.parametrize("T1", [1, 2, 3, 16, 31, 32, 33, 64, 100])
def test_pre_split_calls_bitwise(T1):
    """Two calls chained through the history give one call's bits (every token's arithmetic
    is the same whichever run or call it falls in)."""
    T = 230
    x = make_pre_inputs(T, seed=21)
    d = _dev(x)
    full = _run_gpu(d, T, 1, 1e-6)
    first = dict(d, x=d["x"][:T1].contiguous(), a=d["a"][:T1].contiguous(),
                 b=d["b"][:T1].contiguous())
    r1 = _run_gpu(first, T1, 1, 1e-6)
    second = dict(d, x=d["x"][T1:].contiguous(), a=d["a"][T1:].contiguous(),
                  b=d["b"][T1:].contiguous(), hist=r1["hist_out"])
    r2 = _run_gpu(second, T - T1, 1, 1e-6)
    torch.cuda.synchronize()
    for n in ("q", "k", "v", "g", "beta"):
        assert torch.equal(torch.cat([r1[n], r2[n]]).view(torch.int32),
                           full[n].view(torch.int32)), n
    assert torch.equal(r2["hist_out"].view(torch.int32), full["hist_out"].view(torch.int32))


def test_pre_zero_tokens_copies_history():
    from linear_attention_recurrence_gated_amd import gdn
    x = make_pre_inputs(0, seed=2)
    d = _dev(x)
    r = gdn.pre(d["x"], d["conv_w"], d["hist"], HK, HV, hist_out=_nan(tuple(d["hist"].shape)))
    torch.cuda.synchronize()
    assert torch.equal(r["hist_out"], d["hist"])


def test_pre_feeds_the_layer():
    """gdn_pre's outputs as the recurrence's inputs: the one-call layer on them is within
    the chunked gate of the oracle recurrence on the same (GPU-made) inputs, and the keys it
    produced have unit norm."""
    import oracle
    from linear_attention_recurrence_gated_amd import gdn, make_inputs
    T = 2100
    x = make_pre_inputs(T, seed=33)
    r = _run_gpu(_dev(x), T, 1, 1e-6)
    torch.cuda.synchronize()
    kn = torch.linalg.vector_norm(r["k"].double(), dim=-1)
    assert float((kn - 1).abs().max()) <= 1e-6
    rest = make_inputs(1, seed=34, with_norm=True)  # S0 and the norm weight
    s0 = torch.from_numpy(rest["s0"]).cuda()
    w = torch.from_numpy(rest["w"]).cuda()
    z = torch.randn((T, HV, 128), generator=torch.Generator(device="cuda").manual_seed(35),
                    device="cuda")
    y, o, s = gdn.layer_chunked(r["q"], r["k"], r["v"], r["g"], r["beta"], s0, z, w, eps=1e-6)
    torch.cuda.synchronize()
    h = {n: r[n].cpu().numpy() for n in ("q", "k", "v", "g", "beta")}
    o_ref, s_ref = oracle.recurrence(h["q"], h["k"], h["v"], h["g"], h["beta"], rest["s0"])
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(s.cpu().numpy(), s_ref)
    log("pre -> layer: out %.3e state %.3e" % (eo, es))
    assert eo <= CHUNKED_TOL and es <= CHUNKED_TOL
