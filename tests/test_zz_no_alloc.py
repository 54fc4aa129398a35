"""gdn_layer_chunked_noalloc (the one-call layer with the library's static workspace) against
gdn_layer_chunked with a caller workspace, through the C ABI, on the GPU.

The two share every kernel, so their results must agree bit for bit: o, the final state
and y, on consecutive calls whose second input is smaller than the first (the static array
keeps the first call's contents, which the second must not depend on), at the largest head
count the array holds, and against the oracle within the chunked gate.  Outputs are
NaN-filled before each call.  A repeated call leaves the device's free memory unchanged.
"""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import CHUNKED_TOL, log, to_dev
from linear_attention_recurrence_gated_amd.inputs import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_gated_amd import gdn
    gdn.lib()  # raises if the library is not built: no fallback


def _nan_outputs(d):
    return (torch.full_like(d["s0"], float("nan")), torch.full_like(d["v"], float("nan")),
            torch.full(d["v"].shape, float("nan"), dtype=torch.float16, device=d["v"].device))


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.float16 else t.view(torch.int32)


def _compare(x, d, tag):
    from linear_attention_recurrence_gated_amd import gdn
    Hk, Hv = x["q"].shape[1], x["v"].shape[1]
    ws = gdn.workspace(d["q"].device, Hk, Hv)
    ws.view(torch.float32).fill_(float("nan"))
    s1, o1, y1 = _nan_outputs(d)
    gdn.layer_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["z"], d["w"],
                      eps=1e-6, state_out=s1, o=o1, y=y1, ws=ws)
    s2, o2, y2 = _nan_outputs(d)
    log("noalloc %s T=%d Hk=%d Hv=%d" % (tag, x["q"].shape[0], Hk, Hv))
    gdn.layer_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["z"], d["w"],
                              state_out=s2, o=o2, y=y2, eps=1e-6)
    torch.cuda.synchronize()
    for a, b, n in ((y1, y2, "y"), (o1, o2, "o"), (s1, s2, "state")):
        assert torch.equal(_bits(a), _bits(b)), (tag, n)
    return o2, s2


def test_noalloc_two_calls_second_smaller():
    """Two calls in a row, 4100 tokens (three super-blocks, a ragged last chunk) then 1000
    tokens: each gives gdn_layer_chunked's bits, and the second is within the chunked gate
    of the oracle."""
    import oracle
    for T, seed in ((4100, 61), (1000, 62)):
        x = make_inputs(T, seed=seed, with_norm=True)
        d = to_dev(x)
        o, s = _compare(x, d, "call T=%d" % T)
    o_ref, s_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"])
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(s.cpu().numpy(), s_ref)
    log("  second call vs oracle: out %.3e state %.3e" % (eo, es))
    assert eo <= CHUNKED_TOL and es <= CHUNKED_TOL


def test_noalloc_largest_head_count():
    """64 value heads (16 key heads x 4), the most the static array holds, over two
    super-blocks."""
    x = make_inputs(2100, seed=63, n_k_heads=16, n_v_heads=64, with_norm=True)
    _compare(x, to_dev(x), "max heads")


def test_noalloc_repeated_call_allocates_nothing():
    """After a first call on the device, further calls leave the device's free memory
    unchanged (nothing is allocated or freed by the call)."""
    from linear_attention_recurrence_gated_amd import gdn
    x = make_inputs(3000, seed=64, with_norm=True)
    d = to_dev(x)
    s, o, y = _nan_outputs(d)

    def call():
        gdn.layer_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["z"],
                                  d["w"], state_out=s, o=o, y=y, eps=1e-6)

    call()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    y_first = y.clone()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    log("noalloc free memory before %d after %d" % (free0, free1))
    assert free1 == free0
    assert torch.equal(_bits(y), _bits(y_first))
    assert np.isfinite(o.cpu().numpy()).all()
