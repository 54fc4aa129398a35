"""gdn_layer_chunked_noalloc captured in a HIP graph (the kind of caller it is for): every
replay gives the bits of the same call made eagerly.

The graph is replayed several times, with NaN-filled outputs and unrelated eager library
work between the replays, and each replay is compared with the eager result.
"""
import pytest

from gpu_util import log, to_dev
from linear_attention_recurrence_gated_amd.inputs import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_attention_recurrence_gated_amd import gdn
    gdn.lib()  # raises if the library is not built: no fallback


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.float16 else t.view(torch.int32)


def test_noalloc_layer_replayed_from_a_graph():
    from linear_attention_recurrence_gated_amd import gdn
    T = 4100  # three super-blocks, a ragged last chunk
    x = make_inputs(T, seed=31, with_norm=True)
    d = to_dev(x)
    st = torch.empty_like(d["s0"])
    o = torch.empty_like(d["v"])
    y = torch.empty(d["v"].shape, dtype=torch.float16, device=d["v"].device)

    def call():
        gdn.layer_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["z"],
                                  d["w"], state_out=st, o=o, y=y, eps=1e-6)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # eager, on the stream the graph is captured on: the reference
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (st, o, y)]

    log("capture noalloc layer T=%d" % T)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    other = make_inputs(700, seed=32, with_norm=True)
    od = to_dev(other)
    for rep in range(4):
        for t in (st, o, y):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        log("replay %d" % rep)
        graph.replay()
        torch.cuda.synchronize()
        for a, b, n in zip((st, o, y), ref, ("state", "o", "y")):
            assert torch.equal(_bits(a), _bits(b)), (rep, n)
        # unrelated eager work between the replays (the same static workspace included)
        gdn.layer_chunked_noalloc(od["q"], od["k"], od["v"], od["g"], od["beta"], od["s0"],
                                  od["z"], od["w"], state_out=torch.empty_like(od["s0"]),
                                  o=torch.empty_like(od["v"]),
                                  y=torch.empty(od["v"].shape, dtype=torch.float16,
                                                device=od["v"].device), eps=1e-6)
        torch.cuda.synchronize()
