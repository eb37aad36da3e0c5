"""HIP graph capture of the layer's forward.

moe_forward is recorded once into a graph through stream capture, the latent
down projection and the shared experts forked onto a second stream by events
and joined back, then replayed on new inputs written into the captured input
buffer.  The forward is deterministic, so each replay must equal the eager
forward of the same input bit for bit: y, the routing (ids, weights, cutoffs,
logits) and the dispatch (counts, offsets, perm, inv_perm).  Eager work and a
synchronisation sit between the replays, and the first input comes back last.
"""
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

KEYS = ("idx", "w", "cutoff", "logits", "counts", "offsets", "perm", "inv_perm")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _inputs(cfg, seeds):
    return [synth.device_layer(cfg, s, names=["x"])["x"] for s in seeds]


@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", {}),
    ("mid_bf16", {}),
    ("mid_bf16", {"bt": 64}),            # short batch: split-K dense GEMMs + their reduction
    ("mid_bf16", {"weight": "fp8"}),
    ("mid_bf16", {"weight": "mxfp4"}),
])
@pytest.mark.parametrize("two_streams", [True, False])
def test_forward_graph_replays_match_eager(name, over, two_streams):
    cfg = synth.CONFIGS[name].with_(**over)
    say(f"graph capture: {name} {over} two_streams={two_streams}")
    layer, x0 = parity.device_layer(cfg, seed=0, cutoff="batch")
    xs = [x0] + _inputs(cfg, (11, 12))
    side = torch.cuda.Stream() if two_streams else None

    # eager references (also the warm-up: workspace, kernel attributes, event pool)
    ref = []
    for x in xs:
        y, r = layer.forward(x, shared_stream=side, return_routing=True)
        ref.append((y.clone(), {k: r[k].clone() for k in KEYS}))
    torch.cuda.synchronize()

    x_buf = xs[0].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_buf, r_buf = layer.forward(x_buf, shared_stream=side, return_routing=True)
    torch.cuda.synchronize()

    for i in (1, 2, 0):
        x_buf.copy_(xs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_ref, r_ref = ref[i]
        assert torch.equal(y_buf, y_ref), f"replay of input {i}: y"
        for k in KEYS:
            assert torch.equal(r_buf[k], r_ref[k]), f"replay of input {i}: {k}"
        # eager work between replays on the same buffers the graph reads
        y_e = layer.forward(xs[i], shared_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(y_e, y_ref)
    del g
