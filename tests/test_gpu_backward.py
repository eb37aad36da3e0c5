"""GPU parity of the backward pass (moe_backward) against the fp64 backward
oracle: every gradient, normwise max relative error within the bf16 bound,
with the routing the GPU chose (itself checked against the oracle's routing:
equal, or a near tie that is a valid top-k of the oracle's scores)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import backward as ob
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = parity.TOL["bf16"]


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bf16_dy(cfg, seed):
    """dL/dy, normal values rounded to bf16: the raw bits and their fp64 values."""
    v = np.random.default_rng(seed).normal(0, 1, (cfg.bt, cfg.d)).astype(np.float32)
    bits = (v.view(np.uint32) + 0x7FFF + ((v.view(np.uint32) >> 16) & 1)) >> 16
    bits = bits.astype(np.uint16)
    return bits, oracle.decode(bits)


def _check(cfg, cutoff, seed=0):
    say("backward", cfg.name, "bt", cfg.bt, "cutoff", cutoff, "S", cfg.n_shared)
    layer, x = parity.device_layer(cfg, seed=seed, cutoff=cutoff)
    bits, dy64 = _bf16_dy(cfg, seed + 7)
    dy = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    r = layer.route(x)
    g = layer.backward(x, dy, route=r)
    torch.cuda.synchronize()
    idx = parity.to_np(r["idx"])
    ref_route = parity.oracle_routing_full(cfg, seed=seed, cutoff=cutoff)
    _, bad = parity.routing_mismatches(idx, ref_route["idx"], ref_route["z32"],
                                       ref_route["alpha"])
    assert not bad, f"tokens whose expert set is not a valid top-k: {bad[:8]}"
    host = synth.host_layer(cfg, seed)
    p = ob.decode_layer(cfg, host)
    ref = ob.backward(cfg, p, oracle.decode(host["x"]), idx.astype(np.int64), dy64)
    worst = 0.0
    for name in ob.GRAD_NAMES:
        if cfg.n_shared == 0 and name.startswith("sh_"):
            continue
        got = parity.to_np(g[name]).astype(np.float64)
        want = ref[name]
        assert got.shape == want.shape, name
        err = parity.normwise_err(got, want)
        worst = max(worst, err)
        say(f"  {name:13s} normwise {err:.2e}")
        assert err <= TOL, (name, err)
    return worst


@pytest.mark.parametrize("cutoff", ["batch", "given"])
def test_backward_mid(cutoff):
    """2048 tokens, 64 experts of 512 x 512, top 8, two shared experts."""
    _check(synth.CONFIGS["mid_bf16"].with_(bt=2048), cutoff)


@pytest.mark.parametrize("bt", [1, 37])
def test_backward_ragged_and_empty_experts(bt):
    """One token (most experts unchosen: zero gradients) and 37 tokens (ragged
    expert groups, partial tiles everywhere)."""
    _check(synth.CONFIGS["mid_bf16"].with_(bt=bt), "batch")


def test_backward_without_shared_experts():
    _check(synth.CONFIGS["mid_bf16"].with_(bt=256, n_shared=0), "batch")


def test_backward_zero_tokens_writes_zero_gradients():
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=0)
    layer, _ = parity.device_layer(cfg.with_(bt=8), seed=0)
    x = torch.empty((0, cfg.d), dtype=torch.bfloat16, device="cuda")
    grads = {n: torch.full(s, 7.0, dtype=torch.float32, device="cuda")
             for n, s in layer.grad_shapes(0).items()}
    route = dict(idx=torch.empty((0, cfg.top_k), dtype=torch.int32, device="cuda"),
                 w=torch.empty((0, cfg.top_k), dtype=torch.float32, device="cuda"))
    gs = moe.MoeGrads(*(grads[n].data_ptr() if grads[n].numel() else 0
                        for n in moe.GRAD_FIELDS))
    st = moe.moe_backward(layer.cfg, layer.w, 0, 0, 0, 0, 0, gs, 0, 0,
                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for n, t in grads.items():
        if n != "dx":
            assert bool((t == 0).all()), n
    del route, x
