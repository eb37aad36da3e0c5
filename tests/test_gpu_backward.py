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


def _reduced_host_layer(cfg, tokens, idx, seed):
    """The host layer cut down to what the listed tokens touch: the dense
    weights whole, and the router rows, biases and matrices of the experts those
    tokens chose (re-indexed in ascending id).  A token's forward and its dx only
    involve its own experts, and an expert's weight gradients only the tokens
    that chose it."""
    experts = sorted({int(e) for t in tokens for e in idx[t]})
    remap = {e: i for i, e in enumerate(experts)}
    sp = synth.specs(cfg)
    lay = {n: synth.host_tensor(cfg, n, seed).reshape(sp[n].shape)
           for n in ("w_down_proj", "w_up_proj", "sh_gate", "sh_up", "sh_down")}
    lay["w_router"] = synth.host_tensor(cfg, "w_router", seed).reshape(sp["w_router"].shape)[
        experts]
    for n in ("w_gate", "w_up", "w_down"):
        lay[n] = np.stack([synth.host_matrix(cfg, n, e, seed) for e in experts])
    bias = synth.router_bias(cfg)
    if bias is not None:
        lay["router_bias"] = np.asarray(bias)[experts]
    lay["gamma"] = synth.gamma(cfg)
    sub_idx = np.array([[remap[int(e)] for e in idx[t]] for t in tokens], np.int64)
    return cfg.with_(n_experts=len(experts), bt=len(tokens)), lay, remap, sub_idx


def test_backward_k3_decode_sampled():
    """K3 decode shapes (64 tokens, 896 experts of 3072 x 3584, top 16, d 7168):
    an expert chosen by two tokens, and those tokens.  The oracle computes the
    two tokens' dx and the expert's gate / up / down / router gradients in full
    from the 32 or fewer experts they touch."""
    cfg = synth.CONFIGS["k3_decode_bf16"]
    seed = 0
    say("backward K3 decode, sampled")
    layer, x = parity.device_layer(cfg, seed=seed)
    bits, dy64 = _bf16_dy(cfg, seed + 7)
    dy = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    r = layer.route(x)
    g = layer.backward(x, dy, route=r)
    torch.cuda.synchronize()
    idx = parity.to_np(r["idx"])
    ref_route = parity.oracle_routing_full(cfg, seed=seed)
    _, bad = parity.routing_mismatches(idx, ref_route["idx"], ref_route["z32"],
                                       ref_route["alpha"])
    assert not bad, f"tokens whose expert set is not a valid top-k: {bad[:8]}"
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
    e_star = int(np.nonzero(counts == 2)[0][0])
    tokens = [int(t) for t in np.nonzero((idx == e_star).any(axis=1))[0]]
    say("  expert", e_star, "tokens", tokens)
    sub, lay, remap, sub_idx = _reduced_host_layer(cfg, tokens, idx, seed)
    p = ob.decode_layer(sub, lay)
    xs = oracle.decode(synth.host_rows(cfg, "x", tokens, seed))
    ref = ob.backward(sub, p, xs, sub_idx, dy64[tokens])
    es = remap[e_star]
    pairs = [("dx", parity.to_np(g["dx"][tokens]), ref["dx"])]
    for n in ("w_gate", "w_up", "w_down", "w_router"):
        pairs.append((n, parity.to_np(g[n][e_star]), ref[n][es]))
    for name, got, want in pairs:
        err = parity.normwise_err(got.astype(np.float64), want)
        say(f"  {name:9s} normwise {err:.2e}")
        assert err <= TOL, (name, err)
    gb = float(g["router_bias"][e_star])
    assert abs(gb - ref["router_bias"][es]) <= TOL * max(1e-30, abs(ref["router_bias"][es]))
    del layer, g


def test_backward_k3_prefill_sampled_tokens():
    """K3 prefill shapes (16384 tokens, Zipf(1.1) offsets, batch quantile
    cutoffs), the launch the backward bench times: the first and the last
    token's dx against the oracle on the experts they chose."""
    cfg = synth.CONFIGS["k3_prefill_bf16"]
    seed = 0
    say("backward K3 prefill, sampled tokens")
    layer, x = parity.device_layer(cfg, seed=seed)
    bits, dy64 = _bf16_dy(cfg, seed + 7)
    dy = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    r = layer.route(x)
    g = layer.backward(x, dy, route=r)
    torch.cuda.synchronize()
    idx = parity.to_np(r["idx"])
    tokens = [0, cfg.bt - 1]
    dx = parity.to_np(g["dx"][tokens])
    del g, layer
    torch.cuda.empty_cache()
    ref_route = parity.oracle_routing_full(cfg, seed=seed)
    _, bad = parity.routing_mismatches(idx, ref_route["idx"], ref_route["z32"],
                                       ref_route["alpha"])
    assert not bad, f"tokens whose expert set is not a valid top-k: {bad[:8]}"
    sub, lay, _, sub_idx = _reduced_host_layer(cfg, tokens, idx, seed)
    xs = oracle.decode(synth.host_rows(cfg, "x", tokens, seed))
    ref = ob.backward(sub, ob.decode_layer(sub, lay), xs, sub_idx, dy64[tokens])
    err = parity.normwise_err(dx.astype(np.float64), ref["dx"])
    say(f"  dx normwise {err:.2e}")
    assert err <= TOL


def test_backward_k3_widths_large_expert_groups():
    """K3 widths (d 7168, L 3584, I 3072, two shared of 3072, Zipf(1.1)
    offsets, batch cutoffs) with prefill-sized expert groups: 1024 tokens over
    32 experts, top 16, about 512 pairs an expert (K3 prefill has about 293).
    The least-loaded expert's gate / up / down / router gradients in full and
    the dx of every token that chose it, against the oracle on those tokens
    and the experts they touch."""
    cfg = synth.CONFIGS["k3_prefill_bf16"].with_(bt=1024, n_experts=32)
    seed = 0
    say("backward K3 widths, 32 experts, 1024 tokens")
    layer, x = parity.device_layer(cfg, seed=seed)
    bits, dy64 = _bf16_dy(cfg, seed + 7)
    dy = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    r = layer.route(x)
    g = layer.backward(x, dy, route=r)
    torch.cuda.synchronize()
    idx = parity.to_np(r["idx"])
    ref_route = parity.oracle_routing_full(cfg, seed=seed)
    _, bad = parity.routing_mismatches(idx, ref_route["idx"], ref_route["z32"],
                                       ref_route["alpha"])
    assert not bad, f"tokens whose expert set is not a valid top-k: {bad[:8]}"
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
    e_star = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    tokens = [int(t) for t in np.nonzero((idx == e_star).any(axis=1))[0]]
    say("  expert", e_star, "tokens", len(tokens))
    got = {"dx": parity.to_np(g["dx"][tokens])}
    for n in ("w_gate", "w_up", "w_down", "w_router"):
        got[n] = parity.to_np(g[n][e_star])
    gb = float(g["router_bias"][e_star])
    del g, layer
    torch.cuda.empty_cache()
    sub, lay, remap, sub_idx = _reduced_host_layer(cfg, tokens, idx, seed)
    xs = oracle.decode(synth.host_rows(cfg, "x", tokens, seed))
    ref = ob.backward(sub, ob.decode_layer(sub, lay), xs, sub_idx, dy64[tokens])
    es = remap[e_star]
    for name in got:
        want = ref[name] if name == "dx" else ref[name][es]
        err = parity.normwise_err(got[name].astype(np.float64), want)
        say(f"  {name:9s} normwise {err:.2e}")
        assert err <= TOL, (name, err)
    assert abs(gb - ref["router_bias"][es]) <= TOL * max(1e-30, abs(ref["router_bias"][es]))
