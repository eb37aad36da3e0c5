"""GPU tests of expert tiering (moe_tier_*): routed experts in pinned host
memory, an HBM cache of the popular ones, every expert read through the
address table.  Reading an expert from its slot or from host memory gives the
same bytes to the same kernels, so a tiered forward must equal the forward on
HBM-resident weights bit for bit, whatever the cache holds at that moment.
Tiered outputs are also checked against the oracle directly: the oracle's
routing of the same tokens and its output on them, from regenerated weights."""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _host_experts(layer, mx):
    names = ["w_gate", "w_up", "w_down"] + (["e8_gate", "e8_up", "e8_down"] if mx else [])
    return {n: layer.tensors[n].cpu().pin_memory() for n in names}


def _tiered_layer(moe, layer, tier):
    t = {n: v for n, v in layer.tensors.items()
         if n not in ("w_gate", "w_up", "w_down", "e8_gate", "e8_up", "e8_down")}
    t["expert_tab"] = tier.table
    return moe.StableLatentMoE(layer.cfg, t)


def _expert_bytes(cfg):
    """Bytes of one expert's three matrices (and E8M0 codes for MX weights)."""
    n = cfg.expert_inter * cfg.latent
    return {"bf16": 3 * 2 * n, "mxfp4": 3 * (n // 2 + n // 32),
            "mxfp8": 3 * (n + n // 32)}[cfg.weight]


def _check_against_oracle(cfg, tl, x, x_seed, y):
    """The tiered layer's routing and output on this batch against the oracle
    (weights of seed 0, tokens of x_seed), every token."""
    r = tl.route(x)
    torch.cuda.synchronize()
    xh = synth.host_tensor(cfg, "x", x_seed).reshape(cfg.bt, cfg.d)
    ref = parity.oracle_routing_full(cfg, seed=0, x=xh)
    idx = parity.to_np(r["idx"])
    diff, bad = parity.routing_mismatches(idx, ref["idx"], ref["z32"], ref["alpha"])
    assert not bad
    keep = np.setdiff1d(np.arange(cfg.bt), diff)
    yref = parity.oracle_tokens(cfg, keep, ref["idx"], ref["w"], seed=0, x=xh)
    parity.assert_close(parity.y_to_f64(y)[keep], yref, parity.tol_of(cfg), "tiered y")


def _dispatch_bufs(cfg, bt):
    E, P = cfg.n_experts, bt * cfg.top_k
    return dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                perm=torch.empty(P, dtype=torch.int32, device="cuda"),
                inv_perm=torch.empty(P, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("weight,frac,side_copy", [
    ("bf16", 0.25, True), ("bf16", 0.0, False), ("bf16", 1.0, True),
    ("mxfp4", 0.25, True), ("mxfp8", 0.25, False)])
def test_tiered_forward_equals_resident(weight, frac, side_copy):
    """Eight decode-sized batches with Zipf-skewed routing: after each forward
    the counts feed the cache, between forwards copies land and the table
    switches; every output equals the resident layer's bit for bit.  With a
    cache of a quarter of the experts the popular ones end up in HBM and serve
    most routed pairs."""
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=32, bias="zipf1.1", weight=weight,
                                          act_quant="mxfp8" if weight == "mxfp8" else "none")
    say("tier", weight, "slots", frac, "side copy stream", side_copy)
    layer, _ = parity.device_layer(cfg, seed=0)
    mx = weight != "bf16"
    n_slots = int(round(frac * cfg.n_experts))
    tier = moe.ExpertTier(layer.cfg, _host_experts(layer, mx), n_slots, decay=0.9, max_loads=8)
    tl = _tiered_layer(moe, layer, tier)
    copy = torch.cuda.Stream() if side_copy else None
    bufs = _dispatch_bufs(cfg, cfg.bt)
    for step in range(8):
        x = synth.device_layer(cfg, seed=100 + step, names=["x"])["x"]
        y_ref = layer.forward(x)
        tier.plan(copy)
        y = tl.forward(x, dispatch=bufs)
        tier.observe(bufs["counts"])
        torch.cuda.synchronize()
        same = torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        assert same, f"step {step}: tiered output differs"
        if step in (0, 7):
            _check_against_oracle(cfg, tl, x, 100 + step, y)
    for _ in range(2):  # start the last harvest, then fold it
        tier.plan(copy)
        torch.cuda.synchronize()
    st = tier.stats()
    say("  stats", st)
    assert st["forwards"] == 8 and st["harvested"] == 8
    assert st["pairs"] == 8 * cfg.bt * cfg.top_k
    assert 0 <= st["resident"] <= n_slots and st["loads"] >= st["resident"]
    if n_slots == 0:
        assert st["resident"] == 0 and st["pairs_hbm"] == 0 and st["bytes_loaded"] == 0
    else:
        assert st["resident"] > 0 and st["pairs_hbm"] > 0
        assert st["bytes_loaded"] == st["loads"] * _expert_bytes(cfg)
    if frac == 0.25:
        # Zipf(1.1) routing: the cached quarter serves most pairs once warm
        assert st["pairs_hbm"] > 0.4 * st["pairs"]
        # popularity moves (the bias rolled by half the experts): the cache
        # evicts the old favourites while outputs stay bit-exact
        moved = {n: v for n, v in layer.tensors.items()}
        moved["router_bias"] = torch.roll(layer.tensors["router_bias"], cfg.n_experts // 2)
        layer = moe.StableLatentMoE(layer.cfg, moved)
        tl = _tiered_layer(moe, layer, tier)
        for step in range(12):
            x = synth.device_layer(cfg, seed=200 + step, names=["x"])["x"]
            y_ref = layer.forward(x)
            tier.plan(copy)
            y = tl.forward(x, dispatch=bufs)
            tier.observe(bufs["counts"])
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"moved {step}"
        st2 = tier.stats()
        say("  after the shift", st2)
        assert st2["evictions"] > 0 and st2["resident"] <= n_slots
    tier.close()


def test_tiered_forward_equals_resident_k3_mxfp4_decode():
    """K3 decode with MXFP4 experts (15.7 GB of pinned host experts, 112 cached):
    four steps of fresh tokens, each equal to the resident layer's output."""
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["k3_decode_mxfp4_tier"]
    say("tier K3 mxfp4 decode")
    layer, _ = parity.device_layer(cfg, seed=0)
    tier = moe.ExpertTier(layer.cfg, _host_experts(layer, True), cfg.tier_slots, max_loads=64)
    tl = _tiered_layer(moe, layer, tier)
    bufs = _dispatch_bufs(cfg, cfg.bt)
    for step in range(4):
        x = synth.device_layer(cfg, seed=300 + step, names=["x"])["x"]
        y_ref = layer.forward(x)
        tier.plan()
        y = tl.forward(x, dispatch=bufs)
        tier.observe(bufs["counts"])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"step {step}"
        if step in (0, 3):
            _check_against_oracle(cfg, tl, x, 300 + step, y)
    st = tier.stats()
    say("  stats", st)
    assert st["resident"] > 0
    tier.close()


def test_tier_rejects_pageable_host_memory():
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=8)
    layer, _ = parity.device_layer(cfg, seed=0, names=["w_gate", "w_up", "w_down"])
    host = {n: layer.tensors[n].cpu() for n in ("w_gate", "w_up", "w_down")}  # not pinned
    with pytest.raises(moe.MoeError) as ei:
        moe.ExpertTier(layer.cfg, host, 4)
    assert ei.value.status == -1
