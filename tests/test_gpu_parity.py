"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle."""
import numpy as np
import pytest

import oracle
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


# ---- input generator ---------------------------------------------------------------

@pytest.mark.parametrize("name,routing", [("x", "normal"), ("w_gate", "normal"),
                                          ("x", "dyadic"), ("w_router", "dyadic")])
@pytest.mark.parametrize("cfg_name", ["tiny_fp32", "mid_bf16", "k3_prefill_fp8"])
def test_synth_device_matches_host(cfg_name, name, routing):
    cfg = synth.CONFIGS[cfg_name]
    if cfg_name == "k3_prefill_fp8":
        cfg = cfg.with_(bt=64, n_experts=2)
    say("synth", cfg_name, name, routing)
    dev = synth.device_layer(cfg, seed=3, routing=routing, names=[name])[name]
    torch.cuda.synchronize()
    host = synth.host_tensor(cfg, name, seed=3, routing=routing)
    got = dev.view(torch.uint8 if dev.dtype == torch.uint8 else
                   (torch.int16 if dev.dtype == torch.bfloat16 else torch.int32)).cpu().numpy()
    np.testing.assert_array_equal(got.reshape(-1).view(host.dtype), host)


# ---- routing -------------------------------------------------------------------------------

ROUTE_CASES = [("tiny_fp32", "batch"), ("tiny_fp32", "given"), ("mid_bf16", "given"),
               ("mid_bf16", "batch"), ("k3_decode_bf16", "given"),
               ("k3_prefill_bf16", "batch")]


@pytest.mark.parametrize("cfg_name,cutoff", ROUTE_CASES)
def test_route_dyadic_bit_exact(cfg_name, cutoff):
    """Dyadic x and W_r make every logit exact in fp32 on any accumulation order:
    logits, cutoffs, indices and dispatch must then equal the oracle's bit for bit."""
    cfg = synth.CONFIGS[cfg_name]
    if cfg_name == "k3_prefill_bf16":
        cfg = cfg.with_(bt=2048)
    say("route dyadic", cfg.name, cfg.bt, cutoff)
    layer, x = parity.device_layer(cfg, seed=1, routing="dyadic", cutoff=cutoff,
                                   names=["x", "w_router"])
    r = layer.route(x, want_logits=True)
    torch.cuda.synchronize()
    ref = parity.oracle_routing_full(cfg, seed=1, routing="dyadic", cutoff=cutoff)
    np.testing.assert_array_equal(parity.to_np(r["logits"]), ref["z32"])
    np.testing.assert_array_equal(parity.to_np(r["cutoff"]), ref["alpha"])
    np.testing.assert_array_equal(parity.to_np(r["idx"]), ref["idx"])
    np.testing.assert_allclose(parity.to_np(r["w"]), ref["w"], rtol=2e-6, atol=1e-7)
    d = layer.dispatch(r["idx"])
    torch.cuda.synchronize()
    for n in ("counts", "offsets", "perm", "inv_perm"):
        np.testing.assert_array_equal(parity.to_np(d[n]), ref[n], err_msg=n)


@pytest.mark.parametrize("cfg_name,cutoff", ROUTE_CASES)
def test_route_normal_inputs(cfg_name, cutoff):
    """Gaussian inputs: logits within 1e-5 of the fp64 oracle; expert sets equal
    except near ties (logged)."""
    cfg = synth.CONFIGS[cfg_name]
    if cfg_name == "k3_prefill_bf16":
        cfg = cfg.with_(bt=2048)
    say("route normal", cfg.name, cfg.bt, cutoff)
    layer, x = parity.device_layer(cfg, seed=2, cutoff=cutoff, names=["x", "w_router"])
    r = layer.route(x, want_logits=True)
    torch.cuda.synchronize()
    ref = parity.oracle_routing_full(cfg, seed=2, cutoff=cutoff)
    z = parity.to_np(r["logits"])
    dz = np.abs(z.astype(np.float64) - ref["z64"]).max()
    say(f"  max |z - z_ref| = {dz:.3e}")
    assert dz <= (1e-5 if cfg.act != "f32" else 1e-5)
    assert np.abs(parity.to_np(r["cutoff"]) - ref["alpha"]).max() <= dz
    diff, bad = parity.routing_mismatches(parity.to_np(r["idx"]), ref["idx"], ref["z32"],
                                          ref["alpha"])
    say(f"  near-tie tokens: {len(diff)}")
    assert not bad, f"tokens routed differently beyond the near-tie band: {bad[:10]}"


# ---- dispatch ----------------------------------------------------------------------------

@pytest.mark.parametrize("bt,k,E,hot", [(64, 2, 16, 0), (100, 8, 64, 0), (129, 8, 64, 6),
                                        (1, 16, 896, 0), (4096, 16, 896, 20),
                                        (16384, 16, 896, 0), (3000, 64, 64, 0),
                                        (70, 1, 1, 0)])
def test_dispatch_fixture_bit_exact(bt, k, E, hot):
    say("dispatch", bt, k, E, hot)
    import sparse_moe_layer_quantile_amd as moe
    cfg = moe.make_config(256, 64, E, k, 64, 0, 0, act="bf16")
    idx = synth.routing_fixture(bt, k, E, seed=5, hot=hot)
    layer = moe.StableLatentMoE(cfg, {})
    d = layer.dispatch(torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E)
    for n, r in zip(("counts", "offsets", "perm", "inv_perm"), ref):
        np.testing.assert_array_equal(parity.to_np(d[n]), r, err_msg=n)


# ---- whole layer, small shapes ------------------------------------------------------------

@pytest.mark.parametrize("cfg_name,cutoff,routing", [
    ("tiny_fp32", "batch", "normal"), ("tiny_fp32", "given", "normal"),
    ("tiny_fp32", "batch", "dyadic"), ("mid_bf16", "given", "normal"),
    ("mid_bf16", "batch", "dyadic")])
def test_forward_small_all_tokens(cfg_name, cutoff, routing):
    cfg = synth.CONFIGS[cfg_name]
    say("forward", cfg.name, cutoff, routing)
    layer, x = parity.device_layer(cfg, seed=0, routing=routing, cutoff=cutoff)
    y, r = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(cfg, synth.host_layer(cfg, 0, routing),
                         cutoff=oracle.BATCH if cutoff == "batch" else oracle.GIVEN)
    idx = parity.to_np(r["idx"])
    diff, bad = parity.routing_mismatches(idx, ref["idx"], ref["z32"], ref["zeta"])
    assert not bad
    if routing == "dyadic":
        assert not diff
    if not diff:
        for n in ("counts", "offsets", "perm", "inv_perm"):
            np.testing.assert_array_equal(parity.to_np(r[n]), ref[n], err_msg=n)
    else:
        parity.check_dispatch_valid(idx, *(parity.to_np(r[n]) for n in
                                           ("counts", "offsets", "perm", "inv_perm")),
                                    cfg.n_experts)
    keep = np.setdiff1d(np.arange(cfg.bt), diff)
    err = parity.normwise_err(parity.y_to_f64(y)[keep], ref["y"][keep])
    say(f"  normwise err {err:.3e} (tol {parity.tol_of(cfg)}), near ties {len(diff)}")
    assert err <= parity.tol_of(cfg)
