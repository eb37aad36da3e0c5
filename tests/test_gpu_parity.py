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
@pytest.mark.parametrize("cfg_name", ["tiny_fp32", "mid_bf16", "k3_prefill_fp8",
                                      "k3_prefill_mxfp4", "k3_prefill_mxfp8"])
def test_synth_device_matches_host(cfg_name, name, routing):
    cfg = synth.CONFIGS[cfg_name]
    if cfg_name.startswith("k3_prefill"):
        cfg = cfg.with_(bt=64, n_experts=2)
    say("synth", cfg_name, name, routing)
    lay = synth.device_layer(cfg, seed=3, routing=routing, names=[name])
    dev = lay[name]
    torch.cuda.synchronize()
    host = synth.host_tensor(cfg, name, seed=3, routing=routing)
    got = dev.view(torch.uint8 if dev.dtype == torch.uint8 else
                   (torch.int16 if dev.dtype == torch.bfloat16 else torch.int32)).cpu().numpy()
    np.testing.assert_array_equal(got.reshape(-1).view(host.dtype), host)
    if "scale:" + name in lay:  # block scales / E8M0 codes too
        hs = synth.host_scales(cfg, name, seed=3)
        np.testing.assert_array_equal(lay["scale:" + name].cpu().numpy(), hs)


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
    say(f"  near ties {len(diff)}")
    parity.assert_close(parity.y_to_f64(y)[keep], ref["y"][keep], parity.tol_of(cfg), "y")


@pytest.mark.parametrize("bt,cutoff", [(4096, "batch"), (64, "given"), (100, "batch")])
def test_forward_fp8_weights_mid(bt, cutoff):
    """fp8 e4m3 weights with 128 x 128 block scales at the mid shapes: the
    prefill-sized batch runs the 320-row grouped tiles, the short ones the
    32-row tiles and split-K dense GEMMs."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="fp8", bt=bt)
    say("forward fp8", bt, cutoff)
    layer, x = parity.device_layer(cfg, seed=0, cutoff=cutoff)
    y, r = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(cfg, synth.host_layer(cfg, 0),
                         cutoff=oracle.BATCH if cutoff == "batch" else oracle.GIVEN)
    diff, bad = parity.routing_mismatches(parity.to_np(r["idx"]), ref["idx"], ref["z32"],
                                          ref["zeta"])
    assert not bad
    keep = np.setdiff1d(np.arange(cfg.bt), diff)
    say(f"  near ties {len(diff)}")
    parity.assert_close(parity.y_to_f64(y)[keep], ref["y"][keep], parity.tol_of(cfg), "y")


@pytest.mark.parametrize("bt,cutoff,shape", [(4096, "batch", None), (64, "given", None),
                                             (100, "batch", None), (300, "batch", (640, 384)),
                                             (16, "given", None), (8, "batch", (640, 384))])
def test_forward_mxfp4_experts_mid(bt, cutoff, shape):
    """MXFP4 routed experts (E2M1 codes, E8M0 scales per 32) at the mid shapes:
    the prefill-sized batch runs the 320-row grouped tiles, the 64-token one
    the 32-row tiles with the deep ring, 16 and 8 tokens (two rows an expert)
    the 8-row short tiles, the others the 192-row tiles; the (640, 384) cases
    have a partial N tile in the down GEMM and K ranges of 20 and 12 scale
    blocks."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4", bt=bt)
    if shape is not None:
        cfg = cfg.with_(latent=shape[0], expert_inter=shape[1])
    say("forward mxfp4", bt, cutoff, cfg.latent, cfg.expert_inter)
    _mxfp4_check(cfg, cutoff)


@pytest.mark.parametrize("shape_id", ["0", "1", "6", "7", "7-bk128"])
def test_forward_mxfp4_every_tile_shape(shape_id, monkeypatch):
    """Each MXFP4 tile shape (forced) on one batch of about 25 rows an expert:
    several M tiles an expert for the short shapes, a partial one for the long;
    the 8-row tile with its 256-wide K tiles and with 128-wide ones."""
    monkeypatch.setenv("MOE_GEMM_MX4", shape_id.split("-")[0])
    if shape_id.endswith("bk128"):
        monkeypatch.setenv("MOE_GEMM_MX4_BK128", "1")
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4", bt=200)
    say("forward mxfp4 forced shape", shape_id)
    _mxfp4_check(cfg, "batch")


def _mxfp4_check(cfg, cutoff, elem_floor=parity.ELEM_FLOOR_ASSERT):
    layer, x = parity.device_layer(cfg, seed=0, cutoff=cutoff)
    y, r = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(cfg, synth.host_layer(cfg, 0),
                         cutoff=oracle.BATCH if cutoff == "batch" else oracle.GIVEN)
    diff, bad = parity.routing_mismatches(parity.to_np(r["idx"]), ref["idx"], ref["z32"],
                                          ref["zeta"])
    assert not bad
    keep = np.setdiff1d(np.arange(cfg.bt), diff)
    say(f"  near ties {len(diff)}")
    parity.assert_close(parity.y_to_f64(y)[keep], ref["y"][keep], parity.tol_of(cfg), "y",
                        elem_floor=elem_floor)


# ---- MX FP8 expert inputs (MXFP4 weights, block-scaled MFMA) --------------------------------

def _mx8_inputs(n, seed):
    """n bf16 values (uint16 bit patterns), blocks of 32 drawn from a mix that
    reaches every branch of the conversion: normal data at scales 2^-133 ..
    2^120 (bf16 subnormal to near the top of its range), all-zero blocks,
    blocks with one non-zero, blocks with signed zeros, and values that sit
    exactly on e4m3 rounding midpoints after scaling."""
    rng = np.random.default_rng(seed)
    nb = n // 32
    v = rng.normal(size=(nb, 32)).astype(np.float32)
    kind = rng.integers(0, 8, size=nb)
    scale = np.ldexp(np.float32(1), rng.integers(-133, 121, size=nb)).astype(np.float32)
    v *= scale[:, None]
    v[kind == 0] = 0.0
    v[kind == 1] = -0.0
    one = kind == 2
    v[one, 1:] = 0.0
    # midpoints: m.5 steps of a 3-bit mantissa at the block's scale
    mid = kind == 3
    m = rng.integers(0, 16, size=(int(mid.sum()), 32)).astype(np.float32)
    e = rng.integers(-10, 9, size=(int(mid.sum()), 32))
    sign = np.where(rng.random((int(mid.sum()), 32)) < 0.5, -1, 1).astype(np.float32)
    v[mid] = sign * np.ldexp((8 + m + 0.5) / 8, e).astype(np.float32) * 0.5
    # bf16 of each value (round to nearest even; no overflow at these scales)
    u = v.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16).reshape(-1)


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("n,seed", [(32, 0), (32 * 37, 1), (32 * 1000 + 32 * 3, 2),
                                     ((1 << 21) + 32 * 5, 3)])
def test_mx8_quantize_bit_exact(n, seed):
    """The MX FP8 quantiser's codes and E8M0 scales equal the oracle's bit for
    bit (its input is bf16, exact in the oracle's fp64; both compute the same
    rounding), over one block, ragged grids and a 2M-element input."""
    import sparse_moe_layer_quantile_amd as moe
    say("mx8 quantize", n, seed)
    bits = _mx8_inputs(n, seed)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    codes, scales = moe.mx8_quantize(x)
    torch.cuda.synchronize()
    rc, rs = oracle.mx8_quantize(_bf16_to_f64(bits))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.nonzero(got != rc)[0]
    assert bad.size == 0, (f"{bad.size} codes differ, first at {bad[:4]}: got "
                           f"{got[bad[:4]]} want {rc[bad[:4]]} from {_bf16_to_f64(bits)[bad[:4]]}")


def test_mx8_quantize_argument_errors():
    import sparse_moe_layer_quantile_amd as moe
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(64, dtype=torch.uint8, device="cuda")
    s = torch.empty(2, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert moe.moe_mx8_quantize(x.data_ptr(), 48, c.data_ptr(), s.data_ptr(), stream) == -1
    assert moe.moe_mx8_quantize(x.data_ptr(), -32, c.data_ptr(), s.data_ptr(), stream) == -1
    assert moe.moe_mx8_quantize(0, 32, c.data_ptr(), s.data_ptr(), stream) == -1
    assert moe.moe_mx8_quantize(x.data_ptr() + 2, 32, c.data_ptr(), s.data_ptr(), stream) == -1
    assert moe.moe_mx8_quantize(0, 0, 0, 0, stream) == 0


@pytest.mark.parametrize("bt,cutoff,shape", [(4096, "batch", None), (64, "given", None),
                                             (300, "batch", (640, 384)), (8, "batch", None)])
def test_forward_mxfp4_mx8_inputs_mid(bt, cutoff, shape):
    """MXFP4 experts with MX FP8 inputs (x_lat and h quantised in the layer, the
    block-scaled MFMA): the oracle quantises its fp64 x_lat and h the same
    way.  256-row tiles: several per expert at 4096 tokens, a partial one
    at 64; (640, 384) has a partial N tile in the down GEMM and K ranges of
    five and three 128-wide K tiles."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4", act_quant="mxfp8", bt=bt)
    if shape is not None:
        cfg = cfg.with_(latent=shape[0], expert_inter=shape[1])
    say("forward mxfp4 + mx8 inputs", bt, cutoff, cfg.latent, cfg.expert_inter)
    _mxfp4_check(cfg, cutoff)


@pytest.mark.parametrize("weight", ["mxfp4", "mxfp8"])
def test_forward_mx8_inputs_against_codes_on_exact_values(weight, monkeypatch):
    """The same layers against an oracle that decides every MX FP8 code on the
    exact fp64 x_lat and h (the plain MX conversion) instead of on their bf16
    roundings: the two oracles differ only where a bf16 rounding moves a value
    across a code boundary, and the GPU stays within the fp8 tolerance of
    both."""
    monkeypatch.setattr(oracle, "MX_CODES_ON_BF16", False)
    cfg = synth.CONFIGS["mid_bf16"].with_(weight=weight, act_quant="mxfp8", bt=4096)
    say("forward mx8 inputs, oracle codes on exact values", weight)
    # normwise only: a code decided on a value one bf16 rounding away moves by a
    # whole e4m3 step (about 6 %), and the two oracles differ by 2-5 % of an
    # expert's largest output (measured on the CPU)
    _mxfp4_check(cfg, "batch", elem_floor=None)


@pytest.mark.parametrize("weight", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("bt", [1, 2, 63, 129])
def test_forward_mx8_inputs_ragged_batches(weight, bt):
    """MX FP8 expert inputs on ragged batches: one row in most experts' tiles,
    a single token (BATCH mode: the k lowest ids), partial 32-row sub-blocks."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight=weight, act_quant="mxfp8", bt=bt)
    say("forward mx8 inputs ragged", weight, bt)
    _mxfp4_check(cfg, "batch")


@pytest.mark.parametrize("shape_id", ["11", "12", "13"])
def test_forward_mxfp4_mx8_every_tile_shape(shape_id, monkeypatch):
    """Each tile shape of the block-scaled engine (forced): 256, 320 and 192 rows
    on a batch of 512 rows an expert (several M tiles each, a ragged last one)."""
    monkeypatch.setenv("MOE_GEMM_A8", shape_id)
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4", act_quant="mxfp8", bt=4096)
    say("forward mxfp4 + mx8 inputs, forced shape", shape_id)
    _mxfp4_check(cfg, "batch")


@pytest.mark.parametrize("bt,cutoff,shape", [(4096, "batch", None), (64, "given", None),
                                             (300, "batch", (640, 384)), (8, "batch", None)])
def test_forward_mxfp8_experts_mid(bt, cutoff, shape):
    """MX FP8 experts (e4m3 codes, E8M0 scales per 32) reading MX FP8 inputs: both
    operands on the block-scaled MFMA (W8A8).  The 4096-token batch runs the
    320-row tiles, the others the 192-row ones; (640, 384) has a partial N tile
    in the down GEMM."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp8", act_quant="mxfp8", bt=bt)
    if shape is not None:
        cfg = cfg.with_(latent=shape[0], expert_inter=shape[1])
    say("forward mxfp8 experts", bt, cutoff, cfg.latent, cfg.expert_inter)
    _mxfp4_check(cfg, cutoff)


@pytest.mark.parametrize("shape_id", ["12", "14", "15"])
def test_forward_mxfp8_every_tile_shape(shape_id, monkeypatch):
    """Each tile shape of the W8A8 engine (forced): 320, 256 and 192 rows."""
    monkeypatch.setenv("MOE_GEMM_A8", shape_id)
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp8", act_quant="mxfp8", bt=4096)
    say("forward mxfp8 experts, forced shape", shape_id)
    _mxfp4_check(cfg, "batch")


# ---- edge cases ----------------------------------------------------------------------------

def _small_forward_check(cfg, cutoff, seed=0, alpha=None, routing="normal"):
    layer, x = parity.device_layer(cfg, seed=seed, cutoff=cutoff, alpha=alpha,
                                   routing=routing)
    y, r = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(cfg, synth.host_layer(cfg, seed, routing),
                         cutoff=oracle.BATCH if cutoff == "batch" else oracle.GIVEN,
                         alpha=alpha)
    diff, bad = parity.routing_mismatches(parity.to_np(r["idx"]), ref["idx"], ref["z32"],
                                          ref["zeta"])
    assert not bad
    keep = np.setdiff1d(np.arange(cfg.bt), diff)
    say(f"  {cfg.name} bt={cfg.bt} {cutoff}: near ties {len(diff)}")
    parity.assert_close(parity.y_to_f64(y)[keep], ref["y"][keep], parity.tol_of(cfg), "y")
    return r, ref


@pytest.mark.parametrize("bt", [1, 2, 63, 100, 129, 1000])
@pytest.mark.parametrize("cutoff", ["batch", "given"])
def test_forward_ragged_batches(bt, cutoff):
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=bt)
    say("ragged", bt, cutoff)
    r, ref = _small_forward_check(cfg, cutoff)
    if bt == 1 and cutoff == "batch":
        # m = 1: every cutoff equals the token's own logit, all r = 0, so the
        # k lowest expert ids are chosen
        assert (parity.to_np(r["idx"]) == np.arange(cfg.top_k)).all()


def test_forward_given_nonzero_cutoffs():
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=512)
    alpha = np.random.default_rng(3).normal(size=cfg.n_experts).astype(np.float32)
    say("given cutoffs")
    r, ref = _small_forward_check(cfg, "given", alpha=alpha)
    np.testing.assert_array_equal(parity.to_np(r["cutoff"]), alpha)


@pytest.mark.parametrize("n_shared,shared_inter", [(0, 0), (1, 256), (3, 128)])
def test_forward_shared_expert_counts(n_shared, shared_inter):
    cfg = synth.CONFIGS["mid_bf16"].with_(bt=300, n_shared=n_shared, shared_inter=shared_inter)
    say("shared", n_shared, shared_inter)
    _small_forward_check(cfg, "batch")


def test_forward_k_equals_E_and_single_expert():
    for cfg in (synth.CONFIGS["mid_bf16"].with_(bt=200, n_experts=8, top_k=8),
                synth.CONFIGS["mid_bf16"].with_(bt=200, n_experts=1, top_k=1)):
        say("k=E", cfg.n_experts)
        _small_forward_check(cfg, "batch")


def test_forward_bt_zero_is_a_no_op():
    cfg = synth.CONFIGS["mid_bf16"]
    layer, x = parity.device_layer(cfg, seed=0)
    y = layer.forward(x[:0])
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.d)


def test_forward_deterministic_and_stream_independent():
    cfg = synth.CONFIGS["mid_bf16"]
    layer, x = parity.device_layer(cfg, seed=0, cutoff="batch")
    y1 = layer.forward(x).clone()
    side = torch.cuda.Stream()
    y2 = layer.forward(x, shared_stream=side).clone()
    y3 = layer.forward(x, shared_stream=side).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y2, y3)


def test_forward_output_bounded_for_large_inputs():
    """SiTU-GLU caps the expert activations: x scaled x100 still gives finite
    outputs matching the oracle."""
    cfg = synth.CONFIGS["tiny_fp32"]
    layer, x = parity.device_layer(cfg, seed=0, cutoff="batch")
    y = layer.forward(x * 100.0)
    torch.cuda.synchronize()
    lay = synth.host_layer(cfg, 0)
    lay["x"] = (lay["x"] * np.float32(100.0)).astype(np.float32)
    ref = oracle.forward(cfg, lay, cutoff=oracle.BATCH)
    assert torch.isfinite(y).all()
    parity.assert_close(parity.y_to_f64(y), ref["y"], parity.tol_of(cfg), "y of x * 100")


def test_error_codes():
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["mid_bf16"]
    layer, x = parity.device_layer(cfg, seed=0)
    y = torch.empty((cfg.bt, cfg.d), dtype=x.dtype, device="cuda")
    ws = layer.workspace(cfg.bt)
    stream = torch.cuda.current_stream().cuda_stream
    st = moe.moe_forward(layer.cfg, layer.w, x.data_ptr(), cfg.bt, y.data_ptr(), None, None,
                         ws.data_ptr(), 1024, stream)
    assert st == -3
    st = moe.moe_forward(layer.cfg, moe.MoeWeights(), x.data_ptr(), cfg.bt, y.data_ptr(), None,
                         None, ws.data_ptr(), ws.numel(), stream)
    assert st == -1
    bad = parity.abi_config(cfg.with_(latent=500))
    st = moe.moe_forward(bad, layer.w, x.data_ptr(), cfg.bt, y.data_ptr(), None, None,
                         ws.data_ptr(), ws.numel(), stream)
    assert st == -2
    st = moe.moe_forward(layer.cfg, layer.w, x.data_ptr(), cfg.bt, y.data_ptr(), None, None,
                         ws.data_ptr() + 8, ws.numel() - 8, stream)
    assert st == -3
