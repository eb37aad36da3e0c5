"""GPU parity at the full K3 layer shapes (d=7168, L=3584, 896 experts, top 16,
I=3072, 2 shared experts of 3072), in the launch configuration the benchmark
times (one stream), and the prefill case on two streams as well.  Routing is
checked on every token against the full-batch oracle; the layer output on every
token (decode) or on a seeded sample of tokens the oracle computes one by one
(prefill)."""
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
    yield
    torch.cuda.empty_cache()


def _selection_on_gpu_logits(cfg, got):
    """Routing stage 1, free of any tolerance: the oracle's quantile, top-k and
    dispatch run on the GPU's own fp32 logits of the whole batch, and the
    cutoffs, expert ids, counts, offsets and both permutations must equal the
    GPU's bit for bit; the combine weights are the sigmoid of the same logits."""
    z = got["logits"]
    if cfg.cutoff == "batch":
        alpha = oracle.quantile(z, cfg.quantile_rank)
    else:
        alpha = np.zeros(cfg.n_experts, np.float32)
    np.testing.assert_array_equal(got["cutoff"], alpha, err_msg="cutoffs")
    idx, w = oracle.topk(z, cfg.top_k, alpha=alpha)
    np.testing.assert_array_equal(got["idx"], idx, err_msg="expert ids")
    for n, v in zip(("counts", "offsets", "perm", "inv_perm"), oracle.dispatch(idx, cfg.n_experts)):
        np.testing.assert_array_equal(got[n], v, err_msg=n)
    np.testing.assert_allclose(got["w"], w, rtol=2e-6, atol=0)
    say(f"  stage 1: cutoffs, ids and dispatch bit-exact on {cfg.bt} tokens")


def _run_k3(cfg_name, n_sample, seed=0, two_streams=False):
    cfg = synth.CONFIGS[cfg_name]
    say("k3 parity", cfg.name, "bt", cfg.bt, "sample", n_sample, "two streams", two_streams)
    layer, x = parity.device_layer(cfg, seed=seed)
    side = torch.cuda.Stream() if two_streams else None
    y, r = layer.forward(x, shared_stream=side, return_routing=True)
    torch.cuda.synchronize()
    yg = parity.y_to_f64(y)
    got = {n: parity.to_np(v) for n, v in r.items()}
    del layer, x, y, r
    torch.cuda.empty_cache()
    say("  gpu done; oracle selection on the GPU's logits")
    _selection_on_gpu_logits(cfg, got)
    say("  oracle routing")
    ref = parity.oracle_routing_full(cfg, seed=seed)
    dz = np.abs(got["logits"].astype(np.float64) - ref["z64"]).max()
    say(f"  max |z - z_ref| = {dz:.3e}")
    assert dz <= 1e-5
    assert np.abs(got["cutoff"] - ref["alpha"]).max() <= dz
    diff, bad = parity.routing_mismatches(got["idx"], ref["idx"], ref["z32"], ref["alpha"])
    say(f"  near-tie tokens {len(diff)}: {diff[:8]}")
    assert not bad, f"routing beyond the near-tie band on tokens {bad[:8]}"
    if not diff:
        for n in ("counts", "offsets", "perm", "inv_perm"):
            np.testing.assert_array_equal(got[n], ref[n], err_msg=n)
    else:
        parity.check_dispatch_valid(got["idx"], got["counts"], got["offsets"], got["perm"],
                                    got["inv_perm"], cfg.n_experts)
    np.testing.assert_allclose(got["w"], ref["w"], rtol=1e-5, atol=1e-6)
    rng = np.random.default_rng(seed + 1)
    pool = np.setdiff1d(np.arange(cfg.bt), diff)
    tokens = np.sort(rng.choice(pool, size=min(n_sample, pool.size), replace=False))
    if cfg.bt > 1:  # always include the first and the last token (tile edges)
        tokens = np.unique(np.concatenate([tokens, [pool[0], pool[-1]]]))
    say(f"  oracle y on {len(tokens)} tokens")
    yref = parity.oracle_tokens(cfg, tokens, ref["idx"], ref["w"], seed=seed, x=ref["x"])
    parity.assert_close(yg[tokens], yref, parity.tol_of(cfg), "y")
    return cfg, got


def test_k3_decode_all_tokens():
    cfg, got = _run_k3("k3_decode_bf16", n_sample=64)
    say("  experts touched", int((got["counts"] > 0).sum()))


@pytest.mark.parametrize("two_streams", [False, True])
def test_k3_prefill_zipf_batch_cutoffs(two_streams):
    cfg, got = _run_k3("k3_prefill_bf16", n_sample=10, two_streams=two_streams)
    # the batch cutoffs balance the Zipf-skewed load: every expert near bt*k/E
    mean = cfg.bt * cfg.top_k / cfg.n_experts
    say(f"  load max/mean {got['counts'].max() / mean:.3f} min/mean {got['counts'].min() / mean:.3f}")
    assert got["counts"].max() < 1.5 * mean and got["counts"].min() > 0.5 * mean


def test_k3_prefill_fp8_weights():
    _run_k3("k3_prefill_fp8", n_sample=10)


def test_k3_decode_mxfp4_experts():
    """K3 decode with the routed experts in MXFP4 (the weight format of the
    released checkpoint), every token checked."""
    _run_k3("k3_decode_mxfp4", n_sample=64)


def test_k3_prefill_mxfp4_experts():
    _run_k3("k3_prefill_mxfp4", n_sample=10)


def test_k3_prefill_mxfp4_mx8_inputs():
    """MXFP4 experts with their inputs quantised to MX FP8 (block-scaled MFMA)."""
    _run_k3("k3_prefill_mxfp4_a8", n_sample=10)


def test_k3_prefill_mxfp8_experts():
    """MX FP8 experts with MX FP8 inputs (W8A8 on the block-scaled MFMA)."""
    _run_k3("k3_prefill_mxfp8", n_sample=10)


@pytest.mark.parametrize("weight", ["mxfp4", "mxfp8"])
def test_k3_decode_mx8_inputs(weight):
    """K3 decode (64 tokens) with MX FP8 expert inputs, every token checked."""
    _run_k3("k3_decode_mxfp4_a8" if weight == "mxfp4" else "k3_decode_mxfp8", n_sample=64)


def test_k3_expert_parallel_share():
    """One GPU's share of 8-way expert parallelism: 112 experts with about 2341
    rows each, so every expert spans several M tiles of the grouped GEMMs."""
    cfg, got = _run_k3("k3_ep8_share_bf16", n_sample=10)
    say(f"  rows per expert: min {got['counts'].min()} max {got['counts'].max()}")
    assert got["counts"].min() > 320  # several M tiles per expert
