"""The measurement harness on the CPU: its algorithmic work against the totals
the workloads' own arithmetic gives, its roofline choice, its refusal of more
than one GPU, the near-tie count, and that counters taken on other kernel
sources are not reported."""
import numpy as np

import bench
import synth


def _sum_flops(cfg, touched):
    return sum(f for f, _ in bench.phase_work(cfg, touched).values())


def _layer_flops(cfg):
    """2 bt d E + 2 bt d L + 2 P 3 L I + 2 bt L d + 2 bt 3 d S I_s: router,
    W_down, the experts' three matrices, W_up and the shared experts' three."""
    bt, d, L, E = cfg.bt, cfg.d, cfg.latent, cfg.n_experts
    P, I, S, Is = cfg.bt * cfg.top_k, cfg.expert_inter, cfg.n_shared, cfg.shared_inter
    return 2 * bt * d * E + 2 * bt * d * L + 2 * P * 3 * L * I + 2 * bt * L * d + 2 * bt * 3 * d * S * Is


def test_phase_flops_sum_to_the_layer():
    for name in ("tiny_fp32", "mid_bf16", "k3_decode_bf16", "k3_prefill_bf16", "k3_prefill_fp8"):
        cfg = synth.CONFIGS[name]
        assert _sum_flops(cfg, cfg.n_experts) == _layer_flops(cfg), name


def test_headline_totals():
    # K3 prefill (bt 16384): 23 540.7 GFLOP; the fp8 batch (bt 8192) half of it
    assert abs(_sum_flops(synth.CONFIGS["k3_prefill_bf16"], 896) - 23540.7e9) < 0.1e9
    assert abs(_sum_flops(synth.CONFIGS["k3_prefill_fp8"], 896) - 11770.4e9) < 0.1e9
    assert abs(_sum_flops(synth.CONFIGS["mid_bf16"], 64) - 172.9e9) < 0.1e9


def test_expert_weight_bytes_count_each_touched_expert_once():
    cfg = synth.CONFIGS["k3_decode_bf16"]
    w = bench.phase_work(cfg, 613)
    w2 = bench.phase_work(cfg, 614)
    per_expert = 3 * cfg.latent * cfg.expert_inter * 2
    got = (w2["expert_gateup"][1] + w2["expert_down"][1]) - (w["expert_gateup"][1] + w["expert_down"][1])
    assert got == per_expert


def test_roofline_bound_and_fractions():
    r = bench.roofline_of("expert_gateup", 11.544872091648e12, 41.18806528e9, 12.3)
    assert r["bound"] == "hbm"  # 280 FLOP/B, under the 312 FLOP/B ridge
    assert abs(r["frac"] - r["hbm_frac"]) < 1e-12
    assert abs(r["hbm_frac"] - 41.18806528e9 / 12.3e-3 / 8e12) < 1e-9
    r = bench.roofline_of("x", 2.5e12, 1e9, 1.0)
    assert r["bound"] == "mfma" and abs(r["frac"] - 1.0) < 1e-9


def test_backward_flops_at_k3_prefill():
    assert abs(bench.backward_flops(synth.CONFIGS["k3_prefill_bf16"]) - 68.1e12) < 0.05e12


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one MI355X" in capsys.readouterr().err


def test_near_tie_count_and_load():
    cfg = synth.CONFIGS["tiny_fp32"].with_(bt=3, n_experts=4, top_k=2)
    z = np.array([[3.0, 1.0, 1.0, -2.0],    # 2nd and 3rd best equal: a near tie
                  [3.0, 2.0, 1.0, 0.0],
                  [0.5, 0.4, 0.3, 0.2]], np.float32)
    res = {"counts": np.array([3, 2, 1, 0]), "logits": z, "cutoff": np.zeros(4, np.float32)}
    st = bench.routing_stats(cfg, res)
    assert st["near_tie_tokens"] == 1
    assert st["load_max_over_mean"] == 3 / (3 * 2 / 4)
    assert st["load_min_over_mean"] == 0.0


def test_counters_of_other_kernel_sources_are_not_reported(monkeypatch):
    traffic, method = bench.measured_traffic("k3_prefill_bf16", "expert_gateup")
    if traffic is not None:  # the committed counters match these sources
        assert method.startswith("TCC_EA0_RDREQ")
        assert 40e9 < traffic < 50e9
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000000000000000")
    assert bench.measured_traffic("k3_prefill_bf16", "expert_gateup") == (None, None)
