"""The seeded input generator: Philox known answers, encodings, statistics."""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth


def _philox(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    synth.lib_host().synth_philox_host(c, k)
    return list(c)


def test_philox_known_answers():
    """Known-answer vectors published with Random123 for philox4x32_10."""
    assert _philox([0, 0, 0, 0], [0, 0]) == [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]
    assert _philox([0xffffffff] * 4, [0xffffffff] * 2) == [0x408f276d, 0x41c83b0e,
                                                            0xa20bc7c6, 0x6d5451fd]
    assert _philox([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344],
                   [0xa4093822, 0x299f31d0]) == [0xd16cfe09, 0x94fdcceb, 0x5001e420,
                                                 0x24126ea1]


def test_bf16_encoding_round_to_nearest_even():
    enc = synth.lib_host().synth_bf16_host
    assert enc(1.0) == 0x3F80
    assert enc(1.0 + 2 ** -8) == 0x3F80          # tie -> even
    assert enc(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert enc(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert enc(-2.0) == 0xC000


def test_e4m3_encoding_roundtrip_and_rounding():
    enc = synth.lib_host().synth_e4m3_host
    for code in list(range(0x7F)) + list(range(0x80, 0xFF)):
        v = oracle.e4m3_to_double(code)
        if code == 0x80:
            continue  # -0 encodes as 0x80 too, checked below
        assert enc(v) == code, hex(code)
    assert enc(-0.0) == 0x80
    assert enc(1000.0) == 0x7E and enc(-1000.0) == 0xFE      # saturating
    assert enc(1.0625) == 0x38                               # tie 1.0 / 1.125 -> even
    assert enc(1.1875) == 0x3A                               # tie 1.125 / 1.25 -> even
    assert enc(2 ** -10) == 0x00 and enc(3 * 2 ** -10) == 0x02  # subnormal ties
    assert enc(460.0) == 0x7E


def test_e2m1_encoding_roundtrip_and_rounding():
    enc = synth.lib_host().synth_e2m1_host
    vals = [oracle.e2m1_to_double(c) for c in range(16)]
    for code in range(16):
        if code == 8:
            continue  # -0 encodes as 8 too, checked below
        assert enc(vals[code]) == code, hex(code)
    assert enc(-0.0) == 8
    assert enc(100.0) == 7 and enc(-100.0) == 15 and enc(7.0) == 7  # saturating
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0,
    # 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0
    for v, c in ((0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)):
        assert enc(v) == c and enc(-v) == (c | 8 if c else 8), v
    # nearest grid point (brute force) for random values
    rng = np.random.default_rng(3)
    grid = np.array(vals[:8])
    for x in np.float32(rng.normal(0, 3, 4000)):
        d = np.abs(grid - min(abs(float(x)), 6.0))
        assert enc(float(x)) & 7 == int(np.argmin(d)), x


def test_mxfp4_layer_packing_and_scales():
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4", n_experts=2, latent=256,
                                          expert_inter=128)
    sp = synth.specs(cfg)
    assert sp["w_gate"].shape == (2, 128, 128) and sp["w_down"].shape == (2, 256, 64)
    assert sp["w_down_proj"].dtype == synth.BF16 and sp["sh_up"].dtype == synth.BF16
    codes = synth.host_matrix(cfg, "w_gate", 1)
    # byte i of the matrix holds draws 2i and 2i + 1 of the tensor, encoded
    kind, scale, _ = synth.draw_params(cfg, "w_gate")
    enc = synth.lib_host().synth_e2m1_host
    off = sp["w_gate"].mat_rows * sp["w_gate"].mat_cols  # first element of expert 1
    for i in (0, 1, 77, codes.size - 1):
        lo = synth.lib_host().synth_normal_int_host(0, synth.TID["w_gate"], off + 2 * i)
        hi = synth.lib_host().synth_normal_int_host(0, synth.TID["w_gate"], off + 2 * i + 1)
        want = enc(float(np.float32(lo) * np.float32(scale))) | (
            enc(float(np.float32(hi) * np.float32(scale))) << 4)
        assert codes.ravel()[i] == want
    sc = synth.host_scales(cfg, "w_gate")
    assert sc.dtype == np.uint8 and sc.shape == (2, 128, 8)
    c = synth.mx_centre(cfg, "w_gate")
    assert set(np.unique(sc)) == {c - 1, c, c + 1}
    deq = oracle.decode(codes, sc[1])
    assert abs(deq.std() * math.sqrt(cfg.latent) - 1.0) < 0.45


def test_mxfp8_layer_codes_and_scales():
    """MX FP8 experts: one e4m3 code a weight (the draw at standard deviation 16,
    rounded as the fp8 path rounds), E8M0 codes per row and 32 inputs around a
    centre that gives decoded weights ~ 1/sqrt(fan_in); dense weights bf16."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp8", act_quant="mxfp8", n_experts=2,
                                          latent=256, expert_inter=128)
    sp = synth.specs(cfg)
    assert sp["w_gate"].shape == (2, 128, 256) and sp["w_down"].shape == (2, 256, 128)
    assert sp["w_gate"].dtype == synth.MXFP8 and sp["w_down_proj"].dtype == synth.BF16
    codes = synth.host_matrix(cfg, "w_gate", 1)
    assert codes.dtype == np.uint8 and codes.shape == (128, 256)
    kind, scale, _ = synth.draw_params(cfg, "w_gate")
    off = sp["w_gate"].mat_rows * sp["w_gate"].mat_cols  # first element of expert 1
    for i in (0, 1, 77, codes.size - 1):
        v = synth.lib_host().synth_normal_int_host(0, synth.TID["w_gate"], off + i)
        want = oracle.double_to_e4m3(float(np.float32(v) * np.float32(scale)))
        assert codes.ravel()[i] == want, i
    sc = synth.host_scales(cfg, "w_gate")
    assert sc.dtype == np.uint8 and sc.shape == (2, 128, 8)
    c = synth.mx_centre(cfg, "w_gate")
    assert set(np.unique(sc)) == {c - 1, c, c + 1}
    deq = oracle.decode(codes, sc[1])
    assert abs(deq.std() * math.sqrt(cfg.latent) - 1.0) < 0.45


def test_normal_draw_statistics():
    cfg = synth.CONFIGS["tiny_fp32"]
    x = synth.host_tensor(cfg, "x")
    assert abs(x.mean()) < 0.03 and abs(x.std() - 1.0) < 0.02
    assert np.abs(x).max() <= synth.NORMAL_INT_MAX / synth.NORMAL_INT_STD + 1e-6
    # weights: sigma = 1/sqrt(fan_in)
    mid = synth.CONFIGS["mid_bf16"]
    w = synth.host_tensor(mid, "w_down", count=1 << 18)
    f = (w.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.std() * math.sqrt(mid.expert_inter) - 1.0) < 0.01


def test_slices_are_index_addressable():
    cfg = synth.CONFIGS["mid_bf16"]
    full = synth.host_tensor(cfg, "w_gate", count=3 * cfg.expert_inter * cfg.latent)
    e1 = synth.host_matrix(cfg, "w_gate", 1)
    np.testing.assert_array_equal(e1.reshape(-1), full[cfg.expert_inter * cfg.latent:
                                                       2 * cfg.expert_inter * cfg.latent])
    rows = synth.host_rows(cfg, "x", [5, 2])
    x = synth.host_tensor(cfg, "x", count=6 * cfg.d).reshape(6, cfg.d)
    np.testing.assert_array_equal(rows, x[[5, 2]])


def test_dyadic_router_logits_are_exact_in_fp32():
    """Dyadic x and W_r: every partial sum is a small multiple of 2^-q, so fp32
    accumulation in any order gives the exact logit."""
    cfg = synth.CONFIGS["k3_decode_bf16"]
    x = synth.host_rows(cfg, "x", [0, 1], routing="dyadic")
    W = synth.host_tensor(cfg, "w_router", routing="dyadic", count=4 * cfg.d).reshape(4, cfg.d)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = synth.dyadic_router_shift(cfg.d)
    assert np.all(Wf * 2 ** q == np.round(Wf * 2 ** q)) and np.abs(Wf * 2 ** q).max() <= 8
    assert np.all(xf == np.round(xf)) and np.abs(xf).max() <= 2
    z = xf @ Wf.T
    assert np.abs(z).max() * 2 ** q < 2 ** 24
    assert 0.5 < z.std() < 2.0


def test_fp8_layer_scales_give_unit_fan_in_variance():
    cfg = synth.CONFIGS["k3_prefill_fp8"].with_(d=256, latent=128, expert_inter=256,
                                                 n_experts=2, shared_inter=128)
    codes = synth.host_matrix(cfg, "w_gate", 0)
    sc = synth.host_scales(cfg, "w_gate")[0]
    vals = np.vectorize(oracle.e4m3_to_double)(codes)
    deq = vals * np.repeat(np.repeat(sc, 128, 0), 128, 1)
    assert abs(deq.std() * math.sqrt(cfg.latent) - 1.0) < 0.15
    assert np.abs(vals).max() <= 448


def test_routing_fixture_valid():
    idx = synth.routing_fixture(500, 16, 896, seed=1)
    assert (np.diff(idx, axis=1) > 0).all() and idx.min() >= 0 and idx.max() < 896
    hot = synth.routing_fixture(500, 8, 64, seed=1, hot=10)
    counts = np.bincount(hot.reshape(-1), minlength=64)
    assert counts[:10].min() > counts[10:].max()
    with pytest.raises(ValueError):
        synth.routing_fixture(4, 9, 8)


def test_zipf_offsets():
    b = synth.router_bias(synth.CONFIGS["k3_prefill_bf16"])
    assert b[0] == pytest.approx(5.09, abs=0.01) and b[-1] == pytest.approx(-2.39, abs=0.01)
    p = np.exp(b.astype(np.float64)) / len(b)
    assert p.sum() == pytest.approx(1.0, rel=1e-6)
    assert np.all(np.diff(b) < 0)
