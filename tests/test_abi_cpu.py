"""The C-ABI library on the host: exported symbols, struct layouts, validation.

No compute is launched: these run without a GPU.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import synth
from tests import parity

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("sparse_moe_layer_quantile_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_forward",
            "moe_status_str"} <= set(names)
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(moe.EXPORTED) == set(names)


def test_struct_layouts_match_header():
    """sizeof / offsetof of every ABI struct, from gcc on the header, equal the
    ctypes mirrors used by the binding."""
    structs = {"moe_config": moe.MoeConfig, "moe_weights": moe.MoeWeights,
               "moe_route_out": moe.MoeRouteOut, "moe_dispatch_out": moe.MoeDispatchOut,
               "moe_ffn_config": moe.MoeFfnConfig, "moe_ffn_weights": moe.MoeFfnWeights,
               "moe_tier_desc": moe.MoeTierDesc, "moe_tier_stats": moe.MoeTierStats,
               "moe_grads": moe.MoeGrads}
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void){"]
    for s, cls in structs.items():
        src.append(f'printf("{s} %zu\\n", sizeof({s}));')
        for f, _ in cls._fields_:
            src.append(f'printf("{s}.{f} %zu\\n", offsetof({s}, {f}));')
    src.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.split() for line in out.strip().splitlines())
    for s, cls in structs.items():
        assert int(got[s]) == ctypes.sizeof(cls), s
        for f, _ in cls._fields_:
            assert int(got[f"{s}.{f}"]) == getattr(cls, f).offset, f"{s}.{f}"


def test_workspace_sizes():
    for name, cfg in synth.CONFIGS.items():
        c = parity.abi_config(cfg)
        n = moe.workspace_bytes(c, cfg.bt)
        assert n > 0, name
        assert moe.workspace_bytes(c, cfg.bt * 2) > n
    k3 = parity.abi_config(synth.CONFIGS["k3_prefill_bf16"])
    assert 3.5e9 < moe.workspace_bytes(k3, 16384) < 4.5e9


@pytest.mark.parametrize("change,code", [
    (dict(latent=500), -2),                 # not a multiple of 64
    (dict(n_experts=2000), -2),             # more than 1024 experts
    (dict(top_k=0), -1),
    (dict(top_k=65, n_experts=128), -2),    # k above 64
    (dict(d=-1), -1),
    (dict(beta=0.0), -1),
    (dict(latent=4160), -2),                # latent row over the LDS staging limit
])
def test_invalid_configs_rejected_on_host(change, code):
    cfg = synth.CONFIGS["mid_bf16"].with_(**change)
    c = parity.abi_config(cfg)
    assert moe.workspace_bytes(c, 64) == 0
    out = moe.MoeRouteOut(1, 1, 0, 0)
    assert moe.moe_route(c, moe.MoeWeights(w_router=1), 1, 64, out, 256, 1 << 30, 0) == code


def test_dtype_combinations():
    base = synth.CONFIGS["mid_bf16"]
    ok = parity.abi_config(base)
    assert moe.workspace_bytes(ok, 64) > 0
    bad = moe.make_config(2048, 512, 64, 8, 512, 2, 1024, act="f32", weight="bf16")
    assert moe.workspace_bytes(bad, 64) == 0
    bad = moe.make_config(2048, 512, 64, 8, 512, 2, 1024, act="bf16", weight="f32")
    assert moe.workspace_bytes(bad, 64) == 0
    fp8_odd = moe.make_config(2048, 576, 64, 8, 512, 2, 1024, act="bf16", weight="fp8")
    assert moe.workspace_bytes(fp8_odd, 64) == 0  # fp8 needs multiples of 128
    # the combine keeps a latent row per wavefront in registers
    assert moe.workspace_bytes(moe.make_config(2048, 4096, 64, 8, 512, 2, 1024), 64) > 0
    assert moe.workspace_bytes(moe.make_config(2048, 4160, 64, 8, 512, 2, 1024), 64) == 0
    assert moe.workspace_bytes(moe.make_config(256, 2048, 16, 2, 64, 1, 128, act="f32",
                                               weight="f32"), 64) > 0
    assert moe.workspace_bytes(moe.make_config(256, 2112, 16, 2, 64, 1, 128, act="f32",
                                               weight="f32"), 64) == 0


def test_mxfp4_a8_workspace_and_limits():
    """MX FP8 expert inputs add their codes and E8M0 scales to the workspace:
    x_lat (bt L bytes + bt L / 32) and h (bt k I + bt k I / 32), and drop the
    bf16 h (the gate/up epilogue writes h in MX FP8 directly)."""
    cfg = synth.CONFIGS["mid_bf16"].with_(weight="mxfp4")
    c4 = parity.abi_config(cfg)
    c8 = parity.abi_config(cfg.with_(act_quant="mxfp8"))
    assert c8.weight_dtype == moe.MOE_MXFP4_A8
    bt = 1024
    extra = bt * cfg.latent * 33 // 32 + bt * cfg.top_k * cfg.expert_inter * 33 // 32 - \
        2 * bt * cfg.top_k * cfg.expert_inter
    diff = moe.workspace_bytes(c8, bt) - moe.workspace_bytes(c4, bt)
    assert extra - 256 <= diff <= extra + 4 * 256
    # K ranges of whole 128-element groups, as for MXFP4
    assert moe.workspace_bytes(parity.abi_config(cfg.with_(act_quant="mxfp8", latent=576)),
                               64) == 0
    with pytest.raises(AssertionError):
        parity.abi_config(synth.CONFIGS["mid_bf16"].with_(act_quant="mxfp8"))
    # MX FP8 experts (W8A8): the same workspace as W4A8, MX FP8 inputs required
    c88 = parity.abi_config(cfg.with_(weight="mxfp8", act_quant="mxfp8"))
    assert c88.weight_dtype == moe.MOE_MXFP8
    assert moe.workspace_bytes(c88, bt) == moe.workspace_bytes(c8, bt)
    with pytest.raises(AssertionError):
        parity.abi_config(cfg.with_(weight="mxfp8"))


def test_mx8_quantize_argument_errors_on_host():
    """Rejected before any launch: n not a multiple of 32, negative, NULL or
    misaligned pointers; n = 0 is a no-op."""
    assert moe.moe_mx8_quantize(256, 48, 256, 256, 0) == -1
    assert moe.moe_mx8_quantize(256, -32, 256, 256, 0) == -1
    assert moe.moe_mx8_quantize(0, 32, 256, 256, 0) == -1
    assert moe.moe_mx8_quantize(256, 32, 0, 256, 0) == -1
    assert moe.moe_mx8_quantize(258, 32, 256, 256, 0) == -1
    assert moe.moe_mx8_quantize(0, 0, 0, 0, 0) == 0


def test_tier_select_policy():
    """The expert cache policy (host only): free slots fill with the best
    candidates; a full cache swaps only when a candidate beats the worst
    resident by more than 1.25x; max_loads caps a call; ties are ordered by id."""
    sel = moe.tier_select
    score = np.array([0, 5, 3, 3, 9, 0, 1], np.float32)
    res = np.zeros(7, np.uint8)
    load, vic = sel(score, res, 3, 8)
    assert load.tolist() == [4, 1, 2] and vic.tolist() == [-1, -1, -1]
    load, vic = sel(score, res, 3, 2)  # max_loads
    assert load.tolist() == [4, 1]
    # full cache {1, 2, 4}: candidate 3 (3.0) does not beat victim 2 (3.0) x 1.25
    res[[1, 2, 4]] = 1
    load, vic = sel(score, res, 3, 8)
    assert load.size == 0
    score[3] = 3.8  # beats 3.0 x 1.25 = 3.75
    load, vic = sel(score, res, 3, 8)
    assert load.tolist() == [3] and vic.tolist() == [2]
    # equal-score victims: the higher id goes first
    score = np.array([4, 4, 0, 9, 9], np.float32)
    res = np.array([1, 1, 0, 0, 0], np.uint8)
    load, vic = sel(score, res, 2, 8)
    assert load.tolist() == [3, 4] and vic.tolist() == [1, 0]
    # a free slot first, then a swap
    res = np.array([1, 0, 0, 0, 0], np.uint8)
    load, vic = sel(score, res, 2, 8)
    assert load.tolist() == [3, 4] and vic.tolist() == [-1, 0]
    # zero scores are never loaded; invalid arguments
    load, vic = sel(np.zeros(4, np.float32), np.zeros(4, np.uint8), 4, 4)
    assert load.size == 0
    with pytest.raises(moe.MoeError):
        sel(score, np.ones(5, np.uint8), 2, 8)  # more resident than slots


def test_tier_slot_bytes_and_unsupported_dtypes():
    """A slot holds one expert's three matrices (and E8M0 codes for MX dtypes),
    each 256-byte aligned; fp32 and fp8-block experts are not tiered, and a
    forward with an expert table on them is rejected before any launch."""
    base = synth.CONFIGS["mid_bf16"]
    n = base.expert_inter * base.latent
    assert moe.tier_slot_bytes(parity.abi_config(base)) == 3 * 2 * n
    mx4 = parity.abi_config(base.with_(weight="mxfp4"))
    assert moe.tier_slot_bytes(mx4) == 3 * (n // 2) + 3 * (n // 32)
    mx8 = parity.abi_config(base.with_(weight="mxfp8", act_quant="mxfp8"))
    assert moe.tier_slot_bytes(mx8) == 3 * n + 3 * (n // 32)
    fp8 = parity.abi_config(synth.CONFIGS["k3_prefill_fp8"])
    assert moe.tier_slot_bytes(fp8) == 0
    assert moe.tier_slot_bytes(parity.abi_config(synth.CONFIGS["tiny_fp32"])) == 0
    need = moe.workspace_bytes(fp8, 64)
    w = moe.MoeWeights(**{f: 256 for f in moe.WEIGHT_FIELDS})
    assert moe.moe_forward(fp8, w, 256, 64, 256, None, None, 256, need, 0) == -2


def test_argument_errors_before_any_launch():
    c = parity.abi_config(synth.CONFIGS["mid_bf16"])
    need = moe.workspace_bytes(c, 64)
    w = moe.MoeWeights(w_router=1)
    out = moe.MoeRouteOut(1, 1, 0, 0)
    # missing weights, outputs, workspace
    assert moe.moe_route(c, moe.MoeWeights(), 1, 64, out, 256, need, 0) == -1
    assert moe.moe_route(c, w, 1, 64, moe.MoeRouteOut(0, 1, 0, 0), 256, need, 0) == -1
    assert moe.moe_route(c, w, 1, 64, out, 0, need, 0) == -3
    assert moe.moe_route(c, w, 1, 64, out, 256, need - 1, 0) == -3
    assert moe.moe_route(c, w, 1, 64, out, 257, need, 0) == -3       # misaligned
    assert moe.moe_route(c, w, 1, -1, out, 256, need, 0) == -1
    d = moe.MoeDispatchOut(1, 1, 1, 0)
    assert moe.moe_dispatch(c, 1, 64, d, 256, need, 0) == -1
    assert moe.moe_forward(c, w, 1, 64, 1, None, None, 256, need, 0) == -1  # no expert weights
    assert moe.status_str(-3).startswith("workspace")
    assert moe.status_str(7) == "unknown status"


def test_backward_workspace_and_argument_errors():
    """moe_backward: bf16 only; every error returned before any launch."""
    mid = synth.CONFIGS["mid_bf16"]
    c = parity.abi_config(mid)
    need = moe.backward_workspace_bytes(c, 64)
    P, L, I = 64 * mid.top_k, mid.latent, mid.expert_inter
    assert need > 2 * P * (L + I) * 8  # the recomputed pair activations dominate
    assert moe.backward_workspace_bytes(c, 0) > 0
    assert moe.backward_workspace_bytes(c, -1) == 0
    for other in (synth.CONFIGS["tiny_fp32"], mid.with_(weight="fp8", router="bf16"),
                  mid.with_(weight="mxfp4")):
        assert moe.backward_workspace_bytes(parity.abi_config(other), 64) == 0
    full = moe.MoeGrads(*([1] * len(moe.GRAD_FIELDS)))
    w = moe.MoeWeights(**{n: 1 for n in ("w_router", "w_down_proj", "w_gate", "w_up",
                                         "w_down", "w_up_proj", "sh_gate", "sh_up",
                                         "sh_down")})
    ok = (c, w, 1, 64, 1, 1, 1)
    assert moe.moe_backward(*ok, moe.MoeGrads(), 256, need, 0) == -1         # no gradients
    assert moe.moe_backward(*ok, moe.MoeGrads(*([1] * 11)), 256, need, 0) == -1  # no sh_down
    assert moe.moe_backward(c, moe.MoeWeights(), 1, 64, 1, 1, 1, full, 256, need, 0) == -1
    assert moe.moe_backward(c, w, 1, 64, 0, 1, 1, full, 256, need, 0) == -1  # no routing
    assert moe.moe_backward(*ok, full, 0, need, 0) == -3
    assert moe.moe_backward(*ok, full, 256, need - 1, 0) == -3
    assert moe.moe_backward(*ok, full, 257, need, 0) == -3                  # misaligned
    tab = moe.MoeWeights(**{f: getattr(w, f) or 0 for f, _ in moe.MoeWeights._fields_})
    tab.expert_tab = 1
    assert moe.moe_backward(c, tab, 1, 64, 1, 1, 1, full, 256, need, 0) == -2
    f32 = parity.abi_config(synth.CONFIGS["tiny_fp32"])
    assert moe.moe_backward(f32, w, 1, 64, 1, 1, 1, full, 256, need, 0) == -2


def test_ffn_workspace_and_validation():
    """The dense FFN's host-side checks (no launch)."""
    c = moe.make_ffn_config(7168, 33792)
    ws = moe.ffn_workspace_bytes(c, 16384)
    # n [bt][d] and h [bt][inter] in bf16, no split-K region above 256 rows
    assert ws >= 2 * 16384 * (7168 + 33792) and ws < 2 * 16384 * (7168 + 33792) + 4096
    small = moe.ffn_workspace_bytes(c, 64)
    assert small >= 2 * 64 * (7168 + 33792) + 4 * 16 * 64 * 7168  # with the split-K region
    assert moe.ffn_workspace_bytes(moe.make_ffn_config(7168 + 32, 33792), 8) == 0  # d % 64
    assert moe.ffn_workspace_bytes(moe.make_ffn_config(8192 + 64, 1024), 8) == 0   # d > 8192
    assert moe.ffn_workspace_bytes(moe.make_ffn_config(4096 + 64, 1024, act="f32"), 8) == 0
    assert moe.ffn_workspace_bytes(moe.make_ffn_config(1024, 1000), 8) == 0        # inter % 64
    assert moe.ffn_workspace_bytes(moe.make_ffn_config(1024, 1024), -1) == 0
    w = moe.MoeFfnWeights(0, 0, 0, 0)
    # NULL weights are rejected before anything touches the device
    assert moe.moe_ffn_forward(c, w, 0, 0, 8, 0, 0, 0, 0) == -1


def test_situ_eval_argument_errors_on_host():
    """moe_situ_eval validates before any launch (no GPU needed)."""
    assert moe.moe_situ_eval(0, 0, 0, 4.0, 25.0, 0, 0, 0, 0) == 0      # nothing to do
    assert moe.moe_situ_eval(0, 0, -1, 4.0, 25.0, 0, 0, 0, 0) == -1
    assert moe.moe_situ_eval(0, 0, 16, 4.0, 25.0, 0, 0, 0, 0) == -1     # NULL inputs
    assert moe.moe_situ_eval(8, 8, 16, 4.0, 25.0, 0, 0, 0, 0) == -1     # no output
    assert moe.moe_situ_eval(8, 8, 16, 0.0, 25.0, 8, 0, 0, 0) == -1     # beta <= 0
    assert moe.moe_situ_eval(8, 8, 16, 4.0, -1.0, 8, 0, 0, 0) == -1     # beta_u <= 0
