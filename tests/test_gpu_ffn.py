"""GPU parity of the dense layer-1 FFN (moe_ffn_forward through the C ABI)
against the fp64 oracle: y = r + W_d(phi(W_g n) psi(W_u n)), n = RMSNorm(x) gamma.

mkdocs.reaper.mx "Vue d'ensemble de l'architecture": layer 1 is a dense SiTU-GLU
FFN of intermediate width 33 792 (section "Le décompte des couches"); every
sublayer is pre-normed and summed into the block representation (section "Ce
que fait une couche").  Error bound: normwise max relative error, 1e-4 (fp32)
and 2e-2 (bf16), as for the MoE layer.
"""
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


def _layer(cfg, seed=0):
    import sparse_moe_layer_quantile_amd as moe
    t = synth.ffn_device_layer(cfg, seed)
    c = moe.make_ffn_config(cfg.d, cfg.inter, cfg.beta, cfg.beta_u, cfg.rms_eps, act=cfg.act)
    return moe.DenseFFN(c, t), t


class _Ref:
    """The oracle's FFN over host copies of the same weights."""

    def __init__(self, cfg, seed=0):
        self.cfg = cfg
        sp = synth.ffn_specs(cfg)
        self.m = {n: oracle.Mat(synth.ffn_host_tensor(cfg, n, seed).reshape(sp[n].shape))
                  for n in ("w_gate", "w_up", "w_down")}
        self.gamma = synth.ffn_gamma(cfg)
        self.shape = oracle.FfnShape(cfg.d, cfg.inter, cfg.beta, cfg.beta_u, cfg.rms_eps)
        self.seed = seed

    def rows(self, tokens, with_r=True):
        x = oracle.decode(synth.ffn_host_rows(self.cfg, "x", tokens, self.seed))
        r = oracle.decode(synth.ffn_host_rows(self.cfg, "r", tokens, self.seed)) if with_r \
            else [None] * len(tokens)
        return np.stack([oracle.dense_ffn(self.shape, self.m["w_gate"], self.m["w_up"],
                                          self.m["w_down"], x[i], r[i], self.gamma)
                         for i in range(len(tokens))])


def _check(cfg, y, ref, tokens, with_r=True):
    yg = parity.y_to_f64(y)[tokens]
    yr = ref.rows(tokens, with_r)
    tol = parity.TOL["f32" if cfg.act == "f32" else "bf16"]
    say(f"  {cfg.name} bt {cfg.bt}: {len(tokens)} rows")
    err, _ = parity.assert_close(yg, yr, tol, "y")
    return err


@pytest.mark.parametrize("name", ["ffn_tiny_fp32", "ffn_mid_bf16"])
def test_ffn_all_rows(name):
    cfg = synth.FFN_CONFIGS[name]
    layer, t = _layer(cfg)
    y = layer.forward(t["x"], t["r"])
    torch.cuda.synchronize()
    _check(cfg, y, _Ref(cfg), np.arange(cfg.bt))


def test_ffn_residual_absent_and_in_place():
    cfg = synth.FFN_CONFIGS["ffn_mid_bf16"].with_(bt=300)
    layer, t = _layer(cfg)
    ref = _Ref(cfg)
    rows = np.arange(cfg.bt)
    y0 = layer.forward(t["x"], None)
    torch.cuda.synchronize()
    _check(cfg, y0, ref, rows, with_r=False)
    y1 = layer.forward(t["x"], t["r"])
    r = t["r"].clone()
    y2 = layer.forward(t["x"], r, out=r)  # y written over r
    torch.cuda.synchronize()
    assert y2.data_ptr() == r.data_ptr()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("bt", [1, 3, 100, 256, 257])
def test_ffn_ragged_batches(bt):
    """Short batches (split-K down projection up to 256 rows) and one past it."""
    cfg = synth.FFN_CONFIGS["ffn_mid_bf16"].with_(bt=bt, inter=1024)
    layer, t = _layer(cfg)
    y = layer.forward(t["x"], t["r"])
    torch.cuda.synchronize()
    _check(cfg, y, _Ref(cfg), np.arange(bt))


def test_ffn_bt_zero_and_errors():
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.FFN_CONFIGS["ffn_mid_bf16"].with_(bt=4, inter=1024)
    layer, t = _layer(cfg)
    ws = layer.workspace(4)
    st = moe.moe_ffn_forward(layer.cfg, layer.w, 0, 0, 0, 0, ws.data_ptr(), ws.numel(), 0)
    assert st == 0
    # workspace too small
    st = moe.moe_ffn_forward(layer.cfg, layer.w, t["x"].data_ptr(), 0, 4,
                             t["r"].data_ptr(), ws.data_ptr(), 256, 0)
    assert st == -3
    # unsupported width
    bad = moe.make_ffn_config(2048 + 32, 1024)
    st = moe.moe_ffn_forward(bad, layer.w, t["x"].data_ptr(), 0, 4, t["r"].data_ptr(),
                             ws.data_ptr(), ws.numel(), 0)
    assert st == -2
    # misaligned gamma
    w = moe.MoeFfnWeights(layer.w.w_gate, layer.w.w_up, layer.w.w_down, layer.w.gamma + 4)
    st = moe.moe_ffn_forward(layer.cfg, w, t["x"].data_ptr(), 0, 4, t["r"].data_ptr(),
                             ws.data_ptr(), ws.numel(), 0)
    assert st == -1


def test_ffn_k3_decode_all_rows():
    cfg = synth.FFN_CONFIGS["k3_dense_ffn_decode_bf16"]
    layer, t = _layer(cfg)
    y = layer.forward(t["x"], t["r"])
    torch.cuda.synchronize()
    yc = y.clone()
    del layer, t, y
    torch.cuda.empty_cache()
    _check(cfg, yc, _Ref(cfg), np.arange(cfg.bt))


def test_ffn_k3_prefill_sampled_rows():
    cfg = synth.FFN_CONFIGS["k3_dense_ffn_prefill_bf16"]
    layer, t = _layer(cfg)
    y = layer.forward(t["x"], t["r"])
    torch.cuda.synchronize()
    yc = y.clone()
    del layer, t, y
    torch.cuda.empty_cache()
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([rng.choice(cfg.bt, 10, replace=False), [0, cfg.bt - 1]]))
    _check(cfg, yc, _Ref(cfg), tokens)
