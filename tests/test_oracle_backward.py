"""Pins of the fp64 backward oracle (oracle.backward), CPU only.

* Its forward, given the experts the C oracle chose, equals the C oracle's
  forward (an independent implementation of the same definitions).
* Every gradient equals a central finite difference of sum(dy * y) through
  that forward, entry by entry, for x and each weight: a dropped term, a wrong
  sign or a transposed operand in any step of the chain rule fails here.
* The gradient of an expert no token chose is zero.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import backward as ob

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

SMALL = synth.CONFIGS["mid_bf16"].with_(name="bwd_small", bt=24, d=64, latent=32, n_experts=8,
                                         top_k=2, expert_inter=32, n_shared=2, shared_inter=32,
                                         bias="zipf1.1", cutoff="batch")


def _setup(cfg, seed=0):
    lay = synth.host_layer(cfg, seed)
    ref = oracle.forward(cfg, lay, cutoff=oracle.BATCH)
    p = ob.decode_layer(cfg, lay)
    x = oracle.decode(lay["x"])
    return lay, ref, p, x


def test_forward_equals_c_oracle():
    _, ref, p, x = _setup(SMALL)
    y, tape = ob.forward(SMALL, p, x, ref["idx"])
    np.testing.assert_allclose(tape["w"], ref["w"], rtol=1e-12, atol=0)
    err = np.abs(y - ref["y"]).max() / np.abs(ref["y"]).max()
    assert err < 1e-10, err


def _loss(cfg, p, x, idx, dy):
    y, _ = ob.forward(cfg, p, x, idx)
    return float((dy * y).sum())


@pytest.mark.parametrize("name", ob.GRAD_NAMES)
def test_gradient_equals_finite_difference(name):
    _, ref, p, x = _setup(SMALL)
    idx = ref["idx"]
    rng = np.random.default_rng(5)
    dy = rng.normal(0, 1, (SMALL.bt, SMALL.d))
    gr = ob.backward(SMALL, p, x, idx, dy)
    target = x if name == "dx" else p[name]
    g = gr[name]
    assert g.shape == target.shape
    scale = max(1.0, float(np.abs(g).max()))
    # entries at random, plus the largest-gradient entry
    flat = [int(i) for i in rng.choice(target.size, 8, replace=False)]
    flat.append(int(np.abs(g).argmax()))
    for fi in flat:
        pos = np.unravel_index(fi, target.shape)
        h = 1e-5 * max(1.0, abs(float(target[pos])))
        orig = float(target[pos])
        target[pos] = orig + h
        lp = _loss(SMALL, p, x, idx, dy)
        target[pos] = orig - h
        lm = _loss(SMALL, p, x, idx, dy)
        target[pos] = orig
        fd = (lp - lm) / (2 * h)
        assert abs(fd - g[pos]) <= 1e-6 * scale, (name, pos, fd, g[pos])


def test_unchosen_expert_has_zero_gradient():
    cfg = SMALL.with_(bt=2, top_k=1)
    _, ref, p, x = _setup(cfg)
    idx = ref["idx"]
    gr = ob.backward(cfg, p, x, idx, np.ones((cfg.bt, cfg.d)))
    chosen = set(int(e) for e in idx.ravel())
    assert len(chosen) < cfg.n_experts
    for e in range(cfg.n_experts):
        nz = any(np.abs(gr[m][e]).max() > 0 for m in ("w_gate", "w_up", "w_down"))
        assert nz == (e in chosen), e
        assert (gr["router_bias"][e] != 0) == (e in chosen)


def test_finite_differences_catch_a_planted_mistake(monkeypatch):
    """Plant a mistake in the oracle (phi' without its tanh-cap term; the
    forward only uses phi and psi, so it stays right): the finite difference
    agrees with the true gradient and not with the planted one."""
    _, ref, p, x = _setup(SMALL)
    idx = ref["idx"]
    dy = np.random.default_rng(5).normal(0, 1, (SMALL.bt, SMALL.d))
    good = ob.backward(SMALL, p, x, idx, dy)["w_gate"]
    orig = ob.situ_parts

    def planted(g, u, beta, beta_u):
        phi, dphi, psi, dpsi = orig(g, u, beta, beta_u)
        s = 1.0 / (1.0 + np.exp(-g))
        return phi, dphi - s * (1.0 - np.tanh(g / beta) ** 2), psi, dpsi

    monkeypatch.setattr(ob, "situ_parts", planted)
    wrong = ob.backward(SMALL, p, x, idx, dy)["w_gate"]
    monkeypatch.undo()
    pos = np.unravel_index(int(np.abs(good - wrong).argmax()), good.shape)
    h = 1e-5
    t = p["w_gate"]
    o = float(t[pos])
    t[pos] = o + h
    lp = _loss(SMALL, p, x, idx, dy)
    t[pos] = o - h
    lm = _loss(SMALL, p, x, idx, dy)
    t[pos] = o
    fd = (lp - lm) / (2 * h)
    scale = max(1.0, float(np.abs(good).max()))
    assert abs(fd - good[pos]) <= 1e-6 * scale
    assert abs(fd - wrong[pos]) > 1e-3 * scale


def test_token_and_expert_locality_of_the_gradients():
    """What the full-size sampled GPU check relies on: the oracle on the layer
    cut down to the experts some tokens chose gives those tokens' dx, and the
    full weight gradients of an expert all of whose tokens are among them,
    equal to the oracle on the whole layer."""
    from tests.test_gpu_backward import _reduced_host_layer
    cfg = SMALL.with_(bt=48)
    lay, ref, p, x = _setup(cfg)
    idx = ref["idx"]
    dy = np.random.default_rng(9).normal(0, 1, (cfg.bt, cfg.d))
    full = ob.backward(cfg, p, x, idx, dy)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
    e_star = int(np.argmin(np.where(counts > 0, counts, 10 ** 9)))
    tokens = [int(t) for t in np.nonzero((idx == e_star).any(axis=1))[0]]
    sub, small, remap, sub_idx = _reduced_host_layer(cfg, tokens, idx, 0)
    part = ob.backward(sub, ob.decode_layer(sub, small), x[tokens], sub_idx, dy[tokens])
    np.testing.assert_allclose(part["dx"], full["dx"][tokens], rtol=1e-9, atol=1e-12)
    es = remap[e_star]
    for n in ("w_gate", "w_up", "w_down", "w_router", "router_bias"):
        np.testing.assert_allclose(part[n][es], full[n][e_star], rtol=1e-9, atol=1e-12)
