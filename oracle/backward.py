"""Backward pass of the Stable LatentMoE layer in fp64 -- test infrastructure.

Only tests/, the smoke check and the benchmark's CPU leg use this module; the
product path never imports it.

The pages describe the forward pass only: the router's sigmoid scores and
quantile cutoffs (tech.news18a.com page, figure 2 and the "quantile
balancing" passage), the W-down / experts / RMSNorm / W-up latent path and
the SiTU-GLU activation with its two tanh caps (same page, the architecture
figure and the SiTU formula).  Training is where the pages put the point of
both caps and of the cutoffs (the gradient-explosion passage of that page);
the gradients themselves are the chain rule of that forward, written out
here:

  * routing: the chosen set is a step function of the scores, so it carries
    no gradient; a chosen pair's weight w = sigmoid(z) does (dz = dw w (1-w)),
    the router bias included;
  * experts: h = w phi(g) psi(u) with g = W_g x_lat, u = W_u x_lat, o = W_d h;
    phi(g) = sigmoid(g) beta tanh(g / beta), psi(u) = beta_u tanh(u / beta_u);
  * latent RMSNorm: n = y_lat r gamma, r = (mean y_lat^2 + eps)^(-1/2);
  * shared experts: hs = phi(W_gs x) psi(W_us x); y = W_up n + sum W_ds hs.

The forward here takes the chosen experts as an input (the selection made by
the C oracle's routing), recomputes every other quantity in fp64 without
rounding, and is itself pinned to the C oracle's forward.  Parity: pinned by
central finite differences of sum(dy * y) in the tests.
"""
from __future__ import annotations

import numpy as np

from . import decode

GRAD_NAMES = ("dx", "w_router", "router_bias", "w_down_proj", "w_gate", "w_up", "w_down",
              "latent_gamma", "w_up_proj", "sh_gate", "sh_up", "sh_down")


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def situ_parts(g, u, beta, beta_u):
    """phi, phi', psi, psi' of the SiTU-GLU pre-activations."""
    s = _sigmoid(g)
    tg = np.tanh(g / beta)
    phi = s * beta * tg
    dphi = s * (1.0 - s) * beta * tg + s * (1.0 - tg * tg)
    tu = np.tanh(u / beta_u)
    return phi, dphi, beta_u * tu, 1.0 - tu * tu


def decode_layer(cfg, layer: dict) -> dict:
    """fp64 values of a layer's raw-storage tensors (names of the synthetic layer)."""
    p = {}
    for n in ("w_router", "w_down_proj", "w_gate", "w_up", "w_down", "w_up_proj", "sh_gate",
              "sh_up", "sh_down"):
        if n in layer:
            p[n] = decode(layer[n], layer.get("scale:" + n))
    bias = layer.get("router_bias")
    p["router_bias"] = (np.zeros(cfg.n_experts) if bias is None
                        else np.asarray(bias, np.float64))
    gamma = layer.get("gamma")
    p["latent_gamma"] = (np.ones(cfg.latent) if gamma is None
                         else np.asarray(gamma, np.float64))
    return p


def forward(cfg, p: dict, x, idx):
    """y [bt][d] and the tape of intermediates, for the chosen experts idx [bt][k]."""
    x = np.asarray(x, np.float64)
    bt, k = idx.shape
    z = x @ p["w_router"].T + p["router_bias"]
    w = _sigmoid(np.take_along_axis(z, idx, axis=1))  # [bt][k]
    xl = x @ p["w_down_proj"].T
    L = xl.shape[1]
    ylat = np.zeros((bt, L))
    pairs = {}
    for e in np.unique(idx):
        t, j = np.nonzero(idx == e)
        g = xl[t] @ p["w_gate"][e].T
        u = xl[t] @ p["w_up"][e].T
        phi, dphi, psi, dpsi = situ_parts(g, u, cfg.beta, cfg.beta_u)
        a = phi * psi
        h = w[t, j][:, None] * a
        o = h @ p["w_down"][e].T
        np.add.at(ylat, t, o)
        pairs[int(e)] = dict(t=t, j=j, g=g, u=u, phi=phi, dphi=dphi, psi=psi, dpsi=dpsi,
                             a=a, h=h)
    r = 1.0 / np.sqrt((ylat * ylat).mean(axis=1) + cfg.rms_eps)
    n = ylat * r[:, None] * p["latent_gamma"]
    y = n @ p["w_up_proj"].T
    shared = []
    for s in range(cfg.n_shared):
        gs = x @ p["sh_gate"][s].T
        us = x @ p["sh_up"][s].T
        phi, dphi, psi, dpsi = situ_parts(gs, us, cfg.beta, cfg.beta_u)
        hs = phi * psi
        y = y + hs @ p["sh_down"][s].T
        shared.append(dict(phi=phi, dphi=dphi, psi=psi, dpsi=dpsi, hs=hs))
    tape = dict(x=x, z=z, w=w, xl=xl, ylat=ylat, r=r, n=n, pairs=pairs, shared=shared)
    return y, tape


def backward(cfg, p: dict, x, idx, dy) -> dict:
    """Gradients of sum(dy * y) with respect to x and every weight (GRAD_NAMES)."""
    dy = np.asarray(dy, np.float64)
    _, tp = forward(cfg, p, x, idx)
    x, w, xl, ylat, r, n = tp["x"], tp["w"], tp["xl"], tp["ylat"], tp["r"], tp["n"]
    gamma = p["latent_gamma"]
    L = xl.shape[1]
    gr = {m: np.zeros_like(p[m]) for m in GRAD_NAMES if m in p}
    # y = W_up n + sum_s W_ds,s hs_s
    gr["w_up_proj"] = dy.T @ n
    dn = dy @ p["w_up_proj"]
    dx = np.zeros_like(x)
    for s, sh in enumerate(tp["shared"]):
        gr["sh_down"][s] = dy.T @ sh["hs"]
        dhs = dy @ p["sh_down"][s]
        dgs = dhs * sh["psi"] * sh["dphi"]
        dus = dhs * sh["phi"] * sh["dpsi"]
        gr["sh_gate"][s] = dgs.T @ x
        gr["sh_up"][s] = dus.T @ x
        dx += dgs @ p["sh_gate"][s] + dus @ p["sh_up"][s]
    # n = y_lat r gamma
    gr["latent_gamma"] = (dn * ylat * r[:, None]).sum(axis=0)
    dng = dn * gamma
    dylat = r[:, None] * dng - ylat * (r ** 3)[:, None] * (dng * ylat).sum(axis=1,
                                                                           keepdims=True) / L
    # experts: o = W_d h, h = w phi(g) psi(u)
    dxl = np.zeros_like(xl)
    dw = np.zeros_like(w)
    for e, q in tp["pairs"].items():
        t, j = q["t"], q["j"]
        do = dylat[t]
        gr["w_down"][e] = do.T @ q["h"]
        dh = do @ p["w_down"][e]
        dw[t, j] = (dh * q["a"]).sum(axis=1)
        wt = w[t, j][:, None]
        dg = dh * wt * q["psi"] * q["dphi"]
        du = dh * wt * q["phi"] * q["dpsi"]
        xe = xl[t]
        gr["w_gate"][e] = dg.T @ xe
        gr["w_up"][e] = du.T @ xe
        np.add.at(dxl, t, dg @ p["w_gate"][e] + du @ p["w_up"][e])
    # x_lat = W_down_proj x
    gr["w_down_proj"] = dxl.T @ x
    dx += dxl @ p["w_down_proj"]
    # w = sigmoid(z) of the chosen pairs, z = W_r x + b
    dz = np.zeros_like(tp["z"])
    np.put_along_axis(dz, idx, dw * w * (1.0 - w), axis=1)
    gr["w_router"] = dz.T @ x
    gr["router_bias"] = dz.sum(axis=0)
    dx += dz @ p["w_router"]
    gr["dx"] = dx
    return gr
