"""ctypes binding of the fp64 CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  The oracle
computes the Stable LatentMoE layer forward from its plain definition (see
oracle.h for the steps and the pages they follow).  Inputs are raw storage
arrays (float32, uint16 bf16 bits, uint8 e4m3 codes with fp32 block scales);
a "shape" is any object with the attributes d, latent, n_experts, top_k,
expert_inter, n_shared, shared_inter, beta, beta_u, rms_eps.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
F32, BF16, FP8, MXFP4, MXFP8 = 0, 1, 2, 3, 4
GIVEN, BATCH = 0, 1

_NP_DT = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): FP8}


class OrcMat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_void_p), ("n_mats", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class OrcShape(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("latent", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("expert_inter", ctypes.c_int64), ("n_shared", ctypes.c_int64),
                ("shared_inter", ctypes.c_int64), ("beta", ctypes.c_double),
                ("beta_u", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("act_mx_block", ctypes.c_int64), ("act_mx_exact", ctypes.c_int64)]


class OrcWeights(ctypes.Structure):
    _fields_ = [("w_router", OrcMat), ("router_bias", ctypes.c_void_p),
                ("w_down_proj", OrcMat), ("w_gate", OrcMat), ("w_up", OrcMat),
                ("w_down", OrcMat), ("gamma", ctypes.c_void_p), ("w_up_proj", OrcMat),
                ("sh_gate", OrcMat), ("sh_up", OrcMat), ("sh_down", OrcMat)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        P, I64, D, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int32
        sig = {
            "orc_bf16_to_double": ([ctypes.c_uint16], D),
            "orc_e4m3_to_double": ([ctypes.c_uint8], D),
            "orc_e2m1_to_double": ([ctypes.c_uint8], D),
            "orc_e8m0_to_double": ([ctypes.c_uint8], D),
            "orc_decode": ([P, I64, I64, I64], D),
            "orc_matvec": ([P, I64, P, P], None),
            "orc_sigmoid": ([D], D),
            "orc_phi": ([D, D], D),
            "orc_psi": ([D, D], D),
            "orc_router_logits": ([P, P, P, P, I64, P], ctypes.c_int),
            "orc_quantile": ([P, I64, I64, I64, P], ctypes.c_int),
            "orc_topk": ([P, P, P, I64, I64, I64, P, P], ctypes.c_int),
            "orc_dispatch": ([P, I64, I64, I64, P, P, P, P], ctypes.c_int),
            "orc_expert": ([P, P, P, P, I64, P, P], ctypes.c_int),
            "orc_combine_norm": ([P, P, P, P, P, P], ctypes.c_int),
            "orc_shared": ([P, P, P, P], ctypes.c_int),
            "orc_output": ([P, P, P, P, P], ctypes.c_int),
            "orc_forward": ([P, P, P, I64, I32, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
            "orc_rmsnorm": ([P, I64, P, D, P], None),
            "orc_mx8_quantize": ([P, I64, I64, P, P], ctypes.c_int),
            "orc_double_to_e4m3": ([D], ctypes.c_uint8),
            "orc_round_bf16": ([D], D),
            "orc_dense_ffn": ([P, P, P, P, P, P, P, P], ctypes.c_int),
            "orc_set_threads": ([ctypes.c_int], None),
            "orc_get_threads": ([], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a) if dt is None else np.asarray(a, dtype=dt))
    return a


# MX FP8 expert inputs: decide each code on the input rounded to bf16 (the
# precision the layer stores x_lat and h in) or, when False, on the exact value
MX_CODES_ON_BF16 = True


def shape_of(cfg, mx_codes_on_bf16=None) -> OrcShape:
    g = lambda n, dflt=0: getattr(cfg, n, dflt)
    mx = 32 if getattr(cfg, "act_quant", "none") == "mxfp8" else 0
    on_bf16 = MX_CODES_ON_BF16 if mx_codes_on_bf16 is None else mx_codes_on_bf16
    return OrcShape(g("d"), g("latent"), g("n_experts"), g("top_k"), g("expert_inter"),
                    g("n_shared"), g("shared_inter"), float(g("beta", 4.0)),
                    float(g("beta_u", 25.0)), float(g("rms_eps", 1e-6)), mx,
                    0 if on_bf16 else 1)


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


class Mat:
    """Keeps the arrays behind an OrcMat alive.  A uint8 `scale` (E8M0 codes
    [.., rows, cols / 32]) marks `data` as an MX format: MXFP4 when its rows
    are cols / 2 bytes of two codes each, MX FP8 when they are cols e4m3
    codes."""

    def __init__(self, data: np.ndarray, scale: np.ndarray | None = None, n_mats=None,
                 rows=None, cols=None):
        self.data = np.ascontiguousarray(data)
        mx = scale is not None and np.asarray(scale).dtype == np.uint8
        if scale is None:
            self.scale = None
        else:
            self.scale = np.ascontiguousarray(scale, np.uint8 if mx else np.float32)
        dt = _NP_DT[self.data.dtype]
        if data.ndim == 3:
            n_mats, rows, cols = data.shape
        elif data.ndim == 2:
            n_mats, rows, cols = 1, data.shape[0], data.shape[1]
        if mx:
            blocks = self.scale.shape[-1]
            if cols * 2 == blocks * 32:
                dt, cols = MXFP4, cols * 2
            elif cols == blocks * 32:
                dt = MXFP8
            else:
                raise ValueError("E8M0 scales do not match the MX data's row length")
        self.c = OrcMat(self.data.ctypes.data, dt,
                        None if self.scale is None else self.scale.ctypes.data,
                        n_mats, rows, cols)

    @property
    def ref(self):
        return ctypes.byref(self.c)


class Weights:
    """Oracle view of a layer given as a dict of raw-storage arrays (the
    key names of the GPU ABI's weight set)."""

    def __init__(self, layer: dict):
        def m(name):
            if layer.get(name) is None:
                return None
            return Mat(layer[name], layer.get("scale:" + name))
        self.mats = {n: m(n) for n in ("w_router", "w_down_proj", "w_gate", "w_up", "w_down",
                                       "w_up_proj", "sh_gate", "sh_up", "sh_down")}
        self.bias = _c(layer.get("router_bias"), np.float32)
        self.gamma = _c(layer.get("gamma"), np.float32)
        def cm(n):
            return self.mats[n].c if self.mats[n] is not None else OrcMat()
        self.c = OrcWeights(cm("w_router"),
                            None if self.bias is None else self.bias.ctypes.data,
                            cm("w_down_proj"), cm("w_gate"), cm("w_up"), cm("w_down"),
                            None if self.gamma is None else self.gamma.ctypes.data,
                            cm("w_up_proj"), cm("sh_gate"), cm("sh_up"), cm("sh_down"))

    @property
    def ref(self):
        return ctypes.byref(self.c)


# ---- scalar functions ----------------------------------------------------------

def sigmoid(z):
    return lib().orc_sigmoid(float(z))


def phi(g, beta=4.0):
    return lib().orc_phi(float(g), float(beta))


def psi(u, beta_u=25.0):
    return lib().orc_psi(float(u), float(beta_u))


def bf16_to_double(bits):
    return lib().orc_bf16_to_double(int(bits))


def e4m3_to_double(code):
    return lib().orc_e4m3_to_double(int(code))


def e2m1_to_double(code):
    return lib().orc_e2m1_to_double(int(code))


def e8m0_to_double(code):
    return lib().orc_e8m0_to_double(int(code))


def matvec(mat: Mat, vec, index=0):
    vec = _c(vec, np.float64)
    out = np.empty(mat.c.rows, np.float64)
    lib().orc_matvec(mat.ref, index, _ptr(vec), _ptr(out))
    return out


# ---- steps ----------------------------------------------------------------------

def router_logits(cfg, w: Weights, x: np.ndarray, rows=None) -> np.ndarray:
    """fp64 logits [n_rows][E] of the listed token rows of x (raw storage [bt][d])."""
    xm = Mat(x)
    if rows is None:
        n = x.shape[0]
        rp = None
    else:
        rp = np.ascontiguousarray(rows, np.int64)
        n = rp.size
    out = np.empty((n, cfg.n_experts), np.float64)
    rc = lib().orc_router_logits(ctypes.byref(shape_of(cfg)), w.ref, xm.ref, _ptr(rp), n,
                                 _ptr(out))
    if rc:
        raise ValueError("orc_router_logits rejected its arguments")
    return out


def quantile(z32: np.ndarray, m: int) -> np.ndarray:
    z32 = _c(z32, np.float32)
    bt, E = z32.shape
    out = np.empty(E, np.float32)
    if lib().orc_quantile(_ptr(z32), bt, E, m, _ptr(out)):
        raise ValueError("orc_quantile rejected its arguments")
    return out


def cutoff_update(alpha, zeta, rate: float) -> np.ndarray:
    """One step of the running cutoff (an exponential moving average of the
    batch quantiles; the news18a page's third technique adjusts the cutoff
    dynamically without giving a rule): alpha + rate * (zeta - alpha) in fp32,
    each operation rounded."""
    a = np.asarray(alpha, np.float32)
    z = np.asarray(zeta, np.float32)
    r = np.float32(rate)
    return (a + r * (z - a)).astype(np.float32)


def topk(z32: np.ndarray, k: int, alpha=None, z64=None):
    z32 = _c(z32, np.float32)
    alpha = _c(alpha, np.float32)
    z64 = _c(z64, np.float64)
    bt, E = z32.shape
    idx = np.empty((bt, k), np.int32)
    w = np.empty((bt, k), np.float64)
    if lib().orc_topk(_ptr(z32), _ptr(alpha), _ptr(z64), bt, E, k, _ptr(idx), _ptr(w)):
        raise ValueError("orc_topk rejected its arguments")
    return idx, w


def dispatch(idx: np.ndarray, n_experts: int):
    idx = _c(idx, np.int32)
    bt, k = idx.shape
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    perm = np.empty(bt * k, np.int32)
    inv = np.empty(bt * k, np.int32)
    if lib().orc_dispatch(_ptr(idx), bt, k, n_experts, _ptr(counts), _ptr(offsets),
                          _ptr(perm), _ptr(inv)):
        raise ValueError("orc_dispatch rejected its arguments")
    return counts, offsets, perm, inv


def expert(cfg, gate: Mat, up: Mat, down: Mat, x_lat, index=0,
           mx_codes_on_bf16=None) -> np.ndarray:
    x_lat = _c(x_lat, np.float64)
    o = np.empty(cfg.latent, np.float64)
    if lib().orc_expert(ctypes.byref(shape_of(cfg, mx_codes_on_bf16)), gate.ref, up.ref,
                        down.ref, index, _ptr(x_lat), _ptr(o)):
        raise ValueError("orc_expert rejected its arguments")
    return o


def combine_norm(cfg, o: np.ndarray, w, gamma=None):
    o = _c(o, np.float64)
    w = _c(w, np.float64)
    gamma = _c(gamma, np.float32)
    ylat = np.empty(cfg.latent, np.float64)
    n = np.empty(cfg.latent, np.float64)
    if lib().orc_combine_norm(ctypes.byref(shape_of(cfg)), _ptr(o), _ptr(w), _ptr(gamma),
                              _ptr(ylat), _ptr(n)):
        raise ValueError("orc_combine_norm rejected its arguments")
    return ylat, n


def shared(cfg, w: Weights, x_t) -> np.ndarray:
    x_t = _c(x_t, np.float64)
    out = np.empty(cfg.d, np.float64)
    if lib().orc_shared(ctypes.byref(shape_of(cfg)), w.ref, _ptr(x_t), _ptr(out)):
        raise ValueError("orc_shared rejected its arguments")
    return out


def output(cfg, w: Weights, n, x_t) -> np.ndarray:
    n = _c(n, np.float64)
    x_t = _c(x_t, np.float64)
    y = np.empty(cfg.d, np.float64)
    if lib().orc_output(ctypes.byref(shape_of(cfg)), w.ref, _ptr(n), _ptr(x_t), _ptr(y)):
        raise ValueError("orc_output rejected its arguments")
    return y


def double_to_e4m3(v) -> int:
    return int(lib().orc_double_to_e4m3(float(v)))


def round_bf16(v: float) -> float:
    """Nearest bf16 value of v (ties to even)."""
    return float(lib().orc_round_bf16(float(v)))


def mx8_quantize(x, block=32):
    """(E4M3 codes uint8 [n], E8M0 scales uint8 [n / block]) of x (OCP MX FP8)."""
    x = _c(x, np.float64).ravel()
    codes = np.empty(x.size, np.uint8)
    scales = np.empty(x.size // block, np.uint8)
    if lib().orc_mx8_quantize(_ptr(x), x.size, block, _ptr(codes), _ptr(scales)):
        raise ValueError("orc_mx8_quantize rejected its arguments")
    return codes, scales


def rmsnorm(x, gamma=None, eps=1e-6) -> np.ndarray:
    x = _c(x, np.float64)
    gamma = _c(gamma, np.float32)
    out = np.empty(x.size, np.float64)
    lib().orc_rmsnorm(_ptr(x), x.size, _ptr(gamma), float(eps), _ptr(out))
    return out


class FfnShape:
    """Oracle shape of the dense FFN: width d, intermediate width inter."""

    def __init__(self, d, inter, beta=4.0, beta_u=25.0, rms_eps=1e-6):
        self.d, self.expert_inter, self.latent = d, inter, d
        self.beta, self.beta_u, self.rms_eps = beta, beta_u, rms_eps


def dense_ffn(shape, gate: Mat, up: Mat, down: Mat, x, r=None, gamma=None) -> np.ndarray:
    """y = r + W_d (phi(W_g n) psi(W_u n)), n = RMSNorm(x) gamma, for one row (fp64)."""
    x = _c(x, np.float64)
    r = _c(r, np.float64)
    gamma = _c(gamma, np.float32)
    y = np.empty(shape.d, np.float64)
    if lib().orc_dense_ffn(ctypes.byref(shape_of(shape)), gate.ref, up.ref, down.ref,
                           _ptr(gamma), _ptr(x), _ptr(r), _ptr(y)):
        raise ValueError("orc_dense_ffn rejected its arguments")
    return y


def decode(arr: np.ndarray, scale=None) -> np.ndarray:
    """Exact fp64 value of a raw-storage matrix or stack (uses the oracle's decoders)."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = Mat(a if a.ndim >= 2 else a.reshape(1, -1), scale)
    rows = m.c.n_mats * m.c.rows
    out = np.empty((rows, m.c.cols), np.float64)
    for i in range(rows):
        for c in range(m.c.cols):
            out[i, c] = lib().orc_decode(m.ref, i // m.c.rows, i % m.c.rows, c)
    return out.reshape(a.shape[:-1] + (m.c.cols,))


def forward(cfg, layer: dict, cutoff: int = BATCH, alpha=None):
    """Whole layer on every token of layer['x'] (small shapes).  Returns a dict."""
    w = Weights(layer)
    x = Mat(layer["x"])
    bt = layer["x"].shape[0]
    E, k, P = cfg.n_experts, cfg.top_k, bt * cfg.top_k
    alpha = _c(alpha, np.float32)
    out = dict(z32=np.empty((bt, E), np.float32), zeta=np.empty(E, np.float32),
               idx=np.empty((bt, k), np.int32), w=np.empty((bt, k), np.float64),
               counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               perm=np.empty(P, np.int32), inv_perm=np.empty(P, np.int32),
               y=np.empty((bt, cfg.d), np.float64))
    rc = lib().orc_forward(ctypes.byref(shape_of(cfg)), w.ref, x.ref, bt, cutoff, _ptr(alpha),
                           *(_ptr(out[n]) for n in ("z32", "zeta", "idx", "w", "counts",
                                                    "offsets", "perm", "inv_perm", "y")))
    if rc:
        raise ValueError("orc_forward rejected its arguments")
    return out
