"""Seeded synthetic workloads for the Stable LatentMoE layer.

This module generates inputs only: token activations, layer weights, fp8 block
scales, MXFP4 expert weights with their E8M0 block scales, Zipf logit offsets
and routing-index fixtures.  It holds none of the
layer's arithmetic.  The host generator (``libsynth_host.so``, gcc) and the
device generator (``libsynth_dev.so``, hipcc) expand the same counter-based
Philox-4x32-10 definition in ``synth_rng.h`` and produce identical bits, so the
GPU path can have a 60 GB layer written straight into HBM while the CPU oracle
regenerates any slice of it (one expert, a few token rows) on the host.

Workload shapes follow the five layer configurations of the Kimi K3 Stable
LatentMoE (tech.news18a.com "KimiK3的StableLatentMoE架构解析", forward-flow
figure 2; mkdocs.reaper.mx "Vue d'ensemble de l'architecture", per-token path
steps c-g and the parameter-budget table).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

F32, BF16, FP8, MXFP4, E8M0 = 0, 1, 2, 3, 4
# MX FP8 weights: e4m3 codes (generated as FP8 storage) with E8M0 scales per 32;
# a Python-side tag only (the generators see FP8 for the codes)
MXFP8 = 5
MX_DTYPES = (MXFP4, MXFP8)
NORMAL, DYADIC = 0, 1
NORMAL_INT_STD = 107022.329313
NORMAL_INT_MAX = 524280
FP8_MAX = 448.0
FP8_BLOCK = 128
MX_BLOCK = 32        # MXFP4: elements per E8M0 scale
MX_CODE_SIGMA = 2.0  # MXFP4: standard deviation of the draws rounded to E2M1 codes
# standard deviation of the E2M1 value of a N(0, MX_CODE_SIGMA^2) draw (rounded
# to the grid, saturating at 6), and the rms of 2^u, u uniform in {-1, 0, 1}
MX_CODE_STD = 1.9885
MX_SCALE_RMS = math.sqrt((0.25 + 1.0 + 4.0) / 3.0)
MX8_CODE_SIGMA = 16.0  # MX FP8: standard deviation of the draws rounded to e4m3 codes

# weight="mxfp4": the routed experts in MXFP4, every other weight bf16;
# weight="mxfp8": the routed experts in MX FP8 (with MX FP8 inputs), the rest bf16
DTYPE_NAMES = {"f32": F32, "bf16": BF16, "fp8": FP8, "mxfp4": MXFP4, "mxfp8": MXFP8}
NP_STORAGE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8, MXFP4: np.uint8, MXFP8: np.uint8}
# per storage unit (MXFP4: 2 elements)
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1, MXFP4: 1, MXFP8: 1}
MX_NAMES = ("w_gate", "w_up", "w_down")

# Tensor ids: distinct Philox counter words per tensor.
TID = {
    "x": 1, "w_router": 2, "w_down_proj": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
    "w_up_proj": 7, "sh_gate": 8, "sh_up": 9, "sh_down": 10,
}
SCALE_TID_BASE = 100  # block scales of tensor t use id SCALE_TID_BASE + TID[t]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    bt: int
    d: int
    latent: int
    n_experts: int
    top_k: int
    expert_inter: int
    n_shared: int
    shared_inter: int
    act: str = "bf16"
    weight: str = "bf16"
    router: str = "bf16"
    bias: str = "zero"          # "zero" or "zipf1.1"
    cutoff: str = "given"       # benchmark cutoff mode: "given" (alpha = 0) or "batch"
    # "mxfp8": the expert GEMMs read their inputs (x_lat, h) as OCP MX FP8 with a scale
    # per 32 (with weight="mxfp4" or "mxfp8": the block-scaled MFMA path; weight="mxfp8"
    # requires it); "none": exactly
    act_quant: str = "none"
    # > 0: the routed experts live in pinned host memory with an HBM cache of this
    # many experts (moe_tier_*), the benchmark's tiered-decode workload
    tier_slots: int = 0
    beta: float = 4.0
    beta_u: float = 25.0
    rms_eps: float = 1e-6

    # ---- derived sizes -------------------------------------------------
    @property
    def pairs(self) -> int:
        return self.bt * self.top_k

    @property
    def quantile_rank(self) -> int:
        """m = clamp(ceil(bt*k/E), 1, bt)."""
        m = -(-self.bt * self.top_k // self.n_experts)
        return max(1, min(m, self.bt))

    def flops(self) -> int:
        """Algorithmic FLOPs of one forward (2 per multiply-add of every GEMM)."""
        bt, d, L, E = self.bt, self.d, self.latent, self.n_experts
        return (2 * bt * d * E + 2 * bt * d * L + 2 * self.pairs * 3 * L * self.expert_inter
                + 2 * bt * L * d + 2 * bt * 3 * d * self.n_shared * self.shared_inter)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "tiny_fp32": Config("tiny_fp32", bt=64, d=256, latent=64, n_experts=16, top_k=2,
                        expert_inter=64, n_shared=1, shared_inter=128,
                        act="f32", weight="f32", router="f32", cutoff="batch"),
    "mid_bf16": Config("mid_bf16", bt=4096, d=2048, latent=512, n_experts=64, top_k=8,
                       expert_inter=512, n_shared=2, shared_inter=1024, cutoff="given"),
    "k3_decode_bf16": Config("k3_decode_bf16", bt=64, d=7168, latent=3584, n_experts=896,
                             top_k=16, expert_inter=3072, n_shared=2, shared_inter=3072,
                             cutoff="given"),
    "k3_prefill_bf16": Config("k3_prefill_bf16", bt=16384, d=7168, latent=3584,
                              n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                              shared_inter=3072, bias="zipf1.1", cutoff="batch"),
    "k3_prefill_fp8": Config("k3_prefill_fp8", bt=8192, d=7168, latent=3584, n_experts=896,
                             top_k=16, expert_inter=3072, n_shared=2, shared_inter=3072,
                             weight="fp8", router="bf16", cutoff="batch"),
    # the routed experts in MXFP4 (E2M1 codes, E8M0 scale per 32 inputs), as the
    # released checkpoint stores them; every other weight bf16
    "k3_decode_mxfp4": Config("k3_decode_mxfp4", bt=64, d=7168, latent=3584, n_experts=896,
                              top_k=16, expert_inter=3072, n_shared=2, shared_inter=3072,
                              weight="mxfp4", cutoff="given"),
    "k3_prefill_mxfp4": Config("k3_prefill_mxfp4", bt=16384, d=7168, latent=3584,
                               n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                               shared_inter=3072, weight="mxfp4", bias="zipf1.1",
                               cutoff="batch"),
    # MXFP4 experts read MX FP8 activations: the gfx950 block-scaled MFMA (W4A8)
    "k3_prefill_mxfp4_a8": Config("k3_prefill_mxfp4_a8", bt=16384, d=7168, latent=3584,
                                  n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                                  shared_inter=3072, weight="mxfp4", bias="zipf1.1",
                                  cutoff="batch", act_quant="mxfp8"),
    # decode with MX FP8 expert inputs (MXFP4 or MX FP8 experts)
    "k3_decode_mxfp4_a8": Config("k3_decode_mxfp4_a8", bt=64, d=7168, latent=3584,
                                 n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                                 shared_inter=3072, weight="mxfp4", cutoff="given",
                                 act_quant="mxfp8"),
    "k3_decode_mxfp8": Config("k3_decode_mxfp8", bt=64, d=7168, latent=3584, n_experts=896,
                              top_k=16, expert_inter=3072, n_shared=2, shared_inter=3072,
                              weight="mxfp8", cutoff="given", act_quant="mxfp8"),
    # low-batch decode with Zipf-skewed routing (popular experts), the MXFP4 experts
    # in host DRAM and 112 of them (1/8) cached in HBM
    "k3_decode_mxfp4_tier": Config("k3_decode_mxfp4_tier", bt=8, d=7168, latent=3584,
                                   n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                                   shared_inter=3072, weight="mxfp4", bias="zipf1.1",
                                   cutoff="given", tier_slots=112),
    # the routed experts in MX FP8 (e4m3 codes, E8M0 scale per 32 inputs) reading MX
    # FP8 activations: both operands on the block-scaled MFMA (W8A8)
    "k3_prefill_mxfp8": Config("k3_prefill_mxfp8", bt=16384, d=7168, latent=3584,
                               n_experts=896, top_k=16, expert_inter=3072, n_shared=2,
                               shared_inter=3072, weight="mxfp8", bias="zipf1.1",
                               cutoff="batch", act_quant="mxfp8"),
    # one GPU's share of K3 prefill under 8-way expert parallelism: its own 16384 tokens
    # through the replicated dense parts, and 262144 pairs over its 112 experts
    # (about 2341 rows per expert), so the grouped GEMMs run at the sharded shape
    "k3_ep8_share_bf16": Config("k3_ep8_share_bf16", bt=16384, d=7168, latent=3584,
                                n_experts=112, top_k=16, expert_inter=3072, n_shared=2,
                                shared_inter=3072, cutoff="batch"),
}


# ---- tensor catalogue -------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    shape: tuple          # storage shape, row-major, weights [out][in] (MXFP4: [out][in/2])
    dtype: int
    fan_in: int           # sets sigma = 1/sqrt(fan_in) for weights
    mat_rows: int         # rows / cols (elements) of one matrix (block scales tile these)
    mat_cols: int
    n_mats: int

    @property
    def numel(self) -> int:
        """Storage units (elements; bytes of two elements for MXFP4)."""
        return int(np.prod(self.shape))

    @property
    def mat_units(self) -> int:
        return self.mat_rows * self.mat_cols // (2 if self.dtype == MXFP4 else 1)

    @property
    def nbytes(self) -> int:
        return self.numel * ELEM_BYTES[self.dtype]

    @property
    def n_scale_blocks(self) -> int:
        if self.dtype in MX_DTYPES:
            return self.n_mats * self.mat_rows * (self.mat_cols // MX_BLOCK)
        return self.n_mats * (self.mat_rows // FP8_BLOCK) * (self.mat_cols // FP8_BLOCK)

    @property
    def scale_shape(self) -> tuple:
        if self.dtype in MX_DTYPES:
            return (self.n_mats, self.mat_rows, self.mat_cols // MX_BLOCK)
        return (self.n_mats, self.mat_rows // FP8_BLOCK, self.mat_cols // FP8_BLOCK)


def specs(cfg: Config) -> Dict[str, Spec]:
    d, L, E, I, S, Is = (cfg.d, cfg.latent, cfg.n_experts, cfg.expert_inter, cfg.n_shared,
                         cfg.shared_inter)
    a, w, r = DTYPE_NAMES[cfg.act], DTYPE_NAMES[cfg.weight], DTYPE_NAMES[cfg.router]
    # MXFP4 / MX FP8 apply to the routed experts; the dense weights stay bf16
    xw = w
    if w in MX_DTYPES:
        w = BF16
    h = 2 if xw == MXFP4 else 1  # elements per storage unit of the experts
    return {
        "x": Spec("x", (cfg.bt, d), a, 1, cfg.bt, d, 1),
        "w_router": Spec("w_router", (E, d), r, d, E, d, 1),
        "w_down_proj": Spec("w_down_proj", (L, d), w, d, L, d, 1),
        "w_gate": Spec("w_gate", (E, I, L // h), xw, L, I, L, E),
        "w_up": Spec("w_up", (E, I, L // h), xw, L, I, L, E),
        "w_down": Spec("w_down", (E, L, I // h), xw, I, L, I, E),
        "w_up_proj": Spec("w_up_proj", (d, L), w, L, d, L, 1),
        "sh_gate": Spec("sh_gate", (S, Is, d), w, d, Is, d, S),
        "sh_up": Spec("sh_up", (S, Is, d), w, d, Is, d, S),
        "sh_down": Spec("sh_down", (S, d, Is), w, S * Is, d, Is, S),
    }


WEIGHT_NAMES = ("w_router", "w_down_proj", "w_gate", "w_up", "w_down", "w_up_proj",
                "sh_gate", "sh_up", "sh_down")
FP8_NAMES = ("w_down_proj", "w_gate", "w_up", "w_down", "w_up_proj", "sh_gate", "sh_up",
             "sh_down")


def dyadic_router_shift(d: int) -> int:
    """q such that dyadic router weights k * 2^-q (|k| <= 8) against dyadic
    tokens (|x| <= 2) give logits of roughly unit spread."""
    return int(round(math.log2(math.sqrt(d * 2 * 24))))


def draw_params(cfg: Config, name: str, routing: str = "normal"):
    """(kind, scale, range) of the draw that fills tensor `name`."""
    sp = specs(cfg)[name]
    if routing == "dyadic" and name == "x":
        return DYADIC, 1.0, 2
    if routing == "dyadic" and name == "w_router":
        return DYADIC, 2.0 ** -dyadic_router_shift(cfg.d), 8
    if sp.dtype == FP8:
        return NORMAL, FP8_MAX / NORMAL_INT_MAX, 0
    if sp.dtype == MXFP4:
        return NORMAL, float(np.float32(MX_CODE_SIGMA / NORMAL_INT_STD)), 0
    if sp.dtype == MXFP8:
        return NORMAL, float(np.float32(MX8_CODE_SIGMA / NORMAL_INT_STD)), 0
    sigma = 1.0 if (name == "x" or sp.fan_in == 0) else 1.0 / math.sqrt(sp.fan_in)
    return NORMAL, float(np.float32(sigma / NORMAL_INT_STD)), 0


def mx_centre(cfg: Config, name: str) -> int:
    """Centre E8M0 code of the MXFP4 / MX FP8 block scales of `name`: decoded
    weights then have standard deviation ~ 1/sqrt(fan_in) (within a factor
    sqrt 2)."""
    sp = specs(cfg)[name]
    sigma = 1.0 / math.sqrt(max(sp.fan_in, 1))
    code_std = MX_CODE_STD if sp.dtype == MXFP4 else MX8_CODE_SIGMA
    return 127 + int(round(math.log2(sigma / (code_std * MX_SCALE_RMS))))


def scale_base(cfg: Config, name: str) -> float:
    """Centre of the fp8 block scales of `name`: dequantised codes then have
    standard deviation ~ 1/sqrt(fan_in)."""
    sp = specs(cfg)[name]
    sigma = 1.0 / math.sqrt(max(sp.fan_in, 1))
    return sigma * (NORMAL_INT_MAX / FP8_MAX) / NORMAL_INT_STD


# ---- native libraries ---------------------------------------------------------

_host = None
_dev = None


def lib_host():
    global _host
    if _host is None:
        path = os.path.join(HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_int32]
        lib.synth_fill_host.restype = ctypes.c_int
        lib.synth_philox_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_normal_int_host.argtypes = [ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_uint64]
        lib.synth_normal_int_host.restype = ctypes.c_int32
        lib.synth_bf16_host.argtypes = [ctypes.c_float]
        lib.synth_bf16_host.restype = ctypes.c_uint16
        lib.synth_e4m3_host.argtypes = [ctypes.c_float]
        lib.synth_e4m3_host.restype = ctypes.c_uint8
        lib.synth_e2m1_host.argtypes = [ctypes.c_float]
        lib.synth_e2m1_host.restype = ctypes.c_uint8
        lib.synth_block_scales_host.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.c_uint64, ctypes.c_uint32,
                                                ctypes.c_double]
        lib.synth_zipf_offsets_host.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.c_double]
        lib.synth_routing_host.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                           ctypes.c_int64]
        _host = lib
    return _host


def lib_dev():
    global _dev
    if _dev is None:
        path = os.path.join(HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (torch's HIP runtime first: one runtime per process)
        lib = ctypes.CDLL(path)
        lib.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_float, ctypes.c_int32,
                                          ctypes.c_void_p]
        lib.synth_fill_device.restype = ctypes.c_int
        _dev = lib
    return _dev


# ---- host-side generation -------------------------------------------------------

def host_fill(dtype: int, n: int, seed: int, tid: int, offset: int, kind: int, scale: float,
              rng: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8 if dtype == E8M0 else NP_STORAGE[dtype])
    rc = lib_host().synth_fill_host(out.ctypes.data, FP8 if dtype == MXFP8 else dtype, n, seed,
                                    tid, offset, kind, scale, rng)
    if rc != 0:
        raise ValueError("synth_fill_host rejected its arguments")
    return out


def host_tensor(cfg: Config, name: str, seed: int = 0, routing: str = "normal",
                start: int = 0, count: Optional[int] = None) -> np.ndarray:
    """Raw storage (float32 / uint16 bf16 bits / uint8 e4m3 codes / uint8 bytes
    of two MXFP4 codes) of storage units start..start+count of tensor `name`,
    flat."""
    sp = specs(cfg)[name]
    if count is None:
        count = sp.numel - start
    kind, scale, rng = draw_params(cfg, name, routing)
    return host_fill(sp.dtype, count, seed, TID[name], start, kind, scale, rng)


def host_matrix(cfg: Config, name: str, index: int = 0, seed: int = 0,
                routing: str = "normal") -> np.ndarray:
    """Matrix `index` (an expert, a shared expert) of tensor `name`, 2-D raw storage."""
    sp = specs(cfg)[name]
    n = sp.mat_units
    return host_tensor(cfg, name, seed, routing, index * n, n).reshape(sp.mat_rows,
                                                                      n // sp.mat_rows)


def host_rows(cfg: Config, name: str, rows, seed: int = 0, routing: str = "normal"):
    """Selected rows of a 2-D tensor (e.g. token rows of x), raw storage."""
    sp = specs(cfg)[name]
    cols = sp.shape[-1]
    return np.stack([host_tensor(cfg, name, seed, routing, int(r) * cols, cols)
                     for r in rows]) if len(rows) else np.zeros((0, cols),
                                                                 NP_STORAGE[sp.dtype])


def host_scales(cfg: Config, name: str, seed: int = 0) -> Optional[np.ndarray]:
    """fp32 block scales [n_mats][rows/128][cols/128] of an fp8 tensor, uint8
    E8M0 codes [n_mats][rows][cols/32] of an MXFP4 or MX FP8 tensor, else None."""
    sp = specs(cfg)[name]
    if sp.dtype in MX_DTYPES:
        return host_fill(E8M0, sp.n_scale_blocks, seed, SCALE_TID_BASE + TID[name], 0, NORMAL,
                         0.0, mx_centre(cfg, name)).reshape(sp.scale_shape)
    if sp.dtype != FP8:
        return None
    out = np.empty(sp.n_scale_blocks, dtype=np.float32)
    rc = lib_host().synth_block_scales_host(out.ctypes.data, out.size, seed,
                                            SCALE_TID_BASE + TID[name],
                                            scale_base(cfg, name))
    if rc != 0:
        raise ValueError("synth_block_scales_host rejected its arguments")
    return out.reshape(sp.n_mats, sp.mat_rows // FP8_BLOCK, sp.mat_cols // FP8_BLOCK)


def router_bias(cfg: Config) -> Optional[np.ndarray]:
    """Per-expert logit offsets, or None for a bias-free router."""
    if cfg.bias == "zero":
        return None
    if cfg.bias.startswith("zipf"):
        s = float(cfg.bias[4:])
        out = np.empty(cfg.n_experts, dtype=np.float32)
        lib_host().synth_zipf_offsets_host(out.ctypes.data, cfg.n_experts, s)
        return out
    raise ValueError(cfg.bias)


def gamma(cfg: Config) -> np.ndarray:
    return np.ones(cfg.latent, dtype=np.float32)


def routing_fixture(bt: int, k: int, n_experts: int, seed: int = 0, hot: int = 0,
                    tid: int = 50) -> np.ndarray:
    """[bt][k] int32 expert ids, distinct and ascending per token."""
    out = np.empty((bt, k), dtype=np.int32)
    rc = lib_host().synth_routing_host(out.ctypes.data, bt, k, n_experts, seed, tid, hot)
    if rc != 0:
        raise ValueError("synth_routing_host rejected its arguments")
    return out


def host_layer(cfg: Config, seed: int = 0, routing: str = "normal") -> dict:
    """Every tensor of a (small) layer on the host, raw storage, shaped."""
    out = {}
    for name, sp in specs(cfg).items():
        out[name] = host_tensor(cfg, name, seed, routing).reshape(sp.shape)
        sc = host_scales(cfg, name, seed)
        if sc is not None:
            out["scale:" + name] = sc
    out["router_bias"] = router_bias(cfg)
    out["gamma"] = gamma(cfg)
    return out


# ---- device-side generation (needs torch with a GPU) -------------------------------

def device_layer(cfg: Config, seed: int = 0, routing: str = "normal", device="cuda",
                 names=None) -> dict:
    """Every tensor of the layer generated directly in device memory (torch
    tensors of the raw storage dtype).  Same bits as host_layer()."""
    import torch
    tdt = {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.uint8, MXFP4: torch.uint8,
           MXFP8: torch.uint8}
    stream = torch.cuda.current_stream().cuda_stream

    def fill(t, dtype, n, tid, kind, scale, rng, what):
        rc = lib_dev().synth_fill_device(ctypes.c_void_p(t.data_ptr()),
                                         FP8 if dtype == MXFP8 else dtype, n, seed, tid, 0,
                                         kind, scale, rng, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"synth_fill_device failed ({rc}) for {what}")

    out = {}
    for name, sp in specs(cfg).items():
        if names is not None and name not in names:
            continue
        t = torch.empty(sp.shape, dtype=tdt[sp.dtype], device=device)
        kind, scale, rng = draw_params(cfg, name, routing)
        fill(t, sp.dtype, sp.numel, TID[name], kind, scale, rng, name)
        out[name] = t
        if sp.dtype in MX_DTYPES:
            sc = torch.empty(sp.scale_shape, dtype=torch.uint8, device=device)
            fill(sc, E8M0, sp.n_scale_blocks, SCALE_TID_BASE + TID[name], NORMAL, 0.0,
                 mx_centre(cfg, name), "scale:" + name)
            out["scale:" + name] = sc
            continue
        sc = host_scales(cfg, name, seed)
        if sc is not None:
            out["scale:" + name] = torch.from_numpy(sc).to(device)
    b = router_bias(cfg)
    out["router_bias"] = None if b is None else torch.from_numpy(b).to(device)
    out["gamma"] = torch.from_numpy(gamma(cfg)).to(device)
    return out


# ---- the C ABI's names for a generated layer ----------------------------------------
# (name mapping only: a generated tensor goes to the moe_weights field of the
# same meaning; fp8 block scales to s_*, MX E8M0 codes of the experts to e8_*)

ABI_NAME = {"w_router": "w_router", "router_bias": "router_bias", "w_down_proj": "w_down_proj",
            "w_gate": "w_gate", "w_up": "w_up", "w_down": "w_down", "gamma": "latent_gamma",
            "w_up_proj": "w_up_proj", "sh_gate": "sh_gate", "sh_up": "sh_up",
            "sh_down": "sh_down"}
SCALE_ABI = {"w_down_proj": "s_down_proj", "w_gate": "s_gate", "w_up": "s_up",
             "w_down": "s_down", "w_up_proj": "s_up_proj", "sh_gate": "s_sh_gate",
             "sh_up": "s_sh_up", "sh_down": "s_sh_down"}
MX_ABI = {"w_gate": "e8_gate", "w_up": "e8_up", "w_down": "e8_down"}


def abi_config_args(cfg: Config, cutoff: Optional[str] = None) -> dict:
    """Keyword arguments of the binding's make_config for this workload: the
    weight dtype names the ABI's (MXFP4 experts with MX FP8 inputs are
    "mxfp4_a8")."""
    weight = cfg.weight
    mx8_in = cfg.act_quant == "mxfp8"
    if weight == "mxfp8":
        assert mx8_in, "MX FP8 experts read MX FP8 inputs"
    elif mx8_in:
        assert weight == "mxfp4", "MX FP8 expert inputs go with MX experts"
        weight = "mxfp4_a8"
    return dict(d=cfg.d, latent=cfg.latent, n_experts=cfg.n_experts, top_k=cfg.top_k,
                expert_inter=cfg.expert_inter, n_shared=cfg.n_shared,
                shared_inter=cfg.shared_inter, beta=cfg.beta, beta_u=cfg.beta_u,
                rms_eps=cfg.rms_eps, act=cfg.act, weight=weight, router=cfg.router,
                cutoff=cutoff or cfg.cutoff)


def abi_tensors(cfg: Config, lay: dict) -> dict:
    """A device_layer() dict re-keyed by moe_weights field names (x left out)."""
    t = {}
    for k, v in lay.items():
        if k == "x" or v is None:
            continue
        if k.startswith("scale:"):
            mx = cfg.weight in ("mxfp4", "mxfp8") and k[6:] in MX_ABI
            t[(MX_ABI if mx else SCALE_ABI)[k[6:]]] = v
        else:
            t[ABI_NAME[k]] = v
    return t


# ---- dense layer-1 FFN workloads ----------------------------------------------------------
# mkdocs.reaper.mx "Vue d'ensemble de l'architecture": layer 1 is a dense SiTU-GLU FFN
# of intermediate width 33 792 (section "Le décompte des couches"), pre-RMSNorm with
# its output summed into the block representation (section "Ce que fait une couche").

FFN_TID = {"x": 20, "r": 21, "w_gate": 22, "w_up": 23, "w_down": 24}


@dataclasses.dataclass(frozen=True)
class FfnConfig:
    name: str
    bt: int
    d: int
    inter: int
    act: str = "bf16"
    beta: float = 4.0
    beta_u: float = 25.0
    rms_eps: float = 1e-6

    @property
    def expert_inter(self) -> int:  # the oracle's name for the intermediate width
        return self.inter

    def flops(self) -> int:
        return 2 * self.bt * 3 * self.d * self.inter

    def with_(self, **kw) -> "FfnConfig":
        return dataclasses.replace(self, **kw)


FFN_CONFIGS: Dict[str, FfnConfig] = {
    "ffn_tiny_fp32": FfnConfig("ffn_tiny_fp32", bt=64, d=256, inter=384, act="f32"),
    "ffn_mid_bf16": FfnConfig("ffn_mid_bf16", bt=1024, d=2048, inter=5632),
    "k3_dense_ffn_prefill_bf16": FfnConfig("k3_dense_ffn_prefill_bf16", bt=16384, d=7168,
                                           inter=33792),
    "k3_dense_ffn_decode_bf16": FfnConfig("k3_dense_ffn_decode_bf16", bt=64, d=7168,
                                          inter=33792),
}


def ffn_specs(cfg: FfnConfig) -> Dict[str, Spec]:
    a = DTYPE_NAMES[cfg.act]
    d, I = cfg.d, cfg.inter
    return {
        "x": Spec("x", (cfg.bt, d), a, 1, cfg.bt, d, 1),
        "r": Spec("r", (cfg.bt, d), a, 1, cfg.bt, d, 1),
        "w_gate": Spec("w_gate", (I, d), a, d, I, d, 1),
        "w_up": Spec("w_up", (I, d), a, d, I, d, 1),
        "w_down": Spec("w_down", (d, I), a, I, d, I, 1),
    }


def ffn_draw_params(cfg: FfnConfig, name: str):
    sp = ffn_specs(cfg)[name]
    sigma = 1.0 if name in ("x", "r") else 1.0 / math.sqrt(sp.fan_in)
    return NORMAL, float(np.float32(sigma / NORMAL_INT_STD)), 0


def ffn_gamma(cfg: FfnConfig) -> np.ndarray:
    """RMSNorm gain (7/6)(0.75 + 0.5 u), u uniform in [0, 1): values in [0.875, 1.46),
    so a dropped or misplaced gain shows."""
    out = np.empty(cfg.d, dtype=np.float32)
    lib_host().synth_block_scales_host(out.ctypes.data, cfg.d, 0, 30, 7.0 / 6.0)
    return out


def ffn_host_tensor(cfg: FfnConfig, name: str, seed: int = 0, start: int = 0,
                    count: Optional[int] = None) -> np.ndarray:
    sp = ffn_specs(cfg)[name]
    if count is None:
        count = sp.numel - start
    kind, scale, rng = ffn_draw_params(cfg, name)
    return host_fill(sp.dtype, count, seed, FFN_TID[name], start, kind, scale, rng)


def ffn_host_rows(cfg: FfnConfig, name: str, rows, seed: int = 0) -> np.ndarray:
    sp = ffn_specs(cfg)[name]
    cols = sp.shape[-1]
    return np.stack([ffn_host_tensor(cfg, name, seed, int(r) * cols, cols) for r in rows])


def ffn_host_layer(cfg: FfnConfig, seed: int = 0) -> dict:
    out = {n: ffn_host_tensor(cfg, n, seed).reshape(sp.shape)
           for n, sp in ffn_specs(cfg).items()}
    out["gamma"] = ffn_gamma(cfg)
    return out


def ffn_device_layer(cfg: FfnConfig, seed: int = 0, device="cuda") -> dict:
    """Every tensor of the FFN generated in device memory (same bits as ffn_host_layer)."""
    import torch
    tdt = {F32: torch.float32, BF16: torch.bfloat16}
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, sp in ffn_specs(cfg).items():
        t = torch.empty(sp.shape, dtype=tdt[sp.dtype], device=device)
        kind, scale, rng = ffn_draw_params(cfg, name)
        rc = lib_dev().synth_fill_device(ctypes.c_void_p(t.data_ptr()), sp.dtype, sp.numel, seed,
                                         FFN_TID[name], 0, kind, scale, rng,
                                         ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"synth_fill_device failed ({rc}) for {name}")
        out[name] = t
    out["gamma"] = torch.from_numpy(ffn_gamma(cfg)).to(device)
    return out
