"""Stable LatentMoE layer forward on one MI355X (gfx950).

Python binding of ``libmoe.so``, the C ABI declared in ``include/moe.h``:
``moe_workspace_bytes``, ``moe_route``, ``moe_dispatch``, ``moe_forward``,
``moe_status_str``.  This module only marshals arguments: every step of the
layer runs in the library's HIP kernels.  PyTorch provides device memory and
streams (``tensor.data_ptr()``, ``torch.cuda.current_stream()``).  There is no
fallback: if the library is missing the import of this module fails.

The layer (Kimi K3 Stable LatentMoE): tech.news18a.com
"KimiK3的StableLatentMoE架构解析" figures 1-2 and its three techniques;
mkdocs.reaper.mx "Vue d'ensemble de l'architecture", per-token steps c-g.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8E4M3_B128, MOE_MXFP4, MOE_MXFP4_A8, MOE_MXFP8 = 0, 1, 2, 3, 4, 5
CUTOFF_GIVEN, CUTOFF_BATCH, CUTOFF_RUNNING = 0, 1, 2
# "mxfp4_a8": MXFP4 experts with their inputs quantised to MX FP8 in the layer;
# "mxfp8": MX FP8 experts, inputs likewise
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8E4M3_B128, "mxfp4": MOE_MXFP4,
          "mxfp4_a8": MOE_MXFP4_A8, "mxfp8": MOE_MXFP8}
CUTOFFS = {"given": CUTOFF_GIVEN, "batch": CUTOFF_BATCH, "running": CUTOFF_RUNNING}

_P = ctypes.c_void_p


class MoeConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("latent", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("expert_inter", ctypes.c_int64), ("n_shared", ctypes.c_int64),
                ("shared_inter", ctypes.c_int64), ("beta", ctypes.c_float),
                ("beta_u", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("cutoff_mode", ctypes.c_int32)]


WEIGHT_FIELDS = ("w_router", "router_bias", "cutoff", "w_down_proj", "w_gate", "w_up",
                 "w_down", "latent_gamma", "w_up_proj", "sh_gate", "sh_up", "sh_down",
                 "s_down_proj", "s_gate", "s_up", "s_down", "s_up_proj", "s_sh_gate",
                 "s_sh_up", "s_sh_down", "e8_gate", "e8_up", "e8_down", "expert_tab")


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in WEIGHT_FIELDS]


class MoeFfnConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("inter", ctypes.c_int64), ("beta", ctypes.c_float),
                ("beta_u", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32)]


class MoeFfnWeights(ctypes.Structure):
    _fields_ = [("w_gate", _P), ("w_up", _P), ("w_down", _P), ("gamma", _P)]


class MoeTierDesc(ctypes.Structure):
    _fields_ = [("h_gate", _P), ("h_up", _P), ("h_down", _P), ("h_e8_gate", _P),
                ("h_e8_up", _P), ("h_e8_down", _P), ("n_slots", ctypes.c_int64),
                ("slots", _P), ("table", _P), ("counts_acc", _P), ("counts_host", _P),
                ("decay", ctypes.c_float),
                ("max_loads", ctypes.c_int64)]


TIER_STATS = ("forwards", "harvested", "pairs", "pairs_hbm", "loads", "evictions",
              "bytes_loaded", "resident")


class MoeTierStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in TIER_STATS]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_idx", _P), ("topk_w", _P), ("cutoff", _P), ("logits", _P)]


class MoeDispatchOut(ctypes.Structure):
    _fields_ = [("counts", _P), ("offsets", _P), ("perm", _P), ("inv_perm", _P)]


GRAD_FIELDS = ("dx", "w_router", "router_bias", "w_down_proj", "w_gate", "w_up", "w_down",
               "latent_gamma", "w_up_proj", "sh_gate", "sh_up", "sh_down")


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class MoeGemmDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a", _P), ("lda", ctypes.c_int64), ("a_kouter", ctypes.c_int32),
                ("b", _P), ("ldb", ctypes.c_int64), ("b_kouter", ctypes.c_int32),
                ("c", _P), ("ldc", ctypes.c_int64), ("c_in", _P), ("k_offsets", _P),
                ("n_experts", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    # One HIP runtime per process: torch ships its own libamdhip64, and every
    # HIP library loaded later binds to whichever copy was loaded first.  Load
    # it through torch before this library, so torch's device memory, streams
    # and the library's launches all go through the same runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    CP = ctypes.POINTER
    lib.moe_workspace_bytes.argtypes = [CP(MoeConfig), ctypes.c_int64]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_backward_workspace_bytes.argtypes = [CP(MoeConfig), ctypes.c_int64]
    lib.moe_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_backward.argtypes = [CP(MoeConfig), CP(MoeWeights), _P, ctypes.c_int64, _P, _P, _P,
                                 CP(MoeGrads), _P, ctypes.c_size_t, _P]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_route.argtypes = [CP(MoeConfig), CP(MoeWeights), _P, ctypes.c_int64,
                              CP(MoeRouteOut), _P, ctypes.c_size_t, _P]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [CP(MoeConfig), _P, ctypes.c_int64, CP(MoeDispatchOut), _P,
                                 ctypes.c_size_t, _P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_forward.argtypes = [CP(MoeConfig), CP(MoeWeights), _P, ctypes.c_int64, _P,
                                CP(MoeRouteOut), CP(MoeDispatchOut), _P, ctypes.c_size_t, _P,
                                _P]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [CP(MoeConfig), CP(MoeWeights), _P, ctypes.c_int64, _P,
                                        CP(MoeRouteOut), CP(MoeDispatchOut), _P, _P]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_ffn_workspace_bytes.argtypes = [CP(MoeFfnConfig), ctypes.c_int64]
    lib.moe_ffn_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_ffn_forward.argtypes = [CP(MoeFfnConfig), CP(MoeFfnWeights), _P, _P, ctypes.c_int64,
                                    _P, _P, ctypes.c_size_t, _P]
    lib.moe_ffn_forward.restype = ctypes.c_int
    lib.moe_cutoff_update.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_float, _P]
    lib.moe_cutoff_update.restype = ctypes.c_int
    lib.moe_tier_slot_bytes.argtypes = [CP(MoeConfig)]
    lib.moe_tier_slot_bytes.restype = ctypes.c_size_t
    lib.moe_tier_create.argtypes = [CP(MoeConfig), CP(MoeTierDesc), _P, CP(_P)]
    lib.moe_tier_create.restype = ctypes.c_int
    lib.moe_tier_plan.argtypes = [_P, _P, _P]
    lib.moe_tier_plan.restype = ctypes.c_int
    lib.moe_tier_observe.argtypes = [_P, _P, _P]
    lib.moe_tier_observe.restype = ctypes.c_int
    lib.moe_tier_get_stats.argtypes = [_P, CP(MoeTierStats)]
    lib.moe_tier_get_stats.restype = ctypes.c_int
    lib.moe_tier_destroy.argtypes = [_P]
    lib.moe_tier_destroy.restype = ctypes.c_int
    lib.moe_tier_select.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P,
                                    _P]
    lib.moe_tier_select.restype = ctypes.c_int64
    lib.moe_mx8_quantize.argtypes = [_P, ctypes.c_int64, _P, _P, _P]
    lib.moe_mx8_quantize.restype = ctypes.c_int
    lib.moe_gemm_bf16.argtypes = [CP(MoeGemmDesc), _P]
    lib.moe_gemm_bf16.restype = ctypes.c_int
    lib.moe_situ_eval.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_float, ctypes.c_float, _P, _P,
                                  _P, _P]
    lib.moe_situ_eval.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_profile_enable.argtypes = [ctypes.c_int]
    lib.moe_profile_enable.restype = ctypes.c_int
    lib.moe_profile_read.argtypes = [_P, _P]
    lib.moe_profile_read.restype = ctypes.c_int
    lib.moe_profile_phase_name.argtypes = [ctypes.c_int]
    lib.moe_profile_phase_name.restype = ctypes.c_char_p
    return lib


LIB = _load()

EXPORTED = ("moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_forward",
            "moe_status_str", "moe_profile_enable", "moe_profile_read",
            "moe_profile_phase_name", "moe_ffn_workspace_bytes", "moe_ffn_forward",
            "moe_mx8_quantize", "moe_tier_slot_bytes", "moe_tier_create", "moe_tier_plan",
            "moe_tier_observe", "moe_tier_get_stats", "moe_tier_destroy", "moe_tier_select",
            "moe_cutoff_update", "moe_backward_workspace_bytes", "moe_backward",
            "moe_situ_eval", "moe_forward_noalloc", "moe_gemm_bf16")

# bytes of the library-held workspace of moe_forward_noalloc (one array per GPU)
NOALLOC_SCRATCH_BYTES = 128 << 20


def cutoff_update(alpha, zeta, rate: float):
    """alpha += rate * (zeta - alpha) on the device (fp32 tensors of E)."""
    import torch
    st = LIB.moe_cutoff_update(_P(alpha.data_ptr()), _P(zeta.data_ptr()), alpha.numel(),
                               float(rate), _P(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise MoeError(st, "moe_cutoff_update")


# ---- expert tiering -----------------------------------------------------------------

def tier_slot_bytes(cfg: MoeConfig) -> int:
    return int(LIB.moe_tier_slot_bytes(ctypes.byref(cfg)))


def tier_select(score, resident, n_slots: int, max_loads: int):
    """The cache policy alone (host only): (load ids, victim ids or -1)."""
    import numpy as np
    score = np.ascontiguousarray(score, np.float32)
    resident = np.ascontiguousarray(resident, np.uint8)
    load = np.empty(max(max_loads, 1), np.int32)
    victim = np.empty(max(max_loads, 1), np.int32)
    n = LIB.moe_tier_select(score.ctypes.data, resident.ctypes.data, score.size, n_slots,
                            max_loads, load.ctypes.data, victim.ctypes.data)
    if n < 0:
        raise MoeError(-1, "moe_tier_select")
    return load[:n].copy(), victim[:n].copy()


class ExpertTier:
    """Routed experts in pinned host memory with an HBM cache of n_slots experts
    (moe_tier_*).  `host` maps w_gate / w_up / w_down (and e8_* for the MX
    dtypes) to pinned CPU tensors in the stacked layout.  Pass `table` as the
    layer's expert_tab; call plan() before and observe(counts) after each
    forward."""

    def __init__(self, cfg: MoeConfig, host: dict, n_slots: int, decay: float = 0.9,
                 max_loads: int = 32):
        import torch
        self.cfg = cfg
        self.host = dict(host)
        E = cfg.n_experts
        sb = tier_slot_bytes(cfg)
        if sb == 0:
            raise MoeError(-2, "moe_tier_slot_bytes")
        self.slots = torch.empty(max(n_slots * sb, 256), dtype=torch.uint8, device="cuda")
        self.table = torch.empty(6 * E, dtype=torch.int64, device="cuda")
        self.counts_acc = torch.empty(E + 2, dtype=torch.int32, device="cuda")
        self.counts_host = torch.empty(E + 2, dtype=torch.int32, pin_memory=True)
        desc = MoeTierDesc(*(_ptr(self.host.get(n)) for n in ("w_gate", "w_up", "w_down",
                                                              "e8_gate", "e8_up", "e8_down")),
                           n_slots, self.slots.data_ptr(), self.table.data_ptr(),
                           self.counts_acc.data_ptr(), self.counts_host.data_ptr(), decay,
                           max_loads)
        h = _P()
        st = LIB.moe_tier_create(ctypes.byref(cfg), ctypes.byref(desc),
                                 _P(torch.cuda.current_stream().cuda_stream), ctypes.byref(h))
        if st != 0:
            raise MoeError(st, "moe_tier_create")
        self.handle = h

    def plan(self, copy_stream=None):
        import torch
        st = LIB.moe_tier_plan(self.handle, _P(torch.cuda.current_stream().cuda_stream),
                               _P(copy_stream.cuda_stream if copy_stream is not None else 0))
        if st != 0:
            raise MoeError(st, "moe_tier_plan")

    def observe(self, counts):
        import torch
        st = LIB.moe_tier_observe(self.handle, _P(counts.data_ptr()),
                                  _P(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise MoeError(st, "moe_tier_observe")

    def stats(self) -> dict:
        s = MoeTierStats()
        st = LIB.moe_tier_get_stats(self.handle, ctypes.byref(s))
        if st != 0:
            raise MoeError(st, "moe_tier_get_stats")
        return {n: getattr(s, n) for n in TIER_STATS}

    def close(self):
        if self.handle:
            st = LIB.moe_tier_destroy(self.handle)
            self.handle = None
            if st != 0:
                raise MoeError(st, "moe_tier_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_situ_eval(g: int, u: int, n: int, beta: float, beta_u: float, phi: int, psi: int,
                  h: int, stream: int) -> int:
    return LIB.moe_situ_eval(_P(g or None), _P(u or None), n, float(beta), float(beta_u),
                             _P(phi or None), _P(psi or None), _P(h or None),
                             _P(stream or None))


def gemm_bf16(a, b, a_kouter=False, b_kouter=False, c_in=None, k_offsets=None, out=None):
    """fp32 op(A) op(B) (+ c_in) on the engine: A [M][K] or, K-outer, [K][M];
    B [N][K] or, K-outer, [K][N] (bf16 device tensors).  With k_offsets
    (int32 [E + 1]): E outputs [M][N], expert e over K rows k_offsets[e]..[e+1]."""
    import torch
    M = a.shape[1] if a_kouter else a.shape[0]
    K = a.shape[0] if a_kouter else a.shape[1]
    N = b.shape[1] if b_kouter else b.shape[0]
    E = 0 if k_offsets is None else k_offsets.numel() - 1
    if out is None:
        out = torch.empty(((E,) if E else ()) + (M, N), dtype=torch.float32, device=a.device)
    d = MoeGemmDesc(M, N, K, a.data_ptr(), a.stride(0), int(a_kouter), b.data_ptr(), b.stride(0),
                    int(b_kouter), out.data_ptr(), N, _ptr(c_in), _ptr(k_offsets), E)
    st = LIB.moe_gemm_bf16(ctypes.byref(d), _P(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise MoeError(st, "moe_gemm_bf16")
    return out


def situ_eval(g, u, beta=4.0, beta_u=25.0):
    """(phi(g), psi(u), phi(g) psi(u)) of fp32 device tensors, by the device
    functions of the GEMM epilogues."""
    import torch
    g = g.contiguous()
    u = u.contiguous()
    phi, psi, h = (torch.empty_like(g) for _ in range(3))
    st = moe_situ_eval(g.data_ptr(), u.data_ptr(), g.numel(), beta, beta_u, phi.data_ptr(),
                       psi.data_ptr(), h.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise MoeError(st, "moe_situ_eval")
    return phi, psi, h


def moe_mx8_quantize(x: int, n: int, codes: int, scales: int, stream: int) -> int:
    return LIB.moe_mx8_quantize(_P(x or None), n, _P(codes or None), _P(scales or None),
                                _P(stream or None))


def mx8_quantize(x):
    """MX FP8 codes (uint8, x's shape) and E8M0 scales (uint8, last dim / 32) of
    a bf16 device tensor, blocks of 32 along the last dimension."""
    import torch
    x = x.contiguous()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((*x.shape[:-1], x.shape[-1] // 32), dtype=torch.uint8, device=x.device)
    st = moe_mx8_quantize(x.data_ptr(), x.numel(), codes.data_ptr(), scales.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise MoeError(st, "moe_mx8_quantize")
    return codes, scales
N_PHASES = 14


def status_str(status: int) -> str:
    return LIB.moe_status_str(int(status)).decode()


def make_config(d, latent, n_experts, top_k, expert_inter, n_shared, shared_inter,
                beta=4.0, beta_u=25.0, rms_eps=1e-6, act="bf16", weight="bf16", router=None,
                cutoff="batch") -> MoeConfig:
    router = act if router is None else router
    return MoeConfig(d, latent, n_experts, top_k, expert_inter, n_shared, shared_inter, beta,
                     beta_u, rms_eps, DTYPES[act], DTYPES[weight], DTYPES[router],
                     CUTOFFS[cutoff])


# ---- pointer-level calls (ints are device addresses; 0 = NULL) --------------------

def workspace_bytes(cfg: MoeConfig, bt: int) -> int:
    return int(LIB.moe_workspace_bytes(ctypes.byref(cfg), bt))


def backward_workspace_bytes(cfg: MoeConfig, bt: int) -> int:
    return int(LIB.moe_backward_workspace_bytes(ctypes.byref(cfg), bt))


def moe_backward(cfg, weights: MoeWeights, x: int, bt: int, topk_idx: int, topk_w: int, dy: int,
                 grads: MoeGrads, ws: int, ws_bytes: int, stream: int) -> int:
    return LIB.moe_backward(ctypes.byref(cfg), ctypes.byref(weights), _P(x or None), bt,
                            _P(topk_idx or None), _P(topk_w or None), _P(dy or None),
                            ctypes.byref(grads), _P(ws or None), ws_bytes, _P(stream or None))


def moe_route(cfg, weights: MoeWeights, x: int, bt: int, out: MoeRouteOut, ws: int,
              ws_bytes: int, stream: int) -> int:
    return LIB.moe_route(ctypes.byref(cfg), ctypes.byref(weights), _P(x or None), bt,
                         ctypes.byref(out), _P(ws or None), ws_bytes, _P(stream or None))


def moe_dispatch(cfg, topk_idx: int, bt: int, out: MoeDispatchOut, ws: int, ws_bytes: int,
                 stream: int) -> int:
    return LIB.moe_dispatch(ctypes.byref(cfg), _P(topk_idx or None), bt, ctypes.byref(out),
                            _P(ws or None), ws_bytes, _P(stream or None))


def moe_forward(cfg, weights: MoeWeights, x: int, bt: int, y: int, route, disp, ws: int,
                ws_bytes: int, stream: int, shared_stream: int = 0) -> int:
    return LIB.moe_forward(ctypes.byref(cfg), ctypes.byref(weights), _P(x or None), bt,
                           _P(y or None), ctypes.byref(route) if route is not None else None,
                           ctypes.byref(disp) if disp is not None else None, _P(ws or None),
                           ws_bytes, _P(stream or None), _P(shared_stream or None))


def moe_forward_noalloc(cfg, weights: MoeWeights, x: int, bt: int, y: int, route, disp,
                        stream: int, shared_stream: int = 0) -> int:
    return LIB.moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _P(x or None), bt,
                                   _P(y or None),
                                   ctypes.byref(route) if route is not None else None,
                                   ctypes.byref(disp) if disp is not None else None,
                                   _P(stream or None), _P(shared_stream or None))


def profile_enable(on: bool) -> None:
    """Per-phase HIP-event timing of moe_forward (measurement support)."""
    LIB.moe_profile_enable(1 if on else 0)


def profile_read() -> dict:
    """{phase name: (average ms per call, calls)} since profiling was enabled."""
    ms = (ctypes.c_double * N_PHASES)()
    calls = (ctypes.c_int64 * N_PHASES)()
    st = LIB.moe_profile_read(ms, calls)
    if st != 0:
        raise MoeError(st, "moe_profile_read")
    return {LIB.moe_profile_phase_name(i).decode(): (ms[i], calls[i]) for i in range(N_PHASES)}


# ---- torch-tensor convenience layer (memory and streams only) -----------------------

def _ptr(t):
    return 0 if t is None else t.data_ptr()


def weights_struct(tensors: dict) -> MoeWeights:
    """MoeWeights from a dict of device tensors keyed by the moe_weights field
    names (missing keys -> NULL)."""
    return MoeWeights(*(_ptr(tensors.get(n)) for n in WEIGHT_FIELDS))


class StableLatentMoE:
    """One layer: a config and its device-resident weights.  The caller's
    tensors are borrowed, not copied."""

    def __init__(self, cfg: MoeConfig, tensors: dict):
        self.cfg = cfg
        self.tensors = dict(tensors)
        self.w = weights_struct(self.tensors)
        self._ws = None

    def workspace(self, bt: int):
        import torch
        need = workspace_bytes(self.cfg, bt)
        if need == 0 and bt > 0:
            raise MoeError(-2, "moe_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def route(self, x, want_logits=False):
        import torch
        bt = x.shape[0]
        E, k = self.cfg.n_experts, self.cfg.top_k
        dev = x.device
        idx = torch.empty((bt, k), dtype=torch.int32, device=dev)
        w = torch.empty((bt, k), dtype=torch.float32, device=dev)
        cut = torch.empty(E, dtype=torch.float32, device=dev)
        logits = torch.empty((bt, E), dtype=torch.float32, device=dev) if want_logits else None
        out = MoeRouteOut(idx.data_ptr(), w.data_ptr(), cut.data_ptr(), _ptr(logits))
        ws = self.workspace(bt)
        st = moe_route(self.cfg, self.w, _ptr(x), bt, out, ws.data_ptr(), ws.numel(),
                       torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise MoeError(st, "moe_route")
        return dict(idx=idx, w=w, cutoff=cut, logits=logits)

    def dispatch(self, idx):
        import torch
        bt = idx.shape[0]
        E, P = self.cfg.n_experts, idx.numel()
        dev = idx.device
        res = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(P, dtype=torch.int32, device=dev),
                   inv_perm=torch.empty(P, dtype=torch.int32, device=dev))
        out = MoeDispatchOut(*(res[n].data_ptr() for n in ("counts", "offsets", "perm",
                                                           "inv_perm")))
        ws = self.workspace(bt)
        st = moe_dispatch(self.cfg, idx.data_ptr(), bt, out, ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise MoeError(st, "moe_dispatch")
        return res

    def forward(self, x, shared_stream=None, return_routing=False, out=None, dispatch=None):
        """y; with return_routing also the routing and dispatch results (new
        tensors).  `dispatch` may instead hold caller-owned counts / offsets /
        perm / inv_perm tensors to receive the dispatch results."""
        import torch
        bt = x.shape[0]
        E, k, P = self.cfg.n_experts, self.cfg.top_k, x.shape[0] * self.cfg.top_k
        dev = x.device
        y = out if out is not None else torch.empty((bt, self.cfg.d), dtype=x.dtype, device=dev)
        route = disp = None
        extra = {}
        if return_routing:
            extra = dict(idx=torch.empty((bt, k), dtype=torch.int32, device=dev),
                         w=torch.empty((bt, k), dtype=torch.float32, device=dev),
                         cutoff=torch.empty(E, dtype=torch.float32, device=dev),
                         logits=torch.empty((bt, E), dtype=torch.float32, device=dev),
                         counts=torch.empty(E, dtype=torch.int32, device=dev),
                         offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                         perm=torch.empty(P, dtype=torch.int32, device=dev),
                         inv_perm=torch.empty(P, dtype=torch.int32, device=dev))
            route = MoeRouteOut(*(extra[n].data_ptr() for n in ("idx", "w", "cutoff",
                                                                "logits")))
            disp = MoeDispatchOut(*(extra[n].data_ptr() for n in ("counts", "offsets", "perm",
                                                                  "inv_perm")))
        elif dispatch is not None:
            disp = MoeDispatchOut(*(dispatch[n].data_ptr() for n in ("counts", "offsets", "perm",
                                                                     "inv_perm")))
        ws = self.workspace(bt)
        st = moe_forward(self.cfg, self.w, _ptr(x), bt, y.data_ptr(), route, disp,
                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream,
                         shared_stream.cuda_stream if shared_stream is not None else 0)
        if st != 0:
            raise MoeError(st, "moe_forward")
        return (y, extra) if return_routing else y

    def grad_shapes(self, bt: int) -> dict:
        c = self.cfg
        E, d, L, I = c.n_experts, c.d, c.latent, c.expert_inter
        S, Is = c.n_shared, c.shared_inter
        return dict(dx=(bt, d), w_router=(E, d), router_bias=(E,), w_down_proj=(L, d),
                    w_gate=(E, I, L), w_up=(E, I, L), w_down=(E, L, I), latent_gamma=(L,),
                    w_up_proj=(d, L), sh_gate=(S, Is, d), sh_up=(S, Is, d),
                    sh_down=(S, d, Is))

    def backward(self, x, dy, route=None, grads=None):
        """fp32 gradients of sum(dy * y) (a dict keyed by GRAD_FIELDS) for y =
        forward(x), given the routing of x (route(x) when None).  `grads` may
        hold caller-owned fp32 tensors of grad_shapes() to receive them."""
        import torch
        bt = x.shape[0]
        if route is None:
            route = self.route(x)
        if grads is None:
            grads = {n: torch.empty(s, dtype=torch.float32, device=x.device)
                     for n, s in self.grad_shapes(bt).items()}
        need = backward_workspace_bytes(self.cfg, bt)
        if need == 0:
            raise MoeError(-2, "moe_backward_workspace_bytes")
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        gs = MoeGrads(*(_ptr(grads.get(n)) for n in GRAD_FIELDS))
        st = moe_backward(self.cfg, self.w, _ptr(x), bt, route["idx"].data_ptr(),
                          route["w"].data_ptr(), _ptr(dy), gs, ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise MoeError(st, "moe_backward")
        return grads


# ---- dense layer-1 FFN -----------------------------------------------------------------

def make_ffn_config(d, inter, beta=4.0, beta_u=25.0, rms_eps=1e-6, act="bf16") -> MoeFfnConfig:
    return MoeFfnConfig(d, inter, beta, beta_u, rms_eps, DTYPES[act])


def ffn_workspace_bytes(cfg: MoeFfnConfig, bt: int) -> int:
    return int(LIB.moe_ffn_workspace_bytes(ctypes.byref(cfg), bt))


def moe_ffn_forward(cfg, weights: MoeFfnWeights, x: int, r: int, bt: int, y: int, ws: int,
                    ws_bytes: int, stream: int) -> int:
    return LIB.moe_ffn_forward(ctypes.byref(cfg), ctypes.byref(weights), _P(x or None),
                               _P(r or None), bt, _P(y or None), _P(ws or None), ws_bytes,
                               _P(stream or None))


class DenseFFN:
    """The dense layer-1 FFN: a config and its device-resident weights
    (w_gate, w_up, w_down, gamma), borrowed, not copied."""

    def __init__(self, cfg: MoeFfnConfig, tensors: dict):
        self.cfg = cfg
        self.tensors = dict(tensors)
        self.w = MoeFfnWeights(*(_ptr(self.tensors.get(n)) for n in
                                 ("w_gate", "w_up", "w_down", "gamma")))
        self._ws = None

    def workspace(self, bt: int):
        import torch
        need = ffn_workspace_bytes(self.cfg, bt)
        if need == 0 and bt > 0:
            raise MoeError(-2, "moe_ffn_workspace_bytes")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def forward(self, x, r=None, out=None):
        """y = r + FFN(RMSNorm(x)); out may be r (in place)."""
        import torch
        bt = x.shape[0]
        y = out if out is not None else torch.empty((bt, self.cfg.d), dtype=x.dtype,
                                                    device=x.device)
        ws = self.workspace(bt)
        st = moe_ffn_forward(self.cfg, self.w, _ptr(x), _ptr(r), bt, y.data_ptr(),
                             ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise MoeError(st, "moe_ffn_forward")
        return y
