// api.hip -- the C ABI declared in include/moe.h: argument validation,
// workspace planning and the launch sequence of the Stable LatentMoE forward.
//
// Launch order of moe_forward (tech.news18a.com "KimiK3的StableLatentMoE架构解析",
// figure 2: two parallel paths from the flattened x; mkdocs.reaper.mx "Vue
// d'ensemble de l'architecture", per-token steps c-g):
//   shared_stream: x_lat = x W_down_proj^T                        (step d)
//                  shared gate/up + SiTU -> hs                    (step g, part 1)
//   stream:        router logits -> cutoffs -> top-k -> dispatch  (step c)
//                  join(x_lat)
//                  grouped gate/up + SiTU, x routing weight -> h  (step e; the
//                    weight is applied before W_d, which is linear)
//                  grouped down -> o                              (step e)
//                  combine + latent RMSNorm -> n                  (step f)
//                  join(shared_stream)
//                  y = [n | hs] [W_up_proj | W_ds,0 | W_ds,1]^T   (steps f, g; the final sum)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "gemm.h"
#include "kernels.h"
#include "moe.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kSplitMaxRows = 256;  // batches up to this size may split K

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t elem_size(int32_t dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8E4M3_B128: return 1;
    case MOE_MXFP4:
    case MOE_MXFP4_A8:
    case MOE_MXFP8: return 2;  // the dense weights of an MX layer are bf16
  }
  return 0;
}

struct Plan {
  int path = PATH_BF16;
  bool fp8 = false;
  int dense_wf = WF_BF16;   // weight format of the dense GEMMs
  int expert_wf = WF_BF16;  // and of the routed experts' GEMMs
  int64_t act_bytes = 2;
  // byte offsets into the workspace
  size_t z, zT, alpha, idx, w, w_sorted, counts, offsets, tile_offsets, perm, inv_perm, masks,
      xlat, h, o, n, hs, split, split_sh, xq, xq_sc, hq, hq_sc, total;
  int64_t split_cap = 0;  // floats in each split-K region (0: split K off)
};

moe_status check_config(const moe_config *c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->d <= 0 || c->latent <= 0 || c->n_experts <= 0 || c->top_k <= 0 ||
      c->expert_inter <= 0 || c->n_shared < 0 || (c->n_shared > 0 && c->shared_inter <= 0))
    return MOE_ERR_INVALID_ARG;
  if (c->cutoff_mode != MOE_CUTOFF_GIVEN && c->cutoff_mode != MOE_CUTOFF_BATCH &&
      c->cutoff_mode != MOE_CUTOFF_RUNNING)
    return MOE_ERR_INVALID_ARG;
  if (elem_size(c->act_dtype) == 0 || elem_size(c->weight_dtype) == 0 ||
      elem_size(c->router_dtype) == 0)
    return MOE_ERR_INVALID_ARG;
  if (!(c->beta > 0.0f) || !(c->beta_u > 0.0f) || !(c->rms_eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (c->n_experts > 1024 || c->top_k > c->n_experts || c->top_k > 64 || c->n_shared > 4)
    return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_F32) {
    if (c->weight_dtype != MOE_F32 || c->router_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else if (c->act_dtype == MOE_BF16) {
    if (c->router_dtype != MOE_BF16 || c->weight_dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  const int64_t q = c->weight_dtype == MOE_FP8E4M3_B128 ? 128 : 64;
  if (c->d % 64 || c->latent % q || c->expert_inter % q || (c->n_shared && c->shared_inter % q))
    return MOE_ERR_UNSUPPORTED;
  // MXFP4 experts: K ranges (latent, expert_inter) of whole 128-element groups
  // (a dword of E8M0 codes), with the codes of a B row (K/32 <= 128) in LDS
  const bool mx = c->weight_dtype == MOE_MXFP4 || c->weight_dtype == MOE_MXFP4_A8 ||
                  c->weight_dtype == MOE_MXFP8;
  if (mx && (c->latent % 128 || c->expert_inter % 128 || c->expert_inter > 4096))
    return MOE_ERR_UNSUPPORTED;
  if (c->weight_dtype == MOE_FP8E4M3_B128 && c->d % 128) return MOE_ERR_UNSUPPORTED;
  // fp8 GEMMs stage the block scales of up to 128 K blocks in LDS
  if (c->weight_dtype == MOE_FP8E4M3_B128 &&
      std::max({c->d, c->latent, c->expert_inter, c->shared_inter}) > 16384)
    return MOE_ERR_UNSUPPORTED;
  // the combine holds a latent row per wavefront in registers (8 chunks of 16 B a lane)
  if (c->latent > (c->act_dtype == MOE_F32 ? 2048 : 4096)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status make_plan(const moe_config *c, int64_t bt, Plan *p) {
  moe_status st = check_config(c);
  if (st != MOE_OK) return st;
  if (bt < 0) return MOE_ERR_INVALID_ARG;
  if (bt * c->top_k > INT32_MAX || bt > INT32_MAX / 64) return MOE_ERR_UNSUPPORTED;
  p->path = c->act_dtype == MOE_F32 ? PATH_F32 : PATH_BF16;
  p->fp8 = c->weight_dtype == MOE_FP8E4M3_B128;
  p->dense_wf = p->fp8 ? WF_FP8 : WF_BF16;
  p->expert_wf = c->weight_dtype == MOE_MXFP4      ? WF_MX4
                 : c->weight_dtype == MOE_MXFP4_A8 ? WF_MX4A8
                 : c->weight_dtype == MOE_MXFP8    ? WF_MX8A8
                                                   : p->dense_wf;
  p->act_bytes = elem_size(c->act_dtype);
  const int64_t E = c->n_experts, k = c->top_k, P = bt * k, L = c->latent;
  // the bf16 engine addresses gathered x_lat rows with 32-bit byte offsets
  if (p->path == PATH_BF16 && bt * L * 2 > (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  // MX FP8 A: the E8M0 codes of A rows are addressed from the matrix start
  // with 32-bit offsets
  if ((p->expert_wf == WF_MX4A8 || p->expert_wf == WF_MX8A8) &&
      P * (c->expert_inter / 32) > (int64_t)UINT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  const int64_t nb = (bt + 63) / 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  p->z = take(4 * bt * E);
  p->zT = take(4 * bt * E);
  p->alpha = take(4 * E);
  p->idx = take(4 * P);
  p->w = take(4 * P);
  p->w_sorted = take(4 * P);
  p->counts = take(4 * E);
  p->offsets = take(4 * (E + 1));
  p->tile_offsets = take(4 * (E + 1));
  p->perm = take(4 * P);
  p->inv_perm = take(4 * P);
  p->masks = take(8 * E * nb);
  p->xlat = take(p->act_bytes * bt * L);
  // MX FP8 experts' h goes straight to its codes (hq below): no bf16 copy
  const bool a8 = p->expert_wf == WF_MX4A8 || p->expert_wf == WF_MX8A8;
  p->h = take(a8 ? 0 : p->act_bytes * P * c->expert_inter);
  p->o = take(p->act_bytes * P * L);
  p->n = take(p->act_bytes * bt * L);
  p->hs = take(p->act_bytes * bt * c->n_shared * c->shared_inter);
  // split-K partial sums of the dense bf16 GEMMs of short batches (up to 16
  // splits of the widest output), one region per stream
  if (p->path == PATH_BF16 && bt > 0 && bt <= kSplitMaxRows) {
    const int64_t cols = std::max({E, L, c->d, 2 * c->n_shared * c->shared_inter});
    p->split_cap = 16 * bt * cols;
  }
  p->split = take(4 * p->split_cap);
  p->split_sh = take(4 * p->split_cap);
  // MX FP8 inputs of the routed experts' GEMMs: codes and E8M0 scales
  p->xq = take(a8 ? bt * L : 0);
  p->xq_sc = take(a8 ? bt * L / 32 : 0);
  p->hq = take(a8 ? P * c->expert_inter : 0);
  p->hq_sc = take(a8 ? P * c->expert_inter / 32 : 0);
  p->total = off + kAlign;
  return MOE_OK;
}

moe_status check_ws(const Plan &p, void *ws, size_t ws_bytes) {
  if (!ws || ws_bytes < p.total - kAlign || (reinterpret_cast<uintptr_t>(ws) % kAlign))
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

bool check_weights(const moe_config *c, const moe_weights *w, bool need_experts) {
  if (!w || !w->w_router) return false;
  if (c->cutoff_mode == MOE_CUTOFF_GIVEN) { /* cutoff may be NULL */ }
  if (!need_experts) return true;
  const bool tab = w->expert_tab != nullptr;  // per-expert addresses instead
  if (!w->w_down_proj || !w->latent_gamma || !w->w_up_proj) return false;
  if (!tab && (!w->w_gate || !w->w_up || !w->w_down)) return false;
  if (c->n_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return false;
  if (reinterpret_cast<uintptr_t>(w->latent_gamma) % 16) return false;  // read as float4
  if (c->weight_dtype == MOE_FP8E4M3_B128) {
    if (!w->s_down_proj || !w->s_gate || !w->s_up || !w->s_down || !w->s_up_proj) return false;
    if (c->n_shared > 0 && (!w->s_sh_gate || !w->s_sh_up || !w->s_sh_down)) return false;
  }
  if (!tab && (c->weight_dtype == MOE_MXFP4 || c->weight_dtype == MOE_MXFP4_A8 ||
               c->weight_dtype == MOE_MXFP8)) {
    // E8M0 codes are copied a dword at a time
    for (const uint8_t *e8 : {w->e8_gate, w->e8_up, w->e8_down})
      if (!e8 || reinterpret_cast<uintptr_t>(e8) % 4) return false;
  }
  return true;
}

GemmArgs base_args(const moe_config *c) {
  GemmArgs a = {};
  a.beta = c->beta;
  a.inv_beta = 1.0f / c->beta;
  a.beta_u = c->beta_u;
  a.inv_beta_u = 1.0f / c->beta_u;
  return a;
}

#define MOE_TRY_HIP(expr)                        \
  do {                                           \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// ---- phase timing (measurement support) -------------------------------------------
enum Phase {
  PH_SHARED = 0, PH_ROUTER, PH_CUTOFF, PH_TOPK, PH_DISPATCH, PH_DOWN_PROJ, PH_EXPERT_GATEUP,
  PH_EXPERT_DOWN, PH_COMBINE, PH_OUTPUT, PH_FFN_NORM, PH_FFN_GATEUP, PH_FFN_DOWN, PH_XLAT_QUANT
};
const char *kPhaseNames[MOE_N_PHASES] = {
    "shared_gateup", "router_logits", "cutoff", "topk", "dispatch", "down_proj",
    "expert_gateup", "expert_down", "combine_norm", "output", "ffn_norm", "ffn_gateup",
    "ffn_down", "xlat_quant"};

struct Profiler {
  bool on = false;
  std::mutex mu;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[MOE_N_PHASES];
  std::vector<hipEvent_t> pool;
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records an event pair around its lifetime on `s` while profiling is on.
struct PhaseScope {
  hipEvent_t b = nullptr, e = nullptr;
  hipStream_t s;
  int ph;
  PhaseScope(int phase, hipStream_t stream) : s(stream), ph(phase) {
    if (!g_prof.on) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    b = prof_event();
    e = prof_event();
    if (b && e && hipEventRecord(b, s) != hipSuccess) b = nullptr;
  }
  ~PhaseScope() {
    if (!b || !e) return;
    const bool ok = hipEventRecord(e, s) == hipSuccess;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (ok) g_prof.rec[ph].emplace_back(b, e);
  }
};

// Router: logits (+ transposed copy for the batch quantile), cutoffs, top-k.
moe_status run_route(const moe_config *c, const Plan &p, const moe_weights *w, const void *x,
                     int64_t bt, float *z, int32_t *idx, float *wts, float *cutoff_out, void *ws,
                     hipStream_t s) {
  const int64_t E = c->n_experts;
  // BATCH and RUNNING compute this batch's quantile; RUNNING selects with the
  // caller's alpha and only reports the quantile (in cutoff_out)
  const bool batch = c->cutoff_mode != MOE_CUTOFF_GIVEN;
  const bool running = c->cutoff_mode == MOE_CUTOFF_RUNNING;
  float *zT = at<float>(ws, p.zT);
  GemmArgs a = base_args(c);
  a.M = bt;
  a.N = E;
  a.nseg = 1;
  a.seg[0] = GemmSeg{x, c->d, w->w_router, c->d, nullptr, c->d};
  a.out = z;
  a.ldo = E;
  a.out_t = batch ? zT : nullptr;
  a.bias = w->router_bias;
  a.partial = at<float>(ws, p.split);
  a.partial_cap = p.split_cap;
  const int bm = gemm_bm(p.path);
  {
    PhaseScope ph(PH_ROUTER, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_ROUTER, WF_BF16, (bt + bm - 1) / bm, s));
  }
  const float *alpha;
  {
    PhaseScope ph(PH_CUTOFF, s);
    if (batch) {
      int64_t m = (bt * c->top_k + E - 1) / E;
      m = m < 1 ? 1 : (m > bt ? bt : m);
      float *zeta = cutoff_out ? cutoff_out : at<float>(ws, p.alpha);
      MOE_TRY_HIP(launch_quantile(zT, bt, E, m, zeta, s));
      alpha = running ? w->cutoff : zeta;
    } else {
      alpha = w->cutoff;
      if (cutoff_out) MOE_TRY_HIP(launch_copy_or_zero_f32(cutoff_out, w->cutoff, E, s));
    }
  }
  {
    PhaseScope ph(PH_TOPK, s);
    MOE_TRY_HIP(launch_topk(z, alpha, bt, E, c->top_k, idx, wts, s));
  }
  return MOE_OK;
}

// One pool of events per process for the two-stream join.
std::mutex g_ev_mu;
std::vector<std::pair<int, hipEvent_t>> g_ev_free;

hipError_t ev_get(hipEvent_t *ev) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(g_ev_mu);
    for (size_t i = 0; i < g_ev_free.size(); ++i)
      if (g_ev_free[i].first == dev) {
        *ev = g_ev_free[i].second;
        g_ev_free.erase(g_ev_free.begin() + i);
        return hipSuccess;
      }
  }
  return hipEventCreateWithFlags(ev, hipEventDisableTiming);
}

void ev_put(hipEvent_t ev) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_ev_mu);
  g_ev_free.emplace_back(dev, ev);
}

}  // namespace

MOE_API moe_status moe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  return MOE_OK;
}

MOE_API moe_status moe_profile_read(double *ms_avg, int64_t *calls) {
  if (!ms_avg || !calls) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  moe_status st = MOE_OK;
  for (int p = 0; p < MOE_N_PHASES; ++p) {
    double sum = 0.0;
    int64_t n = 0;
    for (auto &be : g_prof.rec[p]) {
      float ms = 0.0f;
      if (hipEventSynchronize(be.second) != hipSuccess ||
          hipEventElapsedTime(&ms, be.first, be.second) != hipSuccess) {
        st = MOE_ERR_HIP;
      } else {
        sum += ms;
        ++n;
      }
      g_prof.pool.push_back(be.first);
      g_prof.pool.push_back(be.second);
    }
    g_prof.rec[p].clear();
    ms_avg[p] = n ? sum / (double)n : 0.0;
    calls[p] = n;
  }
  return st;
}

MOE_API const char *moe_profile_phase_name(int phase) {
  return (phase >= 0 && phase < MOE_N_PHASES) ? kPhaseNames[phase] : "";
}

MOE_API size_t moe_workspace_bytes(const moe_config *cfg, int64_t bt) {
  Plan p;
  if (make_plan(cfg, bt, &p) != MOE_OK) return 0;
  return p.total - kAlign;
}

MOE_API const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

MOE_API moe_status moe_route(const moe_config *cfg, const moe_weights *w, const void *x,
                             int64_t bt, moe_route_out *out, void *ws, size_t ws_bytes,
                             void *stream) {
  Plan p;
  moe_status st = make_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (!check_weights(cfg, w, false) || !out || !out->topk_idx || !out->topk_w)
    return MOE_ERR_INVALID_ARG;
  if (cfg->cutoff_mode == MOE_CUTOFF_RUNNING && !out->cutoff) return MOE_ERR_INVALID_ARG;
  if (bt > 0 && !x) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bt == 0) {
    if (out->cutoff && cfg->cutoff_mode != MOE_CUTOFF_BATCH)  // GIVEN, RUNNING: alpha
      MOE_TRY_HIP(launch_copy_or_zero_f32(out->cutoff, w->cutoff, cfg->n_experts, s));
    return MOE_OK;
  }
  float *z = out->logits ? out->logits : at<float>(ws, p.z);
  return run_route(cfg, p, w, x, bt, z, out->topk_idx, out->topk_w, out->cutoff, ws, s);
}

MOE_API moe_status moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, int64_t bt,
                                moe_dispatch_out *out, void *ws, size_t ws_bytes,
                                void *stream) {
  Plan p;
  moe_status st = make_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (!out || !out->counts || !out->offsets || !out->perm || !out->inv_perm)
    return MOE_ERR_INVALID_ARG;
  if (bt > 0 && !topk_idx) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(launch_dispatch(topk_idx, nullptr, bt, cfg->top_k, cfg->n_experts,
                              gemm_bm(p.path), at<uint64_t>(ws, p.masks), out->counts,
                              out->offsets, at<int32_t>(ws, p.tile_offsets), out->perm,
                              out->inv_perm, nullptr, s));
  return MOE_OK;
}

MOE_API moe_status moe_cutoff_update(float *alpha, const float *zeta, int64_t n_experts,
                                     float rate, void *stream) {
  if (n_experts < 0 || !(rate >= 0.0f && rate <= 1.0f)) return MOE_ERR_INVALID_ARG;
  if (n_experts == 0) return MOE_OK;
  if (!alpha || !zeta) return MOE_ERR_INVALID_ARG;
  MOE_TRY_HIP(launch_cutoff_update(alpha, zeta, n_experts, rate, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

MOE_API moe_status moe_mx8_quantize(const void *x, int64_t n, uint8_t *codes,
                                    uint8_t *scales, void *stream) {
  if (n < 0 || n % 32) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!x || !codes || !scales || reinterpret_cast<uintptr_t>(x) % 16) return MOE_ERR_INVALID_ARG;
  if (n / 8 > (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  MOE_TRY_HIP(launch_mx8_quant(x, n, codes, scales, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

MOE_API moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x,
                               int64_t bt, void *y, moe_route_out *route,
                               moe_dispatch_out *disp, void *ws, size_t ws_bytes, void *stream,
                               void *shared_stream) {
  Plan p;
  moe_status st = make_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (!check_weights(cfg, w, true)) return MOE_ERR_INVALID_ARG;
  if (bt > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
  if (route && (!route->topk_idx || !route->topk_w)) return MOE_ERR_INVALID_ARG;
  if (cfg->cutoff_mode == MOE_CUTOFF_RUNNING && (!route || !route->cutoff))
    return MOE_ERR_INVALID_ARG;
  if (disp && (!disp->counts || !disp->offsets || !disp->perm || !disp->inv_perm))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  // per-expert address tables: the direct-to-LDS engine with bf16 or MX experts
  const uint64_t *tab = w->expert_tab;
  if (tab && (p.path != PATH_BF16 || p.expert_wf == WF_FP8)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t ss = shared_stream ? static_cast<hipStream_t>(shared_stream) : s;
  if (bt == 0) {
    if (route && route->cutoff && cfg->cutoff_mode != MOE_CUTOFF_BATCH)
      MOE_TRY_HIP(launch_copy_or_zero_f32(route->cutoff, w->cutoff, cfg->n_experts, s));
    return MOE_OK;
  }

  const int64_t E = cfg->n_experts, k = cfg->top_k, P = bt * k, d = cfg->d, L = cfg->latent;
  const int64_t I = cfg->expert_inter, S = cfg->n_shared, Is = cfg->shared_inter;
  const int bm = gemm_bm(p.path);
  const bool fp8 = p.fp8;
  const int dwf = p.dense_wf, ewf = p.expert_wf;
  const int64_t dense_mt = (bt + bm - 1) / bm;

  // ---- second stream: x_lat = x W_down_proj^T, then the shared experts' gate/up -----
  // Neither depends on routing: W_down_proj runs beside the (small, latency-bound)
  // routing kernels, and the shared gate/up beside the routed experts.
  hipEvent_t ev_x = nullptr, ev_lat = nullptr, ev_sh = nullptr;
  const bool two_streams = ss != s;
  hipStream_t side = two_streams ? ss : s;
  if (two_streams) {
    if (ev_get(&ev_x) != hipSuccess || ev_get(&ev_lat) != hipSuccess ||
        ev_get(&ev_sh) != hipSuccess)
      return MOE_ERR_HIP;
    MOE_TRY_HIP(hipEventRecord(ev_x, s));
    MOE_TRY_HIP(hipStreamWaitEvent(ss, ev_x, 0));
  }
  void *xlat = at<void>(ws, p.xlat);
  {
    GemmArgs a = base_args(cfg);
    a.M = bt;
    a.N = L;
    a.nseg = 1;
    a.seg[0] = GemmSeg{x, d, w->w_down_proj, d, w->s_down_proj, d};
    a.partial = at<float>(ws, p.split_sh);
    a.partial_cap = p.split_cap;
    a.out = xlat;
    a.ldo = L;
    PhaseScope ph(PH_DOWN_PROJ, side);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_DENSE, dwf, dense_mt, side));
  }
  // MX FP8 experts' input: x_lat quantised once per token (the gate/up GEMM
  // gathers each token's codes k times)
  const bool a8 = ewf == WF_MX4A8 || ewf == WF_MX8A8;
  uint8_t *xq = at<uint8_t>(ws, p.xq), *xq_sc = at<uint8_t>(ws, p.xq_sc);
  if (a8) {
    PhaseScope ph(PH_XLAT_QUANT, side);
    MOE_TRY_HIP(launch_mx8_quant(xlat, bt * L, xq, xq_sc, side));
  }
  if (two_streams) MOE_TRY_HIP(hipEventRecord(ev_lat, ss));
  void *hs = at<void>(ws, p.hs);
  if (S > 0) {
    GemmArgs a = base_args(cfg);
    a.M = bt;
    a.N = S * Is;
    a.nseg = 1;
    a.seg[0] = GemmSeg{x, d, w->sh_gate, d, w->s_sh_gate, d};
    a.b_up = w->sh_up;
    a.bscale_up = w->s_sh_up;
    a.partial = at<float>(ws, p.split_sh);
    a.partial_cap = p.split_cap;
    a.out = hs;
    a.ldo = S * Is;
    PhaseScope ph(PH_SHARED, side);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_DENSE_SITU, dwf, dense_mt, side));
  }
  if (two_streams) MOE_TRY_HIP(hipEventRecord(ev_sh, ss));

  // ---- routing -----------------------------------------------------------------
  float *z = (route && route->logits) ? route->logits : at<float>(ws, p.z);
  int32_t *idx = route ? route->topk_idx : at<int32_t>(ws, p.idx);
  float *wts = route ? route->topk_w : at<float>(ws, p.w);
  st = run_route(cfg, p, w, x, bt, z, idx, wts, route ? route->cutoff : nullptr, ws, s);
  if (st != MOE_OK) return st;

  // ---- dispatch -----------------------------------------------------------------
  int32_t *counts = disp ? disp->counts : at<int32_t>(ws, p.counts);
  int32_t *offsets = disp ? disp->offsets : at<int32_t>(ws, p.offsets);
  int32_t *perm = disp ? disp->perm : at<int32_t>(ws, p.perm);
  int32_t *inv_perm = disp ? disp->inv_perm : at<int32_t>(ws, p.inv_perm);
  int32_t *tile_offsets = at<int32_t>(ws, p.tile_offsets);
  float *w_sorted = at<float>(ws, p.w_sorted);
  {
    PhaseScope ph(PH_DISPATCH, s);
    MOE_TRY_HIP(launch_dispatch(idx, wts, bt, k, E, grouped_tile_rows(p.path, ewf, P, E),
                                at<uint64_t>(ws, p.masks), counts, offsets, tile_offsets, perm,
                                inv_perm, w_sorted, s));
  }
  if (two_streams) MOE_TRY_HIP(hipStreamWaitEvent(s, ev_lat, 0));  // x_lat ready

  uint8_t *hq = at<uint8_t>(ws, p.hq), *hq_sc = at<uint8_t>(ws, p.hq_sc);
  // ---- routed experts ---------------------------------------------------------------
  const int64_t grouped_mt = (P + bm - 1) / bm + E;
  void *h = at<void>(ws, p.h);
  void *o = at<void>(ws, p.o);
  {
    GemmArgs a = base_args(cfg);
    a.M = P;
    a.N = I;
    a.nseg = 1;
    a.seg[0] = GemmSeg{a8 ? (const void *)xq : xlat, L, w->w_gate, L, w->s_gate, L};
    if (a8) {
      a.a_sc = xq_sc;
      a.lda_sc = L / 32;
    }
    a.b_up = w->w_up;
    a.bscale_up = w->s_up;
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.n_experts = (int32_t)E;
    a.b_estride = I * L;
    a.s_estride = fp8 ? (I / 128) * (L / 128) : (ewf == WF_MX4 || a8) ? I * (L / 32) : 0;
    a.e8 = w->e8_gate;
    a.e8_up = w->e8_up;
    if (tab) {  // rows gate, up, down, e8_gate, e8_up, e8_down of [6][E]
      a.b_tab = tab;
      a.bu_tab = tab + E;
      a.e8_tab = tab + 3 * E;
      a.e8u_tab = tab + 4 * E;
    }
    a.gather = perm;
    a.gather_div = (int32_t)k;
    // h rows carry the routing weight: W_d (w h) = w (W_d h); with MX FP8 h
    // the down GEMM applies it instead (h is quantised as the unweighted row)
    a.row_scale = a8 ? nullptr : w_sorted;
    a.out = h;
    a.ldo = I;
    if (a8) {  // the epilogue writes h as MX FP8 (codes + E8M0 scales) directly
      a.q_codes = hq;
      a.q_scales = hq_sc;
      a.ldq = I;
      a.ldq_sc = I / 32;
    }
    PhaseScope ph(PH_EXPERT_GATEUP, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_EXPERT_SITU, ewf, grouped_mt, s));
  }
  {
    GemmArgs a = base_args(cfg);
    a.M = P;
    a.N = L;
    a.nseg = 1;
    a.seg[0] = GemmSeg{a8 ? (const void *)hq : h, I, w->w_down, I, w->s_down, I};
    if (a8) {
      a.a_sc = hq_sc;
      a.lda_sc = I / 32;
      a.row_scale = w_sorted;
    }
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.n_experts = (int32_t)E;
    a.b_estride = L * I;
    a.s_estride = fp8 ? (L / 128) * (I / 128) : (ewf == WF_MX4 || a8) ? L * (I / 32) : 0;
    a.e8 = w->e8_down;
    if (tab) {
      a.b_tab = tab + 2 * E;
      a.e8_tab = tab + 5 * E;
    }
    a.out = o;
    a.ldo = L;
    PhaseScope ph(PH_EXPERT_DOWN, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_EXPERT_DOWN, ewf, grouped_mt, s));
  }

  // ---- combine + latent RMSNorm -------------------------------------------------------
  void *nrm = at<void>(ws, p.n);
  {
    PhaseScope ph(PH_COMBINE, s);
    MOE_TRY_HIP(launch_combine_norm(o, p.path == PATH_BF16, inv_perm, bt, k, L,
                                    w->latent_gamma, cfg->rms_eps, nrm, s));
  }

  // ---- y = n W_up_proj^T + sum_j hs_j W_ds,j^T ------------------------------------------
  if (two_streams) {
    MOE_TRY_HIP(hipStreamWaitEvent(s, ev_sh, 0));
    ev_put(ev_x);
    ev_put(ev_lat);
    ev_put(ev_sh);
  }
  {
    GemmArgs a = base_args(cfg);
    a.M = bt;
    a.N = d;
    a.nseg = 1;
    a.seg[0] = GemmSeg{nrm, L, w->w_up_proj, L, w->s_up_proj, L};
    const int64_t esz = elem_size(cfg->weight_dtype);
    for (int64_t j = 0; j < S; ++j) {
      GemmSeg &g = a.seg[a.nseg++];
      g.a = static_cast<const char *>(hs) + p.act_bytes * j * Is;
      g.lda = S * Is;
      g.b = static_cast<const char *>(w->sh_down) + esz * j * d * Is;
      g.ldb = Is;
      g.bscale = fp8 ? w->s_sh_down + j * (d / 128) * (Is / 128) : nullptr;
      g.k = Is;
    }
    a.partial = at<float>(ws, p.split);
    a.partial_cap = p.split_cap;
    a.out = y;
    a.ldo = d;
    PhaseScope ph(PH_OUTPUT, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_DENSE, dwf, dense_mt, s));
  }
  return MOE_OK;
}

// ---- moe_forward without a caller workspace ------------------------------------------
// For callers that cannot allocate device memory: the workspace is a
// file-scope device array of MOE_NOALLOC_SCRATCH_BYTES, one per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and kept.

namespace {

__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<std::pair<int, void *>> g_scratch_ptr;  // (device, address of scratch there)

moe_status scratch_of_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (auto &dp : g_scratch_ptr)
    if (dp.first == dev) {
      *out = dp.second;
      return MOE_OK;
    }
  void *ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
    return MOE_ERR_HIP;
  g_scratch_ptr.emplace_back(dev, ptr);
  *out = ptr;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w,
                                       const void *x, int64_t bt, void *y, moe_route_out *route,
                                       moe_dispatch_out *disp, void *stream,
                                       void *shared_stream) {
  Plan p;
  moe_status st = make_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (p.total - kAlign > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void *ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  // moe_forward zeroes what must start at zero (the per-expert counts) itself
  return moe_forward(cfg, w, x, bt, y, route, disp, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                     shared_stream);
}

// ---- dense layer-1 FFN ------------------------------------------------------------
// RMSNorm -> n, gate/up + SiTU -> h, down + residual -> y, all on `stream`
// (mkdocs.reaper.mx "Vue d'ensemble de l'architecture": layer 1 is a dense
// SiTU-GLU FFN of width 33 792; each sublayer is pre-normed and its output is
// summed into the block representation).

namespace {

struct FfnPlan {
  int path = PATH_BF16;
  int64_t act_bytes = 2;
  size_t n, h, split, total;
  int64_t split_cap = 0;
};

moe_status ffn_plan(const moe_ffn_config *c, int64_t bt, FfnPlan *p) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->d <= 0 || c->inter <= 0 || bt < 0) return MOE_ERR_INVALID_ARG;
  if (!(c->beta > 0.0f) || !(c->beta_u > 0.0f) || !(c->rms_eps >= 0.0f))
    return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  p->path = c->act_dtype == MOE_F32 ? PATH_F32 : PATH_BF16;
  p->act_bytes = elem_size(c->act_dtype);
  if (c->d % 64 || c->inter % 64) return MOE_ERR_UNSUPPORTED;
  // the RMSNorm holds a row per wavefront in registers (16 chunks of 16 B a lane)
  if (c->d > (c->act_dtype == MOE_F32 ? 4096 : 8192)) return MOE_ERR_UNSUPPORTED;
  if (bt > INT32_MAX / 64) return MOE_ERR_UNSUPPORTED;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  p->n = take(p->act_bytes * bt * c->d);
  p->h = take(p->act_bytes * bt * c->inter);
  // split-K partial sums of the down projection for short batches (up to 16 splits)
  if (p->path == PATH_BF16 && bt > 0 && bt <= kSplitMaxRows) p->split_cap = 16 * bt * c->d;
  p->split = take(4 * p->split_cap);
  p->total = off + kAlign;
  return MOE_OK;
}

GemmArgs ffn_args(const moe_ffn_config *c) {
  GemmArgs a = {};
  a.beta = c->beta;
  a.inv_beta = 1.0f / c->beta;
  a.beta_u = c->beta_u;
  a.inv_beta_u = 1.0f / c->beta_u;
  return a;
}

}  // namespace

MOE_API size_t moe_ffn_workspace_bytes(const moe_ffn_config *cfg, int64_t bt) {
  FfnPlan p;
  if (ffn_plan(cfg, bt, &p) != MOE_OK) return 0;
  return p.total - kAlign;
}

MOE_API moe_status moe_ffn_forward(const moe_ffn_config *cfg, const moe_ffn_weights *w,
                                   const void *x, const void *r, int64_t bt, void *y, void *ws,
                                   size_t ws_bytes, void *stream) {
  FfnPlan p;
  moe_status st = ffn_plan(cfg, bt, &p);
  if (st != MOE_OK) return st;
  if (!w || !w->w_gate || !w->w_up || !w->w_down || !w->gamma) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(w->gamma) % 16) return MOE_ERR_INVALID_ARG;  // float4 reads
  if (bt > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.total - kAlign || (reinterpret_cast<uintptr_t>(ws) % kAlign))
    return MOE_ERR_WORKSPACE;
  if (bt == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t d = cfg->d, I = cfg->inter;
  const int bm = gemm_bm(p.path);
  const int64_t mt = (bt + bm - 1) / bm;
  void *n = at<void>(ws, p.n);
  void *h = at<void>(ws, p.h);
  {
    PhaseScope ph(PH_FFN_NORM, s);
    MOE_TRY_HIP(launch_combine_norm(x, p.path == PATH_BF16, nullptr, bt, 1, d, w->gamma,
                                    cfg->rms_eps, n, s));
  }
  {
    GemmArgs a = ffn_args(cfg);
    a.M = bt;
    a.N = I;
    a.nseg = 1;
    a.seg[0] = GemmSeg{n, d, w->w_gate, d, nullptr, d};
    a.b_up = w->w_up;
    a.out = h;
    a.ldo = I;
    PhaseScope ph(PH_FFN_GATEUP, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_DENSE_SITU, WF_BF16, mt, s));
  }
  {
    GemmArgs a = ffn_args(cfg);
    a.M = bt;
    a.N = d;
    a.nseg = 1;
    a.seg[0] = GemmSeg{h, I, w->w_down, I, nullptr, I};
    a.partial = at<float>(ws, p.split);
    a.partial_cap = p.split_cap;
    a.resid = r;
    a.ldr = d;
    a.out = y;
    a.ldo = d;
    PhaseScope ph(PH_FFN_DOWN, s);
    MOE_TRY_HIP(gemm_launch(a, p.path, GK_DENSE, WF_BF16, mt, s));
  }
  return MOE_OK;
}
