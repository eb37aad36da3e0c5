// tier.hip -- cold experts in host DRAM, hot ones cached in HBM (moe_tier_*).
//
// bittide.aicompass.dev "稀疏设计", the tiered-memory paragraphs near its end: at low
// batch the most used experts can live in HBM and the others in cheaper DRAM,
// hot experts being loaded on demand; it pays when routing follows a power law
// over experts.
//
// Design: the expert GEMMs read every expert through an address table
// (moe_weights.expert_tab).  An expert whose copy sits in an HBM slot is read
// from there; any other straight from pinned host memory over PCIe.  So a
// forward is correct for any cache state and never waits for the host.  The
// host side here only decides what to cache and moves bytes:
//   observe: a kernel adds the forward's dispatch counts into a device
//            accumulator, with the pairs whose expert the table pointed into
//            the slots (what that forward read from HBM);
//   plan:    harvest the accumulator (async copy to pinned host memory, then
//            zero it) when no harvest is in flight; fold a landed harvest into
//            decayed scores; point the table at the slots of experts whose
//            copies have landed; if no copy is in flight, pick loads
//            (moe_tier_select), point the victims' table entries back at host
//            memory, and copy the new experts into the freed slots on the copy
//            stream once the forwards enqueued so far (which may read those
//            slots) are done.
// Table edits are one small kernel on the compute stream, with the new
// addresses passed by value: no host buffer has to outlive its launch.
#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "common.h"
#include "moe.h"

namespace moe {
namespace {

constexpr int kTabRows = 6;  // gate, up, down, e8_gate, e8_up, e8_down
constexpr int kUpdMax = 32;  // table entries one update launch carries

struct TabUpdate {
  int32_t n;
  int32_t e[kUpdMax];
  uint64_t addr[kUpdMax][kTabRows];
};

__global__ void __launch_bounds__(64) tier_table_update(uint64_t *table, int64_t n_experts,
                                                        TabUpdate u) {
  const int i = threadIdx.x;
  if (i >= u.n) return;
#pragma unroll
  for (int r = 0; r < kTabRows; ++r) table[r * n_experts + u.e[i]] = u.addr[i][r];
}

// table[r][e] = base[r] + e * stride[r]
struct TabInit {
  uint64_t base[kTabRows];
  uint64_t stride[kTabRows];
};

__global__ void __launch_bounds__(256) tier_table_init(uint64_t *table, int64_t n_experts,
                                                       TabInit ti) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_experts) return;
#pragma unroll
  for (int r = 0; r < kTabRows; ++r) table[r * n_experts + e] = ti.base[r] + e * ti.stride[r];
}

// acc[e] += counts[e]; acc[E] += pairs of experts whose table entry points
// into [lo, hi) (the cache slots), acc[E + 1] += all pairs.
__global__ void __launch_bounds__(256) tier_accumulate(uint32_t *acc, const int32_t *counts,
                                                       const uint64_t *table, int64_t n_experts,
                                                       uint64_t lo, uint64_t hi) {
  __shared__ uint32_t part[2][4];
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t c = 0, h = 0;
  if (e < n_experts) {
    c = (uint32_t)max(counts[e], 0);
    acc[e] += c;
    const uint64_t a = table[e];  // the gate row
    if (a >= lo && a < hi) h = c;
  }
  for (int o = 32; o > 0; o >>= 1) {
    c += __shfl_xor(c, o, 64);
    h += __shfl_xor(h, o, 64);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    part[0][w] = h;
    part[1][w] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&acc[n_experts], part[0][0] + part[0][1] + part[0][2] + part[0][3]);
    atomicAdd(&acc[n_experts + 1], part[1][0] + part[1][1] + part[1][2] + part[1][3]);
  }
}

__global__ void __launch_bounds__(256) tier_zero(uint32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Bytes of one expert matrix of rows x cols in the routed experts' dtype, and
// of its E8M0 codes (MX dtypes).
bool expert_bytes(const moe_config *c, size_t *mat, size_t *codes, bool *mx) {
  const size_t n = (size_t)c->expert_inter * (size_t)c->latent;
  switch (c->weight_dtype) {
    case MOE_BF16: *mat = 2 * n; *codes = 0; *mx = false; return c->act_dtype == MOE_BF16;
    case MOE_MXFP4:
    case MOE_MXFP4_A8: *mat = n / 2; *codes = n / 32; *mx = true; return true;
    case MOE_MXFP8: *mat = n; *codes = n / 32; *mx = true; return true;
  }
  return false;
}

}  // namespace
}  // namespace moe

using namespace moe;

struct moe_tier {
  int64_t E = 0, n_slots = 0, max_loads = 1;
  float decay = 1.0f;
  bool mx = false;
  size_t mat = 0, codes = 0, slot_bytes = 0;
  uint64_t host_dev[kTabRows] = {};  // device-visible bases of the host matrices
  const char *host_ptr[kTabRows] = {};
  char *slots = nullptr;
  uint64_t *table = nullptr;
  uint32_t *counts_acc = nullptr, *counts_host = nullptr;
  std::vector<float> score;
  std::vector<uint8_t> resident;      // table points at the expert's slot
  std::vector<int32_t> slot_of;       // slot of a resident or loading expert, else -1
  std::vector<int32_t> free_slots;
  std::vector<std::pair<int32_t, int32_t>> loading;  // (expert, slot) copies in flight
  hipEvent_t ev_counts = nullptr, ev_evict = nullptr, ev_loaded = nullptr;
  bool harvest_pending = false;       // a harvest copy is in flight
  int64_t observed = 0;               // observes since the last harvest was started
  int64_t harvest_forwards = 0;       // forwards the in-flight harvest covers
  moe_tier_stats st = {};

  uint64_t slot_addr(int32_t s, int r) const {
    const size_t off = r < 3 ? (size_t)r * align256(mat) : 3 * align256(mat) + (size_t)(r - 3) * align256(codes);
    return reinterpret_cast<uint64_t>(slots + (size_t)s * slot_bytes + off);
  }
  uint64_t host_addr(int32_t e, int r) const {
    return host_dev[r] + (uint64_t)e * (r < 3 ? mat : codes);
  }
};

namespace {

hipError_t push_updates(moe_tier *t, const std::vector<int32_t> &experts, bool to_slot,
                        hipStream_t s) {
  for (size_t i0 = 0; i0 < experts.size(); i0 += kUpdMax) {
    TabUpdate u;
    std::memset(&u, 0, sizeof(u));
    u.n = (int32_t)std::min<size_t>(kUpdMax, experts.size() - i0);
    for (int i = 0; i < u.n; ++i) {
      const int32_t e = experts[i0 + i];
      u.e[i] = e;
      for (int r = 0; r < kTabRows; ++r) {
        const bool row_used = r < 3 || t->mx;
        u.addr[i][r] = !row_used ? 0 : to_slot ? t->slot_addr(t->slot_of[e], r) : t->host_addr(e, r);
      }
    }
    hipError_t err = launch_kernel(tier_table_update, dim3(1), dim3(64), 0, s, t->table, t->E, u);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Fold a landed harvest (counts of harvest_forwards forwards) into the scores:
// the older scores decay once per forward, the harvested counts enter whole.
void fold_counts(moe_tier *t) {
  float f = 1.0f;
  for (int64_t i = 0; i < t->harvest_forwards; ++i) f *= t->decay;
  for (int64_t e = 0; e < t->E; ++e) t->score[e] = f * t->score[e] + (float)t->counts_host[e];
  t->st.pairs_hbm += t->counts_host[t->E];
  t->st.pairs += t->counts_host[t->E + 1];
  t->st.harvested += t->harvest_forwards;
  t->harvest_pending = false;
}

#define TIER_TRY(expr)                          \
  do {                                          \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

}  // namespace

MOE_API int64_t moe_tier_select(const float *score, const uint8_t *resident, int64_t E,
                                int64_t n_slots, int64_t max_loads, int32_t *load,
                                int32_t *victim) {
  if (!score || !resident || !load || !victim || E <= 0 || n_slots < 0 || n_slots > E ||
      max_loads < 0)
    return -1;
  std::vector<int32_t> cand, vict;
  int64_t held = 0;
  for (int64_t e = 0; e < E; ++e) {
    if (resident[e]) {
      vict.push_back((int32_t)e);
      ++held;
    } else if (score[e] > 0.0f) {
      cand.push_back((int32_t)e);
    }
  }
  if (held > n_slots) return -1;
  std::stable_sort(cand.begin(), cand.end(),
                   [&](int32_t a, int32_t b) { return score[a] > score[b]; });  // ties: lower id
  std::sort(vict.begin(), vict.end(), [&](int32_t a, int32_t b) {
    return score[a] != score[b] ? score[a] < score[b] : a > b;  // ties: higher id first
  });
  int64_t n = 0, free = n_slots - held;
  size_t vi = 0;
  for (size_t ci = 0; ci < cand.size() && n < max_loads; ++ci) {
    const int32_t c = cand[ci];
    if (free > 0) {
      load[n] = c;
      victim[n] = -1;
      --free;
      ++n;
    } else if (vi < vict.size() && score[c] > 1.25f * score[vict[vi]]) {
      load[n] = c;
      victim[n] = vict[vi++];
      ++n;
    } else {
      break;
    }
  }
  return n;
}

MOE_API size_t moe_tier_slot_bytes(const moe_config *cfg) {
  if (!cfg) return 0;
  size_t mat, codes;
  bool mx;
  if (!expert_bytes(cfg, &mat, &codes, &mx)) return 0;
  return 3 * align256(mat) + (mx ? 3 * align256(codes) : 0);
}

MOE_API moe_status moe_tier_create(const moe_config *cfg, const moe_tier_desc *d, void *stream,
                                   moe_tier **out) {
  if (!cfg || !d || !out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  size_t mat, codes;
  bool mx;
  if (cfg->n_experts <= 0 || cfg->latent <= 0 || cfg->expert_inter <= 0)
    return MOE_ERR_INVALID_ARG;
  if (!expert_bytes(cfg, &mat, &codes, &mx)) return MOE_ERR_UNSUPPORTED;
  const int64_t E = cfg->n_experts;
  if (d->n_slots < 0 || d->n_slots > E || !(d->decay > 0.0f && d->decay <= 1.0f) ||
      d->max_loads < 1 || !d->table || !d->counts_acc || !d->counts_host ||
      (d->n_slots > 0 && !d->slots) ||
      !d->h_gate || !d->h_up || !d->h_down ||
      (mx && (!d->h_e8_gate || !d->h_e8_up || !d->h_e8_down)))
    return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(d->slots) % 256 || reinterpret_cast<uintptr_t>(d->table) % 8)
    return MOE_ERR_INVALID_ARG;
  moe_tier *t = new (std::nothrow) moe_tier;
  if (!t) return MOE_ERR_HIP;
  t->E = E;
  t->n_slots = d->n_slots;
  t->max_loads = d->max_loads;
  t->decay = d->decay;
  t->mx = mx;
  t->mat = mat;
  t->codes = codes;
  t->slot_bytes = moe_tier_slot_bytes(cfg);
  t->slots = static_cast<char *>(d->slots);
  t->table = d->table;
  t->counts_acc = d->counts_acc;
  t->counts_host = d->counts_host;
  const void *hp[kTabRows] = {d->h_gate, d->h_up, d->h_down, d->h_e8_gate, d->h_e8_up,
                              d->h_e8_down};
  // every host buffer must be pinned and mapped for the device
  for (int r = 0; r < kTabRows; ++r) {
    if (r >= 3 && !mx) continue;
    void *dev = nullptr;
    if (hipHostGetDevicePointer(&dev, const_cast<void *>(hp[r]), 0) != hipSuccess || !dev ||
        reinterpret_cast<uintptr_t>(dev) % (r < 3 ? 256 : 4)) {
      (void)hipGetLastError();
      delete t;
      return MOE_ERR_INVALID_ARG;
    }
    t->host_dev[r] = reinterpret_cast<uint64_t>(dev);
    t->host_ptr[r] = static_cast<const char *>(hp[r]);
  }
  {
    void *dev = nullptr;
    if (hipHostGetDevicePointer(&dev, d->counts_host, 0) != hipSuccess) {
      (void)hipGetLastError();
      delete t;
      return MOE_ERR_INVALID_ARG;
    }
  }
  t->score.assign(E, 0.0f);
  t->resident.assign(E, 0);
  t->slot_of.assign(E, -1);
  for (int64_t s = d->n_slots - 1; s >= 0; --s) t->free_slots.push_back((int32_t)s);
  if (hipEventCreateWithFlags(&t->ev_counts, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&t->ev_evict, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&t->ev_loaded, hipEventDisableTiming) != hipSuccess) {
    moe_tier_destroy(t);
    return MOE_ERR_HIP;
  }
  TabInit ti;
  for (int r = 0; r < kTabRows; ++r) {
    ti.base[r] = (r < 3 || mx) ? t->host_dev[r] : 0;
    ti.stride[r] = (r < 3 || mx) ? (r < 3 ? mat : codes) : 0;
  }
  if (launch_kernel(tier_table_init, dim3((unsigned)((E + 255) / 256)), dim3(256), 0,
                    static_cast<hipStream_t>(stream), t->table, E, ti) != hipSuccess ||
      launch_kernel(tier_zero, dim3((unsigned)((E + 2 + 255) / 256)), dim3(256), 0,
                    static_cast<hipStream_t>(stream), t->counts_acc, E + 2) != hipSuccess) {
    moe_tier_destroy(t);
    return MOE_ERR_HIP;
  }
  *out = t;
  return MOE_OK;
}

MOE_API moe_status moe_tier_observe(moe_tier *t, const int32_t *counts, void *stream) {
  if (!t || !counts) return MOE_ERR_INVALID_ARG;
  const uint64_t lo = reinterpret_cast<uint64_t>(t->slots);
  const uint64_t hi = lo + (uint64_t)t->n_slots * t->slot_bytes;
  TIER_TRY(launch_kernel(tier_accumulate, dim3((unsigned)((t->E + 255) / 256)), dim3(256), 0,
                         static_cast<hipStream_t>(stream), t->counts_acc, counts,
                         (const uint64_t *)t->table, t->E, lo, hi));
  ++t->observed;
  ++t->st.forwards;
  return MOE_OK;
}

MOE_API moe_status moe_tier_plan(moe_tier *t, void *stream, void *copy_stream) {
  if (!t) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t cs = copy_stream ? static_cast<hipStream_t>(copy_stream) : s;
  // 1. a landed harvest enters the scores; a new one starts when none is in flight
  if (t->harvest_pending) {
    const hipError_t q = hipEventQuery(t->ev_counts);
    if (q == hipSuccess) fold_counts(t);
    else if (q != hipErrorNotReady) return MOE_ERR_HIP;
  }
  if (!t->harvest_pending && t->observed > 0) {
    TIER_TRY(hipMemcpyAsync(t->counts_host, t->counts_acc, sizeof(uint32_t) * (t->E + 2),
                            hipMemcpyDeviceToHost, s));
    TIER_TRY(launch_kernel(tier_zero, dim3((unsigned)((t->E + 2 + 255) / 256)), dim3(256), 0, s,
                           t->counts_acc, t->E + 2));
    TIER_TRY(hipEventRecord(t->ev_counts, s));
    t->harvest_pending = true;
    t->harvest_forwards = t->observed;
    t->observed = 0;
  }
  // 2. copies that have landed: serve those experts from their slots
  if (!t->loading.empty()) {
    const hipError_t q = hipEventQuery(t->ev_loaded);
    if (q == hipErrorNotReady) return MOE_OK;  // still in flight: nothing more this call
    if (q != hipSuccess) return MOE_ERR_HIP;
    std::vector<int32_t> landed;
    for (const auto &es : t->loading) landed.push_back(es.first);
    TIER_TRY(push_updates(t, landed, true, s));
    for (int32_t e : landed) t->resident[e] = 1;
    t->st.resident += (int64_t)landed.size();
    t->loading.clear();
  }
  // 3. choose and start new copies
  if (t->n_slots == 0) return MOE_OK;
  std::vector<int32_t> load(t->max_loads), victim(t->max_loads);
  const int64_t n = moe_tier_select(t->score.data(), t->resident.data(), t->E, t->n_slots,
                                    t->max_loads, load.data(), victim.data());
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  std::vector<int32_t> evicted;
  for (int64_t i = 0; i < n; ++i) {
    if (victim[i] < 0) continue;
    evicted.push_back(victim[i]);
  }
  if (!evicted.empty()) {
    TIER_TRY(push_updates(t, evicted, false, s));  // victims read from host from now on
    for (int32_t v : evicted) {
      t->resident[v] = 0;
      t->free_slots.push_back(t->slot_of[v]);
      t->slot_of[v] = -1;
    }
    t->st.evictions += (int64_t)evicted.size();
    t->st.resident -= (int64_t)evicted.size();
  }
  // the slots are reused once every forward enqueued so far on `stream` is done
  TIER_TRY(hipEventRecord(t->ev_evict, s));
  if (cs != s) TIER_TRY(hipStreamWaitEvent(cs, t->ev_evict, 0));
  for (int64_t i = 0; i < n; ++i) {
    const int32_t e = load[i];
    const int32_t slot = t->free_slots.back();
    t->free_slots.pop_back();
    t->slot_of[e] = slot;
    for (int r = 0; r < kTabRows; ++r) {
      if (r >= 3 && !t->mx) continue;
      const size_t bytes = r < 3 ? t->mat : t->codes;
      void *dst = reinterpret_cast<void *>(t->slot_addr(slot, r));
      const char *src = t->host_ptr[r] + (size_t)e * bytes;
      TIER_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, cs));
      t->st.bytes_loaded += (int64_t)bytes;
    }
    t->loading.emplace_back(e, slot);
  }
  t->st.loads += n;
  TIER_TRY(hipEventRecord(t->ev_loaded, cs));
  return MOE_OK;
}

MOE_API moe_status moe_tier_get_stats(const moe_tier *t, moe_tier_stats *out) {
  if (!t || !out) return MOE_ERR_INVALID_ARG;
  *out = t->st;
  return MOE_OK;
}

MOE_API moe_status moe_tier_destroy(moe_tier *t) {
  if (!t) return MOE_ERR_INVALID_ARG;
  moe_status st = MOE_OK;
  // copies in flight read the caller's host buffers and write its slots
  if (!t->loading.empty() && t->ev_loaded && hipEventSynchronize(t->ev_loaded) != hipSuccess)
    st = MOE_ERR_HIP;
  if (t->harvest_pending && t->ev_counts && hipEventSynchronize(t->ev_counts) != hipSuccess)
    st = MOE_ERR_HIP;
  for (hipEvent_t ev : {t->ev_counts, t->ev_evict, t->ev_loaded})
    if (ev) (void)hipEventDestroy(ev);
  delete t;
  return st;
}
