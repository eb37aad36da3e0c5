/*
 * moe.h -- C ABI of the Stable LatentMoE layer forward on one MI355X (gfx950).
 *
 * The layer (Kimi K3 "Stable LatentMoE"): tech.news18a.com
 * "KimiK3的StableLatentMoE架构解析" -- module structure (figure 1: router,
 * down_proj, experts, latent_norm, up_proj, shared), forward flow (figure 2),
 * SiTU-GLU (first technique), RMSNorm before up (second technique),
 * Quantile Balancing (third technique); mkdocs.reaper.mx "Vue d'ensemble de
 * l'architecture" -- per-token path steps c-g and the parameter-budget
 * table (d = 7168, L = 3584, 896 experts, top 16, 2 shared experts).
 *
 * For a batch of bt token rows x[bt][d] the library computes
 *   z = x W_r^T + b                       router logits (fp32), s = sigmoid(z)
 *   alpha = batch cutoffs (BATCH) or the caller's (GIVEN)
 *   per token: the top_k experts of largest z - alpha (ties: lower id)
 *   x_lat = x W_down_proj^T               (d -> latent)
 *   o_p   = W_d,e (phi(W_g,e x_lat) * psi(W_u,e x_lat)) per (token, expert) pair
 *   n     = RMSNorm(sum_j s_j o_j) * gamma
 *   y     = n W_up_proj^T + sum_{j<S} W_ds,j (phi(W_gs,j x) * psi(W_us,j x))
 * with phi(g) = sigmoid(g) beta tanh(g/beta), psi(u) = beta_u tanh(u/beta_u).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers on the current HIP device, row-major;
 *    weight matrices are [out][in].  Structs and scalars are host memory.
 *  - The caller owns and allocates every buffer, including the workspace of
 *    moe_workspace_bytes() bytes (256-byte aligned).  The library allocates
 *    no device memory and never synchronises the host: work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and is complete when
 *    that stream is.  Inputs are read-only; outputs are fully overwritten.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    error nothing is enqueued and a negative moe_status is returned.
 *    Asynchronous device faults surface at the caller's next synchronisation.
 *  - Calls that share a workspace must be ordered on one stream.
 *  - NaN or Inf inputs are not supported (results unspecified).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL where required, negative size, bad enum */
  MOE_ERR_UNSUPPORTED = -2, /* shape or dtype combination not implemented */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL, too small or misaligned */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8E4M3_B128 = 2, /* OCP e4m3fn codes + fp32 scale per 128x128 block */
  /* Routed experts in OCP MX FP4 (OCP Microscaling Formats (MX) Specification
   * v1.0: E2M1 elements, E8M0 scale, block 32): each [out][in] matrix stored
   * as [out][in/2] bytes, element 2i of a row in the low nibble of byte i and
   * 2i+1 in the high nibble, plus uint8 E8M0 codes [out][in/32], one per 32
   * consecutive elements of a row.  Every other weight is bf16.  The codes
   * are widened to bf16 (code value * 2^(scale - 127), exact for scale codes
   * 2..252) and multiplied on the bf16 MFMA. */
  MOE_MXFP4 = 3,
  /* MOE_MXFP4 weights, and the routed experts' GEMM inputs (x_lat for gate/up,
   * the SiTU-GLU output h for down) quantised in the layer to OCP MX FP8
   * (e4m3 elements, E8M0 scale per 32 consecutive elements along K, the
   * specification's conversion: shared exponent floor(log2 max|x|) - 8, round
   * to nearest even, saturate at 448), so both operands go to the block-scaled
   * MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) at the fp8 rate.  Same weight
   * buffers as MOE_MXFP4; the routing weight multiplies the down GEMM's output
   * rows instead of h. */
  MOE_MXFP4_A8 = 4,
  /* Routed experts in OCP MX FP8: each [out][in] matrix stored as [out][in]
   * OCP e4m3fn codes plus uint8 E8M0 codes [out][in/32] (the same scale layout
   * as MOE_MXFP4); every other weight bf16.  The experts' inputs are quantised
   * to MX FP8 as with MOE_MXFP4_A8, and both operands go to the block-scaled
   * MFMA as stored (W8A8). */
  MOE_MXFP8 = 5
} moe_dtype;

/* Quantile Balancing cutoff (tech.news18a.com page, third technique): BATCH
 * takes alpha[e] = the m-th largest fp32 logit of expert e over the batch,
 * m = clamp(ceil(bt*top_k/E), 1, bt), so each expert's load is driven to
 * bt*top_k/E; GIVEN takes a caller-held alpha (e.g. a running estimate).
 * RUNNING selects with the caller-held alpha, as GIVEN, and also computes this
 * batch's quantile zeta (as BATCH would use it) into moe_route_out.cutoff
 * (required), so the caller can move its running alpha toward it
 * (moe_cutoff_update) -- the cutoff "dynamically adjusted" across steps. */
typedef enum {
  MOE_CUTOFF_GIVEN = 0,
  MOE_CUTOFF_BATCH = 1,
  MOE_CUTOFF_RUNNING = 2
} moe_cutoff_mode;

typedef struct moe_config {
  int64_t d;            /* model width (7168 for K3) */
  int64_t latent;       /* latent width L of the routed path (3584) */
  int64_t n_experts;    /* E routed experts (896), 1 <= E <= 1024 */
  int64_t top_k;        /* k experts per token (16), 1 <= k <= min(E, 64) */
  int64_t expert_inter; /* I, routed expert intermediate width (3072) */
  int64_t n_shared;     /* S shared experts (2), 0 <= S <= 4 */
  int64_t shared_inter; /* I_s per shared expert (3072) */
  float beta;           /* SiTU gate cap (4) */
  float beta_u;         /* SiTU up-branch cap (25) */
  float rms_eps;        /* latent RMSNorm epsilon (1e-6) */
  int32_t act_dtype;    /* x and y: MOE_F32 or MOE_BF16 */
  int32_t weight_dtype; /* W_down_proj, experts, W_up_proj, shared: MOE_F32 (with f32
                           act), MOE_BF16 or MOE_FP8E4M3_B128 (with bf16 act); or
                           MOE_MXFP4 or MOE_MXFP4_A8 (bf16 act): MXFP4 experts,
                           the rest bf16; MOE_MXFP8 (bf16 act): MX FP8 experts */
  int32_t router_dtype; /* W_r: equal to act_dtype */
  int32_t cutoff_mode;  /* moe_cutoff_mode */
} moe_config;
/* Shape limits: bf16/fp8 paths need d, latent, expert_inter, shared_inter
 * multiples of 64 (of 128 with fp8 weights); latent at most 4096 (2048 with
 * fp32 activations); with fp8 weights d, latent, expert_inter and
 * shared_inter at most 16384; with MXFP4 experts latent and expert_inter
 * multiples of 128 and expert_inter at most 4096 (MOE_MXFP4_A8 and MOE_MXFP8:
 * bt * top_k * expert_inter / 32 below 2^32); bt * top_k below 2^31; with bf16
 * activations the latent activations bt * latent * 2 bytes stay below 4 GiB
 * (bt < 599186 at latent 3584).  Else MOE_ERR_UNSUPPORTED. */

typedef struct moe_weights {
  const void *w_router;      /* [E][d] router_dtype */
  const float *router_bias;  /* [E] logit offsets, or NULL (= 0) */
  const float *cutoff;       /* [E] GIVEN-mode alpha in logit units, or NULL (= 0) */
  const void *w_down_proj;   /* [L][d] */
  const void *w_gate;        /* [E][I][L] */
  const void *w_up;          /* [E][I][L] */
  const void *w_down;        /* [E][L][I] */
  const float *latent_gamma; /* [L] RMSNorm gain, 16-byte aligned */
  const void *w_up_proj;     /* [d][L] */
  const void *sh_gate;       /* [S][I_s][d] */
  const void *sh_up;         /* [S][I_s][d] */
  const void *sh_down;       /* [S][d][I_s] */
  /* MOE_FP8E4M3_B128 only (else NULL): fp32 block scales, one per 128x128
   * block of each [out][in] matrix, laid out [matrices][out/128][in/128]. */
  const float *s_down_proj, *s_gate, *s_up, *s_down, *s_up_proj, *s_sh_gate, *s_sh_up,
      *s_sh_down;
  /* MOE_MXFP4, MOE_MXFP4_A8 and MOE_MXFP8 only (else NULL): E8M0 codes of the routed experts' matrices,
   * [E][I][L/32] (gate, up) and [E][L][I/32] (down), 4-byte aligned. */
  const uint8_t *e8_gate, *e8_up, *e8_down;
  /* Optional (NULL: the stacked arrays above): per-expert addresses of the
   * routed experts' matrices, a device array [6][E] of device-visible
   * addresses -- rows gate, up, down, e8_gate, e8_up, e8_down (the e8 rows for
   * the MX dtypes only, else ignored).  Entry e of a row is the start of expert
   * e's matrix in the per-expert form of the stacked layout ([I][L] etc.), in
   * device memory or in device-visible pinned host memory (256-byte aligned;
   * E8M0 codes 4-byte aligned).  When set, w_gate, w_up, w_down and e8_* are
   * not read and may be NULL.  Weight dtypes MOE_BF16 and the MX ones only
   * (else MOE_ERR_UNSUPPORTED).  moe_tier_* maintains such a table. */
  const uint64_t *expert_tab;
} moe_weights;

/* Router results.  The router "computes scores and indices" (tech.news18a.com
 * page, figure 2).  topk_idx lists each token's experts in ascending id;
 * topk_w is sigmoid(z) of each (the bias included, the cutoff excluded, not
 * renormalised). */
typedef struct moe_route_out {
  int32_t *topk_idx; /* [bt][k] required */
  float *topk_w;     /* [bt][k] required */
  float *cutoff;     /* [E] optional: the alpha used (the batch quantile in BATCH mode);
                        RUNNING: required, the batch quantile zeta (alpha when bt = 0) */
  float *logits;     /* [bt][E] optional: fp32 z */
} moe_route_out;

/* Grouping of (token, expert) pairs p = t*k + j by expert -- the single-GPU
 * form of the dispatch exchange (mkdocs.reaper.mx page, section
 * "Vérification de compréhension": dispatch and combine per MoE layer). */
typedef struct moe_dispatch_out {
  int32_t *counts;   /* [E] pairs per expert */
  int32_t *offsets;  /* [E+1] exclusive prefix sum of counts */
  int32_t *perm;     /* [bt*k] pair ids ordered by (expert asc, token asc) */
  int32_t *inv_perm; /* [bt*k] position of pair p in perm */
} moe_dispatch_out;

/* Device bytes of workspace moe_route / moe_dispatch / moe_forward need for
 * bt tokens (the maximum of the three); 0 for an invalid config. */
size_t moe_workspace_bytes(const moe_config *cfg, int64_t bt);

/* Router: logits, cutoffs and top-k of bt tokens x[bt][d] (act_dtype). */
moe_status moe_route(const moe_config *cfg, const moe_weights *w, const void *x, int64_t bt,
                     moe_route_out *out, void *ws, size_t ws_bytes, void *stream);

/* Dispatch of given routing indices topk_idx[bt][k] (each in [0, E) and
 * distinct within a token's row, in any order).  All four outputs are
 * required.  An id out of range, or repeated in its row, leaves that pair out
 * of the grouping: offsets[E] is then below bt * k (the caller's check; the
 * call does not wait for the device), the pair's inv_perm entry is 0, and
 * every write stays inside the four arrays. */
moe_status moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, int64_t bt,
                        moe_dispatch_out *out, void *ws, size_t ws_bytes, void *stream);

/* Whole layer: y[bt][d] (act_dtype).  route / disp may be NULL; when given
 * they receive the routing and dispatch of this call.  The latent down
 * projection and the shared experts' gate/up do not depend on routing: they
 * run on shared_stream (NULL: on `stream`), joined into `stream` before the
 * routed experts and before the output projection respectively.  The call
 * enqueues kernels and event record / wait pairs only (no memset, copy or
 * host wait), so it can be recorded into a HIP graph by capturing `stream`;
 * shared_stream is then forked from and joined back into the capture by those
 * events.  The first call on a device must run outside capture (it sets the
 * kernels' LDS limits and fills the library's event pool). */
moe_status moe_forward(const moe_config *cfg, const moe_weights *w, const void *x, int64_t bt,
                       void *y, moe_route_out *route, moe_dispatch_out *disp, void *ws,
                       size_t ws_bytes, void *stream, void *shared_stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results, with the workspace taken from a library-held
 * device array of MOE_NOALLOC_SCRATCH_BYTES (128 MiB) instead of a caller
 * buffer.  Each GPU the library runs on holds its own array from the first
 * call there until the process ends; the call allocates nothing (no hipMalloc,
 * no hipFree).  Every call on a GPU shares that GPU's array and leaves its
 * contents behind: calls that overlap on one GPU (on different streams or
 * from several host threads) race and give undefined results, so order them
 * on one stream.  A batch whose moe_workspace_bytes(cfg, bt) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE before anything is
 * enqueued (K3 decode shapes, d 7168 and 896 experts, fit up to 64 tokens).
 * The two-stream join takes events from the library's pool (created on first
 * use; events are not device memory). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_config *cfg, const moe_weights *w, const void *x,
                               int64_t bt, void *y, moe_route_out *route,
                               moe_dispatch_out *disp, void *stream, void *shared_stream);

/* ---- backward pass ---------------------------------------------------------------
 * Gradients of a loss with respect to x and every weight, given dL/dy.  The
 * pages describe the forward only (tech.news18a.com page: the architecture
 * figure, the SiTU formula, the quantile-balancing passage; the gradient
 * explosion passage of that page is why its caps exist); the gradients are the
 * chain rule of that forward.  The chosen expert set is piecewise constant in
 * the scores and gets no gradient; each chosen weight w = sigmoid(z) does, and
 * through it the router weights and bias.  Every array is fp32, dense, in the
 * layout of the weight it belongs to (moe_weights), overwritten (not
 * accumulated), all required (sh_* only when n_shared > 0). */
typedef struct moe_grads {
  float *dx;           /* [bt][d] (may be NULL when bt == 0) */
  float *w_router;     /* [E][d] */
  float *router_bias;  /* [E] */
  float *w_down_proj;  /* [L][d] */
  float *w_gate;       /* [E][I][L] */
  float *w_up;         /* [E][I][L] */
  float *w_down;       /* [E][L][I] */
  float *latent_gamma; /* [L] */
  float *w_up_proj;    /* [d][L] */
  float *sh_gate;      /* [S][I_s][d] */
  float *sh_up;        /* [S][I_s][d] */
  float *sh_down;      /* [S][d][I_s] */
} moe_grads;

/* Device bytes of workspace moe_backward needs for bt tokens; 0 for an invalid
 * or unsupported config. */
size_t moe_backward_workspace_bytes(const moe_config *cfg, int64_t bt);

/* Backward of moe_forward for bf16 activations, weights and router
 * (MOE_ERR_UNSUPPORTED otherwise, for an expert_tab, and unless d, latent,
 * expert_inter and shared_inter are multiples of 64 and n_experts of 8).
 * x[bt][d] and dy[bt][d] are bf16; topk_idx / topk_w [bt][k] the routing
 * moe_route (or moe_forward) returned for x (ids in range and distinct per
 * token: a pair with an id out of range or repeated is left out of the
 * gradients).  The forward's intermediate values are recomputed from x, so no
 * activations are kept between the calls.  Same conventions as moe_forward:
 * everything is enqueued on `stream` (the call neither allocates nor waits
 * for the device), and the gradients are complete when `stream` reaches that
 * point.  The contractions run on the layer's GEMM engine, the routed
 * experts' ones grouped by expert from the dispatch offsets on the device.
 * bt == 0 writes zero weight gradients.  The workspace (256-byte aligned)
 * holds the recomputed activations, about 2 (L + I) * 10 bytes a (token,
 * expert) pair. */
moe_status moe_backward(const moe_config *cfg, const moe_weights *w, const void *x, int64_t bt,
                        const int32_t *topk_idx, const float *topk_w, const void *dy,
                        const moe_grads *g, void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *moe_status_str(int status);

/* ---- Dense layer-1 FFN -------------------------------------------------------
 * The first layer of K3 is dense: a full-width SiTU-GLU FFN of intermediate
 * width 33 792, with no routing (mkdocs.reaper.mx "Vue d'ensemble de
 * l'architecture", section "Le décompte des couches").  As every sublayer it is
 * preceded by an RMSNorm and its output is summed into the block representation
 * (same page, section "Ce que fait une couche").  For bt rows x[bt][d]:
 *   n = x / sqrt(mean(x^2) + eps) * gamma
 *   y = r + W_d (phi(W_g n) * psi(W_u n))        phi, psi as for the experts
 * r (the representation the output is summed into) may be NULL (= 0) and may
 * be y itself (in place).  Same conventions as above (device pointers, caller
 * allocates, validation before enqueue, work on `stream`). */
typedef struct moe_ffn_config {
  int64_t d;            /* width (7168 for K3); multiple of 64, at most 8192 (4096 fp32) */
  int64_t inter;        /* intermediate width (33 792); multiple of 64 */
  float beta, beta_u;   /* SiTU caps (4, 25) */
  float rms_eps;        /* 1e-6 */
  int32_t act_dtype;    /* x, r, y and the weights: MOE_F32 or MOE_BF16 */
} moe_ffn_config;

typedef struct moe_ffn_weights {
  const void *w_gate;   /* [inter][d] */
  const void *w_up;     /* [inter][d] */
  const void *w_down;   /* [d][inter] */
  const float *gamma;   /* [d] RMSNorm gain, 16-byte aligned */
} moe_ffn_weights;

/* Device bytes of workspace moe_ffn_forward needs for bt rows; 0 for an invalid config. */
size_t moe_ffn_workspace_bytes(const moe_ffn_config *cfg, int64_t bt);

moe_status moe_ffn_forward(const moe_ffn_config *cfg, const moe_ffn_weights *w, const void *x,
                           const void *r, int64_t bt, void *y, void *ws, size_t ws_bytes,
                           void *stream);

/* Running cutoff step for MOE_CUTOFF_RUNNING: alpha[e] += rate * (zeta[e] -
 * alpha[e]) for e < n_experts, in fp32 with each operation rounded (device
 * arrays, on `stream`; rate in [0, 1]: 1 follows the last batch, 0 freezes).
 * An exponential moving average of the batch quantiles: the "dynamic
 * adjustment" of the cutoff across steps, which the news18a page names
 * without a rule (the reading taken here). */
moe_status moe_cutoff_update(float *alpha, const float *zeta, int64_t n_experts, float rate,
                             void *stream);

/* ---- Expert tiering: cold experts in host DRAM, hot ones cached in HBM -----
 * bittide.aicompass.dev "稀疏设计" (the tiered-memory paragraphs near its end): at low
 * batch, the most used experts can sit in HBM and the rarely used ones in
 * cheaper DRAM, hot experts being loaded as needed -- worthwhile when routing
 * concentrates on popular experts (a power law), not when a large batch
 * lights up most of them.
 *
 * The routed experts live in pinned host memory (hipHostMalloc, e.g. torch
 * pin_memory), stacked as moe_weights' w_gate / w_up / w_down / e8_*.  A
 * caller-allocated HBM cache of n_slots experts holds the popular ones, and
 * moe_forward reads every expert through the address table `table` (pass it
 * as moe_weights.expert_tab): a cached expert from its slot, any other one
 * straight from host memory over PCIe.  A forward is therefore correct
 * whatever the cache holds, and never waits for the host.  Popularity is the
 * routed-pair count of each expert (the dispatch counts of the forwards),
 * decayed by `decay` per observed forward.  Call
 *   moe_tier_plan(t, stream, copy_stream)   before each forward, and
 *   moe_tier_observe(t, counts, stream)     after it (counts: the forward's
 *                                           moe_dispatch_out.counts).
 * Neither blocks the host.  observe adds the counts on the device into
 * counts_acc (and the pairs whose expert the forward read from HBM), so no
 * observation is lost however far the host runs ahead.  plan harvests that
 * accumulator into counts_host (an async copy, then zeroes it) when no harvest
 * is in flight, folds a landed harvest into the scores, points the table at
 * the slots of experts whose copies have landed, and, when no copy is in
 * flight, picks experts to load with moe_tier_select and starts their copies
 * on copy_stream (NULL: stream).
 * Those copies are ordered after the forwards already enqueued on stream,
 * which may still read a slot being reused.  Every table change is a small
 * kernel on `stream`.  The library allocates no device memory; it keeps
 * host-side state and a few events.  Not thread-safe; one tier per layer. */
typedef struct moe_tier moe_tier;

typedef struct moe_tier_desc {
  const void *h_gate, *h_up, *h_down;             /* pinned host, stacked [E][..] */
  const uint8_t *h_e8_gate, *h_e8_up, *h_e8_down; /* pinned host, MX dtypes only */
  int64_t n_slots;      /* experts the HBM cache holds, 0..E */
  void *slots;          /* device, n_slots * moe_tier_slot_bytes(cfg) bytes, 256-aligned */
  uint64_t *table;      /* device, 6 * E entries (moe_weights.expert_tab) */
  uint32_t *counts_acc; /* device, E + 2 entries: counts observed since the last
                           harvest, then the pairs read from HBM and all pairs */
  uint32_t *counts_host;/* pinned host, E + 2 entries: where harvests land */
  float decay;          /* popularity decay per observed forward, in (0, 1] */
  int64_t max_loads;    /* experts a plan call may start loading, >= 1 */
} moe_tier_desc;

typedef struct moe_tier_stats {
  int64_t forwards;     /* observed forwards */
  int64_t harvested;    /* ... whose counts have been folded into the scores */
  int64_t pairs;        /* routed (token, expert) pairs of the harvested forwards */
  int64_t pairs_hbm;    /* ... whose expert the forward read from HBM */
  int64_t loads;        /* experts copied into the cache */
  int64_t evictions;    /* experts switched back to host memory */
  int64_t bytes_loaded; /* host -> HBM bytes copied */
  int64_t resident;     /* experts the table currently points at HBM for */
} moe_tier_stats;

/* Device bytes of one cache slot (one expert's matrices, plus E8M0 codes for
 * the MX dtypes, each 256-byte aligned); 0 for a config tiering does not take. */
size_t moe_tier_slot_bytes(const moe_config *cfg);
/* Validates desc (host buffers must be pinned and device-visible:
 * MOE_ERR_INVALID_ARG otherwise), fills the table with every expert's host
 * address (an empty cache) and zeroes counts_acc on `stream`, returns the
 * handle in *out. */
moe_status moe_tier_create(const moe_config *cfg, const moe_tier_desc *desc, void *stream,
                           moe_tier **out);
moe_status moe_tier_plan(moe_tier *t, void *stream, void *copy_stream);
moe_status moe_tier_observe(moe_tier *t, const int32_t *counts, void *stream);
moe_status moe_tier_get_stats(const moe_tier *t, moe_tier_stats *out);
/* Waits for the tier's copies in flight, then frees its host-side state. */
moe_status moe_tier_destroy(moe_tier *t);
/* The cache policy moe_tier_plan applies (host only; no GPU call).  score[E]
 * >= 0, resident[E] in {0, 1}.  Candidates are the non-resident experts with
 * score > 0, best first; victims the resident ones, worst first (ties: lower
 * id first as candidate, higher id first as victim).  Up to max_loads
 * candidates are chosen: into a free slot while fewer than n_slots experts
 * are resident (victim -1), else replacing the next victim if the candidate's
 * score exceeds 1.25 x the victim's (hysteresis against thrashing), stopping
 * at the first that does not.  Writes load[i], victim[i]; returns the count,
 * or -1 for invalid arguments. */
int64_t moe_tier_select(const float *score, const uint8_t *resident, int64_t E, int64_t n_slots,
                        int64_t max_loads, int32_t *load, int32_t *victim);

/* ---- MX FP8 quantisation -----------------------------------------------------
 * OCP Microscaling Formats (MX) Specification v1.0, conversion of a vector of
 * scalars to MX blocks, with e4m3 elements and block 32 -- the step
 * MOE_MXFP4_A8 and MOE_MXFP8 apply to the routed experts' GEMM inputs.  x: n bf16 values
 * (device, 16-byte aligned; n a multiple of 32, blocks = 32 consecutive
 * elements); codes: n bytes of OCP e4m3fn (device); scales: n / 32 E8M0 bytes
 * (device).  Per block: shared exponent s = floor(log2 max|x|) - 8, clamped to
 * [-127, 127] (-127 for an all-zero block), scale byte s + 127; element code =
 * x / 2^s rounded to the nearest e4m3 value, ties to even, saturated at +-448.
 * Asynchronous on `stream`; the caller owns every buffer.  MOE_ERR_INVALID_ARG
 * for NULL pointers with n > 0, n < 0, n not a multiple of 32 or a misaligned x;
 * MOE_ERR_UNSUPPORTED for n >= 2^35. */
moe_status moe_mx8_quantize(const void *x, int64_t n, uint8_t *codes, uint8_t *scales,
                            void *stream);

/* ---- bf16 contraction on the layer's GEMM engine --------------------------------
 * C = op(A) op(B) (+ C_in) with bf16 operands, fp32 accumulation and output:
 * the forms the backward pass runs its contractions in.  A is [M][K]
 * (a_kouter = 0, row stride lda >= K) or K-outer [K][M] (a_kouter = 1, lda >=
 * M); B is [N][K] (b_kouter = 0, ldb >= K) or K-outer [K][N] (b_kouter = 1,
 * ldb >= N); C [M][ldc] fp32.  c_in (may be c) is added when given.
 * With k_offsets (device, n_experts + 1 ascending row indices), both operands
 * K-outer: n_experts outputs C_e = [M][N] at c + e M ldc, each over the K rows
 * k_offsets[e] .. k_offsets[e + 1] of A and B (an expert without rows gets
 * zeros) -- the routed experts' weight gradients; K is then unused.
 * Limits: K-outer operands' rows (M or N) and the strides multiples of 8;
 * unless both operands are K-outer, K a multiple of 64; a K-outer A needs a
 * K-outer B.  Else MOE_ERR_UNSUPPORTED.  Asynchronous on `stream`; no
 * workspace, no allocation. */
typedef struct moe_gemm_desc {
  int64_t M, N, K;
  const void *a;
  int64_t lda;
  int32_t a_kouter;
  const void *b;
  int64_t ldb;
  int32_t b_kouter;
  float *c;
  int64_t ldc;
  const float *c_in;
  const int32_t *k_offsets;
  int64_t n_experts;
} moe_gemm_desc;
moe_status moe_gemm_bf16(const moe_gemm_desc *desc, void *stream);

/* ---- SiTU-GLU numerics ---------------------------------------------------------
 * The SiTU-GLU factors on the device, elementwise, by the same inline device
 * functions the GEMM epilogues use (tech.news18a.com page, first technique:
 * sigmoid limiting combined with tanh scaling, an output range strictly
 * bounded by beta = 4 and beta_u = 25):
 *   phi[i] = sigmoid(g[i]) beta tanh(g[i] / beta)
 *   psi[i] = beta_u tanh(u[i] / beta_u)
 *   h[i]   = phi[i] psi[i]
 * g, u: n fp32 device values; phi, psi, h: n fp32 device outputs, each may be
 * NULL (not all three).  For every finite input phi <= beta (phi > -0.2698 at
 * beta = 4), |psi| <= beta_u and |h| <= beta beta_u.  Asynchronous on `stream`.
 * MOE_ERR_INVALID_ARG for n < 0, beta or beta_u not positive, or NULL inputs
 * with n > 0. */
moe_status moe_situ_eval(const float *g, const float *u, int64_t n, float beta, float beta_u,
                         float *phi, float *psi, float *h, void *stream);

/* ---- Measurement support (not part of the layer) ----------------------------
 * While enabled, moe_forward and moe_ffn_forward record a timing hipEvent pair
 * around each of their phases on the stream that phase runs on (the shared
 * experts on shared_stream).  moe_profile_read waits for the recorded events,
 * returns the average milliseconds per call of each phase and clears the
 * record.  Phases: 0 shared gate/up, 1 router logits, 2 cutoffs, 3 top-k,
 * 4 dispatch, 5 W_down_proj, 6 expert gate/up, 7 expert down, 8 combine +
 * RMSNorm, 9 output projection; dense FFN: 10 RMSNorm, 11 gate/up, 12 down;
 * MOE_MXFP4_A8 and MOE_MXFP8: 13 MX FP8 quantisation of x_lat (h is written
 * in MX FP8 by the expert gate/up epilogue).
 * Events are created by the library and kept for reuse (no device memory).
 * Not thread-safe against concurrent forwards. */
#define MOE_N_PHASES 14
moe_status moe_profile_enable(int on);
moe_status moe_profile_read(double *ms_avg, int64_t *calls); /* arrays of MOE_N_PHASES */
const char *moe_profile_phase_name(int phase);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
