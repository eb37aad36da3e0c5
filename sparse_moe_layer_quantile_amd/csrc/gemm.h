// gemm.h -- the GEMM engine of the layer: C[m][n] = sum_k A[m][k] B[n][k].
//
// One problem description (GemmArgs) serves every contraction of the layer:
//   dense      router logits, W_down_proj, shared gate/up, output projection
//   grouped    routed experts: the M rows are positions of the expert-sorted
//              (token, expert) pair list; B is the expert's own matrix
//   gathered   A row of position p is x_lat[perm[p] / top_k]
//   dual       B = (gate, up) pair, the epilogue applies SiTU-GLU
//   segmented  K split over up to three (A, B) pairs: [n | hs] x [W_up | W_ds,j]
// and two inner engines: bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16, B in
// bf16, fp8 e4m3 with 128x128 block scales, or MXFP4) and fp32 SIMT.
#pragma once

#include "common.h"

namespace moe {

enum Epi { EPI_STORE = 0, EPI_ROUTER = 1, EPI_SITU = 2 };

struct GemmSeg {
  const void *a;
  int64_t lda;
  const void *b;
  int64_t ldb;
  const float *bscale;  // fp8: block scales of B (expert 0), [rows/128][k/128]
  int64_t k;
};

struct GemmArgs {
  int64_t M, N;
  int32_t nseg;
  GemmSeg seg[5];  // K segments (up to 1 + 4 shared experts)
  const void *b_up;          // dual: the up matrix (same layout as seg[0].b)
  const float *bscale_up;
  const int32_t *offsets;    // grouped: [E+1] row offsets of each expert; NULL = dense
  const int32_t *tile_offsets;  // grouped: [E+1] first M-tile of each expert
  int32_t n_experts;
  int64_t b_estride;         // elements between consecutive experts' B matrices
  int64_t s_estride;         // block scales between consecutive experts
  // MXFP4 B: E8M0 codes [rows][k/32] of seg[0].b and of b_up (expert 0; 4-byte
  // aligned); consecutive experts s_estride codes apart
  const uint8_t *e8, *e8_up;
  // grouped, direct-to-LDS engine: per-expert addresses of seg[0].b, b_up, e8 and
  // e8_up ([n_experts] each; NULL = the stacked layout above).  An address may be
  // device memory or device-visible pinned host memory.
  const uint64_t *b_tab, *bu_tab, *e8_tab, *e8u_tab;
  const int32_t *gather;     // A row of position p = gather[p] / gather_div
  int32_t gather_div;
  void *out;
  int64_t ldo;
  float *out_t;              // router: transposed copy [N][M] (may be NULL)
  const float *bias;         // router: [N] (may be NULL)
  const float *row_scale;    // SiTU and store: factor of output row m (NULL = 1)
  // SiTU (direct-to-LDS engine and its split-K sum): also the raw gate and up
  // sums, fp32 [M][ldgu] each (the backward's recompute; NULL = not written)
  float *out_g, *out_u;
  int64_t ldgu;
  const void *resid;         // store: out = acc + resid[m][ldr] (OutT; NULL = none; may be out)
  int64_t ldr;
  // MX FP8 A (direct-to-LDS engine, BF_MX4A8): E8M0 codes a_sc[row][lda_sc] of the A
  // rows (gathered rows indexed as the A rows), one per 32 elements along K
  const uint8_t *a_sc;
  int64_t lda_sc;
  // SiTU epilogue of the MX FP8 engine: when q_codes is set, the output is
  // written as MX FP8 instead (the next GEMM's A): e4m3 codes q_codes[row][ldq]
  // and E8M0 codes q_scales[row][ldq_sc], blocks of 32 output columns, decided
  // on the bf16-rounded value (as a separate quantisation of the bf16 output)
  uint8_t *q_codes, *q_scales;
  int64_t ldq, ldq_sc;
  float beta, inv_beta, beta_u, inv_beta_u;
  int32_t n_tiles_n;         // N tiles (direct-to-LDS engine: groups of nper N tiles)
  int32_t group_m;           // M tiles per rasterisation group (tiles of a group share B)
  int32_t nper;              // direct-to-LDS short tiles: N tiles a workgroup runs in turn
  // split K (dense bf16 problems with few tiles): K tile range blockIdx.y of
  // ksplit; raw fp32 sums go to partial[split][M][ldp] (a dual problem's up
  // sums at column N + c) and a second kernel reduces them and applies the
  // epilogue.  partial == NULL (or partial_cap too small) disables it.
  float *partial;
  int64_t partial_cap;       // floats available at partial
  int64_t ldp;
  int32_t ksplit;
};

struct Tile {
  int64_t m0, m_end, n0;
  int32_t e;
  bool valid;
};

// Work item of this workgroup: N tile fastest, then M tile (dense) or the
// linear M-tile index over all experts' segments (grouped).
template <int BM, int BN_OUT>
__device__ __forceinline__ Tile map_tile(const GemmArgs &a) {
  Tile t;
  const int64_t bid = blockIdx.x;
  const int64_t mt = bid / a.n_tiles_n;
  t.n0 = (bid - mt * a.n_tiles_n) * BN_OUT;
  if (a.offsets == nullptr) {
    t.e = 0;
    t.m0 = mt * BM;
    t.m_end = min(a.M, t.m0 + BM);
    t.valid = t.m0 < a.M;
    return t;
  }
  const int32_t total = a.tile_offsets[a.n_experts];
  if (mt >= total) {
    t.valid = false;
    return t;
  }
  int lo = 0, hi = a.n_experts;  // tile_offsets[lo] <= mt < tile_offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_offsets[mid] <= mt) lo = mid;
    else hi = mid;
  }
  t.e = lo;
  t.m0 = a.offsets[lo] + (mt - a.tile_offsets[lo]) * BM;
  t.m_end = min((int64_t)a.offsets[lo + 1], t.m0 + BM);
  t.valid = true;
  return t;
}

template <typename OutT>
__device__ __forceinline__ void store_out(void *out, int64_t i, float v) {
  if constexpr (sizeof(OutT) == 4) static_cast<float *>(out)[i] = v;
  else static_cast<uint16_t *>(out)[i] = f32_to_bf16(v);
}

// Element i of an OutT tensor, as fp32 (the residual of a store epilogue).
template <typename OutT>
__device__ __forceinline__ float load_in(const void *p, int64_t i) {
  if constexpr (sizeof(OutT) == 4) return static_cast<const float *>(p)[i];
  else return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

// Epilogue of one output element (row, col).  v: accumulator (gate for
// dual), vu: the up accumulator of a dual problem.
template <int EPI, typename OutT>
__device__ __forceinline__ void epilogue(const GemmArgs &a, int64_t row, int64_t col, float v,
                                         float vu) {
  if constexpr (EPI == EPI_ROUTER) {
    const float z = v + (a.bias ? a.bias[col] : 0.0f);
    static_cast<float *>(a.out)[row * a.ldo + col] = z;
  } else if constexpr (EPI == EPI_SITU) {
    const float f = a.row_scale ? a.row_scale[row] : 1.0f;
    store_out<OutT>(a.out, row * a.ldo + col,
                    f * situ(v, vu, a.beta, a.inv_beta, a.beta_u, a.inv_beta_u));
  } else {
    if (a.row_scale) v *= a.row_scale[row];
    if (a.resid) v += load_in<OutT>(a.resid, row * a.ldr + col);
    store_out<OutT>(a.out, row * a.ldo + col, v);
  }
}

// ============================================================================
// bf16 MFMA engine.  Tile 128 x 128 (B rows) x 64, 256 threads = 4 waves in a
// 2 x 2 layout, each wave 2 x 2 tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16).
// Dual problems put 64 gate rows and the 64 matching up rows in the B tile, so
// a wave holds the gate and up accumulators of the same outputs.
// LDS: two stages of A[128][64] + B[128][64] bf16, rows of 8 chunks of 16 B,
// chunk index XOR-swizzled with (row & 7) so both the 16 B global->LDS stores
// and the MFMA operand reads are bank-conflict free.
// ============================================================================
namespace mf {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
}  // namespace mf

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

template <int EPI, bool DUAL, bool FP8, bool GATHER, typename OutT>
__global__ void __launch_bounds__(256, 2) gemm_mfma_kernel(GemmArgs args) {
  using namespace mf;
  constexpr int BN_OUT = DUAL ? BN / 2 : BN;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const Tile tile = map_tile<BM, BN_OUT>(args);
  if (!tile.valid) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global-load assignment ---------------------------------------------
  // A and bf16 B: chunk lc of rows (tid >> 3) + 32 i, i = 0..3.
  const int lc = tid & 7;
  int64_t arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t m = tile.m0 + (tid >> 3) + 32 * i;
    if (m >= tile.m_end) m = tile.m0;  // clamp: computed, never stored
    if constexpr (GATHER) m = args.gather[m] / args.gather_div;
    arow[i] = m;
  }
  // B rows of this thread (bf16: 4 rows like A; fp8: row tid >> 1, half tid & 1)
  const char *bbase0 = static_cast<const char *>(args.seg[0].b);
  const char *bbase_up = static_cast<const char *>(args.b_up);
  const float *sbase0 = args.seg[0].bscale;
  const float *sbase_up = args.bscale_up;
  if (args.offsets != nullptr) {
    const int64_t eb = (int64_t)tile.e * args.b_estride * (FP8 ? 1 : 2);
    bbase0 += eb;
    if (DUAL) bbase_up += eb;
    if (FP8) {
      sbase0 += (int64_t)tile.e * args.s_estride;
      if (DUAL) sbase_up += (int64_t)tile.e * args.s_estride;
    }
  }
  auto b_row_of = [&](int r, bool &is_up) -> int64_t {
    int64_t n;
    if (DUAL) {
      is_up = r >= BN / 2;
      n = tile.n0 + (is_up ? r - BN / 2 : r);
    } else {
      is_up = false;
      n = tile.n0 + r;
    }
    if (n >= args.N) n = tile.n0;
    return n;
  };

  int ktiles_total = 0;
  for (int s = 0; s < args.nseg; ++s) ktiles_total += (int)(args.seg[s].k / BK);

  uint4 ra[4];
  uint4 rb[4];  // bf16: 4 chunks; fp8: 2 x 16 codes
  float rbs = 1.0f;

  // global -> registers for flattened K tile kt
  auto load_tile = [&](int kt) {
    int s = 0, k0 = kt * BK;
    while (s + 1 < args.nseg && k0 >= args.seg[s].k) { k0 -= (int)args.seg[s].k; ++s; }
    const GemmSeg &sg = args.seg[s];
    const uint16_t *A = static_cast<const uint16_t *>(sg.a);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = *reinterpret_cast<const uint4 *>(A + arow[i] * sg.lda + k0 + lc * 8);
    const char *bb = (s == 0) ? bbase0 : static_cast<const char *>(sg.b);
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool up;
        const int64_t n = b_row_of((tid >> 3) + 32 * i, up);
        const uint16_t *B = reinterpret_cast<const uint16_t *>(up ? bbase_up : bb);
        rb[i] = *reinterpret_cast<const uint4 *>(B + n * sg.ldb + k0 + lc * 8);
      }
    } else {
      bool up;
      const int64_t n = b_row_of(tid >> 1, up);
      const uint8_t *B = reinterpret_cast<const uint8_t *>(up ? bbase_up : bb);
      const uint8_t *p = B + n * sg.ldb + k0 + (tid & 1) * 32;
      rb[0] = *reinterpret_cast<const uint4 *>(p);
      rb[1] = *reinterpret_cast<const uint4 *>(p + 16);
      const float *S = (s == 0) ? (up ? sbase_up : sbase0) : sg.bscale;
      rbs = S[(n >> 7) * (sg.k >> 7) + (k0 >> 7)];
    }
  };

  // registers -> LDS stage
  auto store_tile = [&](int stage) {
    uint16_t *As = lds + stage * STAGE;
    uint16_t *Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4 *>(As + swz(r, lc)) = ra[i];
    }
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *reinterpret_cast<uint4 *>(Bs + swz(r, lc)) = rb[i];
      }
    } else {
      const int r = tid >> 1, c0 = (tid & 1) * 4;
      const uint32_t *w = reinterpret_cast<const uint32_t *>(rb);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 v;
        uint32_t *o = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t word = w[c * 2 + (q >> 1)];
          const uint32_t b0 = (word >> ((q & 1) * 16)) & 0xFFu;
          const uint32_t b1 = (word >> ((q & 1) * 16 + 8)) & 0xFFu;
          o[q] = pack_bf16x2(e4m3_to_f32(b0) * rbs, e4m3_to_f32(b1) * rbs);
        }
        *reinterpret_cast<uint4 *>(Bs + swz(r, c0 + c)) = v;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles_total; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < ktiles_total) load_tile(kt + 1);
    const uint16_t *As = lds + stage * STAGE;
    const uint16_t *Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8 *>(As + swz(r, chunk));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = DUAL ? (j * 64 + wn * 32 + (lane & 31)) : (wn * 64 + j * 32 + (lane & 31));
        bfr[j] = *reinterpret_cast<const bf16x8 *>(Bs + swz(r, chunk));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ktiles_total) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31), rows 8(r/4) + 4(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = tile.m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= tile.m_end) continue;
      if constexpr (DUAL) {
        const int64_t col = tile.n0 + wn * 32 + (lane & 31);
        if (col < args.N) epilogue<EPI, OutT>(args, row, col, acc[i][0][r], acc[i][1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = tile.n0 + wn * 64 + j * 32 + (lane & 31);
          if (col < args.N) epilogue<EPI, OutT>(args, row, col, acc[i][j][r], 0.0f);
        }
      }
    }
  }
  if constexpr (EPI == EPI_ROUTER) {
    // transposed copy z^T[col][row]: four consecutive rows per lane -> 16 B stores
    if (args.out_t != nullptr) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = tile.n0 + wn * 64 + j * 32 + (lane & 31);
          if (col >= args.N) continue;
          const float b = args.bias ? args.bias[col] : 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t row0 = tile.m0 + wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
            float *dst = args.out_t + col * args.M + row0;
            if (row0 + 3 < tile.m_end && ((args.M & 3) == 0)) {
              float4 v = make_float4(acc[i][j][q * 4 + 0] + b, acc[i][j][q * 4 + 1] + b,
                                     acc[i][j][q * 4 + 2] + b, acc[i][j][q * 4 + 3] + b);
              *reinterpret_cast<float4 *>(dst) = v;
            } else {
              for (int u = 0; u < 4; ++u)
                if (row0 + u < tile.m_end) dst[u] = acc[i][j][q * 4 + u] + b;
            }
          }
        }
    }
  }
}

// ============================================================================
// fp32 SIMT engine (fp32 activations and weights).  Tile 64 x 64 (B rows) x 16,
// 256 threads as 16 x 16, each 4 rows x 4 B rows.
// ============================================================================
namespace sf {
constexpr int BM = 64, BN = 64, BK = 16;
}

template <int EPI, bool DUAL, bool GATHER>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs args) {
  using namespace sf;
  constexpr int BN_OUT = DUAL ? BN / 2 : BN;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];

  const Tile tile = map_tile<BM, BN_OUT>(args);
  if (!tile.valid) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  // load assignment: row tid >> 2, k quad (tid & 3) * 4
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int64_t am = tile.m0 + lr;
  if (am >= tile.m_end) am = tile.m0;
  if constexpr (GATHER) am = args.gather[am] / args.gather_div;
  const float *bbase0 = static_cast<const float *>(args.seg[0].b);
  const float *bbase_up = static_cast<const float *>(args.b_up);
  if (args.offsets != nullptr) {
    bbase0 += (int64_t)tile.e * args.b_estride;
    if (DUAL) bbase_up += (int64_t)tile.e * args.b_estride;
  }
  bool bup = false;
  int64_t bn;
  if (DUAL) {
    bup = lr >= BN / 2;
    bn = tile.n0 + (bup ? lr - BN / 2 : lr);
  } else {
    bn = tile.n0 + lr;
  }
  if (bn >= args.N) bn = tile.n0;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int s = 0; s < args.nseg; ++s) {
    const GemmSeg &sg = args.seg[s];
    const float *A = static_cast<const float *>(sg.a);
    const float *B = (s == 0) ? (bup ? bbase_up : bbase0) : static_cast<const float *>(sg.b);
    for (int64_t k0 = 0; k0 < sg.k; k0 += BK) {
      const float4 av = *reinterpret_cast<const float4 *>(A + am * sg.lda + k0 + lk);
      const float4 bv = *reinterpret_cast<const float4 *>(B + bn * sg.ldb + k0 + lk);
      As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
      Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = DUAL ? Bs[kk][(j >> 1) * 32 + tx * 2 + (j & 1)] : Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = tile.m0 + ty * 4 + i;
    if (row >= tile.m_end) continue;
    if constexpr (DUAL) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = tile.n0 + tx * 2 + j;
        if (col < args.N) epilogue<EPI, float>(args, row, col, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = tile.n0 + tx * 4 + j;
        if (col < args.N) epilogue<EPI, float>(args, row, col, acc[i][j], 0.0f);
      }
    }
  }
  if constexpr (EPI == EPI_ROUTER) {
    if (args.out_t != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = tile.m0 + ty * 4 + i;
        if (row >= tile.m_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = tile.n0 + tx * 4 + j;
          if (col < args.N) args.out_t[col * args.M + row] = acc[i][j] + (args.bias ? args.bias[col] : 0.0f);
        }
      }
    }
  }
}

}  // namespace moe
