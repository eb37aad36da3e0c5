// gemm2.h -- bf16 MFMA GEMM engine with direct-to-LDS loads.
//
// Same problem description as gemm.h (GemmArgs: dense / grouped / gathered /
// dual gate-up / K-segmented), for bf16 A operands and B in one of the
// formats of BFmt: bf16; fp8 e4m3 with 128 x 128 block scales; OCP MX FP4
// (E2M1 codes, two per byte, with an E8M0 scale per 32 K elements of a row);
// and, with MX FP8 A, MX FP4 or MX FP8 B on the block-scaled MFMA.  Quantised
// B tiles travel to LDS as stored; for the bf16 MFMA they are widened in
// registers just before it (fp8: exactly, times the power of two of the
// block scale, the scale's significand going on the accumulators).  The
// backward's layouts add operands stored K-outer and per-expert K ranges.
// Tile TM x TN x BK with TM = WM * SUBM * 32 A rows (or MA < 32 rows, see
// below), TN = WN * FRN * 32 B rows and BK = 32 to 256;
// WM x WN waves, each wave SUBM x FRN blocks of
// v_mfma_f32_32x32x16_bf16, with WM x WN = 4 or 8 waves; OCC is the launch
// bound's minimum waves per SIMD (it caps the registers of a wave at 512 / OCC).
//
//  * Global -> LDS with global_load_lds_dwordx4 (gfx950): no staging
//    registers; each wave instruction fills 1 KB = RPI tile rows of 2 BK
//    bytes (CPR 16 B chunks each).  Rows are XOR-swizzled on chunks,
//    slot = chunk ^ swz(row, CPR) (swz below), which puts the 16 rows an
//    MFMA operand read touches per 16 lanes on 16 distinct 16 B bank groups.
//    The DMA writes lane l at slot l % CPR, so lane l fetches the global
//    chunk that belongs there.
//  * STAGES-deep ring of LDS stages: the loads of tile kt + STAGES - 1 are in
//    flight while tile kt is multiplied.  The 1 KB instructions of a stage
//    are dealt round-robin to the waves; each wave issues the same number of
//    them for every tile (LW), so "tile kt landed" is, per wave,
//    s_waitcnt vmcnt(LW (STAGES-2)) followed by a barrier.
//  * Work items are spread over the 8 XCDs in contiguous ranges (workgroup i
//    runs on XCD i % 8), so the N tiles that share an A tile (one expert's
//    gathered tokens, one token block) run on one XCD and share its L2.
//  * Sub-block i of wave row wm holds tile rows (i WM + wm) 32 ..+32, so a
//    partial M tile (an expert's last rows) is shared by all wave rows and
//    skips the MFMAs of its empty sub-blocks.
//  * Single-segment problems address every DMA from a uniform base with a
//    32-bit per-lane offset, which keeps the address registers at one VGPR
//    per load instruction.
//  * Short tiles (MA > 0, one wave row of one sub-block): a tile holds MA < 32
//    rows and stages only those in LDS; the MFMA's 32 rows read them modulo
//    MA, and the rows past MA, never stored, are discarded.  When a few rows
//    stream a large weight matrix (decode), the LDS then goes to a deeper
//    ring of B tiles, i.e. more weight bytes in flight.
#pragma once

#include <type_traits>
#include <utility>

#include "gemm.h"

// kernel-local lambdas are always inlined (an outlined one puts its captures
// on the stack)
#define G2_INL __attribute__((always_inline))

namespace moe {
namespace g2 {

// Swizzle key of tile row `row` with cpr 16-byte chunks a row: rows shorter
// than 256 bytes share a 256-byte bank line 16 / cpr at a time, and each
// group of them takes its own XOR key; rows of 256 bytes or more start on
// bank group 0 and take key row % 16.
__device__ __forceinline__ constexpr int swz(int row, int cpr) {
  return cpr >= 16 ? row % 16 : (row / (16 / cpr)) % cpr;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // gfx9 encoding: vmcnt[3:0] bits 3:0, vmcnt[5:4] bits 15:14; expcnt 6:4 and
  // lgkmcnt 11:8 left at their maxima (no wait).
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
}

__device__ __forceinline__ void barrier() {
  // s_barrier without the memory fence of __syncthreads (which would wait for
  // every outstanding load, in-flight prefetches included); the asm memory
  // clobber keeps LDS accesses on their side of it.
  asm volatile("s_barrier" ::: "memory");
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), unrolled.
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ void dma16(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(g),
                                   (__attribute__((address_space(3))) void *)(lds_wave_base),
                                   16, 0, 0);
}

// Eight fp8 e4m3 codes (lo: codes 0-3, hi: codes 4-7, byte order) times the
// power of two of a block scale s, 2^floor(log2 |s|), as bf16: the B operand
// of one bf16 MFMA.  The gfx950 scaled conversion reads only the exponent of
// s, and every such product is exact in bf16 (three significand bits); the
// rest of s, its signed significand (scale_sig), multiplies the accumulators
// once per 128-wide K block instead of every element.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi, float s) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  u32x4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, false));
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, s, true));
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, false));
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, s, true));
  return __builtin_bit_cast(bf16x8, v);
}

// Signed significand of a block scale, in [1, 2) up to sign: s / 2^floor(log2 |s|).
// (A zero or subnormal scale gives 1: its block then enters at 2^-127 times
// its codes, which is zero to bf16 and fp32 accumulation alike.)
__device__ __forceinline__ float scale_sig(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x7F800000u) == 0 ? 1.0f : __uint_as_float((b & 0x807FFFFFu) | 0x3F800000u);
}

// Eight E2M1 codes (element 2i in the low nibble of byte i) times an E8M0
// block scale, as bf16: the B operand of one bf16 MFMA.  The gfx950
// conversion of byte b puts its low nibble's value in bits 15:0 and its high
// nibble's in bits 31:16, times the scale; with power-of-two scales that keep
// the products in bf16's normal range every result is exact.  The four packed
// words are moved as 32-bit values (no per-element extraction).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w, float s) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  u32x4 v;
  v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
  v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
  v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
  v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((ext_vector_type(8))) int i32x8;

template <int W>
__device__ __forceinline__ uint32_t word_of(const uint4 &v) {
  static_assert(W >= 0 && W < 4, "four words");
  return W == 0 ? v.x : W == 1 ? v.y : W == 2 ? v.z : v.w;
}

// One dword per lane: lane l's 4 bytes land at lds_wave_base + 4 l.
__device__ __forceinline__ void dma4(const void *g, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(g),
                                   (__attribute__((address_space(3))) void *)(lds_wave_base),
                                   4, 0, 0);
}

// The same direct-to-LDS loads written out in assembly (uniform base in
// SGPRs plus a 32-bit lane offset; a per-lane 64-bit address).  They return
// nothing to registers, and the compiler's wait-count pass does not see them:
// with the builtin it must assume that an LDS read may hit the bytes of any
// load still in flight, and where it cannot prove otherwise (the quantised-B
// operand reads, the transposing reads of K-outer operands) it drains every
// load (vmcnt(0)) before the read, which undoes the ring.  The kernels order these loads themselves: wait_vmcnt
// before a stage is read and before the workgroup ends, and a barrier.
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
}
// A wave-uniform address, moved to scalar registers (the SGPR-base form of
// the DMA needs it there when the compiler cannot prove it uniform).
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char *>((uint64_t)hi << 32 | lo);
}
__device__ __forceinline__ void dma16_asm(const char *sbase, uint32_t voff, void *lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_sb_asm(const char *sbase, uint32_t voff, void *lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_asm(const void *g, void *lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_addr(lds_wave_base))
               : "memory", "m0");
}

// Tile coordinates.  The tile list (M tiles x N tiles) is cut into 8
// contiguous ranges, one per XCD (workgroup b runs on XCD b % 8), so all N
// tiles of an M tile -- which share its A rows -- stay in one L2.  Inside a
// range, tiles go in groups with M fastest, so the concurrent workgroups of an
// XCD share A and B slices in its L2: dense problems use groups of group_m M
// tiles; grouped problems use one group per expert, so the M tiles of an
// expert, which read the same expert matrix, run side by side.
template <int TM, int TN_OUT>
__device__ __forceinline__ Tile map_tile_xcd(const GemmArgs &a) {
  const int64_t nt = a.n_tiles_n;
  const bool grouped = a.offsets != nullptr;
  const int64_t mtiles = grouped ? (int64_t)a.tile_offsets[a.n_experts] : (a.M + TM - 1) / TM;
  const int64_t total = mtiles * nt;
  Tile t;
  const int64_t per = (total + 7) / 8;
  const int64_t b = blockIdx.x;
  const int64_t idx = b >> 3;
  const int64_t lin = (b & 7) * per + idx;
  if (idx >= per || lin >= total) {
    t.valid = false;
    return t;
  }
  int64_t first_m, gm, r;
  int e = 0;
  if (!grouped) {
    const int64_t group_m = a.group_m > 0 ? a.group_m : 1;
    const int64_t gsz = group_m * nt;
    const int64_t g = lin / gsz;
    r = lin - g * gsz;
    first_m = g * group_m;
    gm = min(group_m, mtiles - first_m);
  } else {
    // expert e owns the linear range [tile_offsets[e] nt, tile_offsets[e+1] nt)
    const int64_t mt_lin = lin / nt;
    int lo = 0, hi = a.n_experts;  // tile_offsets[lo] <= mt_lin < tile_offsets[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tile_offsets[mid] <= mt_lin) lo = mid;
      else hi = mid;
    }
    e = lo;
    first_m = a.tile_offsets[lo];
    gm = a.tile_offsets[lo + 1] - first_m;
    r = lin - first_m * nt;
  }
  const int64_t mt = first_m + r % gm;
  t.n0 = (r / gm) * TN_OUT * (a.nper > 1 ? a.nper : 1);
  t.e = e;
  if (!grouped) {
    t.m0 = mt * TM;
    t.m_end = min(a.M, t.m0 + TM);
  } else {
    t.m0 = a.offsets[e] + (mt - first_m) * TM;
    t.m_end = min((int64_t)a.offsets[e + 1], t.m0 + TM);
  }
  t.valid = true;
  return t;
}

// Tiles of one [M][N] output per expert (the expert-batched weight
// gradients): the experts' outputs stacked along M, M tile mt being tile
// mt % mte of expert mt / mte.
template <int TM, int TN_OUT>
__device__ __forceinline__ Tile map_tile_kgrp(const GemmArgs &args) {
  GemmArgs ga = args;
  const int64_t mte = (args.M + TM - 1) / TM;
  ga.M = mte * TM * args.n_experts;
  ga.offsets = nullptr;
  Tile t = map_tile_xcd<TM, TN_OUT>(ga);
  if (t.valid) {
    const int64_t mt = t.m0 / TM;
    t.e = (int32_t)(mt / mte);
    t.m0 = (mt % mte) * TM;
    t.m_end = min(args.M, t.m0 + TM);
  }
  return t;
}

// Storage format of the B operand (and of A).
// BF_MX4A8: MXFP4 B with MX FP8 A (e4m3 codes, an E8M0 scale per 32);
// BF_MX8A8: MX FP8 B (e4m3 codes, an E8M0 scale per 32) with MX FP8 A.  Both
// run the gfx950 block-scaled MFMA on the codes as stored.
enum BFmt { BF_BF16 = 0, BF_FP8 = 1, BF_MX4 = 2, BF_MX4A8 = 3, BF_MX8A8 = 4 };

// fp8 B operands: block scales of up to this many 128-wide K blocks (K <= 16384)
constexpr int kMaxKBlocks = 128;
// MXFP4 B operands: E8M0 codes of up to this many 32-wide K blocks per row (K <= 4096)
constexpr int kMaxK32 = 128;

// Extra LDS of a kernel instance past its stage ring: the per-row factors of a
// SiTU epilogue, and the block scales of the B tile over the whole K range
// (fp8: [TN/128][kMaxKBlocks] floats; MXFP4 with K tiles of 64: [TN][kMaxK32]
// E8M0 codes -- wider K tiles carry their codes in the stage instead).
template <int EPI, int TM, int TN, int BF, int BK>
constexpr int extra_lds_bytes() {
  return (EPI == EPI_SITU ? (TM + 63) / 64 * 64 * 4 : 0) +
         (BF == BF_FP8 ? TN / 128 * kMaxKBlocks * 4
                       : (BF == BF_MX4 && BK < 128) ? TN * kMaxK32 : 0);
}

// AKO / BKO: operand A / B stored K-outer ([K][M] / [K][N] row-major, the
// transposed layouts of the backward pass) instead of [M][K] / [N][K];
// KGRP: one [M][N] output per expert e, over the K rows offsets[e] ..
// offsets[e + 1] of K-outer operands (weight gradients of the routed
// experts).
template <int WM, int WN, int SUBM, int FRN, int BK, int STAGES, int OCC, int MA, int EPI,
          bool DUAL, bool GATHER, bool MSEG, int BF, typename OutT, bool AKO = false,
          bool BKO = false, bool KGRP = false>
__global__ void __launch_bounds__(64 * WM * WN, OCC) gemm_dma_kernel(GemmArgs args) {
  static_assert(BK == 32 || BK == 64 || BK == 128 || BK == 256, "K tile of 32 to 256");
  // A is bf16, or (A8) MX FP8: e4m3 codes with an E8M0 scale per 32 along K
  constexpr bool A8 = BF == BF_MX4A8 || BF == BF_MX8A8;
  constexpr int RB = BK * (A8 ? 1 : 2);  // bytes per A tile row
  constexpr int CPR = RB / 16;        // 16 B chunks per A row
  constexpr int RPI = 1024 / RB;      // A rows per DMA wave instruction
  // B is bf16, fp8 e4m3 with 128 x 128 block scales (B8), MXFP4 (MX4) or MX
  // FP8 (MX8); MXB: B with an E8M0 scale per 32 along K
  constexpr bool B8 = BF == BF_FP8, MX4 = BF == BF_MX4 || BF == BF_MX4A8;
  constexpr bool MX8 = BF == BF_MX8A8, MXB = MX4 || MX8;
  constexpr int ESZ_B = (B8 || MX8) ? 1 : 2;  // bytes per B element (bf16, e4m3)
  // B bytes of n elements: n * BNUM / BDEN
  constexpr int BNUM = MX4 ? 1 : ESZ_B, BDEN = MX4 ? 2 : 1;
  constexpr int RB_B = BK * BNUM / BDEN;  // bytes per B tile row
  constexpr int CPR_B = RB_B / 16;
  constexpr int RPI_B = 1024 / RB_B;
  constexpr int TM = MA > 0 ? MA : WM * SUBM * 32, TN = WN * FRN * 32;
  static_assert(MA == 0 || (WM == 1 && SUBM == 1 && 32 % MA == 0 && MA % RPI == 0 && !MSEG),
                "short tiles: one 32-row MFMA block over MA staged rows");
  constexpr int TN_OUT = DUAL ? TN / 2 : TN;
  constexpr int A_BYTES = TM * RB, B_BYTES = TN * RB_B;
  static_assert(!B8 || (BK == 64 && TN_OUT % 128 == 0),
                "fp8 B: K tile 64, whole 128-row scale blocks");
  // MXFP4 B: a lane's 16-byte read of a B row holds 32 codes, one E8M0 block
  static_assert(!MXB || (BK >= 64 && !MSEG && TN % 64 == 0),
                "MXFP4 B: K tile of 64 or more, single segment");
  constexpr int NW = WM * WN;  // waves per workgroup
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  // MXFP4 with K tiles of 128 or more: the E8M0 codes of a tile's B rows
  // (SPR bytes a row) travel with the tile, after its B rows, copied a dword a
  // lane: LS instructions of 256 bytes a wave a tile, besides the operand
  // ones.  K tiles of 64 (2 bytes a row) take a whole-K table loaded up front.
  constexpr bool MXS = MXB && BK >= 128;
  constexpr int SPR = MXS ? BK / 32 : 0;
  // whole rounds of scale instructions: rows past TN are loaded, never used
  constexpr int LS = MXS ? ((TN * SPR + 255) / 256 + NW - 1) / NW : 0;
  constexpr int S_BYTES = LS * NW * 256;
  // A8: the A rows' E8M0 codes (SPR bytes a row) travel after the B codes,
  // LSA dword instructions a wave (rows past TM are loaded and never used)
  static_assert(!A8 || MXS, "MX FP8 A: in-stage scales");
  constexpr int SA_RPI = A8 ? 256 / SPR : 1;  // A rows a scale instruction
  constexpr int LSA = A8 ? ((TM + SA_RPI - 1) / SA_RPI + NW - 1) / NW : 0;
  constexpr int SA_BYTES = LSA * NW * 256;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_BYTES + SA_BYTES;
  // A stage is TA + TB wave instructions of 1 KB each (A rows, then B rows,
  // in LDS order).  Instruction g is issued by wave g % NW as its (g / NW)-th,
  // so a wave issues LMAX or LMAX - 1 of them per stage (plus LS scale ones).
  constexpr int TA = TM / RPI, TB = TN / RPI_B, TT = TA + TB;
  constexpr int LMAX = (TT + NW - 1) / NW;
  constexpr bool EVEN = TT % NW == 0;
  static_assert(TM % RPI == 0 && TN % RPI_B == 0, "whole DMA rows");
  static_assert(!DUAL || (TN / 2) % RPI_B == 0, "gate/up split on a DMA instruction");
  static_assert(!DUAL || !MXS || (TN / 2) % (256 / SPR) == 0,
                "gate/up split on a scale instruction");
  static_assert(LMAX + LS + LSA < 64 / (STAGES > 2 ? STAGES - 2 : 1), "vmcnt range");
  static_assert(!A8 || (BK >= 128 && MA == 0), "MX FP8 A: K tile of 128 or more");
  static_assert(!MSEG || (!DUAL && !A8 && !MXB && MA == 0), "segmented problems: single, bf16 A");
  constexpr int L = LMAX;
  // K-outer operands: a tile row is one k (T bf16 values, T = TM or TN), in
  // rows of whole 16-byte chunks whose index is XORed with 4 (k mod 4), so
  // the transposing fragment reads hit every bank once
  constexpr int RB_AK = TM * 2, RB_BK = TN * 2;  // bytes of a K-outer tile row
  constexpr int RPI_AK = AKO ? 1024 / RB_AK : 1, RPI_BK = BKO ? 1024 / RB_BK : 1;
  constexpr int CPR_AK = RB_AK / 16, CPR_BK = RB_BK / 16;
  static_assert(!AKO || (BF == BF_BF16 && MA == 0 && !GATHER && !MSEG && 1024 % RB_AK == 0 &&
                         RB_AK >= 256),
                "K-outer A: bf16, a tile of 128, 256 or 512 rows");
  static_assert(!BKO || (BF == BF_BF16 && !DUAL && !MSEG && 1024 % RB_BK == 0 && RB_BK >= 256),
                "K-outer B: bf16 single, a tile of 128, 256 or 512 columns");
  static_assert(!KGRP || (AKO && BKO && EPI == EPI_STORE), "expert-batched K: K-outer operands");
  // K tiles past the end of K (or of an expert's rows) are masked on the B
  // fragments; only layouts that can have such a tail carry the code
  constexpr bool KTAIL = AKO || BKO;
  static_assert(!DUAL || FRN % 2 == 0, "dual needs gate and up fragments");
  static_assert(!GATHER || !MSEG, "gathered A has one K segment");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const Tile tile = KGRP ? map_tile_kgrp<TM, TN_OUT>(args) : map_tile_xcd<TM, TN_OUT>(args);
  if (!tile.valid) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- per-row factors of the SiTU epilogue, into LDS past the ring --------
  // (older than every operand load, so the first tile's wait covers them)
  float *rs_lds = reinterpret_cast<float *>(smem + STAGES * STAGE_BYTES);
  const bool use_rs = EPI == EPI_SITU && args.row_scale != nullptr;
  if constexpr (EPI == EPI_SITU) {
    if (use_rs) {
      for (int q = wave; q < (TM + 63) / 64; q += NW) {
        int64_t m = tile.m0 + q * 64 + lane;
        if (m >= tile.m_end) m = tile.m0;  // loaded, never used
        if constexpr (BF == BF_BF16) dma4(args.row_scale + m, rs_lds + q * 64);
        else dma4_asm(args.row_scale + m, rs_lds + q * 64);
      }
    }
  }

  // ---- fp8 B: block scales of this tile's B rows over the whole K range ------
  // sc_lds[b][kb], b = 128-row block of the tile (dual: gate blocks, then up
  // blocks), kb = 128-wide K block; loaded like the row factors
  constexpr int NBL = TN / 128;
  float *sc_lds = rs_lds + (EPI == EPI_SITU ? (TM + 63) / 64 * 64 : 0);
  int kblocks = B8 ? (int)(args.seg[0].k / 128) : 0;
  if constexpr (B8 && MSEG) {
    // segments one after another along K: [NBL][sum of the segments' K blocks]
    // (plain loads into LDS, made visible by the first barrier)
#pragma unroll
    for (int sgi = 1; sgi < 5; ++sgi)
      if (sgi < args.nseg) kblocks += (int)(args.seg[sgi].k / 128);
    int kb0 = 0;
    for (int sgi = 0; sgi < args.nseg; ++sgi) {
      const int kbs = (int)(args.seg[sgi].k / 128);
      const float *bs = args.seg[sgi].bscale;
      for (int i = tid; i < NBL * kbs; i += 64 * NW) {
        const int b = i / kbs, kbl = i - b * kbs;
        int64_t nb = tile.n0 / 128 + b;
        if (nb >= (args.N + 127) / 128) nb = (args.N + 127) / 128 - 1;  // never stored
        sc_lds[b * kblocks + kb0 + kbl] = bs[nb * kbs + kbl];
      }
      kb0 += kbs;
    }
    wait_lgkm0();
  } else if constexpr (B8) {
    const int64_t nblocks = (args.N + 127) / 128;
    for (int q = wave; q * 64 < NBL * kblocks; q += NW) {
      const int i0 = q * 64 + lane;
      const int idx = i0 < NBL * kblocks ? i0 : 0;  // past the table: loaded, never used
      const int b = idx / kblocks, kb = idx - b * kblocks;
      const bool up = DUAL && b >= NBL / 2;
      int64_t nb = tile.n0 / 128 + (DUAL ? b % (NBL / 2) : b);
      if (nb >= nblocks) nb = nblocks - 1;  // rows past N: never stored
      const float *sp = (up ? args.bscale_up : args.seg[0].bscale) +
                        (int64_t)tile.e * args.s_estride + nb * kblocks + kb;
      dma4_asm(sp, sc_lds + q * 64);
    }
  }

  // ---- MXFP4 B: E8M0 codes of this tile's B rows over the whole K range -------
  // mx_lds[r][kb], r = B tile row (dual: gate rows, then up rows), kb = 32-wide
  // K block; K/32 codes a row, copied a dword per lane (rows are contiguous in
  // the tensor, K/32 is a multiple of 4)
  // Persistent N tiles (short tiles with bf16 or in-stage-scaled MXFP4 B): a
  // workgroup runs nper consecutive N tiles of its M tile, one ring over all
  // of their K tiles, storing each N tile's outputs inside the loop
  constexpr bool PN = MA > 0 && !B8 && !MSEG && EPI != EPI_ROUTER && (!MXB || MXS);
  static_assert(!(PN && (AKO || BKO)), "persistent N tiles: K-inner operands");
  const int nper = PN ? max((int)args.nper, 1) : 1;
  uint8_t *mx_lds = reinterpret_cast<uint8_t *>(sc_lds);
  const int kb32 = MXB ? (int)(args.seg[0].k / 32) : 0;
  if constexpr (MX4 && !MXS) {
    const int wpr = kb32 / 4;  // dwords a row
    const int total = TN * wpr;
    const uint8_t *e8g = args.e8_tab ? reinterpret_cast<const uint8_t *>(args.e8_tab[tile.e])
                                     : args.e8 + (int64_t)tile.e * args.s_estride;
    const uint8_t *e8u = !DUAL        ? e8g
                         : args.e8u_tab ? reinterpret_cast<const uint8_t *>(args.e8u_tab[tile.e])
                                        : args.e8_up + (int64_t)tile.e * args.s_estride;
    for (int q = wave; q * 64 < total; q += NW) {
      const int i0 = q * 64 + lane;
      const int i = i0 < total ? i0 : 0;  // past the table: loaded, never used
      const int rr = i / wpr, w4 = i - rr * wpr;
      const bool up = DUAL && rr >= TN / 2;
      int64_t n = tile.n0 + (up ? rr - TN / 2 : rr);
      if (n >= args.N) n = tile.n0;  // rows past N: never stored
      dma4_asm((up ? e8u : e8g) + n * kb32 + 4 * w4, mx_lds + q * 256);
    }
  }

  // the last instruction slot of this wave carries an instruction
  const bool has_last = EVEN || wave + NW * (LMAX - 1) < TT;

  // ---- K segments -------------------------------------------------------------
  // K range: K-outer operands run over the rows kr0 .. kr0 + klen (KGRP: the
  // expert's pair rows), in K tiles of BK, the last possibly partial
  int64_t kr0 = 0, klen = args.seg[0].k;
  if constexpr (KGRP) {
    kr0 = args.offsets[tile.e];
    klen = args.offsets[tile.e + 1] - kr0;
  }
  // B K-outer with two segments (C = A0 B0 + A1 B1, equal strides, whole K
  // tiles): one K range over both, the second segment's sources a fixed
  // distance from the first's (two-segment K-outer form)
  constexpr bool KSEG2 = BKO && !AKO && !KGRP && !MSEG;
  int kt_seg1 = INT32_MAX;
  int64_t seg1_da = 0, seg1_db = 0;
  if constexpr (KSEG2) {
    if (args.nseg == 2) {
      kt_seg1 = (int)(klen / BK);
      klen += args.seg[1].k;
      seg1_da = static_cast<const char *>(args.seg[1].a) - static_cast<const char *>(args.seg[0].a);
      seg1_db = static_cast<const char *>(args.seg[1].b) - static_cast<const char *>(args.seg[0].b);
    }
  }
  int ktiles = (int)((klen + BK - 1) / BK);
  const int ktiles_all = ktiles;
  const int klast = (int)(klen - (int64_t)(ktiles - 1) * BK);  // k values in the last K tile
  if constexpr (MSEG) {
#pragma unroll
    for (int s = 1; s < 5; ++s)
      if (s < args.nseg) ktiles += (int)(args.seg[s].k / BK);
  }

  // split K: this workgroup's range of K tiles (the host makes none empty)
  int k_begin = 0;
  if (args.ksplit > 1) {
    const int kper = (ktiles + args.ksplit - 1) / args.ksplit;
    k_begin = (int)blockIdx.y * kper;
    ktiles = min(ktiles - k_begin, kper);
  }

  // valid 32-row sub-blocks of this wave: sub-block i of wave row wm covers
  // tile rows (i WM + wm) 32 ..+32, so a partial tile spreads over both wave
  // rows; the MFMAs of empty sub-blocks are skipped
  const int rows_valid = (int)(tile.m_end - tile.m0);
  const int sb_left = (rows_valid + 31) / 32 - wm;
  int sub_valid = sb_left <= 0 ? 0 : (sb_left + WM - 1) / WM;
  sub_valid = sub_valid > SUBM ? SUBM : sub_valid;
  sub_valid = __builtin_amdgcn_readfirstlane(sub_valid);

  f32x16 acc[SUBM][FRN];
#pragma unroll
  for (int i = 0; i < SUBM; ++i)
#pragma unroll
    for (int j = 0; j < FRN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Every DMA source is a uniform base plus a 32-bit per-lane byte offset
  // (global_load_lds with an SGPR base).  Contiguous A and B are addressed
  // from the tile's first row, so the offsets stay below TM (TN) rows;
  // gathered A is addressed from the matrix start, which holds as long as the
  // gathered matrix is under 4 GiB.
  const int64_t cur_lda = args.seg[0].lda, cur_ldb = args.seg[0].ldb;
  const char *a_base = nullptr, *b_base = nullptr, *bu_base = nullptr;
  // single segment: byte offset of each instruction slot; K-segmented: the
  // slot's tile row << 8 | its 16-byte chunk (the row stride is the segment's)
  uint32_t off[LMAX];
  // uniform source base of each instruction slot (an integer: a select
  // between captured pointers would be lowered through the stack)
  uint64_t dbase[MSEG ? 1 : LMAX];
  if constexpr (!MSEG) {
    const int64_t a_first = GATHER ? 0 : tile.m0;
    const int64_t kb0 = (int64_t)k_begin * BK;
    if constexpr (AKO)
      a_base = static_cast<const char *>(args.seg[0].a) + ((kr0 + kb0) * cur_lda + tile.m0) * 2;
    else
      a_base = static_cast<const char *>(args.seg[0].a) + (a_first * cur_lda + kb0) * (A8 ? 1 : 2);
    const char *bsrc = static_cast<const char *>(args.seg[0].b);
    const char *busrc = static_cast<const char *>(args.b_up);
    if (args.b_tab != nullptr) {  // per-expert addresses (tiered experts)
      bsrc = reinterpret_cast<const char *>(args.b_tab[tile.e]);
      if (DUAL) busrc = reinterpret_cast<const char *>(args.bu_tab[tile.e]);
    } else if (args.offsets != nullptr) {
      bsrc += (int64_t)tile.e * args.b_estride * BNUM / BDEN;
      if (DUAL) busrc += (int64_t)tile.e * args.b_estride * BNUM / BDEN;
    }
    if constexpr (BKO) b_base = bsrc + ((kr0 + kb0) * cur_ldb + tile.n0) * 2;
    else b_base = bsrc + (tile.n0 * cur_ldb + kb0) * BNUM / BDEN;
    if constexpr (DUAL) bu_base = busrc + (tile.n0 * cur_ldb + kb0) * BNUM / BDEN;
  }
#pragma unroll
  for (int d = 0; d < LMAX; ++d) {
    const int g = wave + NW * d;
    uint32_t o = 0;
    if constexpr (!MSEG) {
      uint64_t bsel = reinterpret_cast<uint64_t>(a_base);
      if (g >= TA)
        bsel = reinterpret_cast<uint64_t>((DUAL && g - TA >= TB / 2) ? bu_base : b_base);
      dbase[d] = bsel;
    }
    // lane l of an instruction fills 16 B slot l % CPR of tile row l / CPR
    // and fetches the chunk that the swizzle puts there
    if (AKO && g < TA) {
      // K-outer A: k row kr of the tile, 16-byte chunk ch of its TM columns
      const int kr = g * RPI_AK + lane / CPR_AK;
      const int ch = (lane % CPR_AK) ^ (4 * (kr & 3));
      int64_t m = tile.m0 + 8 * ch;
      if (m >= tile.m_end) m = tile.m0;  // clamp: loaded, never stored
      o = (uint32_t)kr << 16 | (uint32_t)((m - tile.m0) * 2);
    } else if (BKO && g >= TA && g < TT) {
      const int kr = (g - TA) * RPI_BK + lane / CPR_BK;
      const int ch = (lane % CPR_BK) ^ (4 * (kr & 3));
      int64_t n = tile.n0 + 8 * ch;
      if (n >= args.N) n = tile.n0;
      o = (uint32_t)kr << 16 | (uint32_t)((n - tile.n0) * 2);
    } else if (g < TA) {
      const int r = g * RPI + lane / CPR;
      const int ch = (lane % CPR) ^ swz(r, CPR);
      int64_t m = tile.m0 + r;
      if (m >= tile.m_end) m = tile.m0;  // clamp: loaded, never stored
      if constexpr (MSEG) {
        o = (uint32_t)(m - tile.m0) << 8 | (uint32_t)ch;
      } else {
        const int64_t a_first = GATHER ? 0 : tile.m0;
        if constexpr (GATHER) m = args.gather[m] / args.gather_div;
        o = (uint32_t)((m - a_first) * cur_lda * (A8 ? 1 : 2) + ch * 16);
      }
    } else if (g < TT) {
      // B rows from TN/2 on are the up rows of a dual problem
      const int rb = (g - TA) * RPI_B + lane / CPR_B;
      const int ch = (lane % CPR_B) ^ swz(rb, CPR_B);
      int64_t n = tile.n0 + ((DUAL && rb >= TN / 2) ? rb - TN / 2 : rb);
      if (n >= args.N) n = tile.n0;
      if constexpr (MSEG) o = (uint32_t)(n - tile.n0) << 8 | (uint32_t)ch;
      else o = (uint32_t)((n - tile.n0) * cur_ldb * BNUM / BDEN + ch * 16);
    }
    off[d] = o;
  }
  // K-segmented problems: first global K tile, sources and strides of each
  // segment, read from the kernel arguments once (scalar registers), so that
  // the DMAs select a segment with scalar compares inside the K loop
  int seg_k0[MSEG ? 5 : 1];
  uint64_t seg_a[MSEG ? 5 : 1], seg_b[MSEG ? 5 : 1];
  uint32_t seg_lda[MSEG ? 5 : 1], seg_ldb[MSEG ? 5 : 1];
  if constexpr (MSEG) {
    int k0 = 0;
#pragma unroll
    for (int sgi = 0; sgi < 5; ++sgi) {
      const GemmSeg &sg = args.seg[sgi];
      const bool used = sgi < args.nseg;
      seg_k0[sgi] = used ? k0 : INT32_MAX;
      seg_a[sgi] = reinterpret_cast<uint64_t>(static_cast<const char *>(sg.a) + tile.m0 * sg.lda * 2);
      seg_b[sgi] =
          reinterpret_cast<uint64_t>(static_cast<const char *>(sg.b) + tile.n0 * sg.ldb * BNUM / BDEN);
      seg_lda[sgi] = (uint32_t)(sg.lda * 2);
      seg_ldb[sgi] = (uint32_t)(sg.ldb * BNUM / BDEN);
      if (used) k0 += (int)(sg.k / BK);
    }
  }
  // the sources of the K tile whose DMAs are issued next (K-segmented
  // problems; set once per tile by seg_select, branch-free)
  uint64_t ms_a = 0, ms_b = 0;
  uint32_t ms_lda = 0, ms_ldb = 0;
  auto seg_select = [&](int kt) G2_INL {
    if constexpr (MSEG) {
      const int kg = k_begin + kt;
      uint64_t a = seg_a[0], b = seg_b[0];
      uint32_t la = seg_lda[0], lb = seg_ldb[0];
      int k0 = 0;
#pragma unroll
      for (int sgi = 1; sgi < 5; ++sgi) {
        const bool in = kg >= seg_k0[sgi];
        a = in ? seg_a[sgi] : a;
        b = in ? seg_b[sgi] : b;
        la = in ? seg_lda[sgi] : la;
        lb = in ? seg_ldb[sgi] : lb;
        k0 = in ? seg_k0[sgi] : k0;
      }
      ms_a = a + (uint64_t)(kg - k0) * RB;
      ms_b = b + (uint64_t)(kg - k0) * RB_B;
      ms_lda = la;
      ms_ldb = lb;
    }
  };
  // MXFP4 scale instructions of this wave: instruction gs = wave + NW q fills
  // bytes 256 gs.. of the stage's code area; lane l copies dword w of the
  // codes of tile row rr (the B row numbering: dual up rows from TN/2), from
  // a uniform base (gate or up codes of this expert, from this split's first
  // K block) plus a 32-bit lane offset
  uint32_t soff[MXS ? LS : 1];
  uint64_t sbase[MXS ? LS : 1];
  if constexpr (MXS) {
#pragma unroll
    for (int q = 0; q < LS; ++q) {
      const int gs = wave + NW * q;
      const int i = gs * 64 + lane;
      const int rr = i / (SPR / 4), w = i % (SPR / 4);
      const bool up = DUAL && rr >= TN / 2 && rr < TN;
      int64_t n = tile.n0 + (up ? rr - TN / 2 : rr);
      if (rr >= TN || n >= args.N) n = tile.n0;  // loaded, never used
      soff[q] = (uint32_t)(n * kb32 + 4 * w);
      const uint8_t *e8x =
          args.e8_tab ? reinterpret_cast<const uint8_t *>((up ? args.e8u_tab : args.e8_tab)[tile.e])
                      : (up ? args.e8_up : args.e8) + (int64_t)tile.e * args.s_estride;
      sbase[q] = reinterpret_cast<uint64_t>(e8x + (int64_t)k_begin * BK / 32);
    }
  }
  // A8: scale instructions of the A rows: instruction gs = wave + NW q, lane l
  // copies dword w of the codes of tile row rr (gathered rows addressed from
  // the matrix start, like the A rows)
  uint32_t saoff[A8 ? LSA : 1];
  const char *sa_base = nullptr;
  if constexpr (A8) {
    sa_base = reinterpret_cast<const char *>(args.a_sc) + (int64_t)k_begin * BK / 32;
#pragma unroll
    for (int q = 0; q < LSA; ++q) {
      const int i = (wave + NW * q) * 64 + lane;
      const int rr = i / (SPR / 4), w = i % (SPR / 4);
      int64_t m = tile.m0 + rr;
      if (rr >= TM || m >= tile.m_end) m = tile.m0;  // loaded, never used
      if constexpr (GATHER) m = args.gather[m] / args.gather_div;
      saoff[q] = (uint32_t)(m * args.lda_sc + 4 * w);
    }
  }
  // B bytes from one N tile to the next (persistent N tiles)
  const int64_t nstep_b = PN ? (int64_t)TN_OUT * cur_ldb * BNUM / BDEN : 0;
  // DMA instruction slot d of this wave (instruction g = wave + NW d) of K
  // tile kt of N tile jn (persistent N tiles; else 0) into stage st.
  auto dma_one = [&](auto d_tag, int kt, int st, int jn) G2_INL {
    constexpr int d = decltype(d_tag)::value;
    if constexpr (!EVEN && d == LMAX - 1) {
      if (!has_last) return;
    }
    const int g = wave + NW * d;
    if constexpr (MSEG) {
      // the sources seg_select chose for this K tile
      const bool is_a = g < TA;
      const char *base = uniform_ptr(reinterpret_cast<const char *>(is_a ? ms_a : ms_b));
      uint32_t o = __umul24(off[d] >> 8, is_a ? ms_lda : ms_ldb) + (off[d] & 0xFFu) * 16u;
      if constexpr (BF != BF_BF16) {
        dma16_asm(base, o, smem + st * STAGE_BYTES + g * 1024);
      } else {
        asm volatile("" : "+v"(o));
        dma16(base + o, smem + st * STAGE_BYTES + g * 1024);
      }
      return;
    }
    const char *base = reinterpret_cast<const char *>(dbase[MSEG ? 0 : d]);
    // (builtin form: the empty asm re-issues the 32-bit offset inside the loop
    // body, so the instruction selector sees uniform base + zext(offset) there
    // (SGPR-base form) instead of a 64-bit address hoisted out of the loop)
    uint32_t o = off[d];
    const int kt_glob = kt;  // (K tile over both segments)
    if constexpr (KSEG2) {
      // K tiles of the second segment: its sources, from its own first K tile
      if (k_begin + kt >= kt_seg1) {
        base += g < TA ? seg1_da : seg1_db;
        kt -= kt_seg1 - k_begin;
      }
    }
    if constexpr (AKO || BKO) {
      const bool ko = (AKO && g < TA) || (BKO && g >= TA);
      if (ko) {
        // k rows past the end of K (last tile) re-read the last row; the B
        // fragments mask those k
        const int kv = k_begin + kt_glob == ktiles_all - 1 ? klast : BK;
        const uint32_t kr = min((int)(o >> 16), kv - 1);
        const int64_t ldx = g < TA ? cur_lda : cur_ldb;
        o = __umul24(kr, (uint32_t)(ldx * 2)) + (o & 0xFFFFu);
        asm volatile("" : "+v"(o));
        dma16_asm(uniform_ptr(base + (int64_t)kt * BK * ldx * 2), o,
                  smem + st * STAGE_BYTES + g * 1024);
        return;
      }
    }
    int64_t kb = (int64_t)kt * (g < TA ? RB : RB_B);
    if constexpr (PN) kb += g < TA ? 0 : jn * nstep_b;
    if constexpr (B8 || AKO || BKO) {
      // (the block-scale branch of the fp8 K loop, and the K-outer layouts'
      // clamps, leave the base's uniformity to the compiler's guess: moved to
      // scalar registers explicitly)
      dma16_asm(uniform_ptr(base + kb), o, smem + st * STAGE_BYTES + g * 1024);
    } else if constexpr (BF != BF_BF16) {
      dma16_asm(base + kb, o, smem + st * STAGE_BYTES + g * 1024);
    } else {
      asm volatile("" : "+v"(o));
      dma16(base + kb + o, smem + st * STAGE_BYTES + g * 1024);
    }
  };
  // the MXFP4 scale instructions of K tile kt of N tile jn into stage st
  auto dma_scales = [&](int kt, int st, int jn) G2_INL {
    if constexpr (MXS) {
#pragma unroll
      for (int q = 0; q < LS; ++q)
        dma4_sb_asm(reinterpret_cast<const char *>(sbase[q]) + (int64_t)kt * SPR +
                        (PN ? (int64_t)jn * TN_OUT * kb32 : 0),
                    soff[q],
                    smem + st * STAGE_BYTES + A_BYTES + B_BYTES + (wave + NW * q) * 256);
    }
  };
  // A8: the A scale instructions of K tile kt into stage st
  auto dma_ascales = [&](int kt, int st) G2_INL {
    if constexpr (A8) {
#pragma unroll
      for (int q = 0; q < LSA; ++q)
        dma4_sb_asm(sa_base + (int64_t)kt * SPR, saoff[q],
                    smem + st * STAGE_BYTES + A_BYTES + B_BYTES + S_BYTES +
                        (wave + NW * q) * 256);
    }
  };
  // "tile kt landed": this wave's loads of later tiles may still be in flight
  auto wait_tile = [&]() G2_INL {
    if constexpr (EVEN) {
      wait_vmcnt<(LMAX + LS + LSA) * (STAGES - 2)>();
    } else {
      if (has_last) wait_vmcnt<(LMAX + LS + LSA) * (STAGES - 2)>();
      else wait_vmcnt<(LMAX - 1 + LS + LSA) * (STAGES - 2)>();
    }
  };

  // Operand fragment f of k step ks (f < FRN: B fragment f, else A fragment f - FRN).
  auto read_frag = [&](const char *st, int ks, auto f_tag, bf16x8 *af,
                       bf16x8 *bfr) G2_INL {
    constexpr int f = decltype(f_tag)::value;
    // k order of a step: lane half h takes k 8h..8h+8 of the step's 16; with
    // fp8 B, steps 2p and 2p+1 take the two halves of chunk 2p + h instead
    // (one 16-byte B read per lane per two steps); with MXFP4 B, steps 4g ..
    // 4g+3 take the four quarters of K range 64g + 32h ..+32 (B chunk 2g + h:
    // one 16-byte read and one E8M0 block per lane per four steps).  A follows
    // the same order.
    const int chunk = B8 ? 4 * (ks >> 1) + 2 * (lane >> 5) + (ks & 1)
                      : MX4 ? 8 * (ks >> 2) + 4 * (lane >> 5) + (ks & 3)
                            : ks * 2 + (lane >> 5);
    int r;
    const char *base;
    if constexpr (f < FRN) {
      constexpr int j = f;
      if (DUAL) r = (j < FRN / 2) ? ((wn * (FRN / 2) + j) * 32 + (lane & 31))
                                  : (TN / 2 + (wn * (FRN / 2) + j - FRN / 2) * 32 + (lane & 31));
      else r = (wn * FRN + j) * 32 + (lane & 31);
      base = st + A_BYTES;
    } else {
      r = MA > 0 ? (lane & 31) % MA : ((f - FRN) * WM + wm) * 32 + (lane & 31);
      base = st;
    }
    bf16x8 v;
    constexpr bool KO = f < FRN ? BKO : AKO;
    if constexpr (KO) {
      // K-outer operand: the fragment's 32 columns c0.. over k 16 ks ..+16,
      // two transposing reads of four k each.  Lane (g, s) of a 16-lane group
      // g supplies k row 8 (g / 2) + s / 4 (+ 4), columns 16 (g % 2) + 4 (s % 4)
      // ..+4; lane i of the group receives element i % 4 of the chunks of
      // lanes i / 4 + 4 j, j = 0..3: column c0 + (lane % 32), k 8 (lane / 32) + j
      constexpr int RBX = f < FRN ? RB_BK : RB_AK;
      const int c0 = r - (lane & 31);
      const int g16 = lane >> 4, sx = lane & 15;
      const int col = c0 + 16 * (g16 & 1) + 4 * (sx & 3);
      const int kr = 16 * ks + 8 * (g16 >> 1) + (sx >> 2);  // kr % 4 == sx / 4
      const char *p0 = base + kr * RBX + (((col >> 3) ^ (4 * (sx >> 2))) << 4) + (col & 7) * 2;
      typedef __attribute__((ext_vector_type(4))) short s4;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4 *)(uintptr_t)lds_addr(p0));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4 *)(uintptr_t)lds_addr(p0 + 4 * RBX));
      typedef __attribute__((ext_vector_type(8))) short s8;
      v = __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    } else {
      v = *reinterpret_cast<const bf16x8 *>(base + r * RB + ((chunk ^ swz(r, CPR)) << 4));
    }
    if constexpr (f < FRN) bfr[f] = v;
    else af[f - FRN] = v;
  };
  // fp8 B: tile row of B fragment j for this lane (dual: gate fragments, then up)
  auto b_row_of = [&](auto j_tag) G2_INL {
    constexpr int j = decltype(j_tag)::value;
    if constexpr (DUAL)
      return j < FRN / 2 ? (wn * (FRN / 2) + j) * 32 + (lane & 31)
                         : TN / 2 + (wn * (FRN / 2) + j - FRN / 2) * 32 + (lane & 31);
    else
      return (wn * FRN + j) * 32 + (lane & 31);
  };
  // quantised B: 16 bytes of fragment j's row at chunk 2p + h -- fp8: the codes
  // of k-step pair p; MXFP4: the 32 codes of k-step group p (steps 4p..4p+3)
  auto read_b8 = [&](const char *st, int p, auto j_tag, uint4 *raw) G2_INL {
    constexpr int j = decltype(j_tag)::value;
    const int r = b_row_of(j_tag);
    const int chunk = 2 * p + (lane >> 5);
    // (read with the operand type of the bf16 reads: the compiler then keeps
    // its LDS accesses independent of the DMA writes in flight, as for those)
    raw[j] = __builtin_bit_cast(uint4, *reinterpret_cast<const bf16x8 *>(
                                           st + A_BYTES + r * RB_B + ((chunk ^ swz(r, CPR_B)) << 4)));
  };
  // fp8 B: block scale of fragment j for K tile kt (uniform per wave)
  auto scale_b8 = [&](int kt, auto j_tag) G2_INL {
    const int rb = b_row_of(j_tag) - (lane & 31);
    return sc_lds[(rb / 128) * kblocks + ((k_begin + kt) * BK) / 128];
  };
  // MXFP4 B: E8M0 scale of this lane's row and K block (chunk 2g + h of K tile
  // kt, in stage st) for fragment j, as an fp32 power of two (codes 1..254)
  auto scale_b4 = [&](const char *st, int kt, int g, auto j_tag) G2_INL {
    const int r = b_row_of(j_tag);
    uint32_t e;
    if constexpr (MXS)
      e = *reinterpret_cast<const uint8_t *>(st + A_BYTES + B_BYTES + r * SPR + 2 * g +
                                             (lane >> 5));
    else
      e = mx_lds[r * kb32 + (k_begin + kt) * (BK / 32) + 2 * g + (lane >> 5)];
    return __uint_as_float(e << 23);
  };
  // ---- stores of the output tile at columns n0.. (the epilogue; with
  // persistent N tiles also called inside the K loop): lane holds column
  // (lane & 31), rows 8(r/4) + 4(lane/32) + r%4 of each 32 x 32 block.  Row
  // quantities are formed once per row, column ones once per block column;
  // the SiTU row factors come from LDS.
  constexpr int JN = DUAL ? FRN / 2 : FRN;  // output block columns of this wave
  auto store_tile = [&](int64_t n0) G2_INL {
    int64_t col[JN];
    bool col_ok[JN];
    float bias[JN];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      col[j] = n0 + (wn * JN + j) * 32 + (lane & 31);
      col_ok[j] = col[j] < args.N;
      bias[j] = (EPI == EPI_ROUTER && args.bias && col_ok[j]) ? args.bias[col[j]] : 0.0f;
    }
    OutT *out = static_cast<OutT *>(args.out) + (KGRP ? (int64_t)tile.e * args.M * args.ldo : 0);
    // the plain store (no row factor, no residual): the common case, kept free
    // of the per-row loads of the general one
    const bool plain_store = args.resid == nullptr && args.row_scale == nullptr;
    if constexpr (A8 && EPI == EPI_SITU) {
      if (args.q_codes != nullptr) {
        // MX FP8 output.  The 32 columns of each of this wave's JN block
        // columns make one MX block per row: each wave stages its SiTU outputs
        // (bf16, as they would be stored) in LDS as [rows][JN * 32], then every
        // lane quantises whole (row, block) pairs -- no cross-lane exchange.
        // The ring is reused for the staging once every DMA has landed and
        // every wave has left the loop.
        constexpr int RW = JN * 32;  // staged columns a row
        static_assert(NW * SUBM * 32 * RW * 2 <= STAGES * STAGE_BYTES, "staging fits the ring");
        wait_vmcnt<0>();
        barrier();
        uint16_t *wl = reinterpret_cast<uint16_t *>(smem) + wave * (SUBM * 32 * RW);
#pragma unroll
        for (int i = 0; i < SUBM; ++i) {
          if (i >= sub_valid) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float f = use_rs ? rs_lds[(i * WM + wm) * 32 + lr - i * 32] : 1.0f;
#pragma unroll
            for (int j = 0; j < JN; ++j)
              wl[lr * RW + j * 32 + (lane & 31)] = f32_to_bf16(
                  f * situ(acc[i][j][r], acc[i][j + FRN / 2][r], args.beta, args.inv_beta,
                           args.beta_u, args.inv_beta_u));
          }
        }
        for (int it = lane; it < sub_valid * 32 * JN; it += 64) {
          const int lr = it / JN, j = it % JN;
          const int64_t c0 = n0 + (wn * JN + j) * 32;  // first column of the block
          const int64_t row = tile.m0 + ((lr >> 5) * WM + wm) * 32 + (lr & 31);
          if (c0 < args.N && row < tile.m_end) {
            const uint4 *src = reinterpret_cast<const uint4 *>(wl + lr * RW + j * 32);
            float v[32];
            float amax = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint4 w4 = src[q];
              const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                v[8 * q + 2 * h] = bf16_to_f32((uint16_t)(w[h] & 0xFFFFu));
                v[8 * q + 2 * h + 1] = bf16_to_f32((uint16_t)(w[h] >> 16));
                amax = fmaxf(amax, fmaxf(fabsf(v[8 * q + 2 * h]), fabsf(v[8 * q + 2 * h + 1])));
              }
            }
            const int shared = mx8_shared_exp(amax);
            const float inv = __uint_as_float((uint32_t)(127 - shared) << 23);
            uint32_t code[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              code[q] = 0;
#pragma unroll
              for (int b = 0; b < 4; ++b) code[q] |= f32_to_e4m3_sat(v[4 * q + b] * inv) << (8 * b);
            }
            uint4 *dst = reinterpret_cast<uint4 *>(args.q_codes + row * args.ldq + c0);
            dst[0] = make_uint4(code[0], code[1], code[2], code[3]);
            dst[1] = make_uint4(code[4], code[5], code[6], code[7]);
            args.q_scales[row * args.ldq_sc + c0 / 32] = (uint8_t)(shared + 127);
          }
        }
        return;
      }
    }
    // one loop nest per store form, so that the plain store's code carries
    // none of the waits that the general form's loads would put at every join
    auto rows_loop = [&](auto general_tag) G2_INL {
      constexpr bool GEN = decltype(general_tag)::value;
#pragma unroll
      for (int i = 0; i < SUBM; ++i) {
        if (i >= sub_valid) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t row = tile.m0 + rr;
          if (row >= tile.m_end) continue;
          OutT *orow = out + row * args.ldo;
          if constexpr (EPI == EPI_SITU) {
            const float f = use_rs ? rs_lds[rr] : 1.0f;
#pragma unroll
            for (int j = 0; j < JN; ++j)
              if (col_ok[j]) {
                store_out<OutT>(orow, col[j],
                                f * situ(acc[i][j][r], acc[i][j + FRN / 2][r], args.beta,
                                         args.inv_beta, args.beta_u, args.inv_beta_u));
                if constexpr (GEN) {  // and the raw gate and up sums
                  args.out_g[row * args.ldgu + col[j]] = acc[i][j][r];
                  args.out_u[row * args.ldgu + col[j]] = acc[i][j + FRN / 2][r];
                }
              }
          } else if constexpr (EPI == EPI_ROUTER) {
#pragma unroll
            for (int j = 0; j < JN; ++j)
              if (col_ok[j]) store_out<float>(orow, col[j], acc[i][j][r] + bias[j]);
          } else if constexpr (!GEN) {
#pragma unroll
            for (int j = 0; j < JN; ++j)
              if (col_ok[j]) store_out<OutT>(orow, col[j], acc[i][j][r]);
          } else {
            // store (times the row's factor, when given), plus the residual row
            // (read before the write: it may be the output)
            const void *rrow = args.resid ? static_cast<const char *>(args.resid) +
                                                row * args.ldr * (int64_t)sizeof(OutT)
                                          : nullptr;
            const float f = args.row_scale ? args.row_scale[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < JN; ++j)
              if (col_ok[j])
                store_out<OutT>(orow, col[j],
                                f * acc[i][j][r] + (rrow ? load_in<OutT>(rrow, col[j]) : 0.0f));
          }
        }
      }
    };
    if constexpr (EPI == EPI_STORE) {
      if (plain_store) rows_loop(std::false_type{});
      else rows_loop(std::true_type{});
    } else if constexpr (EPI == EPI_SITU) {
      if (args.out_g != nullptr) rows_loop(std::true_type{});
      else rows_loop(std::false_type{});
    } else {
      rows_loop(std::false_type{});
    }
    if constexpr (EPI == EPI_ROUTER) {
      if (args.out_t != nullptr) {
#pragma unroll
        for (int i = 0; i < SUBM; ++i)
#pragma unroll
          for (int j = 0; j < FRN; ++j) {
            const int64_t c = col[j];
            if (!col_ok[j]) continue;
            const float b = bias[j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t row0 = tile.m0 + (i * WM + wm) * 32 + 8 * q + 4 * (lane >> 5);
              float *dst = args.out_t + c * args.M + row0;
              if (row0 + 3 < tile.m_end && (args.M & 3) == 0) {
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(acc[i][j][q * 4 + 0] + b, acc[i][j][q * 4 + 1] + b,
                                acc[i][j][q * 4 + 2] + b, acc[i][j][q * 4 + 3] + b);
              } else {
                for (int u = 0; u < 4; ++u)
                  if (row0 + u < tile.m_end) dst[u] = acc[i][j][q * 4 + u] + b;
              }
            }
          }
      }
    }
  };

  // K loop for NS active sub-blocks.  Single-segment problems run one
  // straight-line schedule per stage: MFMAs one at a time, with the fragment
  // reads of the next k step and the DMA instructions of the tile STAGES - 1
  // ahead placed between them, so the in-order issue hides them behind the
  // MFMA pipe.  The prefetch is unconditional (past the end it re-reads the
  // last tile into a stage nobody reads again), so every wave has a fixed
  // number of loads per tile in flight and the wait count is a constant.
  auto mainloop = [&](auto ns_tag) G2_INL {
    constexpr int NS = decltype(ns_tag)::value;
    constexpr int NA = NS > 0 ? NS : 1;
    constexpr int KS = BK / 16;   // k steps per stage
    constexpr int NF = NS + FRN;  // fragment reads per k step
    constexpr int Q = NS * FRN;   // MFMAs per k step
    {
      // tile t of the T = nper ktiles of this workgroup: N tile t / ktiles,
      // K tile t % ktiles
      const int T = nper * ktiles;
#pragma unroll
      for (int p = 0; p < STAGES - 1; ++p) {
        const int tp = p < T ? p : T - 1;
        const int jp = PN ? tp / ktiles : 0;
        seg_select(tp - jp * ktiles);
        static_for<L>([&](auto d) G2_INL { dma_one(d, tp - jp * ktiles, p, jp); });
        dma_scales(tp - jp * ktiles, p, jp);
        dma_ascales(tp - jp * ktiles, p);
      }
      int kt = 0, jn = 0;  // K tile and N tile of t
      for (int t = 0; t < T; ++t) {
        wait_tile();
        barrier();
        const char *st = smem + (t % STAGES) * STAGE_BYTES;
        const int kd = t + STAGES - 1;
        const int kdt = kd < T ? kd : T - 1;
        const int dj = PN ? kdt / ktiles : 0;
        const int kdc = kdt - dj * ktiles;
        const int dst = kd % STAGES;
        seg_select(kdc);
        if constexpr (A8) {
          // block-scaled MFMA: all loads of the tile STAGES - 1 ahead first, then
          // per 64-wide k step the operands and scales of NS x FRN
          // v_mfma_scale_f32_32x32x64_f8f6f4 (A e4m3, B E2M1 or e4m3 as stored).
          // Scale block b of the step (its k 32 b.. 32 b + 31, MX block 2 S + b)
          // is, for E2M1 B, B lane half b (one 16-byte chunk of 32 codes,
          // 2 S + b), and for e4m3 operands bytes 16 b.. 16 b + 15 of both lane
          // halves (half h: k 32 b + 16 h ..+16, so a lane reads chunks 4 S + h
          // and 4 S + 2 + h); the scale of block b comes from lane half b, on
          // both operands.
          static_for<L>([&](auto d) G2_INL { dma_one(d, kdc, dst, dj); });
          dma_scales(kdc, dst, dj);
          dma_ascales(kdc, dst);
          if constexpr (NS > 0) {
            const uint8_t *sa_st = reinterpret_cast<const uint8_t *>(
                st + A_BYTES + B_BYTES + S_BYTES);
            static_for<BK / 64>([&](auto s_tag) G2_INL {
              constexpr int S = decltype(s_tag)::value;
              i32x8 bq[FRN];
              int bs[FRN];
              static_for<FRN>([&](auto j) G2_INL {
                if constexpr (MX8) {
                  // e4m3 B: the A lane layout (chunks 4 S + h and 4 S + 2 + h)
                  const int rb = b_row_of(j);
                  const char *br = st + A_BYTES + rb * RB_B;
                  const int c0 = 4 * S + (lane >> 5);
                  const uint4 lo =
                      *reinterpret_cast<const uint4 *>(br + ((c0 ^ swz(rb, CPR_B)) << 4));
                  const uint4 hi =
                      *reinterpret_cast<const uint4 *>(br + (((c0 + 2) ^ swz(rb, CPR_B)) << 4));
                  bq[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                } else {
                  uint4 raw[FRN];
                  read_b8(st, S, j, raw);
                  bq[j] = i32x8{(int)raw[j].x, (int)raw[j].y, (int)raw[j].z, (int)raw[j].w,
                                0, 0, 0, 0};
                }
                bs[j] = (int)*reinterpret_cast<const uint8_t *>(
                    st + A_BYTES + B_BYTES + b_row_of(j) * SPR + 2 * S + (lane >> 5));
              });
#pragma unroll
              for (int i = 0; i < NS; ++i) {
                const int r = (i * WM + wm) * 32 + (lane & 31);
                const int c0 = 4 * S + (lane >> 5);
                const char *ar = st + r * RB;
                const uint4 lo = *reinterpret_cast<const uint4 *>(ar + ((c0 ^ swz(r, CPR)) << 4));
                const uint4 hi =
                    *reinterpret_cast<const uint4 *>(ar + (((c0 + 2) ^ swz(r, CPR)) << 4));
                const i32x8 aq = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                const int as = (int)sa_st[r * SPR + 2 * S + (lane >> 5)];
#pragma unroll
                for (int j = 0; j < FRN; ++j)
                  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                      aq, bq[j], acc[i][j], 0 /* A e4m3 */, MX8 ? 0 /* B e4m3 */ : 4 /* B e2m1 */,
                      0, as, 0, bs[j]);
              }
              // keep the next k step's LDS reads after these MFMAs (registers)
              __builtin_amdgcn_sched_barrier(0);
            });
          }
        } else if constexpr (NS == 0) {
          static_for<L>([&](auto d) G2_INL { dma_one(d, kdc, dst, dj); });
          dma_scales(kdc, dst, dj);
        } else {
          bf16x8 fa[2][NA], fb[2][FRN];
          uint4 braw[B8 || MX4 ? FRN : 1];
          float bsc[B8 || MX4 ? FRN : 1];
          // MXFP4: codes and scale of the next group of four k steps
          uint4 braw2[MX4 && KS > 4 ? FRN : 1];
          float bsc2[MX4 && KS > 4 ? FRN : 1];
          if constexpr (MX4) {
            // the codes of the first four k steps, one read per fragment
            static_for<FRN>([&](auto j) G2_INL {
              bsc[j] = scale_b4(st, kt, 0, j);
              read_b8(st, 0, j, braw);
            });
            static_for<NF>([&](auto f) G2_INL {
              if constexpr (f >= FRN) read_frag(st, 0, f, fa[0], fb[0]);
            });
            static_for<FRN>([&](auto j) G2_INL {
              fb[0][j] = e2m1x8_to_bf16(braw[j].x, bsc[j]);
            });
          } else if constexpr (B8) {
            static_for<FRN>([&](auto j) G2_INL {
              bsc[j] = scale_b8(kt, j);
              read_b8(st, 0, j, braw);
            });
            // the first K tile of a 128-wide block after another: the
            // accumulators, in units of the previous block's scale significand,
            // change to this block's
            if (kt > 0 && ((k_begin + kt) & 1) == 0) {
              static_for<FRN>([&](auto j_tag) G2_INL {
                constexpr int j = decltype(j_tag)::value;
                const float ratio = scale_sig(scale_b8(kt - 1, j_tag)) / scale_sig(bsc[j]);
#pragma unroll
                for (int i = 0; i < NS; ++i)
#pragma unroll
                  for (int r = 0; r < 16; ++r) acc[i][j][r] *= ratio;
              });
            }
            static_for<NF>([&](auto f) G2_INL {
              if constexpr (f >= FRN) read_frag(st, 0, f, fa[0], fb[0]);
            });
            static_for<FRN>([&](auto j) G2_INL {
              fb[0][j] = e4m3x8_to_bf16(braw[j].x, braw[j].y, bsc[j]);
            });
          } else {
            static_for<NF>([&](auto f) G2_INL { read_frag(st, 0, f, fa[0], fb[0]); });
          }
          // a partial last K tile: k values past the end read as zero on B
          const bool tail = KTAIL && k_begin + kt == ktiles_all - 1 && klast < BK;
          static_for<KS>([&](auto s_tag) G2_INL {
            constexpr int S = decltype(s_tag)::value;
            if constexpr (KTAIL) {
              if (tail) {
                const int k8 = 16 * S + 8 * (lane >> 5);
                static_for<FRN>([&](auto j) G2_INL {
#pragma unroll
                  for (int e = 0; e < 8; ++e)
                    if (k8 + e >= klast) fb[S & 1][j][e] = (__bf16)0.0f;
                });
              }
            }
            static_for<Q>([&](auto q_tag) G2_INL {
              constexpr int q = decltype(q_tag)::value;
              constexpr int i = q / FRN, j = q % FRN;
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[S & 1][i], fb[S & 1][j],
                                                                  acc[i][j], 0, 0, 0);
              // next step's fragments from the first MFMAs on (one per MFMA when
              // they fit), so they have landed when the step starts
              if constexpr (S + 1 < KS) {
                static_for<NF>([&](auto f_tag) G2_INL {
                  constexpr int f = decltype(f_tag)::value;
                  constexpr bool mine = NF <= Q ? (f == q) : (f >= q * NF / Q && f < (q + 1) * NF / Q);
                  if constexpr (mine) {
                    if constexpr (MX4 && f < FRN) {
                      // MXFP4 B: widen the next step's codes (in registers: the
                      // group's read two steps ahead of its first step)
                      constexpr int G = (S + 1) / 4, W = (S + 1) % 4;
                      if constexpr (G % 2 == 0)
                        fb[(S + 1) & 1][f] = e2m1x8_to_bf16(word_of<W>(braw[f]), bsc[f]);
                      else
                        fb[(S + 1) & 1][f] = e2m1x8_to_bf16(word_of<W>(braw2[f]), bsc2[f]);
                      if constexpr ((S + 2) % 4 == 0 && S + 2 < KS) {
                        constexpr int G2 = (S + 2) / 4;
                        if constexpr (G2 % 2 == 0) {
                          read_b8(st, G2, f_tag, braw);
                          bsc[f] = scale_b4(st, kt, G2, f_tag);
                        } else {
                          read_b8(st, G2, f_tag, braw2);
                          bsc2[f] = scale_b4(st, kt, G2, f_tag);
                        }
                      }
                    } else if constexpr (B8 && f < FRN) {
                      // fp8 B: an even step reads the pair's codes, an odd step
                      // converts the upper half read one step earlier
                      if constexpr ((S + 1) % 2 == 0) read_b8(st, (S + 1) / 2, f_tag, braw);
                      else fb[(S + 1) & 1][f] = e4m3x8_to_bf16(braw[f].z, braw[f].w, bsc[f]);
                    } else {
                      read_frag(st, S + 1, f_tag, fa[(S + 1) & 1], fb[(S + 1) & 1]);
                    }
                  }
                });
                if constexpr (B8 && (S + 1) % 2 == 0) {
                  // lower half of the codes read above, late in the step
                  static_for<FRN>([&](auto j_tag) G2_INL {
                    constexpr int j = decltype(j_tag)::value;
                    constexpr int at = Q - FRN + j > j ? Q - FRN + j : j;
                    if constexpr (q == at)
                      fb[(S + 1) & 1][j] = e4m3x8_to_bf16(braw[j].x, braw[j].y, bsc[j]);
                  });
                }
              }
              // DMAs of the tile STAGES - 1 ahead: with two stages that tile is
              // needed at the next barrier, so they all go out in the first k
              // step; deeper rings spread them over the whole stage
              constexpr int DS = STAGES == 2 ? 1 : KS;  // k steps that carry DMAs
              if constexpr (S < DS) {
                constexpr int g = S * Q + q;
                static_for<L>([&](auto d_tag) G2_INL {
                  constexpr int d = decltype(d_tag)::value;
                  if constexpr (d >= g * L / (DS * Q) && d < (g + 1) * L / (DS * Q))
                    dma_one(d_tag, kdc, dst, dj);
                });
                if constexpr (g == 0) dma_scales(kdc, dst, dj);
              }
              __builtin_amdgcn_sched_barrier(0);
            });
          });
        }
        if constexpr (PN) {
          // the last K tile of N tile jn: store it, start the next one afresh
          // (the row factors in LDS landed before the first tile: older loads)
          if (kt == ktiles - 1) {
            store_tile(tile.n0 + (int64_t)jn * TN_OUT);
#pragma unroll
            for (int i = 0; i < SUBM; ++i)
#pragma unroll
              for (int j = 0; j < FRN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
            kt = 0;
            ++jn;
          } else {
            ++kt;
          }
        } else {
          ++kt;
        }
      }
      wait_vmcnt<0>();  // no DMA may still write LDS when the workgroup ends
      if constexpr (B8 && NS > 0) {
        // the last block's scale significand
        static_for<FRN>([&](auto j_tag) G2_INL {
          constexpr int j = decltype(j_tag)::value;
          const float sig = scale_sig(scale_b8(ktiles - 1, j_tag));
#pragma unroll
          for (int i = 0; i < NS; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] *= sig;
        });
      }
    }
  };
  // one specialised copy of the K loop per number of active sub-blocks
  static_assert(SUBM <= 5, "mainloop dispatch covers up to 5 sub-blocks");
  if (!KGRP || ktiles > 0) switch (sub_valid) {
    case 0: mainloop(std::integral_constant<int, 0>{}); break;
    case 1: mainloop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (SUBM >= 2) mainloop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (SUBM >= 3) mainloop(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (SUBM >= 4) mainloop(std::integral_constant<int, 4>{}); break;
    default: if constexpr (SUBM >= 5) mainloop(std::integral_constant<int, 5>{}); break;
  }
  if constexpr (PN) return;  // stored inside the K loop


  // ---- epilogue: lane holds column (lane & 31), rows 8(r/4) + 4(lane/32) + r%4
  // of each 32 x 32 block.  Row quantities are formed once per row, column
  // ones once per block column; the SiTU row factors come from LDS.
  if (args.ksplit > 1) {
    // split K: raw sums of this K range; the reduction applies the epilogue
    float *part = args.partial + (int64_t)blockIdx.y * args.M * args.ldp;
#pragma unroll
    for (int i = 0; i < SUBM; ++i) {
      if (i >= sub_valid) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row =
            tile.m0 + (i * WM + wm) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= tile.m_end) continue;
#pragma unroll
        for (int j = 0; j < FRN; ++j) {
          constexpr int JH = DUAL ? FRN / 2 : FRN;
          const int jo = j % JH;
          const int64_t col = tile.n0 + (wn * JH + jo) * 32 + (lane & 31);
          if (col < args.N) part[row * args.ldp + col + (j >= JH ? args.N : 0)] = acc[i][j][r];
        }
      }
    }
    return;
  }
  if constexpr (EPI == EPI_SITU) {
    if (use_rs) {
      wait_vmcnt<0>();
      barrier();
    }
  }
  store_tile(tile.n0);
}

// Split-K reduction: out[m][c] = epilogue(sum over splits, in split order),
// one output element per thread; eight partial sums are loaded ahead of
// their (ordered) additions so each thread keeps several loads in flight.
template <int EPI, bool DUAL, typename OutT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs a) {
  const int64_t total = a.M * a.N;
  const int64_t plane = a.M * a.ldp;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t row = idx / a.N;
    const int64_t col = idx - row * a.N;
    const float *p = a.partial + row * a.ldp + col;
    float g = 0.0f, u = 0.0f;
    for (int s0 = 0; s0 < a.ksplit; s0 += 8) {
      float vg[8], vu[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = s0 + q < a.ksplit;
        vg[q] = ok ? p[(s0 + q) * plane] : 0.0f;
        vu[q] = (DUAL && ok) ? p[(s0 + q) * plane + a.N] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (s0 + q < a.ksplit) {
          g += vg[q];
          if (DUAL) u += vu[q];
        }
      }
    }
    if constexpr (EPI == EPI_ROUTER) {
      const float z = g + (a.bias ? a.bias[col] : 0.0f);
      static_cast<float *>(a.out)[row * a.ldo + col] = z;
      if (a.out_t) a.out_t[col * a.M + row] = z;
    } else if constexpr (EPI == EPI_SITU) {
      const float f = a.row_scale ? a.row_scale[row] : 1.0f;
      store_out<OutT>(a.out, row * a.ldo + col,
                      f * situ(g, u, a.beta, a.inv_beta, a.beta_u, a.inv_beta_u));
      if (a.out_g != nullptr) {
        a.out_g[row * a.ldgu + col] = g;
        a.out_u[row * a.ldgu + col] = u;
      }
    } else {
      if (a.row_scale) g *= a.row_scale[row];
      if (a.resid) g += load_in<OutT>(a.resid, row * a.ldr + col);
      store_out<OutT>(a.out, row * a.ldo + col, g);
    }
  }
}

}  // namespace g2
}  // namespace moe
