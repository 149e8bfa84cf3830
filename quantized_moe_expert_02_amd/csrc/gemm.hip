// Prefill path (large batches): the experts of the batch union as grouped
// GEMMs on the fp16 matrix cores.
//
// Each unique expert is applied to all of its tokens at once (the batch-wise
// MoE union, "Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com,
// section 実装済み機能); its weights are decoded in registers, straight into
// matrix-core operands -- the in-register decode of the Ornith engine ("GTX
// 1070向け35BパラメータMoEモデル推論エンジン公開", section "VRAMとシステムメモリで
// 重みを分割する設計") -- and multiplied on v_mfma_f32_16x16x32_f16 with fp32
// accumulation:
//   integer codes u = q + OFF (offset binary) are masked into binary16
//     subnormals u * 2^(2j-24) (j = the field's bit position / 2 within its
//     half) with no arithmetic; the activations are divided by 2^(2j) when
//     they are staged, so every product is x * u * 2^-24, and the epilogue
//     forms sum x q = 2^24 acc - OFF * sum x from per-token activation sums
//     (the matrix cores keep subnormal inputs, checked on the hardware);
//   e2m1 codes times their e4m3 block scale are exact binary16 values (at
//     most 6 significant bits).
// Row scales (integer formats) or the tensor scale (e2m1) are applied in the
// epilogue, as is the SwiGLU.
//
//   k_expert_gemm<.., 2, ..>:  tile = 64 tokens of one expert x 512 gate rows
//                              + 512 up rows -> h (binary16, one row per pair)
//   k_expert_gemm<.., 1, ..>:  tile = 128 tokens (int2: 64) x 512 down rows
//                              -> per-pair fp32 outputs, times the routing
//                              weight
//   k_combine:  y[t] = sum over slots j (in slot order) + shared -> binary16
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 guint4;

// Per-format shape of one K-slice of the main loop: SC columns, WPS 16-byte
// chunks of the packed layout per lane, row block and matrix, SC / 32 MFMA
// K-steps.  Integer codes (offset binary, code = q + OFF) use the subnormal
// decode; E2M1 codes are converted and scaled.
template <int FMT>
struct Slice {
  static constexpr int SC = FMT == MOE_W_INT2_ROW ? 64 : 32;
  static constexpr int WPS = FMT == MOE_W_INT8_ROW ? 2 : 1;
  static constexpr int STEPS = SC / 32;
  static constexpr int XP = SC + 8;  // halves per LDS token row (8 pad)
  static constexpr bool SUB = FMT != MOE_W_E2M1_B16;
  static constexpr int OFF = FMT == MOE_W_INT8_ROW ? 128 : FMT == MOE_W_INT4_ROW ? 8 : 2;
};

struct GemmArgs {
  const SlotEntry* slots;
  const int32_t* pairs;
  const int32_t* tiles;      // gate/up tiles: [tile] = (slot, m0) pairs
  const int32_t* tiles_dn;   // down tiles
  const int32_t* n_tiles;    // [2]: gate/up tiles, down tiles
  const float* topk_w;
  const int32_t* topk_idx;
  const uint16_t* x;         // [T][H]
  uint16_t* h;               // [rows_total][I]
  float* part;               // [rows_total][H]
  uint16_t* y;               // [T][H]
  int T, H, I, k, S;
  int rows_total;
  Layout L;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// e2m1 codes (byte b = columns 2b, 2b+1) times a block scale -> 8 binary16.
__device__ __forceinline__ half8_t dequant_e2m1(uint32_t d, half2_t s) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ half2_t e4m3_half2(uint32_t byte) {
  const _Float16 h = (_Float16)__builtin_amdgcn_cvt_f32_fp8(byte, 0);
  return half2_t{h, h};
}

// 4x4 transpose across the lane groups {n, 16+n, 32+n, 48+n} and the four
// dwords: afterwards lane 16a+n dword b holds what lane 16b+n dword a held.
// Two v_permlane32_swap (exchange of the upper half's first operand with the
// lower half's second) then two v_permlane16_swap (odd rows' first operand
// with even rows' second).
__device__ __forceinline__ void transpose4(uint32_t& d0, uint32_t& d1, uint32_t& d2, uint32_t& d3) {
  auto r02 = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
  auto r13 = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
  d0 = r02[0];
  d2 = r02[1];
  d1 = r13[0];
  d3 = r13[1];
  auto r01 = __builtin_amdgcn_permlane16_swap(d0, d1, false, false);
  auto r23 = __builtin_amdgcn_permlane16_swap(d2, d3, false, false);
  d0 = r01[0];
  d1 = r01[1];
  d2 = r23[0];
  d3 = r23[1];
}

// An activation piece: PH consecutive binary16 values of one token row
// (PH = 8 or 16, starting at a multiple of PH), staged by one thread.
template <int PH>
struct Piece {
  uint32_t w[PH / 2];
};

// Binary16 factors that put the activations of a piece on the scale of the
// subnormal weight decode below: the column at position j of an 8-column
// group decodes to u * 2^-24 * class(j), so its activation is divided by
// class(j) (exactly, unless it becomes subnormal).  Pair k of a piece (PH
// halves, starting at a multiple of 8 for int2): int4 class 16 for odd k;
// int2 class 4^(k % 4).
template <int FMT, int PH>
__device__ __forceinline__ Piece<PH> prescale(Piece<PH> v) {
  auto mul = [](uint32_t p, float f) {
    return __builtin_bit_cast(uint32_t, as_h2(p) * half2_t{(_Float16)f, (_Float16)f});
  };
  if (FMT == MOE_W_INT4_ROW) {
#pragma unroll
    for (int k = 1; k < PH / 2; k += 2) v.w[k] = mul(v.w[k], 1.0f / 16);
  } else if (FMT == MOE_W_INT2_ROW) {
    static_assert(FMT != MOE_W_INT2_ROW || PH % 8 == 0, "int2 pieces are whole 8-column groups");
#pragma unroll
    for (int k = 0; k < PH / 2; ++k)
      if (k % 4) v.w[k] = mul(v.w[k], k % 4 == 1 ? 1.0f / 4 : k % 4 == 2 ? 1.0f / 16 : 1.0f / 64);
  }
  return v;
}

// Sum of the values of a piece, in fp32.
template <int PH>
__device__ __forceinline__ float piece_sum(Piece<PH> v) {
  const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < PH / 2; ++k) acc = __builtin_amdgcn_fdot2(as_h2(v.w[k]), one, acc, false);
  return acc;
}

// One K-slice of a 64-row block, rearranged for the MFMA B operands: after
// the transposes, lane 16g+n holds in d[q] (and f[q] for int8) the dword of
// row 16q+n that MFMA lane group g needs:
//   4-bit: one chunk, dword b = columns 8b..8b+7 -> group g takes columns
//     8g..8g+7;
//   int8: two chunks, dword b = columns 4b..4b+3 of each -> group g takes
//     columns 4g..4g+3 and 16+4g..16+4g+3;
//   int2: one chunk of 64 columns, dword b = columns 16b..16b+15 -> group g
//     takes columns 16g+8s .. 16g+8s+7 in step s.
// E2M1: s[q] holds the block-scale byte of those columns.
struct RawBlock {
  uint32_t d[4], f[4], s[4];
};

// A copy the compiler cannot fold: the transposes below work in place, and
// copying first ends the life of the loaded registers here, so that the next
// load can reuse them (otherwise the loop would copy every load result at its
// back edge, after waiting for it).
__device__ __forceinline__ uint32_t fresh(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

template <int FMT>
__device__ __forceinline__ RawBlock to_raw(const u32x4 (&w)[Slice<FMT>::WPS], uint32_t sc) {
  RawBlock r;
  r.d[0] = fresh(w[0].x), r.d[1] = fresh(w[0].y), r.d[2] = fresh(w[0].z), r.d[3] = fresh(w[0].w);
  transpose4(r.d[0], r.d[1], r.d[2], r.d[3]);
  if (FMT == MOE_W_INT8_ROW) {
    constexpr int P = Slice<FMT>::WPS - 1;
    r.f[0] = fresh(w[P].x), r.f[1] = fresh(w[P].y), r.f[2] = fresh(w[P].z), r.f[3] = fresh(w[P].w);
    transpose4(r.f[0], r.f[1], r.f[2], r.f[3]);
  }
  if (FMT == MOE_W_E2M1_B16) {
    r.s[0] = sc & 0xFF, r.s[1] = sc & 0xFF, r.s[2] = (sc >> 8) & 0xFF, r.s[3] = (sc >> 8) & 0xFF;
    transpose4(r.s[0], r.s[1], r.s[2], r.s[3]);
  }
  return r;
}

// B operand of MFMA step `st` for the 16-row group q.  Integer codes u
// (offset binary) become binary16 subnormals by masking alone: a field whose
// lowest bit sits at bit 2j of its half is u * 2^(2j-24) (the activation
// was divided by 2^(2j) to match, see prescale); the offset is removed in
// the epilogue.  E2M1: code times block scale, exactly (at most 6 significant
// bits).
template <int FMT>
__device__ __forceinline__ half8_t b_operand(const RawBlock& r, int q, int st) {
  if (FMT == MOE_W_INT4_ROW) {
    const uint32_t d = r.d[q], e = d >> 8;
    return __builtin_bit_cast(half8_t, u32x4{d & 0x000F000Fu, d & 0x00F000F0u, e & 0x000F000Fu, e & 0x00F000F0u});
  } else if (FMT == MOE_W_INT8_ROW) {
    const uint32_t d = r.d[q], f = r.f[q];
    return __builtin_bit_cast(half8_t,
                              u32x4{d & 0x00FF00FFu, (d >> 8) & 0x00FF00FFu, f & 0x00FF00FFu, (f >> 8) & 0x00FF00FFu});
  } else if (FMT == MOE_W_INT2_ROW) {
    const uint32_t e = st ? r.d[q] >> 8 : r.d[q];
    return __builtin_bit_cast(half8_t, u32x4{e & 0x00030003u, e & 0x000C000Cu, e & 0x00300030u, e & 0x00C000C0u});
  } else {
    return dequant_e2m1(r.d[q], e4m3_half2(r.s[q]));
  }
}

// A operand of MFMA step `st` for token row `r` of an LDS slice, matching
// b_operand's columns for lane group g.
template <int FMT>
__device__ __forceinline__ half8_t a_operand(const _Float16* row, int g, int st) {
  if (FMT == MOE_W_INT8_ROW) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    const half4_t lo = *reinterpret_cast<const half4_t*>(row + 4 * g);
    const half4_t hi = *reinterpret_cast<const half4_t*>(row + 16 + 4 * g);
    return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  if (FMT == MOE_W_INT2_ROW) return *reinterpret_cast<const half8_t*>(row + 16 * g + 8 * st);
  return *reinterpret_cast<const half8_t*>(row + 8 * g);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Token `m` of a tile: its activation row and its output row (pair id, or
// T*k + t for the shared expert).  Returns false past the slot's tokens.
__device__ __forceinline__ bool tile_token(const GemmArgs& a, const SlotEntry& se, int m, int& act_row, int& out_row) {
  if (m >= se.n) return false;
  if (se.p0 < 0) {
    act_row = m;
    out_row = a.T * a.k + m;
  } else {
    const int p = a.pairs[se.p0 + m];
    act_row = p / a.k;
    out_row = p;
  }
  return true;
}

// Grouped GEMM over the tokens of one expert.  512 threads = 8 wavefronts;
// wavefront w owns the 64-row block rb = 8*group + w of each of the NM
// matrices and all BT tokens of its tile:
//   NM == 2 (gate and up, K = H, activations x): BT = 64, one half of a
//     128-token tile; epilogue: row scales, SwiGLU -> h.
//   NM == 1 (down, K = I, activations h): BT = 128; epilogue: row scale,
//     routing weight -> part.
// (accumulators: NM x 64 rows x BT tokens = 128 per lane either way.)  Per
// K-slice: each wavefront streams its NM weight blocks (one 128-bit load per
// lane and chunk, DEPTH slices ahead) and decodes them into B operands just
// before their MFMAs; the tile's activation rows (gathered by token) pass
// through three LDS slices shared by the workgroup: slice c+2 is written and
// slice c+1's A operands are read while slice c is multiplied, one barrier
// per slice.  Integer formats accumulate sum x * u * 2^-24 over codes u = q +
// OFF; the epilogue forms sum x q = 2^24 acc - OFF * sum x from the tile's
// per-token activation sums.
constexpr int kGemmWaves = 8;

template <int FMT, int NM, int DEPTH, int BT, int NW>
__global__ __launch_bounds__(64 * NW) void k_expert_gemm(GemmArgs a, int nx) {
  typedef Slice<FMT> SL;
  // BT tokens per tile: kPrefillTileRows (64) or kDownTileRows (128); the
  // accumulators take NM x 64 rows x BT tokens per wavefront
  static_assert(BT == kPrefillTileRows || BT == kDownTileRows, "a tile height with a tile list");
  constexpr int GMAX = BT / 16;              // 16-token groups per tile
  constexpr int NT = 64 * NW;
  constexpr int SC = SL::SC, WPS = SL::WPS, XP = SL::XP, STEPS = SL::STEPS;
  constexpr int PH = SC * BT / NT;  // halves per thread and slice (every thread stages one piece)
  constexpr int PPR = SC / PH;      // pieces per token row of a slice
  static_assert(PH == 4 || PH == 8 || PH == 16, "activation piece of 8, 16 or 32 bytes");
  // activation slices wait XR slices in registers before they are staged
  // (one for 32-byte pieces, whose slices carry twice the matrix work)
  constexpr int XR = PH == 16 ? 1 : 2;
  static_assert(DEPTH % XR == 0, "the activation ring slot is c % XR");
  // the launcher picks DEPTH so that it divides the slice count K / SC
  typedef Piece<PH> P;
  __shared__ __attribute__((aligned(16))) _Float16 sx[3][BT][XP];
  __shared__ int s_act[BT], s_out[BT];
  __shared__ float s_w[BT], s_sum[BT];
  // XCD-aware order: workgroups are spread round-robin over the 8 XCDs, so
  // map block b to tile 8*(l/nx) + b%8 and row group l%nx with l = b/8: all
  // row groups of one token tile run on one XCD and share its L2 copy of the
  // tile's activations.
  const int32_t* tl = BT == kPrefillTileRows ? a.tiles : a.tiles_dn;
  const int bid = blockIdx.x, xcd = bid & 7, loc = bid >> 3;
  const int tile = 8 * (loc / nx) + xcd;
  const int ngrp = loc % nx;
  if (tile >= a.n_tiles[BT == kPrefillTileRows ? 0 : 1]) return;
  const int slot = tl[2 * tile], m0 = tl[2 * tile + 1];
  const SlotEntry se = a.slots[slot];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = (NM == 2) ? a.H : a.I;
  const int R = (NM == 2) ? a.I : a.H;  // rows per matrix
  // A tile with one filled 16-token group does little matrix work per
  // slice: each wavefront then takes two row blocks (rb, rb + 1), so a
  // slice moves twice the weights against the same activation staging and
  // barrier, and the tile needs half of its row groups (the others exit).
  // (the down GEMM only: the gate/up loop, with two matrices per block,
  // measured slower in pairs)
  const bool pair = NM == 1 && min(se.n - m0, BT) <= 16;
  if (pair && 2 * ngrp * NW * 64 >= R) return;  // uniform over the workgroup
  const int rb = pair ? 2 * (ngrp * NW + wave) : ngrp * NW + wave;
  const bool active = rb * 64 < R;
  const bool active1 = pair && (rb + 1) * 64 < R;  // the second block of a pair
  if (tid < BT) {
    int ar = -1, orow = -1;
    const bool ok = tile_token(a, se, m0 + tid, ar, orow);
    s_act[tid] = ok ? (NM == 2 ? ar : orow) : -1;  // activation row (x row, or h row = output row of GU)
    s_out[tid] = ok ? orow : -1;
    s_w[tid] = ok ? (se.p0 < 0 ? 1.0f : a.topk_w[orow]) : 0.0f;
  }
  __syncthreads();
  const uint16_t* act = (NM == 2) ? a.x : a.h;
  const int nch = K / SC;  // slices (at least 2: K >= 128)
  // this thread's activation piece: token xm, columns PH*xq .. +PH-1 of a slice
  const int xm = tid / PPR, xq = tid % PPR;
  const int xrow = s_act[xm];
  const bool xv = xrow >= 0;
  const P* xsrc = reinterpret_cast<const P*>(act + (size_t)(xv ? xrow : 0) * K + PH * xq);  // row 0 stands in for padding
  const int xoff = xm * XP + PH * xq;
  float xsum = 0.f;
  auto load_x = [&](int c) -> P { return xsrc[(size_t)c * PPR]; };
  auto stage = [&](P v, _Float16* buf, bool live) {
    if (!xv) v = P{};
    if (SL::SUB) {
      const float s = piece_sum<PH>(v);
      xsum += live ? s : 0.f;
      v = prescale<FMT, PH>(v);
    }
    *reinterpret_cast<P*>(buf + xoff) = v;
  };
  // weights: lane's 16 bytes of block (rb, chunk c) of matrix m; a slice is
  // WPS chunks, nch * WPS chunks per row
  const guint4* wsrc;
  const uint8_t* ssrc = nullptr;
  if (NM == 2) {
    wsrc = (const guint4*)(se.base + a.L.gu_off) + (size_t)rb * nch * WPS * 2 * 64 + lane;
    if (FMT == MOE_W_E2M1_B16) ssrc = se.base + a.L.sgu_off + ((size_t)rb * (K / 128) * 2 * 64 + lane) * 8;
  } else {
    wsrc = (const guint4*)(se.base + a.L.d_off) + (size_t)rb * nch * WPS * 64 + lane;
    if (FMT == MOE_W_E2M1_B16) ssrc = se.base + a.L.sdd_off + ((size_t)rb * (K / 128) * 64 + lane) * 8;
  }
  // the pair's second block (a block past the matrix re-reads the first; its
  // results are not stored)
  const size_t rb_step = active1 ? 1 : 0;
  const guint4* wsrc1 = wsrc + rb_step * nch * WPS * NM * 64;
  const uint8_t* ssrc1 = FMT == MOE_W_E2M1_B16 ? ssrc + rb_step * (K / 128) * NM * 64 * 8 : nullptr;
  auto load_w = [&](int c, int m, int p, int b) -> u32x4 {
    return __builtin_nontemporal_load((b ? wsrc1 : wsrc) + ((size_t)(c * WPS + p) * NM + m) * 64);
  };
  auto load_s = [&](int c, int m, int b) -> uint32_t {  // the two scale bytes of the slice, one 16-bit global load
    typedef __attribute__((address_space(1))) const uint16_t gu16;
    return *(gu16*)((b ? ssrc1 : ssrc) + ((size_t)(c / 4) * NM + m) * 64 * 8 + 2 * (c & 3));
  };

  f32x4 acc[NM][4][GMAX];  // [matrix][row group q][token group mt]
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mt = 0; mt < GMAX; ++mt) acc[m][q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ring[DEPTH][NM][WPS], ring1[DEPTH][NM][WPS];  // ring1: the pair's second block
  uint32_t sring[DEPTH][NM], sring1[DEPTH][NM];
  P xring[XR];
  half8_t av[GMAX], av1[GMAX];  // A operands of K-steps 0 and 1 (int2)
  const int n = lane & 15, g = lane >> 4;
  auto read_a = [&](half8_t (&dst)[GMAX], int buf, int st, auto MTC) {
#pragma unroll
    for (int mt = 0; mt < decltype(MTC)::value; ++mt) dst[mt] = a_operand<FMT>(&sx[buf][16 * mt + n][0], g, st);
  };
  // The loop body is straight-line code (loads past the last slice re-read
  // it and go unused), so that the load counters stay exact across slices.
  auto run = [&](auto ACTIVE, auto MTC, auto PAIRC) {
    constexpr int MT = decltype(MTC)::value;  // 16-token groups of the tile that hold tokens
    constexpr bool PR = decltype(PAIRC)::value;  // two row blocks (MT == 1; second in acc[.][.][1])
    static_assert(!PR || MT == 1, "pairs of row blocks for one-group tiles");
    // slice c+1's A operands are read during slice c, except where they
    // would not fit beside the accumulators (int2: two K-steps per slice;
    // more than 4 token groups)
    constexpr bool kPrefetchA = STEPS == 1 && MT <= 4;
    // prologue loads in the order of the loop's refills (activation slice
    // j+2, then weight slice j), so that the load counters the loop waits on
    // are the same on entry as in steady state
    const P v0 = load_x(0), v1 = load_x(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      if (j < XR) xring[j] = load_x(j + 2 < nch ? j + 2 : nch - 1);
      if (ACTIVE) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int cj = j < nch ? j : nch - 1;
#pragma unroll
          for (int p = 0; p < WPS; ++p) ring[j][m][p] = load_w(cj, m, p, 0);
          sring[j][m] = FMT == MOE_W_E2M1_B16 ? load_s(cj, m, 0) : 0u;
          if (PR) {
#pragma unroll
            for (int p = 0; p < WPS; ++p) ring1[j][m][p] = load_w(cj, m, p, 1);
            sring1[j][m] = FMT == MOE_W_E2M1_B16 ? load_s(cj, m, 1) : 0u;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    stage(v0, &sx[0][0][0], true);
    stage(v1, &sx[1][0][0], true);
    __syncthreads();
    if (kPrefetchA) read_a(av, 0, 0, MTC);
    int b1 = 1, b2 = 2;  // LDS slices of c+1 and c+2
    for (int c0 = 0; c0 < nch; c0 += DEPTH) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        const int c = c0 + j;
        // each ring slot is consumed (copied out) before it is refilled, so
        // that the refill lands in the same registers
        stage(xring[j % XR], &sx[b2][0][0], c + 2 < nch);
        __builtin_amdgcn_sched_barrier(0);
        xring[j % XR] = load_x(c + 2 + XR < nch ? c + 2 + XR : nch - 1);
        const int b0 = b1 == 0 ? 2 : b1 - 1;  // LDS slice of c
        half8_t avn[GMAX];
        if (kPrefetchA) {
          read_a(avn, b1, 0, MTC);
        } else {
          read_a(av, b0, 0, MTC);
          if (STEPS == 2) read_a(av1, b0, 1, MTC);
        }
        if (ACTIVE) {
          const int cn = c + DEPTH < nch ? c + DEPTH : nch - 1;
          // transpose every matrix (which ends the slot's registers), refill
          // the slot, then multiply
          RawBlock rw[NM], rw1[NM];
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            rw[m] = to_raw<FMT>(ring[j][m], sring[j][m]);
            if (PR) rw1[m] = to_raw<FMT>(ring1[j][m], sring1[j][m]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int p = 0; p < WPS; ++p) ring[j][m][p] = load_w(cn, m, p, 0);
            if (FMT == MOE_W_E2M1_B16) sring[j][m] = load_s(cn, m, 0);
            if (PR) {
#pragma unroll
              for (int p = 0; p < WPS; ++p) ring1[j][m][p] = load_w(cn, m, p, 1);
              if (FMT == MOE_W_E2M1_B16) sring1[j][m] = load_s(cn, m, 1);
            }
          }
          // the loads above issue before the matrix work below
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int st = 0; st < STEPS; ++st)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const half8_t b = b_operand<FMT>(rw[m], q, st);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                  acc[m][q][mt] =
                      __builtin_amdgcn_mfma_f32_16x16x32_f16(st ? av1[mt] : av[mt], b, acc[m][q][mt], 0, 0, 0);
                if (PR) {
                  const half8_t b1 = b_operand<FMT>(rw1[m], q, st);
                  acc[m][q][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(st ? av1[0] : av[0], b1, acc[m][q][1], 0, 0, 0);
                }
              }
          // the barrier below stays after the matrix work
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        if (kPrefetchA) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) av[mt] = avn[mt];
        }
        b1 = b2;
        b2 = b2 == 2 ? 0 : b2 + 1;
      }
    }
  };
  // the loop is specialised on the number of 16-token groups that hold
  // tokens (1-4, and 6 or 8 in 128-token tiles), so that a partly filled
  // tile skips the matrix work of its empty groups (their accumulators stay
  // zero; the epilogue skips padding tokens)
  typedef std::true_type on;
  typedef std::false_type off;
  const int ng = (min(se.n - m0, BT) + 15) >> 4;
  if (!active)
    run(off{}, std::integral_constant<int, 1>{}, off{});
  else if (NM == 1 && pair)
    run(on{}, std::integral_constant<int, 1>{}, std::integral_constant<bool, NM == 1>{});
  else if (ng <= 1)
    run(on{}, std::integral_constant<int, 1>{}, off{});
  else if (ng == 2)
    run(on{}, std::integral_constant<int, 2>{}, off{});
  else if (ng == 3)
    run(on{}, std::integral_constant<int, 3>{}, off{});
  else if (GMAX == 4 || ng == 4)
    run(on{}, std::integral_constant<int, 4>{}, off{});
  else if (ng <= 6)
    run(on{}, std::integral_constant<int, GMAX == 8 ? 6 : 4>{}, off{});
  else
    run(on{}, std::integral_constant<int, GMAX>{}, off{});
  if (SL::SUB) {  // per-token activation sums: the PPR pieces of a token sit in adjacent lanes
    float s = xsum;
#pragma unroll
    for (int o = 1; o < PPR; o <<= 1) s += __shfl_xor(s, o);
    if (xq == 0) s_sum[xm] = s;
    __syncthreads();
  }
  if (!active) return;
  // epilogue: lane (n, g) holds tokens 16 mt + 4 g + i of row 64 rb + 16 q + n
  // in acc[.][q][mt]; the second block of a pair holds its token group 0 in
  // acc[.][q][1]
  constexpr float kSub = 16777216.0f;  // 2^24
  const int gn = (min(se.n - m0, BT) + 15) >> 4;  // token groups that can hold tokens
  auto epilogue = [&](int rbx, auto ABC) {
    constexpr int AB = decltype(ABC)::value;     // accumulator index of token group 0
    constexpr int NG = AB ? 1 : GMAX;            // token groups held
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = rbx * 64 + 16 * q + n;
      if (NM == 2) {
        float sgv, suv;
        if (row_scaled(FMT)) {
          sgv = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.sg_off)[row]);
          suv = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.su_off)[row]);
        } else {
          const float* g3 = reinterpret_cast<const float*>(se.base + a.L.g3_off);
          sgv = g3[0];
          suv = g3[1];
        }
#pragma unroll
        for (int mt = 0; mt < NG; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int mm = 16 * mt + 4 * g + i;
            if (mt >= gn) continue;
            const int orow = s_out[mm];
            if (orow < 0) continue;
            float ga = acc[0][q][AB + mt][i], ua = acc[NM - 1][q][AB + mt][i];
            if (SL::SUB) {
              const float off = SL::OFF * s_sum[mm];
              ga = ga * kSub - off;
              ua = ua * kSub - off;
            }
            const float gv = ga * sgv, uv = ua * suv;
            a.h[(size_t)orow * a.I + row] = __builtin_bit_cast(uint16_t, (_Float16)(silu(gv) * uv));
          }
      } else {
        float sd;
        if (row_scaled(FMT))
          sd = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.sd_off)[row]);
        else
          sd = reinterpret_cast<const float*>(se.base + a.L.g3_off)[2];
#pragma unroll
        for (int mt = 0; mt < NG; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int mm = 16 * mt + 4 * g + i;
            if (mt >= gn) continue;
            const int orow = s_out[mm];
            if (orow < 0) continue;
            float da = acc[0][q][AB + mt][i];
            if (SL::SUB) da = da * kSub - SL::OFF * s_sum[mm];
            // streamed out (non-temporal): read once, by the combine
            __builtin_nontemporal_store(s_w[mm] * (sd * da), a.part + (size_t)orow * a.H + row);
          }
      }
    }
  };
  epilogue(rb, std::integral_constant<int, 0>{});
  if (active1) epilogue(rb + 1, std::integral_constant<int, 1>{});
}

// y[t][c] = sum_j part[t*k + j][c] (slot order) + part[T*k + t][c].  A
// thread owns 2 columns (measured faster than 1 or 4); a token's slot rows
// and its shared row are requested before they are added (a slot dropped by
// top-p has topk_idx < 0: its row is read but not added).
__global__ __launch_bounds__(256) void k_combine(GemmArgs a) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 2;
  if (c >= a.H) return;
  uint32_t keep = 0;  // slots kept (k <= 32)
  for (int j = 0; j < a.k; ++j) keep |= (uint32_t)(a.topk_idx[t * a.k + j] >= 0) << j;
  const size_t row = a.H / 2;  // float2 per partial row
  const float2* pt = reinterpret_cast<const float2*>(a.part + (size_t)t * a.k * a.H + c);
  const float2 sh = a.S ? reinterpret_cast<const float2*>(a.part + ((size_t)a.T * a.k + t) * a.H + c)[0] : float2{0.f, 0.f};
  float2 acc = {0.f, 0.f};
  for (int j0 = 0; j0 < a.k; j0 += 8) {
    float2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      typedef float f2v __attribute__((ext_vector_type(2)));
      const f2v u = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(pt + (size_t)min(j0 + i, a.k - 1) * row));
      v[i] = float2{u.x, u.y};
    }
    __builtin_amdgcn_sched_barrier(0);  // all eight loads in flight before the first add
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool use = j0 + i < a.k && ((keep >> (j0 + i)) & 1u);
      const float2 s = acc + v[i];
      acc = use ? s : acc;
    }
  }
  acc += sh;
  *reinterpret_cast<uint32_t*>(a.y + (size_t)t * a.H + c) = __builtin_bit_cast(uint32_t, half2_t{(_Float16)acc.x, (_Float16)acc.y});
}

}  // namespace

hipError_t launch_prefill_experts(const moe_dims_t& d, const Plan& p, const moe_weights_t& w,
                                  const uint16_t* x, const Route& r, void* ws, uint16_t* y, hipStream_t s,
                                  const StageEvents& se) {
  (void)w;
  GemmArgs a{};
  a.slots = r.slots;
  a.pairs = r.pairs;
  a.tiles = r.tiles;
  a.tiles_dn = r.tiles_dn;
  a.n_tiles = r.n_tiles;
  a.topk_w = r.topk_w;
  a.topk_idx = r.topk_idx;
  a.x = x;
  a.h = (uint16_t*)((char*)ws + p.h_off);
  a.part = (float*)((char*)ws + p.p_dn_off);
  a.y = y;
  a.T = p.T;
  a.H = p.H;
  a.I = p.I;
  a.k = p.k;
  a.S = p.S;
  a.rows_total = p.rows_total;
  a.L = layout_of(d);
  const int mt8 = (prefill_max_tiles(p.T, p.k, p.E, p.S) + 7) / 8 * 8;
  const int mt8_dn = (prefill_max_tiles(p.T, p.k, p.E, p.S, kDownTileRows) + 7) / 8 * 8;
  // one launch of kernel k over the tile list of BT-token tiles, NW
  // wavefronts (64 rows each) per workgroup, R rows per matrix
  auto gemm = [&](auto k, int BT, int NW, int R, hipEvent_t start, hipEvent_t stop) {
    const int nx = (R + 64 * NW - 1) / (64 * NW);
    launch_k(k, dim3((BT == kDownTileRows ? mt8_dn : mt8) * nx), dim3(64 * NW), s, start, stop, a, nx);
  };
  auto gemms = [&](auto gu, auto dn, int dn_rows, int dn_waves) {
    gemm(gu, kPrefillTileRows, kGemmWaves, p.I, se.start(1), se.stop(1));
    gemm(dn, dn_rows, dn_waves, p.H, se.start(2), nullptr);
  };
  // Ring depth (K-slices of weights in flight per wavefront): 4 slices for
  // the int4 gate/up, 2 for the others (deeper rings spill beside the 128
  // accumulators).  Down tiles hold 128 tokens, except int2 (64: its
  // 32-byte activation pieces leave no registers for 128).
  constexpr int G = kPrefillTileRows, D = kDownTileRows, W = kGemmWaves;
  switch (d.wfmt) {
    case MOE_W_INT4_ROW: gemms(k_expert_gemm<MOE_W_INT4_ROW, 2, 4, G, W>, k_expert_gemm<MOE_W_INT4_ROW, 1, 2, D, W>, D, W); break;
    case MOE_W_INT8_ROW: gemms(k_expert_gemm<MOE_W_INT8_ROW, 2, 2, G, W>, k_expert_gemm<MOE_W_INT8_ROW, 1, 2, D, W>, D, W); break;
    case MOE_W_INT2_ROW: gemms(k_expert_gemm<MOE_W_INT2_ROW, 2, 2, G, W>, k_expert_gemm<MOE_W_INT2_ROW, 1, 2, G, W>, G, W); break;
    default: gemms(k_expert_gemm<MOE_W_E2M1_B16, 2, 2, G, W>, k_expert_gemm<MOE_W_E2M1_B16, 1, 2, D, W>, D, W); break;
  }
  launch_k(k_combine, dim3((p.H / 2 + 255) / 256, p.T), dim3(256), s, nullptr, se.stop(2), a);
  return hipGetLastError();
}

}  // namespace moe
