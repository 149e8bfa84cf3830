// Prefill path (large batches): the experts of the batch union as grouped
// GEMMs on the fp16 matrix cores.
//
// Each unique expert is applied to all of its tokens at once (the batch-wise
// MoE union, "Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com,
// section 実装済み機能); its weights are decoded in registers, straight into
// matrix-core operands, as exact binary16 values (int8/int4/int2 codes are
// small integers; e2m1 x e4m3 has at most 6 significant bits) -- the in-register
// decode of the Ornith engine ("GTX 1070向け35BパラメータMoEモデル推論エンジン公開",
// section "VRAMとシステムメモリで重みを分割する設計") -- and multiplied on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation.  Row scales (integer
// formats) or the tensor scale (e2m1) are applied in the epilogue, as is the
// SwiGLU.
//
//   k_expert_gemm<.., 2>:  tile = 64 tokens of one expert x 512 gate rows +
//                          512 up rows -> h (binary16, one row per pair)
//   k_expert_gemm<.., 1>:  tile = 64 tokens x 512 down rows -> per-pair fp32
//                          outputs, already multiplied by the routing weight
//   k_combine:  y[t] = sum over slots j (in slot order) + shared -> binary16
#include "common.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 guint4;

constexpr int BM = kPrefillTileRows;  // tokens per tile

// Per-format shape of one K-slice of the main loop: SC columns, WPS 16-byte
// pieces (chunks of the packed layout) per lane and matrix, SC / 32 MFMA
// K-steps; kDepth slices of weights in flight (a multiple of the activation
// ring's depth, 2).
template <int FMT>
struct Slice {
  static constexpr int SC = FMT == MOE_W_INT2_ROW ? 64 : 32;
  static constexpr int WPS = FMT == MOE_W_INT8_ROW ? 2 : 1;
  static constexpr int STEPS = SC / 32;
  static constexpr int XP = SC + 8;  // halves per LDS token row (8 pad)
  static constexpr int kDepth = WPS == 1 ? 6 : 2;
};

struct GemmArgs {
  const SlotEntry* slots;
  const int32_t* pairs;
  const int32_t* tiles;      // [tile] = (slot, m0) pairs
  const int32_t* n_tiles;    // [1]
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

// Field masks held in VGPRs, so that each mask-and-insert below is one
// v_and_or_b32 (a VOP3 instruction takes no literal on gfx9 and at most one
// scalar operand; the magic constant takes that slot).
struct DecMasks {
  uint32_t m[4];
};

__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

template <int FMT>
__device__ __forceinline__ DecMasks dec_masks() {
  DecMasks k{};
  if (FMT == MOE_W_INT4_ROW) {
    k.m[0] = in_vgpr(0x000F000Fu);
    k.m[1] = in_vgpr(0x00F000F0u);
  } else if (FMT == MOE_W_INT8_ROW) {
    k.m[0] = in_vgpr(0x00FF00FFu);
  } else if (FMT == MOE_W_INT2_ROW) {
#pragma unroll
    for (int j = 0; j < 4; ++j) k.m[j] = in_vgpr(0x00030003u << (2 * j));
  }
  return k;
}

// int4 (device order, offset binary) -> 8 consecutive binary16 values.
__device__ __forceinline__ half8_t dequant_int4(uint32_t d, const DecMasks& mk) {
  const half2_t k1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t d8 = d >> 8;
  const half2_t p0 = as_h2((d & mk.m[0]) | 0x64006400u) + k1032;
  const half2_t p1 = as_h2((d & mk.m[1]) | 0x54005400u) + k72;
  const half2_t p2 = as_h2((d8 & mk.m[0]) | 0x64006400u) + k1032;
  const half2_t p3 = as_h2((d8 & mk.m[1]) | 0x54005400u) + k72;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// int8 (bytes 0, 2 = columns 0, 1; bytes 1, 3 = columns 2, 3; offset
// binary) -> 4 consecutive binary16 values: 1024 + u - 1152 = q.
__device__ __forceinline__ void dequant_int8(uint32_t d, const DecMasks& mk, half2_t& p0, half2_t& p1) {
  const half2_t k1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  p0 = as_h2((d & mk.m[0]) | 0x64006400u) + k1152;
  p1 = as_h2(((d >> 8) & mk.m[0]) | 0x64006400u) + k1152;
}

// int2 (column 2j in bits 2j, column 2j+1 in bits 16+2j, offset binary) ->
// columns 8h .. 8h+7 of the dword's 16 as binary16: the field at bit 2j
// lands in the mantissa of 1024, 256, 64 or 16 (unit in the last place
// 2^-2j), and base + u - (base + 2) = q.
__device__ __forceinline__ half8_t dequant_int2(uint32_t d, int h, const DecMasks& mk) {
  const uint32_t e = h ? d >> 8 : d;
  const half2_t p0 = as_h2((e & mk.m[0]) | 0x64006400u) + half2_t{(_Float16)-1026.0f, (_Float16)-1026.0f};
  const half2_t p1 = as_h2((e & mk.m[1]) | 0x5C005C00u) + half2_t{(_Float16)-258.0f, (_Float16)-258.0f};
  const half2_t p2 = as_h2((e & mk.m[2]) | 0x54005400u) + half2_t{(_Float16)-66.0f, (_Float16)-66.0f};
  const half2_t p3 = as_h2((e & mk.m[3]) | 0x4C004C00u) + half2_t{(_Float16)-18.0f, (_Float16)-18.0f};
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

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

// One K-slice of a 64-row block in a wavefront -> the B operands of the
// v_mfma_f32_16x16x32_f16 steps, b[step][q] for the 16-row group q: lane
// 16g+n receives row 16q+n and eight columns that depend on the format (the
// A operands are read from LDS to match, see a_operand):
//   4-bit: one chunk, dword b = columns 8b..8b+7 -> lane group g takes
//     columns 8g..8g+7;
//   int8: two chunks, dword b = columns 4b..4b+3 of each -> lane group g
//     takes columns 4g..4g+3 and 16+4g..16+4g+3;
//   int2: one chunk of 64 columns, dword b = columns 16b..16b+15 -> lane
//     group g takes columns 16g+8s .. 16g+8s+7 in step s.
// E2M1: `sc` holds this lane's two block-scale bytes (columns 0-15, 16-31).
template <int FMT>
__device__ __forceinline__ void block_to_operands(const u32x4 (&w)[Slice<FMT>::WPS], uint32_t sc, const DecMasks& mk,
                                                  half8_t (&b)[Slice<FMT>::STEPS][4]) {
  uint32_t d0 = w[0].x, d1 = w[0].y, d2 = w[0].z, d3 = w[0].w;
  transpose4(d0, d1, d2, d3);
  const uint32_t d[4] = {d0, d1, d2, d3};
  if (FMT == MOE_W_INT4_ROW) {
#pragma unroll
    for (int q = 0; q < 4; ++q) b[0][q] = dequant_int4(d[q], mk);
  } else if (FMT == MOE_W_INT8_ROW) {
    uint32_t f0 = w[Slice<FMT>::WPS - 1].x, f1 = w[Slice<FMT>::WPS - 1].y, f2 = w[Slice<FMT>::WPS - 1].z,
             f3 = w[Slice<FMT>::WPS - 1].w;
    transpose4(f0, f1, f2, f3);
    const uint32_t f[4] = {f0, f1, f2, f3};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half2_t p0, p1, p2, p3;
      dequant_int8(d[q], mk, p0, p1);
      dequant_int8(f[q], mk, p2, p3);
      b[0][q] = half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  } else if (FMT == MOE_W_INT2_ROW) {
#pragma unroll
    for (int st = 0; st < Slice<FMT>::STEPS; ++st)
#pragma unroll
      for (int q = 0; q < 4; ++q) b[st][q] = dequant_int2(d[q], st, mk);
  } else {
    uint32_t t0 = sc & 0xFF, t1 = sc & 0xFF, t2 = (sc >> 8) & 0xFF, t3 = (sc >> 8) & 0xFF;
    transpose4(t0, t1, t2, t3);
    b[0][0] = dequant_e2m1(d[0], e4m3_half2(t0));
    b[0][1] = dequant_e2m1(d[1], e4m3_half2(t1));
    b[0][2] = dequant_e2m1(d[2], e4m3_half2(t2));
    b[0][3] = dequant_e2m1(d[3], e4m3_half2(t3));
  }
}

// A operand of MFMA step `st` for token row `r` of an LDS slice, matching
// block_to_operands' columns for lane group g.
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

// Grouped GEMM over one tile of BM tokens of one expert.  512 threads = 8
// wavefronts; wavefront w owns the 64-row block rb = 8*group + w of each
// of the NM matrices (gate and up for NM = 2, down for NM = 1) and all BM
// tokens.  Per 32-column slice: each wavefront streams its NM weight blocks
// (one 128-bit load per lane each) and decodes them into MFMA operands in
// registers; the tile's activation rows (gathered by token) pass through a
// double-buffered LDS slice shared by the eight wavefronts.
//   NM == 2: K = H, activations x, epilogue: row scales, SwiGLU -> h.
//   NM == 1: K = I, activations h, epilogue: row scale, routing weight -> part.
constexpr int kGemmWaves = 8;  // wavefronts per workgroup, 64 rows each

template <int FMT, int NM>
__global__ __launch_bounds__(64 * kGemmWaves) void k_expert_gemm(GemmArgs a, int nx) {
  typedef Slice<FMT> SL;
  constexpr int SC = SL::SC, WPS = SL::WPS, XP = SL::XP;
  __shared__ __attribute__((aligned(16))) _Float16 sx[2][BM][XP];
  __shared__ int s_act[BM], s_out[BM];
  __shared__ float s_w[BM];
  // XCD-aware order: workgroups are spread round-robin over the 8 XCDs, so
  // map block b to tile 8*(l/nx) + b%8 and row group l%nx with l = b/8: all
  // row groups of one token tile run on one XCD and share its L2 copy of the
  // tile's activations.
  const int bid = blockIdx.x, xcd = bid & 7, loc = bid >> 3;
  const int tile = 8 * (loc / nx) + xcd;
  const int ngrp = loc % nx;
  if (tile >= *a.n_tiles) return;
  const int slot = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const SlotEntry se = a.slots[slot];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = (NM == 2) ? a.H : a.I;
  const int R = (NM == 2) ? a.I : a.H;  // rows per matrix
  const int rb = ngrp * kGemmWaves + wave;
  const bool active = rb * 64 < R;
  if (tid < BM) {
    int ar = -1, orow = -1;
    const bool ok = tile_token(a, se, m0 + tid, ar, orow);
    s_act[tid] = ok ? (NM == 2 ? ar : orow) : -1;  // activation row (x row, or h row = output row of GU)
    s_out[tid] = ok ? orow : -1;
    s_w[tid] = ok ? (se.p0 < 0 ? 1.0f : a.topk_w[orow]) : 0.0f;
  }
  __syncthreads();
  const uint16_t* act = (NM == 2) ? a.x : a.h;
  const int nch = K / SC;  // slices
  // this thread's 16-byte share of an activation slice: token tid/(SC/8),
  // columns 8*(tid%(SC/8)) (threads past BM*SC/8 only compute)
  constexpr int XQ = SC / 8;
  const bool xload = tid < XQ * BM;
  const int xm = (tid / XQ) & (BM - 1), xq = tid % XQ;
  const int xrow = xload ? s_act[xm] : -1;
  const uint16_t* xsrc = act + (size_t)(xrow < 0 ? 0 : xrow) * K + 8 * xq;
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
  auto load_w = [&](int c, int m, int p) -> u32x4 {
    return __builtin_nontemporal_load(wsrc + ((size_t)(c * WPS + p) * NM + m) * 64);
  };
  auto load_s = [&](int c, int m) -> uint32_t {
    const uint8_t* p = ssrc + ((size_t)(c / 4) * NM + m) * 64 * 8 + 2 * (c & 3);
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
  };
  auto load_x = [&](int c) -> u32x4 {
    return xrow < 0 ? u32x4{0, 0, 0, 0} : *reinterpret_cast<const u32x4*>(xsrc + SC * c);
  };

  f32x4 acc[NM][4][4];  // [matrix][row group q][token group mt]
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[m][q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weights stream through a ring of kDepth register slices (loads issued
  // kDepth slices ahead); activations through a double-buffered LDS slice.
  constexpr int kDepth = SL::kDepth;
  u32x4 ring[kDepth][NM][WPS];
  uint32_t sring[kDepth][NM];
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      sring[j][m] = 0;
      if (active && j < nch) {
#pragma unroll
        for (int p = 0; p < WPS; ++p) ring[j][m][p] = load_w(j, m, p);
        if (FMT == MOE_W_E2M1_B16) sring[j][m] = load_s(j, m);
      }
    }
  // activation slices: register ring kXDepth deep feeding the LDS double buffer
  constexpr int kXDepth = 2;
  static_assert(kDepth % kXDepth == 0, "xring slot j % kXDepth must hold slice c + 1");
  u32x4 xring[kXDepth];
#pragma unroll
  for (int j = 0; j < kXDepth; ++j) xring[j] = (j + 1 < nch) ? load_x(j + 1) : u32x4{0, 0, 0, 0};
  if (xload) *reinterpret_cast<u32x4*>(&sx[0][xm][8 * xq]) = load_x(0);
  __syncthreads();
  const int n = lane & 15, g = lane >> 4;
  const DecMasks mk = dec_masks<FMT>();
  for (int c0 = 0; c0 < nch; c0 += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int c = c0 + j;
      if (c >= nch) break;
      // slice c+1 sits in xring[j % kXDepth]; refill it with slice c+1+kXDepth
      const u32x4 xn = xring[j % kXDepth];
      if (c + 1 + kXDepth < nch) xring[j % kXDepth] = load_x(c + 1 + kXDepth);
      if (active) {
        u32x4 wv[NM][WPS];
        uint32_t sv[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int p = 0; p < WPS; ++p) wv[m][p] = ring[j][m][p];
          sv[m] = sring[j][m];
          if (c + kDepth < nch) {
#pragma unroll
            for (int p = 0; p < WPS; ++p) ring[j][m][p] = load_w(c + kDepth, m, p);
            if (FMT == MOE_W_E2M1_B16) sring[j][m] = load_s(c + kDepth, m);
          }
        }
        half8_t av[SL::STEPS][4];
#pragma unroll
        for (int st = 0; st < SL::STEPS; ++st)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) av[st][mt] = a_operand<FMT>(&sx[c & 1][16 * mt + n][0], g, st);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          half8_t b[SL::STEPS][4];
          block_to_operands<FMT>(wv[m], sv[m], mk, b);
#pragma unroll
          for (int st = 0; st < SL::STEPS; ++st)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int mt = 0; mt < 4; ++mt)
                acc[m][q][mt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st][mt], b[st][q], acc[m][q][mt], 0, 0, 0);
        }
      }
      if (xload && c + 1 < nch) *reinterpret_cast<u32x4*>(&sx[(c + 1) & 1][xm][8 * xq]) = xn;
      __syncthreads();
    }
  }
  if (!active) return;
  // epilogue: lane (n, g) holds tokens 16 mt + 4 g + i of row 64 rb + 16 q + n
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = rb * 64 + 16 * q + n;
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
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mm = 16 * mt + 4 * g + i;
          const int orow = s_out[mm];
          if (orow < 0) continue;
          const float gv = acc[0][q][mt][i] * sgv, uv = acc[NM - 1][q][mt][i] * suv;
          a.h[(size_t)orow * a.I + row] = __builtin_bit_cast(uint16_t, (_Float16)(silu(gv) * uv));
        }
    } else {
      float sd;
      if (row_scaled(FMT))
        sd = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.sd_off)[row]);
      else
        sd = reinterpret_cast<const float*>(se.base + a.L.g3_off)[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mm = 16 * mt + 4 * g + i;
          const int orow = s_out[mm];
          if (orow < 0) continue;
          a.part[(size_t)orow * a.H + row] = s_w[mm] * (sd * acc[0][q][mt][i]);
        }
    }
  }
}

// y[t][c] = sum_j part[t*k + j][c] (slot order) + part[T*k + t][c].
__global__ __launch_bounds__(256) void k_combine(GemmArgs a) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.H) return;
  float acc = 0.f;
  for (int j = 0; j < a.k; ++j)
    if (a.topk_idx[t * a.k + j] >= 0) acc += a.part[((size_t)t * a.k + j) * a.H + c];  // < 0: dropped by top-p
  if (a.S) acc += a.part[((size_t)a.T * a.k + t) * a.H + c];
  a.y[(size_t)t * a.H + c] = __builtin_bit_cast(uint16_t, (_Float16)acc);
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
  const int rows_per_wg = 64 * kGemmWaves;
  const int nx_gu = (p.I + rows_per_wg - 1) / rows_per_wg, nx_dn = (p.H + rows_per_wg - 1) / rows_per_wg;
  const dim3 blk(64 * kGemmWaves);
  auto gemms = [&](auto gu, auto dn) {
    launch_k(gu, dim3(mt8 * nx_gu), blk, s, se.start(1), se.stop(1), a, nx_gu);
    launch_k(dn, dim3(mt8 * nx_dn), blk, s, se.start(2), nullptr, a, nx_dn);
  };
  switch (d.wfmt) {
    case MOE_W_INT4_ROW: gemms(k_expert_gemm<MOE_W_INT4_ROW, 2>, k_expert_gemm<MOE_W_INT4_ROW, 1>); break;
    case MOE_W_INT8_ROW: gemms(k_expert_gemm<MOE_W_INT8_ROW, 2>, k_expert_gemm<MOE_W_INT8_ROW, 1>); break;
    case MOE_W_INT2_ROW: gemms(k_expert_gemm<MOE_W_INT2_ROW, 2>, k_expert_gemm<MOE_W_INT2_ROW, 1>); break;
    default: gemms(k_expert_gemm<MOE_W_E2M1_B16, 2>, k_expert_gemm<MOE_W_E2M1_B16, 1>); break;
  }
  launch_k(k_combine, dim3((p.H + 255) / 256, p.T), dim3(256), s, nullptr, se.stop(2), a);
  return hipGetLastError();
}

}  // namespace moe
