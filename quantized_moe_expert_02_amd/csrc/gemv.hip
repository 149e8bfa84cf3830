// Decode path (small batches): the experts of the batch union as split-K
// GEMVs that stream the packed 4-bit weights once per unique expert.
//
// Weights are decoded in registers right before the dot products, never
// expanded to fp16 in memory -- the design the Ornith engine uses for its
// NVFP4 weights ("GTX 1070向け35BパラメータMoEモデル推論エンジン公開",
// 648news.com, section "VRAMとシステムメモリで重みを分割する設計") -- and each
// unique expert of the batch is read once and applied to all of its tokens
// (the batch-wise MoE union, "Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
// hakusoku.com, section 実装済み機能).
//
// Work split.  A unit is one wavefront: (expert slot, block of 64 output
// rows, K-segment).  Lane l owns output row 64*rb + l and streams that row's
// 32-column chunks as 128-bit loads (one contiguous KiB per wavefront per
// load).  Activations are wave-uniform, so they are read through the scalar
// cache.  Each unit writes fp32 partial sums; the last unit of a group (a
// device-scope atomic counter, fence-protected) reduces the partials in a
// fixed order, so results are deterministic and no float atomics are used.
//
//   k_gu_gemv:  gate and up rows together -> SwiGLU -> h (binary16)
//   k_dn_gemv:  down rows -> scaled partials -> routing-weighted combine of
//               the k slots plus the shared expert -> y (binary16)
#include "common.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
constexpr int kMaxSplit = 8;  // largest split-K factor of the GEMV kernels
// Global-address-space views, so weight loads compile to global_load (not
// flat_load, which also occupies the LDS/scalar wait counter).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 guint4;
typedef __attribute__((address_space(1))) const u32x2 guint2;

struct GemvArgs {
  const SlotEntry* slots;
  const int32_t* n_unique;
  const int32_t* uniq_ids;
  const int32_t* uniq_off;
  const int32_t* pairs;
  const float* topk_w;
  float* part;        // partials
  uint32_t* counters;
  uint16_t* h;        // [rows_total][I]
  uint16_t* y;        // [T][H]
  int T, H, I, k, S;
  int ks;             // K-segments per row block
  int cpu;            // 32-column chunks per unit
  int rows_total;
  int fmt;
  Layout L;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// The two nibble masks live in VGPRs so that each mask-and-insert below is a
// single v_and_or_b32 (a VOP3 instruction takes no literal on gfx9, and only
// one scalar operand).
struct Int4Masks {
  uint32_t lo, hi;
};

__device__ __forceinline__ Int4Masks int4_masks() {
  Int4Masks m;
  asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(m.lo));
  asm volatile("v_mov_b32 %0, 0x00F000F0" : "=v"(m.hi));
  return m;
}

// int4 (device order, offset binary) -> four half2 pairs of exact integers.
// (d & 0x000F000F) | 0x6400 gives 1024 + u; (d & 0x00F000F0) | 0x5400 gives
// 64 + u; subtracting 1032 / 72 leaves q = u - 8 exactly.
__device__ __forceinline__ void dec_int4(uint32_t d, const Int4Masks& mk, half2_t& p0, half2_t& p1, half2_t& p2,
                                         half2_t& p3) {
  const half2_t k1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t d8 = d >> 8;
  p0 = as_h2((d & mk.lo) | 0x64006400u) + k1032;
  p1 = as_h2((d & mk.hi) | 0x54005400u) + k72;
  p2 = as_h2((d8 & mk.lo) | 0x64006400u) + k1032;
  p3 = as_h2((d8 & mk.hi) | 0x54005400u) + k72;
}

// e2m1 codes (byte b = columns 2b, 2b+1) -> four half2 pairs, multiplied by
// the block scale (exact: e2m1 * e4m3 has at most 6 significant bits).
__device__ __forceinline__ void dec_e2m1(uint32_t d, half2_t s, half2_t& p0, half2_t& p1, half2_t& p2,
                                         half2_t& p3) {
  p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s;
  p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s;
  p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s;
  p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s;
}

__device__ __forceinline__ half2_t e4m3_pair(uint32_t bytes, int sel) {
  float f;
  switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_f32_fp8(bytes, 0); break;
    case 1: f = __builtin_amdgcn_cvt_f32_fp8(bytes, 1); break;
    case 2: f = __builtin_amdgcn_cvt_f32_fp8(bytes, 2); break;
    default: f = __builtin_amdgcn_cvt_f32_fp8(bytes, 3); break;
  }
  const _Float16 h = (_Float16)f;
  return half2_t{h, h};
}

__device__ __forceinline__ float dot8(half2_t p0, half2_t p1, half2_t p2, half2_t p3, uint4 xv, float acc) {
  acc = __builtin_amdgcn_fdot2(p0, as_h2(xv.x), acc, false);
  acc = __builtin_amdgcn_fdot2(p1, as_h2(xv.y), acc, false);
  acc = __builtin_amdgcn_fdot2(p2, as_h2(xv.z), acc, false);
  acc = __builtin_amdgcn_fdot2(p3, as_h2(xv.w), acc, false);
  return acc;
}

// Streams `nch` chunks for NM matrices (gate+up: NM=2) and NT activation rows.
//   w: this lane's 16 bytes in the first chunk of matrix 0; matrix m of
//      chunk c is at w + (c*NM + m)*64 (uint4 units).
//   sc: E2M1 only: this lane's 8 scale bytes of the first 4-chunk group of
//      matrix 0; matrix m of group g is at sc + (g*NM + m)*64 (uint2 units).
//   act[t]: wave-uniform activation rows, already offset to column 32*c0.
template <int FMT, int NM, int U>
__device__ __forceinline__ void load_batch(const guint4* __restrict__ w, const guint2* __restrict__ sc, int c,
                                           u32x4 (&wv)[U][NM], u32x2 (&sv)[NM]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < NM; ++m) wv[u][m] = __builtin_nontemporal_load(w + ((c + u) * NM + m) * 64);
  if (FMT == MOE_W_E2M1_B16) {
#pragma unroll
    for (int m = 0; m < NM; ++m) sv[m] = sc[((c / U) * NM + m) * 64];
  }
}

template <int FMT, int NM, int NT, int U>
__device__ __forceinline__ void compute_batch(const u32x4 (&wv)[U][NM], const u32x2 (&sv)[NM], int c,
                                              const uint4* const* act, const Int4Masks& mk, float (&acc)[NM][NT]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint4 xv[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[t][i] = act[t][(c + u) * 4 + i];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t dw[4] = {wv[u][m].x, wv[u][m].y, wv[u][m].z, wv[u][m].w};
      half2_t s0, s1;
      if (FMT == MOE_W_E2M1_B16) {
        const uint32_t sb = (u < 2) ? sv[m].x : sv[m].y;
        s0 = e4m3_pair(sb, (u & 1) * 2);
        s1 = e4m3_pair(sb, (u & 1) * 2 + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t p0, p1, p2, p3;
        if (FMT == MOE_W_INT4_ROW) dec_int4(dw[i], mk, p0, p1, p2, p3);
        else dec_e2m1(dw[i], i < 2 ? s0 : s1, p0, p1, p2, p3);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = dot8(p0, p1, p2, p3, xv[t][i], acc[m][t]);
      }
    }
  }
}

// Streams `nch` chunks (a multiple of 4) for NM matrices (gate+up: NM=2) and
// NT activation rows, keeping the next 4-chunk batch of weights in flight
// while the current one is decoded and multiplied.
//   w: this lane's 16 bytes in the first chunk of matrix 0; matrix m of
//      chunk c is at w + (c*NM + m)*64 (uint4 units).
//   sc: E2M1 only: this lane's 8 scale bytes of the first 4-chunk group of
//      matrix 0; matrix m of group g is at sc + (g*NM + m)*64 (uint2 units).
//   act[t]: wave-uniform activation rows, already offset to column 32*c0.
template <int FMT, int NM, int NT>
__device__ __forceinline__ void stream_chunks(const guint4* __restrict__ w, const guint2* __restrict__ sc,
                                              const uint4* const* act, int nch, float (&acc)[NM][NT]) {
  const Int4Masks mk = int4_masks();
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = 0.f;
  constexpr int U = 4;  // chunks per batch (one E2M1 scale group)
  u32x4 wa[U][NM], wb[U][NM];
  u32x2 sa[NM], sb[NM];
  load_batch<FMT, NM, U>(w, sc, 0, wa, sa);
  for (int c = 0; c < nch; c += 2 * U) {
    const bool has_b = c + U < nch;
    if (has_b) load_batch<FMT, NM, U>(w, sc, c + U, wb, sb);
    compute_batch<FMT, NM, NT, U>(wa, sa, c, act, mk, acc);
    if (!has_b) break;
    if (c + 2 * U < nch) load_batch<FMT, NM, U>(w, sc, c + 2 * U, wa, sa);
    compute_batch<FMT, NM, NT, U>(wb, sb, c + U, act, mk, acc);
  }
}

// Expert and token list of a slot, from the slot table the union step
// wrote: one 16-byte wave-uniform load.  Returns false for unused slots.
struct SlotInfo {
  const uint8_t* base;
  int n;            // tokens
  int p0;           // first entry in pairs (routed) or -1 (shared)
};

__device__ __forceinline__ bool resolve_slot(const GemvArgs& a, int slot, SlotInfo& si) {
  const SlotEntry e = a.slots[slot];
  si.base = e.base;
  si.n = e.n;
  si.p0 = e.p0;
  return si.n > 0;
}

// Token index and output row (pair id, or T*k + t for the shared expert) of
// the i-th token of a slot.
__device__ __forceinline__ void slot_token(const GemvArgs& a, const SlotInfo& si, int i, int& t, int& row) {
  if (si.p0 < 0) {
    t = i;
    row = a.T * a.k + i;
  } else {
    const int p = a.pairs[si.p0 + i];
    t = p / a.k;
    row = p;
  }
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Publishes this unit's partial stores and reports whether it is the last of
// `total` units of its group; the last one resets the counter for the next
// call.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total) {
  if (publish_arrival(counter) != total - 1) return false;
  if ((threadIdx.x & 63) == 0) st_dev(counter, 0u);
  return true;
}

template <int FMT, int NT>
__device__ void gu_tile(const GemvArgs& a, const SlotInfo& si, int rb, int c0, int ks, int i0,
                        const uint16_t* __restrict__ x) {
  const int lane = threadIdx.x & 63;
  const guint4* w = (const guint4*)(si.base + a.L.gu_off) + ((size_t)rb * (a.H / 32) + c0) * 2 * 64 + lane;
  const guint2* sc = nullptr;
  if (FMT == MOE_W_E2M1_B16)
    sc = (const guint2*)(si.base + a.L.sgu_off) + ((size_t)rb * (a.H / 128) + c0 / 4) * 2 * 64 + lane;
  const uint4* act[NT];
  int rows[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int tok, row;
    slot_token(a, si, i0 + t, tok, row);
    tok = __builtin_amdgcn_readfirstlane(tok);
    rows[t] = __builtin_amdgcn_readfirstlane(row);
    act[t] = reinterpret_cast<const uint4*>(x + (size_t)tok * a.H + 32 * c0);
  }
  float acc[2][NT];
  stream_chunks<FMT, 2, NT>(w, sc, act, a.cpu, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float* pr = a.part + (((size_t)ks * a.rows_total + rows[t]) * 2) * a.I + 64 * rb + lane;
    st_dev(pr, acc[0][t]);
    st_dev(pr + a.I, acc[1][t]);
  }
}

template <int FMT, int NT>
__device__ void dn_tile(const GemvArgs& a, const SlotInfo& si, int rb, int c0, int ks, int i0, float scale) {
  const int lane = threadIdx.x & 63;
  const guint4* w = (const guint4*)(si.base + a.L.d_off) + ((size_t)rb * (a.I / 32) + c0) * 64 + lane;
  const guint2* sc = nullptr;
  if (FMT == MOE_W_E2M1_B16)
    sc = (const guint2*)(si.base + a.L.sdd_off) + ((size_t)rb * (a.I / 128) + c0 / 4) * 64 + lane;
  const uint4* act[NT];
  int rows[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int tok, row;
    slot_token(a, si, i0 + t, tok, row);
    rows[t] = __builtin_amdgcn_readfirstlane(row);
    act[t] = reinterpret_cast<const uint4*>(a.h + (size_t)rows[t] * a.I + 32 * c0);
  }
  float acc[1][NT];
  stream_chunks<FMT, 1, NT>(w, sc, act, a.cpu, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t)
    st_dev(a.part + ((size_t)ks * a.rows_total + rows[t]) * a.H + 64 * rb + lane, acc[0][t] * scale);
}

// Grid: x = (I/64) * ks units of (row block, K-segment); y = expert slots.
// Block: one wavefront.
template <int FMT>
__global__ __launch_bounds__(64) void k_gu_gemv(GemvArgs a, const uint16_t* __restrict__ x) {
  SlotInfo si;
  const int slot = blockIdx.y;
  if (!resolve_slot(a, slot, si)) return;
  const int rb = blockIdx.x / a.ks, ks = blockIdx.x % a.ks;
  const int c0 = ks * a.cpu;
  const int lane = threadIdx.x & 63;
  for (int i0 = 0; i0 < si.n; i0 += 4) {
    switch (min(4, si.n - i0)) {
      case 1: gu_tile<FMT, 1>(a, si, rb, c0, ks, i0, x); break;
      case 2: gu_tile<FMT, 2>(a, si, rb, c0, ks, i0, x); break;
      case 3: gu_tile<FMT, 3>(a, si, rb, c0, ks, i0, x); break;
      default: gu_tile<FMT, 4>(a, si, rb, c0, ks, i0, x); break;
    }
  }
  if (!arrive_last(a.counters + (size_t)slot * (a.I / 64) + rb, a.ks)) return;
  // Last K-segment of this (slot, row block): reduce in segment order, apply
  // the row scales, SwiGLU, store h.
  const int r = 64 * rb + lane;
  float sg, su;
  if (FMT == MOE_W_INT4_ROW) {
    sg = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(si.base + a.L.sg_off)[r]);
    su = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(si.base + a.L.su_off)[r]);
  } else {
    const float* g3 = reinterpret_cast<const float*>(si.base + a.L.g3_off);
    sg = g3[0];
    su = g3[1];
  }
  for (int i = 0; i < si.n; ++i) {
    int tok, row;
    slot_token(a, si, i, tok, row);
    // issue every partial load before summing (they are independent)
    float pg[kMaxSplit], pu[kMaxSplit];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (s < a.ks) {
        const float* pr = a.part + (((size_t)s * a.rows_total + row) * 2) * a.I + r;
        pg[s] = ld_dev(pr);
        pu[s] = ld_dev(pr + a.I);
      }
    }
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (s < a.ks) {
        g += pg[s];
        u += pu[s];
      }
    }
    g *= sg;
    u *= su;
    const float hv = silu(g) * u;
    a.h[(size_t)row * a.I + r] = __builtin_bit_cast(uint16_t, (_Float16)hv);
  }
}

// Grid: x = (H/64) * ks, y = expert slots.  Block: one wavefront.
template <int FMT>
__global__ __launch_bounds__(64) void k_dn_gemv(GemvArgs a) {
  SlotInfo si;
  const int slot = blockIdx.y;
  if (!resolve_slot(a, slot, si)) return;
  const int rb = blockIdx.x / a.ks, ks = blockIdx.x % a.ks;
  const int c0 = ks * a.cpu;
  const int lane = threadIdx.x & 63;
  const int r = 64 * rb + lane;
  float scale;
  if (FMT == MOE_W_INT4_ROW)
    scale = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(si.base + a.L.sd_off)[r]);
  else
    scale = reinterpret_cast<const float*>(si.base + a.L.g3_off)[2];
  for (int i0 = 0; i0 < si.n; i0 += 4) {
    switch (min(4, si.n - i0)) {
      case 1: dn_tile<FMT, 1>(a, si, rb, c0, ks, i0, scale); break;
      case 2: dn_tile<FMT, 2>(a, si, rb, c0, ks, i0, scale); break;
      case 3: dn_tile<FMT, 3>(a, si, rb, c0, ks, i0, scale); break;
      default: dn_tile<FMT, 4>(a, si, rb, c0, ks, i0, scale); break;
    }
  }
  const uint32_t total = (uint32_t)a.ks * (uint32_t)(a.S + *a.n_unique);
  if (!arrive_last(a.counters + rb, total)) return;
  // Last unit of this row block: y[t] = sum_j w[t][j] * o_j + o_shared, in
  // slot order, each o summed over K-segments in order.
  for (int t = 0; t < a.T; ++t) {
    float acc = 0.f;
    for (int j0 = 0; j0 < a.k + a.S; j0 += 8) {
      // up to 8 slots' partials in flight at once, summed in slot order
      float o[8][kMaxSplit];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        const int row = (j < a.k) ? t * a.k + j : a.T * a.k + t;
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
          if (j < a.k + a.S && s < a.ks) o[jj][s] = ld_dev(a.part + ((size_t)s * a.rows_total + row) * a.H + r);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj;
        if (j >= a.k + a.S) break;
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
          if (s < a.ks) v += o[jj][s];
        acc += (j < a.k) ? a.topk_w[t * a.k + j] * v : v;
      }
    }
    a.y[(size_t)t * a.H + r] = __builtin_bit_cast(uint16_t, (_Float16)acc);
  }
}

}  // namespace

hipError_t launch_decode_experts(const moe_dims_t& d, const Plan& p, const moe_weights_t& w,
                                 const uint16_t* x, const Route& r, void* ws, uint16_t* y, hipStream_t s,
                                 const StageEvents& se) {
  GemvArgs a{};
  a.slots = r.slots;
  a.n_unique = r.n_unique;
  a.uniq_ids = r.uniq_ids;
  a.uniq_off = r.uniq_off;
  a.pairs = r.pairs;
  a.topk_w = r.topk_w;
  a.T = p.T;
  a.H = p.H;
  a.I = p.I;
  a.k = p.k;
  a.S = p.S;
  a.rows_total = p.rows_total;
  a.fmt = d.wfmt;
  a.L = layout_of(d);
  a.h = (uint16_t*)((char*)ws + p.h_off);
  a.y = y;
  // gate/up
  a.part = (float*)((char*)ws + p.p_gu_off);
  a.counters = (uint32_t*)ws + p.c_gu;
  a.ks = p.ks_gu;
  a.cpu = (p.H / 32) / p.ks_gu;
  dim3 g1((unsigned)((p.I / 64) * p.ks_gu), (unsigned)p.slots_max);
  se.record(1, s);
  if (d.wfmt == MOE_W_INT4_ROW) hipLaunchKernelGGL(k_gu_gemv<MOE_W_INT4_ROW>, g1, dim3(64), 0, s, a, x);
  else hipLaunchKernelGGL(k_gu_gemv<MOE_W_E2M1_B16>, g1, dim3(64), 0, s, a, x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // down + combine
  a.part = (float*)((char*)ws + p.p_dn_off);
  a.counters = (uint32_t*)ws + p.c_dn;
  a.ks = p.ks_dn;
  a.cpu = (p.I / 32) / p.ks_dn;
  dim3 g2((unsigned)((p.H / 64) * p.ks_dn), (unsigned)p.slots_max);
  se.record(2, s);
  if (d.wfmt == MOE_W_INT4_ROW) hipLaunchKernelGGL(k_dn_gemv<MOE_W_INT4_ROW>, g2, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(k_dn_gemv<MOE_W_E2M1_B16>, g2, dim3(64), 0, s, a);
  e = hipGetLastError();
  se.record(3, s);
  return e;
}

}  // namespace moe
