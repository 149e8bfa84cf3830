// Decode path (small batches): the experts of the batch union as split-K
// GEMVs that stream the packed weights (4-, 8- or 2-bit codes) once per
// unique expert.
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
// 16-byte chunks as 128-bit loads (one contiguous KiB per wavefront per
// load).  Activations are wave-uniform: x is read through the scalar cache,
// h through LDS.  Partial sums are reduced in a fixed order (LDS within a
// workgroup, device-scope arrival counters across workgroups), so results
// are deterministic and no float atomics are used.  The three launches are
// described below, before the kernels.
#include <utility>

#include "wave.h"

namespace moe {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
constexpr int kMaxSplit = 8;  // largest split-K factor of the down projection
// Global-address-space views, so weight loads compile to global_load (not
// flat_load, which also occupies the LDS/scalar wait counter).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 guint4;
typedef __attribute__((address_space(1))) const u32x2 guint2;
typedef __attribute__((address_space(4))) const u32x4 cu32x4;
typedef __attribute__((address_space(3))) const u32x4 lu32x4;


__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Per-format constants of the packed layout (common.h): C columns per
// 1 KiB chunk, XPC activation vectors (8 binary16 each) per chunk, U chunks
// per ring batch (128 columns for int2, else 4 chunks; an E2M1 scale group
// is 4 chunks).  NCLS accumulator classes and the code offset OFF of the
// integer decode below.
template <int FMT>
struct Fmt {
  static constexpr int C = 128 / code_bits(FMT);
  static constexpr int XPC = C / 8;
  static constexpr int U = FMT == MOE_W_INT2_ROW ? 2 : 4;
  static constexpr int NCLS = FMT == MOE_W_INT2_ROW ? 4 : FMT == MOE_W_INT4_ROW ? 2 : 1;
  static constexpr float OFF = FMT == MOE_W_INT2_ROW ? 2.f : FMT == MOE_W_INT4_ROW ? 8.f : 128.f;
};

// Integer codes are decoded without any arithmetic: masking a dword leaves
// the offset-binary code u of two adjacent columns in the low mantissa bits
// of a half2, i.e. the binary16 subnormals u * 2^-24 * 2^b for a field at bit
// b of the 16-bit half (exact while the field stays below bit 10).  The dot
// products accumulate these per bit position b (a "class"), each class is
// scaled back by 2^24 / 2^b (exact), and the offset is removed once per
// K-segment as OFF * sum(x), which the callers compute alongside:
// sum (u - OFF) x = sum u x - OFF sum x.
//   INT4_ROW: fields at bits 0 and 4 of d and of d >> 8 (classes 2^0, 2^4);
//   INT8_ROW: bytes 0/2 of d and of d >> 8 (one class);
//   INT2_ROW: fields at bits 0, 2, 4, 6 of d and of d >> 8 (classes 4^j).
template <int FMT>
__device__ __forceinline__ constexpr float class_scale(int j) {
  return FMT == MOE_W_INT2_ROW ? 16777216.0f / (float)(1 << (2 * j))
         : FMT == MOE_W_INT4_ROW ? 16777216.0f / (float)(1 << (4 * j))
         : FMT == MOE_W_INT8_ROW ? 16777216.0f : 1.0f;
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

__device__ __forceinline__ float dot8(half2_t p0, half2_t p1, half2_t p2, half2_t p3, u32x4 xv, float acc) {
  acc = __builtin_amdgcn_fdot2(p0, as_h2(xv.x), acc, false);
  acc = __builtin_amdgcn_fdot2(p1, as_h2(xv.y), acc, false);
  acc = __builtin_amdgcn_fdot2(p2, as_h2(xv.z), acc, false);
  acc = __builtin_amdgcn_fdot2(p3, as_h2(xv.w), acc, false);
  return acc;
}

// Requests chunks c .. c+U-1 of NM matrices (and, for E2M1, their scale
// group) with non-temporal loads: the weights are read once per call.
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

__device__ __forceinline__ float fdot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2(as_h2(w), as_h2(x), acc, false);
}

// acc + the sum of the eight binary16 values in v.
__device__ __forceinline__ float sum8(u32x4 v, float acc) {
  constexpr uint32_t kOnes = 0x3C003C00u;  // (1.0, 1.0)
  acc = fdot2(v.x, kOnes, acc);
  acc = fdot2(v.y, kOnes, acc);
  acc = fdot2(v.z, kOnes, acc);
  return fdot2(v.w, kOnes, acc);
}

// Dword i of a chunk of matrix m against the chunk's activations xv, into
// the class accumulators cl[m][t][class].
template <int FMT, int NM, int NT, int XPC, int NCLS>
__device__ __forceinline__ void dot_dword(uint32_t d, int i, int m, half2_t s, const u32x4 (&xv)[NT][XPC],
                                          float (&cl)[NM][NT][NCLS]) {
  const uint32_t d8 = d >> 8;
  if constexpr (FMT == MOE_W_INT8_ROW) {  // columns 4i .. 4i+3
    const uint32_t e0 = d & 0x00FF00FFu, e1 = d8 & 0x00FF00FFu;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 v = xv[t][i / 2];
      cl[m][t][0] = fdot2(e0, (i & 1) ? v.z : v.x, cl[m][t][0]);
      cl[m][t][0] = fdot2(e1, (i & 1) ? v.w : v.y, cl[m][t][0]);
    }
  } else if constexpr (FMT == MOE_W_INT2_ROW) {  // columns 16i .. 16i+15: pair j of d, pair 4+j of d >> 8
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = d & (0x00030003u << (2 * j));
      e[4 + j] = d8 & (0x00030003u << (2 * j));
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 a = xv[t][2 * i], b = xv[t][2 * i + 1];
      const uint32_t xa[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) cl[m][t][j & 3] = fdot2(e[j], xa[j], cl[m][t][j & 3]);
    }
  } else if constexpr (FMT == MOE_W_INT4_ROW) {  // columns 8i .. 8i+7
    const uint32_t e0 = d & 0x000F000Fu, e1 = d & 0x00F000F0u, e2 = d8 & 0x000F000Fu, e3 = d8 & 0x00F000F0u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 v = xv[t][i];
      cl[m][t][0] = fdot2(e0, v.x, cl[m][t][0]);
      cl[m][t][1] = fdot2(e1, v.y, cl[m][t][1]);
      cl[m][t][0] = fdot2(e2, v.z, cl[m][t][0]);
      cl[m][t][1] = fdot2(e3, v.w, cl[m][t][1]);
    }
  } else {  // E2M1: columns 8i .. 8i+7, block scale s
    half2_t p0, p1, p2, p3;
    dec_e2m1(d, s, p0, p1, p2, p3);
#pragma unroll
    for (int t = 0; t < NT; ++t) cl[m][t][0] = dot8(p0, p1, p2, p3, xv[t][i], cl[m][t][0]);
  }
}

template <int FMT, int NM, int NT, int U, typename AP>
__device__ __forceinline__ void compute_batch(const u32x4 (&wv)[U][NM], const u32x2 (&sv)[NM], int c,
                                              const AP* act, float (&cl)[NM][NT][Fmt<FMT>::NCLS]) {
  constexpr int XPC = Fmt<FMT>::XPC;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // keep each chunk's activation loads next to their use: hoisting them
    // over the whole batch needs U*XPC*4*NT registers at once
    __builtin_amdgcn_sched_barrier(0);
    u32x4 xv[NT][XPC];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < XPC; ++i) xv[t][i] = act[t][(c + u) * XPC + i];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t dw[4] = {wv[u][m].x, wv[u][m].y, wv[u][m].z, wv[u][m].w};
      half2_t s0{}, s1{};
      if (FMT == MOE_W_E2M1_B16) {
        const uint32_t sb = (u < 2) ? sv[m].x : sv[m].y;
        s0 = e4m3_pair(sb, (u & 1) * 2);
        s1 = e4m3_pair(sb, (u & 1) * 2 + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) dot_dword<FMT, NM, NT, XPC>(dw[i], i, m, i < 2 ? s0 : s1, xv, cl);
    }
  }
}

// Streams `nch` chunks (a multiple of U) for NM matrices (gate+up: NM=2) and
// NT activation rows and adds sum_c u[c] * x[c] to acc (integer formats: u
// is the code before its offset is removed), through a ring of D batches of
// U chunks: the first D batches are requested at once, then `pre()` runs (a
// caller's own loads, overlapping the weights in flight), and every batch is
// reloaded with the batch D ahead right after it has been decoded and
// multiplied.
//   w: this lane's 16 bytes in the first chunk of matrix 0; matrix m of
//      chunk c is at w + (c*NM + m)*64 (uint4 units).
//   sc: E2M1 only: this lane's 8 scale bytes of the first 4-chunk group of
//      matrix 0; matrix m of group g is at sc + (g*NM + m)*64 (uint2 units).
//   act[t]: wave-uniform activation rows, already offset to the first
//      chunk's columns.  Rows that stay unchanged for the whole launch are
//      passed as constant-address-space pointers, which makes their loads
//      scalar.
template <int FMT, int NM, int NT, int D, typename AP, typename Pre>
__device__ __forceinline__ void stream_ring(const guint4* __restrict__ w, const guint2* __restrict__ sc,
                                            const AP* act, int nch, float (&acc)[NM][NT], Pre&& pre) {
  constexpr int U = Fmt<FMT>::U, NCLS = Fmt<FMT>::NCLS;
  u32x4 wv[D][U][NM];
  u32x2 sv[D][NM];
  float cl[NM][NT][NCLS];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NCLS; ++j) cl[m][t][j] = 0.f;
  const int nb = nch / U;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nb) load_batch<FMT, NM, U>(w, sc, d * U, wv[d], sv[d]);
  pre();
  for (int b0 = 0; b0 < nb; b0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int b = b0 + d;
      if (b < nb) {
        compute_batch<FMT, NM, NT, U>(wv[d], sv[d], b * U, act, cl);
        if (b + D < nb) load_batch<FMT, NM, U>(w, sc, (b + D) * U, wv[d], sv[d]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NCLS; ++j) acc[m][t] += cl[m][t][j] * class_scale<FMT>(j);
}

// ===========================================================================
// Decode path: three launches per layer.  Workgroups are four wavefronts
// (fewer workgroups to dispatch per launch).
//   k_route_phase  router workgroups: four independent router units each
//                  (fp64 partial logits of one expert over one column
//                  segment, for all tokens); the last router unit to finish
//                  takes every token's top-k and forms the batch union and
//                  slot table.  Shared-expert workgroups: gate/up of one
//                  64-row block over four K-segments, which need no routing.
//   k_gu_phase     one workgroup per (routed slot, 64-row block): its
//                  wavefronts stream the K-segments, reduce through LDS in a
//                  fixed order and form h (row scales, SwiGLU)
//   k_dn_phase     one workgroup per (slot, 64-row output block): K-segments
//                  reduced through LDS into the slot's scaled row, which is
//                  added, routing-weighted, to the token's output row as an
//                  exact fixed-point sum; the slot that completes a row
//                  writes it to y
// "Last" is decided by device-scope arrival counters, which that unit
// returns to zero, so every call starts from zeroed counters.  Data handed
// to another workgroup of the same launch is written with device-coherent
// stores and read with device-coherent loads after the arrival that
// publishes it (common.h); the launch boundaries order the phases, so no
// unit ever waits for another.
// ===========================================================================

constexpr int kWpg = 4;           // wavefronts per workgroup
constexpr int kStageCols = 1024;  // h columns staged in LDS per step
constexpr int kStageVec = kStageCols / 8;  // ... as 16-byte vectors per token
constexpr int kRingChunks = 8;    // chunks in flight per matrix (gate/up: 16 KiB, down: 8 KiB)
constexpr int kSumPieces = 4;     // 16-byte activation pieces per lane held for the offset sum
constexpr int kSyRouter = 64;     // router arrival counters (uint32 index in the sync region):
constexpr int kRouterGroups = 8;  //   top counter, then one per group of router workgroups

struct DecArgs {
  const float* Wr;
  const float* rbias;
  const uint16_t* x;
  const void* const* experts;
  const void* shared;
  int T, H, I, E, k, S;
  float top_p;
  int top_p_on;       // 0 < top_p < 1: slots may be dropped
  Layout L;
  uint16_t* y;
  int32_t* topk_idx;
  float* topk_w;
  double* z;
  int32_t* n_unique;
  int32_t* uniq_ids;
  int32_t* uniq_off;
  int32_t* pairs;
  SlotEntry* slots;
  uint16_t* h;
  float* p_gu;        // one partial plane per group of K-segments (shared and routed rows)
  uint64_t* y_acc;    // [T][H] output accumulators (fixed point + arrivals), zero between calls
  uint32_t* sync;
  uint32_t* gu_cnt;   // [slot][I/64] arrivals of K-segment groups
  int ks_gu, ks_sgu, ks_dn;     // K-segments: routed gate/up, shared gate/up, down
  int cpu_gu, cpu_sgu, cpu_dn;  // chunks per K-segment
  int slots_max, rows_total;
  int rsplit, seg4;   // router units per expert, 16-byte columns per router unit
  int n_router;       // E * rsplit
  int n_router_wg;    // workgroups of router units
  int with_slots;     // forward: also write the slot table (moe_route: no)
  int gu_routes;      // one token: the routed gate/up workgroups take the top-k
                      // themselves (the routing launch ends with its router units)
  int n_sgu_in_gu;    // shared gate/up workgroups placed in the routed gate/up launch
};

struct SlotInfo {
  const uint8_t* base;
  int n;     // tokens
  int p0;    // first entry in pairs (routed) or -1 (shared)
  int pair;  // >= 0: the pair of a one-token slot, known without the pairs table
};

// Tables that an earlier launch wrote (slot table, pairs) are read with
// scalar loads through constant-address-space pointers: they wait on the
// scalar memory counter, so a lookup issued after the weight loads does not
// wait for those (vector loads complete in order).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Slot s of the call: the shared expert needs no routing; routed slots come
// from the table the route phase wrote.  Returns false for unused slots.
__device__ __forceinline__ bool get_slot(const DecArgs& a, int s, SlotInfo& si) {
  if (a.S && s == 0) {
    si.base = (const uint8_t*)a.shared;
    si.n = a.T;
    si.p0 = -1;
    si.pair = -1;
    return true;
  }
  static_assert(sizeof(SlotEntry) == 16, "slot entry is one 16-byte scalar load");
  const u32x4 e = ld_const(reinterpret_cast<const u32x4*>(a.slots), s);
  si.base = reinterpret_cast<const uint8_t*>((uint64_t)e.x | ((uint64_t)e.y << 32));
  si.n = (int)e.z;
  si.p0 = (int)e.w;
  si.pair = -1;
  return si.n > 0;
}

// Token index and output row (pair id, or T*k + t for the shared expert)
// of the i-th token of a slot.
__device__ __forceinline__ void slot_token(const DecArgs& a, const SlotInfo& si, int i, int& t, int& row) {
  if (si.pair >= 0) {
    t = si.pair / a.k;
    row = si.pair;
  } else if (si.p0 < 0) {
    t = i;
    row = a.T * a.k + i;
  } else {
    const int p = ld_const(a.pairs, si.p0 + i);
    t = p / a.k;
    row = p;
  }
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Arrival on a counter shared by `total` units: true for the last one, which
// also returns the counter to zero.  Called by one whole wavefront.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total) {
  if (publish_arrival(counter) != total - 1) return false;
  if ((threadIdx.x & 63) == 0) st_dev(counter, 0u);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // no load moves above the arrival
  return true;
}

// Orders one wavefront's LDS accesses at this point (the other wavefronts of
// the workgroup run independent units, so no workgroup barrier is used).
// A wavefront's LDS operations complete in issue order; this keeps the
// compiler from moving them across.
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- batch union ----------------------------------------------------------
// Unique experts in ascending order, their pair lists (pairs of one expert
// in token order) and the slot table, from per-expert token bitmasks in LDS:
// the rank of pair (t, j) within its expert is the number of earlier tokens
// that chose the same expert.  pe[] holds the expert of every pair.  Run by
// one wavefront.
struct UnionLds {
  uint32_t mask[kMaxExperts];  // tokens per expert (bit t)
  int base[kMaxExperts];       // first pair of each expert
  int pe[kDecodeMaxTokens * kMaxTopK];
  const uint8_t* ep[kMaxExperts];  // packed expert pointers, staged by the caller
  RankSlots<1> rank[kWpg];         // top-k scratch of each wavefront
};

// Lane l owns experts [l*per, l*per + per).
constexpr int kMaxPer = kMaxExperts / 64;
__device__ __forceinline__ void union_step(const DecArgs& a, UnionLds& ls) {
  const int lane = threadIdx.x & 63;
  const int P = a.T * a.k;
  const int per = (a.E + 63) / 64;
  const int e0 = lane * per, e1 = min(a.E, e0 + per);
  for (int e = e0; e < e1; ++e) ls.mask[e] = 0;
  wave_lds_sync();
  for (int p = lane; p < P; p += 64)
    if (ls.pe[p] >= 0) atomicOr(&ls.mask[ls.pe[p]], 1u << (p / a.k));  // < 0: dropped by top-p
  wave_lds_sync();
  int cnt = 0, pres = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = __popc(ls.mask[e]);
    cnt += c;
    pres += c > 0;
  }
  // inclusive scan of (present << 16 | count) across the wavefront
  int v = wave_inclusive_scan((pres << 16) | cnt);
  const int excl = v - ((pres << 16) | cnt);
  int up = excl >> 16, uc = excl & 0xFFFF;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = e0 + i;
    if (i < per && e < e1) {
      const int c = __popc(ls.mask[e]);
      ls.base[e] = uc;
      if (c > 0) {
        a.uniq_ids[up] = e;
        a.uniq_off[up] = uc;
        if (a.with_slots) {
          SlotEntry se;
          se.base = ls.ep[e];
          se.n = c;
          se.p0 = uc;
          a.slots[a.S + up] = se;
        }
        ++up;
      }
      uc += c;
    }
  }
  const int tot = __builtin_amdgcn_readlane(v, 63);
  const int nu = tot >> 16;
  if (lane == 0) {
    *a.n_unique = nu;
    a.uniq_off[nu] = tot & 0xFFFF;
  }
  if (a.with_slots)
    for (int sl = a.S + nu + lane; sl < a.slots_max; sl += 64) a.slots[sl].n = 0;
  wave_lds_sync();
  for (int p = lane; p < P; p += 64) {
    const int e = ls.pe[p];
    if (e < 0) continue;
    const int t = p / a.k;
    a.pairs[ls.base[e] + __popc(ls.mask[e] & ((1u << t) - 1u))] = p;
  }
}

// The same outputs for a single token, whose k slots name distinct experts:
// slot j (kept, pe[j] >= 0) is pair j, and its expert's place in the union
// is the number of kept slots with a smaller expert.  Run by one wavefront,
// from registers: one LDS read and the stores.
__device__ __forceinline__ void union_one(const DecArgs& a, UnionLds& ls) {
  const int lane = threadIdx.x & 63;
  const int k = a.k;
  const int e = lane < k ? ls.pe[lane] : -1;
  int r = 0;
  for (int j = 0; j < k; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    r += (ej >= 0 && ej < e) ? 1 : 0;
  }
  const int nu = __popcll(__ballot(e >= 0));
  if (e >= 0) {
    a.uniq_ids[r] = e;
    a.uniq_off[r] = r;
    if (a.with_slots) {
      SlotEntry se;
      se.base = ls.ep[e];
      se.n = 1;
      se.p0 = r;
      a.slots[a.S + r] = se;
    }
    a.pairs[r] = lane;
  }
  if (lane == 0) {
    *a.n_unique = nu;
    a.uniq_off[nu] = nu;
  }
  if (a.with_slots)
    for (int sl = a.S + nu + lane; sl < a.slots_max; sl += 64) a.slots[sl].n = 0;
}

// ---- router unit: fp64 partial logits of expert e over one column segment --
// Segment s of expert e writes plane s of z ([plane][T][E]); the top-k step
// adds the planes in order and the bias.  One wavefront.
constexpr int kLogitsBatch = 12;  // 16-byte router loads in flight per lane
// Arrival of a router workgroup (after all of its units): five hundred
// arrivals on one counter queue up behind each other at the memory, so the
// workgroups arrive on one of kRouterGroups group counters and the last of
// each group on the top counter.  True for the last workgroup overall.
// Called by wavefront 0 after a workgroup barrier; every wavefront has
// waited for its own logit stores before that barrier.
__device__ __forceinline__ bool router_arrive(const DecArgs& a) {
  const int b = blockIdx.x;
  const int ng = min(kRouterGroups, a.n_router_wg), g = b % ng;
  const uint32_t in_group = (uint32_t)((a.n_router_wg - g + ng - 1) / ng);
  if (!arrive_last(a.sync + kSyRouter + 16 * (1 + g), in_group)) return false;
  return arrive_last(a.sync + kSyRouter, (uint32_t)ng);
}

__device__ __forceinline__ void router_unit(const DecArgs& a, int it) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int e = it / a.rsplit, seg = it % a.rsplit;
  const int lane = threadIdx.x & 63;
  double acc[kDecodeMaxTokens];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTokens; ++t) acc[t] = 0.0;
  const f32x4* wr = reinterpret_cast<const f32x4*>(a.Wr + (size_t)e * a.H);
  const int n4 = min(a.H / 4, (seg + 1) * a.seg4);
  for (int base = seg * a.seg4; base < n4; base += 64 * kLogitsBatch) {
    f32x4 w[kLogitsBatch];
#pragma unroll
    for (int i = 0; i < kLogitsBatch; ++i) {
      const int c4 = base + lane + 64 * i;
      w[i] = (c4 < n4) ? __builtin_nontemporal_load(wr + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < kDecodeMaxTokens; ++t) {
      if (t < a.T) {
        double s0 = acc[t], s1 = 0.0;
#pragma unroll
        for (int i = 0; i < kLogitsBatch; ++i) {
          const int c4 = base + lane + 64 * i;
          const uint2 xv = (c4 < n4) ? *reinterpret_cast<const uint2*>(a.x + (size_t)t * a.H + 4 * c4) : make_uint2(0, 0);
          const _Float16 x0 = __builtin_bit_cast(_Float16, (uint16_t)(xv.x & 0xFFFF));
          const _Float16 x1 = __builtin_bit_cast(_Float16, (uint16_t)(xv.x >> 16));
          const _Float16 x2 = __builtin_bit_cast(_Float16, (uint16_t)(xv.y & 0xFFFF));
          const _Float16 x3 = __builtin_bit_cast(_Float16, (uint16_t)(xv.y >> 16));
          s0 = fma((double)x0, (double)w[i].x, s0);
          s1 = fma((double)x1, (double)w[i].y, s1);
          s0 = fma((double)x2, (double)w[i].z, s0);
          s1 = fma((double)x3, (double)w[i].w, s1);
        }
        acc[t] = s0 + s1;
      }
    }
  }
  // the tokens' sums, four butterflies at a time interleaved (independent
  // chains; each token's sum in the same order as wave_sum; tokens past T
  // hold zeros)
#pragma unroll
  for (int t0 = 0; t0 < kDecodeMaxTokens; t0 += 4) {
    if (t0 < a.T) {
      double v[4] = {acc[t0], acc[t0 + 1], acc[t0 + 2], acc[t0 + 3]};
      wave_sum_n(v);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane == 0 && t0 + i < a.T) st_dev(a.z + ((size_t)seg * a.T + t0 + i) * a.E + e, v[i]);
    }
  }
}

// Router units of one workgroup; the last workgroup then takes the top-k of
// every token (tokens spread over its wavefronts) and forms the union.
__device__ __forceinline__ void router_workgroup(const DecArgs& a, UnionLds& ls) {
  __shared__ int s_last;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int it = blockIdx.x * kWpg + wave;
  if (it < a.n_router) router_unit(a, it);
  if (a.gu_routes) return;  // the routed gate/up launch ranks the token
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's logit stores are done
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (wave == 0) {
    const bool last = router_arrive(a);
    if (lane == 0) s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // The last wavefront stages the expert pointers the union needs in LDS
  // (wavefront 0, which ranks the first token, does not wait for them).
  if (wave == kWpg - 1 && a.with_slots)
    for (int e = lane; e < a.E; e += 64) ls.ep[e] = (const uint8_t*)a.experts[e];
  const int tpw = (a.T + kWpg - 1) / kWpg;
  const int t0 = wave * tpw, t1 = min(a.T, t0 + tpw);
  for (int t = t0; t < t1; ++t)
    topk_tokens(a.z + (size_t)t * a.E, a.rsplit, (size_t)a.T * a.E, a.rbias, a.E, a.k, a.top_p, 1,
                a.topk_idx + t * a.k, a.topk_w + t * a.k, ls.pe + t * a.k, ls.rank[wave]);
  __syncthreads();
  if (wave == 0) {
    if (a.T == 1) union_one(a, ls);
    else union_step(a, ls);
  }
}

// ---- one token: top-k by the four wavefronts of a workgroup -------------------
// Experts are ordered by (logit descending, index ascending), a total order.
// Fast path (E <= 256, k <= 16): wavefront w holds experts 64w .. 64w+63,
// one per lane; an expert's rank in that group is the number of members
// whose key has a larger high word, counted against every lane through row
// rotations (DPP) of the four row arrangements of the wavefront; the k first
// of every group are candidates; every wavefront ranks the 4k candidates the
// same way (no barrier afterwards).  That is exact as long as no two of the experts involved share a
// high word: every expert above a true top-k member is then a candidate of
// its group, and a non-member counts k or more.  Two candidates on one rank
// show such a tie (or keys that differ only in their low words), and then
// -- as for larger E or k -- every expert is ranked exactly against all E
// keys in LDS, index included.
struct TopkLds {
  uint64_t key[kMaxExperts];
  const uint8_t* ep[kMaxExperts];  // packed expert pointers, loaded beside the logits
  uint32_t chi[kWpg * 16];         // fast path: each group's candidates by rank, high words
  int cidx[kWpg * 16];             //   and experts (-1: none)
  int tie[kWpg];
  int se[kWpg][kMaxTopK];          // fast path: each wavefront's slot experts
  uint64_t sk[kMaxTopK];           // exact path: slot j, key and expert
  int sx[kMaxTopK];
};

// Expert f (key kf) comes before expert e (key ke).
__device__ __forceinline__ bool comes_before(uint64_t kf, int f, uint64_t ke, int e) {
  return kf > ke || (kf == ke && f < e);
}

// Logit key of expert e (the planes added in order, then the bias, as the
// serial top-k adds them).  The planes were written by the previous launch:
// plain loads, so that the workgroups of one XCD share its L2 copy (every
// workgroup of the launch reads the same few KiB at once).
__device__ __forceinline__ uint64_t logit_key(const DecArgs& a, int e) {
  // every plane slot is loaded (a slot past rsplit re-reads plane 0 and is
  // not added), so that the loads issue together: one memory latency
  double zs[kMaxLogitParts];
#pragma unroll
  for (int s = 0; s < kMaxLogitParts; ++s) zs[s] = a.z[(size_t)(s < a.rsplit ? s : 0) * a.E + e];
  const float b = a.rbias ? a.rbias[e] : 0.0f;
  double v = 0.0;
#pragma unroll
  for (int s = 0; s < kMaxLogitParts; ++s)
    if (s < a.rsplit) v += zs[s];
  if (a.rbias) v += (double)b;
  return order_key(v);
}

// Number of lanes whose value is larger than this lane's (values held one
// per lane): every lane is reached by one of 16 row rotations of one of the
// four row arrangements (rows as they are, swapped by 16, by 32, by 48).
template <int... R>
__device__ __forceinline__ int count_larger_rot(uint32_t v, uint32_t h, std::integer_sequence<int, R...>) {
  // row_ror:r for r = 1..15 (DPP control 0x120 + r)
  return ((((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121 + R, 0xF, 0xF, false) > h) ? 1 : 0) + ...);
}

// NQ = 4: all 64 lanes; NQ = 2: lanes 0-31 (rows 0 and 1) only, for values
// held in those lanes.
template <int NQ>
__device__ __forceinline__ int count_larger(uint32_t h) {
  const uint32_t x16 = (uint32_t)partner<16>((int)h);
  uint32_t v[4] = {h, x16, 0u, 0u};
  if (NQ == 4) v[2] = (uint32_t)partner<32>((int)h), v[3] = (uint32_t)partner<32>((int)x16);
  int c = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) c += (v[q] > h ? 1 : 0) + count_larger_rot(v[q], h, std::make_integer_sequence<int, 15>{});
  return c;
}

// Every lane ends with the OR of the lanes' values.
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v |= (uint32_t)partner<1>((int)v);
  v |= (uint32_t)partner<2>((int)v);
  v |= (uint32_t)partner<4>((int)v);
  v |= (uint32_t)partner<8>((int)v);
  v |= (uint32_t)partner<16>((int)v);
  v |= (uint32_t)partner<32>((int)v);
  return v;
}

// Called by the whole workgroup.  On the fast path (returns true) lane l of
// every wavefront holds candidate l: its expert ci (-1: none) and its rank R
// among all experts (the slots are the candidates with R < k); with
// `slots`, lane j < k also gets slot j's key (kj) and expert (ej).  On the
// exact path (returns false) lane j < k gets kj and ej.  Every wavefront
// ranks the candidates itself (the same data, the same result), so the fast
// path ends without a barrier.  ls.ep holds the expert pointers.
__device__ __forceinline__ bool topk_parallel(const DecArgs& a, TopkLds& ls, bool slots, int& R, int& ci, uint64_t& kj,
                                              int& ej) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int E = a.E, k = a.k;
  constexpr int NT = kWpg * 64;
  for (int e = tid; e < E; e += NT) {
    ls.key[e] = logit_key(a, e);
    ls.ep[e] = (const uint8_t*)a.experts[e];
  }
  // fast path: group w is experts 64w .. 64w+63, held by wavefront w (the
  // thread of expert e wrote its key above)
  const bool try_fast = E <= NT && k <= 16;
  if (try_fast) {
    // 0: empty, below every real high word
    const uint32_t h = tid < E ? (uint32_t)(ls.key[tid] >> 32) : 0u;
    const int gt = count_larger<4>(h);
    const bool cand = tid < E && gt < k;
    if (lane < 16) ls.chi[wave * 16 + lane] = 0u, ls.cidx[wave * 16 + lane] = -1;
    if (cand) {
      ls.chi[wave * 16 + gt] = h;
      ls.cidx[wave * 16 + gt] = tid;
    }
    const uint32_t taken = wave_or_u32(cand ? 1u << gt : 0u);
    const int ncand = __popcll(__ballot(cand));  // (a ballot outside any lane branch)
    if (lane == 0) ls.tie[wave] = __popc(taken) != ncand;
  }
  __syncthreads();
  bool fast = try_fast;
  if (fast) {
#pragma unroll
    for (int w = 0; w < kWpg; ++w) fast = fast && !ls.tie[w];
  }
  if (fast) {
    // lane l holds candidate (group l / k, rank l % k)
    const int nc = kWpg * k;
    const uint32_t h = lane < nc ? ls.chi[(lane / k) * 16 + lane % k] : 0u;
    ci = lane < nc ? ls.cidx[(lane / k) * 16 + lane % k] : -1;
    R = nc <= 32 ? count_larger<2>(h) : count_larger<4>(h);
    const bool top = ci >= 0 && R < k;
    const uint32_t taken = wave_or_u32(top ? 1u << R : 0u);
    fast = __popcll(__ballot(top)) == k && __popc(taken) == k;  // the same in every wavefront
    if (fast && slots) {
      if (top) ls.se[wave][R] = ci;
      wave_lds_sync();
      if (lane < k) {
        ej = ls.se[wave][lane];
        kj = ls.key[ej];
      }
    }
  }
  if (!fast) {  // exact ranks of every expert against all E keys
    for (int e = tid; e < E; e += NT) {
      const uint64_t ke = ls.key[e];
      int r = 0;
      for (int f = 0; f < E; ++f) r += comes_before(ls.key[f], f, ke, e) ? 1 : 0;
      if (r < k) {
        ls.sk[r] = ke;
        ls.sx[r] = e;
      }
    }
    __syncthreads();
    if (lane < k) {
      kj = ls.sk[lane];
      ej = ls.sx[lane];
    }
  }
  return fast;
}

// ---- one token: routing inside the routed gate/up launch ----------------------
// Every routed gate/up workgroup ranks the token itself from the partial
// logits that the routing launch wrote (the same fp64 logits and order as
// the routing leader would use, so every workgroup reaches the same slots)
// and takes the expert of its slot j (pair j of the token; the order of the
// gate/up work does not matter, the down launch reads the union).  The
// routing launch therefore ends with its router units: no arrival chain, no
// leader, no slot-table lookup before the weight stream.  Workgroup 0 also
// writes the routing outputs, the union and the slot table that the down
// launch reads.  Returns false for a slot dropped by top-p.
struct RouteOneLds {
  TopkLds tk;
};

__device__ __forceinline__ bool route_one(const DecArgs& a, int j, bool writer, SlotInfo& si, RouteOneLds& ls) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // the ranking shares its SIMDs with the shared expert's streaming
  // wavefronts: it goes first while it runs
  __builtin_amdgcn_s_setprio(3);
  const bool out = writer && wave == 0;
  // slots in lane order are needed for the weights: where they are written,
  // or where they decide which slots top-p keeps
  const bool need_w = out || a.top_p_on;
  int R = 0, ci = -1, ej = -1;
  uint64_t kj = 0;
  const bool fast = topk_parallel(a, ls.tk, need_w, R, ci, kj, ej);
  int e_j;  // slot j's expert, or -1 when top-p drops it
  if (fast && !need_w) {
    const uint64_t hit = __ballot(ci >= 0 && R == j);
    e_j = __builtin_amdgcn_readlane(ci, __ffsll((unsigned long long)hit) - 1);
  } else {
    const SlotWeight sw = need_w ? slot_weights(from_order_key(kj), a.k, a.top_p) : SlotWeight{a.k, 0.0f};
    const int e = lane < sw.m ? ej : -1;  // kept slots
    e_j = __builtin_amdgcn_readlane(e, j);
    if (out) {  // the routing outputs, the union of one token (as union_one) and the slot table
      int r = 0;  // kept experts below e
      for (int jj = 0; jj < a.k; ++jj) {
        const int e2 = __builtin_amdgcn_readlane(e, jj);
        r += (e2 >= 0 && e2 < e) ? 1 : 0;
      }
      const int nu = __popcll(__ballot(e >= 0));
      if (lane < a.k) {
        a.topk_idx[lane] = e;
        a.topk_w[lane] = sw.w;
      }
      if (e >= 0) {
        a.uniq_ids[r] = e;
        a.uniq_off[r] = r;
        SlotEntry se;
        se.base = ls.tk.ep[e];
        se.n = 1;
        se.p0 = r;
        a.slots[a.S + r] = se;
        a.pairs[r] = lane;
      }
      if (lane == 0) {
        *a.n_unique = nu;
        a.uniq_off[nu] = nu;
      }
      for (int sl = a.S + nu + lane; sl < a.slots_max; sl += 64) a.slots[sl].n = 0;
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if (e_j < 0) return false;  // the same in every wavefront
  si.base = ls.tk.ep[e_j];
  si.n = 1;
  si.p0 = -1;  // unused: the pair is known
  si.pair = j;
  return true;
}

// ---- gate/up: one (slot, 64-row block) per workgroup --------------------------
// Wavefront w streams K-segment q0 + w of the block for a tile of NT tokens;
// the four results meet in LDS and wavefront 0 adds them in segment order.
template <int KT>
struct GuLds {
  float r[kWpg][2][KT][64];
};

template <int FMT, int NT>
__device__ __forceinline__ void gu_stream(const DecArgs& a, const uint16_t* __restrict__ x, const SlotInfo& si,
                                          int rb, int ks, int nch, int i0, float (&acc)[2][NT]) {
  const int lane = threadIdx.x & 63;
  const int c0 = ks * nch;
  constexpr int C = Fmt<FMT>::C;
  const guint4* w = (const guint4*)(si.base + a.L.gu_off) + ((size_t)rb * (a.H / C) + c0) * 2 * 64 + lane;
  const guint2* sc = nullptr;
  if (FMT == MOE_W_E2M1_B16)
    sc = (const guint2*)(si.base + a.L.sgu_off) + ((size_t)rb * (a.H / 128) + c0 / 4) * 2 * 64 + lane;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[0][t] = acc[1][t] = 0.f;
  // The weights are requested first; the tokens' rows are looked up while
  // they are in flight.  Integer formats also need the sum of the segment's
  // activations (code offset): the lanes request its 16-byte pieces after
  // the first weights and add them up after the stream.
  const cu32x4* act[NT];  // x is read-only during the launch
  const u32x4* xg[NT];
  const int npc = nch * Fmt<FMT>::XPC;
  u32x4 xp[NT][kSumPieces];
  stream_ring<FMT, 2, NT, kRingChunks / Fmt<FMT>::U>(w, sc, act, nch, acc, [&] {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int tok, row;
      slot_token(a, si, i0 + t, tok, row);
      xg[t] = reinterpret_cast<const u32x4*>(x + (size_t)tok * a.H + C * c0);
      act[t] = (const cu32x4*)xg[t];
      if (row_scaled(FMT)) {
#pragma unroll
        for (int i = 0; i < kSumPieces; ++i) {
          const int q = lane + 64 * i;
          xp[t][i] = xg[t][q < npc ? q : 0];
        }
      }
    }
  });
  if (!row_scaled(FMT)) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float xs = 0.f;
#pragma unroll
    for (int i = 0; i < kSumPieces; ++i) xs = (lane + 64 * i < npc) ? sum8(xp[t][i], xs) : xs;
    for (int q = lane + 64 * kSumPieces; q < npc; q += 64) xs = sum8(xg[t][q], xs);
    const float off = Fmt<FMT>::OFF * wave_sum_f32(xs);
    acc[0][t] -= off;
    acc[1][t] -= off;
  }
}

// Gate and up scales of this lane's row of block rb, as stored (binary16
// row scales, or the E2M1 fp32 tensor scales).  Requested before the
// weights and converted only where they are used, so that nothing waits
// for them before the weight stream starts.
struct GuScales {
  uint32_t g, u;
};

template <int FMT>
__device__ __forceinline__ GuScales gu_scales(const DecArgs& a, const SlotInfo& si, int rb) {
  typedef __attribute__((address_space(1))) const uint16_t gu16;
  typedef __attribute__((address_space(1))) const uint32_t gu32;
  const int r = 64 * rb + (threadIdx.x & 63);
  if (row_scaled(FMT))
    return GuScales{(uint32_t)((gu16*)(si.base + a.L.sg_off))[r], (uint32_t)((gu16*)(si.base + a.L.su_off))[r]};
  gu32* g3 = (gu32*)(si.base + a.L.g3_off);
  return GuScales{g3[0], g3[1]};
}

template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t bits) {
  return row_scaled(FMT) ? (float)__builtin_bit_cast(_Float16, (uint16_t)bits) : __builtin_bit_cast(float, bits);
}

// h for token row `row` of this block from its gate/up sums (wavefront 0).
template <int FMT>
__device__ __forceinline__ void gu_finish(const DecArgs& a, GuScales gs, int rb, int row, float g, float u) {
  const int r = 64 * rb + (threadIdx.x & 63);
  // opaque from here on: keeps the conversion (and the wait for the load)
  // from being hoisted in front of the weight stream
  asm volatile("" : "+v"(gs.g), "+v"(gs.u));
  const float hv = silu(g * scale_value<FMT>(gs.g)) * (u * scale_value<FMT>(gs.u));
  a.h[(size_t)row * a.I + r] = __builtin_bit_cast(uint16_t, (_Float16)hv);  // read by the next launch
}

// K-segments [grp*nw, grp*nw + nw) of (slot s, row block rb), nw <= kWpg
// wavefronts (the others only join the barriers).  With ngrp == 1 the
// workgroup forms h; otherwise each group writes its sum as partial plane
// grp and the last workgroup to arrive (of all groups and token tiles)
// adds the planes in order and forms h for every token of the slot.
template <int FMT, int NT, int KT>
__device__ __forceinline__ void gu_tile_group(const DecArgs& a, const uint16_t* __restrict__ x, const SlotInfo& si,
                                              int s, int rb, int grp, int ngrp, int nw, int nch, int i0,
                                              GuScales gs, GuLds<KT>& ls) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave < nw) {
    float acc[2][NT];
    gu_stream<FMT, NT>(a, x, si, rb, grp * nw + wave, nch, i0, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ls.r[wave][0][t][lane] = acc[0][t];
      ls.r[wave][1][t][lane] = acc[1][t];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float g = 0.f, u = 0.f;
      for (int q = 0; q < nw; ++q) {
        g += ls.r[q][0][t][lane];
        u += ls.r[q][1][t][lane];
      }
      int tok, row;
      slot_token(a, si, i0 + t, tok, row);
      if (ngrp == 1) {
        gu_finish<FMT>(a, gs, rb, row, g, u);
      } else {
        float* pr = a.p_gu + (((size_t)grp * a.rows_total + row) * 2) * a.I + 64 * rb + lane;
        st_dev(pr, g);
        st_dev(pr + a.I, u);
      }
    }
  }
  __syncthreads();  // LDS is reused by the next tile
}

template <int FMT, int KT>
__device__ __forceinline__ void gu_group(const DecArgs& a, const uint16_t* __restrict__ x, int s, const SlotInfo& si,
                                         int rb, int grp, int ngrp, int nw, int nch, int tile, int ntiles,
                                         GuLds<KT>& ls) {
  const GuScales gs = gu_scales<FMT>(a, si, rb);
  // token tiles tile, tile + ntiles, ... of the slot (several workgroups
  // share a slot's tiles when ntiles > 1)
  for (int i0 = tile * KT; i0 < si.n; i0 += KT * ntiles) {
    if (KT == 1 || si.n - i0 == 1) gu_tile_group<FMT, 1, KT>(a, x, si, s, rb, grp, ngrp, nw, nch, i0, gs, ls);
    else gu_tile_group<FMT, KT, KT>(a, x, si, s, rb, grp, ngrp, nw, nch, i0, gs, ls);
  }
  if (ngrp == 1 || threadIdx.x >= 64) return;
  if (!arrive_last(a.gu_cnt + (size_t)s * (a.I / 64) + rb, (uint32_t)(ngrp * ntiles))) return;
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < si.n; ++i) {
    int tok, row;
    slot_token(a, si, i, tok, row);
    float g = 0.f, u = 0.f;
    for (int q0 = 0; q0 < ngrp; q0 += 8) {  // planes in order, loaded 8 at a time
      float pg[8], pu[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q0 + q < ngrp) {
          const float* pr = a.p_gu + (((size_t)(q0 + q) * a.rows_total + row) * 2) * a.I + 64 * rb + lane;
          pg[q] = ld_dev(pr);
          pu[q] = ld_dev(pr + a.I);
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < ngrp) {
          g += pg[q];
          u += pu[q];
        }
    }
    gu_finish<FMT>(a, gs, rb, row, g, u);
  }
}

// ---- down: one (slot, 64-row output block) per workgroup ------------------------
// Wavefront w streams K-segment w for a tile of NT tokens, with its h row
// pieces staged in its own LDS region: vector loads of h mixed into the
// weight stream would make every weight batch wait for them (the vector
// memory counter retires in order), so each step of kStageCols columns
// requests its first weight batches, then stages h while those are in
// flight, then streams.
// ---- output combine -----------------------------------------------------------
// Every (token, slot) pair adds its routing-weighted down row w*o to the
// token's output row in one 64-bit atomic add per element, as a fixed-point
// integer (29 fraction bits, rounded to nearest) together with one arrival:
//   bits  0..55  the sum, two's complement (|sum| < 2^55)
//   bits 56..61  arrivals (at most kMaxTopK + 1)
//   bits 62, 63  a term reached +kFixLimit / -kFixLimit (both: not a number)
// Integer sums are exact and order-free, so the output does not depend on
// which slot arrives when (deterministic and batch-invariant), and the one
// round trip that adds a term also tells its lane whether the row is
// complete: that lane converts the sum to binary16, writes y and returns the
// word to zero.  Each term is held to 2^-30 absolute, below a quarter of the
// smallest binary16 step (2^-24), for any output size.
constexpr double kFixLimit = 1048576.0;  // 2^20: 33 terms of 2^49 units stay below 2^55
constexpr uint64_t kArrival = 1ull << 56;

__device__ __forceinline__ void combine_add(const DecArgs& a, int tok, int r, float w, float o, uint32_t target) {
  uint64_t* cell = a.y_acc + (size_t)tok * a.H + r;
  const double t = (double)w * (double)o;  // exact
  uint64_t add = kArrival;
  if (__builtin_fabs(t) < kFixLimit) {
    const double q = __builtin_rint(t * 0x1p29);  // |q| < 2^49
    const double hi = __builtin_floor(q * 0x1p-32);
    add += ((uint64_t)(int64_t)(int32_t)hi << 32) | (uint64_t)(uint32_t)(q - hi * 0x1p32);
  } else {  // out of range, or not a number: flag it before the arrival that may complete the row
    const uint64_t flag = t >= kFixLimit ? 1ull << 62 : t <= -kFixLimit ? 1ull << 63 : 3ull << 62;
    __hip_atomic_fetch_or(cell, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  const uint64_t tot = __hip_atomic_fetch_add(cell, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
  const uint64_t low = tot & ((1ull << 62) - 1);
  const uint32_t n = (uint32_t)((low + (1ull << 55)) >> 56);
  if (n != target) return;
  float yv;
  const uint32_t f = (uint32_t)(tot >> 62);
  if (f == 0)
    yv = (float)((double)(int64_t)(low - ((uint64_t)n << 56)) * 0x1p-29);
  else
    yv = f == 1 ? __builtin_inff() : f == 2 ? -__builtin_inff() : __builtin_nanf("");
  a.y[(size_t)tok * a.H + r] = __builtin_bit_cast(uint16_t, (_Float16)yv);
  __hip_atomic_store(cell, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KT>
struct DnLds {
  u32x4 h[kWpg][KT * kStageVec];  // per wavefront: KT tokens x kStageCols binary16
  float r[kWpg][KT][64];
};

template <int FMT, int NT, int KT>
__device__ __forceinline__ void dn_tile(const DecArgs& a, const SlotInfo& si, int rb, int seg, int i0, float scale,
                                        DnLds<KT>& ls) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const bool active = rb < a.H / 64;  // the last workgroup of a slot may overhang
  // the combine's tokens, routing weights and arrival counts, looked up
  // before the stream
  int tk[NT];
  float wt[NT];
  uint32_t target[NT];
  if (active && seg == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int tok, row;
      slot_token(a, si, i0 + t, tok, row);
      tk[t] = tok;
      wt[t] = row < a.T * a.k ? ld_const(a.topk_w, row) : 1.f;
      uint32_t kept = a.k;
      if (a.top_p_on) {
        kept = 0;
        for (int j = 0; j < a.k; ++j) kept += ld_const(a.topk_idx, tok * a.k + j) >= 0 ? 1 : 0;
      }
      target[t] = (uint32_t)a.S + kept;
    }
  }
  if (active) {
    const int c0 = seg * a.cpu_dn;
    constexpr int C = Fmt<FMT>::C, XPC = Fmt<FMT>::XPC, kStage = kStageCols / C;
    const guint4* w = (const guint4*)(si.base + a.L.d_off) + ((size_t)rb * (a.I / C) + c0) * 64 + lane;
    const guint2* sc = nullptr;
    if (FMT == MOE_W_E2M1_B16)
      sc = (const guint2*)(si.base + a.L.sdd_off) + ((size_t)rb * (a.I / 128) + c0 / 4) * 64 + lane;
    u32x4* hl = ls.h[wave];
    const lu32x4* act[NT];  // LDS
#pragma unroll
    for (int t = 0; t < NT; ++t) act[t] = (const lu32x4*)(hl + t * kStageVec);
    float acc[1][NT], hs[NT];  // hs: this lane's share of the h sum (code offset)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[0][t] = hs[t] = 0.f;
    for (int p0 = 0; p0 < a.cpu_dn; p0 += kStage) {
      const int np = min(kStage, a.cpu_dn - p0);
      wave_lds_sync();  // the previous step's LDS reads are done
      stream_ring<FMT, 1, NT, kRingChunks / Fmt<FMT>::U>(
          w + (size_t)p0 * 64, FMT == MOE_W_E2M1_B16 ? sc + (size_t)(p0 / 4) * 64 : sc, act, np, acc, [&] {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              int tok, row;
              slot_token(a, si, i0 + t, tok, row);
              const u32x4* src = reinterpret_cast<const u32x4*>(a.h + (size_t)row * a.I + C * c0);
              for (int q = lane; q < np * XPC; q += 64) {
                const u32x4 v = src[p0 * XPC + q];
                hl[t * kStageVec + q] = v;
                if (row_scaled(FMT)) hs[t] = sum8(v, hs[t]);
              }
            }
            wave_lds_sync();
          });
    }
    if (row_scaled(FMT)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[0][t] -= Fmt<FMT>::OFF * wave_sum_f32(hs[t]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) ls.r[wave][t][lane] = acc[0][t];
  }
  __syncthreads();
  if (active && seg == 0) {  // first wavefront of this row block adds its segments in order
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float v = 0.f;
      for (int q = 0; q < a.ks_dn; ++q) v += ls.r[wave + q][t][lane];
      combine_add(a, tk[t], 64 * rb + lane, wt[t], v * scale, target[t]);
    }
  }
  __syncthreads();  // LDS is reused by the next tile
}

// Workgroup = (slot s, kWpg / ks_dn consecutive output row blocks); wavefront
// w takes row block rbg * (kWpg / ks_dn) + w / ks_dn, K-segment w % ks_dn.
template <int FMT, int KT>
__device__ __forceinline__ void dn_unit(const DecArgs& a, int s, int rbg, DnLds<KT>& ls) {
  SlotInfo si;
  if (!get_slot(a, s, si)) return;  // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int rb = rbg * (kWpg / a.ks_dn) + wave / a.ks_dn, seg = wave % a.ks_dn;
  const int r = 64 * min(rb, a.H / 64 - 1) + lane;
  float scale;
  if (row_scaled(FMT))
    scale = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(si.base + a.L.sd_off)[r]);
  else
    scale = reinterpret_cast<const float*>(si.base + a.L.g3_off)[2];
  for (int i0 = 0; i0 < si.n; i0 += KT) {
    if (KT == 1 || si.n - i0 == 1) dn_tile<FMT, 1, KT>(a, si, rb, seg, i0, scale, ls);
    else dn_tile<FMT, KT, KT>(a, si, rb, seg, i0, scale, ls);
  }
}

// Shared expert gate/up, workgroup j of its grid: workgroup = (token tile,
// row block, group of kWpg K-segments); the tiles of one (row block, group)
// are n_rbg workgroups apart, a multiple of 8, so they run on one XCD and
// share its L2 copy of the weights.
template <int FMT, int KT>
__device__ __forceinline__ void shared_gu(const DecArgs& a, const uint16_t* __restrict__ x, int j, GuLds<KT>& gl) {
  const int nw = min(kWpg, a.ks_sgu), ngrp = a.ks_sgu / nw, n_rbg = (a.I / 64) * ngrp;
  const int r = j % n_rbg;
  SlotInfo si;
  get_slot(a, 0, si);
  gu_group<FMT, KT>(a, x, 0, si, r / ngrp, r % ngrp, ngrp, nw, a.cpu_sgu, j / n_rbg, (a.T + KT - 1) / KT, gl);
}

// Workgroups of the shared expert's gate/up.
inline int shared_gu_workgroups(const DecArgs& a, int KT) {
  const int nw = std::min(kWpg, a.ks_sgu);
  return a.S * (a.I / 64) * (a.ks_sgu / nw) * ((a.T + KT - 1) / KT);
}

// ---- kernels ---------------------------------------------------------------------
template <int FMT, int KT>
__global__ __launch_bounds__(64 * kWpg) void k_route_phase(DecArgs a, const uint16_t* __restrict__ x) {
  __shared__ UnionLds ul;
  __shared__ GuLds<KT> gl;
  const int b = blockIdx.x;
  if (b < a.n_router_wg) {
    router_workgroup(a, ul);
    return;
  }
  shared_gu<FMT, KT>(a, x, b - a.n_router_wg, gl);
}

// moe_route on small batches: the router workgroups of k_route_phase alone
// (no shared expert, no slot table).
__global__ __launch_bounds__(64 * kWpg) void k_route_only(DecArgs a) {
  __shared__ UnionLds ul;
  router_workgroup(a, ul);
}

template <int FMT, int KT>
__global__ __launch_bounds__(64 * kWpg) void k_gu_phase(DecArgs a, const uint16_t* __restrict__ x) {
  __shared__ GuLds<KT> gl;
  __shared__ RouteOneLds rl;
  // workgroup = (slot, row block, group of kWpg K-segments)
  // with gu_routes, the shared expert's gate/up workgroups come first (they
  // stream while the routed workgroups rank the token); one gu_group call
  // serves both kinds
  const int b = blockIdx.x - a.n_sgu_in_gu;
  SlotInfo si;
  int s, r, ngrp, nw, nch, tile, ntiles;
  if (b < 0) {
    nw = min(kWpg, a.ks_sgu), ngrp = a.ks_sgu / nw;
    const int n_rbg = (a.I / 64) * ngrp;
    r = blockIdx.x % n_rbg, s = 0, nch = a.cpu_sgu, tile = blockIdx.x / n_rbg, ntiles = (a.T + KT - 1) / KT;
    get_slot(a, 0, si);
  } else {
    nw = min(kWpg, a.ks_gu), ngrp = a.ks_gu / nw;
    // slot u: the union's u-th expert, or with gu_routes the token's u-th
    // ranked slot
    const int per_slot = (a.I / 64) * ngrp, u = b / per_slot;
    r = b % per_slot, s = a.S + u, nch = a.cpu_gu, tile = 0, ntiles = 1;
    if (a.gu_routes) {
      if (!route_one(a, u, b == 0, si, rl)) return;  // uniform over the workgroup
    } else if (!get_slot(a, s, si)) {
      return;
    }
  }
  gu_group<FMT, KT>(a, x, s, si, r / ngrp, r % ngrp, ngrp, nw, nch, tile, ntiles, gl);
}

template <int FMT, int KT>
__global__ __launch_bounds__(64 * kWpg) void k_dn_phase(DecArgs a) {
  __shared__ DnLds<KT> dl;
  const int rpw = kWpg / a.ks_dn, per_slot = (a.H / 64 + rpw - 1) / rpw;
  dn_unit<FMT, KT>(a, blockIdx.x / per_slot, blockIdx.x % per_slot, dl);
}

template <int FMT, int KT>
hipError_t launch_phases(DecArgs a, const uint16_t* x, hipStream_t s, const StageEvents& se) {
  const int sgu_wg = shared_gu_workgroups(a, KT);
  // one token: the shared gate/up moves to the routed gate/up launch
  a.n_sgu_in_gu = a.gu_routes ? sgu_wg : 0;
  const dim3 blk(64 * kWpg);
  launch_k(k_route_phase<FMT, KT>, dim3(a.n_router_wg + sgu_wg - a.n_sgu_in_gu), blk, s, se.start(0), se.stop(0), a,
           x);
  const int gu_wg = (a.slots_max - a.S) * (a.I / 64) * (a.ks_gu / min(kWpg, a.ks_gu));
  launch_k(k_gu_phase<FMT, KT>, dim3(a.n_sgu_in_gu + gu_wg), blk, s, se.start(1), se.stop(1), a, x);
  const int rpw = kWpg / a.ks_dn;
  launch_k(k_dn_phase<FMT, KT>, dim3(a.slots_max * ((a.H / 64 + rpw - 1) / rpw)), blk, s, se.start(2), se.stop(2), a);
  return hipGetLastError();
}

DecArgs dec_args(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x, const Route& r,
                 void* ws, uint16_t* y, bool with_slots) {
  DecArgs a{};
  a.Wr = w.router_w;
  a.rbias = w.router_b;
  a.x = x;
  a.experts = w.experts;
  a.shared = w.shared;
  a.T = p.T;
  a.H = p.H;
  a.I = p.I;
  a.E = p.E;
  a.k = p.k;
  a.S = p.S;
  a.top_p = d.top_p;
  a.top_p_on = d.top_p > 0.0f && d.top_p < 1.0f;
  a.L = layout_of(d);
  a.y = y;
  a.topk_idx = r.topk_idx;
  a.topk_w = r.topk_w;
  a.z = r.z;
  a.n_unique = r.n_unique;
  a.uniq_ids = r.uniq_ids;
  a.uniq_off = r.uniq_off;
  a.pairs = r.pairs;
  a.slots = r.slots;
  a.h = (uint16_t*)((char*)ws + p.h_off);
  a.p_gu = (float*)((char*)ws + p.p_gu_off);
  a.y_acc = (uint64_t*)((char*)ws + p.acc_off);
  a.sync = (uint32_t*)ws;
  a.gu_cnt = a.sync + p.c_gu;
  a.ks_gu = p.ks_gu;
  a.ks_sgu = p.ks_sgu;
  a.ks_dn = p.ks_dn;
  const int C = 128 / code_bits(d.wfmt);  // columns per chunk
  a.cpu_gu = (p.H / C) / p.ks_gu;
  a.cpu_sgu = (p.H / C) / p.ks_sgu;
  a.cpu_dn = (p.I / C) / p.ks_dn;
  a.slots_max = p.slots_max;
  a.rows_total = p.rows_total;
  // router units: enough column segments that each needs one batch of loads,
  // and at least two per expert (short rows: more units in flight)
  const int n4 = p.H / 4, per = 64 * kLogitsBatch;
  a.rsplit = std::min(kMaxLogitParts, std::max(2, (n4 + per - 1) / per));
  a.seg4 = (n4 + a.rsplit - 1) / a.rsplit;
  a.n_router = p.E * a.rsplit;
  a.n_router_wg = (a.n_router + kWpg - 1) / kWpg;
  a.with_slots = with_slots ? 1 : 0;
  a.gu_routes = (with_slots && p.T == 1) ? 1 : 0;
  return a;
}

}  // namespace

hipError_t launch_decode_route(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                               const Route& r, void* ws, hipStream_t s) {
  const DecArgs a = dec_args(d, p, w, x, r, ws, nullptr, false);
  hipLaunchKernelGGL(k_route_only, dim3(a.n_router_wg), dim3(64 * kWpg), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                         const Route& r, void* ws, uint16_t* y, hipStream_t s, const StageEvents& se) {
  const DecArgs a = dec_args(d, p, w, x, r, ws, y, true);
  // a single token never needs the two-token tiles, which cost registers
  switch (d.wfmt) {
    case MOE_W_INT4_ROW:
      return p.T == 1 ? launch_phases<MOE_W_INT4_ROW, 1>(a, x, s, se) : launch_phases<MOE_W_INT4_ROW, 2>(a, x, s, se);
    case MOE_W_INT8_ROW:
      return p.T == 1 ? launch_phases<MOE_W_INT8_ROW, 1>(a, x, s, se) : launch_phases<MOE_W_INT8_ROW, 2>(a, x, s, se);
    case MOE_W_INT2_ROW:
      return p.T == 1 ? launch_phases<MOE_W_INT2_ROW, 1>(a, x, s, se) : launch_phases<MOE_W_INT2_ROW, 2>(a, x, s, se);
    default:
      return p.T == 1 ? launch_phases<MOE_W_E2M1_B16, 1>(a, x, s, se) : launch_phases<MOE_W_E2M1_B16, 2>(a, x, s, se);
  }
}

}  // namespace moe
