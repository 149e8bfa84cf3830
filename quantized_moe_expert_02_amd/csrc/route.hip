// Router (sigmoid top-k) and batch expert union.
//
// The router is the DeepSeek-V3-style sigmoid router and the union is the
// batch-wise MoE union of the Colibrì engine ("Show HN: 低速のコンピュータでGLM
// 5.2を動かす方法", hakusoku.com, section 実装済み機能): every unique expert
// chosen by the batch is listed once with all the (token, slot) pairs that
// chose it.  The top-k is fixed and deterministic, as the vLLM recipe
// requires of its MoE placement order ("GLM-5.3-Flash 320B MoEを4枚のCMP 170HX
// で動かすvLLMレシピ", 648news.com, section "Ampere世代のGPU向けに最適化された
// 独自カーネル群").
//
// Readings taken where the pages are silent: logits accumulate in fp64 so the
// discrete choice does not depend on summation order; ties go to the lower
// expert index; kept slots are in descending-score order; the kept sigmoid
// scores are renormalised to sum to one; an optional fp32 logit bias is
// added before ranking.
#include "wave.h"

namespace moe {
namespace {

struct RouteArgs {
  const float* Wr;
  const float* b;
  const uint16_t* x;
  int T, H, E, k, S;
  float top_p;
  double* z;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_unique;
  int32_t* uniq_ids;
  int32_t* uniq_off;
  int32_t* pairs;
  int32_t* ucnt;
  int32_t* ubase;
  uint32_t* counter;
  int n_chunks;
  // slot table and grouped-GEMM tile list (forward only)
  SlotEntry* slots;
  int32_t* tiles;     // gate/up tiles (kPrefillTileRows tokens)
  int32_t* tiles_dn;  // down tiles (kDownTileRows tokens)
  int32_t* n_tiles;   // [2]
  int slots_max;
  const void* const* experts;
  const void* shared;
};

// Slot table for the expert kernels: shared expert first, then the union.
__device__ __forceinline__ void write_slot(const RouteArgs& a, int slot, int expert, int n, int p0) {
  SlotEntry se;
  se.base = (const uint8_t*)(expert < 0 ? a.shared : a.experts[expert]);
  se.n = n;
  se.p0 = p0;
  a.slots[slot] = se;
}

// ---- large batches -------------------------------------------------------

// fp64 logits for large batches on the matrix cores (v_mfma_f64_16x16x4_f64,
// D = A·B + C with A 16x4, B 4x16, D 16x16 fp64): block (128 tokens, 64
// experts, K-split ks) accumulates columns [ks*Kc, (ks+1)*Kc) into a partial
// sum per (token, expert); partials are added in K-split order by
// k_logits_sum.  Wavefront w owns tokens 32w .. 32w+31 (two 16-token groups)
// x the 64 experts (four 16-expert groups).  K runs in chunks of 16 columns;
// MFMA step s of a chunk gives lane group g column 4g + s, so a lane loads 4
// consecutive binary16 activations and 4 consecutive fp32 weights per group
// and chunk, and widens them to fp64 (exact).  Lane layout: A[i][k] and
// B[k][j] in lane i (or j) + 16k; D[i][j] in lane j + 16*(i % 4), element
// i / 4 (checked on the hardware).
constexpr int kLogitSplit = 8;
constexpr int LGT = 128, LGE = 64;
static_assert(kLogitSplit + 1 <= kZPlanes, "z holds the logits and the K-split partials");
typedef double f64x4 __attribute__((ext_vector_type(4)));

// A copy the compiler cannot fold (ends the life of a loaded register before
// its refill, so that the refill reuses it).
__device__ __forceinline__ uint32_t fresh_u32(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

__global__ __launch_bounds__(256) void k_logits_tiled(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * LGT + wave * 32, e0 = blockIdx.y * LGE;
  const int kc = a.H / kLogitSplit;  // a multiple of 16 (H is a multiple of 128)
  const int kb = blockIdx.z * kc + 4 * g;
  // this lane's rows (clamped into range; results outside are not stored)
  const uint2* xr[2];
  const float4* wr[4];
#pragma unroll
  for (int mg = 0; mg < 2; ++mg) {
    const int tt = min(t0 + 16 * mg + n, a.T - 1);
    xr[mg] = reinterpret_cast<const uint2*>(a.x + (size_t)tt * a.H + kb);
  }
#pragma unroll
  for (int ng = 0; ng < 4; ++ng) {
    const int ee = min(e0 + 16 * ng + n, a.E - 1);
    wr[ng] = reinterpret_cast<const float4*>(a.Wr + (size_t)ee * a.H + kb);
  }
  const int nch = kc / 16;
  f64x4 acc[2][4];
#pragma unroll
  for (int mg = 0; mg < 2; ++mg)
#pragma unroll
    for (int ng = 0; ng < 4; ++ng) acc[mg][ng] = f64x4{0.0, 0.0, 0.0, 0.0};
  // two chunks in flight; chunk c of a row is 4 uint2 / 4 float4 further on
  uint2 xv[2][2];
  float4 wv[2][4];
  auto load = [&](int slot, int c) {
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) xv[slot][mg] = xr[mg][4 * c];
#pragma unroll
    for (int ng = 0; ng < 4; ++ng) wv[slot][ng] = wr[ng][4 * c];
  };
  // widen slot `slot` to fp64 operands (copies first, so the slot can be refilled)
  auto widen = [&](int slot, double (&xa)[2][4], double (&wb)[4][4]) {
#pragma unroll
    for (int mg = 0; mg < 2; ++mg) {
      const uint32_t lo = fresh_u32(xv[slot][mg].x), hi = fresh_u32(xv[slot][mg].y);
      xa[mg][0] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(lo & 0xFFFF));
      xa[mg][1] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(lo >> 16));
      xa[mg][2] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(hi & 0xFFFF));
      xa[mg][3] = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)(hi >> 16));
    }
#pragma unroll
    for (int ng = 0; ng < 4; ++ng) {
      wb[ng][0] = (double)__builtin_bit_cast(float, fresh_u32(__builtin_bit_cast(uint32_t, wv[slot][ng].x)));
      wb[ng][1] = (double)__builtin_bit_cast(float, fresh_u32(__builtin_bit_cast(uint32_t, wv[slot][ng].y)));
      wb[ng][2] = (double)__builtin_bit_cast(float, fresh_u32(__builtin_bit_cast(uint32_t, wv[slot][ng].z)));
      wb[ng][3] = (double)__builtin_bit_cast(float, fresh_u32(__builtin_bit_cast(uint32_t, wv[slot][ng].w)));
    }
  };
  auto multiply = [&](const double (&xa)[2][4], const double (&wb)[4][4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mg = 0; mg < 2; ++mg)
#pragma unroll
        for (int ng = 0; ng < 4; ++ng)
          acc[mg][ng] = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[mg][s], wb[ng][s], acc[mg][ng], 0, 0, 0);
  };
  load(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(1, nch > 1 ? 1 : 0);
  __builtin_amdgcn_sched_barrier(0);
  const int nfull = nch & ~1;  // whole pairs; an odd last chunk waits in slot 0
  for (int c0 = 0; c0 < nfull; c0 += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      double xa[2][4], wb[4][4];
      widen(j, xa, wb);
      __builtin_amdgcn_sched_barrier(0);
      const int cn = c0 + j + 2;
      load(j, cn < nch ? cn : nch - 1);  // past the end: re-read the last chunk, unused
      __builtin_amdgcn_sched_barrier(0);
      multiply(xa, wb);
    }
  }
  if (nch & 1) {
    double xa[2][4], wb[4][4];
    widen(0, xa, wb);
    multiply(xa, wb);
  }
  double* zp = a.z + (size_t)blockIdx.z * a.T * a.E;
#pragma unroll
  for (int mg = 0; mg < 2; ++mg)
#pragma unroll
    for (int ng = 0; ng < 4; ++ng)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + 16 * mg + 4 * r + g, ee = e0 + 16 * ng + n;
        if (tt < a.T && ee < a.E) zp[(size_t)tt * a.E + ee] = acc[mg][ng][r];
      }
}

// Adds the K-split partial logits (in split order) and the bias: z[t][e].
__global__ __launch_bounds__(256) void k_logits_sum(RouteArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)a.T * a.E;
  if (i >= n) return;
  double v = 0.0;
  for (int s = 0; s < kLogitSplit; ++s) v += a.z[(size_t)(s + 1) * n + i];
  a.z[i] = v + (a.b ? (double)a.b[i % a.E] : 0.0);
}

// One wavefront per token.
__global__ __launch_bounds__(256) void k_topk(RouteArgs a) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= a.T) return;
  topk_any<false>(a.z + (size_t)t * a.E, 1, 0, nullptr, a.E, a.k, a.top_p, a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k,
                  nullptr);
}

// Union for large batches, a stable counting sort in three passes over
// chunks of 32 tokens.  Pass 1: per-chunk expert counts.
__global__ __launch_bounds__(256) void k_union_count(RouteArgs a) {
  __shared__ uint32_t s_mask[kMaxExperts];
  const int c = blockIdx.x;
  const int t0 = c * 32;
  const int nt = min(32, a.T - t0);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) s_mask[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nt * a.k; i += blockDim.x) {
    const int t = t0 + i / a.k;
    const int e = a.topk_idx[(size_t)t * a.k + i % a.k];
    if (e >= 0) atomicOr(&s_mask[e], 1u << (i / a.k));  // e < 0: slot dropped by top-p
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.ucnt[(size_t)c * a.E + e] = __popc(s_mask[e]);
}

// Exclusive prefix of v over a block of kScanThreads threads (every thread
// calls it), and the block total.  s_wave: kScanThreads / 64 ints of LDS.
constexpr int kScanThreads = 1024;
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kScanThreads / 64; ++i) {
    const int s = s_wave[i];
    base += i < w ? s : 0;
    tot += s;
  }
  total = tot;
  return base + inc - v;
}

// Grouped-GEMM tile list of BT-token tiles, longest first: a tile's class is
// its number of filled 16-token groups (BT / 16 for a full tile), tiles are
// listed by class in descending order, and within a class by expert, the
// shared expert (slot 0, all T tokens) first, then the union in order; an
// expert's full tiles precede its partial one.  So the launch dispatches the
// long tiles first and ends on short ones.  One block-wide prefix sum per
// class; every thread places its own expert's tiles (tot tokens, union slot
// `slot`).  Returns the number of tiles.
template <int BT>
__device__ int write_tile_list(const RouteArgs& a, int32_t* list, int tot, int slot, int (*s_buf)[kScanThreads / 64]) {
  constexpr int G = BT / 16;
  const int nfull = tot / BT, rest = tot % BT, pcls = (rest + 15) / 16;  // pcls 0: no partial tile
  const int sfull = a.S ? a.T / BT : 0, srest = a.S ? a.T % BT : 0, spcls = (srest + 15) / 16;
  int base = 0;
  for (int c = G; c >= 1; --c) {
    const int cnt = (c == G ? nfull : 0) + (pcls == c ? 1 : 0);
    const int sh = (c == G ? sfull : 0) + (spcls == c ? 1 : 0);
    int total;
    const int ex = block_exclusive_scan(cnt, s_buf[c & 1], total);
    if (threadIdx.x == 0)
      for (int i = 0; i < sh; ++i) {
        const int pos = base + i;
        list[2 * pos] = 0;
        list[2 * pos + 1] = (c == G && i < sfull) ? BT * i : BT * sfull;
      }
    for (int i = 0; i < cnt; ++i) {
      const int pos = base + sh + ex + i;
      list[2 * pos] = slot;
      list[2 * pos + 1] = (c == G && i < nfull) ? BT * i : BT * nfull;
    }
    base += sh + total;
  }
  return base;
}

// Pass 2 (one block, thread e = expert e): per-expert totals over the
// chunks; block-wide prefix sums give each expert's pair offset, its place
// in the union and the places of its tiles in each grouped-GEMM tile list
// (write_tile_list), so every thread writes its own expert's entries; then
// each (chunk, expert) base offset.
__global__ __launch_bounds__(kScanThreads) void k_union_scan(RouteArgs a) {
  __shared__ int s_wave[2][kScanThreads / 64];
  __shared__ int s_cls[2][kScanThreads / 64];
  static_assert(kMaxExperts <= kScanThreads, "one thread per expert");
  const int e = threadIdx.x;
  int tot = 0;  // pairs of expert e (16 independent loads in flight)
  if (e < a.E)
    for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (c0 + i < a.n_chunks) ? a.ucnt[(size_t)(c0 + i) * a.E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) tot += v[i];
    }
  const int used = tot > 0 ? 1 : 0;
  int off_all, nu_all;
  const int off = block_exclusive_scan(tot, s_wave[0], off_all);
  const int u = block_exclusive_scan(used, s_wave[1], nu_all);
  if (used) {
    a.uniq_ids[u] = e;
    a.uniq_off[u] = off;
    if (a.slots) {
      SlotEntry sl;
      sl.base = (const uint8_t*)a.experts[e];
      sl.n = tot;
      sl.p0 = off;
      a.slots[a.S + u] = sl;
    }
  }
  if (a.tiles) {  // (uniform) grouped-GEMM tile lists, longest tiles first
    const int nt = write_tile_list<kPrefillTileRows>(a, a.tiles, tot, a.S + u, s_cls);
    const int nd = write_tile_list<kDownTileRows>(a, a.tiles_dn, tot, a.S + u, s_cls);
    if (e == 0) {
      a.n_tiles[0] = nt;
      a.n_tiles[1] = nd;
    }
  }
  if (e == 0) {
    *a.n_unique = nu_all;
    a.uniq_off[nu_all] = off_all;
    if (a.slots && a.S) write_slot(a, 0, -1, a.T, -1);
  }
  if (a.slots)
    for (int sl = a.S + nu_all + e; sl < a.slots_max; sl += kScanThreads) write_slot(a, sl, 0, 0, 0);
  // base of each (chunk, expert) = expert base + earlier chunks' counts
  if (e < a.E) {
    int run = off;
    for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (c0 + i < a.n_chunks) ? a.ucnt[(size_t)(c0 + i) * a.E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < a.n_chunks) a.ubase[(size_t)(c0 + i) * a.E + e] = run;
        run += v[i];
      }
    }
  }
}

// Pass 3: scatter pair ids to their stable positions.
__global__ __launch_bounds__(256) void k_union_scatter(RouteArgs a) {
  __shared__ uint32_t s_mask[kMaxExperts];
  const int c = blockIdx.x;
  const int t0 = c * 32;
  const int nt = min(32, a.T - t0);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) s_mask[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nt * a.k; i += blockDim.x) {
    const int t = t0 + i / a.k;
    const int e = a.topk_idx[(size_t)t * a.k + i % a.k];
    if (e >= 0) atomicOr(&s_mask[e], 1u << (i / a.k));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * a.k; i += blockDim.x) {
    const int tl = i / a.k;
    const int t = t0 + tl;
    const int e = a.topk_idx[(size_t)t * a.k + i % a.k];
    if (e < 0) continue;
    const int rank = __popc(s_mask[e] & ((1u << tl) - 1u));
    a.pairs[a.ubase[(size_t)c * a.E + e] + rank] = t * a.k + i % a.k;
  }
}

}  // namespace

hipError_t launch_route(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                        const Route& r, bool with_slots, hipStream_t s, hipEvent_t ev_start,
                        hipEvent_t ev_stop) {
  RouteArgs a{};
  a.Wr = w.router_w;
  a.b = w.router_b;
  a.x = x;
  a.T = p.T;
  a.H = p.H;
  a.E = p.E;
  a.k = p.k;
  a.top_p = d.top_p;
  a.z = r.z;
  a.topk_idx = r.topk_idx;
  a.topk_w = r.topk_w;
  a.n_unique = r.n_unique;
  a.uniq_ids = r.uniq_ids;
  a.uniq_off = r.uniq_off;
  a.pairs = r.pairs;
  a.ucnt = r.ucnt;
  a.ubase = r.ubase;
  a.counter = r.counter;
  a.n_chunks = (p.T + 31) / 32;
  a.S = p.S;
  a.slots = with_slots ? r.slots : nullptr;
  a.tiles = with_slots ? r.tiles : nullptr;
  a.tiles_dn = with_slots ? r.tiles_dn : nullptr;
  a.n_tiles = r.n_tiles;
  a.slots_max = p.slots_max;
  a.experts = w.experts;
  a.shared = w.shared;
  {
    RouteArgs b = a;
    b.z = r.z + (size_t)p.T * p.E;  // K-split partials live after z
    launch_k(k_logits_tiled, dim3((p.T + LGT - 1) / LGT, (p.E + LGE - 1) / LGE, kLogitSplit), dim3(256), s, ev_start,
             nullptr, b);
    const size_t n = (size_t)p.T * p.E;
    hipLaunchKernelGGL(k_logits_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(k_topk, dim3((p.T + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_count, dim3(a.n_chunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(kScanThreads), 0, s, a);
  launch_k(k_union_scatter, dim3(a.n_chunks), dim3(256), s, nullptr, ev_stop, a);
  return hipGetLastError();
}

}  // namespace moe
