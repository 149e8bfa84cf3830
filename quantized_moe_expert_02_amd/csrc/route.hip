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
#include "common.h"

namespace moe {
namespace {

constexpr int kWave = 64;

struct RouteArgs {
  const float* Wr;
  const float* b;
  const uint16_t* x;
  int T, H, E, k, S;
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
  uint32_t* zero_from;
  int zero_count;
  int n_chunks;
  // slot table and grouped-GEMM tile list (forward only)
  SlotEntry* slots;
  int32_t* tiles;
  int32_t* n_tiles;
  int slots_max;
  const void* const* experts;
  const void* shared;
};

// ---- wavefront exchange helpers -------------------------------------------
// Value held by the partner lane of a butterfly step.  Steps 1 and 2 use
// quad permutes, 4 and 8 the half-row / row mirrors (which pair lanes of
// groups that earlier steps already made uniform), 16 and 32 the gfx950
// row-swap instructions.
template <int STEP>
__device__ __forceinline__ int partner(int v) {
  if constexpr (STEP == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  else if constexpr (STEP == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  else if constexpr (STEP == 4) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else if constexpr (STEP == 8) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);  // row_mirror
  else if constexpr (STEP == 16) {
    auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

template <int STEP>
__device__ __forceinline__ double partner_d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)partner<STEP>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)partner<STEP>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// (value, index) ordering of the router: larger logit first, then lower index.
__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int STEP>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
  const double ov = partner_d<STEP>(v);
  const int oi = partner<STEP>(i);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Every lane ends with the wave-wide best (value, index) (large batches).
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
  argmax_step<1>(v, i);
  argmax_step<2>(v, i);
  argmax_step<4>(v, i);
  argmax_step<8>(v, i);
  argmax_step<16>(v, i);
  argmax_step<32>(v, i);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)partner<1>((int)v));
  v = max(v, (uint32_t)partner<2>((int)v));
  v = max(v, (uint32_t)partner<4>((int)v));
  v = max(v, (uint32_t)partner<8>((int)v));
  v = max(v, (uint32_t)partner<16>((int)v));
  v = max(v, (uint32_t)partner<32>((int)v));
  return v;
}

// Order-preserving map of a finite double onto uint64: a > b  <=>  key(a) > key(b).
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double from_order_key(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __builtin_bit_cast(double, u);
}

// Every lane ends with the wave-wide best (key, index): the largest key, ties
// to the lower index.  The high key word is reduced first; only when more than
// one lane holds that high word are the low word and the index reduced too.
__device__ __forceinline__ void wave_argmax_key(uint64_t& key, int& idx) {
  const uint32_t hi = (uint32_t)(key >> 32);
  const uint32_t hmax = wave_max_u32(hi);
  const uint64_t cand = __ballot(hi == hmax);
  if (__popcll(cand) == 1) {
    const int l = __ffsll((unsigned long long)cand) - 1;
    key = ((uint64_t)__shfl((int)(uint32_t)(key >> 32), l, 64) << 32) | (uint32_t)__shfl((int)(uint32_t)key, l, 64);
    idx = __shfl(idx, l, 64);
    return;
  }
  const uint32_t lo = (uint32_t)key;
  const uint32_t lmax = wave_max_u32(hi == hmax ? lo : 0u);
  const bool c2 = (hi == hmax) && (lo == lmax);
  const uint32_t best_inv = wave_max_u32(c2 ? ~(uint32_t)idx : 0u);
  key = ((uint64_t)hmax << 32) | lmax;
  idx = (int)~best_inv;
}

// Top-k of one token's logits by one wavefront: k rounds of a wave-wide
// argmax over the experts not yet taken.  Lane l holds experts l + 64 i.
// Writes idx/w for slots 0..k-1 and the chosen experts to slot_expert.
// The routing weights are formed in fp32: sigmoid of the fp64 logit, then
// renormalised over the kept slots.
template <int kPer, bool kCoherent>
__device__ void topk_wave(const double* zrow, int E, int k, int32_t* idx_out, float* w_out, int* slot_expert) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    key[i] = (e < E) ? order_key(kCoherent ? ld_dev(zrow + e) : zrow[e]) : 0ull;  // 0: below every finite key
  }
  uint64_t my_key = 0;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint64_t bk = 0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {  // ascending index, so '>' keeps the lower index on ties
      if (key[i] > bk) {
        bk = key[i];
        bi = lane + i * kWave;
      }
    }
    wave_argmax_key(bk, bi);
    if ((bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + i * kWave == bi) key[i] = 0;
    }
    if (lane == j) {
      my_key = bk;
      my_e = bi;
    }
  }
  const double my_z = from_order_key(my_key);
  const float s = (lane < k) ? 1.0f / (1.0f + expf(-(float)my_z)) : 0.0f;
  float tot = s;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) tot += __shfl_xor(tot, m, kWave);
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = s / tot;
    if (slot_expert) slot_expert[lane] = my_e;
  }
}

template <bool kCoherent>
__device__ void topk_any(const double* zrow, int E, int k, int32_t* idx_out, float* w_out, int* slot_expert) {
  if (E <= 64) topk_wave<1, kCoherent>(zrow, E, k, idx_out, w_out, slot_expert);
  else if (E <= 128) topk_wave<2, kCoherent>(zrow, E, k, idx_out, w_out, slot_expert);
  else if (E <= 256) topk_wave<4, kCoherent>(zrow, E, k, idx_out, w_out, slot_expert);
  else if (E <= 512) topk_wave<8, kCoherent>(zrow, E, k, idx_out, w_out, slot_expert);
  else topk_wave<16, kCoherent>(zrow, E, k, idx_out, w_out, slot_expert);
}

// Slot table for the expert kernels: shared expert first, then the union.
__device__ __forceinline__ void write_slot(const RouteArgs& a, int slot, int expert, int n, int p0) {
  SlotEntry se;
  se.base = (const uint8_t*)(expert < 0 ? a.shared : a.experts[expert]);
  se.n = n;
  se.p0 = p0;
  a.slots[slot] = se;
}

// ---- decode-size routing ------------------------------------------------

// Decode-size logits of expert e by a 256-thread block: thread i covers the
// float4 columns i + 256 q; all of a batch's router loads (non-temporal:
// the router is streamed once per call) are issued before any arithmetic.
// Per-thread fp64 partials are reduced through LDS in a fixed tree.
constexpr int kLogitsBatch = 8;
__device__ void logits_block(const RouteArgs& a, int e, double (*s_part)[256], double (*s_red)[16]) {
  const int tid = threadIdx.x;
  const int n4 = a.H / 4;
  double acc[kRouteSmallMaxTokens];
#pragma unroll
  for (int t = 0; t < kRouteSmallMaxTokens; ++t) acc[t] = 0.0;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4* wr = reinterpret_cast<const f32x4*>(a.Wr + (size_t)e * a.H);
  for (int base = 0; base < n4; base += 256 * kLogitsBatch) {
    f32x4 w[kLogitsBatch];
#pragma unroll
    for (int i = 0; i < kLogitsBatch; ++i) {
      const int c4 = base + tid + 256 * i;
      w[i] = (c4 < n4) ? __builtin_nontemporal_load(wr + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < kRouteSmallMaxTokens; ++t) {
      if (t < a.T) {
        uint2 xv[kLogitsBatch];
#pragma unroll
        for (int i = 0; i < kLogitsBatch; ++i) {
          const int c4 = base + tid + 256 * i;
          xv[i] = (c4 < n4) ? *reinterpret_cast<const uint2*>(a.x + (size_t)t * a.H + 4 * c4) : make_uint2(0, 0);
        }
        double s0 = acc[t], s1 = 0.0;
#pragma unroll
        for (int i = 0; i < kLogitsBatch; ++i) {
          const _Float16 x0 = __builtin_bit_cast(_Float16, (uint16_t)(xv[i].x & 0xFFFF));
          const _Float16 x1 = __builtin_bit_cast(_Float16, (uint16_t)(xv[i].x >> 16));
          const _Float16 x2 = __builtin_bit_cast(_Float16, (uint16_t)(xv[i].y & 0xFFFF));
          const _Float16 x3 = __builtin_bit_cast(_Float16, (uint16_t)(xv[i].y >> 16));
          s0 = fma((double)x0, (double)w[i].x, s0);
          s1 = fma((double)x1, (double)w[i].y, s1);
          s0 = fma((double)x2, (double)w[i].z, s0);
          s1 = fma((double)x3, (double)w[i].w, s1);
        }
        acc[t] = s0 + s1;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouteSmallMaxTokens; ++t)
    if (t < a.T) s_part[t][tid] = acc[t];
  __syncthreads();
  for (int i = tid; i < a.T * 16; i += 256) {
    const int t = i / 16, j = i % 16;
    double v = 0.0;
    for (int q = 0; q < 16; ++q) v += s_part[t][16 * j + q];
    s_red[t][j] = v;
  }
  __syncthreads();
  if (tid < a.T) {
    double v = 0.0;
    for (int j = 0; j < 16; ++j) v += s_red[tid][j];
    st_dev(a.z + (size_t)tid * a.E + e, v + (a.b ? (double)a.b[e] : 0.0));
  }
}

// Union of T*k pairs (T <= 16): per-expert token bitmasks built in LDS; one
// wavefront scans them for the unique experts and their offsets; the rank
// of pair (t, j) within its expert is the number of earlier tokens that
// chose the same expert.
__device__ void union_small(const RouteArgs& a, const int* s_pe, uint32_t* s_mask, int* s_base) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int P = a.T * a.k;
  for (int e = tid; e < a.E; e += nt) s_mask[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) atomicOr(&s_mask[s_pe[p]], 1u << (p / a.k));
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    const int per = (a.E + kWave - 1) / kWave;
    const int e0 = lane * per, e1 = min(a.E, e0 + per);
    int cnt = 0, pres = 0;
    for (int e = e0; e < e1; ++e) {
      const int c = __popc(s_mask[e]);
      cnt += c;
      pres += c > 0;
    }
    // inclusive scan of (present << 16 | count) across the wave
    int v = (pres << 16) | cnt;
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(v, off, kWave);
      if (lane >= off) v += o;
    }
    const int excl = v - ((pres << 16) | cnt);
    int up = excl >> 16, uc = excl & 0xFFFF;
    for (int e = e0; e < e1; ++e) {
      const int c = __popc(s_mask[e]);
      s_base[e] = uc;
      if (c > 0) {
        a.uniq_ids[up] = e;
        a.uniq_off[up] = uc;
        if (a.slots) write_slot(a, a.S + up, e, c, uc);
        ++up;
      }
      uc += c;
    }
    const int tot = __shfl(v, kWave - 1, kWave);
    const int nu = tot >> 16;
    if (lane == 0) {
      *a.n_unique = nu;
      a.uniq_off[nu] = tot & 0xFFFF;
      if (a.slots && a.S) write_slot(a, 0, -1, a.T, -1);
    }
    if (a.slots)
      for (int s = a.S + nu + lane; s < a.slots_max; s += kWave) write_slot(a, s, 0, 0, 0);
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = s_pe[p];
    const int t = p / a.k;
    a.pairs[s_base[e] + __popc(s_mask[e] & ((1u << t) - 1u))] = p;
  }
}

// Decode-size routing in one launch: block e computes the logits of expert e
// for all tokens; the last block to finish (device counter; logits handed
// over with device-coherent stores/loads) does the top-k, the union and the
// slot table, and clears the expert kernels' completion counters.
// Grid: E blocks of 256 threads.
__global__ __launch_bounds__(256) void k_route_small(RouteArgs a) {
  __shared__ double s_part[kRouteSmallMaxTokens][256];
  __shared__ double s_red[kRouteSmallMaxTokens][16];
  __shared__ int s_pe[kRouteSmallMaxTokens * kMaxTopK];
  __shared__ uint32_t s_mask[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_last;
  const int wave = threadIdx.x / kWave;
  logits_block(a, blockIdx.x, s_part, s_red);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) st_dev(a.counter, 0u);
  for (int i = threadIdx.x; i < a.zero_count; i += blockDim.x) a.zero_from[i] = 0;
  for (int t = wave; t < a.T; t += 4)
    topk_any<true>(a.z + (size_t)t * a.E, a.E, a.k, a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k,
                   s_pe + t * a.k);
  __syncthreads();
  union_small(a, s_pe, s_mask, s_base);
}

// ---- large batches -------------------------------------------------------

// fp64 logits for large batches: block (tile of 64 tokens, tile of 64
// experts, K-split ks) accumulates columns [ks*Kc, (ks+1)*Kc) into a partial
// sum per (token, expert); partials are added in K-split order by k_topk.
// Each thread owns 4 tokens x 4 experts; operands are staged in LDS as fp32
// (binary16 -> fp32 is exact) and widened to fp64 for the FMA.
constexpr int LT = 64, LE = 64, LK = 32;
constexpr int kLogitSplit = 4;
__global__ __launch_bounds__(256) void k_logits_tiled(RouteArgs a) {
  __shared__ __attribute__((aligned(16))) float sx[LK][LT];
  __shared__ __attribute__((aligned(16))) float sw[LK][LE];
  const int t0 = blockIdx.x * LT, e0 = blockIdx.y * LE;
  const int kc = a.H / kLogitSplit;
  const int kbeg = blockIdx.z * kc;
  const int tid = threadIdx.x;
  const int tt = (tid & 15) * 4;  // token offset in tile
  const int te = (tid >> 4) * 4;  // expert offset in tile
  double acc[4][4] = {};
  // staging: thread loads 8 consecutive columns of one row (x: 64 rows; w: 64 rows)
  const int sr = tid >> 2, sc8 = (tid & 3) * 8;
  for (int k0 = kbeg; k0 < kbeg + kc; k0 += LK) {
    {
      const int t = t0 + sr;
      float v[8] = {};
      if (t < a.T) {
        const uint4 xv = *reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H + k0 + sc8);
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[i] & 0xFFFF));
          v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w4[i] >> 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sx[sc8 + i][sr] = v[i];
      const int e = e0 + sr;
      float u[8] = {};
      if (e < a.E) {
        const float4 w0 = *reinterpret_cast<const float4*>(a.Wr + (size_t)e * a.H + k0 + sc8);
        const float4 w1 = *reinterpret_cast<const float4*>(a.Wr + (size_t)e * a.H + k0 + sc8 + 4);
        u[0] = w0.x; u[1] = w0.y; u[2] = w0.z; u[3] = w0.w;
        u[4] = w1.x; u[5] = w1.y; u[6] = w1.z; u[7] = w1.w;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sw[sc8 + i][sr] = u[i];
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < LK; ++c) {
      const float4 xv = *reinterpret_cast<const float4*>(&sx[c][tt]);
      const float4 wv = *reinterpret_cast<const float4*>(&sw[c][te]);
      const double xd[4] = {xv.x, xv.y, xv.z, xv.w};
      const double wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(xd[i], wd[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* zp = a.z + (size_t)blockIdx.z * a.T * a.E;
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tt + i;
    if (t >= a.T) continue;
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + te + j;
      if (e < a.E) zp[(size_t)t * a.E + e] = acc[i][j];
    }
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
  topk_any<false>(a.z + (size_t)t * a.E, a.E, a.k, a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k,
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
    atomicOr(&s_mask[a.topk_idx[(size_t)t * a.k + i % a.k]], 1u << (i / a.k));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.ucnt[(size_t)c * a.E + e] = __popc(s_mask[e]);
}

// Pass 2 (one block of 1024 threads): per-expert prefix over chunks, then
// the prefix over experts gives the union arrays and each (chunk, expert)
// base offset.
__global__ __launch_bounds__(1024) void k_union_scan(RouteArgs a) {
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_pre[kMaxExperts];
  __shared__ int s_prs[kMaxExperts];
  __shared__ const uint8_t* s_ptr[kMaxExperts];
  const int tid = threadIdx.x;
  if (a.slots)
    for (int e = tid; e < a.E; e += blockDim.x) s_ptr[e] = (const uint8_t*)a.experts[e];
  // pass 1: per-expert totals (16 independent loads in flight per thread)
  for (int e = tid; e < a.E; e += blockDim.x) {
    int run = 0;
    for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (c0 + i < a.n_chunks) ? a.ucnt[(size_t)(c0 + i) * a.E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) run += v[i];
    }
    s_tot[e] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, nu = 0;
    for (int e = 0; e < a.E; ++e) {
      s_pre[e] = off;
      s_prs[e] = nu;
      if (s_tot[e] > 0) {
        a.uniq_ids[nu] = e;
        a.uniq_off[nu] = off;
        if (a.slots) {
          SlotEntry sl;
          sl.base = s_ptr[e];
          sl.n = s_tot[e];
          sl.p0 = off;
          a.slots[a.S + nu] = sl;
        }
        ++nu;
      }
      off += s_tot[e];
    }
    *a.n_unique = nu;
    a.uniq_off[nu] = off;
    s_prs[0] = nu;
    if (a.slots && a.S) write_slot(a, 0, -1, a.T, -1);
    if (a.tiles) {
      // grouped-GEMM tiles: shared expert first, then the union in order
      int nt = 0;
      if (a.S)
        for (int m0 = 0; m0 < a.T; m0 += kPrefillTileRows) {
          a.tiles[2 * nt] = 0;
          a.tiles[2 * nt + 1] = m0;
          ++nt;
        }
      int u = 0;
      for (int e = 0; e < a.E; ++e) {
        if (s_tot[e] == 0) continue;
        for (int m0 = 0; m0 < s_tot[e]; m0 += kPrefillTileRows) {
          a.tiles[2 * nt] = a.S + u;
          a.tiles[2 * nt + 1] = m0;
          ++nt;
        }
        ++u;
      }
      *a.n_tiles = nt;
    }
  }
  __syncthreads();
  if (a.slots)
    for (int sl = a.S + s_prs[0] + tid; sl < a.slots_max; sl += blockDim.x) write_slot(a, sl, 0, 0, 0);
  __syncthreads();
  // pass 2: base of each (chunk, expert) = expert base + earlier chunks' counts
  for (int e = tid; e < a.E; e += blockDim.x) {
    int run = s_pre[e];
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
    atomicOr(&s_mask[a.topk_idx[(size_t)t * a.k + i % a.k]], 1u << (i / a.k));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * a.k; i += blockDim.x) {
    const int tl = i / a.k;
    const int t = t0 + tl;
    const int e = a.topk_idx[(size_t)t * a.k + i % a.k];
    const int rank = __popc(s_mask[e] & ((1u << tl) - 1u));
    a.pairs[a.ubase[(size_t)c * a.E + e] + rank] = t * a.k + i % a.k;
  }
}

// Zero a counter range (used on the large-batch path, where no route kernel
// runs a last-block step).
__global__ void k_zero_u32(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_route(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                        const Route& r, bool with_slots, uint32_t* zero_from, size_t zero_count, hipStream_t s) {
  RouteArgs a{};
  a.Wr = w.router_w;
  a.b = w.router_b;
  a.x = x;
  a.T = p.T;
  a.H = p.H;
  a.E = p.E;
  a.k = p.k;
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
  a.zero_from = zero_from;
  a.zero_count = (int)zero_count;
  a.n_chunks = (p.T + 31) / 32;
  a.S = p.S;
  a.slots = with_slots ? r.slots : nullptr;
  a.tiles = with_slots ? r.tiles : nullptr;
  a.n_tiles = r.n_tiles;
  a.slots_max = p.slots_max;
  a.experts = w.experts;
  a.shared = w.shared;
  if (p.T <= kRouteSmallMaxTokens) {
    hipLaunchKernelGGL(k_route_small, dim3(p.E), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (zero_count > 0) {
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((zero_count + 255) / 256)), dim3(256), 0, s, zero_from,
                       (int)zero_count);
  }
  {
    RouteArgs b = a;
    b.z = r.z + (size_t)p.T * p.E;  // K-split partials live after z
    hipLaunchKernelGGL(k_logits_tiled, dim3((p.T + LT - 1) / LT, (p.E + LE - 1) / LE, kLogitSplit), dim3(256), 0, s, b);
    const size_t n = (size_t)p.T * p.E;
    hipLaunchKernelGGL(k_logits_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(k_topk, dim3((p.T + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_count, dim3(a.n_chunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(k_union_scatter, dim3(a.n_chunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
