// Wavefront-level helpers shared by the router kernels: DPP / permlane
// butterflies, order-preserving keys for fp64 logits, and the top-k of one
// token by one wavefront (k rounds of a wave-wide argmax).
#pragma once

#include "common.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxLogitParts = 5;  // partial-logit planes the workspace holds

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

// Every lane ends with the wave-wide fp32 sum, added as a pairwise tree
// (lanes 2i and 2i+1 first, then pairs of pairs, ...), the same on every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, partner<1>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, partner<2>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, partner<4>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, partner<8>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, partner<16>(__builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, partner<32>(__builtin_bit_cast(int, v)));
  return v;
}

// Every lane ends with the wave-wide fp64 sum, added in a fixed butterfly order.
__device__ __forceinline__ double wave_sum(double v) {
  v += partner_d<1>(v);
  v += partner_d<2>(v);
  v += partner_d<4>(v);
  v += partner_d<8>(v);
  v += partner_d<16>(v);
  v += partner_d<32>(v);
  return v;
}

// wave_sum of N values at once, the N butterflies interleaved step by step.
template <int N>
__device__ __forceinline__ void wave_sum_n(double (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<2>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<4>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<8>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<16>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += partner_d<32>(v[i]);
}

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Routing weights of the k ranked slots, slot j held by lane j (z: its fp64
// logit; lanes >= k hold nothing).  In fp64: s = sigmoid(z), w = s / sum(s)
// over the kept slots, rounded to fp32 at the end.  Adaptive expert top-p
// ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com, section
// 実行・チューニングパラメータ, the --topp option), for 0 < top_p < 1: the kept
// slots are the shortest prefix whose cumulative weight s_j / sum(s), summed
// in slot order, reaches top_p (the reading taken); the others are dropped.
// Returns the kept count m (k without top-p) and this lane's weight (0 for
// lanes >= m).
struct SlotWeight {
  int m;
  float w;
};
__device__ __forceinline__ SlotWeight slot_weights(double z, int k, float top_p) {
  const int lane = threadIdx.x & 63;
  const double s = lane < k ? 1.0 / (1.0 + exp(-z)) : 0.0;
  double tot = wave_sum(s);
  int m = k;
  if (top_p > 0.0f && top_p < 1.0f) {
    const double p = (double)top_p, w = s / tot;
    double cum = 0.0;
    for (int j = 0; j < k; ++j) {
      cum += readlane_d(w, j);
      if (cum >= p) {
        m = j + 1;
        break;
      }
    }
    if (m < k) tot = wave_sum(lane < m ? s : 0.0);
  }
  return SlotWeight{m, lane < m ? (float)(s / tot) : 0.0f};
}

// Inclusive prefix sum over the lanes (lane l gets v_0 + ... + v_l): row
// shifts within each row of 16 lanes, then the row broadcasts of lanes 15
// and 31 into the rows above.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Every lane ends with the wave-wide best (key, index): the largest key, ties
// to the lower index.  The high key word is reduced first; only when more than
// one lane holds that high word are the low word and the index reduced too.
__device__ __forceinline__ void wave_argmax_key(uint64_t& key, int& idx) {
  const uint32_t hi = (uint32_t)(key >> 32);
  const uint32_t hmax = wave_max_u32(hi);
  const uint64_t cand = __ballot(hi == hmax);
  if (__popcll(cand) == 1) {
    const int l = __ffsll((unsigned long long)cand) - 1;  // wave-uniform
    key = ((uint64_t)hmax << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, l);
    idx = __builtin_amdgcn_readlane(idx, l);
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
// The routing weights are formed by slot_weights (fp64).
// The logit of expert e is zrow[e], or with kCoherent the sum of nz partial
// logits zrow[s * zstride + e] (s ascending) plus bias[e] when bias is set.
template <int kPer, bool kCoherent>
__device__ void topk_wave(const double* zrow, int nz, size_t zstride, const float* bias, int E, int k, float top_p,
                          int32_t* idx_out, float* w_out, int* slot_expert) {
  // kCoherent: zrow holds partial logits written during this kernel by
  // other workgroups (published before this wavefront waited, and not read
  // before), and idx_out / w_out are read back by other workgroups of this
  // kernel, so they are written with device-coherent stores.
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t key[kPer];
  if (kCoherent) {
    // planes are loaded PG at a time, so that at most ~20 doubles per lane
    // are in flight
    constexpr int PG = kPer >= 20 ? 1 : (20 / kPer < kMaxLogitParts ? 20 / kPer : kMaxLogitParts);
    double v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = 0.0;
    for (int s0 = 0; s0 < nz; s0 += PG) {
      double zs[kPer][PG];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
#pragma unroll
        for (int s = 0; s < PG; ++s) {
          const int e = lane + i * kWave;
          if (e < E && s0 + s < nz) zs[i][s] = ld_dev(zrow + (s0 + s) * zstride + e);
        }
#pragma unroll
      for (int i = 0; i < kPer; ++i)
#pragma unroll
        for (int s = 0; s < PG; ++s)
          if (s0 + s < nz) v[i] += zs[i][s];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + i * kWave;
      if (bias && e < E) v[i] += (double)bias[e];
      key[i] = (e < E) ? order_key(v[i]) : 0ull;  // 0: below every finite key
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + i * kWave;
      key[i] = (e < E) ? order_key(zrow[e]) : 0ull;
    }
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
  const SlotWeight sw = slot_weights(from_order_key(my_key), k, top_p);
  if (lane < k) {
    const int32_t e_out = lane < sw.m ? my_e : -1;
    const float w = sw.w;
    if (kCoherent) {
      st_dev(idx_out + lane, e_out);
      st_dev(w_out + lane, w);
    } else {
      idx_out[lane] = e_out;
      w_out[lane] = w;
    }
    if (slot_expert) slot_expert[lane] = e_out;
  }
}

template <bool kCoherent>
__device__ void topk_any(const double* zrow, int nz, size_t zstride, const float* bias, int E, int k, float top_p,
                         int32_t* idx_out, float* w_out, int* slot_expert) {
  if (E <= 64) topk_wave<1, kCoherent>(zrow, nz, zstride, bias, E, k, top_p, idx_out, w_out, slot_expert);
  else if (E <= 128) topk_wave<2, kCoherent>(zrow, nz, zstride, bias, E, k, top_p, idx_out, w_out, slot_expert);
  else if (E <= 256) topk_wave<4, kCoherent>(zrow, nz, zstride, bias, E, k, top_p, idx_out, w_out, slot_expert);
  else if (E <= 512) topk_wave<8, kCoherent>(zrow, nz, zstride, bias, E, k, top_p, idx_out, w_out, slot_expert);
  else topk_wave<16, kCoherent>(zrow, nz, zstride, bias, E, k, top_p, idx_out, w_out, slot_expert);
}


// LDS scratch of one wavefront's top-k: the winner of round j writes its
// key and expert to slot j, and lane j reads them back after the rounds.
template <int NT>
struct RankSlots {
  uint64_t key[NT][kMaxTopK];
  int e[NT][kMaxTopK];
};

// Top-k of NT tokens at once by one wavefront (the NT rank searches are
// independent chains, so interleaving them hides their latency).  Same
// result as topk_wave per token.  Token t's logit of expert e is the sum of
// nz partial logits z[s * zstride + t * E + e] (s ascending) plus bias[e]
// when bias is set; partial logits were written by other workgroups of this
// kernel and published before this wavefront read them.  Each lane first
// sorts the kPer logits it holds (descending; equal logits keep ascending
// expert order), then each of the k rounds takes the wave-wide largest head
// (ties to the lower expert index): the lane holding it recognises itself
// from the wave-wide maximum, records it in slot j of rs and pops it, so a
// round's dependent chain is the reduction, one compare and the pop.
// Outputs are written with device-coherent stores: idx_out[t * k + j] and
// w_out[...] if idx_out is set, and slot_expert[t * k + j] (LDS) if set.
template <int kPer, int NT>
__device__ __forceinline__ void topk_multi(const double* z, int nz, size_t zstride, const float* bias, int E, int k,
                                           float top_p, int32_t* idx_out, float* w_out, int* slot_expert,
                                           RankSlots<NT>& rs) {
  const int lane = threadIdx.x & (kWave - 1);
  double v[NT][kPer];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[t][i] = 0.0;
  // all planes are requested at once (one memory latency), then added in
  // plane order
  constexpr int PG = kPer * NT * kMaxLogitParts <= 40 ? kMaxLogitParts : 1;
  for (int s0 = 0; s0 < nz; s0 += PG) {
    double zs[PG][NT][kPer];
#pragma unroll
    for (int s = 0; s < PG; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int e = lane + i * kWave;
          zs[s][t][i] = (e < E && s0 + s < nz) ? ld_dev(z + (s0 + s) * zstride + (size_t)t * E + e) : 0.0;
        }
#pragma unroll
    for (int s = 0; s < PG; ++s)
      if (s0 + s < nz) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < kPer; ++i) v[t][i] += zs[s][t][i];
      }
  }
  uint64_t key[NT][kPer];
  int idx[NT][kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    const double b = (bias && e < E) ? (double)bias[e] : 0.0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      key[t][i] = (e < E) ? order_key(bias ? v[t][i] + b : v[t][i]) : 0ull;  // 0: below every finite key
      idx[t][i] = e;
    }
  }
  // per-lane sort, descending; a swap only on a strictly larger key keeps
  // equal keys in ascending expert order
#pragma unroll
  for (int pass = 0; pass < kPer - 1; ++pass)
#pragma unroll
    for (int i = 0; i < kPer - 1 - pass; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool sw = key[t][i + 1] > key[t][i];
        const uint64_t k0 = key[t][i], k1 = key[t][i + 1];
        const int i0 = idx[t][i], i1 = idx[t][i + 1];
        key[t][i] = sw ? k1 : k0;
        key[t][i + 1] = sw ? k0 : k1;
        idx[t][i] = sw ? i1 : i0;
        idx[t][i + 1] = sw ? i0 : i1;
      }
  for (int j = 0; j < k; ++j) {
    uint32_t hmax[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) hmax[t] = wave_max_u32((uint32_t)(key[t][0] >> 32));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t hi = (uint32_t)(key[t][0] >> 32);
      bool win = hi == hmax[t];
      if (__popcll(__ballot(win)) != 1) {  // equal high words: compare the low words, then the expert index
        const uint32_t lo = (uint32_t)key[t][0];
        const uint32_t lmax = wave_max_u32(win ? lo : 0u);
        const bool c2 = win && (lo == lmax);
        const uint32_t best_inv = wave_max_u32(c2 ? ~(uint32_t)idx[t][0] : 0u);
        win = c2 && (uint32_t)idx[t][0] == ~best_inv;  // expert indices are distinct: one lane
      }
      if (win) {
        rs.key[t][j] = key[t][0];
        rs.e[t][j] = idx[t][0];
#pragma unroll
        for (int i = 0; i < kPer - 1; ++i) {
          key[t][i] = key[t][i + 1];
          idx[t][i] = idx[t][i + 1];
        }
        key[t][kPer - 1] = 0;
      }
    }
  }
  // this wavefront's LDS writes above complete before its reads below
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint64_t my_key[NT];
  int my_e[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    my_key[t] = lane < k ? rs.key[t][lane] : 0ull;
    my_e[t] = lane < k ? rs.e[t][lane] : -1;
  }
  // the weights are needed for the outputs, or to decide which slots top-p keeps
  const bool need_w = idx_out || (top_p > 0.0f && top_p < 1.0f);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const SlotWeight sw = need_w ? slot_weights(from_order_key(my_key[t]), k, top_p) : SlotWeight{k, 0.0f};
    if (lane < k) {
      const int32_t e_out = lane < sw.m ? my_e[t] : -1;
      if (idx_out) {
        st_dev(idx_out + t * k + lane, e_out);
        st_dev(w_out + t * k + lane, sw.w);
      }
      if (slot_expert) slot_expert[t * k + lane] = e_out;
    }
  }
}

// Top-k of T tokens (z, outputs and slot_expert indexed as in topk_multi),
// one token at a time (ranking several together gains little: the rounds
// are bound by instruction issue, not latency).
template <int kPer>
__device__ __forceinline__ void topk_tokens_per(const double* z, int nz, size_t zstride, const float* bias, int E,
                                                int k, float top_p, int T, int32_t* idx_out, float* w_out,
                                                int* slot_expert, RankSlots<1>& rs) {
  for (int t0 = 0; t0 < T; ++t0)
    topk_multi<kPer, 1>(z + (size_t)t0 * E, nz, zstride, bias, E, k, top_p, idx_out ? idx_out + t0 * k : nullptr,
                        w_out ? w_out + t0 * k : nullptr,
                        slot_expert + t0 * k, rs);
}

__device__ __forceinline__ void topk_tokens(const double* z, int nz, size_t zstride, const float* bias, int E, int k,
                                            float top_p, int T, int32_t* idx_out, float* w_out, int* slot_expert,
                                            RankSlots<1>& rs) {
  if (E <= 64) topk_tokens_per<1>(z, nz, zstride, bias, E, k, top_p, T, idx_out, w_out, slot_expert, rs);
  else if (E <= 128) topk_tokens_per<2>(z, nz, zstride, bias, E, k, top_p, T, idx_out, w_out, slot_expert, rs);
  else if (E <= 256) topk_tokens_per<4>(z, nz, zstride, bias, E, k, top_p, T, idx_out, w_out, slot_expert, rs);
  else if (E <= 512) topk_tokens_per<8>(z, nz, zstride, bias, E, k, top_p, T, idx_out, w_out, slot_expert, rs);
  else topk_tokens_per<16>(z, nz, zstride, bias, E, k, top_p, T, idx_out, w_out, slot_expert, rs);
}

}  // namespace moe
