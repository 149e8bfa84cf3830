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
  int T, H, E, k;
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
  int chunk_tokens;
  int n_chunks;
};

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
  return __shfl_xor(v, m, kWave);
}

// (value, index) ordering of the router: larger logit first, then lower index.
__device__ __forceinline__ bool better(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Top-k of one token's logits by one wavefront: k rounds of a wave-wide
// argmax over the experts not yet taken.  Writes idx/w for slots 0..k-1 and,
// if `slot_expert` is non-null, the chosen experts to it.
__device__ void topk_wave(const double* zrow, int E, int k, int32_t* idx_out, float* w_out, int* slot_expert) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kPer = kMaxExperts / kWave;  // 16 values per lane at most
  double v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    v[i] = (e < E) ? zrow[e] : 0.0;
    if (e >= E) taken |= 1u << i;
  }
  double my_z = 0.0;
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + i * kWave;
      if (!(taken >> i & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const double ov = shfl_xor_d(bv, m);
      const int oi = __shfl_xor(bi, m, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_z = bv;
      my_e = bi;
    }
  }
  // s_j = sigmoid(z_j); w_j = s_j / sum_j s_j  (sum by a fixed butterfly).
  double s = (lane < k) ? 1.0 / (1.0 + exp(-my_z)) : 0.0;
  double tot = s;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) tot += shfl_xor_d(tot, m);
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = (float)(s / tot);
    if (slot_expert) slot_expert[lane] = my_e;
  }
}

// fp64 logits of one expert for all T (<= kRouteSmallMaxTokens) tokens by
// one wavefront; lane l covers columns 4l + 256i.
__device__ void logits_wave(const RouteArgs& a, int e) {
  const int lane = threadIdx.x & (kWave - 1);
  double acc[kRouteSmallMaxTokens];
#pragma unroll
  for (int t = 0; t < kRouteSmallMaxTokens; ++t) acc[t] = 0.0;
  const float4* wr = reinterpret_cast<const float4*>(a.Wr + (size_t)e * a.H);
  const int n4 = a.H / 4;
  for (int c4 = lane; c4 < n4; c4 += kWave) {
    const float4 w = wr[c4];
#pragma unroll
    for (int t = 0; t < kRouteSmallMaxTokens; ++t) {
      if (t < a.T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(a.x + (size_t)t * a.H + 4 * c4);
        const _Float16 x0 = __builtin_bit_cast(_Float16, (uint16_t)(xv.x & 0xFFFF));
        const _Float16 x1 = __builtin_bit_cast(_Float16, (uint16_t)(xv.x >> 16));
        const _Float16 x2 = __builtin_bit_cast(_Float16, (uint16_t)(xv.y & 0xFFFF));
        const _Float16 x3 = __builtin_bit_cast(_Float16, (uint16_t)(xv.y >> 16));
        double s = acc[t];
        s = fma((double)x0, (double)w.x, s);
        s = fma((double)x1, (double)w.y, s);
        s = fma((double)x2, (double)w.z, s);
        s = fma((double)x3, (double)w.w, s);
        acc[t] = s;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouteSmallMaxTokens; ++t) {
    if (t < a.T) {
      double v = acc[t];
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) v += shfl_xor_d(v, m);
      if (lane == 0) a.z[(size_t)t * a.E + e] = v + (a.b ? (double)a.b[e] : 0.0);
    }
  }
}

// Union of T*k pairs by one workgroup, using per-expert token bitmasks:
// the rank of pair (t, j) among the pairs of its expert is the number of
// earlier tokens that chose the same expert.  Requires T <= 32.
__device__ void union_small(const RouteArgs& a, const int* s_pe, uint32_t* s_mask, int* s_base, int* s_scan) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int P = a.T * a.k;
  for (int e = tid; e < a.E; e += nt) s_mask[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) atomicOr(&s_mask[s_pe[p]], 1u << (p / a.k));
  __syncthreads();
  // Each thread owns a contiguous run of experts; a block-wide inclusive
  // scan of the per-run (present, count) totals gives every run its base.
  const int per = (a.E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(a.E, e0 + per);
  int my_present = 0, my_count = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = __popc(s_mask[e]);
    my_present += c > 0;
    my_count += c;
  }
  s_scan[tid] = my_present;
  s_scan[nt + tid] = my_count;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    int vp = 0, vc = 0;
    if (tid >= off) {
      vp = s_scan[tid - off];
      vc = s_scan[nt + tid - off];
    }
    __syncthreads();
    s_scan[tid] += vp;
    s_scan[nt + tid] += vc;
    __syncthreads();
  }
  int up = s_scan[tid] - my_present;
  int uc = s_scan[nt + tid] - my_count;
  for (int e = e0; e < e1; ++e) {
    const int c = __popc(s_mask[e]);
    s_base[e] = uc;
    if (c > 0) {
      a.uniq_ids[up] = e;
      a.uniq_off[up] = uc;
      ++up;
    }
    uc += c;
  }
  if (tid == nt - 1) {
    *a.n_unique = s_scan[tid];
    a.uniq_off[s_scan[tid]] = s_scan[nt + tid];
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = s_pe[p];
    const int t = p / a.k;
    a.pairs[s_base[e] + __popc(s_mask[e] & ((1u << t) - 1u))] = p;
  }
}

// Decode-size routing in one launch: each wavefront computes one expert's
// logits for all tokens; the last workgroup to finish does the top-k and
// the union.  Grid: ceil(E / 4) blocks of 256 threads.
__global__ __launch_bounds__(256) void k_route_small(RouteArgs a) {
  __shared__ int s_pe[kRouteSmallMaxTokens * kMaxTopK];
  __shared__ uint32_t s_mask[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_scan[2 * 256];
  __shared__ int s_last;
  const int wave = threadIdx.x / kWave;
  const int e = blockIdx.x * 4 + wave;
  if (e < a.E) logits_wave(a, e);
  // Zero the completion counters that the expert kernels of this call use.
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.zero_count; i += gridDim.x * blockDim.x)
    a.zero_from[i] = 0;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(a.counter, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) *a.counter = 0;
  for (int t = wave; t < a.T; t += 4)
    topk_wave(a.z + (size_t)t * a.E, a.E, a.k, a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k,
              s_pe + t * a.k);
  __syncthreads();
  union_small(a, s_pe, s_mask, s_base, s_scan);
}

// ---- large batches -------------------------------------------------------

// fp64 logits, tiled: 32 tokens x 64 experts per 256-thread block; each
// thread owns 2 tokens x 4 experts.  Operands are staged in LDS as fp32
// (binary16 -> fp32 is exact) and widened to fp64 for the FMA.
constexpr int LT = 32, LE = 64, LK = 32;
__global__ __launch_bounds__(256) void k_logits_tiled(RouteArgs a) {
  __shared__ float sx[LK][LT + 4];
  __shared__ float sw[LK][LE + 4];
  const int t0 = blockIdx.x * LT, e0 = blockIdx.y * LE;
  const int tid = threadIdx.x;
  const int tt = (tid & 15) * 2;   // token offset in tile
  const int te = (tid >> 4) * 4;   // expert offset in tile
  double acc[2][4] = {};
  for (int k0 = 0; k0 < a.H; k0 += LK) {
    // x tile: 32 tokens x 32 columns = 1024 values, 4 per thread
    for (int i = tid; i < LT * LK; i += 256) {
      const int r = i / LK, c = i % LK;
      const int t = t0 + r;
      float v = 0.f;
      if (t < a.T) v = (float)__builtin_bit_cast(_Float16, a.x[(size_t)t * a.H + k0 + c]);
      sx[c][r] = v;
    }
    for (int i = tid; i < LE * LK; i += 256) {
      const int r = i / LK, c = i % LK;
      const int e = e0 + r;
      sw[c][r] = (e < a.E) ? a.Wr[(size_t)e * a.H + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < LK; ++c) {
      const double x0 = sx[c][tt], x1 = sx[c][tt + 1];
      const double w0 = sw[c][te], w1 = sw[c][te + 1], w2 = sw[c][te + 2], w3 = sw[c][te + 3];
      acc[0][0] = fma(x0, w0, acc[0][0]);
      acc[0][1] = fma(x0, w1, acc[0][1]);
      acc[0][2] = fma(x0, w2, acc[0][2]);
      acc[0][3] = fma(x0, w3, acc[0][3]);
      acc[1][0] = fma(x1, w0, acc[1][0]);
      acc[1][1] = fma(x1, w1, acc[1][1]);
      acc[1][2] = fma(x1, w2, acc[1][2]);
      acc[1][3] = fma(x1, w3, acc[1][3]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + tt + i;
    if (t >= a.T) continue;
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + te + j;
      if (e < a.E) a.z[(size_t)t * a.E + e] = acc[i][j] + (a.b ? (double)a.b[e] : 0.0);
    }
  }
}

// One wavefront per token.
__global__ __launch_bounds__(256) void k_topk(RouteArgs a) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= a.T) return;
  topk_wave(a.z + (size_t)t * a.E, a.E, a.k, a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k, nullptr);
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
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += blockDim.x) {
    int run = 0;
    for (int c = 0; c < a.n_chunks; ++c) {
      const int v = a.ucnt[(size_t)c * a.E + e];
      a.ubase[(size_t)c * a.E + e] = run;
      run += v;
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
        ++nu;
      }
      off += s_tot[e];
    }
    *a.n_unique = nu;
    a.uniq_off[nu] = off;
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += blockDim.x) {
    const int base = s_pre[e];
    for (int c = 0; c < a.n_chunks; ++c) a.ubase[(size_t)c * a.E + e] += base;
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
                        const Route& r, uint32_t* zero_from, size_t zero_count, hipStream_t s) {
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
  a.chunk_tokens = 32;
  a.n_chunks = (p.T + 31) / 32;
  if (p.T <= kRouteSmallMaxTokens) {
    hipLaunchKernelGGL(k_route_small, dim3((p.E + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (zero_count > 0) {
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((zero_count + 255) / 256)), dim3(256), 0, s, zero_from,
                       (int)zero_count);
  }
  hipLaunchKernelGGL(k_logits_tiled, dim3((p.T + LT - 1) / LT, (p.E + LE - 1) / LE), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_topk, dim3((p.T + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_count, dim3(a.n_chunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_union_scan, dim3(1), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(k_union_scatter, dim3(a.n_chunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
