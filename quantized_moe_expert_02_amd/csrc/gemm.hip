// Prefill path (large batches): the experts of the batch union as grouped
// GEMMs on the fp16 matrix cores.
//
// Each unique expert is applied to all of its tokens at once (the batch-wise
// MoE union, "Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com,
// section 実装済み機能); its 4-bit weights are decoded once per tile into LDS
// as exact binary16 values (int4 codes are small integers; e2m1 x e4m3 has at
// most 6 significant bits) and multiplied on v_mfma_f32_16x16x32_f16 with
// fp32 accumulation.  Row scales (int4) or the tensor scale (e2m1) are applied
// in the epilogue, as is the SwiGLU.
//
//   k_gu_gemm:  tile = 64 tokens of one expert x 64 gate rows + 64 up rows
//               -> h (binary16, one row per (token, slot) pair)
//   k_dn_gemm:  tile = 64 tokens x 128 down rows -> per-pair fp32 outputs,
//               already multiplied by the pair's routing weight
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
constexpr int BK = 64;    // columns per K step (two 32-column chunks)
constexpr int LDS_PITCH = BK + 8;  // halves per LDS row (16-byte pad against bank conflicts)

struct GemmArgs {
  const SlotEntry* slots;
  const int32_t* pairs;
  const int32_t* tiles;      // [tile] = (slot, m0) pairs
  const int32_t* n_tiles;    // [1]
  const float* topk_w;
  const uint16_t* x;         // [T][H]
  uint16_t* h;               // [rows_total][I]
  float* part;               // [rows_total][H]
  uint16_t* y;               // [T][H]
  int T, H, I, k, S;
  int rows_total;
  Layout L;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// int4 (device order, offset binary) -> 8 consecutive binary16 values.
__device__ __forceinline__ u32x4 dequant_int4(uint32_t d) {
  const half2_t k1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t d8 = d >> 8;
  const half2_t p0 = as_h2((d & 0x000F000Fu) | 0x64006400u) + k1032;
  const half2_t p1 = as_h2((d & 0x00F000F0u) | 0x54005400u) + k72;
  const half2_t p2 = as_h2((d8 & 0x000F000Fu) | 0x64006400u) + k1032;
  const half2_t p3 = as_h2((d8 & 0x00F000F0u) | 0x54005400u) + k72;
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
               __builtin_bit_cast(uint32_t, p3)};
}

// e2m1 codes (byte b = columns 2b, 2b+1) times the block scale -> 8 binary16.
__device__ __forceinline__ u32x4 dequant_e2m1(uint32_t d, half2_t s) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s;
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
               __builtin_bit_cast(uint32_t, p3)};
}

__device__ __forceinline__ half2_t e4m3_half2(uint32_t byte) {
  const _Float16 h = (_Float16)__builtin_amdgcn_cvt_f32_fp8(byte, 0);
  return half2_t{h, h};
}

// Decodes this lane's 16 bytes of a 64-row x 32-column block (row `lane`) and
// stores the 32 binary16 values to LDS row `lane` at column offset `col`.
// E2M1: `sbytes` holds the row's two block scales of this chunk.
template <int FMT>
__device__ __forceinline__ void decode_to_lds(u32x4 w, uint32_t sbytes, _Float16* lds_row, int col) {
  u32x4 o[4];
  if (FMT == MOE_W_INT4_ROW) {
    o[0] = dequant_int4(w.x);
    o[1] = dequant_int4(w.y);
    o[2] = dequant_int4(w.z);
    o[3] = dequant_int4(w.w);
  } else {
    const half2_t s0 = e4m3_half2(sbytes & 0xFF), s1 = e4m3_half2((sbytes >> 8) & 0xFF);
    o[0] = dequant_e2m1(w.x, s0);
    o[1] = dequant_e2m1(w.y, s0);
    o[2] = dequant_e2m1(w.z, s1);
    o[3] = dequant_e2m1(w.w, s1);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(lds_row + col);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = o[i];
}

// E2M1 block-scale bytes of chunk c for row `lane`: two bytes of the lane's
// 8-byte group (see the packed layout).
__device__ __forceinline__ uint32_t e2m1_scale_pair(const uint8_t* sregion, size_t group_idx, int lane, int c) {
  const uint8_t* p = sregion + (group_idx * 64 + lane) * 8 + 2 * (c & 3);
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8);
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

// Gate/up: grid (I/64, max tiles); 256 threads = 4 waves; wave w owns gate
// and up rows 16w..16w+15 of the row block, all 64 tokens of the tile.
template <int FMT>
__global__ __launch_bounds__(256) void k_gu_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 sx[BM][LDS_PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sw[2][64][LDS_PITCH];
  __shared__ int s_act[BM], s_out[BM];
  const int tile = blockIdx.y;
  if (tile >= *a.n_tiles) return;
  const int slot = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const SlotEntry se = a.slots[slot];
  const int rb = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid & 63;
  if (tid < BM) {
    int ar = -1, orow = -1;
    if (!tile_token(a, se, m0 + tid, ar, orow)) ar = -1;
    s_act[tid] = ar;
    s_out[tid] = orow;
  }
  __syncthreads();
  const int n_ch = a.H / 32;
  const guint4* wbase = (const guint4*)(se.base + a.L.gu_off) + (size_t)rb * n_ch * 2 * 64 + lane;
  const uint8_t* sregion = se.base + a.L.sgu_off;
  f32x4 acc_g[4], acc_u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_g[i] = acc_u[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.H; k0 += BK) {
    // weights: wave w decodes chunk (k0/32 + w/2) of matrix w%2 (gate 0, up 1)
    {
      const int c = k0 / 32 + (wave >> 1), m = wave & 1;
      const u32x4 wv = __builtin_nontemporal_load(wbase + ((size_t)c * 2 + m) * 64);
      uint32_t sb = 0;
      if (FMT == MOE_W_E2M1_B16)
        sb = e2m1_scale_pair(sregion, ((size_t)rb * (a.H / 128) + c / 4) * 2 + m, lane, c);
      decode_to_lds<FMT>(wv, sb, &sw[m][lane][0], 32 * (wave >> 1));
    }
    // activations: 64 tokens x 64 columns, 16 bytes per thread x 2
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r;  // 0..511
      const int m = idx >> 3, q = idx & 7;
      const int ar = s_act[m];
      u32x4 v = {0, 0, 0, 0};
      if (ar >= 0) v = *reinterpret_cast<const u32x4*>(a.x + (size_t)ar * a.H + k0 + 8 * q);
      *reinterpret_cast<u32x4*>(&sx[m][8 * q]) = v;
    }
    __syncthreads();
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      const half8_t bg = *reinterpret_cast<const half8_t*>(&sw[0][16 * wave + n][kk + 8 * g]);
      const half8_t bu = *reinterpret_cast<const half8_t*>(&sw[1][16 * wave + n][kk + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const half8_t av = *reinterpret_cast<const half8_t*>(&sx[16 * mt + n][kk + 8 * g]);
        acc_g[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bg, acc_g[mt], 0, 0, 0);
        acc_u[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bu, acc_u[mt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // epilogue: lane holds tokens 16 mt + 4 g + i for weight row 16 wave + n
  const int n = lane & 15, g = lane >> 4;
  const int row = rb * 64 + 16 * wave + n;
  float sgv, suv;
  if (FMT == MOE_W_INT4_ROW) {
    sgv = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.sg_off)[row]);
    suv = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.su_off)[row]);
  } else {
    const float* g3 = reinterpret_cast<const float*>(se.base + a.L.g3_off);
    sgv = g3[0];
    suv = g3[1];
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * mt + 4 * g + i;
      const int orow = s_out[m];
      if (s_act[m] < 0) continue;
      const float gv = acc_g[mt][i] * sgv, uv = acc_u[mt][i] * suv;
      a.h[(size_t)orow * a.I + row] = __builtin_bit_cast(uint16_t, (_Float16)(silu(gv) * uv));
    }
  }
}

// Down: grid (H/128, max tiles); 256 threads = 4 waves; wave w owns down rows
// 32w..32w+31 of the 128-row tile (two 64-row blocks), all 64 tokens.
template <int FMT>
__global__ __launch_bounds__(256) void k_dn_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 sx[BM][LDS_PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sw[128][LDS_PITCH];
  __shared__ int s_out[BM];
  __shared__ float s_w[BM];
  const int tile = blockIdx.y;
  if (tile >= *a.n_tiles) return;
  const int slot = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const SlotEntry se = a.slots[slot];
  const int nb = blockIdx.x;  // 128-row tile
  const int tid = threadIdx.x, wave = tid / 64, lane = tid & 63;
  if (tid < BM) {
    int ar = -1, orow = -1;
    const bool ok = tile_token(a, se, m0 + tid, ar, orow);
    s_out[tid] = ok ? orow : -1;
    s_w[tid] = ok ? (se.p0 < 0 ? 1.0f : a.topk_w[orow]) : 0.0f;
  }
  __syncthreads();
  const int n_ch = a.I / 32;
  const guint4* wbase = (const guint4*)(se.base + a.L.d_off) + lane;
  const uint8_t* sregion = se.base + a.L.sdd_off;
  f32x4 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.I; k0 += BK) {
    // weights: wave w decodes row block (2 nb + w/2), chunk (k0/32 + w%2)
    {
      const int rb = 2 * nb + (wave >> 1), c = k0 / 32 + (wave & 1);
      const u32x4 wv = __builtin_nontemporal_load(wbase + ((size_t)rb * n_ch + c) * 64);
      uint32_t sb = 0;
      if (FMT == MOE_W_E2M1_B16) sb = e2m1_scale_pair(sregion, (size_t)rb * (a.I / 128) + c / 4, lane, c);
      decode_to_lds<FMT>(wv, sb, &sw[64 * (wave >> 1) + lane][0], 32 * (wave & 1));
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + 256 * r;
      const int m = idx >> 3, q = idx & 7;
      const int orow = s_out[m];
      u32x4 v = {0, 0, 0, 0};
      if (orow >= 0) v = *reinterpret_cast<const u32x4*>(a.h + (size_t)orow * a.I + k0 + 8 * q);
      *reinterpret_cast<u32x4*>(&sx[m][8 * q]) = v;
    }
    __syncthreads();
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      half8_t b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const half8_t*>(&sw[32 * wave + 16 * j + n][kk + 8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const half8_t av = *reinterpret_cast<const half8_t*>(&sx[16 * mt + n][kk + 8 * g]);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[j], acc[j][mt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = nb * 128 + 32 * wave + 16 * j + n;
    float sd;
    if (FMT == MOE_W_INT4_ROW)
      sd = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(se.base + a.L.sd_off)[row]);
    else
      sd = reinterpret_cast<const float*>(se.base + a.L.g3_off)[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * g + i;
        const int orow = s_out[m];
        if (orow < 0) continue;
        a.part[(size_t)orow * a.H + row] = s_w[m] * (sd * acc[j][mt][i]);
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
  for (int j = 0; j < a.k; ++j) acc += a.part[((size_t)t * a.k + j) * a.H + c];
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
  const unsigned mt = (unsigned)prefill_max_tiles(p.T, p.k, p.E, p.S);
  se.record(1, s);
  if (d.wfmt == MOE_W_INT4_ROW)
    hipLaunchKernelGGL(k_gu_gemm<MOE_W_INT4_ROW>, dim3(p.I / 64, mt), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_gu_gemm<MOE_W_E2M1_B16>, dim3(p.I / 64, mt), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  se.record(2, s);
  if (d.wfmt == MOE_W_INT4_ROW)
    hipLaunchKernelGGL(k_dn_gemm<MOE_W_INT4_ROW>, dim3(p.H / 128, mt), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_dn_gemm<MOE_W_E2M1_B16>, dim3(p.H / 128, mt), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_combine, dim3((p.H + 255) / 256, p.T), dim3(256), 0, s, a);
  e = hipGetLastError();
  se.record(3, s);
  return e;
}

}  // namespace moe
