// moe_pack / moe_unpack: canonical expert tensors <-> packed device layout.
// A bijective re-encoding of the codes (the layout is described in common.h); the
// converter role it plays is that of the offline FP8 -> int4 converter of the
// Colibrì engine ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
// hakusoku.com, section 実装済み機能), minus the quantisation itself.
#include "common.h"

namespace moe {
namespace {

// Device nibble position p holds canonical element kSrc[p] of the dword.
__device__ __forceinline__ uint32_t int4_to_device(uint32_t c) {
  uint32_t o = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int e = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
    o |= (((c >> (4 * e)) & 0xFu) ^ 0x8u) << (4 * p);
  }
  return o;
}

__device__ __forceinline__ uint32_t int4_from_device(uint32_t d) {
  uint32_t o = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int e = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
    o |= (((d >> (4 * p)) & 0xFu) ^ 0x8u) << (4 * e);
  }
  return o;
}

// int8: canonical bytes (columns 0, 1, 2, 3) -> device bytes (0, 2, 1, 3),
// offset binary.  The byte swap is its own inverse.
__device__ __forceinline__ uint32_t int8_swap(uint32_t c) {
  return (c & 0xFF0000FFu) | ((c & 0x0000FF00u) << 8) | ((c & 0x00FF0000u) >> 8);
}
__device__ __forceinline__ uint32_t int8_to_device(uint32_t c) { return int8_swap(c) ^ 0x80808080u; }
__device__ __forceinline__ uint32_t int8_from_device(uint32_t d) { return int8_swap(d ^ 0x80808080u); }

// int2: canonical column m at bits 2m -> device column 2j at bits 2j and
// column 2j+1 at bits 16+2j, offset binary (code ^ 2).
__device__ __forceinline__ int int2_pos(int m) { return (m & 1) * 16 + 2 * (m >> 1); }
__device__ __forceinline__ uint32_t int2_to_device(uint32_t c) {
  uint32_t o = 0;
#pragma unroll
  for (int m = 0; m < 16; ++m) o |= (((c >> (2 * m)) & 3u) ^ 2u) << int2_pos(m);
  return o;
}
__device__ __forceinline__ uint32_t int2_from_device(uint32_t d) {
  uint32_t o = 0;
#pragma unroll
  for (int m = 0; m < 16; ++m) o |= (((d >> int2_pos(m)) & 3u) ^ 2u) << (2 * m);
  return o;
}

__device__ __forceinline__ uint32_t to_device(int fmt, uint32_t c) {
  switch (fmt) {
    case MOE_W_INT4_ROW: return int4_to_device(c);
    case MOE_W_INT8_ROW: return int8_to_device(c);
    case MOE_W_INT2_ROW: return int2_to_device(c);
    default: return c;
  }
}
__device__ __forceinline__ uint32_t from_device(int fmt, uint32_t d) {
  switch (fmt) {
    case MOE_W_INT4_ROW: return int4_from_device(d);
    case MOE_W_INT8_ROW: return int8_from_device(d);
    case MOE_W_INT2_ROW: return int2_from_device(d);
    default: return d;
  }
}

struct PackArgs {
  const uint8_t* qg;
  const uint8_t* qu;
  const uint8_t* qd;
  uint8_t* qg_w;  // unpack outputs
  uint8_t* qu_w;
  uint8_t* qd_w;
  uint8_t* packed;
  const uint8_t* packed_r;
  int H, I, fmt, bits;
  size_t gu_off, d_off;
};

// 16-byte lane pieces of the GU and D regions.
inline int64_t gu_pieces(const moe_dims_t& d) { return (int64_t)d.inter * d.hidden * code_bits(d.wfmt) / 64; }
inline int64_t d_pieces(const moe_dims_t& d) { return (int64_t)d.hidden * d.inter * code_bits(d.wfmt) / 128; }

// One thread per 16-byte lane chunk of the GU and D regions.
template <bool kUnpack>
__global__ __launch_bounds__(256) void k_pack_weights(PackArgs a) {
  const int64_t n_gu = (int64_t)a.I * a.H * a.bits / 64;
  const int64_t n_d = (int64_t)a.H * a.I * a.bits / 128;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_gu + n_d) return;
  int64_t canon_off;
  size_t dev_off;
  int which;  // 0 gate, 1 up, 2 down
  if (i < n_gu) {
    const int64_t blk = i >> 6;
    const int lane = (int)(i & 63);
    const int64_t step = blk >> 1;
    which = (int)(blk & 1);
    const int64_t cpr = (int64_t)a.H * a.bits / 128;  // chunks per row
    const int64_t rb = step / cpr, c = step % cpr;
    canon_off = (rb * 64 + lane) * ((int64_t)a.H * a.bits / 8) + c * 16;
    dev_off = a.gu_off + (size_t)i * 16;
  } else {
    const int64_t j = i - n_gu;
    const int64_t blk = j >> 6;
    const int lane = (int)(j & 63);
    const int64_t cpr = (int64_t)a.I * a.bits / 128;
    const int64_t rb = blk / cpr, c = blk % cpr;
    which = 2;
    canon_off = (rb * 64 + lane) * ((int64_t)a.I * a.bits / 8) + c * 16;
    dev_off = a.d_off + (size_t)j * 16;
  }
  if (!kUnpack) {
    const uint8_t* src = (which == 0 ? a.qg : which == 1 ? a.qu : a.qd) + canon_off;
    uint4 v = *reinterpret_cast<const uint4*>(src);
    v.x = to_device(a.fmt, v.x);
    v.y = to_device(a.fmt, v.y);
    v.z = to_device(a.fmt, v.z);
    v.w = to_device(a.fmt, v.w);
    *reinterpret_cast<uint4*>(a.packed + dev_off) = v;
  } else {
    uint4 v = *reinterpret_cast<const uint4*>(a.packed_r + dev_off);
    v.x = from_device(a.fmt, v.x);
    v.y = from_device(a.fmt, v.y);
    v.z = from_device(a.fmt, v.z);
    v.w = from_device(a.fmt, v.w);
    uint8_t* dst = (which == 0 ? a.qg_w : which == 1 ? a.qu_w : a.qd_w) + canon_off;
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

struct ScaleArgs {
  const uint8_t* sg;
  const uint8_t* su;
  const uint8_t* sd;
  uint8_t* sg_w;
  uint8_t* su_w;
  uint8_t* sd_w;
  const float* g3;
  float* g3_w;
  uint8_t* packed;
  const uint8_t* packed_r;
  int H, I, fmt;
  Layout L;
};

// Row-scaled formats: one thread per binary16 scale.  E2M1_B16: one thread
// per 8-byte lane group of block scales (8 consecutive canonical scale bytes).
template <bool kUnpack>
__global__ __launch_bounds__(256) void k_pack_scales(ScaleArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row_scaled(a.fmt)) {
    const int64_t n = 2LL * a.I + a.H;
    if (i >= n) return;
    const uint16_t* src;
    uint16_t* dst;
    if (i < a.I) {
      src = kUnpack ? (const uint16_t*)(a.packed_r + a.L.sg_off) + i : (const uint16_t*)a.sg + i;
      dst = kUnpack ? (uint16_t*)a.sg_w + i : (uint16_t*)(a.packed + a.L.sg_off) + i;
    } else if (i < 2LL * a.I) {
      const int64_t r = i - a.I;
      src = kUnpack ? (const uint16_t*)(a.packed_r + a.L.su_off) + r : (const uint16_t*)a.su + r;
      dst = kUnpack ? (uint16_t*)a.su_w + r : (uint16_t*)(a.packed + a.L.su_off) + r;
    } else {
      const int64_t r = i - 2LL * a.I;
      src = kUnpack ? (const uint16_t*)(a.packed_r + a.L.sd_off) + r : (const uint16_t*)a.sd + r;
      dst = kUnpack ? (uint16_t*)a.sd_w + r : (uint16_t*)(a.packed + a.L.sd_off) + r;
    }
    *dst = *src;
    return;
  }
  const int64_t n_gu = (int64_t)a.I * a.H / 64;  // 8-byte groups, gate + up
  const int64_t n_d = (int64_t)a.H * a.I / 128;
  if (i == n_gu + n_d) {  // tensor scales
    for (int m = 0; m < 3; ++m) {
      if (kUnpack) {
        if (a.g3_w) a.g3_w[m] = ((const float*)(a.packed_r + a.L.g3_off))[m];
      } else {
        ((float*)(a.packed + a.L.g3_off))[m] = a.g3 ? a.g3[m] : 1.0f;
      }
    }
    return;
  }
  if (i > n_gu + n_d) return;
  int64_t canon_off;
  size_t dev_off;
  int which;
  if (i < n_gu) {
    const int64_t blk = i >> 6;  // 64 lanes per (rb, group, matrix)
    const int lane = (int)(i & 63);
    const int64_t step = blk >> 1;
    which = (int)(blk & 1);
    const int64_t gpr = a.H / 128;
    const int64_t rb = step / gpr, grp = step % gpr;
    canon_off = (rb * 64 + lane) * (a.H / 16) + grp * 8;
    dev_off = a.L.sgu_off + (size_t)i * 8;
  } else {
    const int64_t j = i - n_gu;
    const int64_t blk = j >> 6;
    const int lane = (int)(j & 63);
    const int64_t gpr = a.I / 128;
    const int64_t rb = blk / gpr, grp = blk % gpr;
    which = 2;
    canon_off = (rb * 64 + lane) * (a.I / 16) + grp * 8;
    dev_off = a.L.sdd_off + (size_t)j * 8;
  }
  if (!kUnpack) {
    const uint8_t* src = (which == 0 ? a.sg : which == 1 ? a.su : a.sd) + canon_off;
    *reinterpret_cast<uint2*>(a.packed + dev_off) = *reinterpret_cast<const uint2*>(src);
  } else {
    uint8_t* dst = (which == 0 ? a.sg_w : which == 1 ? a.su_w : a.sd_w) + canon_off;
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(a.packed_r + dev_off);
  }
}

inline unsigned blocks_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

}  // namespace

hipError_t launch_pack(const moe_dims_t& d, const void* qg, const void* sg, const void* qu, const void* su,
                       const void* qd, const void* sd, const float* g3, void* out, hipStream_t s) {
  const Layout L = layout_of(d);
  PackArgs a{};
  a.qg = (const uint8_t*)qg;
  a.qu = (const uint8_t*)qu;
  a.qd = (const uint8_t*)qd;
  a.packed = (uint8_t*)out;
  a.H = d.hidden;
  a.I = d.inter;
  a.fmt = d.wfmt;
  a.bits = code_bits(d.wfmt);
  a.gu_off = L.gu_off;
  a.d_off = L.d_off;
  const int64_t nw = gu_pieces(d) + d_pieces(d);
  hipLaunchKernelGGL(k_pack_weights<false>, dim3(blocks_for(nw, 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScaleArgs b{};
  b.sg = (const uint8_t*)sg;
  b.su = (const uint8_t*)su;
  b.sd = (const uint8_t*)sd;
  b.g3 = g3;
  b.packed = (uint8_t*)out;
  b.H = d.hidden;
  b.I = d.inter;
  b.fmt = d.wfmt;
  b.L = L;
  const int64_t ns = row_scaled(d.wfmt) ? 2LL * d.inter + d.hidden
                                              : (int64_t)d.inter * d.hidden / 64 + (int64_t)d.hidden * d.inter / 128 + 1;
  hipLaunchKernelGGL(k_pack_scales<false>, dim3(blocks_for(ns, 256)), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_unpack(const moe_dims_t& d, const void* packed, void* qg, void* sg, void* qu, void* su,
                         void* qd, void* sd, float* g3, hipStream_t s) {
  const Layout L = layout_of(d);
  PackArgs a{};
  a.qg_w = (uint8_t*)qg;
  a.qu_w = (uint8_t*)qu;
  a.qd_w = (uint8_t*)qd;
  a.packed_r = (const uint8_t*)packed;
  a.H = d.hidden;
  a.I = d.inter;
  a.fmt = d.wfmt;
  a.bits = code_bits(d.wfmt);
  a.gu_off = L.gu_off;
  a.d_off = L.d_off;
  const int64_t nw = gu_pieces(d) + d_pieces(d);
  hipLaunchKernelGGL(k_pack_weights<true>, dim3(blocks_for(nw, 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScaleArgs b{};
  b.sg_w = (uint8_t*)sg;
  b.su_w = (uint8_t*)su;
  b.sd_w = (uint8_t*)sd;
  b.g3_w = g3;
  b.packed_r = (const uint8_t*)packed;
  b.H = d.hidden;
  b.I = d.inter;
  b.fmt = d.wfmt;
  b.L = L;
  const int64_t ns = row_scaled(d.wfmt) ? 2LL * d.inter + d.hidden
                                              : (int64_t)d.inter * d.hidden / 64 + (int64_t)d.hidden * d.inter / 128 + 1;
  hipLaunchKernelGGL(k_pack_scales<true>, dim3(blocks_for(ns, 256)), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace moe
