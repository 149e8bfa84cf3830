// Reference rates for the rooflines the benchmark reports beside the
// published peaks: what a plain streaming read and a pure matrix-core loop
// reach on this GPU.  Measurement support, not part of the layer.
#include "common.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadUnroll = 8;

// Every 16-byte vector of buf read once (non-temporal 128-bit loads, grid
// stride, kReadUnroll loads in flight per thread); the XOR of a thread's
// data goes to sink[thread] so that no load can be dropped.
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ buf, size_t n, uint32_t* sink) {
  const size_t nth = (size_t)gridDim.x * 256, tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  size_t i = tid;
  for (; i + (kReadUnroll - 1) * nth < n; i += kReadUnroll * nth) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * nth);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u];
  }
  for (; i < n; i += nth) x ^= __builtin_nontemporal_load(buf + i);
  sink[tid] = x.x ^ x.y ^ x.z ^ x.w;
}

constexpr int kMfmaChains = 16;

// Independent chains of v_mfma_f32_16x16x32_f16 (16 x 16 x 32 multiply-adds
// each) on register operands, `iters` rounds of kMfmaChains per wavefront;
// the accumulators' sum goes to sink[thread].
__global__ __launch_bounds__(512) void k_probe_mfma(uint32_t* sink, int iters) {
  const int tid = blockIdx.x * 512 + threadIdx.x;
  const _Float16 h = (_Float16)(1.0f + (threadIdx.x & 7) * 0x1p-10f);
  const half8_t a = {h, h, h, h, h, h, h, h}, b = {h, h, h, h, h, h, h, h};
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c].x + acc[c].y + acc[c].z + acc[c].w;
  sink[tid] = __builtin_bit_cast(uint32_t, s);
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || ((uintptr_t)sink & 3u) || (bytes & 15u) || blocks < 1)
    return MOE_E_INVAL;
  hipLaunchKernelGGL(moe::k_probe_read, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const moe::u32x4*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_probe_mfma(uint32_t* sink, int32_t blocks, int32_t iters, void* stream) {
  if (!sink || ((uintptr_t)sink & 3u) || blocks < 1 || iters < 1) return MOE_E_INVAL;
  hipLaunchKernelGGL(moe::k_probe_mfma, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream, sink, iters);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // extern "C"
