// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_w4a16.h"

namespace moe {

// ---------------------------------------------------------------------------
// Packed device layout of one expert (written by moe_pack).
//
// Weights are stored in 1 KiB blocks ("chunks") of 64 rows x C columns,
// C = 128 / bits per code (16 for int8, 32 for the 4-bit formats, 64 for
// int2): lane l of a wavefront reads the 16 bytes at offset 16*l, which hold
// row l's C consecutive columns, so one 128-bit load per lane pulls one
// contiguous KiB.
//   GU region:  for rb in [0, I/64), c in [0, H/C): [gate block][up block]
//               (2 KiB per step, so gate row i and up row i sit in one lane)
//   D region:   for rb in [0, H/64), c in [0, I/C): [down block]
// Inside a lane's 16 bytes, dword m holds columns Cc + (C/4)m + (0..C/4-1),
// arranged so that masking the dword yields binary16 pairs of adjacent
// columns:
//   INT4_ROW: nibble position p (bits 4p..4p+3) holds column offset 2p
//     (p < 4) or 2(p-4)+1 (p >= 4), offset binary (q + 8): (d & 0x000F000F)
//     and (d & 0x00F000F0) each yield a pair of adjacent columns.
//   E2M1_B16: byte b of the dword holds columns 2b (low nibble) and 2b+1
//     (high nibble), codes unchanged.
//   INT8_ROW: bytes 0, 2 hold columns 0, 1 and bytes 1, 3 columns 2, 3,
//     offset binary (q + 128).
//   INT2_ROW: column 2j sits in bits 2j..2j+1 and column 2j+1 in bits
//     16+2j..17+2j (j = 0..7), offset binary (q + 2).
// Scales:
//   INT4_ROW, INT8_ROW, INT2_ROW: binary16 gate[I], up[I], down[H].
//   E2M1_B16: e4m3 block scales grouped per 4 chunks (128 columns): for the
//     GU region [rb][H/128][gate: 64 lanes x 8 B][up: 64 lanes x 8 B], for
//     the D region [rb][I/128][64 lanes x 8 B]; byte 2j / 2j+1 of a lane's
//     8 bytes scale columns 32j..32j+15 / 32j+16..32j+31 of the group;
//     then fp32 g[3] (gate, up, down).
// Every region starts on a 256-byte boundary.
// ---------------------------------------------------------------------------
struct Layout {
  size_t gu_off, d_off;        // weight regions
  size_t sg_off, su_off, sd_off;  // INT4_ROW scales
  size_t sgu_off, sdd_off;     // E2M1 block scales
  size_t g3_off;               // E2M1 tensor scales
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Bits per weight code, and whether the format has one binary16 scale per row.
constexpr int code_bits(int wfmt) { return wfmt == MOE_W_INT8_ROW ? 8 : wfmt == MOE_W_INT2_ROW ? 2 : 4; }
constexpr bool row_scaled(int wfmt) { return wfmt != MOE_W_E2M1_B16; }

inline Layout layout_of(const moe_dims_t& d) {
  Layout L{};
  const size_t H = (size_t)d.hidden, I = (size_t)d.inter, b = (size_t)code_bits(d.wfmt);
  size_t off = 0;
  L.gu_off = off; off = align256(off + 2 * I * H * b / 8);  // gate + up
  L.d_off = off;  off = align256(off + H * I * b / 8);
  if (row_scaled(d.wfmt)) {
    L.sg_off = off; off = align256(off + I * 2);
    L.su_off = off; off = align256(off + I * 2);
    L.sd_off = off; off = align256(off + H * 2);
  } else {
    L.sgu_off = off; off = align256(off + 2 * I * (H / 16));
    L.sdd_off = off; off = align256(off + H * (I / 16));
    L.g3_off = off;  off = align256(off + 3 * 4);
  }
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Workspace layout.  The first `sync` bytes hold completion counters that
// every kernel leaves at zero.
// ---------------------------------------------------------------------------
constexpr int kDecodeMaxTokens = 16;   // GEMV path for T <= this
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kPrefillTileRows = 64;   // tokens per gate/up grouped-GEMM tile
constexpr int kDownTileRows = 128;     // tokens per down grouped-GEMM tile
constexpr int kZPlanes = 9;            // fp64 logit planes: z, then up to 8 K-split partials

// Upper bound on grouped-GEMM tiles (slot, first token) of B tokens for T
// tokens.
inline int prefill_max_tiles(int T, int k, int E, int S, int B = kPrefillTileRows) {
  const long P = (long)T * k;
  const long U = P < E ? P : E;
  return (int)((S ? (T + B - 1) / B : 0) + (P + B - 1) / B + U);
}

struct Plan {
  int T, H, I, E, k, S;      // S = has_shared
  int slots_max;             // S + min(E, T*k)
  int rows_total;            // T*k + T: h / partial rows (pair rows then shared rows)
  int ks_gu, ks_sgu, ks_dn;  // split-K factors of the GEMV path (routed / shared gate/up, down)
  bool decode;               // GEMV path
  // counters (uint32), offsets in elements from ws base
  size_t c_route, c_gu, n_counters;
  size_t acc_off;            // byte offset of the decode output accumulators (uint64, in the sync region)
  size_t sync_bytes;
  // byte offsets
  size_t z_off, idx_off, w_off, nu_off, ids_off, off_off, pairs_off;
  size_t ucnt_off, ubase_off, tiles_off, tiles_dn_off, ntiles_off, slots_off;
  size_t h_off, p_gu_off, p_dn_off;
  size_t total;
};

bool make_plan(const moe_dims_t& d, int T, Plan* p);

// One expert slot of a call, written by the union step.  Slot 0 is the
// shared expert when there is one; the routed union follows in ascending
// expert order; slots past the realised union have n == 0.
struct SlotEntry {
  const uint8_t* base;  // packed expert
  int32_t n;            // tokens using it
  int32_t p0;           // first index into pairs, or -1 for the shared expert
};

// Device pointers resolved for one call.
struct Route {
  double* z;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_unique;
  int32_t* uniq_ids;
  int32_t* uniq_off;
  int32_t* pairs;
  int32_t* ucnt;    // union: per-chunk counts
  int32_t* ubase;   // union: per-chunk bases
  SlotEntry* slots; // [slots_max]
  int32_t* tiles;    // [max tiles][2]: (slot, first token) of each gate/up tile (kPrefillTileRows tokens)
  int32_t* tiles_dn; // the same for down tiles (kDownTileRows tokens)
  int32_t* n_tiles;  // [2]: gate/up tiles, down tiles
  uint32_t* counter;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_pack(const moe_dims_t& d, const void* qg, const void* sg, const void* qu, const void* su,
                       const void* qd, const void* sd, const float* g3, void* out, hipStream_t s);
hipError_t launch_unpack(const moe_dims_t& d, const void* packed, void* qg, void* sg, void* qu, void* su,
                         void* qd, void* sd, float* g3, hipStream_t s);
// Routing and union.  With `with_slots`, also fills r.slots from w.experts
// and w.shared (moe_w4a16_forward); moe_route passes false.
hipError_t launch_route(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                        const Route& r, bool with_slots, hipStream_t s, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_stop = nullptr);
// Optional stage events (benchmark timing): ev[2i] / ev[2i+1] take the
// start / end of stage i, recorded by the dispatch packets of the stage's
// first / last kernel (hipExtLaunchKernelGGL); null entries are skipped.
struct StageEvents {
  void* const* ev;
  int n;
  hipEvent_t start(int i) const { return (ev && 2 * i < n) ? (hipEvent_t)ev[2 * i] : nullptr; }
  hipEvent_t stop(int i) const { return (ev && 2 * i + 1 < n) ? (hipEvent_t)ev[2 * i + 1] : nullptr; }
};

// Kernel launch that optionally records events at the dispatch's start and
// end.
template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                     Args... args) {
  if (start || stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Routing and union for T <= kDecodeMaxTokens (moe_route): the router
// workgroups of the decode path's routing launch, without the slot table.
hipError_t launch_decode_route(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                               const Route& r, void* ws, hipStream_t s);
// The whole layer for T <= kDecodeMaxTokens in three launches: route +
// shared gate/up, routed gate/up, down (stages 0, 1, 2).
hipError_t launch_decode(const moe_dims_t& d, const Plan& p, const moe_weights_t& w, const uint16_t* x,
                         const Route& r, void* ws, uint16_t* y, hipStream_t s, const StageEvents& se);
hipError_t launch_prefill_experts(const moe_dims_t& d, const Plan& p, const moe_weights_t& w,
                                  const uint16_t* x, const Route& r, void* ws, uint16_t* y, hipStream_t s,
                                  const StageEvents& se);

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off without L2 maintenance.  The per-XCD L2 caches are
// not coherent with each other for ordinary stores, and a device-scope fence
// writes back and invalidates the whole L2.  Data handed between workgroups
// is therefore written and read with device-scope relaxed atomic accesses
// (st_dev / ld_dev, which bypass the XCD-private cache state and stay
// coherent across XCDs), and a unit publishes its arrival only after all of
// its stores have completed (s_waitcnt 0).  A reader issues its ld_dev loads
// only after the arrival that tells it the data is complete.  No plain load
// ever reads data written by another workgroup of the same launch.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every lane of a wavefront after its st_dev stores: returns the
// counter value before this wavefront's increment (same on all lanes).
__device__ __forceinline__ uint32_t publish_arrival(uint32_t* counter) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): our stores are done
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t prev = 0;
  if ((threadIdx.x & 63) == 0)
    prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);  // lane 0's value (all lanes are active)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return prev;
}

}  // namespace moe
