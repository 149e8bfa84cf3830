// Host side of the C ABI declared in include/moe_w4a16.h: argument
// validation, workspace planning and kernel launches.  Nothing here
// allocates, copies or synchronises.
#include <string.h>

#include <mutex>
#include <new>

#include "common.h"

namespace moe {

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// Largest f <= fmax with (K/128) % f == 0, so every K-segment is a whole
// number of 128-column groups.
int split_factor(int K, int fmax) {
  const int g = K / 128;
  for (int f = fmax; f > 1; --f)
    if (g % f == 0) return f;
  return 1;
}

// Split of the shared expert's gate/up: up to 16 K-segments, in groups of
// four wavefronts (a split above 4 is a multiple of 4).
int shared_split(int K) {
  const int g = K / 128;
  for (int f = 16; f > 4; f -= 4)
    if (g % f == 0) return f;
  return split_factor(K, 4);
}

// Split of the routed experts' gate/up: four K-segments per workgroup, and
// more groups of four (partials handed to the last group) while the launch
// would hold fewer than kGuTargetWaves wavefronts for `slots` experts.  The
// split fixes the order of a token's sums, so it is taken for one token's
// slots at every batch size: a token's output bits do not depend on the
// batch it comes in.
constexpr int kGuTargetWaves = 1024;
int routed_split(int K, int I, int slots) {
  const int g = K / 128;
  int best = split_factor(K, 4);
  for (int f = 8; f <= 16; f += 4) {
    if ((long)slots * (I / 64) * best >= kGuTargetWaves) break;
    if (g % f == 0) best = f;
  }
  return best;
}

int check_dims(const moe_dims_t* d) {
  if (!d) return MOE_E_INVAL;
  if (d->n_experts < 1 || d->top_k < 1 || d->top_k > d->n_experts || d->hidden <= 0 || d->inter <= 0)
    return MOE_E_INVAL;
  if (d->has_shared != 0 && d->has_shared != 1) return MOE_E_INVAL;
  if (!(d->top_p >= 0.0f && d->top_p <= 1.0f)) return MOE_E_INVAL;  // NaN fails too
  if (d->wfmt < MOE_W_INT4_ROW || d->wfmt > MOE_W_INT2_ROW) return MOE_E_UNSUPPORTED;
  if (d->hidden % 128 || d->inter % 128) return MOE_E_UNSUPPORTED;
  if (d->n_experts > kMaxExperts || d->top_k > kMaxTopK) return MOE_E_UNSUPPORTED;
  if ((int64_t)d->hidden * d->inter > (int64_t)1 << 30) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

constexpr int32_t kMaxTokens = 1 << 20;

}  // namespace

bool make_plan(const moe_dims_t& d, int T, Plan* p) {
  Plan q{};
  q.T = T;
  q.H = d.hidden;
  q.I = d.inter;
  q.E = d.n_experts;
  q.k = d.top_k;
  q.S = d.has_shared;
  q.decode = T <= kDecodeMaxTokens;
  q.slots_max = q.S + (int)std::min<int64_t>(q.E, (int64_t)T * q.k);
  q.rows_total = T * q.k + T;
  // decode K-splits: one wavefront per K-segment, four per workgroup
  q.ks_gu = routed_split(q.H, q.I, std::min(q.E, q.k));  // routed experts
  q.ks_sgu = shared_split(q.H);    // shared expert, streamed while routing
  // down: 2 K-segments x 2 row blocks per workgroup; short rows (I <= 1024)
  // take 4 K-segments x 1 row block, or their launch holds too few
  // wavefronts (the segment count divides the 4 wavefronts of a workgroup)
  q.ks_dn = (q.I <= 1024 && (q.I / 128) % 4 == 0) ? 4 : split_factor(q.I, 2);
  // Counters: the first 256 words for route-stage counters, then one per
  // (slot, gate/up row block) for the largest decode batch; then the decode
  // output accumulators, one 64-bit word per output element of the largest
  // decode batch.  All of it starts at zero and every call leaves it so.
  const int slots_decode = q.S + std::min(q.E, kDecodeMaxTokens * q.k);
  q.c_route = 0;
  q.c_gu = 256;
  q.n_counters = q.c_gu + (size_t)slots_decode * (q.I / 64);
  q.acc_off = up256(q.n_counters * 4);
  q.sync_bytes = up256(q.acc_off + (size_t)kDecodeMaxTokens * q.H * 8);
  size_t off = q.sync_bytes;
  const size_t Tk = (size_t)T * q.k;
  const size_t cap = std::max<size_t>(1, std::min<size_t>(q.E, Tk));
  // z plus the K-split partial logits of the batched router
  q.z_off = off; off = up256(off + (size_t)T * q.E * 8 * kZPlanes);
  q.idx_off = off; off = up256(off + Tk * 4);
  q.w_off = off; off = up256(off + Tk * 4);
  q.nu_off = off; off = up256(off + 4);
  q.ids_off = off; off = up256(off + cap * 4);
  q.off_off = off; off = up256(off + (cap + 1) * 4);
  q.pairs_off = off; off = up256(off + std::max<size_t>(1, Tk) * 4);
  const size_t nch = ((size_t)T + 31) / 32;
  q.ucnt_off = off; off = up256(off + nch * q.E * 4);
  q.ubase_off = off; off = up256(off + nch * q.E * 4);
  q.tiles_off = off; off = up256(off + (size_t)prefill_max_tiles(T, q.k, q.E, q.S) * 8);
  q.tiles_dn_off = off; off = up256(off + (size_t)prefill_max_tiles(T, q.k, q.E, q.S, kDownTileRows) * 8);
  q.ntiles_off = off; off = up256(off + 8);
  q.slots_off = off; off = up256(off + (size_t)q.slots_max * sizeof(SlotEntry));
  q.h_off = off; off = up256(off + (size_t)q.rows_total * q.I * 2);
  if (q.decode) {
    const int groups = std::max(q.ks_sgu > 4 ? q.ks_sgu / 4 : 1, q.ks_gu > 4 ? q.ks_gu / 4 : 1);
    q.p_gu_off = off; off = up256(off + (size_t)groups * q.rows_total * 2 * q.I * 4);
    q.p_dn_off = 0;  // the down partials go straight into the output accumulators
  } else {
    q.p_gu_off = 0;
    q.p_dn_off = off; off = up256(off + (size_t)q.rows_total * q.H * 4);
  }
  q.total = off;
  *p = q;
  return true;
}

}  // namespace moe

using namespace moe;

namespace {

Route route_ptrs(const Plan& p, void* ws) {
  char* b = (char*)ws;
  Route r{};
  r.z = (double*)(b + p.z_off);
  r.topk_idx = (int32_t*)(b + p.idx_off);
  r.topk_w = (float*)(b + p.w_off);
  r.n_unique = (int32_t*)(b + p.nu_off);
  r.uniq_ids = (int32_t*)(b + p.ids_off);
  r.uniq_off = (int32_t*)(b + p.off_off);
  r.pairs = (int32_t*)(b + p.pairs_off);
  r.ucnt = (int32_t*)(b + p.ucnt_off);
  r.ubase = (int32_t*)(b + p.ubase_off);
  r.slots = (SlotEntry*)(b + p.slots_off);
  r.tiles = (int32_t*)(b + p.tiles_off);
  r.tiles_dn = (int32_t*)(b + p.tiles_dn_off);
  r.n_tiles = (int32_t*)(b + p.ntiles_off);
  r.counter = (uint32_t*)ws + p.c_route;
  return r;
}

int check_weights(const moe_dims_t* d, const moe_weights_t* w) {
  if (!w || !w->experts || !w->router_w) return MOE_E_INVAL;
  if (!aligned16(w->experts) || !aligned16(w->router_w) || (w->router_b && !aligned16(w->router_b)))
    return MOE_E_INVAL;
  if (d->has_shared ? (!w->shared || ((uintptr_t)w->shared & 255u)) : (w->shared != nullptr)) return MOE_E_INVAL;
  return MOE_OK;
}

// ---- scratch of moe_w4a16_forward_noalloc -----------------------------------
// A fixed array in the library's device code: every GPU the library runs on
// holds its own copy until the process ends.  Its host-side name is only a
// stand-in; the device address comes from hipGetSymbolAddress, once per
// device (with that device current), and is kept per device.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || ((uintptr_t)ptr & 255u)) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void k_zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

extern "C" {

size_t moe_packed_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return layout_of(*d).total;
}

size_t moe_workspace_sync_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  Plan p;
  make_plan(*d, 1, &p);
  return p.sync_bytes;
}

size_t moe_workspace_bytes(const moe_dims_t* d, int32_t T) {
  if (check_dims(d) != MOE_OK || T < 0 || T > kMaxTokens) return 0;
  Plan p;
  make_plan(*d, T, &p);
  return p.total;
}

int32_t moe_decode_max_tokens(void) { return kDecodeMaxTokens; }

int moe_pack(const moe_dims_t* d, const void* q_gate, const void* s_gate, const void* q_up, const void* s_up,
             const void* q_down, const void* s_down, const float* g3, void* packed_out, void* stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  const void* ps[] = {q_gate, s_gate, q_up, s_up, q_down, s_down, packed_out};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return MOE_E_INVAL;
  if (((uintptr_t)packed_out & 255u) || (g3 && ((uintptr_t)g3 & 3u))) return MOE_E_INVAL;
  if (launch_pack(*d, q_gate, s_gate, q_up, s_up, q_down, s_down, g3, packed_out, (hipStream_t)stream) !=
      hipSuccess)
    return MOE_E_HIP;
  return MOE_OK;
}

int moe_unpack(const moe_dims_t* d, const void* packed, void* q_gate, void* s_gate, void* q_up, void* s_up,
               void* q_down, void* s_down, float* g3, void* stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  const void* ps[] = {packed, q_gate, s_gate, q_up, s_up, q_down, s_down};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return MOE_E_INVAL;
  if (((uintptr_t)packed & 255u) || (g3 && ((uintptr_t)g3 & 3u))) return MOE_E_INVAL;
  if (launch_unpack(*d, packed, q_gate, s_gate, q_up, s_up, q_down, s_down, g3, (hipStream_t)stream) != hipSuccess)
    return MOE_E_HIP;
  return MOE_OK;
}

int moe_route(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T, int32_t* topk_idx,
              float* topk_w, int32_t* n_unique, int32_t* uniq_ids, int32_t* uniq_off, int32_t* pairs, void* ws,
              size_t ws_bytes, void* stream) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_E_INVAL;
  if (T > kMaxTokens) return MOE_E_UNSUPPORTED;
  if (!w || !w->router_w || !aligned16(w->router_w) || (w->router_b && !aligned16(w->router_b)))
    return MOE_E_INVAL;
  if (T == 0) return MOE_OK;
  const void* ps[] = {x, topk_idx, topk_w, n_unique, uniq_ids, uniq_off, pairs, ws};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return MOE_E_INVAL;
  Plan p;
  make_plan(*d, T, &p);
  if (ws_bytes < p.total) return MOE_E_WORKSPACE;
  Route r = route_ptrs(p, ws);
  r.topk_idx = topk_idx;
  r.topk_w = topk_w;
  r.n_unique = n_unique;
  r.uniq_ids = uniq_ids;
  r.uniq_off = uniq_off;
  r.pairs = pairs;
  const hipError_t e = p.decode ? launch_decode_route(*d, p, *w, x, r, ws, (hipStream_t)stream)
                               : launch_route(*d, p, *w, x, r, false, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

// Validation of a forward call (no launch); on success *p holds the plan.
static int forward_check(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T, uint16_t* y,
                         int32_t* topk_idx_out, float* topk_w_out, const void* ws, size_t ws_bytes, Plan* p) {
  int st = check_dims(d);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_E_INVAL;
  if (T > kMaxTokens) return MOE_E_UNSUPPORTED;
  st = check_weights(d, w);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const void* ps[] = {x, y, ws};
  for (const void* q : ps)
    if (!q || !aligned16(q)) return MOE_E_INVAL;
  if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out))) return MOE_E_INVAL;
  make_plan(*d, T, p);
  if (ws_bytes < p->total) return MOE_E_WORKSPACE;
  return MOE_OK;
}

// The layer's launches for a validated call.
static int forward_launch(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, uint16_t* y,
                          int32_t* topk_idx_out, float* topk_w_out, void* ws, hipStream_t s, const Plan& p,
                          const StageEvents& se) {
  Route r = route_ptrs(p, ws);
  if (topk_idx_out) r.topk_idx = topk_idx_out;
  if (topk_w_out) r.topk_w = topk_w_out;
  if (p.decode) return launch_decode(*d, p, *w, x, r, ws, y, s, se) == hipSuccess ? MOE_OK : MOE_E_HIP;
  if (launch_route(*d, p, *w, x, r, true, s, se.start(0), se.stop(0)) != hipSuccess) return MOE_E_HIP;
  return launch_prefill_experts(*d, p, *w, x, r, ws, y, s, se) == hipSuccess ? MOE_OK : MOE_E_HIP;
}

static int forward_impl(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T, uint16_t* y,
                        int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream,
                        const StageEvents& se) {
  Plan p;
  const int st = forward_check(d, w, x, T, y, topk_idx_out, topk_w_out, ws, ws_bytes, &p);
  if (st != MOE_OK || T == 0) return st;
  return forward_launch(d, w, x, y, topk_idx_out, topk_w_out, ws, (hipStream_t)stream, p, se);
}

int moe_w4a16_forward(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T, uint16_t* y,
                      int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, w, x, T, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream, StageEvents{nullptr, 0});
}

int moe_w4a16_forward_profiled(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
                               uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                               void* stream, void* const* events, int32_t n_events) {
  if (n_events < 0 || n_events > 6 || (n_events > 0 && !events)) return MOE_E_INVAL;
  return forward_impl(d, w, x, T, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream,
                      StageEvents{events, n_events});
}

int moe_w4a16_forward_noalloc(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
                              uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  Plan p;
  // validated against a stand-in address (the scratch array is 256-byte
  // aligned): nothing touches the device before the call is known to be good
  const int st = forward_check(d, w, x, T, y, topk_idx_out, topk_w_out, (const void*)(uintptr_t)256,
                               kNoAllocScratchBytes, &p);
  if (st != MOE_OK || T == 0) return st;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return MOE_E_HIP;
  const hipStream_t s = (hipStream_t)stream;
  // the completion counters must start at zero (a fill kernel, not a memset
  // node, so that the call can be captured in a graph)
  const size_t words = p.sync_bytes / 4;
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)std::min<size_t>((words + 255) / 256, 64)), dim3(256), 0, s,
                     (uint32_t*)ws, words);
  if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
  return forward_launch(d, w, x, y, topk_idx_out, topk_w_out, ws, s, p, StageEvents{nullptr, 0});
}

// ---- a decode step of several layers as one HIP graph ----------------------
struct moe_step_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int32_t n_layers;
};

int moe_step_graph_create(const moe_dims_t* d, int32_t n_layers, const moe_weights_t* w,
                          const uint16_t* const* x, int32_t T, uint16_t* const* y, void* ws, size_t ws_bytes,
                          moe_step_graph_t* out) {
  if (!out || !w || !x || !y) return MOE_E_INVAL;
  if (n_layers < 1 || n_layers > MOE_STEP_GRAPH_MAX_LAYERS || T < 1) return MOE_E_INVAL;
  // every layer validated before anything touches the device
  Plan p;
  for (int l = 0; l < n_layers; ++l) {
    const int st = forward_check(d, &w[l], x[l], T, y[l], nullptr, nullptr, ws, ws_bytes, &p);
    if (st != MOE_OK) return st;
  }
  // captured on a stream of the library's own (default priority), so that
  // nothing else the caller enqueues lands in the graph
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return MOE_E_HIP;
  int st = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) == hipSuccess ? MOE_OK : MOE_E_HIP;
  const bool capturing = st == MOE_OK;
  for (int l = 0; st == MOE_OK && l < n_layers; ++l)
    st = forward_launch(d, &w[l], x[l], y[l], nullptr, nullptr, ws, s, p, StageEvents{nullptr, 0});
  hipGraph_t g = nullptr;
  if (capturing && hipStreamEndCapture(s, &g) != hipSuccess) st = MOE_E_HIP;
  hipGraphExec_t ge = nullptr;
  if (st == MOE_OK && hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) st = MOE_E_HIP;
  moe_step_graph_s* h = nullptr;
  if (st == MOE_OK) {
    h = new (std::nothrow) moe_step_graph_s{g, ge, n_layers};
    if (!h) st = MOE_E_HIP;
  }
  (void)hipStreamDestroy(s);
  if (st != MOE_OK) {
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();  // the failure is reported through the status
    return st;
  }
  *out = h;
  return MOE_OK;
}

int moe_step_graph_launch(moe_step_graph_t g, void* stream) {
  if (!g) return MOE_E_INVAL;
  return hipGraphLaunch(g->exec, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int moe_step_graph_destroy(moe_step_graph_t g) {
  if (!g) return MOE_OK;
  const bool ok = hipGraphExecDestroy(g->exec) == hipSuccess && hipGraphDestroy(g->graph) == hipSuccess;
  delete g;
  return ok ? MOE_OK : MOE_E_HIP;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_E_INVAL: return "MOE_E_INVAL: invalid argument (null or misaligned pointer, bad size or T)";
    case MOE_E_UNSUPPORTED: return "MOE_E_UNSUPPORTED: shape or format outside the supported set";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_E_HIP: return "MOE_E_HIP: a kernel launch failed";
    default: return "unknown moe status";
  }
}

}  // extern "C"
