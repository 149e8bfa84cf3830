// Tiered expert residency (include/moe_tier.h): per layer, a cache of HBM
// expert slots (LRU, or the most used experts) in front of pinned host
// copies that the GPU reads over PCIe when an expert is not resident.  The split between GPU memory and
// pinned system memory read directly by the GPU, and the look-ahead loads,
// follow the Ornith engine ("GTX 1070向け35BパラメータMoEモデル推論エンジン公開",
// 648news.com, section "VRAMとシステムメモリで重みを分割する設計"); the cache per
// layer with LRU replacement and the asynchronous expert loads follow the
// Colibrì engine ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
// hakusoku.com, sections "Colibrì: 消費者PCで…" and 実装済み機能).
#include <new>
#include <vector>

#include "common.h"
#include "moe_tier.h"

namespace moe {
namespace {

// One table entry, written by one thread with an ordinary vector store.
__global__ void k_table_write(const void** entry, const void* value) { *entry = value; }

// Promotion copy, pinned host memory -> HBM slot, by the GPU itself: its
// reads over PCIe run faster than the copy engine's here (measured), and
// they are the same reads the layer makes from host memory.
constexpr int kCopyBlocks = 512;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_promote_copy(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                     size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)kCopyBlocks * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace
}  // namespace moe

struct moe_tier {
  moe_dims_t d;
  int L = 0, E = 0, C = 0;
  size_t pb = 0;                   // bytes of one packed expert
  bool dry = true;
  std::vector<const void*> hdev;   // [L*E] device addresses of the host copies
  uint8_t* slots = nullptr;
  const void** table = nullptr;
  hipStream_t copy = nullptr;
  std::vector<int> slot_of;        // [L*E] slot within the layer, or -1
  std::vector<int> holder;         // [L*C] expert in the slot, or -1
  std::vector<uint64_t> stamp;     // [L*C] time of last use
  std::vector<uint64_t> seen;      // [E] call id that last saw the expert (deduplication)
  std::vector<float> count;        // [L*E] decayed use counts (MOE_TIER_HOT)
  uint64_t clock = 0, call = 0;
  int policy = MOE_TIER_LRU;
  std::vector<hipEvent_t> ev_ready, ev_free;  // [L*C]
  hipEvent_t ev_all = nullptr;     // copy stream, after the latest promotion
  moe_tier_stats_t st{};

  const void* slot_ptr(int l, int s) const { return slots + ((size_t)l * C + s) * pb; }

  int table_write(int l, int e, const void* v, hipStream_t s) {
    hipLaunchKernelGGL(moe::k_table_write, dim3(1), dim3(1), 0, s, table + (size_t)l * E + e, v);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
  }

  // The slot a promotion into layer l would take: a free one, else the
  // least recently used (LRU) or the least used (HOT) resident.
  int victim_slot(int l) const {
    int best = -1;
    for (int i = 0; i < C; ++i) {
      const int k = l * C + i;
      if (holder[k] < 0) return i;
      if (best < 0) {
        best = i;
        continue;
      }
      const int kb = l * C + best;
      if (policy == MOE_TIER_HOT) {
        const float ci = count[(size_t)l * E + holder[k]], cb = count[(size_t)l * E + holder[kb]];
        if (ci < cb || (ci == cb && stamp[k] < stamp[kb])) best = i;
      } else if (stamp[k] < stamp[kb]) {
        best = i;
      }
    }
    return best;
  }

  // Expert e of layer l into slot `best` of that layer, see moe_tier.h for
  // the ordering.
  int promote(int l, int e, int best, hipStream_t s) {
    const int k = l * C + best;
    const int victim = holder[k];
    if (victim >= 0) {
      slot_of[(size_t)l * E + victim] = -1;
      ++st.evictions;
      if (!dry) {
        if (hipStreamWaitEvent(s, ev_ready[k], 0) != hipSuccess) return MOE_E_HIP;
        if (table_write(l, victim, hdev[(size_t)l * E + victim], s) != MOE_OK) return MOE_E_HIP;
        if (hipEventRecord(ev_free[k], s) != hipSuccess) return MOE_E_HIP;
        if (hipStreamWaitEvent(copy, ev_free[k], 0) != hipSuccess) return MOE_E_HIP;
      }
    }
    holder[k] = e;
    stamp[k] = ++clock;
    slot_of[(size_t)l * E + e] = best;
    ++st.promotions;
    st.bytes_promoted += (int64_t)pb;
    if (!dry) {
      hipLaunchKernelGGL(moe::k_promote_copy, dim3(moe::kCopyBlocks), dim3(256), 0, copy,
                         (moe::u32x4*)slot_ptr(l, best), (const moe::u32x4*)hdev[(size_t)l * E + e], pb / 16);
      if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
      if (table_write(l, e, slot_ptr(l, best), copy) != MOE_OK) return MOE_E_HIP;
      if (hipEventRecord(ev_ready[k], copy) != hipSuccess) return MOE_E_HIP;
      if (hipEventRecord(ev_all, copy) != hipSuccess) return MOE_E_HIP;
    }
    return MOE_OK;
  }

  int visit(int l, const int32_t* experts, int n, bool use, hipStream_t s) {
    ++call;
    if (policy == MOE_TIER_HOT && use) {
      for (int e = 0; e < E; ++e) count[(size_t)l * E + e] *= 15.0f / 16.0f;
      for (int i = 0; i < n; ++i)
        if (seen[experts[i]] != call) {
          seen[experts[i]] = call;
          count[(size_t)l * E + experts[i]] += 1.0f;
        }
      ++call;
    }
    for (int i = 0; i < n; ++i) {
      const int e = experts[i];
      if (seen[e] == call) continue;
      seen[e] = call;
      const int sl = slot_of[(size_t)l * E + e];
      if (sl >= 0) {
        stamp[l * C + sl] = ++clock;
        if (use) ++st.hits;
        continue;
      }
      if (use) ++st.misses;
      else ++st.prefetched;
      if (C == 0) continue;
      const int v = victim_slot(l);
      if (policy == MOE_TIER_HOT && use && holder[l * C + v] >= 0 &&
          !(count[(size_t)l * E + e] > count[(size_t)l * E + holder[l * C + v]]))
        continue;  // not used more than the least used resident
      const int r = promote(l, e, v, s);
      if (r != MOE_OK) return r;
    }
    return MOE_OK;
  }
};

extern "C" {

int moe_tier_create(const moe_dims_t* d, int32_t n_layers, const void* const* host_experts, void* slots,
                    int32_t slots_per_layer, void* table, void* copy_stream, int32_t policy, moe_tier_t** out) {
  if (!out || !host_experts || n_layers < 1) return MOE_E_INVAL;
  if (policy != MOE_TIER_LRU && policy != MOE_TIER_HOT) return MOE_E_INVAL;
  const size_t pb = moe_packed_bytes(d);
  if (pb == 0) return MOE_E_INVAL;
  const int E = d->n_experts;
  if (slots_per_layer < 0 || slots_per_layer > E) return MOE_E_INVAL;
  const bool dry = !slots && !table && !copy_stream;
  if (!dry) {
    if (!table || !copy_stream || ((uintptr_t)table & 7u)) return MOE_E_INVAL;
    if (slots_per_layer > 0 && (!slots || ((uintptr_t)slots & 255u))) return MOE_E_INVAL;
  }
  const size_t n = (size_t)n_layers * E;
  std::vector<const void*> hdev(n);
  for (size_t i = 0; i < n; ++i) {
    const void* h = host_experts[i];
    if (!h || ((uintptr_t)h & 255u)) return MOE_E_INVAL;
    hdev[i] = h;
    if (!dry) {
      void* dp = nullptr;
      if (hipHostGetDevicePointer(&dp, const_cast<void*>(h), 0) != hipSuccess || !dp) {
        (void)hipGetLastError();  // clear the sticky error of the failed lookup
        return MOE_E_INVAL;
      }
      hdev[i] = dp;
    }
  }
  moe_tier* t = new (std::nothrow) moe_tier();
  if (!t) return MOE_E_HIP;
  t->d = *d;
  t->L = n_layers;
  t->E = E;
  t->C = slots_per_layer;
  t->pb = pb;
  t->dry = dry;
  t->hdev = std::move(hdev);
  t->slots = (uint8_t*)slots;
  t->table = (const void**)table;
  t->copy = (hipStream_t)copy_stream;
  t->slot_of.assign(n, -1);
  t->holder.assign((size_t)n_layers * slots_per_layer, -1);
  t->stamp.assign((size_t)n_layers * slots_per_layer, 0);
  t->seen.assign(E, 0);
  t->count.assign(n, 0.0f);
  t->policy = policy;
  if (!dry) {
    const size_t ns = (size_t)n_layers * slots_per_layer;
    if (hipEventCreateWithFlags(&t->ev_all, hipEventDisableTiming) != hipSuccess) {
      moe_tier_destroy(t);
      return MOE_E_HIP;
    }
    t->ev_ready.assign(ns, nullptr);
    t->ev_free.assign(ns, nullptr);
    for (size_t i = 0; i < ns; ++i) {
      if (hipEventCreateWithFlags(&t->ev_ready[i], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&t->ev_free[i], hipEventDisableTiming) != hipSuccess) {
        moe_tier_destroy(t);
        return MOE_E_HIP;
      }
    }
    if (hipMemcpy(table, t->hdev.data(), n * sizeof(void*), hipMemcpyHostToDevice) != hipSuccess) {
      moe_tier_destroy(t);
      return MOE_E_HIP;
    }
  }
  *out = t;
  return MOE_OK;
}

int moe_tier_destroy(moe_tier_t* t) {
  if (!t) return MOE_E_INVAL;
  for (hipEvent_t e : t->ev_ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : t->ev_free)
    if (e) (void)hipEventDestroy(e);
  if (t->ev_all) (void)hipEventDestroy(t->ev_all);
  delete t;
  return MOE_OK;
}

static int tier_check(const moe_tier_t* t, int32_t layer, const int32_t* experts, int32_t n) {
  if (!t || layer < 0 || layer >= t->L || n < 0 || (n > 0 && !experts)) return MOE_E_INVAL;
  for (int32_t i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= t->E) return MOE_E_INVAL;
  return MOE_OK;
}

int moe_tier_use(moe_tier_t* t, int32_t layer, const int32_t* experts, int32_t n, void* stream) {
  const int r = tier_check(t, layer, experts, n);
  if (r != MOE_OK) return r;
  return t->visit(layer, experts, n, true, (hipStream_t)stream);
}

int moe_tier_prefetch(moe_tier_t* t, int32_t layer, const int32_t* experts, int32_t n, void* stream) {
  const int r = tier_check(t, layer, experts, n);
  if (r != MOE_OK) return r;
  return t->visit(layer, experts, n, false, (hipStream_t)stream);
}

int moe_tier_sync(moe_tier_t* t, void* stream) {
  if (!t) return MOE_E_INVAL;
  if (t->dry || !t->ev_all) return MOE_OK;
  return hipStreamWaitEvent((hipStream_t)stream, t->ev_all, 0) == hipSuccess ? MOE_OK : MOE_E_HIP;
}

int32_t moe_tier_slot(const moe_tier_t* t, int32_t layer, int32_t expert) {
  if (!t || layer < 0 || layer >= t->L || expert < 0 || expert >= t->E) return -1;
  return t->slot_of[(size_t)layer * t->E + expert];
}

int moe_tier_stats(const moe_tier_t* t, moe_tier_stats_t* out) {
  if (!t || !out) return MOE_E_INVAL;
  *out = t->st;
  return MOE_OK;
}

}  // extern "C"
