/*
 * moe_tier.h -- tiered expert residency for the MoE FFN layer of
 * moe_w4a16.h on one GPU.
 *
 * The pages keep the most-used experts in GPU memory, the rest in pinned
 * system memory that the GPU reads directly over PCIe, and load the next
 * layer's experts ahead of use ("GTX 1070向け35BパラメータMoEモデル推論エンジン
 * 公開", 648news.com, section "VRAMとシステムメモリで重みを分割する設計"); each
 * layer has its own LRU expert cache in front of a slower store, and expert
 * loads for the next block run asynchronously ("Show HN: 低速のコンピュータで
 * GLM 5.2を動かす方法", hakusoku.com, sections "Colibrì: 消費者PCで…" and
 * 実装済み機能).
 *
 * Here: every layer's packed experts live in pinned host memory (the lower
 * tier); each layer owns `slots_per_layer` expert slots in HBM (the upper
 * tier, a cache with one of the replacement policies below).  The manager keeps a device table [L][E] of expert
 * pointers: entry (l, e) points at the expert's HBM slot when it is
 * resident and at its pinned host copy otherwise, so
 *   moe_weights_t.experts = table + l * E
 * makes moe_w4a16_forward read resident experts from HBM and the others
 * straight from host memory over PCIe (no copy, no synchronisation).  Both
 * copies hold the same bytes, so the layer's output does not depend on
 * residency.
 *
 * Promotions (host -> HBM slot copies) run on the manager's copy stream.
 * Ordering, per slot s:
 *   - a victim's table entry is switched back to its host copy by a kernel
 *     on the caller's stream, after which an event lets the copy stream
 *     overwrite s: forward calls queued earlier on that stream have
 *     finished, and later ones read the host copy;
 *   - the new expert's entry is switched to s by a kernel on the copy
 *     stream after the copy, and a forward call that reads the entry in
 *     between reads the host copy, which holds the same bytes;
 *   - the caller's stream waits for the slot's previous promotion before it
 *     switches that entry back (so the two switches cannot swap order).
 * Forward calls that read a layer's table must be queued on the stream
 * passed to moe_tier_use / moe_tier_prefetch for that layer.
 *
 * This is the one place where the library allocates: the manager's host
 * bookkeeping and its HIP events (released by moe_tier_destroy).  Slots,
 * table and the pinned host copies are the caller's.  A manager is not
 * thread-safe; calls on one manager must come from one host thread.
 */
#ifndef MOE_TIER_H
#define MOE_TIER_H

#include <stddef.h>
#include <stdint.h>

#include "moe_w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_tier moe_tier_t;

/* Replacement policies.
 *   MOE_TIER_LRU: every reported miss is promoted into the layer's slots,
 *     evicting the least recently used expert (the per-layer LRU cache of
 *     the Colibrì engine).  Pair it with moe_tier_sync before the forward
 *     call to load missing experts before they are used.
 *   MOE_TIER_HOT: the layer keeps its most used experts: every report adds
 *     one to the reported experts' use counts after all of the layer's
 *     counts decay by a factor 15/16; a non-resident expert is promoted
 *     only into a free slot or when its count exceeds the lowest count among
 *     the residents (that expert is evicted).  Misses are read over PCIe
 *     (the Ornith engine's most-used experts in GPU memory, the rest read
 *     from pinned system memory). */
typedef enum { MOE_TIER_LRU = 0, MOE_TIER_HOT = 1 } moe_tier_policy_t;

typedef struct {
  int64_t hits;        /* experts resident in HBM when moe_tier_use reported them */
  int64_t misses;      /* experts that were read from host memory              */
  int64_t promotions;  /* host -> HBM copies enqueued (uses and prefetches)      */
  int64_t evictions;   /* resident experts replaced                             */
  int64_t prefetched;  /* promotions requested by moe_tier_prefetch             */
  int64_t bytes_promoted;
} moe_tier_stats_t;

/* Creates a manager for n_layers layers of d->n_experts routed experts.
 *   host_experts: (host) array [n_layers * n_experts] of packed experts
 *     (moe_pack layout, moe_packed_bytes(d) bytes each, 256-byte aligned) in
 *     pinned host memory that the GPU can read (hipHostMalloc); entry
 *     l * n_experts + e is expert e of layer l.
 *   slots: device buffer of n_layers * slots_per_layer * moe_packed_bytes(d)
 *     bytes, 256-byte aligned; layer l owns slots [l * slots_per_layer,
 *     (l + 1) * slots_per_layer).  slots_per_layer may be 0 (every expert
 *     is read from host memory).
 *   table: device buffer of n_layers * n_experts pointers (8-byte aligned),
 *     written by the manager; create fills it with the host copies and
 *     waits for that copy to finish.
 *   copy_stream: hipStream_t for promotions (not NULL).
 *   policy: a moe_tier_policy_t.
 * Dry mode: slots == NULL, table == NULL and copy_stream == NULL keep the
 * bookkeeping only (no HIP call at all; host_experts entries need only be
 * non-NULL) -- the replacement policy on its own, for traces and tests.
 * Returns MOE_OK and *out, MOE_E_INVAL for bad arguments (including a host
 * pointer that the GPU cannot map), MOE_E_HIP on a HIP failure. */
int moe_tier_create(const moe_dims_t* d, int32_t n_layers, const void* const* host_experts, void* slots,
                    int32_t slots_per_layer, void* table, void* copy_stream, int32_t policy, moe_tier_t** out);

/* Releases the manager (its events and host memory).  The caller makes
 * sure that no work it queued through the manager is still pending. */
int moe_tier_destroy(moe_tier_t* t);

/* Reports that a step of layer `layer` uses (or used) the n experts in
 * `experts` (host array, indices in [0, n_experts), repeats allowed):
 * resident ones count as hits and become most recently used; the others
 * count as misses and are promoted as the policy decides.  Kernels and waits
 * go onto `stream` (the stream of the layer's forward calls) and the copy
 * stream; nothing synchronises. */
int moe_tier_use(moe_tier_t* t, int32_t layer, const int32_t* experts, int32_t n, void* stream);

/* Promotes experts ahead of use (the next-layer prefetch): like
 * moe_tier_use, but resident experts are only refreshed and nothing counts
 * as a hit or a miss. */
int moe_tier_prefetch(moe_tier_t* t, int32_t layer, const int32_t* experts, int32_t n, void* stream);

/* Makes `stream` wait until every promotion enqueued so far has been copied
 * and switched in the table, so that forward calls queued afterwards read
 * those experts from HBM. */
int moe_tier_sync(moe_tier_t* t, void* stream);

/* HBM slot index (within the layer) holding expert e of layer l, or -1 when
 * it is read from host memory (the manager's view: a promotion counts from
 * the moment it is enqueued). */
int32_t moe_tier_slot(const moe_tier_t* t, int32_t layer, int32_t expert);

int moe_tier_stats(const moe_tier_t* t, moe_tier_stats_t* out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TIER_H */
