/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) 4-bit-weight Mixture-of-Experts
 * FFN layer.
 *
 * The layer (one MoE FFN block of a large MoE language model):
 *   - weights are 4-bit and activations binary16 ("W4A16": INT4 weights with
 *     FP16 activations; "GLM-5.3-Flash 320B MoEを4枚のCMP 170HXで動かすvLLMレシピ",
 *     648news.com, section "OpenAI互換APIで動く320BパラメータのMoE構成").  Two
 *     weight formats: int4 with one scale per row ("Show HN: 低速のコンピュータで
 *     GLM 5.2を動かす方法", hakusoku.com, section 実装済み機能), and NVFP4-style
 *     e2m1 codes with block scales, decoded in registers inside the matmul
 *     ("GTX 1070向け35BパラメータMoEモデル推論エンジン公開", 648news.com, section
 *     "VRAMとシステムメモリで重みを分割する設計");
 *   - a DeepSeek-V3-style sigmoid router picks top_k of n_experts routed
 *     experts per token, and a shared expert is always added (hakusoku.com,
 *     section 実装済み機能);
 *   - the unique experts chosen across the batch are gathered once and each is
 *     applied to every token that chose it (hakusoku.com, section 実装済み機能,
 *     "batch-wise MoE union");
 *   - each expert is a SwiGLU FFN: h = silu(Wg x) * (Wu x), o = Wd h;
 *   - y[t] = sum_j w[t][j] * o_{e(t,j)} + o_shared, with w the sigmoid scores
 *     of the kept experts renormalised to sum to one.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *     allocates every buffer; the library never allocates or frees memory
 *     (except the graph handle of moe_step_graph_create) and keeps no global
 *     mutable state, so calls on different streams with different workspaces
 *     may run concurrently.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Each call validates its arguments on the host, enqueues its kernels and
 *     returns; outputs are valid once the stream has synchronised.  No call
 *     copies, synchronises or allocates, so every call can be captured in a
 *     HIP graph.
 *   - Validation happens before any launch; on failure the call returns a
 *     negative moe_status_t, launches nothing and leaves outputs untouched.
 *     No call prints or throws.
 *   - Inputs must be finite.  The same inputs give bitwise-identical outputs,
 *     and a token's outputs do not depend on the batch it comes in (decode
 *     batches, T <= 16): no floating-point atomics; reductions run in a
 *     fixed order, and the decode path adds each slot's routing-weighted
 *     down row into the output as an exact 64-bit fixed-point integer (29
 *     fraction bits), which any arrival order sums alike.  A decode output
 *     element to which some slot contributes 2^20 or more in magnitude is
 *     +-inf (NaN where such terms have both signs).
 *   - All device pointers must be 16-byte aligned; packed experts 256-byte.
 *   - The workspace must be zero-filled once before its first use (e.g.
 *     allocated with torch.zeros).  Its first moe_workspace_sync_bytes(d)
 *     bytes hold completion counters and the decode output accumulators,
 *     which every call leaves at zero again,
 *     so a zeroed workspace stays valid for any later call and any T, but
 *     two calls that overlap in time must not share one workspace.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_INVAL = -1,       /* null/misaligned pointer, bad size, T < 0, k > E ... */
  MOE_E_UNSUPPORTED = -2, /* shape or format outside the supported set          */
  MOE_E_WORKSPACE = -3,   /* ws_bytes < moe_workspace_bytes(d, T)               */
  MOE_E_HIP = -4          /* a kernel launch failed                              */
} moe_status_t;

typedef enum {
  /* int4 two's complement in [-8, 7]; one binary16 scale per output row:
   * W[r][c] = q[r][c] * s[r]. */
  MOE_W_INT4_ROW = 0,
  /* OCP FP4 E2M1 codes; one OCP FP8 E4M3 (FN) scale per 16 consecutive
   * weights along the row, and one fp32 tensor scale g per matrix:
   * W[r][c] = e2m1(q[r][c]) * e4m3(s[r][c/16]) * g. */
  MOE_W_E2M1_B16 = 1,
  /* int8 two's complement in [-128, 127], or int2 two's complement in
   * [-2, 1]; one binary16 scale per output row: W[r][c] = q[r][c] * s[r].
   * The int8/int2 kernels with per-row scales of the Colibrì engine
   * ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com,
   * section 実装済み機能). */
  MOE_W_INT8_ROW = 2,
  MOE_W_INT2_ROW = 3
} moe_wfmt_t;

/* Layer shape (host struct).  Supported: hidden and inter multiples of 128,
 * 1 <= top_k <= min(n_experts, 32), n_experts <= 1024, has_shared in {0,1},
 * wfmt a moe_wfmt_t. */
typedef struct {
  int32_t hidden;     /* H: model width                                  */
  int32_t inter;      /* I: expert intermediate width                    */
  int32_t n_experts;  /* E: routed experts                               */
  int32_t top_k;      /* k: routed experts kept per token                */
  int32_t has_shared; /* 1 if a shared expert is added to every token    */
  int32_t wfmt;       /* moe_wfmt_t                                      */
  float top_p;        /* adaptive expert top-p: 0 keeps all top_k slots;
                       * otherwise in (0, 1], see moe_route              */
} moe_dims_t;

/* Weights of one layer (host struct holding device pointers). */
typedef struct {
  /* DEVICE array of n_experts DEVICE pointers; entry e points to routed
   * expert e packed by moe_pack (moe_packed_bytes(d) bytes, 256-B aligned). */
  const void* const* experts;
  /* The packed shared expert; NULL iff has_shared == 0. */
  const void* shared;
  /* Router weights, fp32 [E][H] row-major. */
  const float* router_w;
  /* Router logit bias, fp32 [E], or NULL for none.  It is added to the
   * logits before the top-k and the sigmoid. */
  const float* router_b;
} moe_weights_t;

/* Bytes of one packed expert (gate, up, down and their scales). */
size_t moe_packed_bytes(const moe_dims_t* d);

/* Bytes of scratch memory that moe_route / moe_w4a16_forward need for T
 * tokens (see the zero-fill rule above).  Returns 0 for invalid dims. */
size_t moe_workspace_bytes(const moe_dims_t* d, int32_t T);

/* Bytes at the start of the workspace that hold completion counters. */
size_t moe_workspace_sync_bytes(const moe_dims_t* d);

/* Canonical expert -> packed device layout (a byte permutation; the values
 * are unchanged).  It plays the role of the offline weight converter of the
 * Colibrì engine ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
 * hakusoku.com, section 実装済み機能, the FP8 -> int4 offline conversion
 * tool), minus the quantisation: the codes and scales are given.  Run once
 * per expert when the weights are loaded, not per call.  Errors: MOE_E_INVAL
 * for a null or misaligned pointer (16 B; packed_out 256 B; g3 4 B),
 * MOE_E_UNSUPPORTED / MOE_E_INVAL for dims outside the supported set,
 * MOE_E_HIP if a launch fails.  Canonical inputs, all row-major on the device, with
 * b = 8 (INT8_ROW), 2 (INT2_ROW) or 4 (the others) bits per code:
 *   q_gate, q_up: uint8 [I][H*b/8]; q_down: uint8 [H][I*b/8];
 *     4-bit codes: element 2j in the low nibble of byte j, element 2j+1 in
 *     the high nibble; INT8_ROW: one byte per element; INT2_ROW: element
 *     4j+i in bits 2i..2i+1 of byte j;
 *   INT4_ROW, INT8_ROW, INT2_ROW: s_gate, s_up: binary16 [I]; s_down:
 *     binary16 [H]; g3 ignored;
 *   E2M1_B16: s_gate, s_up: uint8 E4M3 [I][H/16]; s_down: uint8 [H][I/16];
 *     g3: fp32 [3] tensor scales (gate, up, down), or NULL for 1.0.
 * packed_out receives moe_packed_bytes(d) bytes. */
int moe_pack(const moe_dims_t* d, const void* q_gate, const void* s_gate, const void* q_up,
             const void* s_up, const void* q_down, const void* s_down, const float* g3,
             void* packed_out, void* stream);

/* Inverse of moe_pack (for tests): writes the canonical tensors back.
 * g3 may be NULL. */
int moe_unpack(const moe_dims_t* d, const void* packed, void* q_gate, void* s_gate, void* q_up,
               void* s_up, void* q_down, void* s_down, float* g3, void* stream);

/* Router and batch union for T tokens (x: binary16 [T][H]).
 * Logits are accumulated in fp64: z[t][e] = b[e] + sum_h x[t][h]*Wr[e][h].
 * Experts are ranked by (z descending, index ascending); the first k are
 * kept in that order.  w[t][j] = sigmoid(z_j) / sum_j' sigmoid(z_j'),
 * formed in fp64 and rounded to fp32.
 * Adaptive expert top-p ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
 * hakusoku.com, section 実行・チューニングパラメータ, the --topp option), when
 * 0 < d->top_p < 1: only the shortest prefix of the k slots whose
 * cumulative weight (fp64, summed in slot order) reaches top_p is kept, and
 * the kept weights are renormalised over the kept slots; dropped slots get
 * topk_idx = -1 and topk_w = 0.
 * Batches of T <= moe_decode_max_tokens() are routed by the router
 * workgroups and the top-k code of the GEMV path of moe_w4a16_forward,
 * larger ones by the batched router of the grouped-GEMM path.
 * Outputs:
 *   topk_idx int32 [T][k], topk_w fp32 [T][k];
 *   n_unique int32 [1]: distinct experts chosen by the batch;
 *   uniq_ids int32 [min(E, T*k)]: those experts, ascending;
 *   uniq_off int32 [min(E, T*k) + 1]: uniq_off[u]..uniq_off[u+1] is expert
 *     u's range in pairs; uniq_off[n_unique] is the number of kept pairs;
 *   pairs int32 [T*k]: pair ids t*k + j of the kept slots, grouped by
 *     expert and in ascending token order within each group.
 * Entries past n_unique are unspecified.  T == 0 launches nothing and
 * returns MOE_OK (outputs untouched). */
int moe_route(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
              int32_t* topk_idx, float* topk_w, int32_t* n_unique, int32_t* uniq_ids,
              int32_t* uniq_off, int32_t* pairs, void* ws, size_t ws_bytes, void* stream);

/* The whole layer for T tokens: route, union, experts, combine.
 *   x: binary16 [T][H]; y: binary16 [T][H] (output);
 *   topk_idx_out int32 [T][k] and topk_w_out fp32 [T][k]: optional copies of
 *   the routing decision (NULL to skip).
 * Small batches take the GEMV path (weights streamed once per unique
 * expert); larger batches take the grouped-GEMM path on the matrix cores.
 * Both compute the same function.  T == 0 is a no-op. */
int moe_w4a16_forward(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
                      uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream);

/* moe_w4a16_forward with stage timing for benchmarks: `events` is a host
 * array of n_events (0..6) hipEvent_t handles (passed as void*; entries may
 * be NULL).  events[2i] and events[2i+1] take the start and end time of
 * stage i, recorded by the dispatch of the stage's first and last kernel
 * (so the interval holds the stage's kernels and the gaps between them, not
 * the launch overhead around them).  Stages on the decode path (T <=
 * moe_decode_max_tokens()): 0 routing + union + shared expert gate/up,
 * 1 routed gate/up + SwiGLU, 2 down projections + combine; for T == 1,
 * stage 0 holds the router logits alone and stage 1 the top-k, union and
 * every gate/up (shared and routed).  On the
 * grouped-GEMM path: 0 routing + union, 1 gate/up + SwiGLU, 2 down +
 * combine.  Adds no synchronisation.  Same arguments and results as
 * moe_w4a16_forward; n_events outside 0..6 or a NULL array with n_events
 * > 0 gives MOE_E_INVAL. */
int moe_w4a16_forward_profiled(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
                               uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* ws,
                               size_t ws_bytes, void* stream, void* const* events, int32_t n_events);

/* moe_w4a16_forward for callers that cannot allocate memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments (minus the workspace), same kernels, same results as
 * moe_w4a16_forward.  The scratch memory is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's device code, which every GPU
 * the library runs on holds until the process ends; the call allocates
 * nothing.  Each call first clears the array's completion counters with a
 * small fill kernel on `stream`, then runs the layer.
 * Limit: a call with moe_workspace_bytes(d, T) > MOE_NOALLOC_SCRATCH_BYTES
 * returns MOE_E_WORKSPACE and launches nothing (the 6144 x 2048, 256-expert
 * top-8 int4 layer with a shared expert fits up to T = 118).
 * Every call on one GPU uses that GPU's single array: calls that overlap in
 * time on one GPU (several streams or host threads) race and give undefined
 * results; serialise them, e.g. on one stream.  Other errors as
 * moe_w4a16_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moe_w4a16_forward_noalloc(const moe_dims_t* d, const moe_weights_t* w, const uint16_t* x, int32_t T,
                              uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* stream);

/* A decode step of several layers captured once as one HIP graph and then
 * replayed, so that a step costs one graph launch instead of one host launch
 * per kernel: the way the Ornith engine runs each decode step ("GTX 1070向け
 * 35BパラメータMoEモデル推論エンジン公開", 648news.com, section "Pascal世代の
 * 制約をCUDAグラフとカーネル最適化で克服").
 * moe_step_graph_create records, for l = 0 .. n_layers-1 in order,
 *   moe_w4a16_forward(d, &w[l], x[l], T, y[l], NULL, NULL, ws, ws_bytes, .)
 * on a capture stream of its own (nothing else is recorded):
 *   w: (host) array of n_layers weight structs; x, y: (host) arrays of
 *   n_layers device pointers (binary16 [T][H] each).  The pointers and the
 *   shape are fixed at creation; the data behind them is read and written at
 *   every launch.  Passing x[l+1] == y[l] chains the layers (each consumes the
 *   previous one's output); distinct buffers give independent layers.
 *   All layers share the one workspace ws (the zero-fill rule above).
 * Every layer's arguments are validated as moe_w4a16_forward validates them
 * before anything touches the device; errors as there, plus MOE_E_INVAL for
 * n_layers outside 1 .. MOE_STEP_GRAPH_MAX_LAYERS, T < 1, or a NULL array or
 * out; MOE_E_HIP if the capture or the instantiation fails.  On success
 * *out receives the handle; otherwise *out is untouched and nothing is kept.
 * Creation is the one place where the library allocates: the handle and
 * the HIP runtime's graph objects, freed by moe_step_graph_destroy.
 * moe_step_graph_launch enqueues the whole step on `stream` (allocating
 * nothing; MOE_E_INVAL for a NULL handle, MOE_E_HIP if the launch fails).
 * Launches of one graph, or of graphs sharing a workspace, must not overlap
 * in time (one stream serialises them).  moe_step_graph_destroy(NULL) is a
 * no-op; the graph must not be in flight when it is destroyed. */
#define MOE_STEP_GRAPH_MAX_LAYERS 4096
typedef struct moe_step_graph_s* moe_step_graph_t;
int moe_step_graph_create(const moe_dims_t* d, int32_t n_layers, const moe_weights_t* w,
                          const uint16_t* const* x, int32_t T, uint16_t* const* y, void* ws,
                          size_t ws_bytes, moe_step_graph_t* out);
int moe_step_graph_launch(moe_step_graph_t g, void* stream);
int moe_step_graph_destroy(moe_step_graph_t g);

/* Reference rates for the rooflines (measurement support, not part of the
 * layer).  The pages find decode speed bound by memory bandwidth ("GLM 5.3
 * Flash をローカルに導入するには？", vramglass.com, the section on offloading
 * experts to system memory); these two kernels measure what this GPU
 * actually reaches, beside its published peaks:
 *   moe_probe_stream_read: reads every 16-byte vector of buf (bytes, a
 *     multiple of 16; buf 16-byte aligned) once with 128-bit non-temporal
 *     loads over `blocks` workgroups of 256 threads (grid stride); writes one
 *     word per thread to sink (blocks * 256 uint32, 4-byte aligned).
 *   moe_probe_mfma: `blocks` workgroups of 512 threads; every wavefront runs
 *     iters rounds of 16 independent v_mfma_f32_16x16x32_f16 (16 x 16 x 32
 *     multiply-adds each) on register operands and writes one word per
 *     thread to sink (blocks * 512 uint32).
 * Both are stream-ordered launches; MOE_E_INVAL for a null or misaligned
 * pointer, a size that is not a multiple of 16, or blocks / iters < 1;
 * MOE_E_HIP if the launch fails. */
int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);
int moe_probe_mfma(uint32_t* sink, int32_t blocks, int32_t iters, void* stream);

/* Largest T served by the GEMV path of moe_w4a16_forward. */
int32_t moe_decode_max_tokens(void);

/* Static description of a status code; never NULL. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
