/*
 * moert.h — C ABI of the routed-expert MoE step on one MI355X (gfx950).
 *
 * The step, per MoE layer, as the FreeToken pages describe it:
 *   route top-k → one device-side control kernel (dedup the routed
 *   (layer, expert) ids, classify them against the residency table, split the
 *   misses by q, surface the K least-recently-used victim slots, rewrite ids
 *   into slot ids or a CPU flag) → PCIe fills into victims ∥ host execution of
 *   the remaining misses → grouped expert FFN over the slot pool → exact,
 *   fixed-order merge of GPU and host partial sums.  Prefill streams whole
 *   layers into two full-layer buffers carved out of the same pool; the pool
 *   can be rebuilt under a new budget without reloading the host pool.
 *
 * Pages cited (by title and section):
 *   [snackonai] "FreeToken, or why your laptop was never the bottleneck",
 *               https://www.snackonai.com/p/freetoken-or-why-your-laptop-was-never-the-bottleneck
 *   [satyajit]  "FreeToken: a 753B model on one GPU, and the two bandwidths that
 *               decide everything", https://ai.thesatyajit.com/articles/freetoken
 *   [son]       "FreeToken: treat the whole PC as one" (essay, no headings),
 *               https://signalovernoise.tech/p/freetoken-treat-the-whole-pc-as-one
 *   [devto]     "FreeToken runs frontier-scale MoE models by treating the whole PC
 *               as the inference platform", dev.to/khasky
 *
 * Conventions for every call:
 *   - Pointers marked (device) are device addresses (e.g. torch.cuda tensors);
 *     (host) are host addresses.  The caller owns every buffer it passes; the
 *     library keeps no pointer to it after the call returns, except the host
 *     pool given to moe_create (kept until moe_destroy).
 *   - Arguments are validated before anything is enqueued: a bad argument
 *     returns MOE_EINVAL and enqueues nothing.  No C++ exception crosses the
 *     ABI.  A HIP failure returns MOE_EHIP and is latched: every later call on
 *     that context returns MOE_EHIP (moe_last_error() has the text).
 *   - route / plan / ffn / merge / prefill enqueue work on `stream` and never
 *     synchronise the host; plans stay on the device (the host never reads
 *     them on this path) [snackonai, "The Architecture, Unpacked"].  The one
 *     exception is on-demand prefill (see moe_prefill_layer), which must read
 *     a layer's routed experts before it can fetch them.
 *   - One context is driven by one host thread, and its decode calls for a
 *     layer are issued in the order plan → ffn → merge on one stream; a call
 *     out of that order returns MOE_EINVAL.
 *   - Matrices are row-major.  Activations (x, y) use the context's act dtype
 *     (f32 or bf16); router logits and weights are fp32.
 */
#ifndef MOERT_H
#define MOERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;
typedef void* moe_stream; /* a hipStream_t; NULL is the null stream */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument or call order; nothing enqueued      */
  MOE_ENOMEM = -2,       /* device or pinned host allocation failed           */
  MOE_ENOSPC = -3,       /* prefill with an empty slot pool                   */
  MOE_EHIP = -4,         /* HIP runtime error (latched)                       */
  MOE_EBUSY = -5,        /* work still in flight where a safe point is needed */
  MOE_ETIMEDOUT = -6,    /* resize could not drain within timeout_ms          */
  MOE_EUNSUPPORTED = -7  /* device lacks a needed feature                     */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype;

/* Miss handling [satyajit, "Four backends, and the one that has to be
 * measured"]: HYBRID fills q = clamp(round_half_even(m*B_P/B_H), 1, m) misses
 * and runs the rest on the host; OFFLOAD fills every miss; CPU fills none. */
typedef enum { MOE_HYBRID = 0, MOE_OFFLOAD = 1, MOE_CPU = 2 } moe_mode;

typedef struct {
  int32_t n_layers;      /* L: MoE layers; flat expert id u = l*E + e        */
  int32_t n_experts;     /* E (1..1024)                                       */
  int32_t top_k;         /* k (1..min(E, 32))                                 */
  int32_t hidden;        /* H: multiple of 64, at most 512 sixteen-byte chunks
                            per row (F32 2048, BF16 4096, MXFP4 16384)       */
  int32_t inter;         /* I, expert intermediate: same rules as H           */
  int32_t w_dtype;       /* moe_dtype of expert weights: F32, BF16 or MXFP4   */
  int32_t act_dtype;     /* moe_dtype of x and y: F32 or BF16                 */
  int32_t n_slots;       /* initial device slot budget (0..max_slots)         */
  int32_t max_slots;     /* address-space reservation; resize may grow to it  */
  int32_t max_tokens;    /* largest T of a decode layer call (1..256)          */
  int64_t bw_pcie_mbps;  /* B_P, MB/s (> 0)                                   */
  int64_t bw_host_mbps;  /* B_H, MB/s (>= B_P in HYBRID)                      */
  int32_t max_fetch;     /* cap on PCIe fills per layer call; 0 = none        */
  int32_t mode;          /* moe_mode                                          */
  int32_t cpu_threads;   /* host worker threads; 0 = one per available core   */
  int32_t max_prefill_tokens; /* largest prefill chunk; 0 disables prefill    */
  int32_t timing;        /* 1: time every launched phase with HIP events      */
} moe_config;

/* Bytes of one expert bank == one device slot stride (expert bytes rounded up
 * to 256).  A slot is a complete expert, named by its flat id u = l*E + e in
 * every bank [snackonai, "The Architecture, Unpacked", first decision].
 * Bank layout (contraction axis contiguous in every matrix):
 *   F32  : W_gate[I][H] | W_up[I][H] | W_down[H][I]           (float)
 *   BF16 : the same, bfloat16
 *   MXFP4: codes W_gate[I][H/2] | W_up[I][H/2] | W_down[H][I/2], then
 *          scales W_gate[I][H/32] | W_up[I][H/32] | W_down[H][I/32];
 *          OCP MX v1.0 E2M1 codes two per byte (low nibble = even element),
 *          one E8M0 scale per 32 contraction elements.
 * The expert is SwiGLU without biases: p = W_down (silu(W_gate x) * W_up x).
 * Returns 0 for an invalid config. */
size_t moe_expert_bytes(const moe_config* cfg);

/* Pinned, device-mapped host memory for the host expert pool (the source of
 * truth: [son]; [snackonai, "What It Actually Does"]).  The caller fills bank
 * u at offset u * moe_expert_bytes() and then calls moe_create.  The pages pin
 * after filling; this library allocates pinned memory first because
 * registering existing pages is not available on the target platform.
 * Returns MOE_ENOMEM on failure. */
moe_status moe_host_pool_alloc(size_t bytes, void** out /* (host) */);
moe_status moe_host_pool_free(void* p);

/* Create a context on the current HIP device.  host_pool (host) must come
 * from moe_host_pool_alloc and hold L*E banks (host_pool_bytes >=
 * L*E*moe_expert_bytes); the library only reads it.  Reserves device address
 * space for max_slots slots, maps n_slots of them, allocates the residency
 * tables (all slots empty: no warmup [satyajit, "Elastic memory, because the
 * machine is not yours"]), plan buffers sized by max_tokens, staging, side
 * streams and the host worker pool. */
moe_status moe_create(const moe_config* cfg, void* host_pool, size_t host_pool_bytes,
                      moe_ctx** out);
/* Waits for the context's work, then frees everything it owns. */
moe_status moe_destroy(moe_ctx* ctx);

/* Router top-k [snackonai, "The Promise" leaves router design out; a softmax
 * router is assumed].  logits (device) fp32 [T][E]; ids (device) int32 [T][k]
 * receives experts by descending logit, equal logits by ascending index (NaN
 * ranks as -inf); w (device) fp32 [T][k] receives the softmax over the k
 * selected logits.  1 <= T <= max(max_tokens, max_prefill_tokens). */
moe_status moe_route_topk(moe_ctx* ctx, const float* logits, int32_t T, int32_t* ids,
                          float* w, moe_stream stream);

/* The control step of MoE layer `layer` [snackonai, "The Architecture,
 * Unpacked", third decision; satyajit, "Residency that follows the router";
 * snackonai, "The Code, Annotated"]: one kernel deduplicates {layer*E +
 * ids[t][j]} (ascending), classifies them against id2slot, computes q (mode,
 * then max_fetch, then the slots not holding a current hit), refreshes the
 * hits' recency, surfaces the K = min(max_tokens*k, E, n_slots[, max_fetch])
 * least-recently-used slots by (tick, slot) excluding current hits, admits the
 * first q misses into the first q of them and writes slot_map[t][j] (slot id,
 * or -1 = run on the host).  One LRU tick per call.  The call then enqueues
 * the PCIe fill of the q admitted experts into their slots (on `stream`);
 * one more workgroup of that launch hands the remaining misses to the host
 * branch (ids, slot map and activations into pinned memory, then a doorbell
 * that a host thread answers), so the control kernel itself writes no host
 * memory.
 * ids (device) int32 [T][k]; x (device) [T][H] act dtype, read by the host
 * branch.  1 <= T <= max_tokens. */
moe_status moe_cache_plan(moe_ctx* ctx, int32_t layer, const int32_t* ids, int32_t T,
                          const void* x, moe_stream stream);

/* Grouped SwiGLU evaluation of every GPU-resident routed expert of the last
 * plan (hits and fills; each slot's weights read once per call) into the
 * context's fp32 partial rows P_gpu[T][k][H] [snackonai, "The Code,
 * Annotated", "The split policy itself": the GPU path runs the cache update,
 * then the batched copy, then grouped evaluation of the resident experts].
 * It follows the plan's fill on the same stream.  x (device) [T][H] act
 * dtype; layer and T must equal the last moe_cache_plan's.  MOE_EINVAL out of
 * call order (see the conventions above). */
moe_status moe_expert_ffn(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                          moe_stream stream);

/* Graph capture of decode calls [snackonai, "Technical Moats": a policy
 * simple enough to run inside a captured graph; satyajit, "Residency that
 * follows the router"]: moe_route_topk, moe_cache_plan, moe_expert_ffn and moe_merge
 * enqueue only kernels on `stream`, and every value that changes from call to
 * call (LRU tick, plan count, which also numbers the calls for the host
 * branch, counts, slot lists) lives on the device.  A caller may therefore
 * capture any sequence of whole layer calls into a HIP graph and replay it,
 * as long as: the context was created with timing = 0; the inputs of each
 * replay sit at the captured addresses; the last call before the capture was
 * not a prefill layer (run one eager decode layer call after a prefill).  A
 * resize or a prefill layer changes the slot count and buffers: capture again
 * after either.  Replays and eager calls may be interleaved. */

/* Exact merge [snackonai, "What It Actually Does"; satyajit, "Decode: the one
 * equation"]: waits for the host branch, then y[t] = sum over ascending j of
 * w[t][j] * (slot_map[t][j] >= 0 ? P_gpu[t][j] : P_cpu[t][j]) in fp32, rounded
 * once to the act dtype.  w (device) fp32 [T][k]; y (device) [T][H]. */
moe_status moe_merge(moe_ctx* ctx, const float* w, int32_t T, void* y, moe_stream stream);

/* Rebuild the slot pool under a new budget at a safe point [satyajit,
 * "Elastic memory, because the machine is not yours"; snackonai, "Resizing
 * the cache without a restart"].  Drains the context's streams (waiting up to
 * timeout_ms, else MOE_ETIMEDOUT with nothing changed), evicts in LRU victim
 * order until min(new_n_slots, occupied) experts remain, leaves a survivor
 * below the new budget in its slot and moves the survivors beyond it into the
 * free slots below it (both in ascending order; one device-to-device copy
 * kernel, since no move reads a slot another move writes), keeps their
 * recency, and maps or unmaps device memory beyond the new budget.  The host
 * pool is never read or written.  A full-layer slab that a prefill call
 * streamed ahead and no call has consumed yet is admitted first (one tick),
 * as a decode call would admit it.  0 <= new_n_slots <= max_slots.
 * Synchronous. */
moe_status moe_cache_resize(moe_ctx* ctx, int32_t new_n_slots, int32_t timeout_ms);

/* One prefill chunk of MoE layer `layer` [satyajit, "Prefill: hide the pool
 * behind the wire"; snackonai, "It In Action"]: two full-layer buffers are
 * slots [0,E) and [E,2E) of the shared pool; layer l runs out of buffer l%2
 * while a copy stream streams every expert of layer l+1 into the other
 * buffer with one hipMemcpyAsync from the pinned host pool (with one buffer,
 * see moe_prefill_set_buffers, every layer uses slots [0,E) and its copy
 * starts after the previous layer's compute).  The residency tables record the
 * buffer's experts as ordinary slots (one tick per layer), so what survives
 * seeds decode.  Tokens are grouped by expert and evaluated with an MFMA
 * grouped GEMM; y[t] = sum over ascending j of w[t][j] * FFN(x[t]).
 * x (device) [T][H] act dtype; ids (device) int32 [T][k]; w (device) fp32
 * [T][k]; y (device) [T][H].  1 <= T <= max_prefill_tokens.
 * Supported for MXFP4 experts with bf16 activations, H % 256 == 0 and
 * I % 128 == 0 (MOE_EUNSUPPORTED otherwise).  moe_create refuses a
 * max_prefill_tokens with max_prefill_tokens*H*2 or max_prefill_tokens*k*I*2
 * at or above 2^32 (the GEMM's per-row byte offsets are 32-bit).
 * When n_slots < buffers x E the buffers do not fit, and the call falls back
 * to on-demand loading instead of oversubscribing [signalovernoise essay;
 * snackonai, "The Architecture, Unpacked"]: it synchronises `stream` once to
 * read which experts the chunk routes to, then loads them in ascending order,
 * at most n_slots per pass, into slots [0, P) (one tick per pass; occupants
 * evicted, a pass expert resident elsewhere emptied there), and runs the
 * grouped GEMM over each pass's experts on `stream`; nothing is prefetched.
 * Cache hits do not cross the bus [satyajit, "Four backends, and the one that has to
 * be measured", the prefill hit-D2D option]: when a layer's slab goes into
 * its full-layer buffer, each of its experts resident in a slot outside the
 * buffers is copied device to device and only the others cross PCIe (runs of
 * consecutive experts, one copy each); for this the first two-buffer call
 * after any decode call, resize or on-demand pass reads the residency table
 * once (one synchronisation of `stream`).  On demand, in the first pass an
 * expert already in its target slot is not copied and one resident at or
 * beyond slot P is copied device to device.  Only the bytes' source changes;
 * the tables are the same.  moe_ctx_stats counts the experts by source.
 * MOE_ENOSPC if n_slots == 0. */
moe_status moe_prefill_layer(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                             const int32_t* ids, const float* w, void* y, moe_stream stream);

/* moe_prefill_layer for callers that cannot allocate memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same call, the same kernels and the same results, but the chunk's
 * grouping and GEMM intermediates (per-expert counts, offsets and cursors, the
 * M-tile list, the pair permutation, the bf16 intermediate and the fp32
 * expert rows) live in the library's fixed device scratch instead of the
 * block moe_prefill_layer allocates on its first call.  The call makes no
 * hipMalloc, hipFree or other allocating call; the context's prefill events
 * and pinned staging already exist (moe_create makes them when
 * max_prefill_tokens > 0).
 * Limit: the scratch is 64 MiB per GPU, held from the first moe_create on
 * that GPU until the process ends.  A chunk fits when its T*k routed pairs
 * need at most that: about 4*(4E + T*k/128) + T*k*(4 + 2I + 4H) bytes (each
 * array rounded up to 256 B), i.e. T*k <= 3,275 pairs (T <= 409 at k = 8) for
 * E = 256, H = 4096, I = 2048.  A larger T returns MOE_EINVAL (moe_last_error() gives
 * the limit for the context's shape) and enqueues nothing.
 * Every context on one GPU shares that GPU's scratch, and each call leaves
 * its intermediates there (moe_prefill_view_get shows them until the next
 * prefill call on the context): calls on one GPU whose work overlaps in time
 * (other streams, other contexts, other host threads) race on it; serialise
 * them.  Everything a call reads from the scratch it first writes or zeroes
 * on the device (by kernels, not memset nodes). */
moe_status moe_prefill_layer_noalloc(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                                     const int32_t* ids, const float* w, void* y, moe_stream stream);

/* Full-layer buffers for prefill: 2 (default; the next layer streams while
 * this one computes) or 1 (the ablation the pages measure by disabling the
 * second buffer [snackonai, "It In Action"]: each layer's copy waits for the
 * previous layer's compute, and n_slots >= E suffices).  MOE_EBUSY while a
 * prefetched slab is pending (between two prefill layers of a chunk); call it
 * before a chunk's first layer or after a decode call. */
moe_status moe_prefill_set_buffers(moe_ctx* ctx, int32_t n_buffers);

/* Device addresses of the last plan's fixed-shape outputs and of the
 * residency tables (for inspection and tests; reading them requires the
 * plan's stream to have completed).  Counts layout: see moe_plan_counts. */
typedef struct {
  int32_t n_uniq, n_hit, n_miss, q, n_cpu, n_gpu, K;
  int32_t tick_lo;  /* low 32 bits of the call's LRU tick (the full 64-bit
                       tick is moe_plan_view.tick)                           */
} moe_plan_counts;

typedef struct {
  const moe_plan_counts* counts; /* (device) */
  const int32_t* uniq;       /* [Umax] ascending flat ids                     */
  const int32_t* hits;       /* [Umax] ascending                              */
  const int32_t* misses;     /* [Umax] ascending                              */
  const int32_t* victims;    /* [Kmax] LRU-first, -1 padded to K              */
  const int32_t* fill_u;     /* [Kmax] first q misses                          */
  const int32_t* fill_slot;  /* [Kmax]                                         */
  const int32_t* fill_old;   /* [Kmax] evicted id or -1                        */
  const int32_t* cpu_u;      /* [Umax] misses[q:]                              */
  const int32_t* gpu_u;      /* [Umax] resident after the plan, ascending u    */
  const int32_t* gpu_slot;   /* [Umax]                                         */
  const int32_t* slot_map;   /* [max_tokens*k]                                 */
  const int32_t* id2slot;    /* [L*E]                                          */
  const int32_t* slot2id;    /* [max_slots]                                    */
  const int64_t* slot_ts;    /* [max_slots], -1 = empty                        */
  const int64_t* tick;       /* [1]                                            */
  const float* p_gpu;        /* [max_tokens*k][H] fp32                         */
  const float* p_cpu;        /* [max_tokens*k][H] fp32 (pinned host, mapped)   */
  const void* slot_base;     /* slot s at slot_base + s * moe_expert_bytes()   */
  int32_t n_slots, max_slots, umax, kmax;
  const uint64_t* h_marked;  /* [max_tokens*k][inter] the expert FFN's
                                intermediate silu(gate) * up: fp32 bits in the
                                low word, the low 32 bits of the tick of the
                                call that wrote it in the high word (an entry
                                counts only with its call's mark; every 2^30
                                ticks the control kernel sets all marks to
                                that call's tick with bit 31 flipped)         */
} moe_plan_view;

moe_status moe_plan_view_get(moe_ctx* ctx, moe_plan_view* out);

/* Device addresses of the last prefill layer's grouping of its routed
 * (token, rank) pairs by expert and of its intermediates, for inspection and
 * tests [satyajit, "Prefill: hide the pool behind the wire": the layer's
 * tokens are evaluated expert by expert out of the full-layer buffer].
 * Reading them requires the prefill call's stream to have completed; the next
 * prefill call overwrites them.  MOE_EINVAL before the first prefill call.
 *   counts  [E]    routed pairs per expert
 *   offsets [E+2]  offsets[e] = first position of expert e (exclusive scan of
 *                  counts, offsets[E] = T*k); offsets[E+1] = number of M-tiles
 *   perm    [T*k]  position -> pair index t*k + j, the pairs of expert e at
 *                  positions [offsets[e], offsets[e+1]) in no particular order
 *   tiles   [offsets[E+1]]  (e << 20) | ((m0 / 64) << 1) | half: the 128-row
 *                  M-tiles of each expert in order, m0 its first row within the
 *                  expert, half = 1 for a last tile of at most 64 rows
 *   hmid    [T*k][I] bf16 silu(gate) * up per position
 *   prow    [T*k][H] fp32 expert output per pair */
typedef struct {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tiles;
  const uint16_t* hmid;
  const float* prow;
  int32_t n_experts, max_pairs, max_tiles;
} moe_prefill_view;

moe_status moe_prefill_view_get(moe_ctx* ctx, moe_prefill_view* out);

/* Pool table [snackonai, "Resizing the cache without a restart"]: occupancy
 * and counters accumulated on the device since moe_create.  Synchronises the
 * context's streams; not for the hot path. */
typedef struct {
  int32_t n_slots, occupied;
  int64_t plans, hits, fills, cpu, evictions;
  int64_t prefill_layers, resizes;
  /* prefill experts brought into full-layer buffers or on-demand pass slots:
     over PCIe from the host pool, and device to device from a slot that
     already held them (the cache hits that cross no bus) */
  int64_t prefill_h2d_experts, prefill_d2d_experts;
} moe_stats;

moe_status moe_ctx_stats(moe_ctx* ctx, moe_stats* out);

/* Bandwidth calibration [snackonai, "The Code, Annotated": the two rates are
 * measured once per machine on the deployed expert shapes, not taken from
 * spec sheets; "The split policy itself": q uses exactly these two numbers].
 * B_P: the fill kernel pulling n_experts whole experts from the pinned host
 * banks into a scratch device buffer, reps timed launches after one untimed
 * one (HIP events).  B_H: the host branch's own expert arithmetic on its
 * worker pool, one token per expert, reps timed runs after one untimed one
 * (wall clock).  Every run takes a different set of experts spread over the
 * host pool (distinct while L*E >= n_experts*(reps+1)), so no cache serves
 * bytes twice.  If bw_h2d_mbps is not NULL, the same sets are also copied
 * with pinned host-to-device copies (the copy engines, one per expert) and
 * that rate is written there too (the fill itself uses the pull).  All in
 * MB/s of expert bytes (moe_expert_bytes without the slot padding).  Safe-point call: drains the
 * context like moe_cache_resize (60 s limit, MOE_ETIMEDOUT), allocates and
 * frees a scratch buffer of n_experts slots; the slot pool, the residency
 * tables and the configured bandwidths are unchanged.  1 <= n_experts (capped
 * at 64 and at L*E), 1 <= reps <= 1000.  Synchronous. */
moe_status moe_measure_bandwidth(moe_ctx* ctx, int32_t n_experts, int32_t reps,
                                 int64_t* bw_pcie_mbps, int64_t* bw_host_mbps, int64_t* bw_h2d_mbps);

/* The backend rule [snackonai, "The Code, Annotated": recommend hybrid when
 * B_H exceeds threshold x B_P, with threshold 2.0, else offload]: writes
 * MOE_HYBRID or MOE_OFFLOAD to *out.  Pure host arithmetic, no context.
 * MOE_EINVAL for non-positive bandwidths or threshold. */
moe_status moe_recommend_mode(int64_t bw_pcie_mbps, int64_t bw_host_mbps, double threshold,
                              moe_mode* out);

/* Per-layer host decode [satyajit, "Four backends, and the one that has to be
 * measured": a flag names the MoE layers that decode on the CPU]: flags
 * (host) [n_layers], nonzero = that layer's calls run with mode CPU (q = 0:
 * no fills and no admissions; experts of the layer still resident from
 * before stay hits on the GPU until evicted).  NULL clears.  n_layers must
 * equal cfg.n_layers.  Applies from the next moe_cache_plan; a graph
 * captured earlier keeps the modes it was captured with.  No layer call may
 * be open. */
moe_status moe_set_cpu_layers(moe_ctx* ctx, const uint8_t* flags, int32_t n_layers);

/* Replace the bandwidths the control kernel splits misses with, and the mode
 * (for example with measured values and the recommended backend).  Applies
 * from the next moe_cache_plan; a graph captured earlier keeps the values it
 * was captured with (capture again).  No layer call may be open. */
moe_status moe_set_split(moe_ctx* ctx, int64_t bw_pcie_mbps, int64_t bw_host_mbps, moe_mode mode);

/* Device time per phase, summed since creation (or the last reset), when the
 * context was created with cfg.timing = 1: each call brackets the kernels it
 * launches with a pair of HIP events on the stream they run on.  HOST is the
 * wall time of the host branch (poller thread) per call with host work;
 * PREFILL_GEMM covers the two grouped GEMM kernels only.  Synchronises the device; not for
 * the hot path.  MOE_EINVAL if timing is off. */
enum {
  MOE_T_ROUTE = 0, MOE_T_PLAN = 1, MOE_T_FILL = 2, MOE_T_FFN = 3, MOE_T_MERGE = 4,
  MOE_T_HOST = 5, MOE_T_PREFILL_COPY = 6, MOE_T_PREFILL_GROUP = 7, MOE_T_PREFILL_GEMM = 8,
  MOE_T_PREFILL_MERGE = 9, MOE_T_COUNT = 10
};
typedef struct {
  int64_t calls[MOE_T_COUNT];
  double ms[MOE_T_COUNT];
} moe_timing;

moe_status moe_ctx_timing(moe_ctx* ctx, moe_timing* out, int32_t reset);

const char* moe_strerror(moe_status s);
/* Text of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOERT_H */
