// Internal declarations of the routed-expert MoE library (gfx950, HIP).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moert.h"

namespace moert {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxSlots = 32768;
constexpr int kMaxDecodeTokens = 256;
constexpr int kPlanThreads = 1024;
// the expert FFN's intermediate entries carry the low 32 bits of their
// call's tick; every 2^kHMarkEpochBits ticks the control kernel rewrites all
// marks to one that no tick of the new epoch has
constexpr int kHMarkEpochBits = 30;

// Device-resident scalars the control kernel owns: the LRU tick and the
// running counters of the pool table.
struct DevState {
  int64_t tick;
  int64_t plans, hits, fills, cpu, evictions;
  int64_t prefill_layers;
  int32_t n_slots;   // current budget, read by the control kernel
  int32_t pad;
  int64_t h_epoch;   // tick >> kHMarkEpochBits when the marks were last rewritten
};

// Everything the host branch needs from one plan, in pinned host memory that
// the fill kernel's hand-off workgroup writes directly after the control
// kernel.  `seq` is the doorbell: it is written last (after a system-scope
// fence), and only when the call has host work.
struct HostBlockHeader {
  int64_t seq;
  moe_plan_counts c;
  int32_t layer, T;
};

// Completion word of the host branch (pinned, mapped): the poller publishes
// the doorbell value it finished; the merge kernel waits for it; a merge that
// gives up after its time limit sets `error`.
struct HostSync {
  int64_t done;
  int32_t error;
  int32_t pad[13];
};

// Fixed-shape plan outputs in device memory (one allocation).
struct PlanBufs {
  moe_plan_counts* counts;
  int32_t *uniq, *hits, *misses, *victims, *fill_u, *fill_slot, *fill_old;
  int32_t *cpu_u, *gpu_u, *gpu_slot, *slot_map;
  uint64_t* h_marked;     // [h_words] the expert FFN's marked intermediate
  int64_t h_words;
  int32_t* host_work;     // [1] set by the control kernel: the host branch has work
  // host block in pinned, device-mapped memory, written by the fill kernel's
  // hand-off workgroup:
  // header | ids[maxTk] | slot_map[maxTk] | x[max_tokens][H] (act dtype)
  uint8_t* hblock;        // device address of the mapping
  size_t hblock_bytes;    // header + ids + slot map
  size_t x_offset;        // byte offset of the activations copy
  int act_bytes;          // bytes per activation element
};

// One physical chunk of the slot pool mapped into the reserved range.
struct PoolChunk {
  hipMemGenericAllocationHandle_t h;
  size_t offset, bytes;
};

struct SlotPool {
  uint8_t* base = nullptr;     // start of the reserved (or allocated) range
  size_t reserved = 0;         // bytes of address space
  size_t mapped = 0;           // bytes currently backed
  size_t gran = 0;             // chunk size (multiple of the VMM granularity)
  bool vmm = false;            // false: one plain allocation of `reserved`
  std::vector<PoolChunk> chunks;
};

// Device intermediates of one prefill chunk: the grouping of its routed
// pairs by expert and the two GEMMs' outputs.  One block carved into
// 256-byte aligned arrays (prefill_layout).
struct PrefillBufs {
  int32_t* counts = nullptr;   // [E] pairs per expert
  int32_t* offsets = nullptr;  // [E+2] exclusive scan; [E+1] = M-tile count
  int32_t* cursor = nullptr;   // [E] scatter cursors
  int32_t* slot_of = nullptr;  // [E] on-demand pass: slot of each expert, -1 outside
  int32_t* tiles = nullptr;    // [max_tiles] M-tile list
  int32_t* perm = nullptr;     // [max_pairs] position -> pair index
  uint16_t* hmid = nullptr;    // [max_pairs][I] bf16 intermediate
  float* prow = nullptr;       // [max_pairs][H] fp32 expert rows
  int32_t max_tiles = 0;
  int64_t max_pairs = 0;
};

// Bytes of the intermediates of a chunk with `pairs` routed pairs; when
// `base` is given, `out` is pointed into it.
size_t prefill_layout(const moe_config& c, int64_t pairs, uint8_t* base, PrefillBufs* out);

// The library's fixed device scratch for moe_prefill_layer_noalloc
// (prefill.hip): its device address on `device`, looked up once per device
// by prefill_scratch_init (called by moe_create with the device current).
constexpr size_t kPrefillScratchBytes = (size_t)64 << 20;
hipError_t prefill_scratch_init(int device);
uint8_t* prefill_scratch_ptr(int device);

struct CpuPool;     // host worker pool (cpu_branch.cpp)
struct HostBranch;  // doorbell poller (cpu_branch.cpp)

enum CallState { kIdle = 0, kPlanned = 1, kEvaluated = 2 };

// Ring of event pairs bracketing launched phases (timing mode only).
struct Timing {
  static constexpr int kRing = 2048;
  std::vector<hipEvent_t> a, b;
  std::vector<int> phase;
  int head = 0, used = 0;
  int64_t calls[MOE_T_COUNT] = {};
  double ms[MOE_T_COUNT] = {};
  std::atomic<int64_t> host_ns{0}, host_calls{0};
};

}  // namespace moert

struct moe_ctx {
  moe_config cfg;
  int device = 0;
  size_t stride = 0;          // slot / bank stride
  size_t expert_bytes = 0;
  int64_t n_ids = 0;
  int32_t n_slots = 0;
  int32_t umax = 0;           // plan list bound: min(max_tokens*k, E)
  int32_t kmax = 0;           // victim list bound for the largest budget
  int32_t cpu_threads = 0;

  // host expert pool (caller-owned, pinned + mapped)
  uint8_t* host_pool = nullptr;
  const uint8_t* host_pool_dev = nullptr;
  size_t host_pool_bytes = 0;

  moert::SlotPool pool;

  // residency tables (device)
  int32_t* id2slot = nullptr;
  int32_t* slot2id = nullptr;
  int64_t* slot_ts = nullptr;
  moert::DevState* dstate = nullptr;

  moert::PlanBufs plan{};
  uint8_t* plan_alloc = nullptr;

  // partial rows and decode intermediate
  float* p_gpu = nullptr;      // device [max_tokens*k][H]
  float* p_cpu = nullptr;      // pinned host, mapped [max_tokens*k][H]
  const float* p_cpu_dev = nullptr;
  uint64_t* h_mid = nullptr;   // device [max_tokens*k][I] {fp32 bits, tick mark}

  // host block (pinned, mapped): the fill launch's hand-off workgroup writes it, the
  // host branch reads it
  uint8_t* hstage = nullptr;   // host address
  uint8_t* xstage = nullptr;   // host address of its activations copy

  // host branch hand-off
  moert::HostSync* sync = nullptr;        // host address
  moert::HostSync* sync_dev = nullptr;    // device address
  uint64_t wait_ticks = 0;                // merge's wait limit in wall-clock ticks
  uint64_t ffn_wait_ticks = 0;            // expert FFN down items' wait limit

  hipStream_t copy = nullptr;  // prefill transfers
  std::vector<uint8_t> cpu_layers;  // [L] nonzero: the layer decodes its misses on the host, never fills

  moert::CpuPool* cpu = nullptr;
  moert::HostBranch* hb = nullptr;

  // decode call order
  int state = moert::kIdle;
  int32_t cur_layer = -1, cur_T = 0;

  // prefill: events and pinned staging at creation (max_prefill_tokens > 0);
  // the intermediates of moe_prefill_layer allocated on its first call
  struct Prefill {
    bool ready = false;                    // events and staging exist
    int32_t buffers = 2;                   // full-layer buffers in use (1: no prefetch)
    int32_t buf_layer[2] = {-1, -1};      // layer whose slab was issued into buffer b
    bool admitted[2] = {false, false};     // tables already describe buffer b
    hipEvent_t ev_copied[2] = {nullptr, nullptr};
    hipEvent_t ev_start = nullptr;
    int32_t* counts_host = nullptr;        // [2E] pinned: counts, then the layer's id2slot row (on-demand)
    uint8_t* own_block = nullptr;          // moe_prefill_layer's intermediates (one allocation)
    moert::PrefillBufs own;
    const moert::PrefillBufs* last = nullptr;  // the set the last prefill call used
    moert::PrefillBufs scratch;            // moe_prefill_layer_noalloc's, in the device scratch
    // residency snapshot for the hit-D2D slab copies: id2slot as of the
    // first two-buffer call since the last decode call, resize or on-demand
    // pass (pinned [L*E]); entries of a layer admitted since are cleared
    int32_t* snap = nullptr;
    bool snap_valid = false;
    int64_t h2d_experts = 0, d2d_experts = 0;
  } pf;
  int64_t n_resizes = 0;

  moert::Timing* timing = nullptr;
  // a timing context's FFN launch: the ring slot's two events, bound to the
  // kernel's own dispatch (its start and end), set only around that launch
  hipEvent_t ffn_ev[2] = {nullptr, nullptr};

  moe_status err = MOE_OK;     // latched HIP error
  std::string err_msg;
};

namespace moert {

// error helpers --------------------------------------------------------------
void set_last_error(const std::string& s);
moe_status fail(moe_ctx* ctx, moe_status s, const std::string& msg);
moe_status hip_fail(moe_ctx* ctx, hipError_t e, const char* what);

#define MOE_HIP(ctx, expr)                                   \
  do {                                                       \
    hipError_t _e = (expr);                                  \
    if (_e != hipSuccess) return ::moert::hip_fail((ctx), _e, #expr); \
  } while (0)

inline int dtype_bytes(int d) { return d == MOE_F32 ? 4 : 2; }

// kernel launchers (defined in the .hip files) -------------------------------
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);
hipError_t launch_plan(moe_ctx* ctx, int layer, const int32_t* ids, int T, const void* x,
                       hipStream_t s);
// the fill of the last plan, plus its hand-off to the host branch (one more
// workgroup: the host block and the doorbell, when the plan has host work)
hipError_t launch_fill(moe_ctx* ctx, int layer, const int32_t* ids, int T, const void* x, hipStream_t s);
// resize compaction: n_moves (from, to) slot pairs (device, int32 [n][2]),
// no slot both read and written
hipError_t launch_slot_moves(moe_ctx* ctx, const int32_t* moves, int n_moves, hipStream_t s);
// the fill kernel on explicit lists: q = counts->q experts fill_u[i] of the
// mapped host banks to dst + fill_slot[i] * stride
hipError_t launch_fill_lists(const uint8_t* host_dev, uint8_t* dst, size_t stride,
                             const moe_plan_counts* counts, const int32_t* fill_u,
                             const int32_t* fill_slot, hipStream_t s);
double host_expert_seconds(moe_ctx* ctx, const int32_t* us, int n, int reps);
hipError_t launch_ffn(moe_ctx* ctx, const void* x, int T, hipStream_t s);
hipError_t launch_ffn_f32(moe_ctx* ctx, const void* x, int T, hipStream_t s);
hipError_t launch_ffn_bf16(moe_ctx* ctx, const void* x, int T, hipStream_t s);
hipError_t launch_ffn_mx(moe_ctx* ctx, const void* x, int T, hipStream_t s);
hipError_t launch_merge(moe_ctx* ctx, const float* w, int T, void* y, hipStream_t s);
hipError_t launch_prefill_admit(moe_ctx* ctx, int layer, int b, hipStream_t s);
// the full-layer buffer of a prefill layer: layer % 2 with two buffers, else 0
inline int prefill_buffer(const moe_ctx* ctx, int layer);
hipError_t launch_prefill_compute(moe_ctx* ctx, const PrefillBufs& pb, int layer, const void* x, int T,
                                  const int32_t* ids, const float* w, void* y, hipStream_t s);
// the three phases of launch_prefill_compute: grouping of the routed pairs;
// GEMM1 + GEMM2 over the experts of the layer's buffer (slot_of == nullptr)
// or over the experts slot_of maps (others skipped); the merge
hipError_t launch_prefill_group(moe_ctx* ctx, const PrefillBufs& pb, const int32_t* ids, int T,
                                hipStream_t s);
hipError_t launch_prefill_gemm(moe_ctx* ctx, const PrefillBufs& pb, int layer, const void* x, int T,
                               const int32_t* slot_of, hipStream_t s);
hipError_t launch_prefill_merge(moe_ctx* ctx, const PrefillBufs& pb, const int32_t* ids, const float* w,
                                int T, void* y, hipStream_t s);
hipError_t launch_prefill_pass_admit(moe_ctx* ctx, const PrefillBufs& pb, int layer, int p0, int P,
                                     hipStream_t s);
hipError_t launch_table_reset(moe_ctx* ctx, hipStream_t s);
moe_status prefill_settle(moe_ctx* ctx, hipStream_t s);

// timing mode: bracket a launch; no-ops when timing is off
hipError_t timing_begin(moe_ctx* ctx, int phase, hipStream_t s);
hipError_t timing_end(moe_ctx* ctx, hipStream_t s);
// A ring slot's two events for a launch to bind (not recorded here; both
// null without timing), and the slot's release once the launch is queued.
hipError_t timing_pair(moe_ctx* ctx, int phase, hipEvent_t* ev0, hipEvent_t* ev1);
void timing_commit(moe_ctx* ctx);

// host branch -----------------------------------------------------------------
CpuPool* cpu_pool_create(int threads);
void cpu_pool_destroy(CpuPool* p);
// Start / stop the doorbell poller of a context (worker 0 of its pool).
bool host_branch_start(moe_ctx* ctx);
void host_branch_stop(moe_ctx* ctx);
// True when every rung doorbell has been answered.
bool host_branch_idle(moe_ctx* ctx);

}  // namespace moert

inline int moert::prefill_buffer(const moe_ctx* ctx, int layer) {
  return ctx->pf.buffers == 2 ? (layer & 1) : 0;
}
