// Context lifecycle, slot pool, entry points and resize of the routed-expert
// MoE library.  Kernels live in the .hip files, the host branch in
// cpu_branch.cpp.
#include <unistd.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <thread>

#include "internal.h"

using namespace moert;

namespace moert {

static thread_local std::string g_last_error;

void set_last_error(const std::string& s) { g_last_error = s; }

moe_status fail(moe_ctx* ctx, moe_status s, const std::string& msg) {
  set_last_error(msg);
  if (ctx && s == MOE_EHIP) {
    ctx->err = MOE_EHIP;
    ctx->err_msg = msg;
  }
  return s;
}

moe_status hip_fail(moe_ctx* ctx, hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  if (e == hipErrorOutOfMemory) {
    set_last_error(m);
    return MOE_ENOMEM;
  }
  return fail(ctx, MOE_EHIP, m);
}

}  // namespace moert

// ------------------------------------------------------------------ config
static size_t expert_bytes_of(const moe_config* c) {
  size_t H = (size_t)c->hidden, I = (size_t)c->inter;
  switch (c->w_dtype) {
    case MOE_F32: return 12 * H * I;
    case MOE_BF16: return 6 * H * I;
    case MOE_MXFP4: return 3 * H * I / 2 + 3 * H * I / 32;
    default: return 0;
  }
}

// Row chunk (elements per 16-byte weight load) of a weight dtype.
static int chunk_elems(int w_dtype) { return w_dtype == MOE_F32 ? 4 : w_dtype == MOE_BF16 ? 8 : 32; }

// The decode GEMV gives every lane of a wave up to 8 of the NCH = K / chunk
// 16-byte chunks of a row, so NCH <= 512.
static bool row_split_ok(int K, int w_dtype) {
  int ch = chunk_elems(w_dtype);
  return K % ch == 0 && K / ch <= 512;
}

static std::string validate(const moe_config* c) {
  if (!c) return "config is NULL";
  if (c->n_layers < 1) return "n_layers must be >= 1";
  if (c->n_experts < 1 || c->n_experts > kMaxExperts) return "n_experts must be in 1..1024";
  if (c->top_k < 1 || c->top_k > std::min(c->n_experts, kMaxTopK)) return "top_k must be in 1..min(E,32)";
  if (c->w_dtype < MOE_F32 || c->w_dtype > MOE_MXFP4) return "w_dtype must be F32, BF16 or MXFP4";
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return "act_dtype must be F32 or BF16";
  if (c->hidden < 1 || c->inter < 1) return "hidden and inter must be positive";
  if (c->hidden % 64 || c->inter % 64) return "hidden and inter must be multiples of 64";
  if (!row_split_ok(c->hidden, c->w_dtype) || !row_split_ok(c->inter, c->w_dtype))
    return "hidden/inter too large for the decode GEMV (at most 512 sixteen-byte chunks per row)";
  if (c->max_slots < 0 || c->max_slots > kMaxSlots) return "max_slots must be in 0..32768";
  if (c->n_slots < 0 || c->n_slots > c->max_slots) return "n_slots must be in 0..max_slots";
  if (c->max_tokens < 1 || c->max_tokens > kMaxDecodeTokens) return "max_tokens must be in 1..256";
  if ((int64_t)c->max_tokens * c->top_k > 4096) return "max_tokens*top_k must be <= 4096";
  if (c->bw_pcie_mbps <= 0 || c->bw_host_mbps <= 0) return "bandwidths must be positive";
  if (c->bw_pcie_mbps > (int64_t)1 << 40 || c->bw_host_mbps > (int64_t)1 << 40) return "bandwidth too large";
  if (c->mode < MOE_HYBRID || c->mode > MOE_CPU) return "mode must be HYBRID, OFFLOAD or CPU";
  if (c->max_fetch < 0) return "max_fetch must be >= 0";
  if (c->cpu_threads < 0) return "cpu_threads must be >= 0";
  if (c->max_prefill_tokens < 0 || c->max_prefill_tokens > 65536) return "max_prefill_tokens must be in 0..65536";
  if ((int64_t)c->n_layers * c->n_experts > (int64_t)1 << 30) return "too many expert ids";
  // the grouped GEMM addresses an activation row (token rows of x, pair rows
  // of the intermediate) with a 32-bit byte offset from the tensor's base
  if (c->max_prefill_tokens > 0 &&
      ((int64_t)c->max_prefill_tokens * c->hidden * 2 >= ((int64_t)1 << 32) ||
       (int64_t)c->max_prefill_tokens * c->top_k * c->inter * 2 >= ((int64_t)1 << 32)))
    return "max_prefill_tokens too large: max_prefill_tokens*hidden*2 and "
           "max_prefill_tokens*top_k*inter*2 must stay below 2^32 bytes";
  return "";
}

extern "C" size_t moe_expert_bytes(const moe_config* cfg) {
  if (!validate(cfg).empty()) return 0;
  return (expert_bytes_of(cfg) + 255) / 256 * 256;
}

extern "C" const char* moe_strerror(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument or call order";
    case MOE_ENOMEM: return "out of memory";
    case MOE_ENOSPC: return "prefill needs at least one slot";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_EBUSY: return "busy";
    case MOE_ETIMEDOUT: return "timed out";
    case MOE_EUNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

extern "C" const char* moe_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ host pool
extern "C" moe_status moe_host_pool_alloc(size_t bytes, void** out) {
  if (!out || bytes == 0) return fail(nullptr, MOE_EINVAL, "moe_host_pool_alloc: bad arguments");
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess) {
    set_last_error(std::string("hipHostMalloc: ") + hipGetErrorString(e));
    return MOE_ENOMEM;
  }
  *out = p;
  return MOE_OK;
}

extern "C" moe_status moe_host_pool_free(void* p) {
  if (!p) return MOE_OK;
  hipError_t e = hipHostFree(p);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipHostFree");
  return MOE_OK;
}

// ------------------------------------------------------------------ slot pool
static bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && v[0] != '0';
}

static moe_status pool_map_to(moe_ctx* ctx, size_t need) {
  SlotPool& P = ctx->pool;
  if (!P.vmm) return need <= P.reserved ? MOE_OK : fail(ctx, MOE_ENOMEM, "slot pool exhausted");
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = ctx->device;
  while (P.mapped < need) {
    PoolChunk c{};
    c.offset = P.mapped;
    c.bytes = P.gran;
    MOE_HIP(ctx, hipMemCreate(&c.h, c.bytes, &prop, 0));
    hipError_t e = hipMemMap(P.base + c.offset, c.bytes, 0, c.h, 0);
    if (e != hipSuccess) {
      (void)hipMemRelease(c.h);
      return hip_fail(ctx, e, "hipMemMap");
    }
    hipMemAccessDesc acc = {};
    acc.location = prop.location;
    acc.flags = hipMemAccessFlagsProtReadWrite;
    MOE_HIP(ctx, hipMemSetAccess(P.base + c.offset, c.bytes, &acc, 1));
    P.chunks.push_back(c);
    P.mapped += c.bytes;
  }
  return MOE_OK;
}

static moe_status pool_unmap_to(moe_ctx* ctx, size_t need) {
  SlotPool& P = ctx->pool;
  if (!P.vmm) return MOE_OK;
  while (!P.chunks.empty() && P.chunks.back().offset >= need) {
    PoolChunk c = P.chunks.back();
    MOE_HIP(ctx, hipMemUnmap(P.base + c.offset, c.bytes));
    MOE_HIP(ctx, hipMemRelease(c.h));
    P.chunks.pop_back();
    P.mapped = c.offset;
  }
  return MOE_OK;
}

static moe_status pool_create(moe_ctx* ctx) {
  SlotPool& P = ctx->pool;
  size_t want = (size_t)ctx->cfg.max_slots * ctx->stride;
  int vmm = 0;
  (void)hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, ctx->device);
  P.vmm = vmm && !env_flag("MOERT_NO_VMM");
  if (P.vmm) {
    hipMemAllocationProp prop = {};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = ctx->device;
    size_t g = 0;
    if (hipMemGetAllocationGranularity(&g, &prop, hipMemAllocationGranularityMinimum) != hipSuccess ||
        g == 0) {
      P.vmm = false;
    } else {
      // chunks of 1/64 of the reserved range, 64 MiB to 1 GiB: every map or
      // unmap call costs about a quarter of a millisecond whatever its size,
      // so a large pool resizes in few calls and a small one keeps a fine
      // granularity
      const size_t chunk = std::min<size_t>((size_t)1 << 30, std::max<size_t>((size_t)64 << 20, want / 64));
      P.gran = (chunk + g - 1) / g * g;
      P.reserved = std::max<size_t>(P.gran, (want + P.gran - 1) / P.gran * P.gran);
      void* base = nullptr;
      if (hipMemAddressReserve(&base, P.reserved, 0, nullptr, 0) != hipSuccess) {
        P.vmm = false;
      } else {
        P.base = (uint8_t*)base;
      }
    }
  }
  if (!P.vmm) {
    P.reserved = std::max<size_t>(256, want);
    void* b = nullptr;
    MOE_HIP(ctx, hipMalloc(&b, P.reserved));
    P.base = (uint8_t*)b;
    P.mapped = P.reserved;
    return MOE_OK;
  }
  return pool_map_to(ctx, (size_t)ctx->cfg.n_slots * ctx->stride);
}

static void pool_destroy(moe_ctx* ctx) {
  SlotPool& P = ctx->pool;
  if (!P.base) return;
  if (P.vmm) {
    pool_unmap_to(ctx, 0);
    (void)hipMemAddressFree(P.base, P.reserved);
  } else {
    (void)hipFree(P.base);
  }
  P.base = nullptr;
}

// ------------------------------------------------------------------ create
static int32_t victim_bound(const moe_config& c, int32_t n_slots) {
  int64_t K = std::min<int64_t>((int64_t)c.max_tokens * c.top_k, c.n_experts);
  K = std::min<int64_t>(K, n_slots);
  if (c.max_fetch > 0) K = std::min<int64_t>(K, c.max_fetch);
  return (int32_t)K;
}

// Largest number of routed pairs whose prefill intermediates fit the fixed
// device scratch.
static int64_t scratch_pairs(const moe_config& c) {
  int64_t lo = 0, hi = (int64_t)65536 * kMaxTopK;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (prefill_layout(c, mid, nullptr, nullptr) <= kPrefillScratchBytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

static void free_all(moe_ctx* ctx);
static moe_status timing_create(moe_ctx* ctx);
static void timing_destroy(moe_ctx* ctx);

extern "C" moe_status moe_create(const moe_config* cfg, void* host_pool, size_t host_pool_bytes,
                                 moe_ctx** out) {
  std::string why = validate(cfg);
  if (!why.empty()) return fail(nullptr, MOE_EINVAL, "moe_create: " + why);
  if (!out) return fail(nullptr, MOE_EINVAL, "moe_create: out is NULL");
  size_t stride = moe_expert_bytes(cfg);
  int64_t n_ids = (int64_t)cfg->n_layers * cfg->n_experts;
  if (!host_pool || host_pool_bytes < (size_t)n_ids * stride)
    return fail(nullptr, MOE_EINVAL, "moe_create: host pool smaller than L*E banks");

  moe_ctx* ctx = new (std::nothrow) moe_ctx();
  if (!ctx) return fail(nullptr, MOE_ENOMEM, "moe_create: out of host memory");
  ctx->cfg = *cfg;
  ctx->stride = stride;
  ctx->expert_bytes = expert_bytes_of(cfg);
  ctx->n_ids = n_ids;
  ctx->n_slots = cfg->n_slots;
  ctx->umax = std::min(cfg->max_tokens * cfg->top_k, cfg->n_experts);
  ctx->kmax = std::max(1, victim_bound(*cfg, cfg->max_slots));
  ctx->host_pool = (uint8_t*)host_pool;
  ctx->host_pool_bytes = host_pool_bytes;
  moe_status st = MOE_OK;
  auto bail = [&](moe_status s) {
    free_all(ctx);
    delete ctx;
    return s;
  };
  (void)hipGetDevice(&ctx->device);

  void* hp_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&hp_dev, host_pool, 0);
  if (e != hipSuccess) {
    set_last_error(std::string("host pool is not pinned, mapped memory (hipHostGetDevicePointer: ") +
                   hipGetErrorString(e) + ")");
    delete ctx;
    return MOE_EUNSUPPORTED;
  }
  ctx->host_pool_dev = (const uint8_t*)hp_dev;

  if ((st = pool_create(ctx)) != MOE_OK) return bail(st);

  const int H = cfg->hidden, I = cfg->inter, k = cfg->top_k;
  const int maxTk = cfg->max_tokens * k;
#define ALLOC(ptr, bytes)                                                   \
  do {                                                                      \
    hipError_t _e = hipMalloc((void**)&(ptr), (bytes));                     \
    if (_e != hipSuccess) return bail(hip_fail(ctx, _e, "hipMalloc " #ptr)); \
  } while (0)
  ALLOC(ctx->id2slot, sizeof(int32_t) * n_ids);
  ALLOC(ctx->slot2id, sizeof(int32_t) * std::max(1, cfg->max_slots));
  ALLOC(ctx->slot_ts, sizeof(int64_t) * std::max(1, cfg->max_slots));
  ALLOC(ctx->dstate, sizeof(DevState));
  ALLOC(ctx->p_gpu, sizeof(float) * maxTk * H);
  ALLOC(ctx->h_mid, sizeof(uint64_t) * maxTk * I);

  // plan buffers: one allocation, 256-byte aligned sub-arrays
  {
    size_t off = 0;
    auto take = [&](size_t bytes) {
      size_t o = off;
      off += (bytes + 255) / 256 * 256;
      return o;
    };
    size_t o_counts = take(sizeof(moe_plan_counts));
    size_t o_uniq = take(4 * ctx->umax), o_hits = take(4 * ctx->umax), o_miss = take(4 * ctx->umax);
    size_t o_vic = take(4 * ctx->kmax), o_fu = take(4 * ctx->kmax), o_fs = take(4 * ctx->kmax),
           o_fo = take(4 * ctx->kmax);
    size_t o_cpu = take(4 * ctx->umax), o_gu = take(4 * ctx->umax), o_gs = take(4 * ctx->umax);
    size_t o_sm = take(4 * maxTk);
    size_t o_hw = take(4);
    ALLOC(ctx->plan_alloc, off);
    uint8_t* b = ctx->plan_alloc;
    PlanBufs& p = ctx->plan;
    p.counts = (moe_plan_counts*)(b + o_counts);
    p.uniq = (int32_t*)(b + o_uniq);
    p.hits = (int32_t*)(b + o_hits);
    p.misses = (int32_t*)(b + o_miss);
    p.victims = (int32_t*)(b + o_vic);
    p.fill_u = (int32_t*)(b + o_fu);
    p.fill_slot = (int32_t*)(b + o_fs);
    p.fill_old = (int32_t*)(b + o_fo);
    p.cpu_u = (int32_t*)(b + o_cpu);
    p.gpu_u = (int32_t*)(b + o_gu);
    p.gpu_slot = (int32_t*)(b + o_gs);
    p.slot_map = (int32_t*)(b + o_sm);
    p.h_marked = ctx->h_mid;
    p.h_words = (int64_t)maxTk * I;
    p.host_work = (int32_t*)(b + o_hw);
    p.hblock_bytes = sizeof(HostBlockHeader) + 2 * 4 * (size_t)maxTk;
    p.x_offset = (p.hblock_bytes + 255) / 256 * 256;
    p.act_bytes = dtype_bytes(cfg->act_dtype);
  }
#undef ALLOC

  // pinned, device-mapped memory: the host block (the fill launch's hand-off
  // workgroup -> host branch) and the host branch's output rows (host branch
  // -> merge)
  {
    void* p = nullptr;
    size_t hb = ctx->plan.x_offset + (size_t)cfg->max_tokens * H * ctx->plan.act_bytes;
    e = hipHostMalloc(&p, hb, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostMalloc host block"));
    ctx->hstage = (uint8_t*)p;
    ctx->xstage = ctx->hstage + ctx->plan.x_offset;
    memset(p, 0, hb);
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostGetDevicePointer host block"));
    ctx->plan.hblock = (uint8_t*)d;
    e = hipHostMalloc(&p, sizeof(HostSync), hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostMalloc host sync"));
    ctx->sync = (HostSync*)p;
    memset(p, 0, sizeof(HostSync));
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostGetDevicePointer host sync"));
    ctx->sync_dev = (HostSync*)d;
    e = hipHostMalloc(&p, sizeof(float) * maxTk * H, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostMalloc p_cpu"));
    ctx->p_cpu = (float*)p;
    memset(p, 0, sizeof(float) * maxTk * H);
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipHostGetDevicePointer p_cpu"));
    ctx->p_cpu_dev = (const float*)d;
  }

  e = hipStreamCreateWithFlags(&ctx->copy, hipStreamNonBlocking);
  if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipStreamCreate copy"));
  {
    int khz = 0;
    (void)hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, ctx->device);
    if (khz <= 0) khz = 100000;
    ctx->wait_ticks = (uint64_t)khz * 1000ull * 10ull;  // the merge waits at most 10 s
    ctx->ffn_wait_ticks = (uint64_t)khz * 1000ull;      // an FFN down item waits at most 1 s
  }

  // empty tables, tick 0
  e = launch_table_reset(ctx, ctx->copy);
  if (e != hipSuccess) return bail(hip_fail(ctx, e, "table reset"));
  e = hipStreamSynchronize(ctx->copy);
  if (e != hipSuccess) return bail(hip_fail(ctx, e, "table reset sync"));

  // Host expert bandwidth saturates well before every core is busy, and the
  // caller's issue thread and the HIP runtime threads need cores too: by
  // default use half the available cores, at most 8.
  int threads = cfg->cpu_threads;
  if (threads == 0) {
    cpu_set_t cs;
    int avail = (sched_getaffinity(0, sizeof cs, &cs) == 0) ? CPU_COUNT(&cs) : 1;
    threads = std::max(1, std::min(8, avail / 2));
  }
  ctx->cpu_threads = threads;
  ctx->cpu = cpu_pool_create(threads);
  if (!ctx->cpu) return bail(fail(nullptr, MOE_ENOMEM, "host worker pool"));
  if (!host_branch_start(ctx)) return bail(fail(nullptr, MOE_ENOMEM, "host branch poller"));
  if (cfg->timing && (st = timing_create(ctx)) != MOE_OK) return bail(st);
  if (cfg->max_prefill_tokens > 0) {
    // the prefill path's events and pinned staging, and the device address of
    // the library's fixed scratch on this device (the no-allocation prefill
    // entry point); moe_prefill_layer's own intermediates wait for its first call
    auto& pf = ctx->pf;
    for (int b = 0; b < 2 && e == hipSuccess; ++b)
      e = hipEventCreateWithFlags(&pf.ev_copied[b], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&pf.ev_start, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipHostMalloc((void**)&pf.counts_host, 8 * (size_t)cfg->n_experts, hipHostMallocDefault);
    if (e == hipSuccess)
      e = hipHostMalloc((void**)&pf.snap, 4 * (size_t)n_ids, hipHostMallocDefault);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "prefill events and staging"));
    e = prefill_scratch_init(ctx->device);
    if (e != hipSuccess) return bail(hip_fail(ctx, e, "hipGetSymbolAddress of the prefill scratch"));
    uint8_t* base = prefill_scratch_ptr(ctx->device);
    const int64_t pairs = std::min<int64_t>((int64_t)cfg->max_prefill_tokens * cfg->top_k,
                                            scratch_pairs(*cfg));
    if (base && pairs > 0) prefill_layout(*cfg, pairs, base, &pf.scratch);
    pf.ready = true;
  }
  *out = ctx;
  return MOE_OK;
}

static void free_all(moe_ctx* ctx) {
  if (ctx->copy) (void)hipStreamSynchronize(ctx->copy);
  host_branch_stop(ctx);
  timing_destroy(ctx);
  if (ctx->cpu) cpu_pool_destroy(ctx->cpu);
  ctx->cpu = nullptr;
  auto F = [](void* p) {
    if (p) (void)hipFree(p);
  };
  F(ctx->id2slot); F(ctx->slot2id); F(ctx->slot_ts); F(ctx->dstate);
  F(ctx->p_gpu); F(ctx->h_mid); F(ctx->plan_alloc);
  auto& pf = ctx->pf;
  F(pf.own_block);
  if (pf.counts_host) (void)hipHostFree(pf.counts_host);
  if (pf.snap) (void)hipHostFree(pf.snap);
  for (int b = 0; b < 2; ++b)
    if (pf.ev_copied[b]) (void)hipEventDestroy(pf.ev_copied[b]);
  if (pf.ev_start) (void)hipEventDestroy(pf.ev_start);
  if (ctx->hstage) (void)hipHostFree(ctx->hstage);
  if (ctx->p_cpu) (void)hipHostFree(ctx->p_cpu);
  if (ctx->sync) (void)hipHostFree(ctx->sync);
  if (ctx->copy) (void)hipStreamDestroy(ctx->copy);
  pool_destroy(ctx);
}

extern "C" moe_status moe_destroy(moe_ctx* ctx) {
  if (!ctx) return MOE_OK;
  (void)hipDeviceSynchronize();
  free_all(ctx);
  delete ctx;
  return MOE_OK;
}

// ------------------------------------------------------------------ timing
static moe_status timing_create(moe_ctx* ctx) {
  ctx->timing = new (std::nothrow) Timing();
  if (!ctx->timing) return fail(ctx, MOE_ENOMEM, "timing ring");
  Timing& T = *ctx->timing;
  T.a.resize(Timing::kRing);
  T.b.resize(Timing::kRing);
  T.phase.resize(Timing::kRing);
  // timing-only events: no system-scope fence (cache write-back and
  // invalidate) on record, which would also slow the work that follows
  for (int i = 0; i < Timing::kRing; ++i) {
    MOE_HIP(ctx, hipEventCreateWithFlags(&T.a[i], hipEventDisableSystemFence));
    MOE_HIP(ctx, hipEventCreateWithFlags(&T.b[i], hipEventDisableSystemFence));
  }
  return MOE_OK;
}

static void timing_destroy(moe_ctx* ctx) {
  if (!ctx->timing) return;
  for (auto e : ctx->timing->a) (void)hipEventDestroy(e);
  for (auto e : ctx->timing->b) (void)hipEventDestroy(e);
  delete ctx->timing;
  ctx->timing = nullptr;
}

// fold the oldest recorded pair into the totals
static hipError_t timing_harvest_one(Timing& T) {
  int idx = (T.head - T.used + Timing::kRing) % Timing::kRing;
  hipError_t e = hipEventSynchronize(T.b[idx]);
  if (e != hipSuccess) return e;
  float ms = 0.f;
  e = hipEventElapsedTime(&ms, T.a[idx], T.b[idx]);
  if (e != hipSuccess) return e;
  T.ms[T.phase[idx]] += ms;
  T.calls[T.phase[idx]] += 1;
  T.used -= 1;
  return hipSuccess;
}

hipError_t moert::timing_begin(moe_ctx* ctx, int phase, hipStream_t s) {
  if (!ctx->timing) return hipSuccess;
  Timing& T = *ctx->timing;
  if (T.used == Timing::kRing) {
    hipError_t e = timing_harvest_one(T);
    if (e != hipSuccess) return e;
  }
  T.phase[T.head] = phase;
  return hipEventRecord(T.a[T.head], s);
}

hipError_t moert::timing_pair(moe_ctx* ctx, int phase, hipEvent_t* ev0, hipEvent_t* ev1) {
  *ev0 = *ev1 = nullptr;
  if (!ctx->timing) return hipSuccess;
  Timing& T = *ctx->timing;
  if (T.used == Timing::kRing) {
    hipError_t e = timing_harvest_one(T);
    if (e != hipSuccess) return e;
  }
  T.phase[T.head] = phase;
  *ev0 = T.a[T.head];
  *ev1 = T.b[T.head];
  return hipSuccess;
}

void moert::timing_commit(moe_ctx* ctx) {
  if (!ctx->timing) return;
  Timing& T = *ctx->timing;
  T.head = (T.head + 1) % Timing::kRing;
  T.used += 1;
}

hipError_t moert::timing_end(moe_ctx* ctx, hipStream_t s) {
  if (!ctx->timing) return hipSuccess;
  Timing& T = *ctx->timing;
  hipError_t e = hipEventRecord(T.b[T.head], s);
  T.head = (T.head + 1) % Timing::kRing;
  T.used += 1;
  return e;
}

extern "C" moe_status moe_ctx_timing(moe_ctx* ctx, moe_timing* out, int32_t reset) {
  if (!ctx || !out) return fail(nullptr, MOE_EINVAL, "moe_ctx_timing: NULL argument");
  if (!ctx->timing) return fail(ctx, MOE_EINVAL, "moe_ctx_timing: context created without timing");
  MOE_HIP(ctx, hipDeviceSynchronize());
  Timing& T = *ctx->timing;
  while (T.used > 0) MOE_HIP(ctx, timing_harvest_one(T));
  for (int i = 0; i < MOE_T_COUNT; ++i) {
    out->calls[i] = T.calls[i];
    out->ms[i] = T.ms[i];
  }
  out->calls[MOE_T_HOST] = T.host_calls.load();
  out->ms[MOE_T_HOST] = T.host_ns.load() * 1e-6;
  if (reset) {
    for (int i = 0; i < MOE_T_COUNT; ++i) {
      T.calls[i] = 0;
      T.ms[i] = 0;
    }
    T.host_calls = 0;
    T.host_ns = 0;
  }
  return MOE_OK;
}

// ------------------------------------------------------------------ calls
#define CHECK_CTX(ctx)                                                        \
  do {                                                                        \
    if (!(ctx)) return fail(nullptr, MOE_EINVAL, "context is NULL");          \
    if ((ctx)->sync && ((volatile HostSync*)(ctx)->sync)->error && (ctx)->err == MOE_OK) \
      fail((ctx), MOE_EHIP, ((volatile HostSync*)(ctx)->sync)->error == 2                \
                                ? "expert FFN gave up waiting for its gate/up items (1 s limit)" \
                                : "merge gave up waiting for the host branch (10 s limit)");      \
    if ((ctx)->err != MOE_OK) {                                               \
      set_last_error((ctx)->err_msg);                                         \
      return (ctx)->err;                                                      \
    }                                                                         \
  } while (0)

extern "C" moe_status moe_route_topk(moe_ctx* ctx, const float* logits, int32_t T, int32_t* ids,
                                     float* w, moe_stream stream) {
  CHECK_CTX(ctx);
  int tmax = std::max(ctx->cfg.max_tokens, ctx->cfg.max_prefill_tokens);
  if (!logits || !ids || !w || T < 1 || T > tmax)
    return fail(ctx, MOE_EINVAL, "moe_route_topk: bad arguments");
  MOE_HIP(ctx, timing_begin(ctx, MOE_T_ROUTE, (hipStream_t)stream));
  MOE_HIP(ctx, launch_route_topk(logits, T, ctx->cfg.n_experts, ctx->cfg.top_k, ids, w,
                                 (hipStream_t)stream));
  MOE_HIP(ctx, timing_end(ctx, (hipStream_t)stream));
  return MOE_OK;
}

extern "C" moe_status moe_cache_plan(moe_ctx* ctx, int32_t layer, const int32_t* ids, int32_t T,
                                     const void* x, moe_stream stream) {
  CHECK_CTX(ctx);
  if (!ids || !x || layer < 0 || layer >= ctx->cfg.n_layers || T < 1 || T > ctx->cfg.max_tokens)
    return fail(ctx, MOE_EINVAL, "moe_cache_plan: bad arguments");
  if (((uintptr_t)x & 15) || ((uintptr_t)ids & 3))
    return fail(ctx, MOE_EINVAL, "moe_cache_plan: x must be 16-byte aligned, ids 4-byte aligned");
  if (ctx->state != kIdle)
    return fail(ctx, MOE_EINVAL, "moe_cache_plan: previous layer call was not merged");
  hipStream_t s = (hipStream_t)stream;
  moe_status pst = prefill_settle(ctx, s);
  if (pst != MOE_OK) return pst;
  ctx->pf.snap_valid = false;  // fills may overwrite any slot outside the call's hits
  // The control kernel decides; the next launch hands the host branch its
  // work (doorbell in pinned memory, answered by the poller thread) while it
  // fills the admitted experts.
  MOE_HIP(ctx, timing_begin(ctx, MOE_T_PLAN, s));
  MOE_HIP(ctx, launch_plan(ctx, layer, ids, T, x, s));
  MOE_HIP(ctx, timing_end(ctx, s));
  // GPU miss path: batched copy of the admitted experts into their slots;
  // one more workgroup of the same launch hands the CPU set to the host branch
  MOE_HIP(ctx, timing_begin(ctx, MOE_T_FILL, s));
  MOE_HIP(ctx, launch_fill(ctx, layer, ids, T, x, s));
  MOE_HIP(ctx, timing_end(ctx, s));
  ctx->state = kPlanned;
  ctx->cur_layer = layer;
  ctx->cur_T = T;
  return MOE_OK;
}

extern "C" moe_status moe_expert_ffn(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                                     moe_stream stream) {
  CHECK_CTX(ctx);
  if (!x || ctx->state != kPlanned || layer != ctx->cur_layer || T != ctx->cur_T)
    return fail(ctx, MOE_EINVAL, "moe_expert_ffn: must follow moe_cache_plan of the same layer and T");
  if ((uintptr_t)x & 15) return fail(ctx, MOE_EINVAL, "moe_expert_ffn: x must be 16-byte aligned");
  // timed by events bound to the kernel's own dispatch (its start and end),
  // not recorded around it on the stream
  MOE_HIP(ctx, timing_pair(ctx, MOE_T_FFN, &ctx->ffn_ev[0], &ctx->ffn_ev[1]));
  const hipError_t le = launch_ffn(ctx, x, T, (hipStream_t)stream);
  ctx->ffn_ev[0] = ctx->ffn_ev[1] = nullptr;
  MOE_HIP(ctx, le);
  timing_commit(ctx);
  ctx->state = kEvaluated;
  return MOE_OK;
}

extern "C" moe_status moe_merge(moe_ctx* ctx, const float* w, int32_t T, void* y,
                                moe_stream stream) {
  CHECK_CTX(ctx);
  if (!w || !y || ctx->state != kEvaluated || T != ctx->cur_T)
    return fail(ctx, MOE_EINVAL, "moe_merge: must follow moe_expert_ffn with the same T");
  hipStream_t s = (hipStream_t)stream;
  MOE_HIP(ctx, timing_begin(ctx, MOE_T_MERGE, s));
  MOE_HIP(ctx, launch_merge(ctx, w, T, y, s));
  MOE_HIP(ctx, timing_end(ctx, s));
  ctx->state = kIdle;
  return MOE_OK;
}

extern "C" moe_status moe_plan_view_get(moe_ctx* ctx, moe_plan_view* v) {
  if (!ctx || !v) return fail(nullptr, MOE_EINVAL, "moe_plan_view_get: NULL argument");
  PlanBufs& p = ctx->plan;
  v->counts = p.counts;
  v->uniq = p.uniq; v->hits = p.hits; v->misses = p.misses; v->victims = p.victims;
  v->fill_u = p.fill_u; v->fill_slot = p.fill_slot; v->fill_old = p.fill_old;
  v->cpu_u = p.cpu_u; v->gpu_u = p.gpu_u; v->gpu_slot = p.gpu_slot; v->slot_map = p.slot_map;
  v->id2slot = ctx->id2slot; v->slot2id = ctx->slot2id; v->slot_ts = ctx->slot_ts;
  v->tick = &ctx->dstate->tick;
  v->p_gpu = ctx->p_gpu; v->p_cpu = ctx->p_cpu;
  v->slot_base = ctx->pool.base;
  v->n_slots = ctx->n_slots; v->max_slots = ctx->cfg.max_slots;
  v->umax = ctx->umax; v->kmax = ctx->kmax;
  v->h_marked = ctx->h_mid;
  return MOE_OK;
}

extern "C" moe_status moe_prefill_view_get(moe_ctx* ctx, moe_prefill_view* v) {
  if (!ctx || !v) return fail(nullptr, MOE_EINVAL, "moe_prefill_view_get: NULL argument");
  const PrefillBufs* pb = ctx->pf.last;
  if (!pb) return fail(ctx, MOE_EINVAL, "moe_prefill_view_get: no prefill layer has run");
  v->counts = pb->counts;
  v->offsets = pb->offsets;
  v->perm = pb->perm;
  v->tiles = pb->tiles;
  v->hmid = pb->hmid;
  v->prow = pb->prow;
  v->n_experts = ctx->cfg.n_experts;
  v->max_pairs = (int32_t)pb->max_pairs;
  v->max_tiles = pb->max_tiles;
  return MOE_OK;
}

extern "C" moe_status moe_ctx_stats(moe_ctx* ctx, moe_stats* out) {
  CHECK_CTX(ctx);
  if (!out) return fail(ctx, MOE_EINVAL, "moe_ctx_stats: out is NULL");
  MOE_HIP(ctx, hipDeviceSynchronize());
  DevState ds;
  MOE_HIP(ctx, hipMemcpy(&ds, ctx->dstate, sizeof ds, hipMemcpyDeviceToHost));
  std::vector<int32_t> s2i(std::max(1, ctx->n_slots));
  if (ctx->n_slots)
    MOE_HIP(ctx, hipMemcpy(s2i.data(), ctx->slot2id, 4 * (size_t)ctx->n_slots, hipMemcpyDeviceToHost));
  out->n_slots = ctx->n_slots;
  out->occupied = 0;
  for (int s = 0; s < ctx->n_slots; ++s) out->occupied += s2i[s] >= 0;
  out->plans = ds.plans; out->hits = ds.hits; out->fills = ds.fills; out->cpu = ds.cpu;
  out->evictions = ds.evictions; out->prefill_layers = ds.prefill_layers;
  out->resizes = ctx->n_resizes;
  out->prefill_h2d_experts = ctx->pf.h2d_experts;
  out->prefill_d2d_experts = ctx->pf.d2d_experts;
  return MOE_OK;
}

// ------------------------------------------------------------------ resize
static moe_status drain(moe_ctx* ctx, int32_t timeout_ms) {
  auto t0 = std::chrono::steady_clock::now();
  hipEvent_t ev;
  MOE_HIP(ctx, hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  // everything enqueued on the device so far, on any stream
  hipError_t e = hipEventRecord(ev, nullptr);
  if (e != hipSuccess) {
    (void)hipEventDestroy(ev);
    return hip_fail(ctx, e, "hipEventRecord");
  }
  for (;;) {
    bool done = hipEventQuery(ev) == hipSuccess && hipStreamQuery(ctx->copy) == hipSuccess &&
                host_branch_idle(ctx);
    if (done) break;
    double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (timeout_ms >= 0 && ms > timeout_ms) {
      (void)hipEventDestroy(ev);
      return fail(ctx, MOE_ETIMEDOUT, "moe_cache_resize: work still in flight");
    }
    std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
  (void)hipEventDestroy(ev);
  MOE_HIP(ctx, hipDeviceSynchronize());
  return MOE_OK;
}

extern "C" moe_status moe_cache_resize(moe_ctx* ctx, int32_t new_n, int32_t timeout_ms) {
  CHECK_CTX(ctx);
  if (new_n < 0 || new_n > ctx->cfg.max_slots)
    return fail(ctx, MOE_EINVAL, "moe_cache_resize: new_n_slots out of 0..max_slots");
  if (ctx->state != kIdle) return fail(ctx, MOE_EINVAL, "moe_cache_resize: a layer call is open");
  moe_status st = drain(ctx, timeout_ms);
  if (st != MOE_OK) return st;
  // a slab streamed ahead for the next prefill layer and not yet consumed is
  // in its buffer now (drain waited for the copy stream): admit it, as a
  // decode call would, so the tables describe every slot's bytes before the
  // keep set is chosen
  if ((st = prefill_settle(ctx, ctx->copy)) != MOE_OK) return st;
  MOE_HIP(ctx, hipStreamSynchronize(ctx->copy));
  const int32_t n = ctx->n_slots;
  std::vector<int32_t> s2i(std::max(1, n));
  std::vector<int64_t> ts(std::max(1, n));
  if (n) {
    MOE_HIP(ctx, hipMemcpy(s2i.data(), ctx->slot2id, 4 * (size_t)n, hipMemcpyDeviceToHost));
    MOE_HIP(ctx, hipMemcpy(ts.data(), ctx->slot_ts, 8 * (size_t)n, hipMemcpyDeviceToHost));
  }
  // evict in victim order, (tick, slot) ascending, until new_n remain
  std::vector<int32_t> occ;
  for (int s = 0; s < n; ++s)
    if (s2i[s] >= 0) occ.push_back(s);
  std::vector<int32_t> lru = occ;
  std::stable_sort(lru.begin(), lru.end(), [&](int a, int b) {
    return ts[a] != ts[b] ? ts[a] < ts[b] : a < b;
  });
  size_t n_keep = std::min<size_t>((size_t)new_n, occ.size());
  std::vector<char> keep(std::max(1, n), 0);
  for (size_t i = lru.size() - n_keep; i < lru.size(); ++i) keep[lru[i]] = 1;
  // new tables: a survivor below new_n keeps its slot; the survivors at or
  // beyond it take the free slots below it, both in ascending order, so the
  // fewest bytes move and no move reads a slot another move writes
  std::vector<int32_t> i2s((size_t)ctx->n_ids, -1);
  std::vector<int32_t> ns2i(std::max(1, new_n), -1);
  std::vector<int64_t> nts(std::max(1, new_n), -1);
  std::vector<int32_t> moves;  // (from, to) pairs
  for (int s = 0; s < std::min(n, new_n); ++s) {
    if (!keep[s]) continue;
    ns2i[s] = s2i[s];
    nts[s] = ts[s];
    i2s[s2i[s]] = s;
  }
  int32_t hole = 0;
  for (int s = new_n; s < n; ++s) {
    if (!keep[s]) continue;
    while (ns2i[hole] >= 0) ++hole;  // a free slot below new_n exists: kept <= new_n
    ns2i[hole] = s2i[s];
    nts[hole] = ts[s];
    i2s[s2i[s]] = hole;
    moves.push_back(s);
    moves.push_back(hole);
  }
  const int n_moves = (int)moves.size() / 2;
  // grow the mapping first, move the survivors, then release the tail
  size_t need = (size_t)std::max(new_n, n) * ctx->stride;
  if ((st = pool_map_to(ctx, need)) != MOE_OK) return st;
  int32_t* moves_dev = nullptr;
  if (n_moves) {
    MOE_HIP(ctx, hipMalloc((void**)&moves_dev, 4 * moves.size()));
    hipError_t e = hipMemcpyAsync(moves_dev, moves.data(), 4 * moves.size(), hipMemcpyHostToDevice, ctx->copy);
    if (e == hipSuccess) e = launch_slot_moves(ctx, moves_dev, n_moves, ctx->copy);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->copy);
    (void)hipFree(moves_dev);
    MOE_HIP(ctx, e);
  }
  MOE_HIP(ctx, hipMemcpyAsync(ctx->id2slot, i2s.data(), 4 * i2s.size(), hipMemcpyHostToDevice, ctx->copy));
  if (new_n) {
    MOE_HIP(ctx, hipMemcpyAsync(ctx->slot2id, ns2i.data(), 4 * (size_t)new_n, hipMemcpyHostToDevice, ctx->copy));
    MOE_HIP(ctx, hipMemcpyAsync(ctx->slot_ts, nts.data(), 8 * (size_t)new_n, hipMemcpyHostToDevice, ctx->copy));
  }
  int32_t nn = new_n;
  MOE_HIP(ctx, hipMemcpyAsync(&ctx->dstate->n_slots, &nn, 4, hipMemcpyHostToDevice, ctx->copy));
  MOE_HIP(ctx, hipStreamSynchronize(ctx->copy));
  if ((st = pool_unmap_to(ctx, (size_t)new_n * ctx->stride)) != MOE_OK) return st;
  ctx->n_slots = new_n;
  ctx->pf.snap_valid = false;
  ctx->n_resizes += 1;
  return MOE_OK;
}

// ------------------------------------------------------------------ bandwidths
extern "C" moe_status moe_measure_bandwidth(moe_ctx* ctx, int32_t n_experts, int32_t reps,
                                            int64_t* bw_pcie_mbps, int64_t* bw_host_mbps,
                                            int64_t* bw_h2d_mbps) {
  CHECK_CTX(ctx);
  if (!bw_pcie_mbps || !bw_host_mbps || n_experts < 1 || reps < 1 || reps > 1000)
    return fail(ctx, MOE_EINVAL, "moe_measure_bandwidth: bad arguments");
  if (ctx->state != kIdle) return fail(ctx, MOE_EINVAL, "moe_measure_bandwidth: a layer call is open");
  moe_status st = drain(ctx, 60000);
  if (st != MOE_OK) return st;
  const int n = (int)std::min<int64_t>({(int64_t)n_experts, ctx->n_ids, 64});
  // reps + 1 sets of n experts spread over the host pool, distinct while the
  // pool has enough ids, so neither side re-reads bytes a cache may hold
  const int64_t total = (int64_t)n * (reps + 1);
  std::vector<int32_t> us(total), slots(n);
  for (int64_t i = 0; i < total; ++i)
    us[i] = (int32_t)(total <= ctx->n_ids ? i * ctx->n_ids / total : i % ctx->n_ids);
  for (int i = 0; i < n; ++i) slots[i] = i;
  const double bytes = (double)n * (double)ctx->expert_bytes;

  // PCIe: the fill kernel pulling each set into a scratch device buffer (the
  // slot pool and the tables are not touched)
  const size_t o_cnt = (size_t)n * ctx->stride, o_fs = o_cnt + 256, o_fu = o_fs + 256;
  uint8_t* buf = nullptr;
  MOE_HIP(ctx, hipMalloc(&buf, o_fu + 4 * (size_t)total));
  moe_plan_counts cnt{};
  cnt.q = n;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.f;
  hipError_t e = hipMemcpy(buf + o_cnt, &cnt, sizeof cnt, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(buf + o_fu, us.data(), 4 * (size_t)total, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(buf + o_fs, slots.data(), 4 * (size_t)n, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  auto pull = [&](int r) {
    return launch_fill_lists(ctx->host_pool_dev, buf, ctx->stride, (const moe_plan_counts*)(buf + o_cnt),
                             (const int32_t*)(buf + o_fu) + (size_t)r * n, (const int32_t*)(buf + o_fs),
                             ctx->copy);
  };
  if (e == hipSuccess) e = pull(0);  // untimed
  if (e == hipSuccess) e = hipEventRecord(e0, ctx->copy);
  for (int r = 1; r <= reps && e == hipSuccess; ++r) e = pull(r);
  if (e == hipSuccess) e = hipEventRecord(e1, ctx->copy);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  // the same sets as pinned host-to-device copies (the copy engines), one per expert
  float ms_h2d = 0.f;
  if (bw_h2d_mbps) {
    auto copy_set = [&](int r) {
      hipError_t ce = hipSuccess;
      for (int i = 0; i < n && ce == hipSuccess; ++i)
        ce = hipMemcpyAsync(buf + (size_t)i * ctx->stride,
                            ctx->host_pool + (size_t)us[(size_t)r * n + i] * ctx->stride, ctx->expert_bytes,
                            hipMemcpyHostToDevice, ctx->copy);
      return ce;
    };
    if (e == hipSuccess) e = copy_set(0);
    if (e == hipSuccess) e = hipEventRecord(e0, ctx->copy);
    for (int r = 1; r <= reps && e == hipSuccess; ++r) e = copy_set(r);
    if (e == hipSuccess) e = hipEventRecord(e1, ctx->copy);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms_h2d, e0, e1);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(buf);
  if (e != hipSuccess) return hip_fail(ctx, e, "moe_measure_bandwidth (PCIe pull)");
  const double pcie = bytes * reps / (ms * 1e-3) / 1e6;

  // host: the host branch's expert arithmetic on its worker pool
  const double secs = host_expert_seconds(ctx, us.data(), n, reps);
  const double host = bytes / secs / 1e6;
  *bw_pcie_mbps = std::max<int64_t>(1, (int64_t)std::llround(pcie));
  if (bw_h2d_mbps) *bw_h2d_mbps = std::max<int64_t>(1, (int64_t)std::llround(bytes * reps / (ms_h2d * 1e-3) / 1e6));
  *bw_host_mbps = std::max<int64_t>(1, (int64_t)std::llround(host));
  return MOE_OK;
}

extern "C" moe_status moe_recommend_mode(int64_t bw_pcie_mbps, int64_t bw_host_mbps, double threshold,
                                         moe_mode* out) {
  if (!out || bw_pcie_mbps <= 0 || bw_host_mbps <= 0 || !(threshold > 0.0))
    return fail(nullptr, MOE_EINVAL, "moe_recommend_mode: bad arguments");
  *out = (double)bw_host_mbps > threshold * (double)bw_pcie_mbps ? MOE_HYBRID : MOE_OFFLOAD;
  return MOE_OK;
}

extern "C" moe_status moe_set_cpu_layers(moe_ctx* ctx, const uint8_t* flags, int32_t n_layers) {
  CHECK_CTX(ctx);
  if (flags && n_layers != ctx->cfg.n_layers)
    return fail(ctx, MOE_EINVAL, "moe_set_cpu_layers: n_layers must equal the context's layer count");
  if (ctx->state != kIdle) return fail(ctx, MOE_EINVAL, "moe_set_cpu_layers: a layer call is open");
  if (!flags) ctx->cpu_layers.clear();
  else ctx->cpu_layers.assign(flags, flags + n_layers);
  return MOE_OK;
}

extern "C" moe_status moe_set_split(moe_ctx* ctx, int64_t bw_pcie_mbps, int64_t bw_host_mbps,
                                    moe_mode mode) {
  CHECK_CTX(ctx);
  if (bw_pcie_mbps <= 0 || bw_host_mbps <= 0 || bw_pcie_mbps > (int64_t)1 << 40 ||
      bw_host_mbps > (int64_t)1 << 40 || mode < MOE_HYBRID || mode > MOE_CPU)
    return fail(ctx, MOE_EINVAL, "moe_set_split: bad arguments");
  if (ctx->state != kIdle) return fail(ctx, MOE_EINVAL, "moe_set_split: a layer call is open");
  ctx->cfg.bw_pcie_mbps = bw_pcie_mbps;
  ctx->cfg.bw_host_mbps = bw_host_mbps;
  ctx->cfg.mode = mode;
  return MOE_OK;
}

// ------------------------------------------------------------------ prefill
// moe_prefill_layer's intermediates, sized for max_prefill_tokens, allocated
// on its first call (one block).
static moe_status prefill_setup(moe_ctx* ctx) {
  auto& pf = ctx->pf;
  if (pf.own_block) return MOE_OK;
  const moe_config& c = ctx->cfg;
  const int64_t pairs = (int64_t)c.max_prefill_tokens * c.top_k;
  uint8_t* block = nullptr;
  MOE_HIP(ctx, hipMalloc((void**)&block, prefill_layout(c, pairs, nullptr, nullptr)));
  prefill_layout(c, pairs, block, &pf.own);
  pf.own_block = block;
  return MOE_OK;
}

// Issue the slab copy of `layer` into its buffer on the copy stream.
// It waits for everything enqueued on the caller's stream before this call
// (ev_start): earlier readers of that buffer, decode work on those slots.
// Experts of the layer resident in a slot outside the full-layer buffers (by
// the residency snapshot) come device to device; the others cross PCIe from
// the host pool, one copy per run of consecutive experts (satyajit, "Four
// backends, and the one that has to be measured": cache hits cross no bus).
// A source slot outside the buffers is written only by decode fills and
// resizes, and both invalidate the snapshot and wait for this copy first.
static moe_status prefill_issue(moe_ctx* ctx, int32_t layer) {
  auto& pf = ctx->pf;
  const int b = prefill_buffer(ctx, layer);
  const int E = ctx->cfg.n_experts;
  const int outside = pf.buffers * E;  // first slot outside the buffers
  const size_t st = ctx->stride;
  uint8_t* dst = ctx->pool.base + (size_t)b * E * st;
  const int32_t* res = pf.snap_valid ? pf.snap + (size_t)layer * E : nullptr;
  auto resident = [&](int e) { return res && res[e] >= outside ? res[e] : -1; };
  MOE_HIP(ctx, hipStreamWaitEvent(ctx->copy, pf.ev_start, 0));
  MOE_HIP(ctx, timing_begin(ctx, MOE_T_PREFILL_COPY, ctx->copy));
  for (int e = 0; e < E;) {
    const int from = resident(e);
    if (from >= 0) {
      MOE_HIP(ctx, hipMemcpyAsync(dst + (size_t)e * st, ctx->pool.base + (size_t)from * st, st,
                                  hipMemcpyDeviceToDevice, ctx->copy));
      pf.d2d_experts += 1;
      ++e;
      continue;
    }
    int j = e + 1;
    while (j < E && resident(j) < 0) ++j;
    MOE_HIP(ctx, hipMemcpyAsync(dst + (size_t)e * st, ctx->host_pool + ((size_t)layer * E + e) * st,
                                (size_t)(j - e) * st, hipMemcpyHostToDevice, ctx->copy));
    pf.h2d_experts += j - e;
    e = j;
  }
  MOE_HIP(ctx, timing_end(ctx, ctx->copy));
  MOE_HIP(ctx, hipEventRecord(pf.ev_copied[b], ctx->copy));
  pf.buf_layer[b] = layer;
  pf.admitted[b] = false;
  return MOE_OK;
}

// A prefetched slab that no prefill call consumed is admitted before decode
// touches the pool, so the tables describe what the slots hold.
moe_status moert::prefill_settle(moe_ctx* ctx, hipStream_t s) {
  auto& pf = ctx->pf;
  if (!pf.ready) return MOE_OK;
  for (int b = 0; b < 2; ++b) {
    if (pf.buf_layer[b] >= 0 && !pf.admitted[b]) {
      MOE_HIP(ctx, hipStreamWaitEvent(s, pf.ev_copied[b], 0));
      MOE_HIP(ctx, launch_prefill_admit(ctx, pf.buf_layer[b], b, s));
      pf.admitted[b] = true;
    }
    pf.buf_layer[b] = -1;  // decode fills may overwrite the buffer from here on
  }
  return MOE_OK;
}

// On-demand prefill, used when the pool cannot hold the full-layer buffers
// (signalovernoise essay; snackonai, "The Architecture, Unpacked"): the
// layer's routed experts are known only after routing, so the host reads the
// per-expert counts and the layer's row of id2slot (one stream
// synchronisation per layer), then loads the routed experts in ascending
// order, at most n_slots per pass, into slots [0, P), and runs the grouped
// GEMM over that pass's experts only.  Each pass writes the partial rows of
// its own pairs, so one merge after the last pass sees every pair once.
// Cache hits cross no bus (satyajit, "Four backends, and the one that has
// to be measured": the prefill hit-D2D option): in the first pass an expert already in its target
// slot is not copied, and one resident in a slot at or beyond P (which no copy
// of the pass writes) is copied device to device; every other expert comes
// from its host bank, one copy per run of consecutive experts.  Later passes
// find nothing of theirs resident: the first pass filled every slot.
static moe_status prefill_on_demand(moe_ctx* ctx, const PrefillBufs& pb, int32_t layer, const void* x,
                                    int32_t T, const int32_t* ids, const float* w, void* y, hipStream_t s) {
  auto& pf = ctx->pf;
  const int E = ctx->cfg.n_experts;
  moe_status st = prefill_settle(ctx, s);
  if (st != MOE_OK) return st;
  pf.snap_valid = false;  // the passes rewrite slots [0, P)
  MOE_HIP(ctx, launch_prefill_group(ctx, pb, ids, T, s));
  int32_t* counts = pf.counts_host;
  int32_t* resident = pf.counts_host + E;
  MOE_HIP(ctx, hipMemcpyAsync(counts, pb.counts, 4 * (size_t)E, hipMemcpyDeviceToHost, s));
  MOE_HIP(ctx, hipMemcpyAsync(resident, ctx->id2slot + (size_t)layer * E, 4 * (size_t)E,
                              hipMemcpyDeviceToHost, s));
  MOE_HIP(ctx, hipStreamSynchronize(s));
  int32_t routed[kMaxExperts];
  int nu = 0;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) routed[nu++] = e;
  const int n = ctx->n_slots;
  for (int p0 = 0; p0 < nu; p0 += n) {
    const int P = std::min(n, nu - p0);
    MOE_HIP(ctx, launch_prefill_pass_admit(ctx, pb, layer, p0, P, s));
    MOE_HIP(ctx, timing_begin(ctx, MOE_T_PREFILL_COPY, s));
    for (int i = 0; i < P;) {
      const int e = routed[p0 + i];
      const int from = p0 == 0 ? resident[e] : -1;
      if (from == i) {  // already in place
        ++i;
        continue;
      }
      if (from >= P) {  // resident beyond the pass's slots: device to device
        MOE_HIP(ctx, hipMemcpyAsync(ctx->pool.base + (size_t)i * ctx->stride,
                                    ctx->pool.base + (size_t)from * ctx->stride, ctx->stride,
                                    hipMemcpyDeviceToDevice, s));
        pf.d2d_experts += 1;
        ++i;
        continue;
      }
      int j = i + 1;  // a run of consecutive experts that cross the bus
      while (j < P && routed[p0 + j] == routed[p0 + j - 1] + 1 &&
             (p0 != 0 || (resident[routed[p0 + j]] != j && resident[routed[p0 + j]] < P)))
        ++j;
      MOE_HIP(ctx, hipMemcpyAsync(ctx->pool.base + (size_t)i * ctx->stride,
                                  ctx->host_pool + ((size_t)layer * E + e) * ctx->stride,
                                  (size_t)(j - i) * ctx->stride, hipMemcpyHostToDevice, s));
      pf.h2d_experts += j - i;
      i = j;
    }
    MOE_HIP(ctx, timing_end(ctx, s));
    MOE_HIP(ctx, launch_prefill_gemm(ctx, pb, layer, x, T, pb.slot_of, s));
  }
  MOE_HIP(ctx, launch_prefill_merge(ctx, pb, ids, w, T, y, s));
  return MOE_OK;
}

extern "C" moe_status moe_prefill_set_buffers(moe_ctx* ctx, int32_t n_buffers) {
  CHECK_CTX(ctx);
  if (n_buffers != 1 && n_buffers != 2)
    return fail(ctx, MOE_EINVAL, "moe_prefill_set_buffers: n_buffers must be 1 or 2");
  if (ctx->state != kIdle) return fail(ctx, MOE_EINVAL, "moe_prefill_set_buffers: a layer call is open");
  auto& pf = ctx->pf;
  for (int b = 0; b < 2; ++b)
    if (pf.buf_layer[b] >= 0 && !pf.admitted[b])
      return fail(ctx, MOE_EBUSY, "moe_prefill_set_buffers: a prefetched slab is pending");
  if (pf.buffers != n_buffers) {
    // a slab issued under the other mapping no longer names its buffer
    pf.buf_layer[0] = pf.buf_layer[1] = -1;
    pf.buffers = n_buffers;
  }
  return MOE_OK;
}

// Argument checks shared by both prefill entry points.
static moe_status prefill_check(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* ids,
                                const float* w, void* y, const char* where) {
  const moe_config& c = ctx->cfg;
  if (!x || !ids || !w || !y || layer < 0 || layer >= c.n_layers || T < 1 || T > c.max_prefill_tokens)
    return fail(ctx, MOE_EINVAL, std::string(where) + ": bad arguments");
  if (ctx->state != kIdle)
    return fail(ctx, MOE_EINVAL, std::string(where) + ": a decode layer call is open");
  if (c.w_dtype != MOE_MXFP4 || c.act_dtype != MOE_BF16 || c.hidden % 256 || c.inter % 128)
    return fail(ctx, MOE_EUNSUPPORTED,
                std::string(where) + ": the grouped GEMM takes MXFP4 experts, bf16 activations, "
                "hidden % 256 == 0 and inter % 128 == 0");
  if (((uintptr_t)x & 15) || ((uintptr_t)ids & 3) || ((uintptr_t)w & 3) || ((uintptr_t)y & 3))
    return fail(ctx, MOE_EINVAL, std::string(where) + ": x must be 16-byte aligned");
  if (ctx->n_slots < 1) return fail(ctx, MOE_ENOSPC, std::string(where) + ": the slot pool is empty");
  return MOE_OK;
}

// One prefill layer on the intermediates `pb`: the two-buffer pipeline, or
// on-demand loading when the buffers do not fit.  No allocation.
static moe_status prefill_layer_run(moe_ctx* ctx, const PrefillBufs& pb, int32_t layer, const void* x,
                                    int32_t T, const int32_t* ids, const float* w, void* y, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  auto& pf = ctx->pf;
  pf.last = &pb;
  if (ctx->n_slots < pf.buffers * c.n_experts) return prefill_on_demand(ctx, pb, layer, x, T, ids, w, y, s);
  moe_status st = MOE_OK;
  const int b = prefill_buffer(ctx, layer);
  if (!pf.snap_valid) {
    // the residency table as this call finds it, for the hit-D2D slab copies
    MOE_HIP(ctx, hipMemcpyAsync(pf.snap, ctx->id2slot, 4 * (size_t)ctx->n_ids, hipMemcpyDeviceToHost, s));
    MOE_HIP(ctx, hipStreamSynchronize(s));
    pf.snap_valid = true;
  }
  MOE_HIP(ctx, hipEventRecord(pf.ev_start, s));
  if (pf.buf_layer[b] != layer && (st = prefill_issue(ctx, layer)) != MOE_OK) return st;
  // with two buffers, stream the next layer into the other one while this
  // one computes; with one, the next layer's copy waits for this compute
  if (pf.buffers == 2 && layer + 1 < c.n_layers && pf.buf_layer[1 - b] != layer + 1 &&
      (st = prefill_issue(ctx, layer + 1)) != MOE_OK)
    return st;
  MOE_HIP(ctx, hipStreamWaitEvent(s, pf.ev_copied[b], 0));
  // every prefill layer call takes one tick and stamps the buffer's experts
  // with it, also when the buffer already holds this layer (a repeated call):
  // the experts are used again, so their recency is refreshed
  MOE_HIP(ctx, launch_prefill_admit(ctx, layer, b, s));
  pf.admitted[b] = true;
  // the admission empties this layer's other slots: no longer copy sources
  for (int e = 0; e < c.n_experts; ++e) pf.snap[(size_t)layer * c.n_experts + e] = -1;
  MOE_HIP(ctx, launch_prefill_compute(ctx, pb, layer, x, T, ids, w, y, s));
  return MOE_OK;
}

extern "C" moe_status moe_prefill_layer(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                                        const int32_t* ids, const float* w, void* y,
                                        moe_stream stream) {
  CHECK_CTX(ctx);
  moe_status st = prefill_check(ctx, layer, x, T, ids, w, y, "moe_prefill_layer");
  if (st != MOE_OK) return st;
  if ((st = prefill_setup(ctx)) != MOE_OK) return st;
  return prefill_layer_run(ctx, ctx->pf.own, layer, x, T, ids, w, y, (hipStream_t)stream);
}

extern "C" moe_status moe_prefill_layer_noalloc(moe_ctx* ctx, int32_t layer, const void* x, int32_t T,
                                                const int32_t* ids, const float* w, void* y,
                                                moe_stream stream) {
  CHECK_CTX(ctx);
  moe_status st = prefill_check(ctx, layer, x, T, ids, w, y, "moe_prefill_layer_noalloc");
  if (st != MOE_OK) return st;
  const auto& sc = ctx->pf.scratch;
  const int64_t pairs = (int64_t)T * ctx->cfg.top_k;
  if (!sc.counts || pairs > sc.max_pairs)
    return fail(ctx, MOE_EINVAL,
                "moe_prefill_layer_noalloc: T*top_k = " + std::to_string(pairs) +
                    " routed pairs exceed the " + std::to_string(sc.max_pairs) +
                    " whose intermediates fit the library's fixed " +
                    std::to_string(kPrefillScratchBytes >> 20) + " MiB device scratch at this shape");
  return prefill_layer_run(ctx, sc, layer, x, T, ids, w, y, (hipStream_t)stream);
}
