// Host branch: the misses the plan assigned to the CPU run where their
// weights already live, on a persistent worker pool, reading the pinned host
// banks directly (snackonai, "The split policy itself": the cpu set executes
// in place; "Technical Moats": a persistent worker pool pinned to cores with
// SIMD and in-kernel dequantisation).
//
// Hand-off without host synchronisation: when a call has host work the control
// kernel writes the plan, ids, slot map and activations into pinned,
// device-mapped memory and then rings a doorbell (a sequence number).  A
// persistent poller thread of the context sees it, runs the host experts with
// its worker pool, writes fp32 rows P_cpu[t*k + j][H] for every pair whose
// slot map is -1 into pinned, device-mapped memory, and publishes the
// sequence number as done.  The merge kernel of that call waits for it (only
// for tokens with host pairs), with a time limit.  The poller never calls HIP.
#include <immintrin.h>
#include <pthread.h>
#include <sched.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>
#include <cstdio>
#include <cstdlib>

#include "internal.h"

namespace moert {

// ------------------------------------------------------------------ pool
struct CpuPool {
  int n = 1;  // workers including the calling thread
  std::vector<std::thread> th;
  std::mutex mu;
  std::condition_variable cv;
  uint64_t gen = 0;                 // guarded by mu
  std::atomic<uint64_t> gen_fast{0};
  std::atomic<int> pending{0};
  bool stop = false;
  std::function<void(int, int)> fn;  // (worker, n)

  void worker(int i) {
    uint64_t seen = 0;
    for (;;) {
      // brief spin for low wake latency, then block
      uint64_t g = gen_fast.load(std::memory_order_acquire);
      for (int spin = 0; g == seen && spin < 20000; ++spin) {
        _mm_pause();
        g = gen_fast.load(std::memory_order_acquire);
      }
      if (g == seen) {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return gen != seen || stop; });
        if (stop) return;
        g = gen;
      }
      seen = g;
      fn(i, n);
      pending.fetch_sub(1, std::memory_order_acq_rel);
    }
  }

  void run(std::function<void(int, int)> f) {
    if (n == 1) {
      f(0, 1);
      return;
    }
    fn = std::move(f);
    pending.store(n - 1, std::memory_order_release);
    {
      std::lock_guard<std::mutex> lk(mu);
      ++gen;
      gen_fast.store(gen, std::memory_order_release);
    }
    cv.notify_all();
    fn(0, n);
    while (pending.load(std::memory_order_acquire) > 0) _mm_pause();
  }
};

CpuPool* cpu_pool_create(int threads) {
  CpuPool* p = new (std::nothrow) CpuPool();
  if (!p) return nullptr;
  p->n = std::max(1, threads);
  cpu_set_t cs;
  std::vector<int> cores;
  if (sched_getaffinity(0, sizeof cs, &cs) == 0)
    for (int c = 0; c < CPU_SETSIZE; ++c)
      if (CPU_ISSET(c, &cs)) cores.push_back(c);
  // Workers 1..n-1 are pinned to the highest cores, one each, when there are
  // enough; the callback thread (worker 0), the caller's issue thread and the
  // HIP runtime threads keep the low cores.
  const bool pin = (int)cores.size() >= p->n + 2;
  for (int i = 1; i < p->n; ++i) {
    p->th.emplace_back([p, i] { p->worker(i); });
    if (pin) {
      cpu_set_t one;
      CPU_ZERO(&one);
      CPU_SET(cores[cores.size() - i], &one);
      pthread_setaffinity_np(p->th.back().native_handle(), sizeof one, &one);
    }
  }
  return p;
}

void cpu_pool_destroy(CpuPool* p) {
  if (!p) return;
  {
    std::lock_guard<std::mutex> lk(p->mu);
    p->stop = true;
  }
  p->cv.notify_all();
  for (auto& t : p->th) t.join();
  delete p;
}

// ------------------------------------------------------------------ dot kernels
static inline float hsum(__m256 v) {
  __m128 a = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  a = _mm_add_ps(a, _mm_movehl_ps(a, a));
  a = _mm_add_ss(a, _mm_shuffle_ps(a, a, 1));
  return _mm_cvtss_f32(a);
}

// dot(row[0..K), x_t[0..K)) for nt vectors at once; K % 16 == 0
static void dot_bf16(const uint16_t* row, const float* const* x, int nt, int K, float* out) {
  for (int t0 = 0; t0 < nt; t0 += 4) {
    const int m = std::min(4, nt - t0);
    __m256 acc[4][2];
    for (int t = 0; t < 4; ++t) acc[t][0] = acc[t][1] = _mm256_setzero_ps();
    for (int c = 0; c < K; c += 16) {
      __m256i w = _mm256_loadu_si256((const __m256i*)(row + c));
      __m256 lo = _mm256_castsi256_ps(
          _mm256_slli_epi32(_mm256_cvtepu16_epi32(_mm256_castsi256_si128(w)), 16));
      __m256 hi = _mm256_castsi256_ps(
          _mm256_slli_epi32(_mm256_cvtepu16_epi32(_mm256_extracti128_si256(w, 1)), 16));
      for (int t = 0; t < m; ++t) {
        acc[t][0] = _mm256_fmadd_ps(lo, _mm256_loadu_ps(x[t0 + t] + c), acc[t][0]);
        acc[t][1] = _mm256_fmadd_ps(hi, _mm256_loadu_ps(x[t0 + t] + c + 8), acc[t][1]);
      }
    }
    for (int t = 0; t < m; ++t) out[t0 + t] = hsum(_mm256_add_ps(acc[t][0], acc[t][1]));
  }
}

static void dot_f32(const float* row, const float* const* x, int nt, int K, float* out) {
  for (int t = 0; t < nt; ++t) {
    __m256 a0 = _mm256_setzero_ps(), a1 = _mm256_setzero_ps();
    for (int c = 0; c < K; c += 16) {
      a0 = _mm256_fmadd_ps(_mm256_loadu_ps(row + c), _mm256_loadu_ps(x[t] + c), a0);
      a1 = _mm256_fmadd_ps(_mm256_loadu_ps(row + c + 8), _mm256_loadu_ps(x[t] + c + 8), a1);
    }
    out[t] = hsum(_mm256_add_ps(a0, a1));
  }
}

// MXFP4 row: codes[K/2], scales[K/32]; x is in "nibble order" per 32-block:
// the 16 even elements, then the 16 odd elements.
static void dot_mx(const uint8_t* codes, const uint8_t* scales, const float* const* x, int nt, int K,
                   float* out) {
  const __m256 lut = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const __m256i seven = _mm256_set1_epi32(7), eight = _mm256_set1_epi32(8);
  for (int t0 = 0; t0 < nt; t0 += 4) {
    const int m = std::min(4, nt - t0);
    __m256 acc[4];
    for (int t = 0; t < 4; ++t) acc[t] = _mm256_setzero_ps();
    for (int b = 0; b < K / 32; ++b) {
      __m128i by = _mm_loadu_si128((const __m128i*)(codes + 16 * b));
      __m128i lo = _mm_and_si128(by, _mm_set1_epi8(0x0F));
      __m128i hi = _mm_and_si128(_mm_srli_epi16(by, 4), _mm_set1_epi8(0x0F));
      __m256 v[4];
      __m128i parts[4] = {lo, _mm_srli_si128(lo, 8), hi, _mm_srli_si128(hi, 8)};
      for (int q = 0; q < 4; ++q) {
        __m256i idx = _mm256_cvtepu8_epi32(parts[q]);
        __m256 mag = _mm256_permutevar8x32_ps(lut, _mm256_and_si256(idx, seven));
        __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(idx, eight), 28);
        v[q] = _mm256_xor_ps(mag, _mm256_castsi256_ps(sgn));
      }
      const uint32_t s = scales[b];
      uint32_t sb = s ? (s << 23) : 0x00400000u;
      float sc;
      memcpy(&sc, &sb, 4);
      const __m256 scv = _mm256_set1_ps(sc);
      for (int t = 0; t < m; ++t) {
        const float* xp = x[t0 + t] + 32 * b;
        __m256 blk = _mm256_mul_ps(v[0], _mm256_loadu_ps(xp));
        blk = _mm256_fmadd_ps(v[1], _mm256_loadu_ps(xp + 8), blk);
        blk = _mm256_fmadd_ps(v[2], _mm256_loadu_ps(xp + 16), blk);
        blk = _mm256_fmadd_ps(v[3], _mm256_loadu_ps(xp + 24), blk);
        acc[t] = _mm256_fmadd_ps(blk, scv, acc[t]);
      }
    }
    for (int t = 0; t < m; ++t) out[t0 + t] = hsum(acc[t]);
  }
}

static inline float silu(float g) { return g / (1.f + std::exp(-g)); }

// ------------------------------------------------------------------ branch
struct Expert {
  int u;
  std::vector<int> pairs;  // t*k + j
};

static void cpu_branch_body(moe_ctx* ctx);

// Opt-in phase trace of the host branch (MOERT_HOST_TRACE=1): averages of the
// gate/up and down phases over calls with host work, on stderr.
struct HostTrace {
  bool on = false;
  int64_t calls = 0, experts = 0;
  double p1 = 0, p2 = 0;
};
static HostTrace g_trace = [] {
  HostTrace t;
  const char* v = getenv("MOERT_HOST_TRACE");
  t.on = v && v[0] == '1';
  return t;
}();

static inline double now_us() {
  return std::chrono::duration<double, std::micro>(
             std::chrono::steady_clock::now().time_since_epoch()).count();
}

struct HostBranch {
  std::thread th;
  std::atomic<bool> stop{false};
  std::atomic<int64_t> last{0};  // last doorbell value answered
};

static void poller(moe_ctx* ctx) {
  HostBranch* hb = ctx->hb;
  // HostBlockHeader::seq, written last by the fill launch's hand-off
  // workgroup after a system-scope release; an acquire load here orders the
  // block's reads
  const int64_t* bell = (const int64_t*)ctx->hstage;
  int64_t last = 0;
  int idle = 0;
  while (!hb->stop.load(std::memory_order_relaxed)) {
    const int64_t s = __atomic_load_n(bell, __ATOMIC_ACQUIRE);
    if (s == last) {
      // spin while calls are arriving; back off to short sleeps when idle
      if (++idle < (1 << 16)) {
        _mm_pause();
      } else {
        std::this_thread::sleep_for(std::chrono::microseconds(20));
      }
      continue;
    }
    idle = 0;
    if (ctx->timing) {
      auto t0 = std::chrono::steady_clock::now();
      cpu_branch_body(ctx);
      auto ns = std::chrono::duration_cast<std::chrono::nanoseconds>(
          std::chrono::steady_clock::now() - t0);
      ctx->timing->host_ns += ns.count();
      ctx->timing->host_calls += 1;
    } else {
      cpu_branch_body(ctx);
    }
    last = s;
    // rows first, then the completion word the merge kernel waits for
    __atomic_store_n(&ctx->sync->done, s, __ATOMIC_RELEASE);
    hb->last.store(s, std::memory_order_release);
  }
}

bool host_branch_start(moe_ctx* ctx) {
  ctx->hb = new (std::nothrow) HostBranch();
  if (!ctx->hb) return false;
  ctx->hb->th = std::thread(poller, ctx);
  // the poller is worker 0: keep it off the workers' cores
  cpu_set_t cs;
  std::vector<int> cores;
  if (sched_getaffinity(0, sizeof cs, &cs) == 0)
    for (int c = 0; c < CPU_SETSIZE; ++c)
      if (CPU_ISSET(c, &cs)) cores.push_back(c);
  if ((int)cores.size() >= ctx->cpu_threads + 2) {
    cpu_set_t one;
    CPU_ZERO(&one);
    CPU_SET(cores[cores.size() - ctx->cpu_threads], &one);
    pthread_setaffinity_np(ctx->hb->th.native_handle(), sizeof one, &one);
  }
  return true;
}

void host_branch_stop(moe_ctx* ctx) {
  if (!ctx->hb) return;
  ctx->hb->stop = true;
  if (ctx->hb->th.joinable()) ctx->hb->th.join();
  delete ctx->hb;
  ctx->hb = nullptr;
}

bool host_branch_idle(moe_ctx* ctx) {
  if (!ctx->hb) return true;
  return ctx->hb->last.load(std::memory_order_acquire) ==
         __atomic_load_n((const int64_t*)ctx->hstage, __ATOMIC_ACQUIRE);
}

// The host branch's arithmetic: SwiGLU of the experts `ex` read in place from
// the pinned host banks, on the worker pool.  Pair p takes its input from row
// p / k of xf (fp32, MXFP4 nibble order) and writes its fp32 row to out + p*H.
// Gate/up rows, then down rows, split evenly over the workers.
static void host_eval(moe_ctx* ctx, const std::vector<Expert>& ex, const float* xf, int k, float* out,
                      double* t_mid) {
  const moe_config& c = ctx->cfg;
  const int H = c.hidden, I = c.inter;
  const int nex = (int)ex.size();
  int max_pair = 0;
  for (const Expert& X : ex)
    for (int p : X.pairs) max_pair = std::max(max_pair, p + 1);
  // intermediate h per pair, fp32 (MXFP4: nibble order per 32-block of I)
  std::vector<float> hmid((size_t)max_pair * I);
  const size_t stride = ctx->stride;
  const uint8_t* pool = ctx->host_pool;
  const size_t eb = c.w_dtype == MOE_F32 ? 4 : 2;

  // phase 1: gate/up rows, split evenly over the workers
  ctx->cpu->run([&](int wi, int nw) {
    const int64_t R = (int64_t)nex * I;
    const int64_t r0 = R * wi / nw, r1 = R * (wi + 1) / nw;
    std::vector<const float*> xs;
    std::vector<float> g, uu;
    for (int64_t r = r0; r < r1; ++r) {
      const Expert& X = ex[r / I];
      const int row = (int)(r % I);
      const int nt = (int)X.pairs.size();
      xs.resize(nt);
      g.resize(nt);
      uu.resize(nt);
      for (int t = 0; t < nt; ++t) xs[t] = xf + (size_t)(X.pairs[t] / k) * H;
      const uint8_t* bank = pool + (size_t)X.u * stride;
      if (c.w_dtype == MOE_MXFP4) {
        const uint8_t* cg = bank + (size_t)row * (H / 2);
        const uint8_t* cu = bank + (size_t)I * H / 2 + (size_t)row * (H / 2);
        const uint8_t* sbase = bank + 3 * (size_t)H * I / 2;
        dot_mx(cg, sbase + (size_t)row * (H / 32), xs.data(), nt, H, g.data());
        dot_mx(cu, sbase + (size_t)I * H / 32 + (size_t)row * (H / 32), xs.data(), nt, H, uu.data());
      } else if (c.w_dtype == MOE_BF16) {
        const uint16_t* wg = (const uint16_t*)bank + (size_t)row * H;
        const uint16_t* wu = (const uint16_t*)bank + (size_t)I * H + (size_t)row * H;
        dot_bf16(wg, xs.data(), nt, H, g.data());
        dot_bf16(wu, xs.data(), nt, H, uu.data());
      } else {
        const float* wg = (const float*)bank + (size_t)row * H;
        const float* wu = (const float*)bank + (size_t)I * H + (size_t)row * H;
        dot_f32(wg, xs.data(), nt, H, g.data());
        dot_f32(wu, xs.data(), nt, H, uu.data());
      }
      for (int t = 0; t < nt; ++t) {
        int col = row;
        if (c.w_dtype == MOE_MXFP4) {  // store in nibble order for the down pass
          const int b = row / 32, i = row % 32;
          col = 32 * b + ((i & 1) ? 16 + i / 2 : i / 2);
        }
        hmid[(size_t)X.pairs[t] * I + col] = silu(g[t]) * uu[t];
      }
    }
  });
  (void)eb;
  if (t_mid) *t_mid = now_us();
  // phase 2: down rows
  ctx->cpu->run([&](int wi, int nw) {
    const int64_t R = (int64_t)nex * H;
    const int64_t r0 = R * wi / nw, r1 = R * (wi + 1) / nw;
    std::vector<const float*> hs;
    std::vector<float> o;
    for (int64_t r = r0; r < r1; ++r) {
      const Expert& X = ex[r / H];
      const int row = (int)(r % H);
      const int nt = (int)X.pairs.size();
      hs.resize(nt);
      o.resize(nt);
      for (int t = 0; t < nt; ++t) hs[t] = hmid.data() + (size_t)X.pairs[t] * I;
      const uint8_t* bank = pool + (size_t)X.u * stride;
      if (c.w_dtype == MOE_MXFP4) {
        const uint8_t* cd = bank + (size_t)I * H + (size_t)row * (I / 2);
        const uint8_t* sd = bank + 3 * (size_t)H * I / 2 + 2 * (size_t)I * H / 32 + (size_t)row * (I / 32);
        dot_mx(cd, sd, hs.data(), nt, I, o.data());
      } else if (c.w_dtype == MOE_BF16) {
        const uint16_t* wd = (const uint16_t*)bank + 2 * (size_t)I * H + (size_t)row * I;
        dot_bf16(wd, hs.data(), nt, I, o.data());
      } else {
        const float* wd = (const float*)bank + 2 * (size_t)I * H + (size_t)row * I;
        dot_f32(wd, hs.data(), nt, I, o.data());
      }
      for (int t = 0; t < nt; ++t) out[(size_t)X.pairs[t] * H + row] = o[t];
    }
  });
}

static void cpu_branch_body(moe_ctx* ctx) {
  const moe_config& c = ctx->cfg;
  const HostBlockHeader* hb = (const HostBlockHeader*)ctx->hstage;
  const int n_cpu = hb->c.n_cpu;
  const int T = hb->T, k = c.top_k, layer = hb->layer, E = c.n_experts;
  const int H = c.hidden;
  const int Tk = T * k;
  const int32_t* ids = (const int32_t*)(ctx->hstage + sizeof(HostBlockHeader));
  const int32_t* smap = ids + Tk;
  // pairs the host must produce; invalid ids get zero rows
  std::vector<Expert> ex;
  bool any = false;
  for (int p = 0; p < Tk; ++p) {
    if (smap[p] >= 0) continue;
    any = true;
    const int e = ids[p];
    if (e < 0 || e >= E) {
      memset(ctx->p_cpu + (size_t)p * H, 0, sizeof(float) * H);
      continue;
    }
    const int u = layer * E + e;
    auto it = std::find_if(ex.begin(), ex.end(), [&](const Expert& x) { return x.u == u; });
    if (it == ex.end()) ex.push_back({u, {p}});
    else it->pairs.push_back(p);
  }
  if (!any || ex.empty()) return;
  (void)n_cpu;
  const int nex = (int)ex.size();
  const double t_start = g_trace.on ? now_us() : 0.0;
  double t_p1 = 0.0, t_p2 = 0.0;

  // activations in fp32 (MXFP4: nibble order per 32-block)
  std::vector<float> xf((size_t)T * H);
  for (int t = 0; t < T; ++t) {
    float* dst = xf.data() + (size_t)t * H;
    if (c.act_dtype == MOE_F32) {
      memcpy(dst, ctx->xstage + (size_t)t * H * 4, sizeof(float) * H);
    } else {
      const uint16_t* src = (const uint16_t*)ctx->xstage + (size_t)t * H;
      for (int h = 0; h < H; ++h) {
        uint32_t b = (uint32_t)src[h] << 16;
        memcpy(dst + h, &b, 4);
      }
    }
  }
  if (c.w_dtype == MOE_MXFP4) {
    std::vector<float> tmp(32);
    for (int t = 0; t < T; ++t) {
      float* v = xf.data() + (size_t)t * H;
      for (int b = 0; b < H / 32; ++b) {
        for (int i = 0; i < 16; ++i) {
          tmp[i] = v[32 * b + 2 * i];
          tmp[16 + i] = v[32 * b + 2 * i + 1];
        }
        memcpy(v + 32 * b, tmp.data(), sizeof(float) * 32);
      }
    }
  }
  host_eval(ctx, ex, xf.data(), k, ctx->p_cpu, g_trace.on ? &t_p1 : nullptr);
  if (g_trace.on) {
    t_p2 = now_us();
    HostTrace& tr = g_trace;
    tr.calls += 1;
    tr.experts += nex;
    tr.p2 += t_p2 - t_p1;
    tr.p1 += t_p1 - t_start;
    (void)tr;
    if (tr.calls % 2000 == 0)
      fprintf(stderr, "[moert host] %lld calls with host work, %.2f experts/call, gate+up %.1f us, "
              "down %.1f us per call (%d threads)\n", (long long)tr.calls,
              (double)tr.experts / tr.calls, tr.p1 / tr.calls, tr.p2 / tr.calls, ctx->cpu_threads);
  }
}

// Seconds per evaluation of n experts (one token each, all reading the same
// input row) by the host branch's arithmetic: set r is us[r*n .. r*n+n), set 0
// untimed, sets 1..reps timed and averaged (distinct sets, so the host caches
// do not serve repeated bytes).  The caller guarantees the host branch is idle.
double host_expert_seconds(moe_ctx* ctx, const int32_t* us, int n, int reps) {
  const int H = ctx->cfg.hidden;
  std::vector<float> xf((size_t)H), out((size_t)n * H);
  for (int h = 0; h < H; ++h) xf[h] = 0.01f * (float)((h * 37) % 101 - 50);
  auto set = [&](int r) {
    std::vector<Expert> ex;
    for (int i = 0; i < n; ++i) ex.push_back({us[r * n + i], {i}});
    return ex;
  };
  host_eval(ctx, set(0), xf.data(), n, out.data(), nullptr);
  double total = 0.0;
  for (int r = 1; r <= reps; ++r) {
    const std::vector<Expert> ex = set(r);
    const auto t0 = std::chrono::steady_clock::now();
    host_eval(ctx, ex, xf.data(), n, out.data(), nullptr);
    total += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  }
  return total / reps;
}

}  // namespace moert
