// Drives the host branch (cpu_branch.cpp: doorbell poller + worker pool) on
// the CPU alone, for a ThreadSanitizer build.  This program plays the part of
// the device (the fill launch's hand-off workgroup): it writes each call's host
// block (header, ids, slot map, activations) and rings the doorbell with a
// release store, then waits for the completion word with acquire loads, as the
// merge kernel does, and copies out the rows of the pairs assigned to the host.
// Meanwhile it polls host_branch_idle() as a resize would.
//
// usage: host_branch_check IN OUT
// IN  (little-endian): int32 L E k H I w_dtype act_dtype T n_calls threads,
//     int64 stride, the host pool (L*E*stride bytes), then per call: int32
//     layer, int32 ids[T*k], int32 slot_map[T*k], activations [T][H] (act dtype)
// OUT: per call float32 rows [T*k][H]; rows of pairs with slot_map >= 0 are 0
#include <immintrin.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../routed_expert_execution_moe_amd/csrc/internal.h"

using namespace moert;

static bool read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 2;
  int32_t h[10];
  int64_t stride = 0;
  if (!read_all(in, h, sizeof h) || !read_all(in, &stride, 8)) return 2;
  const int L = h[0], E = h[1], k = h[2], H = h[3], I = h[4], wdt = h[5], adt = h[6], T = h[7],
            n_calls = h[8], threads = h[9];
  const int Tk = T * k, ab = adt == MOE_F32 ? 4 : 2;
  std::vector<uint8_t> pool((size_t)L * E * stride);
  if (!read_all(in, pool.data(), pool.size())) return 2;

  moe_ctx* ctx = new moe_ctx();
  ctx->cfg.n_layers = L;
  ctx->cfg.n_experts = E;
  ctx->cfg.top_k = k;
  ctx->cfg.hidden = H;
  ctx->cfg.inter = I;
  ctx->cfg.w_dtype = wdt;
  ctx->cfg.act_dtype = adt;
  ctx->cfg.max_tokens = T;
  ctx->stride = (size_t)stride;
  ctx->host_pool = pool.data();
  ctx->cpu_threads = threads;
  // host block laid out as the device's hand-off writes it
  const size_t hbytes = sizeof(HostBlockHeader) + 2 * 4 * (size_t)Tk;
  const size_t x_off = (hbytes + 255) / 256 * 256;
  std::vector<uint8_t> block(x_off + (size_t)T * H * ab + 256, 0);
  ctx->hstage = block.data();
  ctx->xstage = block.data() + x_off;
  HostSync sync{};
  ctx->sync = &sync;
  std::vector<float> prow((size_t)Tk * H, 0.f);
  ctx->p_cpu = prow.data();
  ctx->cpu = cpu_pool_create(threads);
  if (!ctx->cpu || !host_branch_start(ctx)) return 3;

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 2;
  HostBlockHeader* hdr = (HostBlockHeader*)block.data();
  int32_t* ids = (int32_t*)(block.data() + sizeof(HostBlockHeader));
  int32_t* smap = ids + Tk;
  std::vector<float> rows((size_t)Tk * H);
  int64_t idle_polls = 0;
  for (int c = 0; c < n_calls; ++c) {
    int32_t layer = 0;
    if (!read_all(in, &layer, 4) || !read_all(in, ids, 4 * (size_t)Tk) ||
        !read_all(in, smap, 4 * (size_t)Tk) || !read_all(in, ctx->xstage, (size_t)T * H * ab))
      return 2;
    hdr->layer = layer;
    hdr->T = T;
    int n_cpu = 0;
    for (int p = 0; p < Tk; ++p) n_cpu += smap[p] < 0;
    hdr->c.n_cpu = n_cpu;
    const int64_t seq = c + 1;
    __atomic_store_n(&hdr->seq, seq, __ATOMIC_RELEASE);  // ring
    while (__atomic_load_n(&sync.done, __ATOMIC_ACQUIRE) < seq) {
      idle_polls += host_branch_idle(ctx) ? 1 : 0;
      _mm_pause();
    }
    for (int p = 0; p < Tk; ++p) {
      if (smap[p] < 0) memcpy(&rows[(size_t)p * H], &prow[(size_t)p * H], 4 * (size_t)H);
      else memset(&rows[(size_t)p * H], 0, 4 * (size_t)H);
    }
    if (fwrite(rows.data(), 4, rows.size(), out) != rows.size()) return 2;
  }
  if (!host_branch_idle(ctx)) return 4;  // every doorbell answered
  host_branch_stop(ctx);
  cpu_pool_destroy(ctx->cpu);
  ctx->cpu = nullptr;
  delete ctx;
  fclose(out);
  fclose(in);
  fprintf(stderr, "host branch: %d calls answered (%lld idle polls while waiting)\n", n_calls,
          (long long)idle_polls);
  return 0;
}
