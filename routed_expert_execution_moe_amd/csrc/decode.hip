// Decode data path: PCIe fill of admitted experts (with the hand-off of the
// CPU set to the host branch), dispatch of the expert FFN (ffn.h) and the
// fixed-order merge.
//
// Fill (snackonai, "The split policy itself", execution order: cache update,
// then the batched copy, then grouped evaluation): the host never learns
// which slots were chosen (the plan stays on the device), so the copy is a
// device-pull kernel reading the pinned, device-mapped host banks over PCIe.
// The expert FFN follows the fill on the same stream rather than running
// beside it for the experts already resident: with megabytes of host reads in
// flight, an HBM stream launched next to the pull ran 2-4x slower (and was
// sometimes dispatched late), which buys little and blurs the FFN's timing.
#include "internal.h"

namespace moert {

// ------------------------------------------------------------------ fill
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The hand-off of a call's CPU set to the host branch (snackonai, "The split
// policy itself": the CPU branch runs the misses left to it): the host block
// in pinned, device-mapped memory gets the routed ids, the slot map and the
// activations, then the header and, last, the doorbell (the call's sequence
// number, the device plan count).  One workgroup of the fill launch does it,
// only when the control kernel flagged host work.
struct Handoff {
  uint8_t* hblock;                 // device address of the host block; nullptr: no hand-off
  const int32_t* host_work;        // control kernel's flag
  const int32_t* ids;              // [T*k] routed ids
  const int32_t* slot_map;         // [T*k] slot or -1
  const moe_plan_counts* counts;
  const DevState* st;
  const uint8_t* x;                // [T][H] activations
  int64_t x_units;                 // 16-byte units of x
  size_t x_offset;                 // byte offset of the activations in the block
  int32_t Tk, T, layer;
};

__device__ void host_handoff(const Handoff& h) {
  if (*h.host_work == 0) return;  // uniform
  const int tid = threadIdx.x;
  HostBlockHeader* hb = (HostBlockHeader*)h.hblock;
  int32_t* hb_ids = (int32_t*)(h.hblock + sizeof(HostBlockHeader));
  int32_t* hb_map = hb_ids + h.Tk;
  for (int i = tid; i < h.Tk; i += blockDim.x) {
    hb_ids[i] = h.ids[i];
    hb_map[i] = h.slot_map[i];
  }
  const uint4* xs = (const uint4*)h.x;
  uint4* xd = (uint4*)(h.hblock + h.x_offset);
  for (int64_t i = tid; i < h.x_units; i += blockDim.x) xd[i] = xs[i];
  // every thread's block writes complete at system scope before the barrier,
  // then one thread writes the header and rings
  __threadfence_system();
  __syncthreads();
  if (tid == 0) {
    hb->c = *h.counts;
    hb->layer = h.layer;
    hb->T = h.T;
    const int64_t seq = h.st->plans;
    __threadfence_system();
    __hip_atomic_store(&hb->seq, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __threadfence_system();
  }
}

__global__ __launch_bounds__(256) void fill_kernel(const uint8_t* __restrict__ host_dev,
                                                   uint8_t* __restrict__ slots, size_t stride,
                                                   const moe_plan_counts* __restrict__ counts,
                                                   const int32_t* __restrict__ fill_u,
                                                   const int32_t* __restrict__ fill_slot, Handoff h) {
  // the last workgroup (when the launch carries a hand-off) serves the host
  // branch; the others pull the admitted experts
  const int nblk = (int)gridDim.x - (h.hblock ? 1 : 0);
  if ((int)blockIdx.x >= nblk) {
    host_handoff(h);
    return;
  }
  const int q = counts->q;
  if (q == 0) return;
  const size_t units = stride / 16;  // 16-byte units per expert
  const size_t total = (size_t)q * units;
  const size_t nthreads = (size_t)nblk * blockDim.x;
  // 16 loads of 16 bytes in flight per lane over 64 workgroups (4 MB in
  // flight): 54-55 GB/s from pinned host memory, a few % above wider grids
  constexpr int U = 16;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * nthreads < total; i += U * nthreads) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      size_t idx = i + j * nthreads;
      size_t f = idx / units, o = idx - f * units;
      const u32x4* src = (const u32x4*)(host_dev + (size_t)fill_u[f] * stride) + o;
      v[j] = __builtin_nontemporal_load(src);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      size_t idx = i + j * nthreads;
      size_t f = idx / units, o = idx - f * units;
      ((u32x4*)(slots + (size_t)fill_slot[f] * stride))[o] = v[j];
    }
  }
  for (; i < total; i += nthreads) {
    size_t f = i / units, o = i - f * units;
    ((u32x4*)(slots + (size_t)fill_slot[f] * stride))[o] =
        __builtin_nontemporal_load((const u32x4*)(host_dev + (size_t)fill_u[f] * stride) + o);
  }
}

constexpr int kFillBlocks = 64;

hipError_t launch_fill_lists(const uint8_t* host_dev, uint8_t* dst, size_t stride,
                             const moe_plan_counts* counts, const int32_t* fill_u,
                             const int32_t* fill_slot, hipStream_t s) {
  Handoff none{};
  hipLaunchKernelGGL(fill_kernel, dim3(kFillBlocks), dim3(256), 0, s, host_dev, dst, stride, counts,
                     fill_u, fill_slot, none);
  return hipGetLastError();
}

hipError_t launch_fill(moe_ctx* ctx, int layer, const int32_t* ids, int T, const void* x, hipStream_t s) {
  const PlanBufs& pb = ctx->plan;
  Handoff h;
  h.hblock = pb.hblock;
  h.host_work = pb.host_work;
  h.ids = ids;
  h.slot_map = pb.slot_map;
  h.counts = pb.counts;
  h.st = ctx->dstate;
  h.x = (const uint8_t*)x;
  h.x_units = (int64_t)T * ctx->cfg.hidden * pb.act_bytes / 16;
  h.x_offset = pb.x_offset;
  h.Tk = T * ctx->cfg.top_k;
  h.T = T;
  h.layer = layer;
  // no slots or CPU mode: q = 0, the fill workgroups exit at once
  hipLaunchKernelGGL(fill_kernel, dim3(kFillBlocks + 1), dim3(256), 0, s, ctx->host_pool_dev, ctx->pool.base,
                     ctx->stride, pb.counts, pb.fill_u, pb.fill_slot, h);
  return hipGetLastError();
}

// ------------------------------------------------------------------ expert FFN
hipError_t launch_ffn(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  if (ctx->n_slots == 0) return hipSuccess;
  switch (ctx->cfg.w_dtype) {
    case MOE_F32: return launch_ffn_f32(ctx, x, T, s);
    case MOE_BF16: return launch_ffn_bf16(ctx, x, T, s);
    default: return launch_ffn_mx(ctx, x, T, s);
  }
}

// ------------------------------------------------------------------ merge
// y[t] = sum over ascending j of w[t][j] * P[t][j], P from the GPU rows or the
// host rows by the sign of slot_map (snackonai, "What It Actually Does";
// satyajit, "Decode: the one equation").  fp32, one rounding to the output.
// A token with host pairs first waits for the host branch to publish this
// call's sequence number, the device plan count the control kernel left
// (bounded: after wait_ticks it flags an error).
template <int AT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ w,
                                                    const int32_t* __restrict__ slot_map,
                                                    const float* __restrict__ pg,
                                                    const float* pc, int k, int H,
                                                    void* __restrict__ y, HostSync* sync,
                                                    const DevState* st, uint64_t wait_ticks) {
  __shared__ int s_ok;
  const int t = blockIdx.y;
  bool host = false;
  for (int j = 0; j < k; ++j) host |= slot_map[t * k + j] < 0;
  if (host) {
    if (threadIdx.x == 0) {
      const uint64_t t0 = wall_clock64();
      const int64_t seq = st->plans;
      int ok = 1;
      while (__hip_atomic_load(&sync->done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < seq) {
        if (wall_clock64() - t0 > wait_ticks) {
          __hip_atomic_store(&sync->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      s_ok = ok;
    }
    __syncthreads();
  }
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  // eight pairs at a time: their partial values and weights are all
  // requested before the first product, so the loads' latencies overlap
  // (the rows were just written on other XCDs and come from HBM); the sum
  // still runs over ascending j
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float v[8], wv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p = t * k + j0 + q;
      v[q] = 0.f;
      wv[q] = 0.f;
      if (j0 + q < k) {
        wv[q] = w[p];
        // one load form for both sources (a system-scope load is what the
        // host rows need; the device rows, written by an earlier kernel on
        // this stream, read the same through it), so no load waits at a
        // branch join
        const float* src = (slot_map[p] >= 0 ? pg : pc) + (size_t)p * H + h;
        v[q] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (j0 + q < k) acc = fmaf(wv[q], v[q], acc);
  }
  if constexpr (AT == MOE_F32) {
    ((float*)y)[(size_t)t * H + h] = acc;
  } else {
    uint32_t u = __float_as_uint(acc);
    u += 0x7FFFu + ((u >> 16) & 1u);
    ((uint16_t*)y)[(size_t)t * H + h] = (uint16_t)(u >> 16);
  }
}

hipError_t launch_merge(moe_ctx* ctx, const float* w, int T, void* y, hipStream_t s) {
  const int H = ctx->cfg.hidden;
  dim3 grid((H + 255) / 256, T), block(256);
  if (ctx->cfg.act_dtype == MOE_F32)
    hipLaunchKernelGGL(merge_kernel<MOE_F32>, grid, block, 0, s, w, ctx->plan.slot_map, ctx->p_gpu,
                       ctx->p_cpu_dev, ctx->cfg.top_k, H, y, ctx->sync_dev, ctx->dstate, ctx->wait_ticks);
  else
    hipLaunchKernelGGL(merge_kernel<MOE_BF16>, grid, block, 0, s, w, ctx->plan.slot_map, ctx->p_gpu,
                       ctx->p_cpu_dev, ctx->cfg.top_k, H, y, ctx->sync_dev, ctx->dstate, ctx->wait_ticks);
  return hipGetLastError();
}

// Resize compaction: moves[2i] -> moves[2i+1], whole slots of `stride`
// bytes.  No move reads a slot another move writes (the survivors beyond the
// new budget go to free slots below it), so every move runs at once: kParts
// workgroups per move, each copying a contiguous part with four 16-byte
// loads in flight per lane.
constexpr int kMoveParts = 32;

__global__ __launch_bounds__(256) void slot_move_kernel(uint8_t* __restrict__ base, size_t stride,
                                                        const int32_t* __restrict__ moves) {
  const int mv = blockIdx.x / kMoveParts, part = blockIdx.x % kMoveParts;
  const u32x4* src = (const u32x4*)(base + (size_t)moves[2 * mv] * stride);
  u32x4* dst = (u32x4*)(base + (size_t)moves[2 * mv + 1] * stride);
  const size_t n16 = stride / 16, per = (n16 + kMoveParts - 1) / kMoveParts;
  const size_t b = (size_t)part * per, e = b + per < n16 ? b + per : n16;
  size_t i = b + threadIdx.x;
  for (; i + 3 * 256 < e; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    __builtin_nontemporal_store(v0, dst + i);
    __builtin_nontemporal_store(v1, dst + i + 256);
    __builtin_nontemporal_store(v2, dst + i + 512);
    __builtin_nontemporal_store(v3, dst + i + 768);
  }
  for (; i < e; i += 256) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_slot_moves(moe_ctx* ctx, const int32_t* moves, int n_moves, hipStream_t s) {
  if (n_moves <= 0) return hipSuccess;
  hipLaunchKernelGGL(slot_move_kernel, dim3((unsigned)n_moves * kMoveParts), dim3(256), 0, s,
                     ctx->pool.base, ctx->stride, moves);
  return hipGetLastError();
}

}  // namespace moert
