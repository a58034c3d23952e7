// Router top-k and residency-table reset.
//
// Routing: one 64-lane wave per token.  Lane l holds logits e = l, l+64, ...
// in registers; k rounds of a wave arg-max (larger logit first, lower expert
// index on equal logits, NaN ranked as -inf) pick the experts, and the
// softmax over the k selected logits gives the weights.  The pages leave the
// router design out of scope (snackonai, "The Promise"); a softmax router is
// the assumption.
#include "internal.h"

namespace moert {

constexpr int kRouteMaxPerLane = kMaxExperts / 64;  // 16

__device__ inline bool better(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[kRouteMaxPerLane];
  const int per = (E + 63) >> 6;
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    int e = lane + 64 * i;
    float x = -INFINITY;
    if (i < per && e < E) {
      x = row[e];
      if (x != x) x = -INFINITY;
    }
    v[i] = x;
  }
  uint32_t taken = 0;
  float sel0 = 0.f, wsum = 0.f;
  float my_val = 0.f;  // lane j keeps the j-th selected logit
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      int e = lane + 64 * i;
      if (i < per && e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oe = __shfl_xor(be, off);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_val = bv;
      my_id = be;
    }
    if (j == 0) sel0 = bv;
  }
  // softmax over the selected logits (lane j holds the j-th)
  float ex = 0.f;
  if (lane < k) ex = (sel0 == -INFINITY) ? 1.f : expf(my_val - sel0);
  wsum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = ex / wsum;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  dim3 block(256), grid((T + 3) / 4);
  hipLaunchKernelGGL(route_topk_kernel, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- table reset
__global__ void table_reset_kernel(int32_t* id2slot, int64_t n_ids, int32_t* slot2id,
                                   int64_t* slot_ts, int max_slots, DevState* st, int n_slots) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < n_ids; j += stride) id2slot[j] = -1;
  for (int64_t j = i; j < max_slots; j += stride) {
    slot2id[j] = -1;
    slot_ts[j] = -1;
  }
  if (i == 0) {
    st->tick = 0;
    st->plans = st->hits = st->fills = st->cpu = st->evictions = st->prefill_layers = 0;
    st->n_slots = n_slots;
    st->pad = 0;
  }
}

hipError_t launch_table_reset(moe_ctx* ctx, hipStream_t s) {
  hipLaunchKernelGGL(table_reset_kernel, dim3(256), dim3(256), 0, s, ctx->id2slot, ctx->n_ids,
                     ctx->slot2id, ctx->slot_ts, ctx->cfg.max_slots, ctx->dstate, ctx->n_slots);
  return hipGetLastError();
}

}  // namespace moert
