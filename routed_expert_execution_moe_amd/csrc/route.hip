// Router top-k and residency-table reset.
//
// Routing: one 64-lane wave per token.  Lane l holds logits e = l, l+64, ...
// in registers (all loads issued before any is used).  Each logit becomes a
// 64-bit key, its order-preserving unsigned image above the complement of
// its index, so one unsigned maximum ranks larger logits first and equal
// logits by lower index (NaN counts as -inf, -0 as +0).  k rounds of a wave
// maximum pick the experts (DPP within each row of 16 lanes, then the four
// row maxima read as scalars); the winner's key is then cleared.  The
// softmax over the k selected logits gives the weights.  The pages leave the
// router design out of scope (snackonai, "The Promise"); a softmax router is
// the assumption.
#include "internal.h"

namespace moert {

__device__ inline uint64_t route_key(float x, int e) {
  if (x != x) x = -INFINITY;
  if (x == 0.f) x = 0.f;  // -0 ranks with +0
  uint32_t b = __float_as_uint(x);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ inline float route_val(uint64_t key) {
  uint32_t b = (uint32_t)(key >> 32);
  b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;
  return __uint_as_float(b);
}

template <int CTRL>
__device__ inline uint64_t dpp_max(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// the key of lane l as a wave-uniform value
__device__ inline uint64_t lane_key(uint64_t k, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(v[i], e) : 0;  // 0 ranks below every logit
  }
  uint64_t my_key = 0;  // lane j keeps the j-th selected key
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) b = key[i] > b ? key[i] : b;
    b = dpp_max<0xB1>(b);   // quad_perm [1,0,3,2]
    b = dpp_max<0x4E>(b);   // quad_perm [2,3,0,1]
    b = dpp_max<0x141>(b);  // row_half_mirror
    b = dpp_max<0x140>(b);  // row_mirror
    // every lane now holds its row's maximum; the four rows' maxima are
    // read as scalars, so the wave maximum needs no trip through LDS
    const uint64_t r0 = lane_key(b, 0), r1 = lane_key(b, 16), r2 = lane_key(b, 32), r3 = lane_key(b, 48);
    const uint64_t m01 = r0 > r1 ? r0 : r1, m23 = r2 > r3 ? r2 : r3;
    b = m01 > m23 ? m01 : m23;
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = key[i] == b ? 0 : key[i];
    if (lane == j) my_key = b;
  }
  // softmax over the selected logits (lane j holds the j-th); lane 0 holds the max
  const float my_val = route_val(my_key);
  const float sel0 = __shfl(my_val, 0);
  float ex = 0.f;
  if (lane < k) ex = (sel0 == -INFINITY) ? 1.f : expf(my_val - sel0);
  float wsum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = (int32_t)~(uint32_t)my_key;
    w[(size_t)t * k + lane] = ex / wsum;
  }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  dim3 block(256), grid((T + 3) / 4);
  const int per = (E + 63) / 64;
  if (per <= 1) hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (per <= 2) hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (per <= 4) hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (per <= 8) hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
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
    st->h_epoch = -1;  // the first control call writes the intermediate's marks
  }
}

hipError_t launch_table_reset(moe_ctx* ctx, hipStream_t s) {
  hipLaunchKernelGGL(table_reset_kernel, dim3(256), dim3(256), 0, s, ctx->id2slot, ctx->n_ids,
                     ctx->slot2id, ctx->slot_ts, ctx->cfg.max_slots, ctx->dstate, ctx->n_slots);
  return hipGetLastError();
}

}  // namespace moert
