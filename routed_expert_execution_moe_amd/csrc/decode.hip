// Decode data path: PCIe fill of admitted experts, the grouped SwiGLU expert
// GEMV over the slot pool, and the fixed-order merge.
//
// Fill (snackonai, "The split policy itself", execution order: cache update,
// then the batched copy, then grouped evaluation): the host never learns
// which slots were chosen (the plan stays on the device), so the copy is a
// device-pull kernel reading the pinned, device-mapped host banks over PCIe.
//
// Expert GEMV: decode touches each routed expert's complete weights once per
// call, so the kernel is an HBM stream.  A workgroup owns RB row groups of one
// expert; its KS waves split the contraction axis, every lane loads one
// 16-byte chunk per row (coalesced), keeps the input vector chunk of every
// routed token in registers, reduces within its lane group with xor
// shuffles, and the waves combine partials through LDS in a fixed order (no
// atomics, bit-reproducible).  Gate and up rows are read together so the
// SiLU(g) * u epilogue needs no second pass; the down projection reads the
// fp32 intermediate.
#include "internal.h"

namespace moert {

// ------------------------------------------------------------------ fill
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void fill_kernel(const uint8_t* __restrict__ host_dev,
                                                   uint8_t* __restrict__ slots, size_t stride,
                                                   const moe_plan_counts* __restrict__ counts,
                                                   const int32_t* __restrict__ fill_u,
                                                   const int32_t* __restrict__ fill_slot) {
  const int q = counts->q;
  if (q == 0) return;
  const size_t units = stride / 16;  // 16-byte units per expert
  const size_t total = (size_t)q * units;
  const size_t nthreads = (size_t)gridDim.x * blockDim.x;
  constexpr int U = 4;
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

hipError_t launch_fill(moe_ctx* ctx, hipStream_t s) {
  if (ctx->n_slots == 0 || ctx->cfg.mode == MOE_CPU) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(512), dim3(256), 0, s, ctx->host_pool_dev, ctx->pool.base,
                     ctx->stride, ctx->plan.counts, ctx->plan.fill_u, ctx->plan.fill_slot);
  return hipGetLastError();
}

// ------------------------------------------------------------------ weight chunks
// Elements per 16-byte weight chunk.
template <int WT> struct WChunk;
template <> struct WChunk<MOE_F32> { static constexpr int CH = 4; };
template <> struct WChunk<MOE_BF16> { static constexpr int CH = 8; };
template <> struct WChunk<MOE_MXFP4> { static constexpr int CH = 32; };

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// OCP MX E2M1 code (4 bits) to float: sign bit 3, exponent bits 2..1 (bias 1),
// mantissa bit 0; exponent 0 is the subnormal 0 / 0.5.
__device__ inline float e2m1_to_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  uint32_t bits = m >= 2u ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22)) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// OCP MX E8M0 scale 2^(s-127).
__device__ inline float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// Raw chunk as loaded from the slot.
template <int WT> struct Raw { uint4 v; uint32_t scale; };

template <int WT>
__device__ inline Raw<WT> load_chunk(const uint8_t* __restrict__ mat, const uint8_t* __restrict__ sc,
                                     int row, int K, int c) {
  Raw<WT> r;
  if constexpr (WT == MOE_F32) {
    r.v = *(const uint4*)(mat + ((size_t)row * K + (size_t)c * 4) * 4);
    r.scale = 0;
  } else if constexpr (WT == MOE_BF16) {
    r.v = *(const uint4*)(mat + ((size_t)row * K + (size_t)c * 8) * 2);
    r.scale = 0;
  } else {
    r.v = *(const uint4*)(mat + (size_t)row * (K / 2) + (size_t)c * 16);
    r.scale = sc[(size_t)row * (K / 32) + c];
  }
  return r;
}

// dot of a raw chunk with CH input values
template <int WT>
__device__ inline float chunk_dot(const Raw<WT>& r, const float* x) {
  if constexpr (WT == MOE_F32) {
    float a = __uint_as_float(r.v.x) * x[0];
    a = fmaf(__uint_as_float(r.v.y), x[1], a);
    a = fmaf(__uint_as_float(r.v.z), x[2], a);
    a = fmaf(__uint_as_float(r.v.w), x[3], a);
    return a;
  } else if constexpr (WT == MOE_BF16) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a = fmaf(bf16_lo(w[i]), x[2 * i], a);
      a = fmaf(bf16_hi(w[i]), x[2 * i + 1], a);
    }
    return a;
  } else {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (w[i] >> (8 * b)) & 0xFFu;
        a = fmaf(e2m1_to_f32(byte & 15u), x[8 * i + 2 * b], a);
        a = fmaf(e2m1_to_f32(byte >> 4), x[8 * i + 2 * b + 1], a);
      }
    }
    return a * e8m0_to_f32(r.scale);
  }
}

// input chunk: CH values of vector `idx` (token or pair) at chunk c
template <int XT, int CH>
__device__ inline void load_x(const void* __restrict__ x, int idx, int K, int c, float* out) {
  if constexpr (XT == MOE_F32) {
    const float4* p = (const float4*)((const float*)x + (size_t)idx * K + (size_t)c * CH);
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
      float4 v = p[i];
      out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (CH == 4) {
    const uint2 v = *(const uint2*)((const uint16_t*)x + (size_t)idx * K + (size_t)c * CH);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x); out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
  } else {
    const uint4* p = (const uint4*)((const uint16_t*)x + (size_t)idx * K + (size_t)c * CH);
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      uint4 v = p[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[8 * i + 2 * j] = bf16_lo(w[j]);
        out[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      }
    }
  }
}

struct GemvArgs {
  const uint8_t* slot_base;
  size_t stride;
  const moe_plan_counts* counts;
  const int32_t* gpu_slot;
  const int32_t* slot_map;
  int Tk, k;
  int K, rows;          // contraction length, output rows per matrix
  int items;            // row blocks of RW rows per expert
  size_t off0, off1;    // matrix byte offsets inside a slot
  size_t soff0, soff1;  // MX scale offsets
  const void* x;        // input vectors
  int x_by_token;       // 1: index = pair / k (activations), 0: index = pair (intermediate)
  float* out;           // [Tk][rows]
};

__device__ inline float silu(float g) { return g / (1.f + expf(-g)); }

// One item per wave: RW consecutive rows of one GPU expert (of both the gate
// and the up matrix when GLU).  Lane l owns chunks l, l+64, ... (CPL of them)
// of every row; the weights are loaded first and stay in registers while the
// wave loops over the expert's routed tokens, so they are read once however
// many tokens share the expert.  Rows are reduced across the wave with xor
// shuffles; no LDS, no barriers.
template <int WT, int XT, int NT, int RW, int CPL, bool GLU>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr int CH = WChunk<WT>::CH;
  constexpr int NM = GLU ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int g = item / a.items;
  const int n_gpu = a.counts->n_gpu;
  if (g >= n_gpu) return;  // wave-uniform
  const int rb = item - g * a.items;
  const int slot = a.gpu_slot[g];
  const uint8_t* sp = a.slot_base + (size_t)slot * a.stride;
  const int row0 = rb * RW;
  const int nch = a.K / CH;

  Raw<WT> wr[NM][RW][CPL];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int row = min(row0 + i, a.rows - 1);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        wr[0][i][c] = load_chunk<WT>(sp + a.off0, sp + a.soff0, row, a.K, ch);
        if constexpr (GLU) wr[1][i][c] = load_chunk<WT>(sp + a.off1, sp + a.soff1, row, a.K, ch);
      } else {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          wr[m][i][c].v = make_uint4(0, 0, 0, 0);
          wr[m][i][c].scale = 127;
        }
      }
    }
  }

  // the expert's routed pairs, NT at a time (ballots are wave-uniform)
  int base = 0;
  uint64_t bm = __ballot(lane < a.Tk && a.slot_map[lane] == slot);
  for (;;) {
    int pr[NT];
    int nt = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      while (bm == 0 && base + 64 < a.Tk) {
        base += 64;
        bm = __ballot(base + lane < a.Tk && a.slot_map[base + lane] == slot);
      }
      pr[t] = -1;
      if (bm) {
        pr[t] = base + __builtin_ctzll(bm);
        bm &= bm - 1;
        ++nt;
      }
    }
    if (nt == 0) break;
    float acc[NM][RW][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < RW; ++i) acc[m][i][t] = 0.f;
      if (pr[t] < 0) continue;
      const int idx = a.x_by_token ? pr[t] / a.k : pr[t];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        if (ch >= nch) continue;
        float xv[CH];
        load_x<XT, CH>(a.x, idx, a.K, ch, xv);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int i = 0; i < RW; ++i) acc[m][i][t] += chunk_dot<WT>(wr[m][i][c], xv);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < RW; ++i)
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[m][i][t] += __shfl_xor(acc[m][i][t], off);
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (lane == (i * NT + t) % 64 && pr[t] >= 0 && row0 + i < a.rows) {
          const float o = GLU ? silu(acc[0][i][t]) * acc[GLU ? 1 : 0][i][t] : acc[0][i][t];
          a.out[(size_t)pr[t] * a.rows + row0 + i] = o;
        }
  }
}

// chunks per lane for a contraction of K
static int cpl_of(int K, int CH) {
  int nch = K / CH;
  return nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 256 ? 4 : 8;
}

template <int WT, int XT, int NT, bool GLU>
static hipError_t launch_gemv_nt(GemvArgs a, int umax, hipStream_t s) {
  constexpr int CH = WChunk<WT>::CH;
  const int cpl = cpl_of(a.K, CH);
  // about 16 sixteen-byte weight loads in flight per lane
  auto go = [&](auto CPLc, auto RWc) -> hipError_t {
    constexpr int C = decltype(CPLc)::value, R = decltype(RWc)::value;
    a.items = (a.rows + R - 1) / R;
    const int waves = umax * a.items;
    hipLaunchKernelGGL((gemv_kernel<WT, XT, NT, R, C, GLU>), dim3((waves + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  if constexpr (GLU) {
    if (cpl == 1) return go(I1{}, I8{});
    if (cpl == 2) return go(I2{}, I4{});
    if (cpl == 4) return go(I4{}, I2{});
    return go(I8{}, I1{});
  } else {
    if (cpl == 1) return go(I1{}, I16{});
    if (cpl == 2) return go(I2{}, I8{});
    if (cpl == 4) return go(I4{}, I4{});
    return go(I8{}, I2{});
  }
}

template <int WT, int XT, bool GLU>
static hipError_t launch_gemv_t(GemvArgs a, int umax, int T, hipStream_t s) {
  if (T <= 1) return launch_gemv_nt<WT, XT, 1, GLU>(a, umax, s);
  if (T <= 2) return launch_gemv_nt<WT, XT, 2, GLU>(a, umax, s);
  if (T <= 4) return launch_gemv_nt<WT, XT, 4, GLU>(a, umax, s);
  return launch_gemv_nt<WT, XT, 8, GLU>(a, umax, s);
}

template <int WT>
static hipError_t launch_ffn_w(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  const int H = c.hidden, I = c.inter;
  GemvArgs a{};
  a.slot_base = ctx->pool.base;
  a.stride = ctx->stride;
  a.counts = ctx->plan.counts;
  a.gpu_slot = ctx->plan.gpu_slot;
  a.slot_map = ctx->plan.slot_map;
  a.Tk = T * c.top_k;
  a.k = c.top_k;
  // gate / up: rows I, contraction H
  const size_t eb = WT == MOE_F32 ? 4 : 2;
  if constexpr (WT == MOE_MXFP4) {
    a.off0 = 0;
    a.off1 = (size_t)I * H / 2;
    a.soff0 = 3 * (size_t)H * I / 2;
    a.soff1 = a.soff0 + (size_t)I * H / 32;
  } else {
    a.off0 = 0;
    a.off1 = (size_t)I * H * eb;
  }
  a.K = H;
  a.rows = I;
  a.x = x;
  a.x_by_token = 1;
  a.out = ctx->h_mid;
  hipError_t e;
  if (c.act_dtype == MOE_F32) e = launch_gemv_t<WT, MOE_F32, true>(a, ctx->umax, T, s);
  else e = launch_gemv_t<WT, MOE_BF16, true>(a, ctx->umax, T, s);
  if (e != hipSuccess) return e;
  // down: rows H, contraction I, input the fp32 intermediate of each pair
  if constexpr (WT == MOE_MXFP4) {
    a.off0 = (size_t)I * H;
    a.soff0 = 3 * (size_t)H * I / 2 + 2 * (size_t)I * H / 32;
  } else {
    a.off0 = 2 * (size_t)I * H * eb;
  }
  a.K = I;
  a.rows = H;
  a.x = ctx->h_mid;
  a.x_by_token = 0;
  a.out = ctx->p_gpu;
  return launch_gemv_t<WT, MOE_F32, false>(a, ctx->umax, T, s);
}

hipError_t launch_ffn(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  if (ctx->n_slots == 0) return hipSuccess;
  switch (ctx->cfg.w_dtype) {
    case MOE_F32: return launch_ffn_w<MOE_F32>(ctx, x, T, s);
    case MOE_BF16: return launch_ffn_w<MOE_BF16>(ctx, x, T, s);
    default: return launch_ffn_w<MOE_MXFP4>(ctx, x, T, s);
  }
}

// ------------------------------------------------------------------ merge
// y[t] = sum over ascending j of w[t][j] * P[t][j], P from the GPU rows or the
// host rows by the sign of slot_map (snackonai, "What It Actually Does";
// satyajit, "Decode: the one equation").  fp32, one rounding to the output.
// A token with host pairs first waits for the host branch to publish this
// call's sequence number (bounded: after wait_ticks it flags an error).
template <int AT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ w,
                                                    const int32_t* __restrict__ slot_map,
                                                    const float* __restrict__ pg,
                                                    const float* pc, int k, int H,
                                                    void* __restrict__ y, HostSync* sync,
                                                    int64_t seq, uint64_t wait_ticks) {
  __shared__ int s_ok;
  const int t = blockIdx.y;
  bool host = false;
  for (int j = 0; j < k; ++j) host |= slot_map[t * k + j] < 0;
  if (host) {
    if (threadIdx.x == 0) {
      const uint64_t t0 = wall_clock64();
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
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    float v;
    if (slot_map[p] >= 0) v = pg[(size_t)p * H + h];
    else v = __hip_atomic_load(pc + (size_t)p * H + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    acc = fmaf(w[p], v, acc);
  }
  if constexpr (AT == MOE_F32) {
    ((float*)y)[(size_t)t * H + h] = acc;
  } else {
    uint32_t u = __float_as_uint(acc);
    u += 0x7FFFu + ((u >> 16) & 1u);
    ((uint16_t*)y)[(size_t)t * H + h] = (uint16_t)(u >> 16);
  }
}

hipError_t launch_merge(moe_ctx* ctx, const float* w, int T, void* y, int64_t seq, hipStream_t s) {
  const int H = ctx->cfg.hidden;
  dim3 grid((H + 255) / 256, T), block(256);
  if (ctx->cfg.act_dtype == MOE_F32)
    hipLaunchKernelGGL(merge_kernel<MOE_F32>, grid, block, 0, s, w, ctx->plan.slot_map, ctx->p_gpu,
                       ctx->p_cpu_dev, ctx->cfg.top_k, H, y, ctx->sync_dev, seq, ctx->wait_ticks);
  else
    hipLaunchKernelGGL(merge_kernel<MOE_BF16>, grid, block, 0, s, w, ctx->plan.slot_map, ctx->p_gpu,
                       ctx->p_cpu_dev, ctx->cfg.top_k, H, y, ctx->sync_dev, seq, ctx->wait_ticks);
  return hipGetLastError();
}

}  // namespace moert
