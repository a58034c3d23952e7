// Decode expert FFN: one launch per layer call over every GPU-resident routed
// expert of the last plan (snackonai, "The Code, Annotated": grouped
// evaluation after the cache update and the batched copy).
//
// Decode reads each routed expert's complete weights once per call, so the
// launch is an HBM stream with a dependency in the middle: the down
// projection of an expert needs its whole SiLU(gate) * up intermediate.  One
// grid holds both halves:
//   * gate/up items (the first waves of the grid, expert by expert): RW_A rows
//     of W_gate and W_up of one expert.  The wave finds its expert's first
//     routed pair and requests that token's inputs, then loads its weight rows
//     into registers (lane l holds 16-byte chunks l, l+64, ... of each row),
//     evaluates every routed token of the expert, reduces the rows across the
//     wave and stores h = silu(g) * u (fp32) per token;
//   * down items (the later workgroups, four row blocks of one expert each):
//     RW_B rows of W_down per wave.  The waves load their rows first (they
//     stream behind the gate/up weights), then the workgroup collects h of
//     each routed pair into LDS as it becomes valid, and every wave writes
//     its fp32 partial rows.
// Memory serves requests roughly in issue order, so the gate/up halves
// finish while the down weights are still streaming and h is mostly valid
// when a down wave gets its data.  A grid the chip nearly holds at once
// puts every gate/up item first; in a larger one an expert's down items
// follow the gate/up items of a few experts later (ffn_lag).  Workgroups are dispatched in index order
// and every down item follows all gate/up items of its own expert, so a
// waiting down item only waits for items that are already running; the
// wait is still bounded (wall clock) and flags an error instead of hanging.
//
// The intermediate crosses compute dies (each XCD has its own L2), so it
// moves with device-coherent accesses instead of cache-wide fences.  Each
// value travels with its own validity mark: one 64-bit device-scope store of
// {value, low 32 bits of the call's LRU tick}, which a reader sees whole or
// not at all.  A gate/up wave therefore stores and exits, with no wait for
// its stores and no completion counter (a counter has to wait until the
// stores behind it have reached memory, which under a full read queue takes
// microseconds and holds the wave's slot from the down workgroups still to be
// dispatched); a down workgroup polls the entries it needs until their marks
// equal this call's.  The control kernel rewrites every mark once per 2^30
// ticks to a value no tick of the new epoch has, so an entry left from an
// earlier call never matches, also where the low word wraps.
//
// Arithmetic: bf16 x bf16 uses the two-term bf16 dot with fp32 accumulation;
// MXFP4 weights are expanded with the gfx950 scaled FP4 converts (to bf16
// pairs against bf16 activations, to fp32 pairs against fp32 inputs), the
// E8M0 scale applied in the convert; everything accumulates in fp32.  Row
// totals use a transpose reduction: at each cross-lane step a lane keeps half
// of its values and takes the partner's copy of that half, so R rows cost
// R - 1 + 6 - log2(R) lane moves instead of 6 R; the moves are DPP and the
// gfx950 lane swaps, not LDS permutes.
#pragma once

#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace moert {

typedef __bf16 ffn_bf16x2 __attribute__((ext_vector_type(2)));
typedef float ffn_f32x2 __attribute__((ext_vector_type(2)));

struct FfnArgs {
  const uint8_t* slot_base;
  size_t stride;
  const moe_plan_counts* counts;
  const int32_t* gpu_slot;    // [n_gpu] slot of each GPU-resident routed expert
  const int32_t* slot_map;    // [Tk] slot of each (token, rank) pair, -1 = host
  int Tk, k, H, I;
  size_t og, ou, od;          // byte offsets of W_gate, W_up, W_down (codes for MXFP4)
  size_t sg, su, sd;          // byte offsets of their E8M0 scales (MXFP4)
  const void* x;              // [T][H] activations
  uint64_t* h;                // [Tk][I] {fp32 bits, tick mark} intermediate
  float* p;                   // [Tk][H] fp32 partial rows
  HostSync* sync;             // error word (2 = a down item gave up waiting)
  uint64_t wait_ticks;
  int umax;
  int itemsA, itemsB;         // row blocks per expert
  int blocksA;                // workgroups of gate/up items (lag < 0)
  int blocksAe;               // gate/up workgroups per expert (lag >= 0)
  int blocksB;                // down workgroups per expert
  int lag;                    // < 0: all gate/up items first; else per expert, each expert's
                              // down items after the gate/up items of the expert lag places on
                              // (every down item still after its own expert's gate/up items)
  int cplA, cplB;             // 16-byte chunks per lane per row
};

template <int WT> struct FfnChunk;
template <> struct FfnChunk<MOE_F32> { static constexpr int CH = 4; };
template <> struct FfnChunk<MOE_BF16> { static constexpr int CH = 8; };
template <> struct FfnChunk<MOE_MXFP4> { static constexpr int CH = 32; };

// chunk slots per lane: gate/up items hold FfnRegA per matrix, down items
// FfnRegB; rows per wave = slots / chunks per lane of a row, at least one.
// bf16 / fp32: eight loads of 16 B in flight per lane per item, whose
// smaller items leave less arithmetic on the tail of the launch than
// sixteen.  MXFP4 keeps sixteen for gate/up: its kernel's registers are set
// by the FP4 converts, so smaller items bring no more waves per SIMD.
template <int WT> struct FfnRegA { static constexpr int N = WT == MOE_MXFP4 ? 8 : 4; };
template <int WT> struct FfnRegB { static constexpr int N = 8; };
__host__ __device__ constexpr int ffn_rows(int slots, int cpl) { return slots / cpl > 0 ? slots / cpl : 1; }

__device__ inline float ffn_bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float ffn_bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// OCP MX E8M0: 2^(s - 127); s = 0 is 2^-127 (a float subnormal).
__device__ inline float ffn_e8m0(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

struct WChunk16 {
  uint4 v;     // 16 raw bytes
  uint32_t s;  // E8M0 scale byte (MXFP4)
};

// An empty asm that claims to rewrite the chunk: keeps the compiler from
// hoisting its expansion (bf16 or FP4 to fp32) out of the token loop, which
// would hold every weight in fp32 registers and cut occupancy.
template <int WT>
__device__ inline void ffn_pin(WChunk16& c) {
  asm volatile("" : "+v"(c.v.x), "+v"(c.v.y), "+v"(c.v.z), "+v"(c.v.w));
  if constexpr (WT == MOE_MXFP4) asm volatile("" : "+v"(c.s));
}

typedef unsigned int ffn_u32x4 __attribute__((ext_vector_type(4)));

// Weight bytes are read once per call: nontemporal (streaming) loads, which
// a plain 72 MB read of 16 loads in flight per lane completes about 13%
// sooner than with ordinary loads.
__device__ inline uint4 ffn_stream16(const uint8_t* p) {
  const ffn_u32x4 v = __builtin_nontemporal_load((const ffn_u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int WT>
__device__ inline WChunk16 ffn_load_w(const uint8_t* __restrict__ mat, const uint8_t* __restrict__ sc,
                                      int row, int K, int ch) {
  WChunk16 c;
  if constexpr (WT == MOE_F32) {
    c.v = ffn_stream16(mat + ((size_t)row * K + (size_t)ch * 4) * 4);
    c.s = 127;
  } else if constexpr (WT == MOE_BF16) {
    c.v = ffn_stream16(mat + ((size_t)row * K + (size_t)ch * 8) * 2);
    c.s = 127;
  } else {
    c.v = ffn_stream16(mat + (size_t)row * (K / 2) + (size_t)ch * 16);
    c.s = __builtin_nontemporal_load(sc + (size_t)row * (K / 32) + ch);
  }
  return c;
}

// The input values matching one weight chunk, as 32-bit words.
template <int WT, int XT> struct XWords {
  static constexpr int N = FfnChunk<WT>::CH * (XT == MOE_F32 ? 4 : 2) / 4;
  uint32_t w[N];
};

template <int WT, int XT>
__device__ inline void ffn_load_x(const void* __restrict__ x, size_t elem0, int ch, XWords<WT, XT>& o) {
  constexpr int CH = FfnChunk<WT>::CH;
  constexpr int EB = XT == MOE_F32 ? 4 : 2;
  constexpr int N = XWords<WT, XT>::N;
  const uint8_t* p = (const uint8_t*)x + (elem0 + (size_t)ch * CH) * EB;
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 v = ((const uint4*)p)[i];
      o.w[4 * i] = v.x; o.w[4 * i + 1] = v.y; o.w[4 * i + 2] = v.z; o.w[4 * i + 3] = v.w;
    }
  } else {
    const uint2 v = *(const uint2*)p;
    o.w[0] = v.x; o.w[1] = v.y;
  }
}

template <int SEL, int XT>
__device__ inline float ffn_mx_pair(uint32_t word, float scale, const uint32_t* xw, float acc) {
  // elements 2*SEL and 2*SEL+1 of this word's eight (low nibble = even)
  if constexpr (XT == MOE_BF16) {
    const ffn_bf16x2 wp = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, SEL);
    return __builtin_amdgcn_fdot2_f32_bf16(wp, __builtin_bit_cast(ffn_bf16x2, xw[SEL]), acc, false);
  } else {
    const ffn_f32x2 wp = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, SEL);
    acc = fmaf(wp[0], __uint_as_float(xw[2 * SEL]), acc);
    return fmaf(wp[1], __uint_as_float(xw[2 * SEL + 1]), acc);
  }
}

// acc + <weight chunk, input chunk>
template <int WT, int XT>
__device__ inline float ffn_dot(const WChunk16& c, const XWords<WT, XT>& x, float acc) {
  const uint32_t w[4] = {c.v.x, c.v.y, c.v.z, c.v.w};
  if constexpr (WT == MOE_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float xv;
      if constexpr (XT == MOE_F32) xv = __uint_as_float(x.w[i]);
      else xv = (i & 1) ? ffn_bf_hi(x.w[i >> 1]) : ffn_bf_lo(x.w[i >> 1]);
      acc = fmaf(__uint_as_float(w[i]), xv, acc);
    }
  } else if constexpr (WT == MOE_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XT == MOE_BF16) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ffn_bf16x2, w[i]),
                                              __builtin_bit_cast(ffn_bf16x2, x.w[i]), acc, false);
      } else {
        acc = fmaf(ffn_bf_lo(w[i]), __uint_as_float(x.w[2 * i]), acc);
        acc = fmaf(ffn_bf_hi(w[i]), __uint_as_float(x.w[2 * i + 1]), acc);
      }
    }
  } else {
    const float s = ffn_e8m0(c.s);
    constexpr int XPW = XT == MOE_BF16 ? 4 : 8;  // input words per weight word
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* xw = x.w + XPW * i;
      acc = ffn_mx_pair<0, XT>(w[i], s, xw, acc);
      acc = ffn_mx_pair<1, XT>(w[i], s, xw, acc);
      acc = ffn_mx_pair<2, XT>(w[i], s, xw, acc);
      acc = ffn_mx_pair<3, XT>(w[i], s, xw, acc);
    }
  }
  return acc;
}

// Cross-lane steps of the row reduction, all in the vector ALU (an LDS
// permute per step would put a round trip through the LDS unit on every
// step of the tail of the launch).
//
// x of the lane paired with this one at step O = 1, 2, 4, 8 (DPP within a
// row of 16): xor 1 and xor 2 by quad permutes, 4 and 8 by the half-row and
// row mirrors, which pair each lane with one whose bit O differs.
template <int O>
__device__ inline float ffn_dpp_pair(float x) {
  constexpr int ctrl = O == 1 ? 0xB1 : O == 2 ? 0x4E : O == 4 ? 0x141 : 0x140;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
}

// Step O = 16 or 32 by the gfx950 row / half-wave swaps: lanes whose bit O is
// clear get the pair's sum of a, lanes whose bit O is set the pair's sum of b.
template <int O>
__device__ inline float ffn_swap_sum(float a, float b) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// Transpose reduction of N values across the wave (N a power of two <= 64),
// steps O = 32, 16, ..., 1: at each a lane keeps the half of its values that
// its bit O selects and adds the partner's copy of that half.  Afterwards
// lane l holds the wave total of value l >> (6 - log2 N) in v[0].
template <int N, int O = 32>
__device__ inline void ffn_xreduce(float* v, int lane) {
  if constexpr (N > 1) {
    constexpr int HN = N / 2;
    if constexpr (O >= 16) {
#pragma unroll
      for (int i = 0; i < HN; ++i) v[i] = ffn_swap_sum<O>(v[i], v[i + HN]);
    } else {
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < HN; ++i) {
        const float send = up ? v[i] : v[i + HN];
        const float keep = up ? v[i + HN] : v[i];
        v[i] = keep + ffn_dpp_pair<O>(send);
      }
    }
    ffn_xreduce<HN, O / 2>(v, lane);
  } else if constexpr (O >= 1) {
    if constexpr (O >= 16) v[0] = ffn_swap_sum<O>(v[0], v[0]);
    else v[0] += ffn_dpp_pair<O>(v[0]);
    ffn_xreduce<1, O / 2>(v, lane);
  }
}

template <int N> struct Log2 { static constexpr int v = 1 + Log2<N / 2>::v; };
template <> struct Log2<1> { static constexpr int v = 0; };

// Next routed pair of `slot` (ascending pair index), or -1.  `base` / `bm`
// carry the wave's position in slot_map between calls (wave-uniform).
__device__ inline int ffn_next_pair(const FfnArgs& a, int slot, int lane, int& base, uint64_t& bm) {
  while (bm == 0 && base + 64 < a.Tk) {
    base += 64;
    bm = __ballot(base + lane < a.Tk && a.slot_map[base + lane] == slot);
  }
  if (bm == 0) return -1;
  const int p = base + __builtin_ctzll(bm);
  bm &= bm - 1;
  return p;
}

__device__ inline float ffn_silu(float g) { return g / (1.f + expf(-g)); }

template <int WT, int XT, int CPL>
__device__ void ffn_gate_up(const FfnArgs& a, int g, int rb, int lane) {
  constexpr int CH = FfnChunk<WT>::CH;
  constexpr int RW = ffn_rows(FfnRegA<WT>::N, CPL);
  const int K = a.H, nch = K / CH, row0 = rb * RW;
  const uint64_t mark = (uint64_t)(uint32_t)a.counts->tick_lo << 32;

  // the slot and its first routed pair come first, so that pair's inputs
  // are requested ahead of the weights and arrive with them
  const int sm0 = lane < a.Tk ? a.slot_map[lane] : -2;
  const int slot = __builtin_amdgcn_readfirstlane(a.gpu_slot[g]);
  int base = 0;
  uint64_t bm = __ballot(sm0 == slot);
  int p = ffn_next_pair(a, slot, lane, base, bm);
  XWords<WT, XT> xw[CPL];
  if (p >= 0) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      ffn_load_x<WT, XT>(a.x, (size_t)(p / a.k) * K, min(lane + 64 * c, nch - 1), xw[c]);
  }

  // every lane loads (chunks past the row end read a valid chunk and are
  // zeroed), so the loads issue back to back without branches
  const uint8_t* sp = a.slot_base + (size_t)slot * a.stride;
  WChunk16 wg[RW][CPL], wu[RW][CPL];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = min(row0 + r, a.I - 1);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = min(lane + 64 * c, nch - 1);
      wg[r][c] = ffn_load_w<WT>(sp + a.og, sp + a.sg, row, K, ch);
      wu[r][c] = ffn_load_w<WT>(sp + a.ou, sp + a.su, row, K, ch);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (64 * (c + 1) > nch) {  // uniform: only a partial last column of chunks
      const bool ok = lane + 64 * c < nch;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        if (!ok) wg[r][c].v = wu[r][c].v = make_uint4(0, 0, 0, 0);
      }
    }
  }

  while (p >= 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        ffn_pin<WT>(wg[r][c]);
        ffn_pin<WT>(wu[r][c]);
      }
    float v[2 * RW];
#pragma unroll
    for (int i = 0; i < 2 * RW; ++i) v[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        v[r] = ffn_dot<WT, XT>(wg[r][c], xw[c], v[r]);
        v[RW + r] = ffn_dot<WT, XT>(wu[r][c], xw[c], v[RW + r]);
      }
    // gate totals land in lanes 0..31, up totals in lanes 32..63
    ffn_xreduce<2 * RW>(v, lane);
    // lane l < 32 takes lane l + 32's value
    const float up = __uint_as_float(
        __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false)[1]);
    constexpr int SH = 6 - Log2<2 * RW>::v;
    const int r = lane >> SH;
    if (lane < 32 && (lane & ((1 << SH) - 1)) == 0 && row0 + r < a.I)
      __hip_atomic_store(a.h + (size_t)p * a.I + row0 + r, mark | __float_as_uint(ffn_silu(v[0]) * up),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p = ffn_next_pair(a, slot, lane, base, bm);
    if (p >= 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        ffn_load_x<WT, XT>(a.x, (size_t)(p / a.k) * K, min(lane + 64 * c, nch - 1), xw[c]);
    }
  }
}

// h entries per thread of the first routed pair that a down workgroup
// requests together with its weights (all of h for I <= 1,024)
constexpr int kHEarly = 4;

__device__ inline uint64_t ffn_load_h(const uint64_t* e) {
  return __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One entry of h into LDS once it carries this call's mark (v: its first
// reading).  A thread that waits past the bound flags error 2 and goes on
// with what it has (the call then fails).
__device__ inline void ffn_take_h(const FfnArgs& a, const uint64_t* e, uint64_t v, uint32_t want,
                                  uint64_t& t0, float* dst) {
  while ((uint32_t)(v >> 32) != want) {
    if (t0 == 0) t0 = wall_clock64();
    if (wall_clock64() - t0 > a.wait_ticks) {
      __hip_atomic_store(&a.sync->error, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    v = ffn_load_h(e);
  }
  *dst = __uint_as_float((uint32_t)v);
}

// h of pair p into LDS (256 threads); `early` holds the first readings of
// the thread's first kHEarly entries when EARLY.
template <bool EARLY>
__device__ inline void ffn_collect_h(const FfnArgs& a, int p, int K, uint32_t want, float* lds_h,
                                     const uint64_t (&early)[kHEarly]) {
  const uint64_t* hp = a.h + (size_t)p * K;
  uint64_t t0 = 0;
#pragma unroll
  for (int j = 0; j < kHEarly; ++j) {
    const int i = (int)threadIdx.x + 256 * j;
    if (i < K) ffn_take_h(a, hp + i, EARLY ? early[j] : ffn_load_h(hp + i), want, t0, lds_h + i);
  }
  for (int i = (int)threadIdx.x + 256 * kHEarly; i < K; i += 256)
    ffn_take_h(a, hp + i, ffn_load_h(hp + i), want, t0, lds_h + i);
}

// Down items run as whole workgroups of one expert (four row blocks): the
// workgroup collects h of each routed pair in LDS once and every wave reads
// its chunks from there.
template <int WT, int CPL>
__device__ void ffn_down(const FfnArgs& a, int g, int rb, int lane, float* lds_h) {
  constexpr int CH = FfnChunk<WT>::CH;
  constexpr int RW = ffn_rows(FfnRegB<WT>::N, CPL);
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const uint32_t want = (uint32_t)a.counts->tick_lo;
  const int sm0 = lane < a.Tk ? a.slot_map[lane] : -2;
  const int slot = __builtin_amdgcn_readfirstlane(a.gpu_slot[g]);
  const uint8_t* sp = a.slot_base + (size_t)slot * a.stride;
  const int K = a.I, nch = K / CH, row0 = rb * RW;

  // the weights do not depend on h: load them before waiting (row blocks
  // past the end, which pad the workgroup, read the last row and write nothing)
  WChunk16 wd[RW][CPL];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = min(row0 + r, a.H - 1);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      wd[r][c] = ffn_load_w<WT>(sp + a.od, sp + a.sd, row, K, min(lane + 64 * c, nch - 1));
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    if (64 * (c + 1) > nch) {
      const bool ok = lane + 64 * c < nch;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        if (!ok) wd[r][c].v = make_uint4(0, 0, 0, 0);
      }
    }
  }

  // the first pair's h is requested right behind the weights: it is mostly
  // complete by the time the weights arrive, and then comes with them
  int base = 0;
  uint64_t bm = __ballot(sm0 == slot);
  int p = ffn_next_pair(a, slot, lane, base, bm);  // uniform in the workgroup
  uint64_t early[kHEarly];
#pragma unroll
  for (int j = 0; j < kHEarly; ++j) {
    const int i = (int)threadIdx.x + 256 * j;
    early[j] = p >= 0 && i < K ? ffn_load_h(a.h + (size_t)p * K + i) : 0;
  }
  for (bool first = true; p >= 0; p = ffn_next_pair(a, slot, lane, base, bm), first = false) {
    __syncthreads();  // the previous pair's reads of LDS are done
    if (first) ffn_collect_h<true>(a, p, K, want, lds_h, early);
    else ffn_collect_h<false>(a, p, K, want, lds_h, early);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int c = 0; c < CPL; ++c) ffn_pin<WT>(wd[r][c]);
    float v[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) v[i] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      XWords<WT, MOE_F32> hw;
      const int ch = min(lane + 64 * c, nch - 1);
#pragma unroll
      for (int i = 0; i < CH / 4; ++i) {
        const u32x4v q = ((const u32x4v*)lds_h)[ch * (CH / 4) + i];
        hw.w[4 * i] = q[0]; hw.w[4 * i + 1] = q[1]; hw.w[4 * i + 2] = q[2]; hw.w[4 * i + 3] = q[3];
      }
#pragma unroll
      for (int r = 0; r < RW; ++r) v[r] = ffn_dot<WT, MOE_F32>(wd[r][c], hw, v[r]);
    }
    ffn_xreduce<RW>(v, lane);
    constexpr int SH = 6 - Log2<RW>::v;
    const int r = lane >> SH;
    if ((lane & ((1 << SH) - 1)) == 0 && row0 + r < a.H) a.p[(size_t)p * a.H + row0 + r] = v[0];
  }
}

// One kernel per (format, activation type, chunks per lane of the two
// contraction lengths), so each holds only the registers its shape needs.
template <int WT, int XT, int CPLA, int CPLB>
__global__ __launch_bounds__(256) void ffn_kernel(FfnArgs a) {
  extern __shared__ float lds_h[];  // [I] h of one pair (down workgroups)
  const int lane = threadIdx.x & 63;
  // wave-uniform values held in scalar registers: slot addresses then go in
  // the scalar base of each load, the per-lane part in a 32-bit offset
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int n_gpu = a.counts->n_gpu;
  const int w4 = (int)(threadIdx.x >> 6);
  if (a.lag < 0) {
    if ((int)blockIdx.x < a.blocksA) {
      const int g = wave / a.itemsA;
      if (g < n_gpu && g < a.umax) ffn_gate_up<WT, XT, CPLA>(a, g, wave - g * a.itemsA, lane);
    } else {
      // whole workgroups of one expert, four row blocks each
      const int b = (int)blockIdx.x - a.blocksA;
      const int g = b / a.blocksB;
      const int rb = (b - g * a.blocksB) * 4 + w4;
      if (g < n_gpu && g < a.umax) ffn_down<WT, CPLB>(a, g, rb, lane, lds_h);
    }
    return;
  }
  // per expert: the gate/up workgroups of expert j, then the down workgroups
  // of expert j - lag; every down workgroup still follows all gate/up
  // workgroups of its expert in dispatch order
  const int A = a.blocksAe, Bw = a.blocksB, L = a.lag;
  int b = (int)blockIdx.x, g, r;
  bool up;
  if (b < L * A) {
    g = b / A;
    r = b - g * A;
    up = true;
  } else {
    b -= L * A;
    const int pairs = a.umax - L;
    if (b < pairs * (A + Bw)) {
      const int j = b / (A + Bw);
      r = b - j * (A + Bw);
      up = r < A;
      g = up ? L + j : j;
      if (!up) r -= A;
    } else {
      b -= pairs * (A + Bw);
      g = pairs + b / Bw;
      r = b - (g - pairs) * Bw;
      up = false;
    }
  }
  if (g >= n_gpu || g >= a.umax) return;
  const int rb = r * 4 + w4;
  if (up) {
    if (rb < a.itemsA) ffn_gate_up<WT, XT, CPLA>(a, g, rb, lane);
  } else {
    ffn_down<WT, CPLB>(a, g, rb, lane, lds_h);
  }
}

// Dispatch order of the FFN grid (see FfnArgs::lag).  A grid smaller than
// twice the workgroups the chip holds at once puts every gate/up item
// first.  A larger one would start its down items late, queued behind all
// gate/up items; there each expert's down items follow the gate/up items of
// the expert `lag` places on, about 36 MB of gate/up weights later, so its h
// is mostly complete when its own weights arrive.  Measured: 8 tokens of the
// Qwen-shaped experts (6.3 MB of gate/up weights each, a grid about ten
// times what fits): lag 0 / 2 / 4 / 6 / 8 / 16 and all gate/up first gave
// 58.1 / 50.4 / 47.1 / 46.7 / 46.9 / 47.6 / 48.4 us; one token of the
// DeepSeek-shaped MXFP4 experts (2,048 workgroups, twice what fits): lag 5
// 20.2 us against 20.7; one token of the Qwen-shaped experts (2,560
// workgroups, 1,792 resident): all gate/up first 15.8 us against 16.3 at
// lag 6.
inline int ffn_lag(int64_t blocks, int64_t resident, int umax, size_t gate_up_bytes) {
  if (blocks < 2 * resident) return -1;
  const size_t target = (size_t)36 << 20;
  const int lag = (int)((target + gate_up_bytes - 1) / gate_up_bytes);
  return std::max(1, std::min(lag, umax));
}

// Workgroups of one FFN kernel instance the device holds at once (counted
// once per process; every device a context runs on is the same model).
template <int WT, int XT, int CPLA, int CPLB>
int64_t ffn_resident_blocks(size_t lds) {
  static int64_t resident = 0;
  if (resident == 0) {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)ffn_kernel<WT, XT, CPLA, CPLB>,
                                                     256, lds) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 1;  // unknown: treated as a large grid
    resident = std::max<int64_t>(1, (int64_t)per_cu * cus);
  }
  return resident;
}

// chunks per lane for a row of nch 16-byte chunks (nch <= 512)
inline int ffn_cpl(int nch) { return nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 256 ? 4 : 8; }

template <int WT>
hipError_t launch_ffn_typed(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  constexpr int CH = FfnChunk<WT>::CH;
  const moe_config& c = ctx->cfg;
  const int H = c.hidden, I = c.inter;
  FfnArgs a{};
  a.slot_base = ctx->pool.base;
  a.stride = ctx->stride;
  a.counts = ctx->plan.counts;
  a.gpu_slot = ctx->plan.gpu_slot;
  a.slot_map = ctx->plan.slot_map;
  a.Tk = T * c.top_k;
  a.k = c.top_k;
  a.H = H;
  a.I = I;
  if constexpr (WT == MOE_MXFP4) {
    a.og = 0;
    a.ou = (size_t)I * H / 2;
    a.od = (size_t)I * H;
    a.sg = 3 * (size_t)H * I / 2;
    a.su = a.sg + (size_t)I * H / 32;
    a.sd = a.su + (size_t)I * H / 32;
  } else {
    const size_t eb = WT == MOE_F32 ? 4 : 2;
    a.og = 0;
    a.ou = (size_t)I * H * eb;
    a.od = 2 * (size_t)I * H * eb;
  }
  a.x = x;
  a.h = ctx->h_mid;
  a.p = ctx->p_gpu;
  a.sync = ctx->sync_dev;
  a.wait_ticks = ctx->ffn_wait_ticks;
  a.umax = ctx->umax;
  a.cplA = ffn_cpl(H / CH);
  a.cplB = ffn_cpl(I / CH);
  const int rwA = ffn_rows(FfnRegA<WT>::N, a.cplA), rwB = ffn_rows(FfnRegB<WT>::N, a.cplB);
  a.itemsA = (I + rwA - 1) / rwA;
  a.itemsB = (H + rwB - 1) / rwB;
  a.blocksA = (int)(((int64_t)a.umax * a.itemsA + 3) / 4);
  a.blocksAe = (a.itemsA + 3) / 4;
  a.blocksB = (a.itemsB + 3) / 4;
  // gate/up bytes of one expert: two matrices (and their scales)
  const size_t gate_up_bytes = 2 * (a.ou - a.og) + (WT == MOE_MXFP4 ? 2 * (a.su - a.sg) : 0);
  const int64_t blocks_first = a.blocksA + (int64_t)a.umax * a.blocksB;
  const size_t lds = sizeof(float) * (size_t)I;
  const dim3 block(256);
  auto go = [&](auto xt, auto ca, auto cb) {
    constexpr int XT = decltype(xt)::value, CA = decltype(ca)::value, CB = decltype(cb)::value;
    a.lag = ffn_lag(blocks_first, ffn_resident_blocks<WT, XT, CA, CB>(lds), a.umax, gate_up_bytes);
    const int64_t nblocks = a.lag < 0 ? blocks_first : (int64_t)a.umax * (a.blocksAe + a.blocksB);
    if (ctx->ffn_ev[0])
      hipExtLaunchKernelGGL((ffn_kernel<WT, XT, CA, CB>), dim3((unsigned)nblocks), block, lds, s,
                            ctx->ffn_ev[0], ctx->ffn_ev[1], 0, a);
    else
      hipLaunchKernelGGL((ffn_kernel<WT, XT, CA, CB>), dim3((unsigned)nblocks), block, lds, s, a);
  };
  auto by_b = [&](auto xt, auto ca) {
    switch (a.cplB) {
      case 1: go(xt, ca, std::integral_constant<int, 1>{}); break;
      case 2: go(xt, ca, std::integral_constant<int, 2>{}); break;
      case 4: go(xt, ca, std::integral_constant<int, 4>{}); break;
      default: go(xt, ca, std::integral_constant<int, 8>{}); break;
    }
  };
  auto by_a = [&](auto xt) {
    switch (a.cplA) {
      case 1: by_b(xt, std::integral_constant<int, 1>{}); break;
      case 2: by_b(xt, std::integral_constant<int, 2>{}); break;
      case 4: by_b(xt, std::integral_constant<int, 4>{}); break;
      default: by_b(xt, std::integral_constant<int, 8>{}); break;
    }
  };
  if (c.act_dtype == MOE_F32) by_a(std::integral_constant<int, MOE_F32>{});
  else by_a(std::integral_constant<int, MOE_BF16>{});
  return hipGetLastError();
}

}  // namespace moert
