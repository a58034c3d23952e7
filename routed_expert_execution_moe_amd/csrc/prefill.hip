// Prefill compute for one chunk of T tokens of one MoE layer whose E experts
// sit in the full-layer buffer b (layer % 2, or 0 when the context runs one
// buffer), slots [b*E, (b+1)*E)
// (satyajit, "Prefill: hide the pool behind the wire").
//
//   1. group    per-expert counts of the T*k routed pairs, offsets, the list
//               of 128-row M-tiles, and the permutation pos -> pair (pairs of
//               an expert contiguous; order inside an expert is not
//               significant: every output row is computed independently with
//               the same arithmetic);
//   2. GEMM1    per expert, gathered token rows x [n_e, H] times the gate and
//               up matrices [I, H] (MXFP4, dequantised to bf16 in registers)
//               with bf16 MFMA and fp32 accumulation; epilogue
//               h = silu(g) * u rounded to bf16, rows in pos order;
//   3. GEMM2    h [n_e, I] times the down matrix [H, I] -> fp32 rows per pair;
//   4. merge    y[t] = sum over ascending j of w[t][j] * P[t*k + j], fp32,
//               one rounding to the output dtype.
// Everything is deterministic: no atomics touch outputs.
//
// GEMM tiling (gfx950, v_mfma_f32_32x32x16_bf16): a workgroup of 4 waves owns
// a 128-row M-tile of one expert and a 256-column N-tile; each wave takes a
// quarter of the columns and every row, in 32-row MFMA blocks, and computes
// only the ceil(rows / 32) blocks the tile holds (an expert's last tile is
// short).  Each wave converts only its own quarter of the B tile.  K steps of 64
// go through three LDS stages that direct-to-LDS copies fill two steps ahead
// (A rows XOR-swizzled by 16-byte chunk, B as raw MXFP4 codes, a quarter of
// its bf16 size, E8M0 scales per two steps).  Each lane dequantises its B
// fragment right before the MFMA with the hardware scaled FP4 -> bf16
// convert.  For GEMM1 the 256 B-tile rows are 128 gate rows then the
// matching 128 up rows, so a wave's gate and up accumulators share lanes and
// the SiLU * up epilogue needs no exchange.  Each XCD takes a contiguous run
// of M-tiles, N-tile outer over groups of four M-tiles, so the N-tiles of an
// M-tile share its A rows and the M-tiles of an expert share its B slices in
// that XCD's L2.  The down GEMM's fp32 output rows leave through the stage
// buffer (written per wave, read back as 16-byte row pieces), so each lane
// stores 16 bytes at a time; the pair index of each tile row is read once
// into LDS at the start.
#include <mutex>
#include <type_traits>

#include "internal.h"

namespace moert {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kRowBytes = kBK * 2;  // one LDS row: 64 bf16

// ------------------------------------------------------------------ grouping
__global__ void group_zero_kernel(int32_t* counts, int32_t* cursor, int E) {
  int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    counts[e] = 0;
    cursor[e] = 0;
  }
}

// pairs per workgroup in the histogram and the scatter
constexpr int kGroupChunk = 2048;

__global__ __launch_bounds__(256) void group_hist_kernel(const int32_t* __restrict__ ids, int Tk, int E,
                                                         int32_t* counts) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < Tk; i += gridDim.x * blockDim.x) {
    int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (h[e]) atomicAdd(&counts[e], h[e]);
}

// offsets[E+1]; M-tile list tiles[i] = (e << 20) | (m0/64 << 1) | half, half
// marking an expert's last tile when it has at most 64 rows; the tile count
// is written to offsets[E+1].
__global__ __launch_bounds__(1024) void group_scan_kernel(const int32_t* counts, int E,
                                                          int32_t* offsets, int32_t* tiles) {
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_toff[kMaxExperts + 1];
  __shared__ int32_t s_cnt[kMaxExperts];
  // the counts come into LDS in parallel, so the serial walk below reads LDS
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = counts[e];
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0, t = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = o;
      s_toff[e] = t;
      o += s_cnt[e];
      t += (s_cnt[e] + kBM - 1) / kBM;
    }
    s_off[E] = o;
    s_toff[E] = t;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  if (threadIdx.x == 0) offsets[E + 1] = s_toff[E];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = s_cnt[e];
    const int nt = (c + kBM - 1) / kBM;
    for (int m = 0; m < nt; ++m) {
      const int half = c - m * kBM <= kBM / 2;  // a last tile of at most 64 rows
      tiles[s_toff[e] + m] = (e << 20) | ((m * kBM / 64) << 1) | half;
    }
  }
}

// Each workgroup takes a chunk of kGroupChunk consecutive pairs: ranks inside
// the chunk come from LDS atomics, then one global atomic per (workgroup,
// expert) reserves the chunk's run in that expert's range, so the shared
// cursors see at most E atomics per workgroup instead of one per pair.
__global__ __launch_bounds__(256) void group_scatter_kernel(const int32_t* __restrict__ ids, int Tk,
                                                            int E, const int32_t* offsets,
                                                            int32_t* cursor, int32_t* perm) {
  __shared__ int32_t s_n[kMaxExperts];
  constexpr int kPer = kGroupChunk / 256;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_n[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kGroupChunk + threadIdx.x;
  int ex[kPer], rank[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = base + q * 256;
    ex[q] = -1;
    rank[q] = 0;
    if (i < Tk) {
      const int e = ids[i];
      if (e >= 0 && e < E) {
        ex[q] = e;
        rank[q] = atomicAdd(&s_n[e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int n = s_n[e];
    s_n[e] = n ? offsets[e] + atomicAdd(&cursor[e], n) : 0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPer; ++q)
    if (ex[q] >= 0) perm[s_n[ex[q]] + rank[q]] = base + q * 256;
}

// ------------------------------------------------------------------ GEMM
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8 MXFP4 codes (4 bytes, low nibble first) times 2^(s-127) -> 8 bf16 with
// the gfx950 scaled convert; e2m1 * 2^k is exact in bf16.
__device__ inline bf16x8 fp4x8_to_bf16(uint32_t raw, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(raw, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ inline float e8m0_scale(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// A rows: 64 bf16 = 8 chunks of 16 B, chunk index XOR ((row / 2) % 8).  Rows
// are 128 B, so with 64 four-byte banks two consecutive rows fill the banks
// once; keying the XOR on row / 2 gives the 16 rows a 16-lane read phase
// touches 16 distinct 16-byte bank groups (row % 8 repeated every 8 rows and
// cost two-way conflicts: 3.0 -> 0.95 conflict cycles per LDS instruction)
__device__ inline int aswz_key(int row) { return (row >> 1) & 7; }
__device__ inline int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ aswz_key(row)) << 4); }
// B rows: 64 codes = 32 B, two 16-byte halves; a lane reads half kg of row n
// (n = 32 consecutive rows per 32 lanes).  Rows 8 apart share banks, so the
// halves of rows with (n / 8) odd are stored swapped (0.95 -> 0 conflict
// cycles per LDS instruction together with the A swizzle)
__device__ inline int bswz_half(int row, int half) { return half ^ ((row >> 3) & 1); }

struct GemmArgs {
  const uint8_t* slot_base;   // slot s at slot_base + s * stride
  size_t stride;
  int slot0;                  // b * E
  const int32_t* slot_of;     // [E] slot of each expert, -1 = skip; nullptr: slot0 + e
  int E, k;
  int K;                      // contraction: H (GEMM1) or I (GEMM2)
  int N;                      // output columns per matrix: I (GEMM1) or H (GEMM2)
  size_t off0, off1;          // code offsets of matrix 0 (gate / down) and 1 (up)
  size_t soff0, soff1;        // scale offsets
  const int32_t* offsets;     // [E+2]
  const int32_t* tiles;       // M-tile list
  const int32_t* perm;        // pos -> pair
  const uint16_t* a_src;      // GEMM1: x [T][H] (rows by token); GEMM2: h [Tk][I] by pos
  uint16_t* h_out;            // GEMM1 output [Tk][I] by pos
  float* p_out;               // GEMM2 output [Tk][H] by pair
  int n_ntiles;               // N-tiles per M-tile
  int max_mtiles;             // grid bound on M-tiles
};

// Three LDS stages per workgroup; the global -> LDS copies of K step kt+2
// are issued (direct-to-LDS loads, no register staging) while step kt is
// computed, so each copy has two steps of MFMA work to land.  The copies are
// issued from inline asm, so the compiler does not serialise LDS reads
// behind them; completion is tracked by hand with the vector-memory counter
// and a workgroup barrier per step.
constexpr int kStageA = kBM * kRowBytes;  // 16 KB: 128 rows x 64 bf16, swizzled
constexpr int kStageB = kBN * 32;         // 8 KB: 256 rows x 64 fp4 codes
constexpr int kStageS = kBN * 4;          // 1 KB: 4 E8M0 bytes per B row = 2 K steps

// 16 bytes per lane from sbase + voff into LDS at lds + 16 * lane
__device__ inline void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
// 4 bytes per lane into LDS at lds + 4 * lane
__device__ inline void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               ::"v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

template <bool GLU>
__global__ __launch_bounds__(kGemmThreads, 2) void grouped_gemm_kernel(GemmArgs a) {
  // three A and three B stages in one buffer: after the K loop the down
  // GEMM reuses it to stage its output rows
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[3 * kStageA + 3 * kStageB];
  uint8_t* const s_a0 = s_stage;
  uint8_t* const s_a1 = s_stage + kStageA;
  uint8_t* const s_a2 = s_stage + 2 * kStageA;
  uint8_t* const s_b0 = s_stage + 3 * kStageA;
  uint8_t* const s_b1 = s_stage + 3 * kStageA + kStageB;
  uint8_t* const s_b2 = s_stage + 3 * kStageA + 2 * kStageB;
  __shared__ __attribute__((aligned(1024))) uint8_t s_sc[2][kStageS];
  __shared__ int32_t s_rowsrc[kBM];  // A source row per tile row
  __shared__ int32_t s_pair[kBM];    // down: the pair (output row) of each tile row

  // XCD-aware mapping: consecutive workgroups go round-robin over the 8 XCDs.
  // XCD x takes the x-th contiguous eighth of the M-tile list: the N-tiles of
  // an M-tile share its A rows, and the M-tiles of one expert (adjacent in
  // the list) share its B slices, in that XCD's L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int n_mtiles = a.offsets[a.E + 1];
  const int per_xcd = (n_mtiles + 7) >> 3;
  // within the XCD, groups of 4 M-tiles: N-tile outer, M-tile inner, so the
  // up to 4 workgroups that read the same B slice run back to back
  const int grp = local / (4 * a.n_ntiles), rem = local - grp * 4 * a.n_ntiles;
  const int nt = rem >> 2;
  const int ml = grp * 4 + (rem & 3);
  const int mt = xcd * per_xcd + ml;
  if (ml >= per_xcd || mt >= n_mtiles) return;
  const int tile = a.tiles[mt];
  const int e = tile >> 20, m0 = ((tile >> 1) & 0x7FFFF) * 64;
  const bool half = tile & 1;  // a last tile of at most 64 rows
  const int eslot = a.slot_of ? a.slot_of[e] : a.slot0 + e;
  if (eslot < 0) return;  // not in this on-demand pass
  const int pos0 = a.offsets[e] + m0;
  const int rows = min(half ? kBM / 2 : kBM, a.offsets[e + 1] - pos0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // rows past the expert's end (padding of the last M-tile) read the tile's
  // first row: no masked loads, and their results are never written
  if (tid < kBM) {
    const int r = tid < rows ? tid : 0;
    const int p = a.perm[pos0 + r];
    s_rowsrc[tid] = GLU ? p / a.k : pos0 + r;
    s_pair[tid] = p;
  }
  __syncthreads();

  const uint8_t* slot = a.slot_base + (size_t)eslot * a.stride;
  // B tile rows: GLU -> gate rows n0..n0+127 then up rows n0..n0+127 (n0 = nt*128);
  // down -> rows n0..n0+255 (n0 = nt*256)
  const int n0 = GLU ? nt * (kBN / 2) : nt * kBN;
  const int K = a.K;
  const int nk = K / kBK;

  // Copy sources.  A: wave w fills the 1 KB LDS blocks 4w..4w+3 (8 rows
  // each); lane l fills slot l of a block: row 8*blk + l/8, slot l%8, which
  // holds chunk (l%8) ^ aswz_key(row) of that row (the XOR swizzle).  B: wave w
  // fills blocks 2w, 2w+1 (32 rows of 32 bytes); lane l: row 32*blk + l/2,
  // LDS half l%2, which holds the row's half bswz_half(row, l%2).  Scales:
  // wave w fills rows 64w..64w+63, 4 bytes each (the blocks of two K steps).
  // Waves 0-1 copy gate rows, 2-3 up rows (GLU).
  const uint8_t* a_base = (const uint8_t*)a.a_src;
  uint32_t a_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (wave * 4 + q) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ aswz_key(row);
    a_off[q] = (uint32_t)(((size_t)s_rowsrc[row] * K + chunk * 8) * 2);
  }
  const bool up_half = GLU && wave >= 2;
  const uint8_t* b_base = slot + (up_half ? a.off1 : a.off0);
  const uint8_t* s_base = slot + (up_half ? a.soff1 : a.soff0);
  const int mrow_base = n0 - (up_half ? kBN / 2 : 0);
  uint32_t b_off[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    b_off[q] = (uint32_t)((mrow_base + (wave * 2 + q) * 32 + (lane >> 1)) * (K / 2) +
                          bswz_half((wave * 2 + q) * 32 + (lane >> 1), lane & 1) * 16);
  const uint32_t s_off = (uint32_t)((mrow_base + wave * 64 + lane) * (K / 32));

  // the K offset advances the (scalar) base, the per-lane offsets stay fixed
  auto issue = [&](int kt, const uint8_t* la, const uint8_t* lb) {
    const int k0 = kt * kBK;
    const uint8_t* ab = a_base + k0 * 2;
    const uint8_t* bb = b_base + k0 / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(ab, a_off[q], lds_addr(la + (wave * 4 + q) * 1024));
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(bb, b_off[q], lds_addr(lb + (wave * 2 + q) * 1024));
    if ((kt & 1) == 0) dma4(s_base + k0 / 32, s_off, lds_addr(&s_sc[(kt >> 1) & 1][wave * 256]));
  };

  const int lr = lane & 31, kg = lane >> 5;

  // Compute shape: the four waves side by side, each all NI = ceil(rows / 32)
  // row blocks of the tile by 64 columns (NI x 2 MFMA tiles); B rows GLU ->
  // gate 32*w and up 128 + 32*w (a wave's gate and up accumulators share
  // lanes), down -> 64*w + {0,32}.  The copies are the same for every NI (the
  // unused A rows repeat row 0).
  auto run = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;  // 32-row blocks computed: ceil(rows / 32)
    constexpr int NJ = 2;
    const int arow0 = 0;
    int brow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) brow[j] = GLU ? j * (kBN / 2) + wave * 32 : wave * 64 + j * 32;
    f32x16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    // K order inside a step (the same for A and B, so the sum is unchanged):
    // lane half kg at slice ks takes k = 32*kg + 8*ks + [0, 8), i.e. A chunk
    // 4*kg + ks and B code word 4*kg + ks; over the step a lane's B codes are
    // the 16-byte half kg of its row, all under scale block kg.
    auto compute = [&](int kt, const uint8_t* sa, const uint8_t* sb) {
      const uint8_t* ss = s_sc[(kt >> 1) & 1];
      uint4 braw[NJ];
      float bsc[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = brow[j] + lr;
        braw[j] = *(const uint4*)(sb + n * 32 + bswz_half(n, kg) * 16);
        bsc[j] = e8m0_scale(ss[n * 4 + (kt & 1) * 2 + kg]);
      }
      // every A fragment of the step is requested up front, so one LDS
      // latency per step is exposed instead of one per 16-wide slice
      bf16x8 af[kBK / 16][NI];
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < NI; ++i) af[ks][i] = *(const bf16x8*)(sa + swz(arow0 + i * 32 + lr, 4 * kg + ks));
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        bf16x8 bfr[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint32_t w = ks == 0 ? braw[j].x : ks == 1 ? braw[j].y : ks == 2 ? braw[j].z : braw[j].w;
          bfr[j] = fp4x8_to_bf16(w, bsc[j]);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[j], acc[i][j], 0, 0, 0);
      }
    };

    // one K step on stage (sa, sb); the copies for step kt+2 go to (na, nb)
    auto step = [&](int kt, const uint8_t* sa, const uint8_t* sb, const uint8_t* na, const uint8_t* nb) {
      // this wave's copies for step kt are done once at most six (the next
      // step's, one scale copy aside) are still in flight
      if (kt + 1 < nk) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // every wave's copies for step kt are in LDS; step kt-1's reads are done
      if (kt + 2 < nk) issue(kt + 2, na, nb);
      compute(kt, sa, sb);
    };
    issue(0, s_a0, s_b0);
    if (nk > 1) issue(1, s_a1, s_b1);
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
      step(kt, s_a0, s_b0, s_a2, s_b2);
      step(kt + 1, s_a1, s_b1, s_a0, s_b0);
      step(kt + 2, s_a2, s_b2, s_a1, s_b1);
    }
    if (kt < nk) step(kt, s_a0, s_b0, s_a2, s_b2);
    if (kt + 1 < nk) step(kt + 1, s_a1, s_b1, s_a0, s_b0);

    // C element r of lane: row 8*(r/4) + 4*kg + r%4, column lr.
    // Down epilogue: each wave writes 32 of its rows (its NJ*32 columns) to
    // the stage buffer, reads them back as 16-byte row pieces and stores
    // those to the pair's fp32 row, twice (row blocks i = 0, 1).
    if constexpr (!GLU) {
      constexpr int CW = NJ * 32, CS = CW + 4;  // row stride padded by 4 floats
      constexpr int LPR = CW / 4;               // lanes per row
      constexpr int RPI = 64 / LPR;             // rows per read
      static_assert(4 * 32 * CS * 4 <= 3 * kStageA + 3 * kStageB, "staging fits the stage buffer");
      __syncthreads();  // every wave is done reading the stages
      float* cbuf = (float*)s_stage + wave * (32 * CS);
      const int c4 = lane % LPR, rsub = lane / LPR;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) cbuf[(8 * (r >> 2) + 4 * kg + (r & 3)) * CS + j * 32 + lr] = acc[i][j][r];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are in LDS
#pragma unroll
        for (int q = 0; q < 32 / RPI; ++q) {
          const int rl = q * RPI + rsub;
          const float4 v = *(const float4*)&cbuf[rl * CS + c4 * 4];
          const int row = arow0 + i * 32 + rl;
          if (row < rows) *(float4*)&a.p_out[(size_t)s_pair[row] * a.N + n0 + brow[0] + c4 * 4] = v;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block's writes
      }
      return;
    }
    // gate/up epilogue: h = silu(g) * u rounded to bf16, rows in pos order
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = arow0 + i * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
        if (row >= rows) continue;
        if constexpr (GLU) {
#pragma unroll
          for (int j = 0; j < NJ / 2; ++j) {
            const float g = acc[i][j][r], u = acc[i][j + NJ / 2][r];
            const float hv = g * u * __builtin_amdgcn_rcpf(1.f + __expf(-g));
            uint32_t bits = __float_as_uint(hv);
            bits += 0x7FFFu + ((bits >> 16) & 1u);
            const int col = n0 + wave * 32 + lr;
            a.h_out[(size_t)(pos0 + row) * a.N + col] = (uint16_t)(bits >> 16);
          }
        }
      }
    }
  };
  switch ((rows + 31) >> 5) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }
}

// y[t] = sum over ascending j of w[t][j] * P[t*k + j]
template <int AT>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const float* __restrict__ w,
                                                            const int32_t* __restrict__ ids,
                                                            const float* __restrict__ P, int k, int H,
                                                            int E, int T, void* __restrict__ y) {
  // four tokens per workgroup, one wave each; lane l holds columns 4l..4l+3
  // of the workgroup's 256-column slice and reads them as one 16-byte load
  // per pair.  Eight pairs are requested before the first product, so their
  // HBM latencies overlap; the sum still runs over ascending j per column.
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.y * 4 + (threadIdx.x >> 6));
  if (t >= T) return;
  const int h = blockIdx.x * 256 + (threadIdx.x & 63) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
    float wv[8];
    bool ok[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p = t * k + j0 + q;
      ok[q] = false;
      wv[q] = 0.f;
      v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + q < k) {
        const int e = ids[p];
        ok[q] = e >= 0 && e < E;  // pairs of no expert contribute nothing
        if (ok[q]) {
          wv[q] = w[p];
          v[q] = *(const float4*)&P[(size_t)p * H + h];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (ok[q]) {
        a0 = fmaf(wv[q], v[q].x, a0);
        a1 = fmaf(wv[q], v[q].y, a1);
        a2 = fmaf(wv[q], v[q].z, a2);
        a3 = fmaf(wv[q], v[q].w, a3);
      }
  }
  const float acc[4] = {a0, a1, a2, a3};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (AT == MOE_F32) {
      ((float*)y)[(size_t)t * H + h + c] = acc[c];
    } else {
      uint32_t u = __float_as_uint(acc[c]);
      u += 0x7FFFu + ((u >> 16) & 1u);
      ((uint16_t*)y)[(size_t)t * H + h + c] = (uint16_t)(u >> 16);
    }
  }
}

hipError_t launch_prefill_group(moe_ctx* ctx, const PrefillBufs& pf, const int32_t* ids, int T,
                                hipStream_t s) {
  const moe_config& c = ctx->cfg;
  const int E = c.n_experts, Tk = T * c.top_k;
  hipError_t e = timing_begin(ctx, MOE_T_PREFILL_GROUP, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(group_zero_kernel, dim3((E + 255) / 256), dim3(256), 0, s, pf.counts, pf.cursor, E);
  // one workgroup per chunk of pairs: the scatter covers every pair without
  // a stride loop; the histogram takes the same grid (its loop strides)
  const int gb = (Tk + kGroupChunk - 1) / kGroupChunk;
  hipLaunchKernelGGL(group_hist_kernel, dim3(gb), dim3(256), 0, s, ids, Tk, E, pf.counts);
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, s, pf.counts, E, pf.offsets, pf.tiles);
  hipLaunchKernelGGL(group_scatter_kernel, dim3(gb), dim3(256), 0, s, ids, Tk, E, pf.offsets,
                     pf.cursor, pf.perm);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return timing_end(ctx, s);
}

hipError_t launch_prefill_gemm(moe_ctx* ctx, const PrefillBufs& pf, int layer, const void* x, int T,
                               const int32_t* slot_of, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  if (c.w_dtype != MOE_MXFP4 || c.act_dtype != MOE_BF16) return hipErrorNotSupported;
  const int E = c.n_experts, k = c.top_k, H = c.hidden, I = c.inter;
  const int Tk = T * k;
  hipError_t e = timing_begin(ctx, MOE_T_PREFILL_GEMM, s);
  if (e != hipSuccess) return e;
  GemmArgs a{};
  a.slot_base = ctx->pool.base;
  a.stride = ctx->stride;
  a.slot0 = prefill_buffer(ctx, layer) * E;
  a.slot_of = slot_of;
  a.E = E;
  a.k = k;
  a.offsets = pf.offsets;
  a.tiles = pf.tiles;
  a.perm = pf.perm;
  a.max_mtiles = Tk / kBM + E;
  // M-tile slots: 8 XCDs x whole groups of 4 (see the kernel's mapping)
  const int grid_m = (a.max_mtiles + 31) / 32 * 32;
  // GEMM1: gate/up, K = H, N = I
  a.K = H;
  a.N = I;
  a.off0 = 0;
  a.off1 = (size_t)I * H / 2;
  a.soff0 = 3 * (size_t)H * I / 2;
  a.soff1 = a.soff0 + (size_t)I * H / 32;
  a.a_src = (const uint16_t*)x;
  a.h_out = pf.hmid;
  a.n_ntiles = I / (kBN / 2);
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(grid_m * a.n_ntiles), dim3(kGemmThreads), 0, s, a);
  // GEMM2: down, K = I, N = H
  a.K = I;
  a.N = H;
  a.off0 = (size_t)I * H;
  a.soff0 = 3 * (size_t)H * I / 2 + 2 * (size_t)I * H / 32;
  a.a_src = pf.hmid;
  a.p_out = pf.prow;
  a.n_ntiles = H / kBN;
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(grid_m * a.n_ntiles), dim3(kGemmThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return timing_end(ctx, s);
}

hipError_t launch_prefill_merge(moe_ctx* ctx, const PrefillBufs& pf, const int32_t* ids, const float* w,
                                int T, void* y, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  const int E = c.n_experts, k = c.top_k, H = c.hidden;
  hipError_t e = timing_begin(ctx, MOE_T_PREFILL_MERGE, s);
  if (e != hipSuccess) return e;
  // H is a multiple of 256 for every context that runs prefill
  dim3 mg(H / 256, (T + 3) / 4);
  hipLaunchKernelGGL(prefill_merge_kernel<MOE_BF16>, mg, dim3(256), 0, s, w, ids, pf.prow, k, H, E, T, y);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return timing_end(ctx, s);
}

hipError_t launch_prefill_compute(moe_ctx* ctx, const PrefillBufs& pb, int layer, const void* x, int T,
                                  const int32_t* ids, const float* w, void* y, hipStream_t s) {
  const moe_config& c = ctx->cfg;
  if (c.w_dtype != MOE_MXFP4 || c.act_dtype != MOE_BF16) return hipErrorNotSupported;
  hipError_t e = launch_prefill_group(ctx, pb, ids, T, s);
  if (e == hipSuccess) e = launch_prefill_gemm(ctx, pb, layer, x, T, nullptr, s);
  if (e == hipSuccess) e = launch_prefill_merge(ctx, pb, ids, w, T, y, s);
  return e;
}

// ------------------------------------------------------------------ intermediates
size_t prefill_layout(const moe_config& c, int64_t pairs, uint8_t* base, PrefillBufs* out) {
  const size_t E = (size_t)c.n_experts;
  const int64_t max_tiles = pairs / kBM + c.n_experts;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t o_counts = take(4 * E), o_off = take(4 * (E + 2)), o_cur = take(4 * E),
               o_slot = take(4 * E), o_tiles = take(4 * (size_t)max_tiles), o_perm = take(4 * (size_t)pairs),
               o_hmid = take(2 * (size_t)pairs * c.inter), o_prow = take(4 * (size_t)pairs * c.hidden);
  if (base && out) {
    out->counts = (int32_t*)(base + o_counts);
    out->offsets = (int32_t*)(base + o_off);
    out->cursor = (int32_t*)(base + o_cur);
    out->slot_of = (int32_t*)(base + o_slot);
    out->tiles = (int32_t*)(base + o_tiles);
    out->perm = (int32_t*)(base + o_perm);
    out->hmid = (uint16_t*)(base + o_hmid);
    out->prow = (float*)(base + o_prow);
    out->max_tiles = (int32_t)max_tiles;
    out->max_pairs = pairs;
  }
  return off;
}

// Fixed device scratch for callers that cannot allocate (the no-allocation
// prefill entry point): one array per device, held until the process ends.
// Host code never uses its name as an address: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kPrefillScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_ptr[kMaxDevices] = {};

hipError_t prefill_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = (uint8_t*)p;
  return hipSuccess;
}

uint8_t* prefill_scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace moert
