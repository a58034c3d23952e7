// The per-layer control kernel and prefill buffer admission.
//
// One kernel per MoE-layer call does all routing-dependent control on the
// device (snackonai, "The Architecture, Unpacked", third decision; satyajit,
// "Residency that follows the router"):
//   1. dedup   the flat ids u = layer*E + ids[t][j] via an E-bit mask in LDS;
//              ascending order falls out of wave ballots over the mask bits;
//   2. classify each u against id2slot (hit: resident);
//   3. q       = clamp(round_half_even(m*B_P/B_H), 1, m) in HYBRID, m in
//              OFFLOAD, 0 in CPU; then the fetch cap and the free capacity
//              (snackonai, "The split policy itself");
//   4. victims the K least recently used slots by (tick, slot), current hits
//              excluded, in one pass over the slot table: one radix select of
//              the K-th smallest tick over register-resident keys, then a
//              rank sort of the K survivors;
//   5. rewrite the first q misses take the first q victims; slot_map[t][j]
//              gets the slot, or -1 for the host; a flag says whether the
//              host branch has work (the fill kernel hands it over).
// Recency is one tick per call; hits and fills take that tick.  The 64-bit
// ticks enter the select as 32-bit keys relative to the call's tick
// (lru_key.h), exact across 2^32.
#include "internal.h"
#include "lru_key.h"

namespace moert {

constexpr int kWaves = kPlanThreads / 64;
constexpr int kSmallK = 16;  // victim counts chosen by wave minima instead of the radix select
constexpr uint32_t kSentinel = kLruNoCandidate;

struct PlanArgs {
  const int32_t* ids;
  int32_t T, k, layer, E, K, n, mode, max_fetch;
  int64_t bwp, bwh;
  int32_t* id2slot;
  int32_t* slot2id;
  int64_t* slot_ts;
  DevState* st;
  PlanBufs pb;
};

__device__ inline int64_t rne_div(int64_t a, int64_t b) {
  int64_t q = a / b, r = a - q * b;
  if (2 * r > b || (2 * r == b && (q & 1))) ++q;
  return q;
}

// Exclusive prefix of per-wave totals; returns this wave's offset and the sum.
__device__ inline int wave_offset(const int* cnt, int wave, int* total) {
  int off = 0, sum = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) off += cnt[w];
    sum += cnt[w];
  }
  *total = sum;
  return off;
}

__device__ inline int lane_rank(uint64_t m, int lane) {
  return __builtin_popcountll(m & ((1ull << lane) - 1ull));
}

// Wave minima through DPP lane moves (VALU operand modifiers, a few cycles
// each, instead of LDS-routed permutes): swaps within quads, the half-row
// and row mirrors, then the broadcasts of lane 15 into the next row and of
// lane 31 into the upper half, which leave the wave's minimum in lane 63.
// A DPP step that has no source for a lane (the broadcasts' unselected
// rows) leaves that lane's value unchanged.
template <int CTRL, int ROWS>
__device__ inline int64_t dpp_min64_step(int64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(v >> 32);
  const int tl = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
  const int th = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
  const int64_t t = (int64_t)(((uint64_t)(uint32_t)th << 32) | (uint32_t)tl);
  return min(v, t);
}
template <int CTRL, int ROWS>
__device__ inline int32_t dpp_min32_step(int32_t v) {
  return min(v, __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false));
}

// Wave minimum of a 64-bit value, returned as a wave-uniform value.
__device__ inline int64_t wave_min64(int64_t v) {
  v = dpp_min64_step<0xB1, 0xF>(v);   // quad_perm 1,0,3,2
  v = dpp_min64_step<0x4E, 0xF>(v);   // quad_perm 2,3,0,1
  v = dpp_min64_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_min64_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_min64_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_min64_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(v >> 32), 63);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave minimum of a 32-bit value, returned as a wave-uniform value.
__device__ inline int32_t wave_min32(int32_t v) {
  v = dpp_min32_step<0xB1, 0xF>(v);
  v = dpp_min32_step<0x4E, 0xF>(v);
  v = dpp_min32_step<0x141, 0xF>(v);
  v = dpp_min32_step<0x140, 0xF>(v);
  v = dpp_min32_step<0x142, 0xA>(v);
  v = dpp_min32_step<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// The thread's smallest remaining candidate tick and its index (the lowest
// index among equal ticks, so the lowest slot).
template <int SPT>
__device__ inline int64_t small_k_head(const int64_t (&ct)[SPT], int& hi) {
  int64_t m = ct[0];
  hi = 0;
#pragma unroll
  for (int i = 1; i < SPT; ++i)
    if (ct[i] < m) {
      m = ct[i];
      hi = i;
    }
  return m;
}

// Victims when K is small (at most kSmallK) and each thread holds its slots'
// ticks and occupants (sid_r) in registers: the keff least recently used
// candidate slots by (tick, slot), in that order, straight from the ticks.
// Each wave takes its keff smallest by repeated wave minima: the lowest lane
// holding the minimum has the lowest slot, since a thread's slots are
// contiguous and ascend with the thread index.  Wave 0 then merges the
// sorted lists of all waves, ties broken by slot.  Empty slots (tick -1)
// come first; hits and slots beyond the budget are no candidates.
template <int SPT>
__device__ __forceinline__ void small_k_victims(const PlanArgs& a, const int64_t (&tsr)[SPT],
                                                const int32_t* sid_r, const uint32_t* s_hitbits, int keff,
                                                int64_t (*s_wtick)[kSmallK], int32_t (*s_wslot)[kSmallK],
                                                int32_t (*s_wold)[kSmallK], int32_t* s_vic,
                                                int32_t* s_vicold) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n, s0 = tid * SPT;
  int64_t ct[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int s = s0 + i;
    ct[i] = s < n && !((s_hitbits[s >> 5] >> (s & 31)) & 1u) ? tsr[i] : INT64_MAX;
  }
  int hi;
  int64_t h = small_k_head<SPT>(ct, hi);
  for (int r = 0; r < keff; ++r) {
    const int64_t m = wave_min64(h);
    const int win = __builtin_ctzll(__ballot(h == m));
    if (lane == win) {
      s_wtick[wave][r] = m;  // INT64_MAX: the wave has no candidate left
      s_wslot[wave][r] = s0 + hi;
      s_wold[wave][r] = sid_r[hi];
      ct[hi] = INT64_MAX;
      h = small_k_head<SPT>(ct, hi);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // kWaves * keff sorted entries, up to 4 per lane
    constexpr int kPer = kWaves * kSmallK / 64;
    const int tot = kWaves * keff;
    int64_t et[kPer];
    int32_t es[kPer], eo[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int j = lane + 64 * c;
      const bool ok = j < tot;
      const int w = ok ? j / keff : 0, r = ok ? j % keff : 0;
      et[c] = ok ? s_wtick[w][r] : INT64_MAX;
      es[c] = ok && et[c] != INT64_MAX ? s_wslot[w][r] : INT32_MAX;
      eo[c] = ok ? s_wold[w][r] : -1;
    }
    for (int r = 0; r < keff; ++r) {
      // the lane's smallest entry by (tick, slot)
      int hc = 0;
      int64_t ht = et[0];
      int32_t hs = es[0];
#pragma unroll
      for (int c = 1; c < kPer; ++c) {
        if (et[c] < ht || (et[c] == ht && es[c] < hs)) {
          ht = et[c];
          hs = es[c];
          hc = c;
        }
      }
      const int64_t mt = wave_min64(ht);
      const int32_t ms = wave_min32(ht == mt ? hs : INT32_MAX);
      const int win = __builtin_ctzll(__ballot(ht == mt && hs == ms));
      if (lane == win) {
        int32_t old = -1;
#pragma unroll
        for (int c = 0; c < kPer; ++c)
          if (c == hc) {
            old = eo[c];
            et[c] = INT64_MAX;
            es[c] = INT32_MAX;
          }
        s_vic[r] = hs;
        s_vicold[r] = old;
      }
    }
  }
  __syncthreads();
}

template <int SPT>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ uint32_t s_mask[kMaxExperts / 32];
  __shared__ int32_t s_eslot[kMaxExperts];
  __shared__ int32_t s_miss[kMaxExperts];
  __shared__ int32_t s_vic[kMaxExperts];
  __shared__ int32_t s_vicold[kMaxExperts];  // occupant of each victim slot
  __shared__ int32_t s_selold[kMaxExperts];
  __shared__ uint32_t s_hitbits[kMaxSlots / 32];
  __shared__ uint32_t s_hist[2048];
  __shared__ int32_t s_cnt[3][kWaves];
  __shared__ int32_t s_scan[kPlanThreads];
  __shared__ int32_t s_scan2[kPlanThreads];
  __shared__ uint64_t s_sel[kMaxExperts];
  __shared__ int32_t s_nuniq, s_nhit, s_m, s_q, s_keff, s_evict, s_ngpu, s_bad;
  __shared__ uint32_t s_prefix, s_pmask, s_kk;
  __shared__ int64_t s_tmin[kWaves], s_tmax[kWaves];
  __shared__ bool s_wempty[kWaves];
  __shared__ int64_t s_wtick[kWaves][kSmallK];  // small K: each wave's oldest candidates
  __shared__ int32_t s_wslot[kWaves][kSmallK];
  __shared__ int32_t s_wold[kWaves][kSmallK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, Tk = a.T * a.k, n = a.n;
  const PlanBufs& pb = a.pb;

  // -------------------------------------------------------------- init
  if (tid < kMaxExperts / 32) s_mask[tid] = 0;
  for (int i = tid; i < (n + 31) / 32; i += kPlanThreads) s_hitbits[i] = 0;
  if (tid < E) s_eslot[tid] = -1;
  if (tid == 0) {
    s_evict = 0;
    s_bad = 0;
  }
  // the slot table rows of this thread's slots, requested now so their
  // latency overlaps the dedup and classification (up to 8 slots per
  // thread; beyond, the ticks are read when the victims are chosen and a
  // victim's occupant when it is selected, to spare registers)
  constexpr bool kHold = SPT <= 8;
  const int64_t now = a.st->tick + 1;
  const int64_t h_epoch = a.st->h_epoch;
  int64_t tsr[SPT];
  int32_t sid_r[kHold ? SPT : 1];
  if constexpr (kHold) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int s = tid * SPT + i;
      tsr[i] = s < n ? a.slot_ts[s] : -1;
      sid_r[i] = s < n ? a.slot2id[s] : -1;
    }
  }
  // the first routed id of this thread and the residency of expert tid of
  // this layer are requested here too, so neither costs a round trip after
  // the barrier (nothing in this kernel writes id2slot before classifying)
  const int id0 = tid < Tk ? a.ids[tid] : 0;
  const int slot_pre = tid < E ? a.id2slot[a.layer * E + tid] : -1;
  __syncthreads();
  const int64_t tick = now;

  // -------------------------------------------------------------- 1. dedup
  for (int i = tid; i < Tk; i += kPlanThreads) {
    int e = i == tid ? id0 : a.ids[i];
    if (e >= 0 && e < E) atomicOr(&s_mask[e >> 5], 1u << (e & 31));
    else atomicAdd(&s_bad, 1);  // out-of-range ids: zero rows from the host branch
  }
  __syncthreads();

  // -------------------------------------------------------------- 2. classify
  const int e = tid;
  const bool present = e < E && ((s_mask[e >> 5] >> (e & 31)) & 1u);
  const int u = a.layer * E + e;
  const int slot = present ? slot_pre : -1;
  const bool hit = present && slot >= 0;
  const bool miss = present && slot < 0;
  const uint64_t b_pres = __ballot(present), b_hit = __ballot(hit), b_miss = __ballot(miss);
  if (lane == 0) {
    s_cnt[0][wave] = __builtin_popcountll(b_pres);
    s_cnt[1][wave] = __builtin_popcountll(b_hit);
    s_cnt[2][wave] = __builtin_popcountll(b_miss);
  }
  __syncthreads();
  int n_uniq, n_hit, m;
  const int o_pres = wave_offset(s_cnt[0], wave, &n_uniq);
  const int o_hit = wave_offset(s_cnt[1], wave, &n_hit);
  const int o_miss = wave_offset(s_cnt[2], wave, &m);
  if (present) pb.uniq[o_pres + lane_rank(b_pres, lane)] = u;
  if (hit) {
    pb.hits[o_hit + lane_rank(b_hit, lane)] = u;
    atomicOr(&s_hitbits[slot >> 5], 1u << (slot & 31));
    s_eslot[e] = slot;
    a.slot_ts[slot] = tick;  // a hit refreshes recency
  }
  if (miss) {
    int p = o_miss + lane_rank(b_miss, lane);
    s_miss[p] = u;
    pb.misses[p] = u;
  }

  // -------------------------------------------------------------- 3. q
  if (tid == 0) {
    int q;
    if (m == 0 || a.mode == MOE_CPU) q = 0;
    else if (a.mode == MOE_OFFLOAD) q = m;
    else {
      int64_t r = rne_div((int64_t)m * a.bwp, a.bwh);
      q = (int)min<int64_t>(max<int64_t>(1, r), m);
    }
    if (a.max_fetch > 0) q = min(q, a.max_fetch);
    q = min(q, n - n_hit);
    s_nuniq = n_uniq;
    s_nhit = n_hit;
    s_m = m;
    s_q = q;
    s_keff = min(a.K, n - n_hit);
  }
  __syncthreads();
  const int keff = s_keff;

  // -------------------------------------------------------------- 4. victims
  if (keff > 0) {
    // candidates: this thread's contiguous slots below n that hold no
    // current hit.  The occupied candidates' tick range (64-bit) and whether
    // any candidate is empty, over the block
    const int s0 = tid * SPT;
    if constexpr (!kHold) {
      // only current hits' ticks changed since entry, and hits are no candidates
#pragma unroll
      for (int i = 0; i < SPT; ++i) tsr[i] = s0 + i < n ? a.slot_ts[s0 + i] : -1;
    }
    // small K with the slot table held in registers (pools up to 8 slots
    // per thread): wave minima; otherwise the radix select
    if (kHold && keff <= kSmallK) {  // uniform
      if constexpr (kHold)
        small_k_victims<SPT>(a, tsr, sid_r, s_hitbits, keff, s_wtick, s_wslot, s_wold, s_vic, s_vicold);
    } else {
    int64_t tmin = INT64_MAX, tmax = -1;
    bool empty = false;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int s = s0 + i;
      if (s < n && !((s_hitbits[s >> 5] >> (s & 31)) & 1u)) {
        if (tsr[i] < 0) {
          empty = true;
        } else {
          tmin = min(tmin, tsr[i]);
          tmax = max(tmax, tsr[i]);
        }
      } else {
        tsr[i] = INT64_MIN;  // not a candidate
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      tmin = min(tmin, (int64_t)__shfl_xor((long long)tmin, off));
      tmax = max(tmax, (int64_t)__shfl_xor((long long)tmax, off));
    }
    const bool w_empty = __ballot(empty) != 0;
    if (lane == 0) {
      s_tmin[wave] = tmin;
      s_tmax[wave] = tmax;
      s_wempty[wave] = w_empty;
    }
    __syncthreads();
    tmin = INT64_MAX;
    tmax = -1;
    empty = false;
    for (int w = 0; w < kWaves; ++w) {
      tmin = min(tmin, s_tmin[w]);
      tmax = max(tmax, s_tmax[w]);
      empty |= s_wempty[w];
    }
    // 32-bit keys relative to the oldest occupied candidate (lru_key.h),
    // shifted so the smallest candidate key is 0: the select then only needs
    // the digits that the candidates' age range actually uses
    const uint32_t kmin = empty ? 0u : 1u;
    const uint32_t kmax = tmax >= 0 ? lru_key(tmax, tmin) : 0u;
    uint32_t key[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      key[i] = tsr[i] == INT64_MIN ? kSentinel : lru_key(tsr[i], tmin) - kmin;
    const uint32_t spread = kmax >= kmin ? kmax - kmin : 0;
    const int bits = spread ? 32 - __builtin_clz(spread) : 0;
    const int first_pass = bits > 21 ? 0 : bits > 10 ? 1 : 2;
    const int n_cand = n - s_nhit;
    uint32_t tau = kSentinel;  // keys < tau are all taken
    if (keff < n_cand) {
      // radix select of the keff-th smallest key: 11 + 11 + 10 bits, leading
      // passes whose digit is zero for every candidate skipped
      if (tid == 0) {
        s_prefix = 0;
        s_pmask = first_pass == 0 ? 0u : first_pass == 1 ? 0xFFE00000u : 0xFFFFFC00u;
        s_kk = (uint32_t)keff;
      }
      const int shifts[3] = {21, 10, 0};
      const uint32_t dmask[3] = {0x7FFu, 0x7FFu, 0x3FFu};
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        if (pass < first_pass) continue;  // uniform
        for (int i = tid; i < 2048; i += kPlanThreads) s_hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = s_prefix, pmask = s_pmask;
#pragma unroll
        for (int i = 0; i < SPT; ++i)
          if (key[i] != kSentinel && (key[i] & pmask) == prefix)
            atomicAdd(&s_hist[(key[i] >> shifts[pass]) & dmask[pass]], 1u);
        __syncthreads();
        // block scan over 2048 bins, two per thread
        int c0 = s_hist[2 * tid], c1 = s_hist[2 * tid + 1];
        int v = c0 + c1;
        // inclusive scan of v across the block
        int x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          int y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        if (lane == 63) s_scan[wave] = x;
        __syncthreads();
        int wbase = 0;
        for (int w = 0; w < wave; ++w) wbase += s_scan[w];
        const int incl = wbase + x, excl = incl - v;
        const uint32_t kk = s_kk;
        __syncthreads();
        if ((uint32_t)excl < kk && kk <= (uint32_t)incl) {
          int bin;
          uint32_t before;
          if (kk <= (uint32_t)(excl + c0)) {
            bin = 2 * tid;
            before = excl;
          } else {
            bin = 2 * tid + 1;
            before = excl + c0;
          }
          s_prefix = prefix | ((uint32_t)bin << shifts[pass]);
          s_pmask = pmask | (dmask[pass] << shifts[pass]);
          s_kk = kk - before;
        }
        __syncthreads();
      }
      tau = s_prefix;  // the keff-th smallest key
    }
    // take every key < tau, then the lowest slots with key == tau
    int lt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      lt += key[i] < tau;
      eq += key[i] == tau && key[i] != kSentinel;
    }
    // block exclusive scans of lt and eq in thread (= slot) order
    int xl = lt, xe = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int yl = __shfl_up(xl, off), ye = __shfl_up(xe, off);
      if (lane >= off) {
        xl += yl;
        xe += ye;
      }
    }
    if (lane == 63) {
      s_scan[wave] = xl;
      s_scan2[wave] = xe;
    }
    __syncthreads();
    int bl = 0, be = 0, tl = 0;
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) {
        bl += s_scan[w];
        be += s_scan2[w];
      }
      tl += s_scan[w];
    }
    int pl = bl + xl - lt;        // exclusive position among keys < tau
    int pe = be + xe - eq;        // exclusive position among keys == tau
    const int r = keff - tl;      // keys == tau to take
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const uint32_t kv = key[i];
      const uint64_t packed = ((uint64_t)kv << 32) | (uint32_t)(s0 + i);
      if (kv < tau) {
        s_selold[pl] = kHold ? sid_r[kHold ? i : 0] : a.slot2id[s0 + i];
        s_sel[pl++] = packed;
      } else if (kv == tau && kv != kSentinel) {
        if (pe < r) {
          s_selold[tl + pe] = kHold ? sid_r[kHold ? i : 0] : a.slot2id[s0 + i];
          s_sel[tl + pe] = packed;
        }
        ++pe;
      }
    }
    __syncthreads();
    // rank sort of the keff survivors by (tick, slot)
    if (tid < keff) {
      const uint64_t mine = s_sel[tid];
      int rank = 0;
      for (int j = 0; j < keff; ++j) rank += s_sel[j] < mine;
      s_vic[rank] = (int32_t)(mine & 0xFFFFFFFFu);
      s_vicold[rank] = s_selold[tid];
    }
    __syncthreads();
    }
  }
  if (tid < a.K) pb.victims[tid] = tid < keff ? s_vic[tid] : -1;

  // -------------------------------------------------------------- 5. rewrite
  const int q = s_q;
  if (tid < q) {
    const int uu = s_miss[tid];
    const int s = s_vic[tid];
    const int old = s_vicold[tid];
    if (old >= 0) {
      a.id2slot[old] = -1;
      atomicAdd(&s_evict, 1);
    }
    a.slot2id[s] = uu;
    a.id2slot[uu] = s;
    a.slot_ts[s] = tick;
    s_eslot[uu - a.layer * E] = s;
    pb.fill_u[tid] = uu;
    pb.fill_slot[tid] = s;
    pb.fill_old[tid] = old;
  }
  const int mm = s_m;
  for (int i = q + tid; i < mm; i += kPlanThreads) pb.cpu_u[i - q] = s_miss[i];
  __syncthreads();

  // slot map and GPU list (ascending u).  The host block (ids, slot map,
  // activations) and the doorbell are written by the fill kernel's hand-off
  // workgroup that follows on the stream, so this kernel makes no
  // host-memory writes and no system-scope fences.
  for (int i = tid; i < Tk; i += kPlanThreads) {
    int ee = a.ids[i];
    pb.slot_map[i] = (ee >= 0 && ee < E) ? s_eslot[ee] : -1;
  }
  const bool on_gpu = present && s_eslot[e] >= 0;
  const uint64_t b_gpu = __ballot(on_gpu);
  if (lane == 0) s_cnt[0][wave] = __builtin_popcountll(b_gpu);
  __syncthreads();
  int n_gpu;
  const int o_gpu = wave_offset(s_cnt[0], wave, &n_gpu);
  if (on_gpu) {
    int p = o_gpu + lane_rank(b_gpu, lane);
    pb.gpu_u[p] = u;
    pb.gpu_slot[p] = s_eslot[e];
  }
  // first call of a new tick epoch: every intermediate entry gets a mark no
  // tick of this epoch has (the mark of this tick with the top bit flipped;
  // the epoch spans 2^30 ticks), so no entry left from an earlier call
  // passes for one of a later call of the epoch
  const bool new_epoch = (tick >> kHMarkEpochBits) != h_epoch;
  if (new_epoch) {
    const uint64_t stale = (uint64_t)((uint32_t)tick ^ 0x80000000u) << 32;
    for (int64_t i = tid; i < pb.h_words; i += kPlanThreads) pb.h_marked[i] = stale;
  }
  if (tid == 0) {
    moe_plan_counts c;
    c.n_uniq = s_nuniq;
    c.n_hit = s_nhit;
    c.n_miss = mm;
    c.q = q;
    c.n_cpu = mm - q;
    c.n_gpu = n_gpu;
    c.K = a.K;
    c.tick_lo = (int32_t)tick;
    *pb.counts = c;
    // the host branch has work: misses left to the CPU, or ids outside
    // [0, E) (their rows are zeros from the host branch)
    *pb.host_work = (mm - q > 0 || s_bad > 0) ? 1 : 0;
    // the call's sequence number is the plan count after it: it lives on the
    // device, so a replayed graph of calls numbers its calls correctly
    DevState* st = a.st;
    const int64_t seq = st->plans + 1;
    st->tick = tick;
    st->plans = seq;
    st->hits += s_nhit;
    st->fills += q;
    st->cpu += mm - q;
    st->evictions += s_evict;
    if (new_epoch) st->h_epoch = tick >> kHMarkEpochBits;
  }
}

hipError_t launch_plan(moe_ctx* ctx, int layer, const int32_t* ids, int T, const void* x,
                       hipStream_t s) {
  PlanArgs a;
  (void)x;
  a.ids = ids;
  a.T = T;
  a.k = ctx->cfg.top_k;
  a.layer = layer;
  a.E = ctx->cfg.n_experts;
  a.n = ctx->n_slots;
  int64_t K = std::min<int64_t>((int64_t)ctx->cfg.max_tokens * ctx->cfg.top_k, ctx->cfg.n_experts);
  K = std::min<int64_t>(K, a.n);
  if (ctx->cfg.max_fetch > 0) K = std::min<int64_t>(K, ctx->cfg.max_fetch);
  a.K = (int32_t)K;
  a.mode = (!ctx->cpu_layers.empty() && ctx->cpu_layers[layer]) ? MOE_CPU : ctx->cfg.mode;
  a.max_fetch = ctx->cfg.max_fetch;
  a.bwp = ctx->cfg.bw_pcie_mbps;
  a.bwh = ctx->cfg.bw_host_mbps;
  a.id2slot = ctx->id2slot;
  a.slot2id = ctx->slot2id;
  a.slot_ts = ctx->slot_ts;
  a.st = ctx->dstate;
  a.pb = ctx->plan;
  dim3 g(1), b(kPlanThreads);
  const int n = a.n;
  if (n <= kPlanThreads * 1) hipLaunchKernelGGL(plan_kernel<1>, g, b, 0, s, a);
  else if (n <= kPlanThreads * 2) hipLaunchKernelGGL(plan_kernel<2>, g, b, 0, s, a);
  else if (n <= kPlanThreads * 4) hipLaunchKernelGGL(plan_kernel<4>, g, b, 0, s, a);
  else if (n <= kPlanThreads * 8) hipLaunchKernelGGL(plan_kernel<8>, g, b, 0, s, a);
  else if (n <= kPlanThreads * 16) hipLaunchKernelGGL(plan_kernel<16>, g, b, 0, s, a);
  else hipLaunchKernelGGL(plan_kernel<32>, g, b, 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- prefill admission
// Buffer b (layer % 2 with two buffers, 0 with one) is slots [b*E, (b+1)*E);
// expert e of the layer sits in
// slot b*E + e with one tick for the layer.  The buffer's previous occupants
// are evicted and any other slot still holding an expert of this layer is
// emptied (satyajit, "Prefill: hide the pool behind the wire").
__global__ __launch_bounds__(kMaxExperts) void prefill_admit_kernel(int layer, int b, int E, int32_t* id2slot,
                                                                    int32_t* slot2id, int64_t* slot_ts,
                                                                    DevState* st) {
  __shared__ int64_t s_tick;
  const int e = threadIdx.x;
  if (e == 0) s_tick = st->tick + 1;
  // other slots holding this layer's experts (outside the buffer) are emptied
  if (e < E) {
    const int u = layer * E + e;
    const int s = id2slot[u];
    if (s >= 0 && (s < b * E || s >= (b + 1) * E)) {
      slot2id[s] = -1;
      slot_ts[s] = -1;
    }
  }
  __syncthreads();
  // evict the buffer's occupants
  if (e < E) {
    const int s = b * E + e;
    const int old = slot2id[s];
    if (old >= 0) id2slot[old] = -1;
  }
  __syncthreads();
  if (e < E) {
    const int s = b * E + e, u = layer * E + e;
    slot2id[s] = u;
    id2slot[u] = s;
    slot_ts[s] = s_tick;
  }
  if (e == 0) {
    st->tick = s_tick;
    st->prefill_layers += 1;
  }
}

// One pass of on-demand prefill (the pool cannot hold the full-layer
// buffers): the experts of `layer` with routed pairs (counts > 0), ranked in
// ascending expert order; ranks [p0, p0 + P) form this pass and go to slots
// [0, P) in rank order, with one tick.  The slots' occupants are evicted and
// a pass expert resident elsewhere is emptied there.  slot_of[e] receives the
// slot of each expert in the pass and -1 for every other expert.
__global__ __launch_bounds__(kMaxExperts) void prefill_pass_admit_kernel(int layer, int E, int p0, int P,
                                                                         const int32_t* counts,
                                                                         int32_t* slot_of, int32_t* id2slot,
                                                                         int32_t* slot2id, int64_t* slot_ts,
                                                                         DevState* st) {
  __shared__ int32_t s_scan[kMaxExperts];
  __shared__ int64_t s_tick;
  const int e = threadIdx.x;
  const int f = (e < E && counts[e] > 0) ? 1 : 0;
  s_scan[e] = f;
  __syncthreads();
  for (int off = 1; off < kMaxExperts; off <<= 1) {  // inclusive scan of the flags
    const int v = e >= off ? s_scan[e - off] : 0;
    __syncthreads();
    s_scan[e] += v;
    __syncthreads();
  }
  const int rank = s_scan[e] - f;
  const int slot = (f && rank >= p0 && rank < p0 + P) ? rank - p0 : -1;
  if (e < E) slot_of[e] = slot;
  if (e == 0) s_tick = st->tick + 1;
  if (e < P) {  // evict the occupants of slots [0, P)
    const int old = slot2id[e];
    if (old >= 0) id2slot[old] = -1;
  }
  __syncthreads();
  if (slot >= 0) {  // a pass expert still resident elsewhere is emptied there
    const int u = layer * E + e;
    const int s = id2slot[u];
    if (s >= 0) {
      slot2id[s] = -1;
      slot_ts[s] = -1;
      id2slot[u] = -1;
    }
  }
  __syncthreads();
  if (slot >= 0) {
    const int u = layer * E + e;
    slot2id[slot] = u;
    id2slot[u] = slot;
    slot_ts[slot] = s_tick;
  }
  if (e == 0) {
    st->tick = s_tick;
    st->prefill_layers += 1;
  }
}

hipError_t launch_prefill_pass_admit(moe_ctx* ctx, const PrefillBufs& pb, int layer, int p0, int P,
                                     hipStream_t s) {
  hipLaunchKernelGGL(prefill_pass_admit_kernel, dim3(1), dim3(kMaxExperts), 0, s, layer,
                     ctx->cfg.n_experts, p0, P, pb.counts, pb.slot_of, ctx->id2slot,
                     ctx->slot2id, ctx->slot_ts, ctx->dstate);
  return hipGetLastError();
}

hipError_t launch_prefill_admit(moe_ctx* ctx, int layer, int b, hipStream_t s) {
  hipLaunchKernelGGL(prefill_admit_kernel, dim3(1), dim3(kMaxExperts), 0, s, layer, b,
                     ctx->cfg.n_experts, ctx->id2slot, ctx->slot2id, ctx->slot_ts, ctx->dstate);
  return hipGetLastError();
}

}  // namespace moert
