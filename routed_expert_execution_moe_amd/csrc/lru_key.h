// 32-bit recency keys for the control kernel's victim selection.
//
// The LRU order is ascending (tick, slot) with empty slots (tick -1) first
// (satyajit, "Residency that follows the router": the K least recently used
// slots are surfaced in one pass).  Ticks are 64-bit and grow by one per
// layer call; the kernel's radix select works on 32-bit keys, so each
// candidate's tick is mapped into 32 bits relative to the oldest occupied
// candidate's tick `tmin` (a block-wide minimum the kernel takes first):
//
//   empty slot (tick < 0)              -> 0
//   tick - tmin <  0xFFFFFFFD          -> 1 + (tick - tmin)
//   tick - tmin >= 0xFFFFFFFD          -> 0xFFFFFFFE
//
// The map preserves the order of ticks exactly while the occupied candidates'
// ticks span fewer than 2^32 - 3 calls, whatever their absolute values (it
// crosses 2^32 unchanged), and empty slots always come first.  Beyond that
// span only the newest candidates share the largest key (they are the last
// victims, ordered among themselves by slot index).  The keys' spread is the
// candidates' age range, so the select skips every digit that range leaves
// zero.  0xFFFFFFFF is left for non-candidates (current hits, slots past the
// budget).
//
// constexpr, so the same function compiles for the device (HIP) and on the
// host (its CPU unit test).
#pragma once

#include <stdint.h>

namespace moert {

constexpr uint32_t kLruNoCandidate = 0xFFFFFFFFu;
constexpr int64_t kLruSpan = 0xFFFFFFFD;

constexpr uint32_t lru_key(int64_t tick, int64_t tmin) {
  return tick < 0 ? 0u : tick - tmin >= kLruSpan ? 0xFFFFFFFEu : (uint32_t)(1 + (tick - tmin));
}

}  // namespace moert
