// 32-bit recency keys for the control kernel's victim selection.
//
// The LRU order is ascending (tick, slot) with empty slots (tick -1) first
// (satyajit, "Residency that follows the router": the K least recently used
// slots are surfaced in one pass).  Ticks are 64-bit and grow by one per
// layer call; the kernel's radix select works on 32-bit keys, so each
// candidate's tick is mapped into 32 bits relative to the call's own tick:
//
//   empty slot (tick < 0)                      -> 0
//   tick <= now - 0xFFFFFFFE                   -> 1 (older than 2^32 - 2 calls)
//   otherwise                                  -> tick - (now - 0xFFFFFFFE) + 1,
//                                                 in 2 .. 0xFFFFFFFE for tick < now
//
// `now` is the tick the current call takes; every candidate has tick < now.
// The map preserves the order of ticks exactly for every slot touched within
// the last 2^32 - 3 calls, whatever the absolute tick (it crosses 2^32
// unchanged), and empty slots always come first.  Slots untouched for longer
// share key 1 and are ordered among themselves by slot index.  0xFFFFFFFF is
// left for non-candidates (current hits, slots past the budget).
//
// constexpr, so the same function compiles for the device (HIP) and on the
// host (its CPU unit test).
#pragma once

#include <stdint.h>

namespace moert {

constexpr uint32_t kLruNoCandidate = 0xFFFFFFFFu;

constexpr uint32_t lru_key(int64_t tick, int64_t now) {
  return tick < 0 ? 0u
         : tick <= now - (int64_t)0xFFFFFFFE ? 1u
         : (uint32_t)(tick - (now - (int64_t)0xFFFFFFFE) + 1);
}

}  // namespace moert
