// Prints the control kernel's 32-bit recency key (lru_key.h, the same header
// the kernel compiles) for (tick, tmin) pairs read from stdin, one per line.
#include <cstdio>

#include "../../routed_expert_execution_moe_amd/csrc/lru_key.h"

int main() {
  long long tick, tmin;
  while (std::scanf("%lld %lld", &tick, &tmin) == 2)
    std::printf("%u\n", moert::lru_key((int64_t)tick, (int64_t)tmin));
  return 0;
}
