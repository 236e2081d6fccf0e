// Exercises the host planners of libgqa (gqa_plan.cpp) over a grid of head counts and tensor-parallel
// degrees, with rank arrays of exactly tp_size entries, and the capacity planners on extreme 64-bit
// inputs, for an AddressSanitizer / UndefinedBehaviorSanitizer build.  Exit status 0 = all consistent.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "gqa.h"

int main() {
  int failures = 0;
  for (int32_t hkv = 1; hkv <= 16; ++hkv)
    for (int32_t g = 1; g <= 8; ++g)
      for (int32_t tp = 1; tp <= 16; ++tp) {
        const int32_t hq = hkv * g;
        std::vector<gqa_tp_rank_t> ranks(tp);
        int32_t held = -1;
        const gqa_status_t st = gqa_tp_plan(hq, hkv, tp, ranks.data(), &held);
        if ((hq % tp == 0) != (st == GQA_OK)) ++failures;
        if (st != GQA_OK) continue;
        int32_t sum = 0;
        for (int32_t r = 0; r < tp; ++r) {
          const gqa_tp_rank_t& k = ranks[r];
          if (k.q_head_end - k.q_head_begin != hq / tp) ++failures;
          if (k.kv_head_begin < 0 || k.kv_head_end > hkv || k.kv_head_begin >= k.kv_head_end) ++failures;
          sum += k.kv_head_end - k.kv_head_begin;
        }
        if (sum != held) ++failures;
      }
  if (gqa_tp_plan(0, 1, 1, nullptr, nullptr) == GQA_OK) ++failures;
  if (gqa_tp_plan(8, 3, 2, nullptr, nullptr) == GQA_OK) ++failures;
  const uint64_t big = ~(uint64_t)0;
  const uint64_t vals[] = {0, 1, 2, 3, 327680, (uint64_t)1 << 32, big - 1, big};
  for (uint64_t a : vals)
    for (uint64_t b : vals) {
      (void)gqa_max_cached_tokens(a, b);
      for (uint64_t c : vals) {
        const uint64_t n = gqa_max_concurrency(a, b, c);
        if ((b == 0 || c == 0) && n != 0) ++failures;
      }
    }
  if (gqa_max_concurrency(big, 2, 3) != big / 6) ++failures;
  if (failures) std::fprintf(stderr, "%d planner check(s) failed\n", failures);
  else std::printf("planner driver: all calls behaved\n");
  return failures ? 1 : 0;
}
