// gqa_plan.cpp -- host-side serving planners of libgqa (no HIP calls): tensor-parallel head sharding
// with KV-head replication, and cache capacity.  Declared in include/gqa.h.
#include <cstdint>

#include "gqa.h"

extern "C" {

// Rank r of tp takes the r-th contiguous slice of Hq / tp query heads and holds every KV head those
// heads read under the contiguous grouping h -> h / G ("Grouped Query Attention: Why 8 KV Heads
// Decide Your Batch Size", section "What breaks when num_kv_heads is smaller than your
// tensor-parallel degree?").  A KV head whose query heads span several ranks is held by each of them.
gqa_status_t gqa_tp_plan(int32_t num_q_heads, int32_t num_kv_heads, int32_t tp_size, gqa_tp_rank_t* ranks,
                         int32_t* kv_heads_held) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || tp_size <= 0) return GQA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0 || num_q_heads % tp_size != 0) return GQA_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t per_rank = num_q_heads / tp_size;
  int32_t held = 0;
  for (int32_t r = 0; r < tp_size; ++r) {
    const int32_t q0 = r * per_rank, q1 = q0 + per_rank;
    const int32_t kv0 = q0 / group, kv1 = (q1 - 1) / group + 1;
    held += kv1 - kv0;
    if (ranks) {
      ranks[r].q_head_begin = q0;
      ranks[r].q_head_end = q1;
      ranks[r].kv_head_begin = kv0;
      ranks[r].kv_head_end = kv1;
    }
  }
  if (kv_heads_held) *kv_heads_held = held;
  return GQA_OK;
}

// free_bytes / (bytes_per_token * context_tokens), rounded down ("Grouped Query Attention: Why 8 KV
// Heads Decide Your Batch Size", section "Why does GQA decide your batch size?").  Dividing twice gives
// the same floor without forming the product, which could overflow.
uint64_t gqa_max_concurrency(uint64_t free_bytes, uint64_t bytes_per_token, uint64_t context_tokens) {
  if (bytes_per_token == 0 || context_tokens == 0) return 0;
  return free_bytes / bytes_per_token / context_tokens;
}

uint64_t gqa_max_cached_tokens(uint64_t free_bytes, uint64_t bytes_per_token) {
  return bytes_per_token == 0 ? 0 : free_bytes / bytes_per_token;
}

}  // extern "C"
