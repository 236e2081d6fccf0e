// gqa_host.h -- small host-side helpers shared by the entry-point sources of libgqa.
#pragma once

#include <cstddef>
#include <cstdint>

#include "gqa.h"

namespace gqa_host {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline bool known_dtype(int dt) { return dt == GQA_F32 || dt == GQA_BF16 || dt == GQA_FP8_E4M3; }

// k with 2^k == x, or -1 when x is not a power of two
inline int log2_exact(int x) {
  int k = 0;
  while (k < 30 && (1 << k) < x) ++k;
  return (1 << k) == x ? k : -1;
}

}  // namespace gqa_host
