// gqa_append.h -- HIP kernel (gfx950) that writes the new token's K and V rows into the cache.
#pragma once

#include "gqa_device.h"

namespace gqa {

// ------------------------------------------------------------------------------------------------
// Cache append: the new token's K and V rows, converted to the cache's storage format, written at
// one position per sequence ("Grouped-Query Attention: How Sharing KV Heads Shrinks Inference
// Memory", section "FP8 KV cache: the other factor of two", for the fp8 format with per-tensor
// scales).

struct AppendParams {
  const void* k_new;  // [B][Hkv][D], f32 or bf16
  const void* v_new;
  void* k_cache;      // dense [B][Hkv][L][D] or pages [num_blocks][Hkv][block_size][D]
  void* v_cache;
  const int32_t* positions;  // [B]; negative: not written
  int32_t* skipped;          // optional: counts positions past the cache or on a page outside the pool
  int B, Hkv, L;
  float k_descale, v_descale;
  const int32_t* block_table;  // paged cache only
  int block_shift, max_blocks, num_blocks;
};

template <typename InT>
__device__ __forceinline__ float load_new(const void* p, size_t i);
template <>
__device__ __forceinline__ float load_new<float>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_new<uint16_t>(const void* p, size_t i) {
  return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
}

// One workgroup per sequence; each thread converts and stores 4 consecutive elements of a row.
// KV: 0 f32, 1 bf16, 2 fp8-e4m3 (cache storage).
template <int D, typename InT, int KV, bool PAGED>
__global__ void __launch_bounds__(256) append_kv_kernel(AppendParams p) {
  const int b = blockIdx.x;
  const int t = p.positions[b];
  if (t < 0) return;
  size_t row0;  // element index of row (b, j = 0, t)
  size_t head_stride;  // elements between rows of consecutive KV heads
  bool ok = t < p.L;
  if constexpr (PAGED) {
    const int page = ok ? p.block_table[(size_t)b * p.max_blocks + (t >> p.block_shift)] : -1;
    ok = ok && (uint32_t)page < (uint32_t)p.num_blocks;
    row0 = (((size_t)(ok ? page : 0) * p.Hkv) << p.block_shift | (size_t)(t & ((1 << p.block_shift) - 1))) * D;
    head_stride = ((size_t)1 << p.block_shift) * D;
  } else {
    row0 = ((size_t)b * p.Hkv * p.L + (size_t)t) * D;
    head_stride = (size_t)p.L * D;
  }
  if (!ok) {
    if (threadIdx.x == 0 && p.skipped) atomicAdd(p.skipped, 1);
    return;
  }
  const int n4 = p.Hkv * D / 4;
  for (int i = threadIdx.x; i < 2 * n4; i += blockDim.x) {
    const bool isv = i >= n4;
    const int e = 4 * (isv ? i - n4 : i);  // element within the sequence's Hkv x D new rows
    const int j = e / D, c = e % D;
    const void* src = isv ? p.v_new : p.k_new;
    void* dst = isv ? p.v_cache : p.k_cache;
    const size_t si = (size_t)b * p.Hkv * D + e;
    const size_t di = row0 + (size_t)j * head_stride + c;
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = load_new<InT>(src, si + u);
    if constexpr (KV == 0) {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(dst) + di) = f32x4_t{x[0], x[1], x[2], x[3]};
    } else if constexpr (KV == 1) {
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(dst) + di) =
          u32x2_t{float_to_bf16_bits(x[0]) | (float_to_bf16_bits(x[1]) << 16),
                  float_to_bf16_bits(x[2]) | (float_to_bf16_bits(x[3]) << 16)};
    } else {
      const float ds = isv ? p.v_descale : p.k_descale;
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) w |= float_to_fp8_e4m3_bits(x[u], ds) << (8 * u);
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(dst) + di) = w;
    }
  }
}

}  // namespace gqa
