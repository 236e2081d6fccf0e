// gqa_kernels.h -- HIP kernels (gfx950 / CDNA4) for single-token grouped-query-attention decode.
//
// Work decomposition (split-K over the cached sequence, one launch):
//   one workgroup per (batch b, KV head j, chunk c of `chunk` cache positions).  Each of its NW waves
//   walks its own tiles of the chunk, keeping the G query rows of group j resident while the K/V tile
//   of head j streams past them once: the tile is read from HBM a single time and serves all G query
//   heads ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch Size", section "Why does GQA
//   speed up decode, not just save memory?").  Softmax is computed online (running max and running
//   sum per query row), the NW wave states are merged in LDS, and the chunk's (max, sum, unnormalised
//   output) is written to the workspace.  The last workgroup of (b, j) to finish -- found with one
//   atomic counter per (b, j) -- merges the chunk partials in chunk order and writes out[b, jG:jG+G].
//   A sequence that fits one chunk writes its output directly.
//
// The arithmetic is scaled dot-product attention per query head with KV head floor(h / G)
// ("Grouped Query Attention (GQA): Efficient Multi-Head Attention", Worked example 2;
// "Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory", section "How
// grouped-query attention works").  Scores are kept in the base-2 domain (scale * log2 e folded into
// one multiplier) so that exp2 is a single v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define GQA_LDS __attribute__((address_space(3)))

// Raw-buffer descriptor word 3 for gfx950 (32-bit data format, no swizzle, range checked).
constexpr int kBufferFlags = 0x00020000;
// Cache policy on the streaming loads: non-temporal (the cache is read once per step).
constexpr int kStreamPolicy = 2;
// Byte offset used for loads of tiles that do not exist: beyond every descriptor's range, so the
// load returns zeros without touching memory.
constexpr uint32_t kNoTile = 0x80000000u;

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  void* out;
  float* part_o;       // [B*Hkv][nchunks][G][D] unnormalised chunk outputs
  float* part_ml;      // [B*Hkv][nchunks][G][2] chunk (max, sum), base-2 domain
  uint32_t* counters;  // [B*Hkv] finished-chunk counters, zero between calls
  int B, Hq, Hkv, L, G;
  int chunk;    // cache positions per chunk
  int nchunks;  // ceil(L / chunk)
  float qk_scale;   // scale * k_descale * log2(e)
  float v_descale;  // applied to the normalised output
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((u >> 16) & 0x8000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp8-e4m3fn codes (the low or high 16 bits of `w`) -> two bf16 in one dword.  Exact: every
// e4m3fn value is representable in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ float wave_max_xor_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) {
  *p = (uint16_t)float_to_bf16_bits(x);
}

// ------------------------------------------------------------------------------------------------
// Shared epilogue.  The NW waves have left, in LDS:
//   ep_m[w][g], ep_l[w][g]   running max (base 2) and running sum of wave w for query row g
//   ep_o[w][g][c]            unnormalised output of wave w (row stride D + 4 floats)
// Waves that saw no token hold (-inf, 0, 0).  Rows g < G are valid.
template <int GT, int D, int NW>
struct EpiLayout {
  static constexpr int kRow = D + 4;
  static constexpr int kBytes = NW * GT * (2 + kRow) * 4;
};

// The last workgroup of a (b, j) stages every chunk's (max, sum) in LDS; the host keeps
// nchunks * G within this many pairs.
constexpr int kCombinePairs = 2048;
constexpr int kCombineBytes = kCombinePairs * 8 + 32 * 4;

// Workspace traffic between workgroups uses agent-scope cache policy (sc1): the bits the compiler
// gives agent-scope atomic loads and stores, which keep them coherent across the per-XCD L2
// caches without a whole-cache write-back or invalidate.
constexpr int kAgentScope = 16;

__device__ __forceinline__ void store4_agent(float* base, uint32_t bytes, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), make_rsrc(base, bytes), off, 0, kAgentScope);
}

template <int GT, int D, int NW, typename OutT>
__device__ void epilogue(const Params& p, float* ep, int b, int j, int c, int nlive) {
  constexpr int NTH = NW * 64;
  constexpr int kRow = EpiLayout<GT, D, NW>::kRow;
  const int tid = threadIdx.x;
  const int G = p.G;
  const int bj = b * p.Hkv + j;
  const float* ep_m = ep;
  const float* ep_l = ep + NW * GT;
  const float* ep_o = ep + 2 * NW * GT;
  OutT* out = reinterpret_cast<OutT*>(p.out) + ((size_t)b * p.Hq + (size_t)j * G) * D;

  // merge of the NW wave states for 4 consecutive columns of one query row
  auto merge4 = [&](int item, float& M, float& l, f32x4_t& o) {
    const int g = (4 * item) / D, cc = (4 * item) % D;
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, ep_m[w * GT + g]);
    l = 0.f;
    o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float s = __builtin_amdgcn_exp2f(ep_m[w * GT + g] - M);
      l += s * ep_l[w * GT + g];
      o += s * *reinterpret_cast<const f32x4_t*>(ep_o + (w * GT + g) * kRow + cc);
    }
  };

  if (nlive == 1) {  // the whole sequence was in this chunk: normalise and store
    for (int item = tid; item < G * D / 4; item += NTH) {
      float M, l;
      f32x4_t o;
      merge4(item, M, l, o);
      const float inv = p.v_descale / l;
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(out + 4 * item + e, o[e] * inv);
    }
    return;
  }

  // Several chunks: publish this chunk's partial result with agent-scope stores.
  float* po = p.part_o + ((size_t)bj * p.nchunks + c) * G * D;
  float* pml = p.part_ml + ((size_t)bj * p.nchunks + c) * G * 2;
  for (int item = tid; item < G * D / 4; item += NTH) {
    float M, l;
    f32x4_t o;
    merge4(item, M, l, o);
    store4_agent(po, G * D * 4, item * 16, o);
    if ((4 * item) % D == 0) {
      const int g = (4 * item) / D;
      __hip_atomic_store(pml + 2 * g, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pml + 2 * g + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every store of this thread has completed at agent scope before the barrier; after it, one
  // thread counts the chunk as finished.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(p.counters + bj, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (done == (uint32_t)(nlive - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // Acquire at agent scope: drop this XCD's cached copies of the workspace lines, so the loads
  // below see what the other workgroups wrote through to memory.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // Last chunk of (b, j) to finish: log-sum-exp merge of all nlive partials, in chunk order.
  float* cm = ep;                        // [nlive][G] chunk max, then its weight
  float* cl = ep + kCombinePairs;        // [nlive][G] chunk sum
  float* cinv = ep + 2 * kCombinePairs;  // [G] v_descale / total sum
  const float* pml0 = p.part_ml + (size_t)bj * p.nchunks * G * 2;
  const float* po0 = p.part_o + (size_t)bj * p.nchunks * G * D;
  const uint32_t o_bytes = (uint32_t)(nlive * G * D * 4);
  for (int i = tid; i < nlive * G; i += NTH) {
    cm[i] = __hip_atomic_load(pml0 + 2 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cl[i] = __hip_atomic_load(pml0 + 2 * i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int g = tid; g < G; g += NTH) {
    float M = -INFINITY;
    for (int k = 0; k < nlive; ++k) M = fmaxf(M, cm[k * G + g]);
    float l = 0.f;
    for (int k = 0; k < nlive; ++k) {
      const float s = __builtin_amdgcn_exp2f(cm[k * G + g] - M);
      cm[k * G + g] = s;
      l += s * cl[k * G + g];
    }
    cinv[g] = p.v_descale / l;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(po0, o_bytes);
  for (int item = tid; item < G * D / 4; item += NTH) {
    const int g = (4 * item) / D;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + 4 <= nlive; k += 4) {  // four partial loads in flight per thread
      u32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, ((k + u) * G * D + 4 * item) * 4, 0, kAgentScope));
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += cm[(k + u) * G + g] * __builtin_bit_cast(f32x4_t, v[u]);
    }
    for (; k < nlive; ++k) {
      const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, (k * G * D + 4 * item) * 4, 0, kAgentScope));
      acc += cm[k * G + g] * __builtin_bit_cast(f32x4_t, v);
    }
    const float inv = cinv[g];
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(out + 4 * item + e, acc[e] * inv);
  }
  if (tid == 0) __hip_atomic_store(p.counters + bj, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Work item of this workgroup.  Returns false when it has nothing to do (after writing the zero rows
// of an empty sequence from chunk 0).
template <int D, typename OutT, int NW>
__device__ __forceinline__ bool decode_work_item(const Params& p, int& b, int& j, int& c, int& n,
                                                 int& nlive) {
  const int wg = blockIdx.x;
  c = wg % p.nchunks;
  const int bj = wg / p.nchunks;
  j = bj % p.Hkv;
  b = bj / p.Hkv;
  n = p.seq_lens[b];
  n = n < 0 ? 0 : (n > p.L ? p.L : n);
  if (n == 0) {
    if (c == 0) {
      OutT* out = reinterpret_cast<OutT*>(p.out) + ((size_t)b * p.Hq + (size_t)j * p.G) * D;
      for (int idx = threadIdx.x; idx < p.G * D; idx += NW * 64) store_out(out + idx, 0.f);
    }
    return false;
  }
  if (c * p.chunk >= n) return false;
  nlive = (n + p.chunk - 1) / p.chunk;
  return true;
}

// ------------------------------------------------------------------------------------------------
// bf16 / fp8 cache: matrix-core kernel.
//
// Per 32-token tile and wave (lane l, quad q = l / 16, r = l % 16):
//   QK^T on v_mfma_f32_16x16x32_bf16 with A = K tile (M = tokens, K = head dim) loaded straight from
//   HBM into the A-operand layout, and B = Q^T (N = query rows of the group, zero-padded to 16).
//   The result leaves lane l holding S[g = r][t = 16h + 4q + i].
//   PV on the same instruction with A = V^T (M = head-dim columns, K = tokens) read from a per-wave
//   LDS copy of the tile with ds_read_b64_tr_b16, and B = P^T, which is exactly S's register layout
//   after exp2 and a bf16 pack.  The accumulator O^T leaves lane l holding O[g = r][c = 16m + 4q + i],
//   so the running max / sum of row g live in the same lanes as its outputs.
// NT = 16-row tiles of query rows (G <= 16 * NT).
template <int D, int NT, bool FP8, typename OutT, int NW>
__global__ void __launch_bounds__(NW * 64, NT == 1 ? 2 : 1) decode_mfma_kernel(Params p) {
  constexpr int TILE = 32;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int MT = D / 16;          // m-tiles of PV
  constexpr int ELT = FP8 ? 1 : 2;    // bytes per cache element
  constexpr int ROWB = D * ELT;       // bytes per cache row
  constexpr int NK = 2 * D * ELT / 64;          // 16-byte K loads per lane per tile
  constexpr int NV = TILE * ROWB / (64 * 16);   // 16-byte V loads per lane per tile
  constexpr int CPR = D / 8;          // 16-byte bf16 chunks per row of the LDS V tile
  constexpr int VTILE = TILE * D * 2;            // bytes of one LDS V tile (bf16)
  constexpr int GT = 16 * NT;
  using Epi = EpiLayout<GT, D, NW>;
  constexpr int SMEM0 = (NW * VTILE > Epi::kBytes) ? NW * VTILE : Epi::kBytes;
  constexpr int SMEM = SMEM0 > kCombineBytes ? SMEM0 : kCombineBytes;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  int b, j, c, n, nlive;
  if (!decode_work_item<D, OutT, NW>(p, b, j, c, n, nlive)) return;

  const int w = threadIdx.x / 64;
  const int l = threadIdx.x % 64;
  const int q = l / 16;
  const int r = l % 16;
  const int G = p.G;

  // ---- query rows of group j, in the B-operand layout of QK^T (zero rows beyond G)
  bf16x8_t bq[NT][KS];
  {
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)b * p.Hq + (size_t)j * G) * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int g = r + 16 * nt;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        // head-dim index of k-slot (8q + e) in k-step s; the K loads below use the same map
        const int d0 = FP8 ? (64 * (s / 2) + 16 * q + 8 * (s % 2)) : (32 * s + 8 * q);
        u32x4_t v = {0, 0, 0, 0};
        if (g < G) v = *reinterpret_cast<const u32x4_t*>(qb + (size_t)g * D + d0);
        bq[nt][s] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  const size_t head = ((size_t)b * p.Hkv + j) * (size_t)p.L * ROWB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(p.k) + head, (uint32_t)n * ROWB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(p.v) + head, (uint32_t)n * ROWB);

  const int tok0 = c * p.chunk;
  const int tok_end = min(tok0 + p.chunk, n);
  const int ntiles = (tok_end - tok0 + TILE - 1) / TILE;
  const int mine = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;  // tiles w, w+NW, ...

  char* vt = smem + w * VTILE;  // this wave's LDS V tile
  const uint32_t vt_lds = (uint32_t)(uintptr_t)(GQA_LDS char*)vt;

  float m_run[NT], l_run[NT];
  f32x4_t o[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  struct Regs {
    u32x4_t k[NK];
    u32x4_t v[NV];
  };
  auto tile_start = [&](int it) { return tok0 + (w + it * NW) * TILE; };
  auto issue = [&](Regs& R, int it) {
    const bool live = it < mine;
    const uint32_t t0 = live ? (uint32_t)tile_start(it) : 0u;
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      // x = h * (NK/2) + u: token subtile h (16 rows), 16-byte column block u of this lane's quad
      const int h = x / (NK / 2), u = x % (NK / 2);
      const uint32_t off = (t0 + 16 * h + r) * ROWB + u * 64 + q * 16;
      R.k[x] = load16(rk, live ? off : kNoTile);
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const uint32_t off = t0 * ROWB + (x * 64 + l) * 16;
      R.v[x] = load16(rv, live ? off : kNoTile);
    }
  };

  auto compute = [&](Regs& R, int it) {
    const int t0 = tile_start(it);
    // -- stage V (as bf16) into the wave's LDS tile, 16-byte chunks XOR-swizzled by row
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int idx = x * 64 + l;  // 16-byte chunk index of the tile in global memory
      if constexpr (!FP8) {
        const int row = idx / CPR, ch = idx % CPR;
        const int pos = ch ^ (2 * (row % (D / 16)));
        *reinterpret_cast<u32x4_t*>(vt + row * D * 2 + pos * 16) = R.v[x];
      } else {
        const int row = idx / (CPR / 2), ch8 = idx % (CPR / 2);
        const u32x4_t a = R.v[x];
        const u32x4_t lo = {fp8x2_to_bf16x2<false>(a[0]), fp8x2_to_bf16x2<true>(a[0]),
                            fp8x2_to_bf16x2<false>(a[1]), fp8x2_to_bf16x2<true>(a[1])};
        const u32x4_t hi = {fp8x2_to_bf16x2<false>(a[2]), fp8x2_to_bf16x2<true>(a[2]),
                            fp8x2_to_bf16x2<false>(a[3]), fp8x2_to_bf16x2<true>(a[3])};
        const int sw = 2 * (row % (D / 16));
        *reinterpret_cast<u32x4_t*>(vt + row * D * 2 + ((2 * ch8) ^ sw) * 16) = lo;
        *reinterpret_cast<u32x4_t*>(vt + row * D * 2 + ((2 * ch8 + 1) ^ sw) * 16) = hi;
      }
    }
    // -- K operands
    bf16x8_t ak[2][KS];
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int h = x / (NK / 2), u = x % (NK / 2);
      if constexpr (!FP8) {
        ak[h][u] = __builtin_bit_cast(bf16x8_t, R.k[x]);
      } else {
        const u32x4_t a = R.k[x];
        const u32x4_t lo = {fp8x2_to_bf16x2<false>(a[0]), fp8x2_to_bf16x2<true>(a[0]),
                            fp8x2_to_bf16x2<false>(a[1]), fp8x2_to_bf16x2<true>(a[1])};
        const u32x4_t hi = {fp8x2_to_bf16x2<false>(a[2]), fp8x2_to_bf16x2<true>(a[2]),
                            fp8x2_to_bf16x2<false>(a[3]), fp8x2_to_bf16x2<true>(a[3])};
        ak[h][2 * u] = __builtin_bit_cast(bf16x8_t, lo);
        ak[h][2 * u + 1] = __builtin_bit_cast(bf16x8_t, hi);
      }
    }
    // -- scores S^T = K Q^T
    f32x4_t sc[2][NT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[h][s], bq[nt][s], acc, 0, 0, 0);
        sc[h][nt] = acc * p.qk_scale;
      }
    if (t0 + TILE > n) {  // ragged last tile: positions >= n get no weight
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 16 * h + 4 * q + i >= n)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sc[h][nt][i] = -INFINITY;
    }
    // -- online softmax; P^T packed to bf16 in the B-operand layout of PV
    bf16x8_t bp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = fmaxf(fmaxf(fmaxf(sc[0][nt][0], sc[0][nt][1]), fmaxf(sc[0][nt][2], sc[0][nt][3])),
                       fmaxf(fmaxf(sc[1][nt][0], sc[1][nt][1]), fmaxf(sc[1][nt][2], sc[1][nt][3])));
      mx = wave_max_xor_16_32(mx);
      const float m_new = fmaxf(m_run[nt], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      m_run[nt] = m_new;
      uint32_t pk[4];
      float psum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const uint32_t lo = float_to_bf16_bits(__builtin_amdgcn_exp2f(sc[h][nt][2 * i2] - m_new));
          const uint32_t hi = float_to_bf16_bits(__builtin_amdgcn_exp2f(sc[h][nt][2 * i2 + 1] - m_new));
          psum += bf16_bits_to_float(lo) + bf16_bits_to_float(hi);  // sum the weights actually used
          pk[2 * h + i2] = lo | (hi << 16);
        }
      l_run[nt] = l_run[nt] * alpha + psum;
      bp[nt] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
    }
    // -- O^T += V^T P^T, V^T read transposed from LDS
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t a[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 16 * h + 4 * q + r / 4;
        const int col = 16 * mt + 4 * (r % 4);
        const int pos = (col / 8) ^ (2 * (row % (D / 16)));
        const uint32_t addr = vt_lds + row * D * 2 + pos * 16 + (col % 8) * 2;
        const i16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS i16x4_t*)(uintptr_t)addr);
        const u32x2_t tt = __builtin_bit_cast(u32x2_t, t);
        a[2 * h] = tt[0];
        a[2 * h + 1] = tt[1];
      }
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, u32x4_t{a[0], a[1], a[2], a[3]});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bp[nt], o[nt][mt], 0, 0, 0);
    }
  };

  // ---- software pipeline: the next tile's loads are in flight while this tile is computed
  Regs A, B;
  issue(A, 0);
  for (int it = 0; it < mine; it += 2) {
    issue(B, it + 1);
    compute(A, it);
    if (it + 1 >= mine) break;
    issue(A, it + 2);
    compute(B, it + 1);
  }

  // ---- wave state -> LDS (canonical layout), then the shared epilogue
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_run[nt] = wave_sum_xor_16_32(l_run[nt]);
  __syncthreads();  // every wave is done with its V tile: the LDS is reused below
  float* ep = reinterpret_cast<float*>(smem);
  constexpr int kRow = Epi::kRow;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int g = r + 16 * nt;
    if (q == 0) {
      ep[w * GT + g] = m_run[nt];
      ep[NW * GT + w * GT + g] = l_run[nt];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4_t*>(ep + 2 * NW * GT + (w * GT + g) * kRow + 16 * mt + 4 * q) = o[nt][mt];
  }
  __syncthreads();
  epilogue<GT, D, NW, OutT>(p, ep, b, j, c, nlive);
}

// ------------------------------------------------------------------------------------------------
// f32 cache: vector-ALU kernel (lane = token for the scores, lane = head-dim column for P V).
// GT >= G query rows are processed; rows g >= G see a zero query and are never stored.
template <int D, int GT, typename OutT, int NW>
__global__ void __launch_bounds__(NW * 64) decode_f32_kernel(Params p) {
  constexpr int TILE = 64;
  constexpr int CPL = D / 64;  // output columns per lane
  using Epi = EpiLayout<GT, D, NW>;
  constexpr int QB = GT * D * 4;
  constexpr int PB = NW * GT * TILE * 4;
  constexpr int MAIN = QB + PB;
  constexpr int SMEM0 = MAIN > Epi::kBytes ? MAIN : Epi::kBytes;
  constexpr int SMEM = SMEM0 > kCombineBytes ? SMEM0 : kCombineBytes;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  int b, j, c, n, nlive;
  if (!decode_work_item<D, OutT, NW>(p, b, j, c, n, nlive)) return;
  const int w = threadIdx.x / 64;
  const int l = threadIdx.x % 64;
  const int G = p.G;

  float* qs = reinterpret_cast<float*>(smem);
  float* ps = reinterpret_cast<float*>(smem + QB) + w * GT * TILE;
  {
    const float* qg = reinterpret_cast<const float*>(p.q) + ((size_t)b * p.Hq + (size_t)j * G) * D;
    for (int idx = threadIdx.x; idx < GT * D; idx += NW * 64) qs[idx] = (idx / D < G) ? qg[idx] : 0.f;
  }
  __syncthreads();

  const float* kh = reinterpret_cast<const float*>(p.k) + ((size_t)b * p.Hkv + j) * (size_t)p.L * D;
  const float* vh = reinterpret_cast<const float*>(p.v) + ((size_t)b * p.Hkv + j) * (size_t)p.L * D;
  const int tok0 = c * p.chunk;
  const int tok_end = min(tok0 + p.chunk, n);

  float m_run[GT], l_run[GT], o[GT][CPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int x = 0; x < CPL; ++x) o[g][x] = 0.f;
  }

  for (int t0 = tok0 + w * TILE; t0 < tok_end; t0 += NW * TILE) {
    const int t = t0 + l;
    const bool valid = t < tok_end;
    float s[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) s[g] = 0.f;
    if (valid) {
      const float4* kr = reinterpret_cast<const float4*>(kh + (size_t)t * D);
      for (int c4 = 0; c4 < D / 4; ++c4) {
        const float4 kv = kr[c4];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float4 qv = *reinterpret_cast<const float4*>(qs + g * D + 4 * c4);
          s[g] += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float sg = valid ? s[g] * p.qk_scale : -INFINITY;
      float mx = sg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[g], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      const float pw = __builtin_amdgcn_exp2f(sg - m_new);
      l_run[g] = l_run[g] * alpha + pw;
#pragma unroll
      for (int x = 0; x < CPL; ++x) o[g][x] *= alpha;
      ps[g * TILE + l] = pw;
    }
    const int cnt = min(TILE, tok_end - t0);
    for (int tt = 0; tt < cnt; ++tt) {
      float vv[CPL];
#pragma unroll
      for (int x = 0; x < CPL; ++x) vv[x] = vh[(size_t)(t0 + tt) * D + 64 * x + l];
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float pw = ps[g * TILE + tt];
#pragma unroll
        for (int x = 0; x < CPL; ++x) o[g][x] += pw * vv[x];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l_run[g] += __shfl_xor(l_run[g], off);

  __syncthreads();
  float* ep = reinterpret_cast<float*>(smem);
  constexpr int kRow = Epi::kRow;
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    if (l == 0) {
      ep[w * GT + g] = m_run[g];
      ep[NW * GT + w * GT + g] = l_run[g];
    }
#pragma unroll
    for (int x = 0; x < CPL; ++x) ep[2 * NW * GT + (w * GT + g) * kRow + 64 * x + l] = o[g][x];
  }
  __syncthreads();
  epilogue<GT, D, NW, OutT>(p, ep, b, j, c, nlive);
}

// ------------------------------------------------------------------------------------------------
// Workspace counter clear (a kernel rather than a memset so that it may be captured in a graph).
__global__ void clear_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// seq_lens range check (test helper).
__global__ void count_bad_seq_lens_kernel(const int32_t* s, int B, int L, int32_t* bad) {
  int cnt = 0;
  for (int i = threadIdx.x; i < B; i += blockDim.x) cnt += (s[i] < 0 || s[i] > L) ? 1 : 0;
  for (int off = 1; off < 64; off <<= 1) cnt += __shfl_xor(cnt, off);
  if (threadIdx.x == 0) *bad = cnt;
}

// Streaming read for bandwidth calibration: workgroup w reads chunk range [lo, hi) of 16-byte
// chunks, eight non-temporal loads in flight per thread.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                          size_t per_wg, uint32_t* sink) {
  const size_t lo = (size_t)blockIdx.x * per_wg;
  const size_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += 256) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int off = 1; off < 64; off <<= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t red[4];
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace gqa
