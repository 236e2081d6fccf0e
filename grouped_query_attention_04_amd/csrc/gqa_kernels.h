// gqa_kernels.h -- HIP kernels (gfx950 / CDNA4) for single-token grouped-query-attention decode.
//
// The arithmetic is scaled dot-product attention per query head, where query head h reads KV head
// floor(h / G) ("Grouped Query Attention (GQA): Efficient Multi-Head Attention", Worked example 2;
// "Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory", section "How
// grouped-query attention works").  A K/V tile is read from HBM once and serves all G query rows of
// its group ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch Size", section "Why does
// GQA speed up decode, not just save memory?").
//
// Work decomposition (one launch).  The cache is cut into tiles of TILE positions; the tiles of all
// (batch b, KV head j) segments, laid end to end in (b, j) order, form one tile space of T tiles
// that the W launched workgroups split into equal contiguous ranges.  Every workgroup therefore
// streams the same number of bytes whatever the mix of sequence lengths.  A range covers pieces of
// one or more segments; its NW waves share each piece tile by tile, keep running softmax state
// (max and sum per query row, base-2 domain) and merge it in LDS when the piece ends.  A piece that
// is a whole segment is normalised and stored at once.  A piece of a segment that several
// workgroups share is published to the workspace; the workgroup that finishes a segment's last
// piece -- found with one atomic counter per (b, j) -- merges the pieces in workgroup order and
// stores the output.  Nothing waits on another workgroup.  Two workgroups fit on a compute unit
// (at most 256 registers per lane), so one's pauses at piece ends can overlap with the other's
// streaming when more than one workgroup per compute unit is launched.
#pragma once

#include "gqa_device.h"

namespace gqa {

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  void* out;
  float* part_o;       // [W][2][G][D] unnormalised outputs of published pieces (G, Hkv: of the segments)
  float* part_ml;      // [W][2][G][2] their (max, sum), base-2 domain
  uint32_t* counters;  // [B*Hkv] finished-piece counters, one per segment, zero between calls
  uint32_t* header;    // workspace header: tag words 0-1, error count word 2
  // Hkv and G describe the kernel's segments: with a query-head split of hs, every KV head of the
  // cache serves hs consecutive segment heads j (cache head j / hs), each with G = Hq / Hkv of its
  // query heads; hs = 1 is the plain layout.
  int B, Hq, Hkv, L, G;
  int hs;
  int W;            // workgroups launched
  float qk_scale;   // scale * k_descale * log2(e)
  float v_descale;  // applied to the normalised output
  // paged cache only: k and v are page pools [num_blocks][Hkv / hs][block_size][D]; block_table is
  // [B][max_blocks]; block_size = 1 << block_shift positions per page.
  const int32_t* block_table;
  int block_shift, max_blocks, num_blocks;
  // fused append (decode_mfma_kernel with APPEND): the new rows k_new, v_new [B][Hkv / hs][D] (bf16) go
  // to position seq_lens[b] - 1, in the cache format (fp8: code of x / enc_descale).
  const void* k_new;
  const void* v_new;
  int32_t* skipped;  // optional: sequences whose new position lies past the cache or on a page outside the pool
  float k_enc_descale, v_enc_descale;
};

// ------------------------------------------------------------------------------------------------
// Workspace header.  gqa_workspace_init clears the counter area and then writes this two-word tag at
// the start of the workspace.  The merge of shared segments relies on counters that start at zero; a
// workspace without the tag (never initialised, or overwritten) is refused by every workgroup, which
// fills its output rows with NaN and counts itself in header word 2 instead of touching a counter.
constexpr uint32_t kWorkspaceTag0 = 0x41514721u, kWorkspaceTag1 = 0x5EED0C7Au;
constexpr int kWorkspaceHeaderWords = 64;  // 256 bytes before the counter area
// Header word 3 holds merge-route flags for tests (zero after initialisation): bit 0 publishes every
// shared piece (the merge from registers of a segment's last piece is off), bit 1 counts the merges
// from registers in header word 4.  The output does not depend on them.
constexpr int kRouteFlagsWord = 3, kShortcutCountWord = 4;
constexpr uint32_t kRouteAlwaysPublish = 1u, kRouteCountShortcuts = 2u;

// Both tag words, read with scalar loads; the caller compares them later, so the load's latency
// overlaps with whatever comes in between.
__device__ __forceinline__ u32x2_t workspace_tag(const Params& p) {
  const GQA_CONST u32x2_t* h = (const GQA_CONST u32x2_t*)(uintptr_t)p.header;
  return *h;
}

__device__ __forceinline__ bool workspace_ok(u32x2_t tag) {
  return tag[0] == kWorkspaceTag0 && tag[1] == kWorkspaceTag1;
}

// The refusal: NaN in the output rows of batch entries b = blockIdx.x + k * W, and one count.
template <int D, typename OutT, int NTH>
__device__ void refuse_workspace(const Params& p) {
  for (int b = blockIdx.x; b < p.B; b += p.W) {
    OutT* out = reinterpret_cast<OutT*>(p.out) + (size_t)b * p.Hq * D;
    for (int i = threadIdx.x; i < p.Hq * D; i += NTH) store_out(out + i, __builtin_nanf(""));
  }
  if (threadIdx.x == 0) __hip_atomic_fetch_add(p.header + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------------------
// Tile space and its split over workgroups.

struct Shared {  // small LDS block every kernel carries
  int red[16];
  int found_b, found_pre;
  int last;
};

__device__ __forceinline__ int seq_len(const Params& p, int b) {
  const int n = p.seq_lens[b];
  return n < 0 ? 0 : (n > p.L ? p.L : n);
}
template <int TILE>
__device__ __forceinline__ int seq_tiles(const Params& p, int b) {
  return (seq_len(p, b) + TILE - 1) / TILE;
}

template <int NTH>
__device__ int block_sum(int x, Shared& sh) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (threadIdx.x % 64 == 0) sh.red[threadIdx.x / 64] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NTH / 64; ++i) t += sh.red[i];
  __syncthreads();
  return uniform(t);
}

// Inclusive prefix sum over the workgroup's threads (thread order); *total receives the sum.
template <int NTH>
__device__ int block_scan(int x, Shared& sh, int* total) {
  const int lane = threadIdx.x % 64;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh.red[threadIdx.x / 64] = x;
  __syncthreads();
  int before = 0, t = 0;
#pragma unroll
  for (int i = 0; i < NTH / 64; ++i) {
    if (i < (int)(threadIdx.x / 64)) before += sh.red[i];
    t += sh.red[i];
  }
  __syncthreads();
  *total = uniform(t);
  return x + before;
}

// This workgroup's tile range [lo, hi) and the batch entry holding tile lo.
struct Range {
  long long T;  // tiles in the whole space
  int weff;     // workgroups that receive tiles: min(W, T)
  long long lo, hi;
  int b, pre;   // batch entry of tile lo, and the tiles of all batch entries before it (per head)
};

__device__ __forceinline__ long long range_lo(long long w, long long T, int weff) { return w * T / weff; }
// Workgroup whose range holds tile x: the largest w with range_lo(w) <= x.
__device__ __forceinline__ int range_owner(long long x, long long T, int weff) {
  return uniform((int)(((x + 1) * weff - 1) / T));
}

template <int TILE, int NTH>
__device__ bool find_range(const Params& p, Shared& sh, Range& r) {
  if (p.B <= NTH) {
    // One pass: thread b holds batch entry b's tile count; one scan gives the total and the
    // entry's prefix, and the thread whose entry holds tile lo reports it.
    const int b = (int)threadIdx.x;
    const int t = b < p.B ? seq_tiles<TILE>(p, b) : 0;
    int total;
    const int incl = block_scan<NTH>(t, sh, &total);
    r.T = (long long)p.Hkv * total;
    r.weff = r.T < p.W ? (int)r.T : p.W;
    const int w = blockIdx.x;
    if (w >= r.weff) return false;
    r.lo = range_lo(w, r.T, r.weff);
    r.hi = range_lo(w + 1, r.T, r.weff);
    const long long s = (long long)p.Hkv * (incl - t), e = (long long)p.Hkv * incl;
    if (t > 0 && s <= r.lo && r.lo < e) {
      sh.found_b = b;
      sh.found_pre = incl - t;
    }
    __syncthreads();
    r.b = uniform(sh.found_b);
    r.pre = uniform(sh.found_pre);
    return true;
  }
  int part = 0;
  for (int b = threadIdx.x; b < p.B; b += NTH) part += seq_tiles<TILE>(p, b);
  r.T = (long long)p.Hkv * block_sum<NTH>(part, sh);
  r.weff = r.T < p.W ? (int)r.T : p.W;
  const int w = blockIdx.x;
  if (w >= r.weff) return false;
  r.lo = range_lo(w, r.T, r.weff);
  r.hi = range_lo(w + 1, r.T, r.weff);
  // batch entry b with Hkv * prefix(b) <= lo < Hkv * prefix(b + 1)
  int carry = 0;
  for (int base = 0; base < p.B; base += NTH) {
    const int b = base + (int)threadIdx.x;
    const int t = b < p.B ? seq_tiles<TILE>(p, b) : 0;
    int total;
    const int incl = block_scan<NTH>(t, sh, &total);
    const long long s = (long long)p.Hkv * (carry + incl - t), e = (long long)p.Hkv * (carry + incl);
    if (t > 0 && s <= r.lo && r.lo < e) {
      sh.found_b = b;
      sh.found_pre = carry + incl - t;
    }
    carry += total;
    __syncthreads();
    if ((long long)p.Hkv * carry > r.lo) break;
  }
  r.b = uniform(sh.found_b);
  r.pre = uniform(sh.found_pre);
  return true;
}

// Zero output rows of empty sequences: batch entries b = blockIdx.x + k * W.
template <int D, typename OutT, int NTH>
__device__ void zero_empty_rows(const Params& p) {
  for (int b = blockIdx.x; b < p.B; b += p.W) {
    if (uniform(seq_len(p, b)) != 0) continue;
    OutT* out = reinterpret_cast<OutT*>(p.out) + (size_t)b * p.Hq * D;
    for (int i = threadIdx.x; i < p.Hq * D; i += NTH) store_out(out + i, 0.f);
  }
}

// ------------------------------------------------------------------------------------------------
// Piece epilogue.  The NW waves have left, in LDS (ep):
//   ep_m[w][g], ep_l[w][g]   running max (base 2) and running sum of wave w for query row g
//   ep_o[w][g][c]            unnormalised output of wave w (row stride D + 4 floats)
// Waves that saw no token hold (-inf, 0, 0).  Rows g < G are valid.
template <int GT, int D, int NW>
struct EpiLayout {
  static constexpr int kRow = D + 4;
  static constexpr int kBytes = NW * GT * (2 + kRow) * 4;
};

struct Piece {
  int b, j;
  long long s, e;  // the segment's tile range in the tile space
  int slot;        // 0: the piece starts this workgroup's range, 1: it ends it
};

// One log-sum-exp combine step: (acc_m, acc_l, acc_o) absorbs a partial (m, l, o) whose weights are
// relative to base-2 maximum m.  Written with explicit fused multiply-adds, so the rounding is the
// same wherever it is inlined: the compiler's free choice of which product to fuse in x * a + y * b
// differs between call sites, and the merges below must agree bit for bit whichever workgroup runs
// them.
__device__ __forceinline__ void lse_combine(float& acc_m, float& acc_l, f32x4_t& acc_o, float m, float l,
                                            f32x4_t o) {
  const float mn = fmaxf(acc_m, m);
  const float a = __builtin_amdgcn_exp2f(acc_m - mn);
  const float sc = __builtin_amdgcn_exp2f(m - mn);
  acc_l = __builtin_fmaf(l, sc, acc_l * a);
#pragma unroll
  for (int c = 0; c < 4; ++c) acc_o[c] = __builtin_fmaf(o[c], sc, acc_o[c] * a);
  acc_m = mn;
}

// Log-sum-exp merge of a segment's npc published pieces (those of workgroups wfirst ..
// wfirst + npc - 1, in that order) into the output rows.  Every thread carries the running (max,
// sum, output) of NI items (4 consecutive columns of one query row each).  The pieces' partials
// stream through PB register sets: piece k is merged, then the loads of piece k + PB go out, so PB
// pieces are always in flight and the merge pays one load latency, not one per group of pieces.
// The piece loop is uniform, so each piece's buffer descriptors stay scalar.  Every load carries
// agent scope (sc1), the form of a relaxed agent-scope atomic load.
template <int D, typename OutT, int NTH, int NI, int PB>
__device__ __forceinline__ void merge_pieces(const Params& p, OutT* out, int nitems, int wfirst, int npc,
                                             int first_slot) {
  const int tid = threadIdx.x;
  const int G = p.G;
  float acc_m[NI], acc_l[NI];
  f32x4_t acc_o[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc_m[i] = -INFINITY;
    acc_l[i] = 0.f;
    acc_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  struct PieceRegs {
    uint32_t m[NI], l[NI];
    u32x4_t o[NI];
  };
  auto load_piece = [&](PieceRegs& R, int k) __attribute__((always_inline)) {
    if (k >= npc) return;
    const size_t sl = (size_t)uniform((wfirst + k) * 2 + (k == 0 ? first_slot : 0));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.part_o + sl * G * D, G * D * 4);
    const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.part_ml + sl * G * 2, G * 2 * 4);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int item = tid + i * NTH;
      if (i > 0 && uniform(i * NTH) >= nitems) break;  // item slots past the group's rows
      const int g = (4 * (item < nitems ? item : 0)) / D;
      // two 4-byte loads: element 1 of a 64-bit buffer load's vector result is not reliable here
      R.m[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rml, g * 8, 0, kAgentScope);
      R.l[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rml, g * 8 + 4, 0, kAgentScope);
      R.o[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, item * 16, 0, kAgentScope));
    }
  };
  auto merge_piece = [&](const PieceRegs& R) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i > 0 && uniform(i * NTH) >= nitems) break;  // not loaded: never stored either
      lse_combine(acc_m[i], acc_l[i], acc_o[i], __builtin_bit_cast(float, R.m[i]),
                  __builtin_bit_cast(float, R.l[i]), __builtin_bit_cast(f32x4_t, R.o[i]));
    }
  };
  PieceRegs R[PB];
#pragma unroll
  for (int u = 0; u < PB; ++u) load_piece(R[u], u);
  for (int k0 = 0; k0 < npc; k0 += PB) {
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (k0 + u >= npc) break;
      merge_piece(R[u]);
      load_piece(R[u], k0 + u + PB);
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int item = tid + i * NTH;
    if (item < nitems) store_out4(out + 4 * item, acc_o[i] * (p.v_descale / acc_l[i]));
  }
}

// Log-sum-exp merge of a segment's npc <= 3 pieces in workgroup order, where piece own_k is this
// workgroup's own, held in registers (own_*), and the others are read from their slots.
template <int D, typename OutT, int NTH, int NI>
__device__ __forceinline__ void merge_with_own(const Params& p, OutT* out, int nitems, int wfirst, int npc,
                                               int first_slot, int own_k, const float* own_m,
                                               const float* own_l, const f32x4_t* own_o) {
  const int tid = threadIdx.x;
  const int G = p.G;
  float acc_m[NI], acc_l[NI];
  f32x4_t acc_o[NI];
  uint32_t pm[2][NI], plv[2][NI];
  u32x4_t po[2][NI];
  // the (up to two) other pieces' partials, loaded together
#pragma unroll
  for (int li = 0; li < 2; ++li) {
    if (li >= npc - 1) break;
    const int kk = uniform(li >= own_k ? li + 1 : li);
    const size_t sl = (size_t)uniform((wfirst + kk) * 2 + (kk == 0 ? first_slot : 0));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.part_o + sl * G * D, G * D * 4);
    const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.part_ml + sl * G * 2, G * 2 * 4);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int item = tid + i * NTH;
      if (i > 0 && uniform(i * NTH) >= nitems) break;
      const int g = (4 * (item < nitems ? item : 0)) / D;
      pm[li][i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rml, g * 8, 0, kAgentScope);
      plv[li][i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rml, g * 8 + 4, 0, kAgentScope);
      po[li][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, item * 16, 0, kAgentScope));
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc_m[i] = -INFINITY;
    acc_l[i] = 0.f;
    acc_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  auto merge_vals = [&](int i, float m, float l, f32x4_t o) __attribute__((always_inline)) {
    lse_combine(acc_m[i], acc_l[i], acc_o[i], m, l, o);
  };
  // pieces in workgroup order: k = 0 .. npc - 1, the own one at own_k
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    if (kk >= npc) break;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i > 0 && uniform(i * NTH) >= nitems) break;
      if (kk == own_k) {
        merge_vals(i, own_m[i], own_l[i], own_o[i]);
      } else {
        const int li = kk > own_k ? kk - 1 : kk;
        merge_vals(i, __builtin_bit_cast(float, li == 0 ? pm[0][i] : pm[1][i]),
                   __builtin_bit_cast(float, li == 0 ? plv[0][i] : plv[1][i]),
                   __builtin_bit_cast(f32x4_t, li == 0 ? po[0][i] : po[1][i]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int item = tid + i * NTH;
    if (item < nitems) store_out4(out + 4 * item, acc_o[i] * (p.v_descale / acc_l[i]));
  }
}

template <int GT, int D, int NW, typename OutT>
__device__ void piece_epilogue(const Params& p, const float* ep, const Range& r, const Piece& pc,
                               Shared& sh, bool known_last = false, uint32_t route_flags = 0) {
  constexpr int NTH = NW * 64;
  constexpr int kRow = EpiLayout<GT, D, NW>::kRow;
  const int tid = threadIdx.x;
  const int G = p.G;
  const int nitems = G * D / 4;  // groups of 4 consecutive columns of one query row
  const float* ep_m = ep;
  const float* ep_l = ep + NW * GT;
  const float* ep_o = ep + 2 * NW * GT;
  OutT* out = reinterpret_cast<OutT*>(p.out) + ((size_t)pc.b * p.Hq + (size_t)pc.j * G) * D;

  // merge of the NW wave states for one item
  auto merge4 = [&](int item, float& M, float& l, f32x4_t& o) {
    const int g = (4 * item) / D, cc = (4 * item) % D;
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, ep_m[w * GT + g]);
    l = 0.f;
    o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      // explicit fused multiply-adds: the publishing and the merging epilogues inline this at
      // different sites and must round alike
      const float s = __builtin_amdgcn_exp2f(ep_m[w * GT + g] - M);
      l = __builtin_fmaf(s, ep_l[w * GT + g], l);
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(ep_o + (w * GT + g) * kRow + cc);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = __builtin_fmaf(s, x[c], o[c]);
    }
  };

  const int wfirst = range_owner(pc.s, r.T, r.weff);
  const int wlast = range_owner(pc.e - 1, r.T, r.weff);
  if (wfirst == wlast) {  // the whole segment was here: normalise and store
    for (int item = tid; item < nitems; item += NTH) {
      float M, l;
      f32x4_t o;
      merge4(item, M, l, o);
      store_out4(out + 4 * item, o * (p.v_descale / l));
    }
    return;
  }

  if (GT == 16 && known_last) {
    // The segment's other pieces (at most two) were all published and counted before this
    // workgroup read the counter: merge them with this one, which is not published, at its place in
    // workgroup order (the same order and arithmetic as the merge below, so the result is bitwise
    // the same).  The counter was read with agent scope after those workgroups' counter updates,
    // which followed the completion of their stores, and the partials below are read with agent
    // scope after it, as in the merge below.  No other workgroup can take this segment as last:
    // this piece is never counted, so the count stays one short for them.
    constexpr int NI = (GT * D / 4 + NTH - 1) / NTH;
    float own_m[NI], own_l[NI];
    f32x4_t own_o[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int item = tid + i * NTH;
      own_m[i] = -INFINITY;
      own_l[i] = 0.f;
      own_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (item < nitems) merge4(item, own_m[i], own_l[i], own_o[i]);
    }
    const int first_slot = uniform(pc.s > range_lo(wfirst, r.T, r.weff) ? 1 : 0);
    merge_with_own<D, OutT, NTH, NI>(p, out, nitems, wfirst, wlast - wfirst + 1, first_slot,
                                     (int)blockIdx.x - wfirst, own_m, own_l, own_o);
    if (tid == 0) {
      __hip_atomic_store(p.counters + pc.b * p.Hkv + pc.j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (route_flags & kRouteCountShortcuts)
        __hip_atomic_fetch_add(p.header + kShortcutCountWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // A shared segment: publish this piece with agent-scope stores.
  const size_t slot = (size_t)blockIdx.x * 2 + pc.slot;
  float* pml = p.part_ml + slot * G * 2;
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(p.part_o + slot * G * D, G * D * 4);
  for (int item = tid; item < nitems; item += NTH) {
    float M, l;
    f32x4_t o;
    merge4(item, M, l, o);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), rpo, item * 16, 0, kAgentScope);
    if ((4 * item) % D == 0) {
      const int g = (4 * item) / D;
      __hip_atomic_store(pml + 2 * g, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pml + 2 * g + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every store of this thread has completed at agent scope before the barrier; after it, one
  // thread counts the piece as finished.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  const int bj = pc.b * p.Hkv + pc.j;
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(p.counters + bj, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = (done == (uint32_t)(wlast - wfirst));
  }
  __syncthreads();
  if (!uniform(sh.last)) return;
  // No acquire fence (it would invalidate this XCD's whole L2, about 2 us): every load of the other
  // pieces below carries agent scope (sc1), the form of a relaxed agent-scope atomic load, which is
  // coherent across the XCDs' L2 caches by itself; and each is issued after the counter update
  // returned (thread 0 waited for it before the barrier), so it sees the stores the other
  // workgroups completed before theirs.  The compiler fence keeps the loads below the barrier.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // Last piece of the segment: log-sum-exp merge of its pieces in workgroup order.  When the
  // group's items fit one per thread (G * D / 4 <= NTH, e.g. G <= 8 at D = 128), the pieces stream
  // through more register sets, so that up to 16 pieces' partials are in flight at once.
  const int npc = wlast - wfirst + 1;
  // Slot of the segment's piece in workgroup w: workgroups after the first hold the segment from
  // their first tile on, i.e. in slot 0; the first one holds it in slot 1 when the segment starts
  // after its first tile.
  const int first_slot = uniform(pc.s > range_lo(wfirst, r.T, r.weff) ? 1 : 0);
  constexpr int NI = (GT * D / 4 + NTH - 1) / NTH;
  if (NI > 1 && nitems <= NTH)
    merge_pieces<D, OutT, NTH, 1, 16>(p, out, nitems, wfirst, npc, first_slot);
  else
    merge_pieces<D, OutT, NTH, NI, (NI > 4 ? 2 : NI > 2 ? 4 : NI == 2 ? 8 : 16)>(p, out, nitems, wfirst, npc,
                                                                              first_slot);
  if (tid == 0) __hip_atomic_store(p.counters + bj, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Walks this workgroup's pieces in order; `body(piece, tile0, ntiles, n)` processes the tiles
// [tile0, tile0 + ntiles) of the piece's segment, whose sequence has n cached positions.
template <int TILE, int NTH, typename Body>
__device__ void for_each_piece(const Params& p, const Range& r, Body&& body) {
  int b = r.b, pre = r.pre;
  int tb = uniform(seq_tiles<TILE>(p, b));
  const long long row0 = (long long)p.Hkv * pre;
  int j = (int)((r.lo - row0) / tb);
  long long seg = row0 + (long long)j * tb;
  long long cur = r.lo;
  while (true) {
    const long long seg_end = seg + tb;
    const long long pend = seg_end < r.hi ? seg_end : r.hi;
    Piece pc;
    pc.b = b;
    pc.j = j;
    pc.s = seg;
    pc.e = seg_end;
    pc.slot = cur == r.lo ? 0 : 1;
    body(pc, (int)(cur - seg), (int)(pend - cur), uniform(seq_len(p, b)));
    cur = pend;
    if (cur >= r.hi) break;
    if (++j == p.Hkv) {
      j = 0;
      pre += tb;
      do {
        ++b;
        tb = uniform(seq_tiles<TILE>(p, b));
      } while (tb == 0);
      seg = (long long)p.Hkv * pre;
    } else {
      seg += tb;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// bf16 / fp8 cache: matrix-core kernel.
//
// Per 16-token tile and wave (lane l, quad q = l / 16, r = l % 16):
//   QK^T on v_mfma_f32_16x16x32_bf16 with A = K tile (M = tokens, K = head dim) loaded straight from
//   HBM into the A-operand layout, and B = Q^T (N = query rows of the group, zero-padded to 16).
//   The result leaves lane l holding S[g = r][t = 4q + i].
//   PV on v_mfma_f32_16x16x16_bf16 with A = V^T (M = head-dim columns, K = tokens) read from a
//   per-wave LDS copy of the tile with ds_read_b64_tr_b16, and B = P^T, which is exactly S's
//   register layout after exp2 and a bf16 pack.  The accumulator O^T leaves lane l holding
//   O[g = r][c = 16m + 4q + i], so the running max / sum of row g live in the same lanes as its
//   outputs.
// NT = 16-row tiles of query rows (G <= 16 * NT).
//
// PAGED: the cache lives in pages of block_size (a power of two, at least TILE) positions, so a tile
// never straddles two pages.  Each register set of the pipeline carries the page-table entry of the
// tile it will receive next (NBUF tiles on in the wave's order): the entry is loaded just ahead of
// the set's own tile loads and moved to a scalar register when that tile is computed, after the
// wait for the tile, so it never costs a wait of its own.  The page's buffer descriptors are built
// per tile; a page number outside the pool yields a descriptor of zero bytes.
template <int D, int NT, bool FP8, typename OutT, int NW, bool PAGED, bool APPEND>
__global__ void __launch_bounds__(NW * 64, NT == 1 ? 2 : 1) decode_mfma_kernel(Params p) {
  constexpr int TILE = 16;
  constexpr int NTH = NW * 64;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int MT = D / 16;          // m-tiles of PV
  constexpr int ELT = FP8 ? 1 : 2;    // bytes per cache element
  constexpr int ROWB = D * ELT;       // bytes per cache row
  constexpr int NK = D * ELT / 64;              // 16-byte K loads per lane per tile
  constexpr int NV = TILE * ROWB / (64 * 16);   // 16-byte V loads per lane per tile
  constexpr int CPR = D / 8;          // 16-byte bf16 chunks per row of the LDS V tile
  constexpr int VTILE = TILE * D * 2;            // bytes of one LDS V tile (bf16)
  constexpr int GT = 16 * NT;
  // register sets of the load pipeline.  Two for both cache formats: keeping three or four fp8 tiles
  // in flight (the bytes in flight of two bf16 tiles) was measured slower on the long fp8 cache
  // (B2 Hq64 Hkv8 L32768: 30.9 us with two sets, 31.3 with three, 32.0 with four, 33.2 with six),
  // and three bf16 sets slower on every bf16 workload (141.2 -> 142.4 us on the 70B layer).
  constexpr int NBUF = 2;
  using Epi = EpiLayout<GT, D, NW>;
  constexpr int SMEM = (NW * VTILE > Epi::kBytes) ? NW * VTILE : Epi::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ Shared sh;
  // fused append: per wave, the new K and V rows in the cache format (unused otherwise)
  __shared__ __attribute__((aligned(16))) char ascr[APPEND ? NW * 2 * ROWB : 16];

  const u32x2_t tag = workspace_tag(p);
  Range rg;
  const bool busy = find_range<TILE, NTH>(p, sh, rg);
  if (!workspace_ok(tag)) {
    refuse_workspace<D, OutT, NTH>(p);
    return;
  }
  if constexpr (APPEND) {
    // sequences whose new position lies past the cache: counted once, by workgroup b mod W
    if (p.skipped && threadIdx.x == 0)
      for (int b = blockIdx.x; b < p.B; b += p.W)
        if (p.seq_lens[b] > p.L) __hip_atomic_fetch_add(p.skipped, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  zero_empty_rows<D, OutT, NTH>(p);
  if (!busy) return;

  const int w = uniform((int)threadIdx.x / 64);  // wave index, scalar: tile addressing derives from it
  const int l = threadIdx.x % 64;
  const int q = l / 16;
  const int r = l % 16;
  const int G = p.G;
  char* vt = smem + w * VTILE;  // this wave's LDS V tile
  const uint32_t vt_lds = (uint32_t)(uintptr_t)(GQA_LDS char*)vt;
  float* ep = reinterpret_cast<float*>(smem);

  for_each_piece<TILE, NTH>(p, rg, [&](const Piece& pc, int tile0, int ntiles, int n) {
    // ---- query rows of group j, in the B-operand layout of QK^T (zero rows beyond G)
    bf16x8_t bq[NT][KS];
    {
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)pc.b * p.Hq + (size_t)pc.j * G) * D;
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
    const int hkv = p.Hkv / p.hs;       // KV heads of the cache
    const int jc = uniform(pc.j / p.hs);  // the cache's KV head of this segment
    const size_t head = PAGED ? 0 : ((size_t)pc.b * hkv + jc) * (size_t)p.L * ROWB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(p.k) + head, (uint32_t)n * ROWB);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(p.v) + head, (uint32_t)n * ROWB);
    const int mine = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;  // piece tiles w, w+NW, ...

    // fused append: position ap = seq_lens[b] - 1 of this segment receives the new rows.  The wave
    // that owns ap's tile loads the rows' bf16 source now, D / 64 elements of each row per lane;
    // when it computes that tile it converts them to the cache format (spread over all lanes, as
    // the fp8 conversion is long), gathers the 16-byte chunks each lane holds of row ap through
    // LDS, puts them in place of the loaded ones and writes them to the cache.  Under a query-head
    // split the hs segments of one cache head each patch their own copy of the tile, and only the
    // first (j % hs == 0) writes the rows to the cache.
    constexpr int EPL = D / 64;         // elements of each new row per lane
    constexpr int CPRB = ROWB / 16;     // 16-byte cache chunks per row
    int ap_it = -1, ap_row = 0;         // the wave's iteration of ap's tile, and ap's row in it
    const bool ap_store = pc.j % p.hs == 0;  // this segment writes the new rows to the cache
    uint32_t kw = 0, vw = 0;            // this lane's source elements (bf16 bits) of the new rows
    if constexpr (APPEND) {
      const int raw = *(const GQA_CONST int32_t*)(uintptr_t)(p.seq_lens + pc.b);  // scalar load
      const int ap = raw - 1;
      const int rel = (ap >= 0 ? ap / TILE : 0) - tile0;
      if (ap >= 0 && ap < p.L && rel >= 0 && rel < ntiles && rel % NW == w) {
        ap_it = rel / NW;
        ap_row = ap % TILE;
        const size_t row = ((size_t)pc.b * hkv + jc) * D;
        if constexpr (EPL == 2) {
          kw = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.k_new) + row)[l];
          vw = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.v_new) + row)[l];
        } else {
          kw = static_cast<const uint16_t*>(p.k_new)[row + l];
          vw = static_cast<const uint16_t*>(p.v_new)[row + l];
        }
      }
    }

    // paged cache: this sequence's page-table row
    __amdgpu_buffer_rsrc_t rtab = rk;
    if constexpr (PAGED)
      rtab = make_rsrc(p.block_table + (size_t)pc.b * p.max_blocks, (uint32_t)p.max_blocks * 4);

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
      int32_t pg;  // paged cache: page-table entry of the next tile this set receives (in flight)
      int page;    // ... the same entry once loaded (scalar)
    };
    auto tile_start = [&](int it) { return (tile0 + w + it * NW) * TILE; };
    auto load_entry = [&](int it) {  // page-table entry of this wave's tile `it` (every lane the same)
      const uint32_t lpage = (uint32_t)(tile_start(it) >> p.block_shift);
      return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rtab, it < mine ? lpage * 4 : kNoTile, 0, 0);
    };
    auto issue = [&](Regs& R, int it) {
      const bool live = it < mine;
      uint32_t t0 = live ? (uint32_t)tile_start(it) : 0u;
      __amdgpu_buffer_rsrc_t tk = rk, tv = rv;
      if constexpr (PAGED) {
        if (live) {
          const int page = R.page;
          const int lpage = (int)(t0 >> p.block_shift);  // logical page of the tile
          const int rows = min(1 << p.block_shift, n - (lpage << p.block_shift));
          const uint32_t bytes = (uint32_t)page < (uint32_t)p.num_blocks ? (uint32_t)rows * ROWB : 0u;
          const size_t pbase = (((size_t)page * hkv + jc) << p.block_shift) * ROWB;
          tk = make_rsrc(static_cast<const char*>(p.k) + pbase, bytes);
          tv = make_rsrc(static_cast<const char*>(p.v) + pbase, bytes);
          t0 &= (1u << p.block_shift) - 1;  // position within the page
        }
      }
      if constexpr (PAGED) R.pg = load_entry(it + NBUF);
#pragma unroll
      for (int x = 0; x < NK; ++x) {  // 16-byte column block x of this lane's quad, token row r
        const uint32_t off = (t0 + r) * ROWB + x * 64 + q * 16;
        R.k[x] = load16(tk, live ? off : kNoTile);
      }
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        const uint32_t off = t0 * ROWB + (x * 64 + l) * 16;
        R.v[x] = load16(tv, live ? off : kNoTile);
      }
    };

    auto compute = [&](Regs& R, int it) {
      const int t0 = tile_start(it);
      if constexpr (APPEND) {
        if (it == ap_it) {
          // the new rows replace the loaded row ap_row of this tile and are written to the cache
          __amdgpu_buffer_rsrc_t tk = rk, tv = rv;
          uint32_t base = (uint32_t)t0;  // position of the tile's row 0 within the descriptors
          bool ok = true;
          if constexpr (PAGED) {
            const int page = R.page;  // this tile's page (the entry for the set's next tile comes below)
            ok = (uint32_t)page < (uint32_t)p.num_blocks;
            const size_t pbase = (((size_t)page * hkv + jc) << p.block_shift) * ROWB;
            const uint32_t bytes = ok ? (uint32_t)ROWB << p.block_shift : 0u;
            tk = make_rsrc(static_cast<const char*>(p.k) + pbase, bytes);
            tv = make_rsrc(static_cast<const char*>(p.v) + pbase, bytes);
            base &= (1u << p.block_shift) - 1;
            // a page outside the pool is neither written nor patched (the tile reads zeros), and
            // the sequence is counted once (by its first KV head)
            if (!ok && pc.j == 0 && l == 0 && p.skipped)
              __hip_atomic_fetch_add(p.skipped, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if (ok) {
            // this lane's elements in the cache format, into the wave's scratch: K row, then V row
            uint32_t ek = 0, ev = 0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float xk = bf16_bits_to_float((kw >> (16 * e)) & 0xffffu);
              const float xv = bf16_bits_to_float((vw >> (16 * e)) & 0xffffu);
              if constexpr (FP8) {
                ek |= float_to_fp8_e4m3_bits(xk, p.k_enc_descale) << (8 * e);
                ev |= float_to_fp8_e4m3_bits(xv, p.v_enc_descale) << (8 * e);
              } else {
                ek |= float_to_bf16_bits(xk) << (16 * e);
                ev |= float_to_bf16_bits(xv) << (16 * e);
              }
            }
            char* as = ascr + w * 2 * ROWB;
            if constexpr (EPL * ELT == 4) {
              *reinterpret_cast<uint32_t*>(as + 4 * l) = ek;
              *reinterpret_cast<uint32_t*>(as + ROWB + 4 * l) = ev;
            } else if constexpr (EPL * ELT == 2) {
              *reinterpret_cast<uint16_t*>(as + 2 * l) = (uint16_t)ek;
              *reinterpret_cast<uint16_t*>(as + ROWB + 2 * l) = (uint16_t)ev;
            } else {
              *reinterpret_cast<uint8_t*>(as + l) = (uint8_t)ek;
              *reinterpret_cast<uint8_t*>(as + ROWB + l) = (uint8_t)ev;
            }
            if (r == ap_row) {  // K: this lane holds row r, bytes x * 64 + q * 16 of chunk x
#pragma unroll
              for (int x = 0; x < NK; ++x) {
                const u32x4_t c = *reinterpret_cast<const u32x4_t*>(as + x * 64 + q * 16);
                R.k[x] = c;
                if (ap_store) __builtin_amdgcn_raw_buffer_store_b128(c, tk, (base + ap_row) * ROWB + x * 64 + q * 16, 0, 0);
              }
            }
            const int lv = (ap_row * CPRB) % 64, xv = ap_row * CPRB / 64;
            if (l >= lv && l < lv + CPRB) {  // V: lanes lv .. lv + CPRB - 1 hold row ap_row's chunks
              const u32x4_t c = *reinterpret_cast<const u32x4_t*>(as + ROWB + (l - lv) * 16);
#pragma unroll
              for (int x = 0; x < NV; ++x)
                if (x == xv) R.v[x] = c;
              if (ap_store) __builtin_amdgcn_raw_buffer_store_b128(c, tv, base * ROWB + (xv * 64 + l) * 16, 0, 0);
            }
          }
        }
      }
      if constexpr (PAGED) R.page = uniform(R.pg);  // loaded ahead of this tile's data
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
          const int sw = 2 * (row % (D / 16));
          *reinterpret_cast<u32x4_t*>(vt + row * D * 2 + ((2 * ch8) ^ sw) * 16) = fp8x8_to_bf16x8(a[0], a[1]);
          *reinterpret_cast<u32x4_t*>(vt + row * D * 2 + ((2 * ch8 + 1) ^ sw) * 16) = fp8x8_to_bf16x8(a[2], a[3]);
        }
      }
      // -- K operands
      bf16x8_t ak[KS];
#pragma unroll
      for (int x = 0; x < NK; ++x) {
        if constexpr (!FP8) {
          ak[x] = __builtin_bit_cast(bf16x8_t, R.k[x]);
        } else {
          const u32x4_t a = R.k[x];
          ak[2 * x] = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(a[0], a[1]));
          ak[2 * x + 1] = __builtin_bit_cast(bf16x8_t, fp8x8_to_bf16x8(a[2], a[3]));
        }
      }
      // -- scores S^T = K Q^T
      f32x4_t sc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[s], bq[nt][s], acc, 0, 0, 0);
        sc[nt] = acc * p.qk_scale;
      }
      if (t0 + TILE > n) {  // ragged last tile: positions >= n get no weight
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 4 * q + i >= n)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sc[nt][i] = -INFINITY;
      }
      // -- online softmax with a lazy reference maximum: the weights are 2^(s - m_run), and m_run
      //    moves (rescaling the row's sum and output) only when the row's tile maximum exceeds it
      //    by more than 8, so weights stay below 2^8 and, past the first tiles, the rescale is
      //    skipped.  P^T is packed to bf16 (nearest even) in the B-operand layout of PV.
      i16x4_t bp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = fmaxf(fmaxf(sc[nt][0], sc[nt][1]), fmaxf(sc[nt][2], sc[nt][3]));
        mx = wave_max_xor_16_32(mx);
        if (mx > m_run[nt] + 8.f) {  // every tile holds a position below n, so mx is finite
          const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mx);
          m_run[nt] = mx;
          l_run[nt] *= alpha;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
        }
        const float m_ref = m_run[nt];
        uint32_t pk[2];
        float psum = 0.f;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          pk[i2] = pack_bf16x2(__builtin_amdgcn_exp2f(sc[nt][2 * i2] - m_ref),
                               __builtin_amdgcn_exp2f(sc[nt][2 * i2 + 1] - m_ref));
          // sum the weights actually used
          psum += __builtin_bit_cast(float, pk[i2] << 16) + __builtin_bit_cast(float, pk[i2] & 0xffff0000u);
        }
        l_run[nt] += psum;
        bp[nt] = __builtin_bit_cast(i16x4_t, u32x2_t{pk[0], pk[1]});
      }
      // -- O^T += V^T P^T, V^T read transposed from LDS (rows 4q..4q+3 = tokens, column 16m + r)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 4 * q + r / 4;
        const int col = 16 * mt + 4 * (r % 4);
        const int pos = (col / 8) ^ (2 * (row % (D / 16)));
        const uint32_t addr = vt_lds + row * D * 2 + pos * 16 + (col % 8) * 2;
        const i16x4_t av = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS i16x4_t*)(uintptr_t)addr);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bp[nt], o[nt][mt], 0, 0, 0);
      }
    };

    // ---- software pipeline: the loads of the next NBUF - 1 tiles are in flight while this tile is
    //      computed; register set u receives tiles u, u + NBUF, ...  (unrolled by NBUF, so every set
    //      is fixed at compile time)
    Regs R[NBUF];
    if constexpr (PAGED) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) R[u].page = uniform(load_entry(u));
    }
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) issue(R[u], u);
    for (int it = 0; it < mine; it += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (it + u >= mine) break;
        issue(R[(u + NBUF - 1) % NBUF], it + u + NBUF - 1);
        compute(R[u], it + u);
      }
    }

    // ---- wave state -> LDS (canonical layout), then the shared epilogue.  For a segment of two or
    //      three pieces thread 0 reads its counter meanwhile: when every other piece has been
    //      counted, this one is the last and is merged without being published (saving its stores,
    //      their wait and the counter update at the end of the step, where the 70B layer's last
    //      workgroups finish: 142.8 -> 141.5 us).  One query tile only: with four, the registers of
    //      the extra merge would spill.
    const int sg_first = range_owner(pc.s, rg.T, rg.weff), sg_last = range_owner(pc.e - 1, rg.T, rg.weff);
    // the merge-route flags of the workspace header (a scalar load, cached)
    const uint32_t route_flags = ((const GQA_CONST uint32_t*)(uintptr_t)p.header)[kRouteFlagsWord];
    const bool sg_check = NT == 1 && sg_first != sg_last && sg_last - sg_first <= 2 &&
                          !(route_flags & kRouteAlwaysPublish);
    uint32_t arrived = 0;
    if (sg_check && threadIdx.x == 0)
      arrived = __hip_atomic_load(p.counters + pc.b * p.Hkv + pc.j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_run[nt] = wave_sum_xor_16_32(l_run[nt]);
    __syncthreads();  // every wave is done with its V tile: the LDS is reused below
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
    if (threadIdx.x == 0) sh.last = sg_check && arrived == (uint32_t)(sg_last - sg_first);
    __syncthreads();
    const bool known_last = NT == 1 && uniform(sh.last);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    piece_epilogue<GT, D, NW, OutT>(p, ep, rg, pc, sh, known_last, route_flags);
    __syncthreads();  // the epilogue's LDS reads finish before the next piece writes V tiles
  });
}

// ------------------------------------------------------------------------------------------------
// f32 cache: vector-ALU kernel (lane = token for the scores, lane = head-dim column for P V).
// GT >= G query rows are processed; rows g >= G see a zero query and are never stored.
template <int D, int GT, typename OutT, int NW>
__global__ void __launch_bounds__(NW * 64) decode_f32_kernel(Params p) {
  constexpr int TILE = 64;
  constexpr int NTH = NW * 64;
  constexpr int CPL = D / 64;  // output columns per lane
  // loads in flight per lane: a whole key row (KL 16-byte loads) and VL value rows at a time for a
  // small group at head dim 64 (each tile's work is then a chain of load round trips: a tiny step is
  // 16.8 us with eight of each in flight), eight of each otherwise (at head dim 128 the larger sets
  // are not fully unrolled and land in scratch).  The arithmetic and its order do not depend on them.
  constexpr bool kWide = GT <= 4 && D == 64;
  constexpr int KL = kWide ? D / 4 : 8;
  constexpr int VL = kWide ? 32 : 8;
  using Epi = EpiLayout<GT, D, NW>;
  constexpr int QB = GT * D * 4;
  constexpr int PB = NW * GT * TILE * 4;
  constexpr int SMEM = QB + PB > Epi::kBytes ? QB + PB : Epi::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ Shared sh;

  const u32x2_t tag = workspace_tag(p);
  Range rg;
  const bool busy = find_range<TILE, NTH>(p, sh, rg);
  if (!workspace_ok(tag)) {
    refuse_workspace<D, OutT, NTH>(p);
    return;
  }
  zero_empty_rows<D, OutT, NTH>(p);
  if (!busy) return;
  const int w = threadIdx.x / 64;
  const int l = threadIdx.x % 64;
  const int G = p.G;
  float* qs = reinterpret_cast<float*>(smem);
  float* ps = reinterpret_cast<float*>(smem + QB) + w * GT * TILE;
  float* ep = reinterpret_cast<float*>(smem);

  for_each_piece<TILE, NTH>(p, rg, [&](const Piece& pc, int tile0, int ntiles, int n) {
    {
      const float* qg = reinterpret_cast<const float*>(p.q) + ((size_t)pc.b * p.Hq + (size_t)pc.j * G) * D;
      for (int idx = threadIdx.x; idx < GT * D; idx += NTH) qs[idx] = (idx / D < G) ? qg[idx] : 0.f;
    }
    __syncthreads();
    // the host never splits the group on this path (hs = 1), so segment heads are cache heads
    const float* kh = reinterpret_cast<const float*>(p.k) + ((size_t)pc.b * p.Hkv + pc.j) * (size_t)p.L * D;
    const float* vh = reinterpret_cast<const float*>(p.v) + ((size_t)pc.b * p.Hkv + pc.j) * (size_t)p.L * D;

    float m_run[GT], l_run[GT], o[GT][CPL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = 0.f;
#pragma unroll
      for (int x = 0; x < CPL; ++x) o[g][x] = 0.f;
    }

    for (int it = w; it < ntiles; it += NW) {
      const int t0 = (tile0 + it) * TILE;
      const int t = t0 + l;
      const bool valid = t < n;
      float s[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) s[g] = 0.f;
      if (valid) {
        // this lane's key row, KL 16-byte loads in flight at a time
        const float4* kr = reinterpret_cast<const float4*>(kh + (size_t)t * D);
        for (int c0 = 0; c0 < D / 4; c0 += KL) {
          float4 kv[KL];
#pragma unroll
          for (int u = 0; u < KL; ++u) kv[u] = kr[c0 + u];
#pragma unroll
          for (int u = 0; u < KL; ++u)
#pragma unroll
            for (int g = 0; g < GT; ++g) {
              const float4 qv = *reinterpret_cast<const float4*>(qs + g * D + 4 * (c0 + u));
              s[g] += qv.x * kv[u].x + qv.y * kv[u].y + qv.z * kv[u].z + qv.w * kv[u].w;
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
      // value rows in groups of VL, their loads in flight together (rows past the tile's last
      // position are not read)
      const int cnt = min(TILE, n - t0);
      for (int t8 = 0; t8 < cnt; t8 += VL) {
        float vv[VL][CPL];
#pragma unroll
        for (int u = 0; u < VL; ++u)
#pragma unroll
          for (int x = 0; x < CPL; ++x)
            vv[u][x] = t8 + u < cnt ? vh[(size_t)(t0 + t8 + u) * D + 64 * x + l] : 0.f;
#pragma unroll
        for (int u = 0; u < VL; ++u) {
          // rows past the tile's last position: with the wide sets they are not skipped (the loop
          // then unrolls) and add fma(0, 0, o) = o, as their weights and value registers are zero
          if constexpr (!kWide) {
            if (t8 + u >= cnt) break;
          }
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            const float pw = ps[g * TILE + t8 + u];
#pragma unroll
            for (int x = 0; x < CPL; ++x) o[g][x] += pw * vv[u][x];
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) l_run[g] += __shfl_xor(l_run[g], off);

    __syncthreads();
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
    piece_epilogue<GT, D, NW, OutT>(p, ep, rg, pc, sh);
    __syncthreads();
  });
}

// ------------------------------------------------------------------------------------------------
// Workspace initialisation: the header and the whole counter area cleared, then the tag written (a
// kernel rather than a memset so that it may be captured in a graph).  n = words to clear.
__global__ void init_workspace_kernel(uint32_t* ws, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ws[i] = i == 0 ? kWorkspaceTag0 : i == 1 ? kWorkspaceTag1 : 0u;
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
