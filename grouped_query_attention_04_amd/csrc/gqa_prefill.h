// gqa_prefill.h -- HIP kernel (gfx950 / CDNA4) for grouped-query-attention prefill over a prompt.
//
// The arithmetic is the scaled_dot_product_attention call with is_causal and enable_gqa of "Grouped
// Query Attention: Why 8 KV Heads Decide Your Batch Size" (section "Why doesn't GQA speed up my
// fine-tuned model?"): query position i of head h attends to key positions t <= i of KV head
// floor(h / G), softmax-weighted over the values.  Unlike decode this is a dense contraction, run on
// the matrix cores.
//
// Work decomposition.  A workgroup owns one (batch b, KV head j, block of BM query positions) and all
// G query heads of the group, so every K/V tile it stages in LDS serves G heads at once -- the
// grouping is used, not expanded (same page, the repeat_kv discussion).  Its 256 rows (G heads x BM
// positions, BM = floor(256 / G), and 256 - G * BM padding rows when G does not divide 256) are split
// over NW waves of NT 16-row tiles each.  Keys are taken
// in blocks of KB through two LDS buffers: while the waves compute on one block, the next one is
// being stored into the other, and the global loads of the block after it are in flight in
// registers.
//
// Per block and wave (lane l, quad q = l / 16, r = l % 16):
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16, one product per 16-key quarter; A = K rows from LDS,
//   B = the wave's query rows (registers).  Lane l holds S[row r][key 16h + 4q + i] of quarter h.
//   O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with each 32-key slab as the contraction: k-slot
//   8q + e is key 4q + e (e < 4) or 16 + 4q + (e - 4) (e >= 4) of the slab, so P^T's B operand is
//   the lane's own eight probabilities, and A = V^T comes from two ds_read_b64_tr_b16 of the V tile.
//   Lane l holds O[row r][d = 16m + 4q + i]; the row's running max lives in the same lanes, and its
//   running sum of (bf16) weights is one more PV product with an all-ones V^T tile.
//   The running max is moved lazily: only when some score of the wave exceeds its row's reference
//   by more than 8 (base 2) are the row maxima reduced and the outputs rescaled, so weights stay
//   below 2^8 and most blocks skip both.  The scale's sign is folded into q by the launcher, so the
//   multiplier applied in the exponent is positive and raw-score maxima are scaled-score maxima.
//
// Latency.  Each wave reads the K fragments of the next 16-key quarter, and all V^T fragments of a
// slab, before it issues the products that use them, so one LDS round trip is paid per group of
// products rather than per product.  The kernel declares its real occupancy (two waves per SIMD:
// one 512-thread workgroup per CU), so that the compiler spends the registers on that read-ahead
// instead of squeezing for an occupancy the workgroup size cannot reach.
#pragma once

#include <type_traits>

#include "gqa_device.h"

namespace gqa {

// Maximum over the four lanes l, l^16, l^32, l^48 (the four quads holding one matrix column).
// v_permlane16_swap(x, x) hands back x of rows {0,0,2,2} and {1,1,3,3} (rows of 16 lanes), and
// v_permlane32_swap(x, x) x of halves {0,0} and {1,1}: the larger of each pair pairs lane l with
// l^16, respectively l^32, without a trip through LDS.  Every lane ends with the same value.  The
// maximum propagates NaN (a NaN score makes NaN weights either way) and so needs no quieting of its
// operands.
__device__ __forceinline__ float quad_max_permlane(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)c[0]), __builtin_bit_cast(float, (uint32_t)c[1]));
}

struct PrefillParams {
  const void* q;  // [B][Hq][S][D] bf16
  const void* k;  // [B][Hkv][S][D] bf16
  const void* v;
  void* out;      // [B][Hq][S][D] OutT
  int B, Hq, Hkv, S, G;
  int bm;         // BM = floor(256 / G) query positions per workgroup (BM * G <= 256 rows)
  int nqb;        // query blocks per (b, j)
  float qk_scale; // |scale| * log2(e), positive (1 * log2(e) for a zero scale)
  uint32_t q_and; // applied to each 32-bit word (two bf16) of q: all ones, or 0 for a zero scale
  uint32_t q_xor; // then: 0, or 0x80008000 (both signs) for a negative scale
};

template <int D, typename OutT, bool CAUSAL, int NW, int NT, int KB>
__global__ void __launch_bounds__(NW * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_mfma_kernel(PrefillParams p) {
  static_assert(NW * NT * 16 == 256, "a workgroup covers 256 rows");
  static_assert(KB % 32 == 0, "keys per block: a multiple of 32");
  constexpr int NTH = NW * 64;
  constexpr int RW = 16 * NT;           // rows per wave
  constexpr int NQ = KB / 16;           // 16-key quarters of a block (S^T tiles)
  constexpr int NS = KB / 32;           // 32-key slabs of a block (PV contractions)
  constexpr int KS = D / 32;            // k-steps of QK^T
  constexpr int MT = D / 16;            // m-tiles of PV (head-dim columns)
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILEB = KB * ROWB;      // bytes of one K (or V) block
  constexpr int NLD = (TILEB / 16 + NTH - 1) / NTH;  // 16-byte loads per thread per block and tensor
  __shared__ __attribute__((aligned(16))) char ks[2][TILEB];
  __shared__ __attribute__((aligned(16))) char vs[2][TILEB];

  // heaviest query blocks first: block index -> (query block, batch, KV head)
  const int nbj = p.B * p.Hkv;
  const int qb = p.nqb - 1 - (int)(blockIdx.x / nbj);
  const int bj = (int)(blockIdx.x % nbj);
  const int b = bj / p.Hkv, j = bj % p.Hkv;
  const int BM = p.bm;
  const int nrows = p.G * BM;  // rows of the workgroup that hold a (head, position); 256 - nrows pad
  const int w = uniform((int)threadIdx.x / 64);
  const int l = threadIdx.x % 64;
  const int q = l / 16;
  const int r = l % 16;

  // the wave's rows: row rho = RW w + 16 nt + r is head g = rho / BM, position qb * BM + rho % BM;
  // rows past nrows (when G does not divide 256) are padding: position S, a zero query, never stored
  int pos[NT];
  int head[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rho = RW * w + 16 * nt + r;
    head[nt] = j * p.G + (rho < nrows ? rho / BM : 0);
    pos[nt] = rho < nrows ? qb * BM + rho % BM : p.S;
  }
  // positions covered by the wave (for skipping blocks it cannot see): its real rows r0 .. r1 cover
  // positions r0 % BM .. r1 % BM of one head, or (when they cross to the next head) the whole block
  const int r0 = RW * w, r1 = min(RW * w + RW, nrows) - 1;
  int lo_rel = 0, hi_rel = -1;  // no real row: every block is skipped
  if (r1 >= r0) {
    if (r0 / BM == r1 / BM) {
      lo_rel = r0 % BM;
      hi_rel = r1 % BM;
    } else {
      lo_rel = 0;
      hi_rel = BM - 1;
    }
  }
  const int wave_lo = uniform(qb * BM + lo_rel);
  const int wave_hi = uniform(hi_rel < 0 ? -1 : min(p.S - 1, qb * BM + hi_rel));
  const int wg_hi = min(p.S, (qb + 1) * BM);  // exclusive
  const int nkb = CAUSAL ? (wg_hi + KB - 1) / KB : (p.S + KB - 1) / KB;

  // query rows in the B-operand layout of QK^T (zero for positions past the prompt)
  bf16x8_t bq[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (((size_t)b * p.Hq + head[nt]) * p.S + pos[nt]) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t v = {0, 0, 0, 0};
      if (pos[nt] < p.S) v = *reinterpret_cast<const u32x4_t*>(qr + 32 * s + 8 * q);
      // the scale's sign goes into q (exact), so the multiplier below is positive and a row's
      // largest raw score is its largest scaled score
      v = (v & p.q_and) ^ p.q_xor;
      bq[nt][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // K/V blocks of this (b, j): buffer descriptors over the prompt (keys past S read as zero)
  const size_t head_off = ((size_t)b * p.Hkv + j) * (size_t)p.S * ROWB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(p.k) + head_off, (uint32_t)p.S * ROWB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(p.v) + head_off, (uint32_t)p.S * ROWB);
  // LDS placement: K chunk c of key row x at chunk c ^ (x % CPR); V as in the decode kernel's tile
  auto store_k = [&](char* dst, const u32x4_t* src) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + NTH * u;
      if (idx >= TILEB / 16) break;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4_t*>(dst + row * ROWB + ((ch ^ (row % CPR)) * 16)) = src[u];
    }
  };
  auto store_v = [&](char* dst, const u32x4_t* src) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = threadIdx.x + NTH * u;
      if (idx >= TILEB / 16) break;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4_t*>(dst + row * ROWB + ((ch ^ (2 * (row % (D / 16)))) * 16)) = src[u];
    }
  };
  auto chunk_off = [&](int blk, int u) __attribute__((always_inline)) {
    const int idx = threadIdx.x + NTH * u;
    return idx < TILEB / 16 ? (uint32_t)blk * TILEB + idx * 16 : kNoTile;
  };
  u32x4_t ldk[2][NLD], ldv[2][NLD];
  auto load_block = [&](int kb, auto setc) __attribute__((always_inline)) {
    constexpr int st = decltype(setc)::value;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      ldk[st][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, chunk_off(kb, u), 0, 0));
      ldv[st][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, chunk_off(kb, u), 0, 0));
    }
  };

  float m_run[NT];      // reference maximum per row, base-2 scaled domain
  float neg_m[NT];      // -m_run, or 0 while the row has seen no key (the exponent's offset)
  f32x4_t lsum[NT];     // running sum of the weights (every element holds the row's sum)
  f32x4_t o[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    neg_m[nt] = 0.f;
    lsum[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  // Lane parts of the LDS read addresses; quarter, slab and half add compile-time offsets.
  // K: quarter h, k-step s reads chunk (4s + q) of key row 16h + r, stored at chunk (4s + q) ^ (r % CPR).
  // V^T: slab sl, half hf, m-tile mt reads columns 16mt + 4(r % 4) .. + 3 of key row
  // 32sl + 16hf + 4q + r / 4, whose row index modulo D / 16 does not depend on sl or hf.
  uint32_t koff[KS], voff[MT];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = r * ROWB + (((4 * s + q) ^ (r % CPR)) * 16);
  {
    const int vrow = 4 * q + r / 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int col = 16 * mt + 4 * (r % 4);
      voff[mt] = vrow * ROWB + (((col / 8) ^ (2 * (vrow % (D / 16)))) * 16) + (col % 8) * 2;
    }
  }
  f32x4_t sc[NQ][NT];   // scores S^T of the block in flight
  bf16x8_t bp[NS][NT];  // its weights P^T in the B-operand layout of PV (k-slot 8q + e, see the header)

  // -- S^T = K Q^T for the 16-key quarters of the block in LDS buffer kt_lds
  auto qk = [&](const char* kt_lds) __attribute__((always_inline)) {
    bf16x8_t ak[2][KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) ak[0][s] = *reinterpret_cast<const bf16x8_t*>(kt_lds + koff[s]);
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) {
      if (hf + 1 < NQ) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          ak[(hf + 1) & 1][s] = *reinterpret_cast<const bf16x8_t*>(kt_lds + 16 * (hf + 1) * ROWB + koff[s]);
      }
      __builtin_amdgcn_sched_barrier(0);  // the next quarter's reads are in flight during these products
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[hf & 1][s], bq[nt][s], acc, 0, 0, 0);
        sc[hf][nt] = acc;  // unscaled: the scale is applied in the exponent
      }
    }
  };
  // -- masks, online softmax (lazy rescale of o and lsum), weights P^T of block kb
  auto softmax = [&](int kb) __attribute__((always_inline)) {
    const int k0 = kb * KB;
    if ((CAUSAL && k0 + KB - 1 > wave_lo) || k0 + KB > p.S) {
      if (CAUSAL) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // keys 16h + i of this lane's quarter columns are visible while 16h + i <= lim
          const int lim = min(pos[nt], p.S - 1) - (k0 + 4 * q);
#pragma unroll
          for (int hf = 0; hf < NQ; ++hf) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * hf + i > lim) sc[hf][nt][i] = -INFINITY;
            // four compares at a time: hoisting them all would hold a scalar register pair each
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 16 * hf + 4 * q + i >= p.S)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) sc[hf][nt][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // This lane's maximum decides whether the reference moves (some score of the wave more than
      // 8 above its row's reference); only then is the row maximum reduced across the quads.
      float mx = -INFINITY;  // NaN-propagating, as in quad_max_permlane
#pragma unroll
      for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = __builtin_elementwise_maximum(mx, sc[hf][nt][i]);
      if (__any(mx * p.qk_scale > m_run[nt] + 8.f)) {  // move the reference maximum (every lane)
        const float m_new = fmaxf(m_run[nt], quad_max_permlane(mx) * p.qk_scale);
        // a row that has seen no key yet (m_new = -inf) keeps alpha = 1
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
        m_run[nt] = m_new;
        neg_m[nt] = m_new == -INFINITY ? 0.f : -m_new;
        lsum[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
      }
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        uint32_t pk[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const f32x4_t& x = sc[2 * sl + h2][nt];
            pk[2 * h2 + i2] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i2], p.qk_scale, neg_m[nt])),
                                          __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * i2 + 1], p.qk_scale, neg_m[nt])));
          }
        bp[sl][nt] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
      }
    }
  };
  // -- O^T += V^T P^T and the row sums, for the block whose V is in LDS buffer vt: V^T rows 16m + r,
  // keys 4q..4q+3 and 16+4q..16+4q+3 of each 32-key slab (two transposed reads).  Each slab's eight
  // fragments are read ahead of its products, so that the LDS latency is paid once per slab; the
  // first slab's are read before the softmax, so that their latency hides behind the exponentials.
  bf16x8_t av[MT];
  auto read_v = [&](const char* vt, int sl) __attribute__((always_inline)) {
    const uint32_t vt_lds = (uint32_t)(uintptr_t)(GQA_LDS const char*)vt;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      i16x4_t part[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t addr = vt_lds + (32 * sl + 16 * hf) * ROWB + voff[mt];
        part[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS i16x4_t*)(uintptr_t)addr);
      }
      av[mt] = __builtin_bit_cast(bf16x8_t, u32x4_t{
          __builtin_bit_cast(u32x2_t, part[0])[0], __builtin_bit_cast(u32x2_t, part[0])[1],
          __builtin_bit_cast(u32x2_t, part[1])[0], __builtin_bit_cast(u32x2_t, part[1])[1]});
    }
  };
  auto pv = [&](const char* vt) __attribute__((always_inline)) {  // slab 0's fragments already in av
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      if (sl > 0) read_v(vt, sl);
      __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) lsum[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bp[sl][nt], lsum[nt], 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bp[sl][nt], o[nt][mt], 0, 0, 0);
    }
  };

  // ---- key blocks through two LDS buffers, global loads two blocks ahead
  load_block(0, std::integral_constant<int, 0>{});
  if (1 < nkb) load_block(1, std::integral_constant<int, 1>{});
  store_k(ks[0], ldk[0]);
  store_v(vs[0], ldv[0]);
  __syncthreads();
  auto step = [&](int kb, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;  // kb % 2: block kb + 1 sits in set 1 - P, kb + 2 goes to set P
    if (kb + 2 < nkb) load_block(kb + 2, par);
    if (!CAUSAL || kb * KB <= wave_hi) {
      qk(ks[P]);
      read_v(vs[P], 0);
      softmax(kb);
      pv(vs[P]);
    }
    if (kb + 1 < nkb) {
      store_k(ks[1 - P], ldk[1 - P]);
      store_v(vs[1 - P], ldv[1 - P]);
    }
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, std::integral_constant<int, 0>{});
    if (kb + 1 >= nkb) break;
    step(kb + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and store the wave's rows
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (pos[nt] >= p.S) continue;
    OutT* orow = static_cast<OutT*>(p.out) + (((size_t)b * p.Hq + head[nt]) * p.S + pos[nt]) * D;
    const float inv = 1.f / lsum[nt][0];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_out4(orow + 16 * mt + 4 * q, o[nt][mt] * inv);
  }
}

}  // namespace gqa
