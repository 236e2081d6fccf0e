// gqa_prefill_api.hip -- host side of libgqa's prefill: argument validation and dispatch of the
// causal (or full) GQA prefill kernel of gqa_prefill.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gqa.h"
#include "gqa_host.h"
#include "gqa_prefill.h"

namespace {

using gqa_host::aligned;
using gqa_host::known_dtype;

constexpr int kPrefillWaves = 8;  // waves per prefill workgroup (256 rows: 16 * 16 / waves each)
constexpr int kPrefillKeys = 64;  // keys per prefill LDS block

}  // namespace

extern "C" {

gqa_status_t gqa_prefill_shape_check(const gqa_prefill_shape_t* s) {
  if (!s) return GQA_ERR_INVALID_ARG;
  if (s->B <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->S <= 0 || s->d <= 0) return GQA_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return GQA_ERR_INVALID_ARG;
  if (!known_dtype(s->dtype) || !known_dtype(s->out_dtype)) return GQA_ERR_INVALID_ARG;
  if (s->causal != 0 && s->causal != 1) return GQA_ERR_INVALID_ARG;
  if (s->dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (s->out_dtype != GQA_BF16 && s->out_dtype != GQA_F32) return GQA_ERR_UNSUPPORTED;
  if (s->d != 64 && s->d != 128) return GQA_ERR_UNSUPPORTED;
  const int G = s->Hq / s->Hkv;
  if (G > 64) return GQA_ERR_UNSUPPORTED;  // any group size up to 64 query heads per KV head
  // per-(batch, KV head) K/V slices are addressed with 32-bit byte offsets
  if ((long long)s->S * s->d * 2 >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  const long long nqb = ((long long)s->S + 256 / G - 1) / (256 / G);
  if (nqb * s->B * s->Hkv >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

gqa_status_t gqa_prefill(const void* q, const void* k, const void* v, float scale, void* out,
                         const gqa_prefill_shape_t* s, void* stream) {
  if (!q || !k || !v || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_prefill_shape_check(s);
  if (st != GQA_OK) return st;
  gqa::PrefillParams pp;
  pp.q = q;
  pp.k = k;
  pp.v = v;
  pp.out = out;
  pp.B = s->B;
  pp.Hq = s->Hq;
  pp.Hkv = s->Hkv;
  pp.S = s->S;
  pp.G = s->Hq / s->Hkv;
  pp.bm = 256 / pp.G;  // query positions per workgroup: G * BM <= 256 rows
  pp.nqb = (s->S + pp.bm - 1) / pp.bm;
  // The kernel takes row maxima before applying the multiplier, so it needs a positive one: a
  // negative scale runs as -q with |scale| (negating bf16 is exact), a zero scale as q = 0 (every
  // score exactly 0, uniform weights over the visible keys).
  pp.q_and = scale == 0.f ? 0u : 0xFFFFFFFFu;
  pp.q_xor = scale < 0.f ? 0x80008000u : 0u;
  pp.qk_scale = (float)((scale == 0.f ? 1.0 : std::fabs((double)scale)) * 1.4426950408889634);
  const unsigned grid = (unsigned)pp.nqb * (unsigned)(s->B * s->Hkv);
  hipStream_t hs = (hipStream_t)stream;
  constexpr int NW = kPrefillWaves, NT = 16 / kPrefillWaves, KB = kPrefillKeys;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(NW * 64), 0, hs, pp);
    return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
  };
  const bool bf = s->out_dtype == GQA_BF16;
  if (s->d == 64) {
    if (s->causal)
      return bf ? go(gqa::prefill_mfma_kernel<64, uint16_t, true, NW, NT, KB>)
                : go(gqa::prefill_mfma_kernel<64, float, true, NW, NT, KB>);
    return bf ? go(gqa::prefill_mfma_kernel<64, uint16_t, false, NW, NT, KB>)
              : go(gqa::prefill_mfma_kernel<64, float, false, NW, NT, KB>);
  }
  if (s->causal)
    return bf ? go(gqa::prefill_mfma_kernel<128, uint16_t, true, NW, NT, KB>)
              : go(gqa::prefill_mfma_kernel<128, float, true, NW, NT, KB>);
  return bf ? go(gqa::prefill_mfma_kernel<128, uint16_t, false, NW, NT, KB>)
            : go(gqa::prefill_mfma_kernel<128, float, false, NW, NT, KB>);
}

}  // extern "C"
