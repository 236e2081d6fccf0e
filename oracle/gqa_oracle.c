/*
 * gqa_oracle.c -- plain, slow, fp64 CPU oracle for single-token grouped-query-attention decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code, header, table or helper with the HIP library and
 * must never be called on the product path.
 *
 * What it computes (written from the pages, not from any kernel):
 *   - Scaled dot-product attention per query head, unchanged by grouping: score_t = (q . k_t) * scale,
 *     softmax over the cached tokens, output = softmax-weighted sum of the value rows.
 *     ("Grouped Query Attention (GQA): Efficient Multi-Head Attention", Worked example 2; "Llama-2 70B
 *     uses 64 query heads ...", section "What stays the same".)
 *   - Query head h reads KV head floor(h / G) with G = Hq / Hkv, i.e. contiguous groups of G query
 *     heads share one K head and one V head.  ("Grouped-Query Attention: How Sharing KV Heads Shrinks
 *     Inference Memory", section "How grouped-query attention works"; "GQA, decode the acronym ...";
 *     "Llama-2 70B uses 64 query heads ...", section "What the choice does to attention".)
 *   - The decode query attends to the cached K/V of the tokens already in the cache, here exactly the
 *     first seq_lens[b] positions.  ("Grouped Query Attention (GQA): Efficient Multi-Head Attention",
 *     section "The bottleneck: autoregressive decoding ...".)
 *   - KV bytes per token = 2 * layers * kv_heads * head_dim * dtype_bytes.  ("Grouped Query Attention:
 *     Why 8 KV Heads Decide Your Batch Size", section "Why does GQA decide your batch size?".)
 *   - An fp8 KV cache stores 8-bit values with per-tensor scales; real value = stored * descale.
 *     ("Grouped-Query Attention: How Sharing KV Heads Shrinks Inference Memory", section "FP8 KV cache:
 *     the other factor of two".)  The 8-bit format is OCP e4m3fn, decoded here from its definition.
 *
 *   - Paged cache ("Grouped Query Attention: Why 8 KV Heads Decide Your Batch Size", section "What
 *     should you do about it?", names paged allocation as a serving lever, with the PagedAttention
 *     paper among the references of "Grouped-Query Attention: How Sharing KV Heads Shrinks Inference
 *     Memory"): the cache positions of a sequence live in fixed-size pages of block_size positions;
 *     logical page t / block_size of sequence b is physical page block_table[b][t / block_size], and
 *     position t sits at row t % block_size of it.  Pages are laid out [num_blocks][Hkv][block_size][d].
 *     The attention itself is the dense one over the un-paged cache.
 *
 *   - Appending the new token's K and V rows to the cache, converted to the cache's storage format; an
 *     fp8 cache stores the code of the value divided by the per-tensor descale ("Grouped-Query Attention:
 *     How Sharing KV Heads Shrinks Inference Memory", section "FP8 KV cache: the other factor of two").
 *
 *   - Causal prefill over a prompt of S tokens ("Grouped Query Attention: Why 8 KV Heads Decide Your
 *     Batch Size", section "Why doesn't GQA speed up my fine-tuned model?", the scaled_dot_product_attention
 *     call with is_causal and enable_gqa): q [B][Hq][S][d], k and v [B][Hkv][S][d]; query position i
 *     of head h attends to key positions t <= i of KV head floor(h / G) (without the mask: all S).
 *
 * Readings where the pages are silent: seq_len 0 yields an all-zero output row; seq_len outside [0, L]
 * is an error (return code 2); a page-table entry of a live page outside [0, num_blocks) is an error
 * (return code 3) while entries of pages past a sequence's length are never read; the output is
 * returned in fp64 so that the caller's comparison includes
 * whatever rounding the device path applies.
 *
 * Every input element is decoded exactly to double; all accumulation is double, in plain index order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2 };

/* bf16 is the upper 16 bits of an IEEE binary32. */
double gqa_oracle_bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0 is
 * subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN; there is no infinity. */
double gqa_oracle_fp8_e4m3_to_double(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

static int elem_size(int dt) {
  switch (dt) {
    case ORACLE_F32: return 4;
    case ORACLE_BF16: return 2;
    case ORACLE_FP8_E4M3: return 1;
    default: return 0;
  }
}

static double load_elem(const void* base, int dt, size_t idx) {
  switch (dt) {
    case ORACLE_F32: {
      float f;
      memcpy(&f, (const char*)base + idx * 4, 4);
      return (double)f;
    }
    case ORACLE_BF16: {
      uint16_t h;
      memcpy(&h, (const char*)base + idx * 2, 2);
      return gqa_oracle_bf16_to_double(h);
    }
    default: return gqa_oracle_fp8_e4m3_to_double(((const uint8_t*)base)[idx]);
  }
}

uint64_t gqa_oracle_kv_bytes_per_token(uint64_t layers, uint64_t kv_heads, uint64_t head_dim,
                                       uint64_t dtype_bytes) {
  /* one K tensor and one V tensor per layer and per KV head */
  return 2u * layers * kv_heads * head_dim * dtype_bytes;
}

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  int q_dtype, kv_dtype;
  double k_descale, v_descale, scale;
  const int32_t* seq_lens;
  int B, Hq, Hkv, L, d;
  /* paged cache (block_table == NULL: dense [B][Hkv][L][d]) */
  const int32_t* block_table; /* [B][max_blocks] */
  int block_size, max_blocks, num_blocks;
} problem_t;

static int check(const problem_t* p) {
  if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->L < 0 || p->d <= 0) return 1;
  if (p->Hq % p->Hkv != 0) return 1;
  if (!elem_size(p->q_dtype) || !elem_size(p->kv_dtype)) return 1;
  if (p->block_table && (p->block_size <= 0 || p->max_blocks < 0 || p->num_blocks < 0)) return 1;
  for (int b = 0; b < p->B; ++b)
    if (p->seq_lens[b] < 0 || p->seq_lens[b] > p->L) return 2;
  if (p->block_table)
    for (int b = 0; b < p->B; ++b) {
      const int live = (p->seq_lens[b] + p->block_size - 1) / p->block_size;
      for (int i = 0; i < live; ++i) {
        const int32_t pg = p->block_table[(size_t)b * p->max_blocks + i];
        if (pg < 0 || pg >= p->num_blocks) return 3;
      }
    }
  return 0;
}

/* Element index of element 0 of cache row (b, j, t). */
static size_t row_index(const problem_t* p, int b, int j, int t) {
  if (!p->block_table) return (((size_t)b * p->Hkv + j) * (size_t)p->L + (size_t)t) * p->d;
  const size_t page = (size_t)p->block_table[(size_t)b * p->max_blocks + t / p->block_size];
  return ((page * p->Hkv + j) * (size_t)p->block_size + (size_t)(t % p->block_size)) * p->d;
}

/* Softmax weights of query head (b, h) over its n cached tokens, written to w[0..n).  Returns n. */
static int head_weights(const problem_t* p, int b, int h, double* w) {
  const int G = p->Hq / p->Hkv;
  const int j = h / G; /* contiguous grouping */
  const int n = p->seq_lens[b];
  const size_t qbase = ((size_t)b * p->Hq + h) * p->d;
  if (n == 0) return 0;
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    const size_t krow = row_index(p, b, j, t);
    double dot = 0.0;
    for (int c = 0; c < p->d; ++c)
      dot += load_elem(p->q, p->q_dtype, qbase + c) *
             (load_elem(p->k, p->kv_dtype, krow + c) * p->k_descale);
    w[t] = dot * p->scale;
    if (w[t] > m) m = w[t];
  }
  double z = 0.0;
  for (int t = 0; t < n; ++t) {
    w[t] = exp(w[t] - m);
    z += w[t];
  }
  for (int t = 0; t < n; ++t) w[t] /= z;
  return n;
}

static void head_output(const problem_t* p, int b, int h, double* w, double* out_row) {
  const int G = p->Hq / p->Hkv;
  const int j = h / G;
  const int n = head_weights(p, b, h, w);
  for (int c = 0; c < p->d; ++c) {
    double acc = 0.0;
    for (int t = 0; t < n; ++t)
      acc += w[t] * (load_elem(p->v, p->kv_dtype, row_index(p, b, j, t) + c) * p->v_descale);
    out_row[c] = acc; /* n == 0 leaves the row at zero */
  }
}

#define FILL_PROBLEM                                                                            \
  problem_t p;                                                                                  \
  p.q = q; p.k = k; p.v = v; p.q_dtype = q_dtype; p.kv_dtype = kv_dtype;                        \
  p.k_descale = k_descale; p.v_descale = v_descale; p.scale = scale; p.seq_lens = seq_lens;     \
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.d = d;                                          \
  p.block_table = NULL; p.block_size = 0; p.max_blocks = 0; p.num_blocks = 0;

/* Full decode: out[B, Hq, d] (fp64).  w_scratch must hold L doubles.  Returns 0, 1 (bad shape or
 * dtype) or 2 (a seq_len outside [0, L]). */
int gqa_oracle_decode(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                      double k_descale, double v_descale, const int32_t* seq_lens, double scale,
                      int B, int Hq, int Hkv, int L, int d, double* w_scratch, double* out) {
  FILL_PROBLEM
  int rc = check(&p);
  if (rc) return rc;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h) head_output(&p, b, h, w_scratch, out + ((size_t)b * Hq + h) * d);
  return 0;
}

/* Selected rows only: rows holds nrows pairs (b, h); out is [nrows, d]. */
int gqa_oracle_decode_rows(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                           double k_descale, double v_descale, const int32_t* seq_lens, double scale,
                           int B, int Hq, int Hkv, int L, int d, const int32_t* rows, int nrows,
                           double* w_scratch, double* out) {
  FILL_PROBLEM
  int rc = check(&p);
  if (rc) return rc;
  for (int r = 0; r < nrows; ++r) {
    int b = rows[2 * r], h = rows[2 * r + 1];
    if (b < 0 || b >= B || h < 0 || h >= Hq) return 1;
    head_output(&p, b, h, w_scratch, out + (size_t)r * d);
  }
  return 0;
}

/* Softmax weights of one query head (b, h): w[0..seq_lens[b]).  Returns the count, or -1/-2. */
int gqa_oracle_weights(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype,
                       double k_descale, double v_descale, const int32_t* seq_lens, double scale,
                       int B, int Hq, int Hkv, int L, int d, int b, int h, double* w) {
  FILL_PROBLEM
  int rc = check(&p);
  if (rc) return -rc;
  if (b < 0 || b >= B || h < 0 || h >= Hq) return -1;
  return head_weights(&p, b, h, w);
}

/* Paged cache: k_pages, v_pages are [num_blocks][Hkv][block_size][d]; block_table is [B][max_blocks];
 * sequences hold at most L = max_blocks * block_size positions.  rows == NULL computes every (b, h) into
 * out[B, Hq, d]; otherwise only the nrows listed (b, h) pairs into out[nrows, d].  w_scratch holds L
 * doubles.  Returns 0, 1 (bad shape or dtype), 2 (a seq_len outside [0, L]) or 3 (a live page-table
 * entry outside [0, num_blocks)). */
int gqa_oracle_decode_paged(const void* q, int q_dtype, const void* k_pages, const void* v_pages,
                            int kv_dtype, double k_descale, double v_descale,
                            const int32_t* block_table, const int32_t* seq_lens, double scale, int B,
                            int Hq, int Hkv, int block_size, int max_blocks, int num_blocks, int d,
                            const int32_t* rows, int nrows, double* w_scratch, double* out) {
  problem_t p;
  p.q = q; p.k = k_pages; p.v = v_pages; p.q_dtype = q_dtype; p.kv_dtype = kv_dtype;
  p.k_descale = k_descale; p.v_descale = v_descale; p.scale = scale; p.seq_lens = seq_lens;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.d = d;
  p.block_table = block_table; p.block_size = block_size; p.max_blocks = max_blocks;
  p.num_blocks = num_blocks;
  p.L = (block_size > 0 && max_blocks >= 0) ? block_size * max_blocks : -1;
  int rc = check(&p);
  if (rc) return rc;
  if (!rows) {
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < Hq; ++h) head_output(&p, b, h, w_scratch, out + ((size_t)b * Hq + h) * d);
    return 0;
  }
  for (int r = 0; r < nrows; ++r) {
    int b = rows[2 * r], h = rows[2 * r + 1];
    if (b < 0 || b >= B || h < 0 || h >= Hq) return 1;
    head_output(&p, b, h, w_scratch, out + (size_t)r * d);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Encoders (storage format of a value), written from the format definitions.
 *
 * bf16: the bf16 value nearest to the binary32 input, ties to the even bit pattern (round to nearest
 *       even, overflowing to infinity as binary formats do); infinities stay; NaN becomes the quiet
 *       NaN 0x7FC0 with the input's sign.
 * fp8 e4m3fn: the input is first divided by the descale in binary32 (correctly rounded, as C does
 *       it), then mapped to the finite e4m3fn value nearest to the quotient, found by trying every
 *       code; ties go to the code with an even mantissa, and between +0 and -0 to the quotient's sign.
 *       Values beyond the largest finite value 448 (infinities included) therefore saturate to +-448.
 *       A NaN input becomes 0x7F with the input's sign bit. */
uint16_t gqa_oracle_encode_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(x)) return (uint16_t)(0x7FC0u | sign);
  if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
  /* candidates: the two bf16 patterns around x (truncation and the next one up in magnitude) */
  const uint16_t lo = (uint16_t)(u >> 16);
  const uint16_t hi = (uint16_t)(lo + 1);
  const double dx = (double)x;
  const double dlo = gqa_oracle_bf16_to_double(lo);
  /* past the largest finite value the next pattern is infinity, which rounding treats as 2^128
   * (the exponent range taken as unbounded), so large enough inputs round to infinity */
  const double dhi = ((hi & 0x7FFFu) == 0x7F80u) ? copysign(ldexp(1.0, 128), dx) : gqa_oracle_bf16_to_double(hi);
  const double elo = fabs(dx - dlo), ehi = fabs(dx - dhi);
  if (elo < ehi) return lo;
  if (ehi < elo) return hi;
  return (lo & 1u) ? hi : lo; /* tie: even pattern */
}

uint8_t gqa_oracle_encode_fp8_e4m3(float x, float descale) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint8_t)(0x7Fu | ((u >> 31) ? 0x80u : 0u));
  const float y = x / descale; /* binary32, correctly rounded */
  memcpy(&u, &y, 4);
  const int neg = (int)(u >> 31);
  /* at or past the largest finite value 448 the nearest finite value is +-448 (checked here so that
   * the distances below stay exact: they are, for |y| < 448, in double) */
  if (fabs((double)y) >= 448.0) return (uint8_t)(neg ? 0xFEu : 0x7Eu);
  int best = -1;
  double best_err = 0.0;
  for (int c = 0; c < 256; ++c) {
    const double v = gqa_oracle_fp8_e4m3_to_double((uint8_t)c);
    if (isnan(v)) continue;
    const double err = fabs((double)y - v);
    if (best < 0 || err < best_err) {
      best = c;
      best_err = err;
    } else if (err == best_err) {
      const double vb = gqa_oracle_fp8_e4m3_to_double((uint8_t)best);
      if (v == vb) { /* +0 and -0: keep the quotient's sign */
        if (((c >> 7) & 1) == neg) best = c;
      } else if ((best & 1) && !(c & 1)) { /* a true tie between neighbours: even mantissa */
        best = c;
      }
    }
  }
  return (uint8_t)best;
}

/* Appends one row per (sequence, KV head): row (b, j) of k_new / v_new ([B][Hkv][d], new_dtype f32 or
 * bf16) is stored, in the cache's format, at position positions[b] of sequence b's cache (dense
 * [B][Hkv][L][d] when block_table is NULL, else pages [num_blocks][Hkv][block_size][d]).  A negative
 * position skips the sequence; a position >= L, or one whose page-table entry lies outside
 * [0, num_blocks), is not written and is counted.  Returns the count of such sequences, or -1 for bad
 * arguments.  Nothing else in the cache changes. */
int gqa_oracle_append(const void* k_new, const void* v_new, int new_dtype, void* k_cache, void* v_cache,
                      int kv_dtype, double k_descale, double v_descale, const int32_t* positions, int B,
                      int Hkv, int L, int d, const int32_t* block_table, int block_size, int max_blocks,
                      int num_blocks) {
  if (B < 0 || Hkv <= 0 || d <= 0 || L < 0) return -1;
  if (new_dtype != ORACLE_F32 && new_dtype != ORACLE_BF16) return -1;
  if (!elem_size(kv_dtype)) return -1;
  if (block_table && (block_size <= 0 || max_blocks < 0 || num_blocks < 0)) return -1;
  const int esz = elem_size(kv_dtype);
  int skipped = 0;
  for (int b = 0; b < B; ++b) {
    const int t = positions[b];
    if (t < 0) continue;
    if (t >= L) {
      ++skipped;
      continue;
    }
    size_t page = 0;
    if (block_table) {
      const int32_t pg = block_table[(size_t)b * max_blocks + t / block_size];
      if (pg < 0 || pg >= num_blocks) {
        ++skipped;
        continue;
      }
      page = (size_t)pg;
    }
    for (int j = 0; j < Hkv; ++j) {
      const size_t row = block_table
          ? ((page * Hkv + j) * (size_t)block_size + (size_t)(t % block_size)) * d
          : (((size_t)b * Hkv + j) * (size_t)L + (size_t)t) * d;
      for (int c = 0; c < d; ++c) {
        const size_t src = ((size_t)b * Hkv + j) * d + c;
        for (int kv = 0; kv < 2; ++kv) {
          const void* in = kv ? v_new : k_new;
          void* cache = kv ? v_cache : k_cache;
          const double descale = kv ? v_descale : k_descale;
          const float x = (float)load_elem(in, new_dtype, src); /* exact: f32 or bf16 input */
          char* dst = (char*)cache + (row + c) * esz;
          if (kv_dtype == ORACLE_F32) {
            memcpy(dst, &x, 4);
          } else if (kv_dtype == ORACLE_BF16) {
            const uint16_t h = gqa_oracle_encode_bf16(x);
            memcpy(dst, &h, 2);
          } else {
            *(uint8_t*)dst = gqa_oracle_encode_fp8_e4m3(x, (float)descale);
          }
        }
      }
    }
  }
  return skipped;
}

/* ------------------------------------------------------------------------------------------------
 * Prefill: out[b][h][i][:] = sum over t < n_i of softmax_t(scale * q[b][h][i] . k[b][j][t]) v[b][j][t],
 * j = floor(h / G), n_i = i + 1 when causal, else S.  rows == NULL: every (b, h, i) into out
 * [B][Hq][S][d]; otherwise the nrows listed triples (b, h, i) into out [nrows][d].  w_scratch holds S
 * doubles.  Returns 0 or 1 (bad arguments). */
int gqa_oracle_prefill(const void* q, const void* k, const void* v, int dtype, double scale, int causal,
                       int B, int Hq, int Hkv, int S, int d, const int32_t* rows, int nrows,
                       double* w_scratch, double* out) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || d <= 0 || Hq % Hkv != 0 || !elem_size(dtype)) return 1;
  const int G = Hq / Hkv;
  const long long total = rows ? nrows : (long long)B * Hq * S;
  for (long long r = 0; r < total; ++r) {
    int b, h, i;
    if (rows) {
      b = rows[3 * r];
      h = rows[3 * r + 1];
      i = rows[3 * r + 2];
      if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= S) return 1;
    } else {
      b = (int)(r / ((long long)Hq * S));
      h = (int)((r / S) % Hq);
      i = (int)(r % S);
    }
    const int j = h / G;
    const int n = causal ? i + 1 : S;
    const size_t qrow = (((size_t)b * Hq + h) * (size_t)S + (size_t)i) * d;
    const size_t kvbase = ((size_t)b * Hkv + j) * (size_t)S * d;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
      double dot = 0.0;
      for (int c = 0; c < d; ++c)
        dot += load_elem(q, dtype, qrow + c) * load_elem(k, dtype, kvbase + (size_t)t * d + c);
      w_scratch[t] = dot * scale;
      if (w_scratch[t] > m) m = w_scratch[t];
    }
    double z = 0.0;
    for (int t = 0; t < n; ++t) {
      w_scratch[t] = exp(w_scratch[t] - m);
      z += w_scratch[t];
    }
    double* o = out + (size_t)r * d;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int t = 0; t < n; ++t) acc += (w_scratch[t] / z) * load_elem(v, dtype, kvbase + (size_t)t * d + c);
      o[c] = acc;
    }
  }
  return 0;
}
