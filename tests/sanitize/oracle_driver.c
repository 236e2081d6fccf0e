/* Exercises every entry point of the C oracle on small and degenerate inputs, in buffers of exactly
 * the documented sizes, so that an AddressSanitizer / UndefinedBehaviorSanitizer build reports any
 * out-of-bounds access, use of uninitialised scratch or undefined arithmetic.  Values are checked by
 * the pinned tests; here only the documented return codes are.  Exit status 0 = every call behaved. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double gqa_oracle_bf16_to_double(uint16_t h);
double gqa_oracle_fp8_e4m3_to_double(uint8_t c);
uint64_t gqa_oracle_kv_bytes_per_token(uint64_t layers, uint64_t kv_heads, uint64_t head_dim, uint64_t dtype_bytes);
int gqa_oracle_decode(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, double k_descale,
                      double v_descale, const int32_t* seq_lens, double scale, int B, int Hq, int Hkv, int L, int d,
                      double* w_scratch, double* out);
int gqa_oracle_decode_rows(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, double k_descale,
                           double v_descale, const int32_t* seq_lens, double scale, int B, int Hq, int Hkv, int L,
                           int d, const int32_t* rows, int nrows, double* w_scratch, double* out);
int gqa_oracle_weights(const void* q, int q_dtype, const void* k, const void* v, int kv_dtype, double k_descale,
                       double v_descale, const int32_t* seq_lens, double scale, int B, int Hq, int Hkv, int L, int d,
                       int b, int h, double* w);
int gqa_oracle_decode_paged(const void* q, int q_dtype, const void* k_pages, const void* v_pages, int kv_dtype,
                            double k_descale, double v_descale, const int32_t* block_table, const int32_t* seq_lens,
                            double scale, int B, int Hq, int Hkv, int block_size, int max_blocks, int num_blocks,
                            int d, const int32_t* rows, int nrows, double* w_scratch, double* out);
uint16_t gqa_oracle_encode_bf16(float x);
uint8_t gqa_oracle_encode_fp8_e4m3(float x, float descale);
int gqa_oracle_append(const void* k_new, const void* v_new, int new_dtype, void* k_cache, void* v_cache,
                      int kv_dtype, double k_descale, double v_descale, const int32_t* positions, int B, int Hkv,
                      int L, int d, const int32_t* block_table, int block_size, int max_blocks, int num_blocks);
int gqa_oracle_prefill(const void* q, const void* k, const void* v, int dtype, double scale, int causal, int B,
                       int Hq, int Hkv, int S, int d, const int32_t* rows, int nrows, double* w_scratch,
                       double* out);

enum { F32 = 0, BF16 = 1, FP8 = 2 };
static const int ESZ[3] = {4, 2, 1};
static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint32_t rng = 12345u;
static uint32_t next_u32(void) { rng = rng * 1664525u + 1013904223u; return rng; }

/* n elements of dtype dt with finite values of moderate size */
static void* fill(int dt, size_t n) {
  void* p = malloc(n * ESZ[dt] + 1);
  for (size_t i = 0; i < n; ++i) {
    float x = ((int)(next_u32() % 2001) - 1000) / 400.0f;
    if (dt == F32) ((float*)p)[i] = x;
    else if (dt == BF16) ((uint16_t*)p)[i] = gqa_oracle_encode_bf16(x);
    else ((uint8_t*)p)[i] = gqa_oracle_encode_fp8_e4m3(x, 1.0f);
  }
  return p;
}

static void decode_cases(void) {
  const int shapes[][5] = {{1, 1, 1, 1, 1}, {2, 4, 2, 5, 3}, {3, 6, 3, 7, 2}, {1, 8, 1, 4, 8}, {2, 2, 2, 3, 1}};
  for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], L = shapes[s][3], d = shapes[s][4];
    for (int qd = 0; qd < 2; ++qd)
      for (int kd = 0; kd < 3; ++kd) {
        void* q = fill(qd, (size_t)B * Hq * d);
        void* k = fill(kd, (size_t)B * Hkv * L * d);
        void* v = fill(kd, (size_t)B * Hkv * L * d);
        int32_t* sl = malloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b) sl[b] = (b * 7 + s) % (L + 1); /* 0 .. L, including empty */
        double* w = malloc(sizeof(double) * L);
        double* out = malloc(sizeof(double) * B * Hq * d);
        EXPECT(gqa_oracle_decode(q, qd, k, v, kd, 0.5, 2.0, sl, 0.7, B, Hq, Hkv, L, d, w, out) == 0);
        for (size_t i = 0; i < (size_t)B * Hq * d; ++i) EXPECT(isfinite(out[i]));
        int32_t rows[4] = {B - 1, Hq - 1, 0, 0};
        double* out2 = malloc(sizeof(double) * 2 * d);
        EXPECT(gqa_oracle_decode_rows(q, qd, k, v, kd, 1.0, 1.0, sl, -0.3, B, Hq, Hkv, L, d, rows, 2, w, out2) == 0);
        int32_t bad_rows[2] = {B, 0};
        EXPECT(gqa_oracle_decode_rows(q, qd, k, v, kd, 1.0, 1.0, sl, 0.3, B, Hq, Hkv, L, d, bad_rows, 1, w, out2) == 1);
        for (int b = 0; b < B; ++b)
          EXPECT(gqa_oracle_weights(q, qd, k, v, kd, 1.0, 1.0, sl, 0.0, B, Hq, Hkv, L, d, b, Hq - 1, w) == sl[b]);
        sl[0] = L + 1; /* outside [0, L] */
        EXPECT(gqa_oracle_decode(q, qd, k, v, kd, 1.0, 1.0, sl, 0.7, B, Hq, Hkv, L, d, w, out) == 2);
        sl[0] = -1;
        EXPECT(gqa_oracle_decode(q, qd, k, v, kd, 1.0, 1.0, sl, 0.7, B, Hq, Hkv, L, d, w, out) == 2);
        sl[0] = 0;
        if ((Hq + 1) % Hkv != 0) /* rejected before any access */
          EXPECT(gqa_oracle_decode(q, qd, k, v, kd, 1.0, 1.0, sl, 0.7, B, Hq + 1, Hkv, L, d, w, out) == 1);
        EXPECT(gqa_oracle_decode(q, qd, k, v, 7, 1.0, 1.0, sl, 0.7, B, Hq, Hkv, L, d, w, out) == 1);
        free(q); free(k); free(v); free(sl); free(w); free(out); free(out2);
      }
  }
}

static void paged_cases(void) {
  const int B = 3, Hq = 4, Hkv = 2, d = 3, bs = 2, max_blocks = 3, num_blocks = 7;
  const int L = bs * max_blocks;
  for (int kd = 0; kd < 3; ++kd) {
    void* q = fill(BF16, (size_t)B * Hq * d);
    void* kp = fill(kd, (size_t)num_blocks * Hkv * bs * d);
    void* vp = fill(kd, (size_t)num_blocks * Hkv * bs * d);
    int32_t table[9] = {4, 0, -1, 6, 2, 5, 3, -7, 99}; /* entries past each sequence are never read */
    int32_t sl[3] = {4, 6, 1};
    double* w = malloc(sizeof(double) * L);
    double* out = malloc(sizeof(double) * B * Hq * d);
    EXPECT(gqa_oracle_decode_paged(q, BF16, kp, vp, kd, 1.0, 1.0, table, sl, 0.4, B, Hq, Hkv, bs, max_blocks,
                                   num_blocks, d, NULL, 0, w, out) == 0);
    int32_t rows[2] = {1, 3};
    EXPECT(gqa_oracle_decode_paged(q, BF16, kp, vp, kd, 1.0, 1.0, table, sl, 0.4, B, Hq, Hkv, bs, max_blocks,
                                   num_blocks, d, rows, 1, w, out) == 0);
    sl[2] = 3; /* now reads entry -7 of sequence 2: a live entry outside the pool */
    EXPECT(gqa_oracle_decode_paged(q, BF16, kp, vp, kd, 1.0, 1.0, table, sl, 0.4, B, Hq, Hkv, bs, max_blocks,
                                   num_blocks, d, NULL, 0, w, out) == 3);
    sl[2] = L + 1;
    EXPECT(gqa_oracle_decode_paged(q, BF16, kp, vp, kd, 1.0, 1.0, table, sl, 0.4, B, Hq, Hkv, bs, max_blocks,
                                   num_blocks, d, NULL, 0, w, out) == 2);
    free(q); free(kp); free(vp); free(w); free(out);
  }
}

static void append_cases(void) {
  const int B = 4, Hkv = 2, L = 5, d = 3;
  for (int nd = 0; nd < 2; ++nd)
    for (int kd = 0; kd < 3; ++kd) {
      void* kn = fill(nd, (size_t)B * Hkv * d);
      void* vn = fill(nd, (size_t)B * Hkv * d);
      void* kc = fill(kd, (size_t)B * Hkv * L * d);
      void* vc = fill(kd, (size_t)B * Hkv * L * d);
      int32_t pos[4] = {0, L - 1, -1, L}; /* first, last, idle, past the end */
      EXPECT(gqa_oracle_append(kn, vn, nd, kc, vc, kd, 0.5, 0.25, pos, B, Hkv, L, d, NULL, 0, 0, 0) == 1);
      /* paged: 3 pages of 2 positions; sequence 3's page is outside the pool */
      void* kp = fill(kd, (size_t)3 * Hkv * 2 * d);
      void* vp = fill(kd, (size_t)3 * Hkv * 2 * d);
      int32_t table[8] = {0, 1, 2, 0, 1, 2, 9, 1};
      int32_t ppos[4] = {3, 0, 1, 0};
      EXPECT(gqa_oracle_append(kn, vn, nd, kp, vp, kd, 1.0, 1.0, ppos, B, Hkv, 4, d, table, 2, 2, 3) == 1);
      EXPECT(gqa_oracle_append(kn, vn, 2, kc, vc, kd, 1.0, 1.0, pos, B, Hkv, L, d, NULL, 0, 0, 0) == -1);
      free(kn); free(vn); free(kc); free(vc); free(kp); free(vp);
    }
}

static void prefill_cases(void) {
  const int shapes[][5] = {{1, 1, 1, 1, 1}, {2, 4, 2, 5, 3}, {1, 6, 3, 4, 2}};
  for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], S = shapes[s][3], d = shapes[s][4];
    for (int dt = 0; dt < 2; ++dt)
      for (int causal = 0; causal < 2; ++causal) {
        void* q = fill(dt, (size_t)B * Hq * S * d);
        void* k = fill(dt, (size_t)B * Hkv * S * d);
        void* v = fill(dt, (size_t)B * Hkv * S * d);
        double* w = malloc(sizeof(double) * S);
        double* out = malloc(sizeof(double) * B * Hq * S * d);
        EXPECT(gqa_oracle_prefill(q, k, v, dt, 0.6, causal, B, Hq, Hkv, S, d, NULL, 0, w, out) == 0);
        EXPECT(gqa_oracle_prefill(q, k, v, dt, -0.6, causal, B, Hq, Hkv, S, d, NULL, 0, w, out) == 0);
        EXPECT(gqa_oracle_prefill(q, k, v, dt, 0.0, causal, B, Hq, Hkv, S, d, NULL, 0, w, out) == 0);
        int32_t rows[3] = {B - 1, Hq - 1, S - 1};
        EXPECT(gqa_oracle_prefill(q, k, v, dt, 0.6, causal, B, Hq, Hkv, S, d, rows, 1, w, out) == 0);
        if ((Hq + 1) % Hkv != 0) /* rejected before any access */
          EXPECT(gqa_oracle_prefill(q, k, v, dt, 0.6, causal, B, Hq + 1, Hkv, S, d, NULL, 0, w, out) == 1);
        free(q); free(k); free(v); free(w); free(out);
      }
  }
}

static void codec_cases(void) {
  for (uint32_t h = 0; h < 65536; ++h) (void)gqa_oracle_bf16_to_double((uint16_t)h);
  for (uint32_t c = 0; c < 256; ++c) {
    const double x = gqa_oracle_fp8_e4m3_to_double((uint8_t)c);
    if (!isnan(x)) EXPECT(gqa_oracle_encode_fp8_e4m3((float)x, 1.0f) == c);
  }
  const float special[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 3.4e38f, -3.4e38f, 1e-45f, 465.0f, -465.0f};
  for (unsigned i = 0; i < sizeof special / sizeof special[0]; ++i) {
    (void)gqa_oracle_encode_bf16(special[i]);
    (void)gqa_oracle_encode_fp8_e4m3(special[i], 1.0f);
    (void)gqa_oracle_encode_fp8_e4m3(special[i], 1e-30f);
  }
  EXPECT(gqa_oracle_kv_bytes_per_token(80, 8, 128, 2) == 327680u);
}

int main(void) {
  decode_cases();
  paged_cases();
  append_cases();
  prefill_cases();
  codec_cases();
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("oracle driver: all calls behaved\n");
  return failures ? 1 : 0;
}
