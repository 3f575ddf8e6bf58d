/* Runs the C oracle (oracle/dsa_oracle.c, built with AddressSanitizer and
 * UBSan) over small decode and prefill cases in both dtypes, on every row
 * and on row subsets, through its error paths, and checks what holds
 * whatever the values: untouched entries past each causal bound, ascending
 * and -1 padded selections within the bound, row subsets equal to the full
 * result, finite attention outputs.  Exit status 0 when every check held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_index_scores(const void* q, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, const int32_t* end_pos, int B, int T, int S_max,
                        int H, int D, float scale, int dtype, const int64_t* rows, int64_t n_rows,
                        float* out);
int oracle_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max, int k,
                const int64_t* rows, int64_t n_rows, int32_t* out);
int oracle_mla(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* kv,
               const uint16_t* pe, const int32_t* idx, const int32_t* end_pos, int B, int T,
               int S_max, int H, int Dc, int Dr, int k, float softmax_scale, const int64_t* rows,
               int64_t n_rows, double* out, double* lse);

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static uint32_t rng = 12345u;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 17;
  rng ^= rng << 5;
  return rng;
}
/* A bf16 value of a small integer in [-4, 4] (exact). */
static uint16_t bf16_int(void) {
  const float v = (float)((int)(next_u32() % 9u) - 4);
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}
/* An e4m3 code of a small integer in [-4, 4]: 0, +-1, +-2, +-3, +-4. */
static uint8_t e4m3_int(void) {
  static const uint8_t pos[5] = {0x00, 0x38, 0x40, 0x44, 0x48};
  const int v = (int)(next_u32() % 9u) - 4;
  return (uint8_t)(v < 0 ? 0x80 | pos[-v] : pos[v]);
}

enum { B = 2, T = 3, S = 40, H = 4, D = 8, K = 16, Dc = 16, Dr = 4 };

static void indexer_and_topk(int dtype) {
  const int32_t end_pos[B] = {35, S};
  const int64_t n = (int64_t)B * T;
  void* q = malloc((size_t)n * H * D * 2);
  void* k = malloc((size_t)B * S * D * 2);
  float w[B * T * H], qs[B * T * H], ks[B * S];
  for (int i = 0; i < B * T * H; ++i) {
    w[i] = (float)((int)(next_u32() % 5u) - 2);
    qs[i] = 0.5f;
  }
  for (int i = 0; i < B * S; ++i) ks[i] = 0.25f;
  for (int64_t i = 0; i < n * H * D; ++i) {
    if (dtype == 0) ((uint16_t*)q)[i] = bf16_int();
    else ((uint8_t*)q)[i] = e4m3_int();
  }
  for (int64_t i = 0; i < (int64_t)B * S * D; ++i) {
    if (dtype == 0) ((uint16_t*)k)[i] = bf16_int();
    else ((uint8_t*)k)[i] = e4m3_int();
  }
  const float* qsp = dtype ? qs : NULL;
  const float* ksp = dtype ? ks : NULL;
  float* all = malloc(sizeof(float) * n * S);
  float* sub = malloc(sizeof(float) * n * S);
  for (int64_t i = 0; i < n * S; ++i) all[i] = sub[i] = NAN;
  EXPECT(oracle_index_scores(q, qsp, w, k, ksp, end_pos, B, T, S, H, D, 0.5f, dtype, NULL, 0, all) == 0);
  const int64_t rows[2] = {4, 1};
  EXPECT(oracle_index_scores(q, qsp, w, k, ksp, end_pos, B, T, S, H, D, 0.5f, dtype, rows, 2, sub) == 0);
  for (int64_t r = 0; r < n; ++r) {
    const int b = (int)(r / T), t = (int)(r % T), bound = end_pos[b] - T + t;
    for (int s = 0; s < S; ++s) {
      const float v = all[r * S + s];
      EXPECT(s <= bound ? isfinite(v) : isnan(v));
      if (r == 4 || r == 1) EXPECT(s > bound ? isnan(sub[r * S + s]) : sub[r * S + s] == v);
      else EXPECT(isnan(sub[r * S + s]));
    }
  }
  /* Selections: k below and above the row lengths, ties from the integers. */
  for (int kk = 1; kk <= S + 5; kk += 7) {
    for (int64_t i = 0; i < n * S; ++i)
      if (isnan(all[i])) all[i] = 0.f; /* the oracle's callers zero the masked tail */
    int32_t* idx = malloc(sizeof(int32_t) * n * kk);
    EXPECT(oracle_topk(all, end_pos, B, T, S, kk, NULL, 0, idx) == 0);
    for (int64_t r = 0; r < n; ++r) {
      const int b = (int)(r / T), t = (int)(r % T), bound = end_pos[b] - T + t;
      const int keff = kk < bound + 1 ? kk : bound + 1;
      for (int j = 0; j < kk; ++j) {
        const int32_t p = idx[r * kk + j];
        if (j < keff) {
          EXPECT(p >= 0 && p <= bound);
          if (j > 0) EXPECT(p > idx[r * kk + j - 1]);
        } else {
          EXPECT(p == -1);
        }
      }
    }
    free(idx);
  }
  /* Error paths. */
  EXPECT(oracle_index_scores(NULL, qsp, w, k, ksp, end_pos, B, T, S, H, D, 1.f, dtype, NULL, 0, all) == -1);
  const int32_t bad_end[B] = {2, S};
  EXPECT(oracle_index_scores(q, qsp, w, k, ksp, bad_end, B, T, S, H, D, 1.f, dtype, NULL, 0, all) == -3);
  const int64_t bad_rows[1] = {(int64_t)B * T};
  EXPECT(oracle_index_scores(q, qsp, w, k, ksp, end_pos, B, T, S, H, D, 1.f, dtype, bad_rows, 1, sub) == -1);
  EXPECT(oracle_topk(all, bad_end, B, T, S, 4, NULL, 0, (int32_t*)sub) == -3);
  free(q);
  free(k);
  free(all);
  free(sub);
}

static void attention(void) {
  const int32_t end_pos[B] = {30, S};
  const int64_t n = (int64_t)B * T;
  uint16_t* qn = malloc(2 * (size_t)n * H * Dc);
  uint16_t* qp = malloc(2 * (size_t)n * H * Dr);
  uint16_t* kv = malloc(2 * (size_t)B * S * Dc);
  uint16_t* pe = malloc(2 * (size_t)B * S * Dr);
  for (int64_t i = 0; i < n * H * Dc; ++i) qn[i] = bf16_int();
  for (int64_t i = 0; i < n * H * Dr; ++i) qp[i] = bf16_int();
  for (int64_t i = 0; i < (int64_t)B * S * Dc; ++i) kv[i] = bf16_int();
  for (int64_t i = 0; i < (int64_t)B * S * Dr; ++i) pe[i] = bf16_int();
  int32_t idx[B * T * K];
  for (int64_t r = 0; r < n; ++r)
    for (int j = 0; j < K; ++j) idx[r * K + j] = j % 3 == 2 ? -1 : j + (int)r; /* within every bound (>= 27); some empty */
  double* out = malloc(sizeof(double) * n * H * Dc);
  double* sub = malloc(sizeof(double) * n * H * Dc);
  double lse[B * T * H], lsub[B * T * H];
  EXPECT(oracle_mla(qn, qp, kv, pe, idx, end_pos, B, T, S, H, Dc, Dr, K, 0.3f, NULL, 0, out, lse) == 0);
  for (int64_t i = 0; i < n * H * Dc; ++i) EXPECT(isfinite(out[i]));
  for (int64_t i = 0; i < n * H; ++i) EXPECT(isfinite(lse[i]));
  const int64_t rows[1] = {5};
  for (int64_t i = 0; i < n * H * Dc; ++i) sub[i] = NAN;
  EXPECT(oracle_mla(qn, qp, kv, pe, idx, end_pos, B, T, S, H, Dc, Dr, K, 0.3f, rows, 1, sub, lsub) == 0);
  for (int64_t i = 5 * H * Dc; i < 6 * H * Dc; ++i) EXPECT(sub[i] == out[i]);
  /* Dense: every valid position, no index list. */
  EXPECT(oracle_mla(qn, qp, kv, pe, NULL, end_pos, B, T, S, H, Dc, Dr, 0, 0.3f, NULL, 0, out, NULL) == 0);
  for (int64_t i = 0; i < n * H * Dc; ++i) EXPECT(isfinite(out[i]));
  /* A list with no valid entry has no defined output. */
  for (int j = 0; j < K; ++j) idx[j] = -1;
  EXPECT(oracle_mla(qn, qp, kv, pe, idx, end_pos, B, T, S, H, Dc, Dr, K, 0.3f, rows, 1, out, lse) == 0);
  EXPECT(oracle_mla(qn, qp, kv, pe, idx, end_pos, B, T, S, H, Dc, Dr, K, 0.3f, NULL, 0, out, lse) == -3);
  EXPECT(oracle_mla(NULL, qp, kv, pe, idx, end_pos, B, T, S, H, Dc, Dr, K, 0.3f, NULL, 0, out, lse) == -1);
  free(qn);
  free(qp);
  free(kv);
  free(pe);
  free(out);
  free(sub);
}

int main(void) {
  indexer_and_topk(0);
  indexer_and_topk(1);
  attention();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
