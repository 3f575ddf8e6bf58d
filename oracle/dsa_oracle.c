/*
 * Plain CPU oracle for the DeepSeek Sparse Attention (DSA) decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * path (the HIP library) never links, loads or calls it, and this file
 * shares no code, header or table with it.
 *
 * What is computed, and where it is defined:
 *
 *  1. Lightning-indexer score (kernelpool's fix in "mlx-lm PR #512
 *     [WIP] deepseek v32"; Indexer.forward excerpt on the model-atlas page
 *     "DeepSeek-V3.2-Exp - Keep top-k positions"):
 *        I[b,t,s] = scale * sum_h w[b,t,h] * ReLU( q[b,t,h,:] . k[b,s,:] )
 *     one shared key per cached token, no head dimension in the output.
 *     For fp8 inputs q and k are the dequantised values code*scale (one
 *     fp32 scale per 128-element block, i.e. per head of q and per key).
 *  2. Causal bound: position s is valid for query t of sequence b iff
 *     s <= end_pos[b] - T + t  (end_pos = start_pos + seqlen, same excerpt).
 *  3. Top-k: topk(min(k, valid count)) of the scores; ties go to the
 *     smaller position, the kept positions are written in ascending order
 *     and the remaining slots hold -1.
 *  4. Absorbed MLA decode ("DeepSeek-V3.2-Exp - Apply sparse mask" page,
 *     MQA decode excerpt): scores over every valid cached position,
 *        z[h,s] = (q_nope[h,:] . kv[s,:] + q_pe[h,:] . pe[s,:]) * softmax_scale
 *     plus an additive index mask (0 on selected positions, -inf elsewhere),
 *     softmax over s, and o[h,:] = sum_s p[h,s] * kv[s,:] (the latent is
 *     both key and value).  The dense variant omits the index mask.
 *
 * Arithmetic: inputs are decoded exactly, every sum is carried in double
 * precision in ascending index order, and the only fp32 step is the final
 * score rounding fl32(fl32(acc) * fl32(scale)).  Built with
 * -ffp-contract=off and without fast-math so IEEE semantics hold.
 *
 * Every function takes its dimensions as arguments (heads, head dim, latent
 * and rope widths), so tiny hand-checkable cases can be run as well as the
 * production shapes.  Every function returns 0 on success or a negative
 * code: -1 bad argument, -2 non-finite input, -3 position out of range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_FP8_E4M3 1

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 holds subnormals m * 2^-9; 0x7F and 0xFF are NaN; there
 * is no infinity and the largest finite magnitude is 448. */
static double e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

static double elem(const void* base, int dtype, size_t i) {
  if (dtype == ORACLE_BF16) return bf16_value(((const uint16_t*)base)[i]);
  return e4m3_value(((const uint8_t*)base)[i]);
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Row list helper: rows == NULL means every (b,t) row. */
static int64_t row_at(const int64_t* rows, int64_t i) { return rows ? rows[i] : i; }

/* ------------------------------------------------------------------------
 * 1+2. Indexer scores.
 * q       [B,T,H,D]  bf16 bits or e4m3 codes
 * q_scale [B,T,H]    fp32 (fp8 only, else NULL): q value = code * q_scale
 * w       [B,T,H]    fp32
 * k       [B,S_max,D] bf16 bits or e4m3 codes
 * k_scale [B,S_max]  fp32 (fp8 only, else NULL): k value = code * k_scale
 * end_pos [B]        int32, T <= end_pos[b] <= S_max
 * out     [B,T,S_max] fp32; entries past the causal bound are not written.
 * ---------------------------------------------------------------------- */
int oracle_index_scores(const void* q, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, const int32_t* end_pos, int B, int T, int S_max,
                        int H, int D, float scale, int dtype, const int64_t* rows, int64_t n_rows,
                        float* out) {
  if (!q || !w || !k || !end_pos || !out || B < 1 || T < 1 || S_max < 1 || H < 1 || D < 1)
    return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_FP8_E4M3) return -1;
  if (dtype == ORACLE_FP8_E4M3 && (!q_scale || !k_scale)) return -1;
  for (int b = 0; b < B; ++b)
    if (end_pos[b] < T || end_pos[b] > S_max) return -3;
  if (!rows) n_rows = (int64_t)B * T;
  int status = 0;
  double* qv = (double*)malloc(sizeof(double) * (size_t)H * D);

  /* Rows one after another; the positions of a row are shared among threads. */
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t row = row_at(rows, i);
    if (row < 0 || row >= (int64_t)B * T) {
      status = -1;
      continue;
    }
    int b = (int)(row / T), t = (int)(row % T);
    int64_t bound = (int64_t)end_pos[b] - T + t;
    for (int h = 0; h < H; ++h) {
      double qs = dtype == ORACLE_FP8_E4M3 ? (double)q_scale[row * H + h] : 1.0;
      for (int d = 0; d < D; ++d) {
        double v = elem(q, dtype, ((size_t)row * H + h) * D + d) * qs;
        if (!isfinite(v)) status = -2;
        qv[h * D + d] = v;
      }
    }
#pragma omp parallel for schedule(static) if (bound >= 4096)
    for (int64_t s = 0; s <= bound; ++s) {
      size_t krow = (size_t)b * S_max + (size_t)s;
      double ks = dtype == ORACLE_FP8_E4M3 ? (double)k_scale[krow] : 1.0;
      double kvals[D];
      for (int d = 0; d < D; ++d) kvals[d] = (elem(k, dtype, krow * D + d) * ks);
      double acc = 0.0;
      for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[h * D + d] * kvals[d];
        double relu = dot > 0.0 ? dot : 0.0;
        acc += (double)w[row * H + h] * relu;
      }
      if (!isfinite(acc)) {
#pragma omp atomic write
        status = -2;
      }
      float acc32 = (float)acc;
      out[(size_t)row * S_max + (size_t)s] = acc32 * scale;
    }
  }
  free(qv);
  return status;
}

/* ------------------------------------------------------------------------
 * 3. Top-k by full sort.
 * scores  [B,T,S_max] fp32 (only entries s <= bound are read)
 * out     [B,T,k] int32: the min(k, bound+1) selected positions in
 *         ascending order, then -1.
 * Order: larger score first; equal scores (IEEE equality, so -0 == +0)
 * keep the smaller position first.
 * ---------------------------------------------------------------------- */
typedef struct {
  float score;
  int32_t pos;
} scored_pos;

static int by_score_then_pos(const void* pa, const void* pb) {
  const scored_pos* a = (const scored_pos*)pa;
  const scored_pos* b = (const scored_pos*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->pos > b->pos) - (a->pos < b->pos);
}

static int ascending_int(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int oracle_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max, int k,
                const int64_t* rows, int64_t n_rows, int32_t* out) {
  if (!scores || !end_pos || !out || B < 1 || T < 1 || S_max < 1 || k < 1) return -1;
  for (int b = 0; b < B; ++b)
    if (end_pos[b] < T || end_pos[b] > S_max) return -3;
  if (!rows) n_rows = (int64_t)B * T;
  int status = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t row = row_at(rows, i);
    if (row < 0 || row >= (int64_t)B * T) {
#pragma omp atomic write
      status = -1;
      continue;
    }
    int b = (int)(row / T), t = (int)(row % T);
    int64_t n = (int64_t)end_pos[b] - T + t + 1;
    scored_pos* cand = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)n);
    for (int64_t s = 0; s < n; ++s) {
      float v = scores[(size_t)row * S_max + (size_t)s];
      if (isnan(v)) {
#pragma omp atomic write
        status = -2;
      }
      cand[s].score = v;
      cand[s].pos = (int32_t)s;
    }
    qsort(cand, (size_t)n, sizeof(scored_pos), by_score_then_pos);
    int64_t keep = n < k ? n : k;
    int32_t* dst = out + (size_t)row * k;
    for (int64_t j = 0; j < keep; ++j) dst[j] = cand[j].pos;
    qsort(dst, (size_t)keep, sizeof(int32_t), ascending_int);
    for (int64_t j = keep; j < k; ++j) dst[j] = -1;
    free(cand);
  }
  return status;
}

/* ------------------------------------------------------------------------
 * 4. Absorbed MLA attention, masked-softmax form.
 * q_nope [B,T,H,Dc] bf16 bits (already absorbed into the latent space)
 * q_pe   [B,T,H,Dr] bf16 bits
 * kv     [B,S_max,Dc] bf16 bits;  pe [B,S_max,Dr] bf16 bits
 * idx    [B,T,k] int32 selected positions (-1 = empty slot), or NULL for
 *        dense attention over every valid position.
 * out    [B,T,H,Dc] double; lse [B,T,H] double = log(sum_s exp(z_s)), or NULL.
 * A query whose mask removes every position has no defined output; it is
 * reported as an error (-3).
 * ---------------------------------------------------------------------- */
int oracle_mla(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* kv,
               const uint16_t* pe, const int32_t* idx, const int32_t* end_pos, int B, int T,
               int S_max, int H, int Dc, int Dr, int k, float softmax_scale,
               const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (!q_nope || !q_pe || !kv || !pe || !end_pos || !out || B < 1 || T < 1 || S_max < 1 ||
      H < 1 || Dc < 1 || Dr < 0 || (idx && k < 1))
    return -1;
  for (int b = 0; b < B; ++b)
    if (end_pos[b] < T || end_pos[b] > S_max) return -3;
  if (!rows) n_rows = (int64_t)B * T;
  int status = 0;
  const double sc = (double)softmax_scale;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows * H; ++i) {
    int64_t row = row_at(rows, i / H);
    int h = (int)(i % H);
    if (row < 0 || row >= (int64_t)B * T) {
#pragma omp atomic write
      status = -1;
      continue;
    }
    int b = (int)(row / T), t = (int)(row % T);
    int64_t n = (int64_t)end_pos[b] - T + t + 1; /* valid positions 0..n-1 */

    /* Index mask as on the pages: -inf everywhere, 0 scattered at the
     * selected positions.  Dense attention keeps every valid position. */
    char* keep = (char*)malloc((size_t)n);
    memset(keep, idx ? 0 : 1, (size_t)n);
    if (idx) {
      const int32_t* sel = idx + (size_t)row * k;
      for (int j = 0; j < k; ++j) {
        if (sel[j] == -1) continue;
        if (sel[j] < 0 || sel[j] >= n) {
#pragma omp atomic write
          status = -3;
          continue;
        }
        keep[sel[j]] = 1;
      }
    }

    const uint16_t* qn = q_nope + ((size_t)row * H + h) * Dc;
    const uint16_t* qp = q_pe + ((size_t)row * H + h) * Dr;
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int64_t s = 0; s < n; ++s) {
      if (!keep[s]) { /* masked: -inf, its dot product is never needed */
        z[s] = -INFINITY;
        continue;
      }
      const uint16_t* kvs = kv + ((size_t)b * S_max + (size_t)s) * Dc;
      const uint16_t* pes = pe + ((size_t)b * S_max + (size_t)s) * Dr;
      double dot = 0.0;
      for (int c = 0; c < Dc; ++c) dot += bf16_value(qn[c]) * bf16_value(kvs[c]);
      double dot_pe = 0.0;
      for (int r = 0; r < Dr; ++r) dot_pe += bf16_value(qp[r]) * bf16_value(pes[r]);
      z[s] = (dot + dot_pe) * sc;
      if (!isfinite(z[s])) {
#pragma omp atomic write
        status = -2;
      }
      if (z[s] > m) m = z[s];
    }
    double* o = out + ((size_t)row * H + h) * Dc;
    if (m == -INFINITY) { /* every position masked */
#pragma omp atomic write
      status = -3;
      for (int c = 0; c < Dc; ++c) o[c] = NAN;
      if (lse) lse[(size_t)row * H + h] = NAN;
      free(z);
      free(keep);
      continue;
    }
    double l = 0.0;
    for (int64_t s = 0; s < n; ++s) {
      z[s] = exp(z[s] - m); /* exp(-inf) == 0 for masked positions */
      l += z[s];
    }
    for (int c = 0; c < Dc; ++c) o[c] = 0.0;
    for (int64_t s = 0; s < n; ++s) {
      if (z[s] == 0.0) continue; /* adds exactly +0 */
      const uint16_t* kvs = kv + ((size_t)b * S_max + (size_t)s) * Dc;
      for (int c = 0; c < Dc; ++c) o[c] += z[s] * bf16_value(kvs[c]);
    }
    for (int c = 0; c < Dc; ++c) o[c] /= l;
    if (lse) lse[(size_t)row * H + h] = m + log(l);
    free(z);
    free(keep);
  }
  return status;
}
