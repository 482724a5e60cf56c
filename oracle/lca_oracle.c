/*
 * lca_oracle.c -- plain CPU oracle (test infrastructure only; see the header).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread -lm.
 * Floating point: the compressor follows its stated fp32 order (the FP8/FP4
 * codes it decides are taken in the same precision on both sides); the
 * indexer score is an exact dot product per head rounded once, then one fp32
 * fma chain over the heads in ascending order (the top-k it decides is
 * compared bit for bit); attention is computed in double and rounded to
 * fp32 once at the end.
 */
#define _GNU_SOURCE
#include "lca_oracle.h"

#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================
 * Number formats.  The workload definitions fix FP8 e4m3 (per-64 fp32 scale)
 * for 448 KV dims, BF16 for the 64 RoPE dims ([AGENT] hybrid-attention
 * section: FP8 storage with BF16 RoPE dims) and FP4 e2m1 with a per-32 scale
 * for the indexer ([AGENT]: the indexer runs in FP4).  Reading: e4m3 is the
 * OCP "fn" flavour (bias 7, max 448, no infinities, S.1111.111 = NaN); the
 * per-32 FP4 scale is an E8M0 power of two (the OCP MX pairing of e2m1 with
 * 32-element blocks).  Encoders round to nearest, ties to even, and
 * saturate.  They are written as a search over the decoded value table so
 * that they follow the definition rather than a bit trick.
 * ====================================================================== */

double orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* bf16 = the top 16 bits of an fp32 after round-to-nearest-even. */
uint16_t orc_bf16_encode(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lo = u & 0xFFFF0000u;          /* truncation toward zero */
  uint32_t hi = lo + 0x10000u;            /* next code away from zero */
  float flo, fhi;
  memcpy(&flo, &lo, 4);
  memcpy(&fhi, &hi, 4);
  double dx = fabs((double)x), dlo = fabs((double)flo), dhi = fabs((double)fhi);
  if ((hi & 0x7F800000u) == 0x7F800000u && (hi & 0x007FFFFFu) == 0) {
    /* the code above is infinity: keep the RNE rule with inf as a neighbour */
    dhi = ldexp(1.0, 128);
  }
  double d_lo = dx - dlo, d_hi = dhi - dx;
  uint32_t pick;
  if (d_lo < d_hi) pick = lo;
  else if (d_hi < d_lo) pick = hi;
  else pick = ((lo >> 16) & 1u) ? hi : lo; /* tie: even code */
  return (uint16_t)(pick >> 16);
}

/* e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits. */
double orc_e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

uint8_t orc_e4m3_encode(float x) {
  double a = fabs((double)x);
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return 0x7F;
  /* Magnitudes 0x00..0x7E are increasing in value; find the neighbours. */
  int lo = 0;
  while (lo < 0x7E && orc_e4m3_value((uint8_t)(lo + 1)) <= a) lo++;
  uint8_t code;
  if (lo == 0x7E) {
    code = 0x7E;                           /* saturate at 448 */
  } else {
    double vlo = orc_e4m3_value((uint8_t)lo), vhi = orc_e4m3_value((uint8_t)(lo + 1));
    double dl = a - vlo, dh = vhi - a;
    if (dl < dh) code = (uint8_t)lo;
    else if (dh < dl) code = (uint8_t)(lo + 1);
    else code = (lo & 1) ? (uint8_t)(lo + 1) : (uint8_t)lo;
  }
  return (uint8_t)(sign | code);
}

/* e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: 0,.5,1,1.5,2,3,4,6. */
double orc_e2m1_value(uint8_t nib) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[nib & 7];
  return (nib & 8) ? -v : v;
}

uint8_t orc_e2m1_encode(float x) {
  double a = fabs((double)x);
  uint8_t sign = signbit(x) ? 8 : 0;
  int lo = 0;
  while (lo < 7 && orc_e2m1_value((uint8_t)(lo + 1)) <= a) lo++;
  uint8_t code;
  if (lo == 7) {
    code = 7;                              /* saturate at 6 */
  } else {
    double vlo = orc_e2m1_value((uint8_t)lo), vhi = orc_e2m1_value((uint8_t)(lo + 1));
    double dl = a - vlo, dh = vhi - a;
    if (dl < dh) code = (uint8_t)lo;
    else if (dh < dl) code = (uint8_t)(lo + 1);
    else code = (lo & 1) ? (uint8_t)(lo + 1) : (uint8_t)lo;
  }
  return (uint8_t)(sign | code);
}

double orc_e8m0_value(uint8_t e) {
  if (e == 255) return NAN;
  return ldexp(1.0, (int)e - 127);
}

/* Per-64 FP8 group.  Reading: the fp32 scale is amax/448 so that the group's
 * largest element lands on the largest finite e4m3 value; codes are
 * e4m3(x * (448/amax)), the product rounded to fp32 first.  An all-zero group
 * stores scale 0 and zero codes. */
void orc_fp8_group_quant(const float *y, uint8_t *codes, float *scale) {
  float amax = 0.0f;
  for (int i = 0; i < ORC_GROUP; i++) {
    float a = fabsf(y[i]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    *scale = 0.0f;
    memset(codes, 0, ORC_GROUP);
    return;
  }
  volatile float inv = 448.0f / amax;      /* fp32 divisions, correctly rounded */
  volatile float s = amax / 448.0f;
  for (int i = 0; i < ORC_GROUP; i++) {
    volatile float t = y[i] * inv;         /* rounded to fp32 before encoding */
    codes[i] = orc_e4m3_encode(t);
  }
  *scale = s;
}

/* One MX block of 32 elements: shared exponent X = floor(log2(amax)) - 2
 * (2 = the largest e2m1 exponent), clamped to the E8M0 range, codes
 * e2m1(x * 2^-X).  Element 2j goes to the low nibble of byte j. */
void orc_mxfp4_quant(const float *y, uint8_t *packed, uint8_t *e8m0) {
  float amax = 0.0f;
  for (int i = 0; i < ORC_MX_BLOCK; i++) {
    float a = fabsf(y[i]);
    if (a > amax) amax = a;
  }
  memset(packed, 0, ORC_MX_BLOCK / 2);
  if (amax == 0.0f) {
    *e8m0 = 0;
    return;
  }
  int ex;
  (void)frexp((double)amax, &ex);          /* amax = f * 2^ex, f in [0.5, 1) */
  int X = (ex - 1) - 2;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  for (int i = 0; i < ORC_MX_BLOCK; i++) {
    float t = ldexpf(y[i], -X);
    uint8_t c = orc_e2m1_encode(t);
    packed[i / 2] |= (uint8_t)((i & 1) ? (c << 4) : c);
  }
  *e8m0 = (uint8_t)(X + 127);
}

/* ======================================================================
 * Compressor.  [AGENT] hybrid-attention section: every m consecutive tokens'
 * KV (m = 4 for CSA, 128 for HCA per [REPORT] 核心技術) are pooled into one
 * entry by softmax-gated pooling with a learned position bias.  Readings:
 * blocks are contiguous and aligned at position 0; the softmax runs over the
 * m tokens of a block separately for every channel, on the per-token gate
 * logit plus the bias of that in-block position and channel; the weights are
 * formed first and then used in an ascending weighted sum.
 * ====================================================================== */

void orc_pool_f32(int m, int C, const float *x, long x_stride,
                  const float *z, long z_stride, const float *bias, float *y) {
  float *a = (float *)malloc(sizeof(float) * (size_t)m);
  float *e = (float *)malloc(sizeof(float) * (size_t)m);
  for (int c = 0; c < C; c++) {
    float M = -INFINITY;                   /* 1. a_i = z_i + bias_i, M = max a_i */
    for (int i = 0; i < m; i++) {
      a[i] = z[(long)i * z_stride + c] + bias[(long)i * C + c];
      if (a[i] > M) M = a[i];
    }
    float S = 0.0f;                        /* 2. e_i = exp(a_i - M), S = sum e_i */
    for (int i = 0; i < m; i++) {
      e[i] = expf(a[i] - M);
      S = S + e[i];
    }
    float acc = 0.0f;                      /* 3. y = sum (e_i / S) * x_i, ascending */
    for (int i = 0; i < m; i++) {
      float w = e[i] / S;
      float t = w * x[(long)i * x_stride + c];
      acc = acc + t;
    }
    y[c] = acc;
  }
  free(a);
  free(e);
}

void orc_pool_f64(int m, int C, const float *x, long x_stride,
                  const float *z, long z_stride, const float *bias, double *y) {
  double *a = (double *)malloc(sizeof(double) * (size_t)m);
  for (int c = 0; c < C; c++) {
    double M = -INFINITY;
    for (int i = 0; i < m; i++) {
      a[i] = (double)z[(long)i * z_stride + c] + (double)bias[(long)i * C + c];
      if (a[i] > M) M = a[i];
    }
    double S = 0.0;
    for (int i = 0; i < m; i++) S += exp(a[i] - M);
    double acc = 0.0;
    for (int i = 0; i < m; i++) acc += exp(a[i] - M) / S * (double)x[(long)i * x_stride + c];
    y[c] = acc;
  }
  free(a);
}

/* One compressed entry: 7 FP8 groups, 64 BF16 RoPE dims, scale slot 7 = 0. */
void orc_make_entry(const float *y, uint8_t *nope, uint16_t *rope, float *scale) {
  for (int g = 0; g < ORC_NGROUPS; g++)
    orc_fp8_group_quant(y + g * ORC_GROUP, nope + g * ORC_GROUP, scale + g);
  scale[ORC_NGROUPS] = 0.0f;
  for (int c = 0; c < ORC_ROPE_DIM; c++) rope[c] = orc_bf16_encode(y[ORC_NOPE_DIM + c]);
}

/* One indexer key: two MXFP4 blocks. */
void orc_make_idx(const float *y, uint8_t *code, uint8_t *e8m0) {
  orc_mxfp4_quant(y, code, e8m0);
  orc_mxfp4_quant(y + ORC_MX_BLOCK, code + ORC_MX_BLOCK / 2, e8m0 + 1);
}

/* Append n tokens to every row: each block completed by the new tokens is
 * pooled and quantized (ascending block order), then the raw tokens enter the
 * ring at slot position % R ([ARCH] 2.1: the window store holds a fixed number
 * of raw tokens and overwrites cyclically), then seq_len grows by n.  Old
 * tokens of a block that straddles calls come from the ring. */
/* Entry placement.  Contiguous layers give each row max_blocks consecutive
 * entries.  Paged layers split a row's entries into runs of page_blocks,
 * run j of row r being pool page page_table[r][j] (the library's layout
 * rule for variable-length batches; it is storage only, so every result
 * equals the contiguous layer's with the same entries). */
long orc_entry_index(const orc_layer *L, int row, long b) {
  if (L->page_blocks == 0) return (long)row * L->max_blocks + b;
  const long pages_per_row = L->max_blocks / L->page_blocks;
  const long page = L->page_table[(long)row * pages_per_row + b / L->page_blocks];
  if (page < 0 || page >= L->pool_pages) return -1;
  return page * L->page_blocks + b % L->page_blocks;
}

int orc_compress_append(orc_layer *L, const uint16_t *kv, const float *gate,
                        const float *ikey, const float *igate, int n) {
  const int m = L->ratio, R = L->ring, C = ORC_KV_DIM, CI = ORC_IDX_DIM;
  if (n < 0 || m < 1) return -1;
  float *xs = (float *)malloc(sizeof(float) * (size_t)m * C);
  float *zs = (float *)malloc(sizeof(float) * (size_t)m * C);
  float *ik = (float *)malloc(sizeof(float) * (size_t)m * CI);
  float *ig = (float *)malloc(sizeof(float) * (size_t)m * CI);
  float y[ORC_KV_DIM], yi[ORC_IDX_DIM];
  int rc = 0;
  for (int b = 0; b < L->batch && rc == 0; b++) {
    const long L0 = L->seq_len[b];
    const long first = L0 / m, end = (L0 + n) / m;
    if (end > L->max_blocks) { rc = -3; break; }
    for (long bk = first; bk < end; bk++) {
      for (int i = 0; i < m; i++) {
        long t = bk * m + i;
        const uint16_t *src_kv;
        const float *src_g, *src_ik = NULL, *src_ig = NULL;
        if (t >= L0) {                     /* a token of this call */
          long j = (long)b * n + (t - L0);
          src_kv = kv + j * C;
          src_g = gate + j * C;
          if (L->has_indexer) { src_ik = ikey + j * CI; src_ig = igate + j * CI; }
        } else {                           /* an earlier token, still in the ring */
          long slot = (long)b * R + (t % R);
          src_kv = L->ring_kv + slot * C;
          src_g = L->ring_gate + slot * C;
          if (L->has_indexer) { src_ik = L->ring_ikey + slot * CI; src_ig = L->ring_igate + slot * CI; }
        }
        for (int c = 0; c < C; c++) xs[(long)i * C + c] = (float)orc_bf16_value(src_kv[c]);
        memcpy(zs + (long)i * C, src_g, sizeof(float) * C);
        if (L->has_indexer) {
          memcpy(ik + (long)i * CI, src_ik, sizeof(float) * CI);
          memcpy(ig + (long)i * CI, src_ig, sizeof(float) * CI);
        }
      }
      long e = orc_entry_index(L, b, bk);
      if (e < 0) { rc = -8; break; }
      orc_pool_f32(m, C, xs, C, zs, C, L->pos_bias, y);
      orc_make_entry(y, L->nope + e * ORC_NOPE_DIM, L->rope + e * ORC_ROPE_DIM,
                     L->kv_scale + e * ORC_SCALE_STRIDE);
      if (L->has_indexer) {
        /* Reading: the indexer key is a separate 64-d per-token stream (fp32)
         * pooled by the same mechanism with its own gate logits and bias. */
        orc_pool_f32(m, CI, ik, CI, ig, CI, L->ipos_bias, yi);
        orc_make_idx(yi, L->idx_code + e * 32, L->idx_scale + e * 2);
      }
    }
    for (int j = 0; j < n; j++) {
      long t = L0 + j;
      long slot = (long)b * R + (t % R);
      long src = (long)b * n + j;
      memcpy(L->ring_kv + slot * C, kv + src * C, sizeof(uint16_t) * C);
      memcpy(L->ring_gate + slot * C, gate + src * C, sizeof(float) * C);
      if (L->has_indexer) {
        memcpy(L->ring_ikey + slot * CI, ikey + src * CI, sizeof(float) * CI);
        memcpy(L->ring_igate + slot * CI, igate + src * CI, sizeof(float) * CI);
      }
    }
    L->seq_len[b] = (int32_t)(L0 + n);
  }
  free(xs); free(zs); free(ik); free(ig);
  return rc;
}

/* ======================================================================
 * Lightning indexer.  [AGENT] hybrid-attention section: an FP4 indexer
 * scores each compressed block by ReLU-scored multi-head dot products and the
 * top-k blocks are kept.  Readings: one shared 64-d key per block; the query
 * has H heads of 64 dims, quantized to MXFP4 in the call; per-head fp32
 * weights; score = sum_h w_h * ReLU(q_h . k).  Order of evaluation (fixed so
 * that the selection can be compared bit for bit; the pages fix none): each
 * head's dot product is the exact dot of the two dequantized MXFP4 vectors
 * rounded once to fp32; ReLU maps it to +0 unless positive; the weighted sum
 * is a single chain of fp32 fused multiply-adds over the heads in ascending
 * order, starting from +0; a zero score is +0.
 * ====================================================================== */

float orc_index_score(const uint8_t *qcode, const uint8_t *qe, const float *w,
                      int H, const uint8_t *kcode, const uint8_t *ke,
                      int *inexact) {
  float score = 0.0f;
  for (int h = 0; h < H; h++) {
    double halfsum[2];
    for (int j = 0; j < 2; j++) {
      double d = 0.0;                      /* exact: products on a 1/4 grid, |sum| < 2^11 */
      for (int i = 0; i < ORC_MX_BLOCK; i++) {
        int el = j * ORC_MX_BLOCK + i;
        uint8_t qb = qcode[h * 32 + el / 2], kb = kcode[el / 2];
        uint8_t qn = (el & 1) ? (qb >> 4) : (qb & 15);
        uint8_t kn = (el & 1) ? (kb >> 4) : (kb & 15);
        d += orc_e2m1_value(qn) * orc_e2m1_value(kn);
      }
      halfsum[j] = ldexp(d, ((int)qe[h * 2 + j] - 127) + ((int)ke[j] - 127));
    }
    double s = halfsum[0] + halfsum[1];
    /* exactness of the double sum (TwoSum error term must vanish) */
    double bv = s - halfsum[0], av = s - bv;
    double err = (halfsum[0] - av) + (halfsum[1] - bv);
    if (err != 0.0 && inexact) *inexact = 1;
    float dot = (float)s;                  /* the single rounding to fp32 */
    float r = dot > 0.0f ? dot : 0.0f;     /* ReLU */
    score = fmaf(w[h], r, score);          /* one chain, ascending heads */
  }
  if (score == 0.0f) score = 0.0f;         /* canonical +0 */
  return score;
}

static uint32_t orc_ord(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

static int orc_cmp_desc(const void *a, const void *b) {
  uint64_t x = *(const uint64_t *)a, y = *(const uint64_t *)b;
  return (x < y) ? 1 : (x > y) ? -1 : 0;
}

static int orc_cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* The k largest (score desc, index asc) of n blocks, emitted in ascending
 * block order and padded with -1 ([AGENT]: the top-k compressed blocks are
 * kept; the order of equal scores is a reading: lowest index first). */
void orc_topk_select(const float *scores, int n, int k, int32_t *out) {
  uint64_t *key = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(n > 0 ? n : 1));
  for (int b = 0; b < n; b++)
    key[b] = ((uint64_t)orc_ord(scores[b]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)b);
  qsort(key, (size_t)n, sizeof(uint64_t), orc_cmp_desc);
  int take = k < n ? k : n;
  for (int i = 0; i < take; i++) out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key[i] & 0xFFFFFFFFu));
  qsort(out, (size_t)take, sizeof(int32_t), orc_cmp_i32);
  for (int i = take; i < k; i++) out[i] = -1;
  free(key);
}

/* Visibility (reading): block b is visible to the query at position p iff all
 * of its m tokens are at positions <= p, i.e. b < floor((p+1)/m).  Queries are
 * the last n_q appended tokens: p = seq_len - n_q + i. */
int orc_indexer_scores(const orc_layer *L, int row, int qi, int n_q,
                       const float *iq, const float *iw, int H, float *scores,
                       int *n_visible) {
  const long p = (long)L->seq_len[row] - n_q + qi;
  if (p < 0) return -1;
  const long nv = (p + 1) / L->ratio;
  uint8_t qcode[32 * 32], qe[32 * 2];
  const float *q = iq + ((long)row * n_q + qi) * (long)H * ORC_IDX_DIM;
  const float *w = iw + ((long)row * n_q + qi) * (long)H;
  for (int h = 0; h < H; h++) orc_make_idx(q + h * ORC_IDX_DIM, qcode + h * 32, qe + h * 2);
  int inexact = 0;
  for (long b = 0; b < nv; b++) {
    long e = orc_entry_index(L, row, b);
    if (e < 0) return -8;
    scores[b] = orc_index_score(qcode, qe, w, H, L->idx_code + e * 32, L->idx_scale + e * 2,
                                &inexact);
  }
  *n_visible = (int)nv;
  return inexact ? -7 : 0;
}

typedef struct {
  const orc_layer *L;
  const float *iq, *iw;
  const uint16_t *q;
  const int32_t *topk;
  int n_q, H, k, mode;
  float scale;
  int32_t *out_idx;
  float *out;
  int next, total, err;
  pthread_mutex_t mu;
} orc_job;

static int orc_take(orc_job *J) {
  pthread_mutex_lock(&J->mu);
  int t = J->next < J->total ? J->next++ : -1;
  pthread_mutex_unlock(&J->mu);
  return t;
}

static void orc_set_err(orc_job *J, int e) {
  pthread_mutex_lock(&J->mu);
  if (J->err == 0) J->err = e;
  pthread_mutex_unlock(&J->mu);
}

static void *orc_indexer_worker(void *arg) {
  orc_job *J = (orc_job *)arg;
  const orc_layer *L = J->L;
  float *scores = (float *)malloc(sizeof(float) * (size_t)(L->max_blocks + 1));
  for (int t; (t = orc_take(J)) >= 0;) {
    int row = t / J->n_q, qi = t % J->n_q, nv = 0;
    int rc = orc_indexer_scores(L, row, qi, J->n_q, J->iq, J->iw, J->H, scores, &nv);
    if (rc) orc_set_err(J, rc);
    orc_topk_select(scores, nv, J->k, J->out_idx + (long)t * J->k);
  }
  free(scores);
  return NULL;
}

static int orc_run(orc_job *J, void *(*fn)(void *), int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  pthread_mutex_init(&J->mu, NULL);
  for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, fn, J);
  for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return J->err;
}

int orc_indexer_topk(const orc_layer *L, const float *iq, const float *iw,
                     int n_q, int H, int k, int32_t *topk, int nthreads) {
  orc_job J;
  memset(&J, 0, sizeof J);
  J.L = L; J.iq = iq; J.iw = iw; J.n_q = n_q; J.H = H; J.k = k; J.out_idx = topk;
  J.total = L->batch * n_q;
  return orc_run(&J, orc_indexer_worker, nthreads);
}

/* ======================================================================
 * Attention.  [ARCH] 2.1: one attention call over the sliding-window KV and
 * the top-k selected compressed KV; [AGENT]/[REPORT]: HCA attends densely to
 * every compressed block.  Readings: keys = the selected (or all visible)
 * blocks in ascending order, then the raw window tokens max(0,p-W+1)..p; the
 * key and the value are the same 512-d vector (448 dequantized FP8 dims,
 * value(code) * scale of its 64-group, then 64 BF16 RoPE dims; a window token
 * is its raw BF16 vector); one softmax over all keys with logit
 * scale * (q . k); output o = sum_j softmax_j * v_j in fp32.
 * ====================================================================== */

void orc_attend_keys(const uint16_t *q, int H, int n_keys, const double *keys,
                     double scale, float *out) {
  double *lg = (double *)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
  double qv[ORC_KV_DIM], o[ORC_KV_DIM];
  for (int h = 0; h < H; h++) {
    for (int c = 0; c < ORC_KV_DIM; c++) qv[c] = orc_bf16_value(q[(long)h * ORC_KV_DIM + c]);
    double M = -INFINITY;
    for (int j = 0; j < n_keys; j++) {
      double d = 0.0;
      for (int c = 0; c < ORC_KV_DIM; c++) d += qv[c] * keys[(long)j * ORC_KV_DIM + c];
      lg[j] = scale * d;
      if (lg[j] > M) M = lg[j];
    }
    double Z = 0.0;
    for (int c = 0; c < ORC_KV_DIM; c++) o[c] = 0.0;
    for (int j = 0; j < n_keys; j++) {
      double pj = exp(lg[j] - M);
      Z += pj;
      for (int c = 0; c < ORC_KV_DIM; c++) o[c] += pj * keys[(long)j * ORC_KV_DIM + c];
    }
    for (int c = 0; c < ORC_KV_DIM; c++)
      out[(long)h * ORC_KV_DIM + c] = (float)(n_keys > 0 ? o[c] / Z : 0.0);
  }
  free(lg);
}

static int orc_entry_vector(const orc_layer *L, int row, long b, double *k) {
  long e = orc_entry_index(L, row, b);
  if (e < 0) return -8;
  const uint8_t *nope = L->nope + e * ORC_NOPE_DIM;
  const float *sc = L->kv_scale + e * ORC_SCALE_STRIDE;
  const uint16_t *rope = L->rope + e * ORC_ROPE_DIM;
  for (int c = 0; c < ORC_NOPE_DIM; c++) k[c] = orc_e4m3_value(nope[c]) * (double)sc[c / ORC_GROUP];
  for (int c = 0; c < ORC_ROPE_DIM; c++) k[ORC_NOPE_DIM + c] = orc_bf16_value(rope[c]);
  return 0;
}

static void orc_window_vector(const orc_layer *L, int row, long pos, double *k) {
  const uint16_t *src = L->ring_kv + ((long)row * L->ring + pos % L->ring) * ORC_KV_DIM;
  for (int c = 0; c < ORC_KV_DIM; c++) k[c] = orc_bf16_value(src[c]);
}

static void *orc_attend_worker(void *arg) {
  orc_job *J = (orc_job *)arg;
  const orc_layer *L = J->L;
  const long cap = (J->mode == 0 ? (long)J->k : L->max_blocks) + L->window;
  double *keys = (double *)malloc(sizeof(double) * (size_t)cap * ORC_KV_DIM);
  for (int t; (t = orc_take(J)) >= 0;) {
    int row = t / J->n_q, qi = t % J->n_q;
    long p = (long)L->seq_len[row] - J->n_q + qi;
    if (p < 0) { orc_set_err(J, -1); continue; }
    long nv = (p + 1) / L->ratio, nk = 0;
    if (J->mode == 0) {
      const int32_t *sel = J->topk + (long)t * J->k;
      for (int i = 0; i < J->k; i++)
        if (sel[i] >= 0 && sel[i] < nv && orc_entry_vector(L, row, sel[i], keys + (nk++) * ORC_KV_DIM)) {
          orc_set_err(J, -8);
          nk--;
        }
    } else {
      for (long b = 0; b < nv; b++)
        if (orc_entry_vector(L, row, b, keys + (nk++) * ORC_KV_DIM)) {
          orc_set_err(J, -8);
          nk--;
        }
    }
    long w0 = p - L->window + 1;
    if (w0 < 0) w0 = 0;
    for (long j = w0; j <= p; j++) orc_window_vector(L, row, j, keys + (nk++) * ORC_KV_DIM);
    orc_attend_keys(J->q + (long)t * J->H * ORC_KV_DIM, J->H, (int)nk, keys, (double)J->scale,
                    J->out + (long)t * J->H * ORC_KV_DIM);
  }
  free(keys);
  return NULL;
}

int orc_csa_attend(const orc_layer *L, const uint16_t *q, int n_q, int H,
                   const int32_t *topk, int k, float scale, float *out,
                   int nthreads) {
  orc_job J;
  memset(&J, 0, sizeof J);
  J.L = L; J.q = q; J.n_q = n_q; J.H = H; J.topk = topk; J.k = k; J.scale = scale;
  J.out = out; J.mode = 0; J.total = L->batch * n_q;
  return orc_run(&J, orc_attend_worker, nthreads);
}

int orc_hca_attend(const orc_layer *L, const uint16_t *q, int n_q, int H,
                   float scale, float *out, int nthreads) {
  orc_job J;
  memset(&J, 0, sizeof J);
  J.L = L; J.q = q; J.n_q = n_q; J.H = H; J.scale = scale; J.out = out; J.mode = 1;
  J.total = L->batch * n_q;
  return orc_run(&J, orc_attend_worker, nthreads);
}
