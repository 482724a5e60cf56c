/*
 * lca_oracle.h -- plain CPU oracle for the compressed-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library: every format, every reduction and every loop here is
 * written again from the definitions, slowly and in the order they are
 * stated, so that a reader can check it against the pages by eye.
 *
 * Sources (cited by page title and section only):
 *   [AGENT]  vibecoco.ai "DeepSeek V4 agent architecture" page, section
 *            "混合注意力" (hybrid attention: the 4x softmax-gated pooling with a
 *            learned position bias, the FP4 lightning indexer with ReLU-scored
 *            multi-head dot products, top-k block selection, the raw sliding
 *            window, the 128x dense path, FP8 KV with BF16 RoPE dims).
 *   [REPORT] agents-report.net "DeepSeek-V4：交錯壓縮注意力與低位元 KV 儲存"
 *            page, section "核心技術" (CSA 4x + indexer top-k; HCA 128x dense).
 *   [ARCH]   pnsm.cn "DeepSeek V4 架构深度解析" page, section 2.1 (two KV
 *            paths: a cyclic sliding window and a compressed path filtered to
 *            top-k; one attention call over both) and 2.2 (HCA at 128:1).
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.  Head counts, dims, scale-block sizes and the
 * gate form come from the workload definitions (16/64 query heads sharing one
 * 512-d entry of 448 FP8 e4m3 dims with a per-64 fp32 scale plus 64 BF16 RoPE
 * dims; an indexer of H_I heads x 64 dims in FP4 e2m1 with a per-32 scale and
 * per-head fp32 weights; gate logits and position bias per in-block position
 * and per channel).
 *
 * Parity status: every function here is pinned by the CPU tests (closed
 * forms, exhaustive format enumeration, brute force on tiny inputs,
 * invariants).  Fidelity to trained model weights is not claimed.
 */
#ifndef LCA_ORACLE_H
#define LCA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_KV_DIM 512
#define ORC_NOPE_DIM 448
#define ORC_ROPE_DIM 64
#define ORC_GROUP 64
#define ORC_NGROUPS 7
#define ORC_SCALE_STRIDE 8
#define ORC_IDX_DIM 64
#define ORC_MX_BLOCK 32

/* ---------------- number formats ---------------- */
double   orc_bf16_value(uint16_t b);
uint16_t orc_bf16_encode(float x);
double   orc_e4m3_value(uint8_t c);
uint8_t  orc_e4m3_encode(float x);
double   orc_e2m1_value(uint8_t nibble);
uint8_t  orc_e2m1_encode(float x);
double   orc_e8m0_value(uint8_t e);
void     orc_fp8_group_quant(const float *y, uint8_t *codes, float *scale);
void     orc_mxfp4_quant(const float *y, uint8_t *packed, uint8_t *e8m0);

/* ---------------- compressor ---------------- */
void orc_pool_f32(int m, int C, const float *x, long x_stride,
                  const float *z, long z_stride, const float *bias, float *y);
void orc_pool_f64(int m, int C, const float *x, long x_stride,
                  const float *z, long z_stride, const float *bias, double *y);
void orc_make_entry(const float *y, uint8_t *nope, uint16_t *rope, float *scale);
void orc_make_idx(const float *y, uint8_t *code, uint8_t *e8m0);

/* One layer's cache, host memory, same plane layout as the library's.
 * Entry planes: [B][max_blocks][...] when page_blocks is 0; otherwise a pool
 * of pool_pages pages of page_blocks entries, [pool_pages * page_blocks][...],
 * and page_table[B][max_blocks / page_blocks] names the pool page holding
 * each run of page_blocks consecutive entries of a row (-1: none). */
typedef struct orc_layer {
  int32_t batch, ratio, window, ring, has_indexer, page_blocks;
  int64_t max_blocks;
  int32_t *seq_len;     /* [B] */
  uint8_t *nope;        /* entry planes (above): 448 e4m3 codes per entry */
  uint16_t *rope;       /* 64 bf16 per entry */
  float *kv_scale;      /* 8 per entry, slot 7 unused (0) */
  uint8_t *idx_code;    /* 32 per entry */
  uint8_t *idx_scale;   /* 2 per entry */
  uint16_t *ring_kv;    /* [B][R][512] */
  float *ring_gate;     /* [B][R][512] */
  float *ring_ikey;     /* [B][R][64] */
  float *ring_igate;    /* [B][R][64] */
  const float *pos_bias;  /* [m][512] */
  const float *ipos_bias; /* [m][64] */
  const int32_t *page_table;  /* [B][max_blocks / page_blocks] when paged */
  int64_t pool_pages;
} orc_layer;

/* Where entry b of a row lives in the entry planes, or -1 when it lies on a
 * page the table does not map (functions meeting one return -8). */
long orc_entry_index(const orc_layer *L, int row, long b);

int orc_compress_append(orc_layer *L, const uint16_t *kv, const float *gate,
                        const float *ikey, const float *igate, int n);

/* ---------------- indexer and top-k ---------------- */
float orc_index_score(const uint8_t *qcode, const uint8_t *qe, const float *w,
                      int H, const uint8_t *kcode, const uint8_t *ke,
                      int *inexact);
void orc_topk_select(const float *scores, int n, int k, int32_t *out);
int orc_indexer_topk(const orc_layer *L, const float *iq, const float *iw,
                     int n_q, int H, int k, int32_t *topk, int nthreads);
int orc_indexer_scores(const orc_layer *L, int row, int q_index, int n_q,
                       const float *iq, const float *iw, int H, float *scores,
                       int *n_visible);

/* ---------------- attention ---------------- */
void orc_attend_keys(const uint16_t *q, int H, int n_keys, const double *keys,
                     double scale, float *out);
int orc_csa_attend(const orc_layer *L, const uint16_t *q, int n_q, int H,
                   const int32_t *topk, int k, float scale, float *out,
                   int nthreads);
int orc_hca_attend(const orc_layer *L, const uint16_t *q, int n_q, int H,
                   float scale, float *out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
