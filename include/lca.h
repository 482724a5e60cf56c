/*
 * lca.h -- C ABI of the MI355X (gfx950) compressed long-context attention
 * library (liblca.so).
 *
 * The library implements the decode/prefill hot path of interleaved
 * compressed attention as described on these pages (cited by title and
 * section):
 *   [AGENT]  vibecoco.ai "DeepSeek V4 agent architecture" page, section
 *            "混合注意力" (hybrid attention): KV compressed 4x along the
 *            sequence by softmax-gated pooling with a learned position bias;
 *            an FP4 lightning indexer (ReLU-scored multi-head dot products)
 *            keeps the top-k compressed blocks; recent tokens stay raw in a
 *            sliding-window branch; HCA compresses 128x and attends densely
 *            to every compressed block; KV is stored in FP8 except the RoPE
 *            dims (BF16); the indexer runs in FP4.
 *   [REPORT] agents-report.net "DeepSeek-V4：交錯壓縮注意力與低位元 KV 儲存"
 *            page, section "核心技術" (CSA: 4x compressor + lightning indexer
 *            top-k; HCA: 128x, dense).
 *   [ARCH]   pnsm.cn "DeepSeek V4 架构深度解析" page, section 2.1 (window KV
 *            overwritten cyclically; the compressor updates the compressed
 *            cache, the index keeps the top-k; one attention over both) and
 *            section 2.2 (HCA, 128:1, layers alternate CSA and HCA).
 *
 * Conventions
 *   - Every entry point returns LCA_OK (0) or a negative LCA_E* code.  On an
 *     error nothing has been enqueued and lca_last_error() returns a message
 *     (thread-local, valid until the next call on the same thread).
 *   - Pointers inside lca_layer and all array arguments are device pointers
 *     owned by the caller, 16-byte aligned, row-major.  The library never
 *     allocates, frees or keeps them after the call returns.
 *   - Work is enqueued on the hipStream_t argument and the call returns
 *     without waiting.  Buffers must stay alive until the stream has executed
 *     the work.  Device faults surface at the caller's next synchronisation.
 *   - Calls on different layers may run concurrently.  Calls that touch the
 *     same layer or the same workspace must be ordered by the caller (same
 *     stream, or events).
 *
 * Fixed dimensions: a KV entry has 512 dims (448 FP8 + 64 BF16 RoPE); an
 * indexer key has 64 dims.
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCA_ABI_VERSION 3

enum {
  LCA_OK = 0,
  LCA_EINVAL = -1,        /* null/misaligned pointer, bad size or argument    */
  LCA_EUNSUPPORTED = -2,  /* valid but outside the supported shape range      */
  LCA_ECAPACITY = -3,     /* cache or ring too small for the request          */
  LCA_EWORKSPACE = -4,    /* workspace missing or smaller than required       */
  LCA_EHIP = -5           /* a HIP runtime call failed                        */
};

/*
 * Status bits of layer.sync[1], set by the device when a call could not do
 * its work exactly (the call itself returned LCA_OK: the condition depends
 * on device data, e.g. lengths that grew inside a replayed graph):
 *   LCA_STATUS_COMPRESS_CAPACITY  a block to finalise lay at or past
 *                                 max_blocks; it was not written
 *   LCA_STATUS_INDEXER_CAPACITY   a query saw more blocks than the call's
 *                                 plan holds (planned from len_max); the
 *                                 newest ones were not scored
 *   LCA_STATUS_ATTEND_CAPACITY    a query's key list was longer than the
 *                                 call's plan (from len_max); its last keys
 *                                 (the newest window tokens) were dropped
 *   LCA_STATUS_FP16_RANGE         attention met an input its fp16 images
 *                                 may not hold to 2^-11 of the vector's
 *                                 largest magnitude: a query head, RoPE
 *                                 group or 64-channel window group whose
 *                                 largest magnitude is 65536 or more (also
 *                                 inf, NaN) or nonzero and below 2^-14; or
 *                                 an FP8 group scale outside [2^-14, 2^8),
 *                                 where the scaled probabilities leave
 *                                 fp16's normal range.  The result may miss
 *                                 the 2e-3 bound
 *   LCA_STATUS_PAGE               a paged layer's block lay on an unmapped
 *                                 page (page-table entry < 0 or not below
 *                                 pool_pages): the compressor did not write
 *                                 it; a visible one read by the indexer or
 *                                 attention gave an unspecified score or key
 * Calls captured in a graph must be planned with len_max set to the longest
 * length they will reach (set the host mirror before capture); the capacity
 * bits report replays that went beyond it.
 */
#define LCA_STATUS_COMPRESS_CAPACITY 1u
#define LCA_STATUS_INDEXER_CAPACITY 2u
#define LCA_STATUS_ATTEND_CAPACITY 4u
#define LCA_STATUS_FP16_RANGE 8u
#define LCA_STATUS_PAGE 16u

#define LCA_KV_DIM 512
#define LCA_NOPE_DIM 448
#define LCA_ROPE_DIM 64
#define LCA_IDX_DIM 64
#define LCA_SCALE_STRIDE 8

/*
 * One attention layer's cache.  Caller-filled; the library reads the sizes
 * and pointers and updates len_min / len_max (host mirrors) in
 * lca_compress_append.
 *
 * Planes (B = batch rows, MB = max_blocks, R = ring, m = ratio):
 *   seq_len    int32   [B]            tokens appended so far, per row (device)
 *   sync       uint32  [2]            zero when created.  sync[0]: a completion
 *                                     counter the library keeps 0 between
 *                                     calls.  sync[1]: status bits (LCA_STATUS_*)
 *                                     that kernels set and never clear; the
 *                                     caller reads (and may reset) them after
 *                                     its work has run
 *   nope       uint8   [B][MB][448]   e4m3fn codes of entry dims 0..447
 *   rope       uint16  [B][MB][64]    bf16 entry dims 448..511
 *   kv_scale   float   [B][MB][8]     fp32 scale of each 64-dim FP8 group
 *                                     (slot 7 unused, written 0)
 *   idx_code   uint8   [B][MB][32]    e2m1 indexer key codes, element 2j in
 *                                     the low nibble of byte j   (CSA only)
 *   idx_scale  uint8   [B][MB][2]     E8M0 exponent of each 32-element half
 *                                     (CSA only)
 *   ring_kv    uint16  [B][R][512]    raw bf16 KV of the last R tokens at slot
 *                                     position % R (window + pooling source)
 *   ring_gate  float   [B][R][512]    their gate logits
 *   ring_ikey  float   [B][R][64]     their indexer-key stream (CSA only)
 *   ring_igate float   [B][R][64]     its gate logits (CSA only)
 *   pos_bias   float   [m][512]       learned in-block position bias
 *   ipos_bias  float   [m][64]        its indexer counterpart (CSA only)
 * Compressed entry b of a row pools tokens b*m .. b*m+m-1.  A query at
 * position p sees entries b < floor((p+1)/m) and the raw tokens
 * max(0, p-W+1) .. p.  Rows may hold different lengths; every call appends
 * the same number of tokens to every row.
 *
 * Paged entries (page_blocks = PB > 0).  Agent traces differ in length and
 * run to about a million tokens ([AGENT] on why agents break down on long
 * tasks), so rows of one batch may draw their compressed entries from one
 * shared pool of pages instead of owning max_blocks each.  The five entry
 * planes (nope, rope, kv_scale, idx_code, idx_scale) then hold pool_pages *
 * PB entries, [pool_pages * PB][...], and
 *   page_table int32   [B][MB / PB]   physical page of each logical page of a
 *                                     row, or -1 (unmapped)
 * places entry b of row r at physical entry
 * page_table[r][b / PB] * PB + b % PB.  PB is a power of two in 64..65536
 * and divides MB; the ring planes stay per row.  The caller maps the pages
 * of every entry a compress_append call completes before the call (device
 * data: a block on an unmapped page is not written and sets
 * LCA_STATUS_PAGE) and may change the table between calls (unmapping pages
 * of entries no query will read again, mapping new ones).
 */
typedef struct lca_layer {
  int32_t batch;        /* B >= 1                                              */
  int32_t ratio;        /* m: power of two, 1..128                             */
  int32_t window;       /* W >= 1                                              */
  int32_t ring;         /* R >= W                                              */
  int32_t has_indexer;  /* 1: CSA layer (indexer planes present); 0: HCA       */
  int32_t page_blocks;  /* 0: entry planes [B][MB][...]; PB: paged (above)     */
  int64_t max_blocks;   /* MB >= 1                                             */
  int64_t len_min;      /* host mirror: min over rows of seq_len               */
  int64_t len_max;      /* host mirror: max over rows of seq_len               */
  int32_t *seq_len;
  uint32_t *sync;
  uint8_t *nope;
  uint16_t *rope;
  float *kv_scale;
  uint8_t *idx_code;
  uint8_t *idx_scale;
  uint16_t *ring_kv;
  float *ring_gate;
  float *ring_ikey;
  float *ring_igate;
  const float *pos_bias;
  const float *ipos_bias;
  const int32_t *page_table;  /* [B][MB / PB] when page_blocks > 0, else NULL  */
  int64_t pool_pages;         /* pages in the entry planes when paged, else 0  */
} lca_layer;

/*
 * lca_compress_append -- [AGENT] hybrid-attention section (softmax-gated
 * pooling with a learned position bias, FP8 entries with BF16 RoPE dims, FP4
 * indexer keys); [ARCH] 2.1 (the compressor updates the compressed cache; the
 * window store overwrites cyclically).
 *
 * Appends n tokens to every row at positions seq_len .. seq_len+n-1, then
 * writes every entry that these tokens complete (blocks b with
 * seq_len < (b+1)*m <= seq_len+n):
 *   a_i = gate[i][c] + pos_bias[i][c];  w_i = softmax_i(a) per channel c;
 *   y_c = sum_i w_i * x_i[c]  (x from bf16 kv; fp32 arithmetic)
 *   dims 0..447 -> e4m3fn codes with a per-64 fp32 scale amax/448;
 *   dims 448..511 -> bf16 (round to nearest even);
 *   CSA: the 64-d indexer stream (ikey, igate, ipos_bias) is pooled the same
 *   way and stored as two MXFP4 blocks (e2m1 codes, E8M0 = floor(log2 amax)-2).
 * Then seq_len += n (on the device) and len_min/len_max += n (on the host).
 *   kv    uint16 [B][n][512] bf16      gate  float [B][n][512]
 *   ikey  float  [B][n][64]            igate float [B][n][64]  (CSA; NULL for HCA)
 * Needs ring >= n + max(window, ratio) - 1 and max_blocks*ratio >= len_max+n.
 * n == 0 is a no-op.  Errors: EINVAL, EUNSUPPORTED, ECAPACITY, EHIP.
 */
int lca_compress_append(lca_layer *layer, const uint16_t *kv, const float *gate,
                        const float *ikey, const float *igate, int32_t n,
                        hipStream_t stream);

/*
 * lca_indexer_topk -- [AGENT] hybrid-attention section (FP4 lightning indexer:
 * ReLU-scored multi-head dot products, top-k compressed blocks kept);
 * [REPORT] 核心技術 (the indexer picks top-k compressed blocks).
 *
 * For each row and each of the last n_q appended tokens (query position
 * p = seq_len - n_q + i), over the visible blocks b < floor((p+1)/m):
 *   q_h = MXFP4(iq[h]) (quantized in the call, same rule as the keys);
 *   dot_h = exact dot of the dequantized q_h and key b, rounded once to fp32;
 *   score = +0, then score = fmaf(iw[h], max(dot_h, 0), score) for
 *           h = 0 .. H_I-1 (one chain, ascending heads); a zero score is +0;
 *   topk = the min(k, visible) largest (score desc, block asc), written in
 *          ascending block order, padded with -1.
 *   iq    float [B][n_q][H_I][64]     iw    float [B][n_q][H_I]
 *   topk  int32 [B][n_q][k]           (output)
 * Needs a CSA layer, 1 <= H_I <= 32, 1 <= k <= 2048, n_q <= len_min and
 * max_blocks <= 524288.  ws must hold lca_indexer_workspace(...) bytes and
 * be used by nothing but lca_indexer_topk.  Its first bytes (out[3] of
 * lca_indexer_layout: per-row counters and one histogram per query) must be
 * zero when a call starts, and every call leaves them zero again.  A call
 * writes its scores and lists after them, so a workspace that served a call
 * with fewer queries (B * n_q) holds non-zero bytes where a call with more
 * queries keeps its counters and histograms: zero-fill it again before such
 * a call (or keep one workspace per query count).  A zero-filled workspace
 * is ready for any call.
 * One query per row and H_I <= 16 (decode): the selection runs in the
 * scoring launch (the row's last scoring workgroup selects from candidates
 * the others kept); LCA_TOPK_FUSED = 0 runs it as a launch of its own.
 * The kernels are chosen from the shapes; for tests and tuning the choice
 * can be forced with lca_set_tuning (keep it unchanged between the workspace
 * query and the call, as the workspace size follows the choice):
 * LCA_SCORE_TILE (0/1: multi-query score kernel), LCA_TOPK_CAND (0/1:
 * candidate lists with it), LCA_TOPK_SLICED (0/1: the selection split over
 * part workgroups), LCA_TOPK_FUSED (0/1: decode selection inside the scoring
 * launch), LCA_SCORE_CPW (chunks of 1024 blocks per scoring workgroup).
 */
size_t lca_indexer_workspace(const lca_layer *layer, int32_t n_q, int32_t H_I, int32_t k);

/*
 * lca_indexer_layout -- where lca_indexer_topk leaves each query's scores in
 * its workspace, for callers that inspect them (host only, enqueues nothing).
 * Same arguments as lca_indexer_workspace; out receives 8 values:
 *   out[0] stride S (key slots per query row); out[1] byte offset of the
 *   scores; out[3] bytes at the start of the workspace that must be zero
 *   when a call starts (per-row counters and per-query histograms; every
 *   call leaves them zero).  A key is the score's order key (the fp32 bits,
 *   all bits flipped for a negative score, the sign bit set otherwise).
 *   out[2] = 0: uint32 keys [B * n_q][S]; slot b holds block b's key for
 *     every visible block b.
 *   out[2] = 1 (candidate lists of multi-query rows): uint32 pairs (key, t)
 *     [B * n_q][S].  The query has out[5] lists; the length of list i is
 *     entry i of the uint32 array [B * n_q][out[5]] at byte offset out[4].
 *     With W = out[6] and span = out[7], list i = 32 (c W + v) + col (c, v,
 *     col with v < W, col < 32) has entry j in slot c * span + 32 v + 32 W j
 *     + col, and that entry's t names block c * span + 32 (v + W t) + col.
 *   out[2] = 2 (candidate segments of one-query rows, the selection inside
 *     the scoring launch): uint32 pairs (key, block) [B * n_q][S]; the query
 *     has out[5] segments of out[7] blocks; segment s holds, from slot
 *     s * out[7] on, count pairs for blocks of its own range in ascending
 *     order, count being entry s of the uint32 array [B * n_q][out[5]] at
 *     byte offset out[4].
 *   For kinds 1 and 2 every block whose key lies in the top-12-bit bin of
 *   the query's k-th largest key, or above it, is kept.  Unused entries of
 *   out are -1 or 0.
 * Returns LCA_OK or LCA_EINVAL (NULL layer or out, n_q < 1).
 */
int lca_indexer_layout(const lca_layer *layer, int32_t n_q, int32_t H_I, int32_t k, int64_t *out);
int lca_indexer_topk(const lca_layer *layer, const float *iq, const float *iw, int32_t n_q,
                     int32_t H_I, int32_t k, int32_t *topk, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * lca_indexer_topk_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops or harnesses that forbid
 * hipMalloc): lca_indexer_topk with the same arguments except the workspace,
 * which is a static device array inside the library of
 * LCA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held until the process ends.
 * Calls whose workspace (lca_indexer_workspace) exceeds that size fail with
 * LCA_EWORKSPACE before anything is enqueued (decode steps fit: 128K context
 * at B = 32 needs about 5 MB; a 4096-query prefill chunk does not).  The
 * call clears the array's histogram part with a fill kernel first, so any
 * sequence of shapes is valid.  All calls on one GPU share the array: calls
 * that may overlap on one GPU (different streams without ordering) race.
 * Results are those of lca_indexer_topk.  Errors: as lca_indexer_topk, plus
 * EWORKSPACE for a call too large for the array and EHIP if the array's
 * address cannot be found.
 */
#define LCA_NOALLOC_SCRATCH_BYTES (32u << 20)
int lca_indexer_topk_noalloc(const lca_layer *layer, const float *iq, const float *iw, int32_t n_q,
                             int32_t H_I, int32_t k, int32_t *topk, hipStream_t stream);

/*
 * lca_decode_append_topk -- one decode step of a CSA layer up to the top-k:
 * the compressor takes the new token and the lightning index selects among
 * the compressed blocks (pnsm.cn "DeepSeek V4 架构深度解析" page, section
 * 2.1: the compressor updates the compressed cache, the index keeps the
 * top-k; vibecoco.ai "DeepSeek V4 agent architecture" page, section
 * 混合注意力).  Exactly lca_compress_append(layer, kv, gate, ikey, igate, 1)
 * followed by lca_indexer_topk(layer, iq, iw, 1, H_I, k, topk, ws, ...),
 * with the same results, arguments, layouts and status bits; in one launch
 * when the decode selection runs inside the scoring launch (H_I <= 16, the
 * automatic choice) and the layer's blocks hold at most 8 tokens (ratio <=
 * 8), else as those two launches.  Needs a CSA layer (has_indexer).  ws
 * holds lca_decode_append_workspace(layer, H_I, k) bytes (the indexer's
 * workspace for the layer one token longer, under the same rules).  Updates
 * len_min / len_max like lca_compress_append.
 */
size_t lca_decode_append_workspace(const lca_layer *layer, int32_t H_I, int32_t k);
int lca_decode_append_topk(lca_layer *layer, const uint16_t *kv, const float *gate, const float *ikey,
                           const float *igate, const float *iq, const float *iw, int32_t H_I, int32_t k,
                           int32_t *topk, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * lca_csa_attend -- [ARCH] 2.1 (one attention over the sliding-window KV and
 * the top-k selected compressed KV); [AGENT] hybrid-attention section (recent
 * tokens at raw precision).
 *
 * For each row, query i (position p = seq_len - n_q + i) and head h: one
 * softmax attention, logit = scale * (q . k), over the keys
 *   { entry b : b listed in topk[row][i][0..k), 0 <= b < floor((p+1)/m) }
 *   then the raw window tokens max(0, p-W+1) .. p,
 * where an entry's vector is e4m3(code)*scale of its 64-group for dims
 * 0..447 and the bf16 RoPE dims 448..511, a window token's vector is its raw
 * bf16 KV, and every key is also its value.  Entries outside the visible
 * range and -1 are skipped; listed indices must be distinct.
 *   q     uint16 [B][n_q][H][512] bf16     out float [B][n_q][H][512]
 * Needs 1 <= H <= 128, 1 <= k <= 2048, n_q <= len_min and
 * n_q + window - 1 <= ring.  ws must hold lca_attend_workspace(...) bytes.
 * The number of key splits (and so the workspace size) follows the shapes;
 * lca_set_tuning("LCA_ATTEND_SPLITS", n) forces it for tests and tuning
 * (keep it unchanged between the query and the call).
 */
size_t lca_attend_workspace(const lca_layer *layer, int32_t n_q, int32_t H, int32_t k);
int lca_csa_attend(const lca_layer *layer, const uint16_t *q, int32_t n_q, int32_t H,
                   const int32_t *topk, int32_t k, float scale, float *out, void *ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * lca_hca_attend -- [AGENT] hybrid-attention section and [REPORT] 核心技術
 * (HCA: 128x compression, no sparse selection, every query attends densely to
 * all compressed blocks), plus the raw window branch.
 *
 * Same as lca_csa_attend with the key set = every visible entry
 * b < floor((p+1)/m), then the window tokens.  Pass k = 0 to
 * lca_attend_workspace for this call.
 */
int lca_hca_attend(const lca_layer *layer, const uint16_t *q, int32_t n_q, int32_t H,
                   float scale, float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * lca_set_tuning -- force a kernel choice (names above: LCA_SCORE_TILE,
 * LCA_TOPK_CAND, LCA_TOPK_SLICED, LCA_TOPK_FUSED, LCA_SCORE_CPW,
 * LCA_ATTEND_SPLITS); value < 0 restores the automatic choice.  The initial
 * values come from environment variables of the same names, read once when
 * the library is loaded.  Process-wide; not meant to change while calls are
 * being made on other threads.  Errors: EINVAL (NULL or unknown name).
 */
int lca_set_tuning(const char *name, int32_t value);

/* Library version and last error (thread-local, never NULL). */
int lca_abi_version(void);
const char *lca_last_error(void);

/*
 * Kernel timing.  Between lca_timing_begin(kernel) and lca_timing_end(), every
 * launch of the named kernel is bracketed by HIP events on its stream;
 * lca_timing_end synchronizes on them and returns the summed duration (ms)
 * and the number of launches.  Kernel names: "indexer_score", "topk_select",
 * "attend", "attend_combine", "compress" ("topk_select" spans the
 * selection's one or two launches).  At most 4096 launches are
 * recorded per session.  Errors: EINVAL (unknown name or nested session),
 * EHIP.
 */
int lca_timing_begin(const char *kernel);
int lca_timing_end(double *total_ms, int64_t *launches);
/*
 * The per-launch durations (ms, launch order) of the session the last
 * lca_timing_end closed: copies min(cap, launches) of them into ms and sets
 * *launches to their number (ms may be NULL when cap is 0).  Errors: EINVAL.
 */
int lca_timing_durations(float *ms, int64_t cap, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif
