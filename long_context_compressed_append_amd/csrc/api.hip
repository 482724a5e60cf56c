// api.hip -- the C ABI of liblca.so: argument validation (before anything is
// enqueued), workspace sizing, launches, kernel timing and error reporting.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <stdlib.h>
#include <vector>

#include "lca_internal.h"

namespace lca {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// ------------------------------------------------------------------ tuning
// Kernel-choice overrides: read once from the environment when the library
// is loaded, changed afterwards only through lca_set_tuning.  -1: automatic.
namespace {
const char* kTuneNames[kTuneCount] = {"LCA_SCORE_TILE", "LCA_TOPK_CAND", "LCA_TOPK_SLICED",
                                      "LCA_TOPK_FUSED", "LCA_SCORE_CPW", "LCA_ATTEND_SPLITS"};
struct Tuning {
  std::atomic<int> v[kTuneCount];
  Tuning() {
    for (int i = 0; i < kTuneCount; i++) {
      const char* e = getenv(kTuneNames[i]);
      v[i].store((e && *e) ? atoi(e) : -1, std::memory_order_relaxed);
    }
  }
};
Tuning g_tuning;
}  // namespace

int tuning(TuneId id) { return g_tuning.v[id].load(std::memory_order_relaxed); }

// ------------------------------------------------------------------ timing
namespace {
struct Timing {
  std::mutex mu;
  std::atomic<int> open{0};   // a session is open: launches take the lock
  int kernel = kKernelNone;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<float> last;    // per-launch durations of the last closed session
};
Timing g_timing;
constexpr int kMaxTimed = 4096;
const char* kKernelNames[kKernelCount] = {"indexer_score", "topk_select", "attend", "attend_combine",
                                          "compress"};
}  // namespace

TimedLaunch::TimedLaunch(KernelId id, hipStream_t s) : slot(-1), stream(s) {
  if (!g_timing.open.load(std::memory_order_acquire)) return;   // no session: no lock, no events
  std::lock_guard<std::mutex> g(g_timing.mu);
  if (g_timing.kernel != id || g_timing.used >= kMaxTimed) return;
  slot = g_timing.used++;
  if (slot >= (int)g_timing.start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      g_timing.used--;
      slot = -1;
      return;
    }
    g_timing.start.push_back(a);
    g_timing.stop.push_back(b);
  }
  hipEventRecord(g_timing.start[slot], stream);
}

int TimedLaunch::done() {
  hipError_t e = hipGetLastError();
  if (slot >= 0) hipEventRecord(g_timing.stop[slot], stream);
  if (e != hipSuccess) return set_error(LCA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return LCA_OK;
}

// ------------------------------------------------------------------ validation

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_layer(const lca_layer* L) {
  if (!L) return set_error(LCA_EINVAL, "layer is NULL");
  if (L->batch < 1) return set_error(LCA_EINVAL, "batch must be >= 1 (got %d)", L->batch);
  if (L->ratio < 1 || L->ratio > 128 || (L->ratio & (L->ratio - 1)))
    return set_error(LCA_EUNSUPPORTED, "ratio must be a power of two in 1..128 (got %d)", L->ratio);
  if (L->window < 1) return set_error(LCA_EINVAL, "window must be >= 1 (got %d)", L->window);
  if (L->ring < L->window)
    return set_error(LCA_ECAPACITY, "ring (%d) must be >= window (%d)", L->ring, L->window);
  if (L->max_blocks < 1) return set_error(LCA_EINVAL, "max_blocks must be >= 1");
  if (L->max_blocks > (int64_t)1 << 31) return set_error(LCA_EUNSUPPORTED, "max_blocks too large");
  if (L->len_min < 0 || L->len_max < L->len_min)
    return set_error(LCA_EINVAL, "len_min/len_max inconsistent (%lld, %lld)", (long long)L->len_min,
                     (long long)L->len_max);
  if (L->len_max > (int64_t)0x7FFFFFFF - 65536) return set_error(LCA_EUNSUPPORTED, "sequence too long");
  if (L->has_indexer != 0 && L->has_indexer != 1) return set_error(LCA_EINVAL, "has_indexer must be 0 or 1");
  const void* must[] = {L->seq_len, L->sync, L->nope, L->rope, L->kv_scale, L->ring_kv, L->ring_gate,
                        L->pos_bias};
  const char* names[] = {"seq_len", "sync", "nope", "rope", "kv_scale", "ring_kv", "ring_gate", "pos_bias"};
  for (int i = 0; i < 8; i++) {
    if (!must[i]) return set_error(LCA_EINVAL, "layer.%s is NULL", names[i]);
    if (!aligned16(must[i])) return set_error(LCA_EINVAL, "layer.%s is not 16-byte aligned", names[i]);
  }
  if (L->has_indexer) {
    const void* im[] = {L->idx_code, L->idx_scale, L->ring_ikey, L->ring_igate, L->ipos_bias};
    const char* in[] = {"idx_code", "idx_scale", "ring_ikey", "ring_igate", "ipos_bias"};
    for (int i = 0; i < 5; i++) {
      if (!im[i]) return set_error(LCA_EINVAL, "layer.%s is NULL on an indexer layer", in[i]);
      if (!aligned16(im[i])) return set_error(LCA_EINVAL, "layer.%s is not 16-byte aligned", in[i]);
    }
  }
  const int32_t pb = L->page_blocks;
  if (pb == 0) {
    if (L->page_table || L->pool_pages)
      return set_error(LCA_EINVAL, "page_table / pool_pages set on a layer with page_blocks 0");
  } else {
    if (pb < 64 || pb > 65536 || (pb & (pb - 1)))
      return set_error(LCA_EUNSUPPORTED, "page_blocks must be 0 or a power of two in 64..65536 (got %d)", pb);
    if (L->max_blocks % pb)
      return set_error(LCA_EINVAL, "max_blocks (%lld) is not a multiple of page_blocks (%d)",
                       (long long)L->max_blocks, pb);
    if (!L->page_table) return set_error(LCA_EINVAL, "layer.page_table is NULL on a paged layer");
    if ((uintptr_t)L->page_table & 3u) return set_error(LCA_EINVAL, "layer.page_table is not 4-byte aligned");
    if (L->pool_pages < 1) return set_error(LCA_EINVAL, "pool_pages must be >= 1 on a paged layer");
    if (L->pool_pages > (((int64_t)1 << 31) - 1) / pb)
      return set_error(LCA_EUNSUPPORTED, "pool_pages * page_blocks must stay below 2^31");
  }
  return LCA_OK;
}

static int check_ptr(const void* p, const char* name) {
  if (!p) return set_error(LCA_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return set_error(LCA_EINVAL, "%s is not 16-byte aligned", name);
  return LCA_OK;
}

int indexer_validate(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                     const int32_t* topk) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!L->has_indexer) return set_error(LCA_EINVAL, "lca_indexer_topk needs an indexer (CSA) layer");
  if (n_q < 1) return set_error(LCA_EINVAL, "n_q must be >= 1 (got %d)", n_q);
  if (H_I < 1 || H_I > 32) return set_error(LCA_EUNSUPPORTED, "H_I must be in 1..32 (got %d)", H_I);
  if (k < 1 || k > 2048) return set_error(LCA_EUNSUPPORTED, "k must be in 1..2048 (got %d)", k);
  if (n_q > L->len_min)
    return set_error(LCA_EINVAL, "n_q (%d) exceeds the shortest row (%lld tokens)", n_q,
                     (long long)L->len_min);
  if (L->max_blocks > 524288) return set_error(LCA_EUNSUPPORTED, "max_blocks above 524288");
  if ((int64_t)L->batch * n_q > 0x7FFFFFFF / 2) return set_error(LCA_EUNSUPPORTED, "too many queries");
  if ((rc = check_ptr(iq, "iq")) || (rc = check_ptr(iw, "iw")) || (rc = check_ptr(topk, "topk")))
    return rc;
  return LCA_OK;
}

}  // namespace lca

using namespace lca;

extern "C" {

int lca_abi_version(void) { return LCA_ABI_VERSION; }

const char* lca_last_error(void) { return g_err; }

// argument checks of an append of n >= 1 tokens per row
static int append_validate(const lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                           const float* igate, int32_t n) {
  int rc;
  if ((rc = check_ptr(kv, "kv")) || (rc = check_ptr(gate, "gate"))) return rc;
  if (L->has_indexer) {
    if ((rc = check_ptr(ikey, "ikey")) || (rc = check_ptr(igate, "igate"))) return rc;
  }
  const int64_t need_ring = (int64_t)n + (L->window > L->ratio ? L->window : L->ratio) - 1;
  if (L->ring < need_ring)
    return set_error(LCA_ECAPACITY, "ring (%d) must be >= n + max(window, ratio) - 1 = %lld", L->ring,
                     (long long)need_ring);
  if ((L->len_max + n) / L->ratio > L->max_blocks)
    return set_error(LCA_ECAPACITY, "max_blocks (%lld) too small for %lld tokens at ratio %d",
                     (long long)L->max_blocks, (long long)(L->len_max + n), L->ratio);
  return LCA_OK;
}

int lca_compress_append(lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                        const float* igate, int32_t n, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (n < 0) return set_error(LCA_EINVAL, "n must be >= 0 (got %d)", n);
  if (n == 0) return LCA_OK;
  if ((rc = append_validate(L, kv, gate, ikey, igate, n))) return rc;
  rc = launch_compress(L, kv, gate, ikey, igate, n, stream);
  if (rc) return rc;
  L->len_min += n;
  L->len_max += n;
  return LCA_OK;
}

size_t lca_indexer_workspace(const lca_layer* L, int32_t n_q, int32_t H_I, int32_t k) {
  if (!L || n_q < 1 || L->ratio < 1 || L->batch < 1) return 0;
  IndexerPlan pl = plan_indexer(L, n_q, H_I, k);
  return pl.total();
}

int lca_indexer_layout(const lca_layer* L, int32_t n_q, int32_t H_I, int32_t k, int64_t* out) {
  if (!L || n_q < 1 || L->ratio < 1 || L->batch < 1) return set_error(LCA_EINVAL, "invalid layer or n_q");
  if (!out) return set_error(LCA_EINVAL, "out is NULL");
  IndexerPlan pl = plan_indexer(L, n_q, H_I, k);
  out[0] = pl.stride;
  out[1] = (int64_t)pl.off_keys;
  out[2] = pl.fused ? 2 : (pl.cand ? 1 : 0);
  out[3] = (int64_t)pl.zero_bytes;
  out[4] = (pl.cand || pl.fused) ? (int64_t)pl.off_cand_count : -1;
  out[5] = pl.fused ? pl.fused_wgs : pl.cand_lists;
  out[6] = pl.cand ? pl.cand_waves : 0;
  out[7] = pl.fused ? pl.fused_span : pl.cand_span;
  return LCA_OK;
}

int lca_indexer_topk(const lca_layer* L, const float* iq, const float* iw, int32_t n_q, int32_t H_I,
                     int32_t k, int32_t* topk, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = indexer_validate(L, iq, iw, n_q, H_I, k, topk);
  if (rc) return rc;
  IndexerPlan pl = plan_indexer(L, n_q, H_I, k);
  const size_t need = pl.total();
  if (!ws || ws_bytes < need)
    return set_error(LCA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return set_error(LCA_EINVAL, "workspace is not 16-byte aligned");
  return launch_indexer(L, iq, iw, n_q, H_I, k, topk, ws, pl, stream);
}

// the layer as the selection of lca_decode_append_topk sees it: one token longer
static lca_layer one_longer(const lca_layer* L) {
  lca_layer a = *L;
  a.len_min += 1;
  a.len_max += 1;
  return a;
}

size_t lca_decode_append_workspace(const lca_layer* L, int32_t H_I, int32_t k) {
  if (!L || L->ratio < 1 || L->batch < 1) return 0;
  const lca_layer after = one_longer(L);
  return plan_indexer(&after, 1, H_I, k).total();
}

int lca_decode_append_topk(lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                           const float* igate, const float* iq, const float* iw, int32_t H_I, int32_t k,
                           int32_t* topk, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!L->has_indexer) return set_error(LCA_EINVAL, "the layer has no indexer (an HCA layer)");
  if ((rc = append_validate(L, kv, gate, ikey, igate, 1))) return rc;
  const lca_layer after = one_longer(L);
  if ((rc = indexer_validate(&after, iq, iw, 1, H_I, k, topk))) return rc;
  IndexerPlan pl = plan_indexer(&after, 1, H_I, k);
  const size_t need = pl.total();
  if (!ws || ws_bytes < need)
    return set_error(LCA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return set_error(LCA_EINVAL, "workspace is not 16-byte aligned");
  rc = launch_decode_append(L, &after, kv, gate, ikey, igate, iq, iw, H_I, k, topk, ws, pl, stream);
  if (rc) return rc;
  L->len_min += 1;
  L->len_max += 1;
  return LCA_OK;
}

size_t lca_attend_workspace(const lca_layer* L, int32_t n_q, int32_t H, int32_t k) {
  if (!L || n_q < 1 || H < 1 || L->ratio < 1 || L->batch < 1) return 0;
  AttendPlan pl = plan_attend(L, n_q, H, k, k > 0);
  if (pl.splits <= 1) return 0;
  return ((pl.ml_bytes + 255) & ~(size_t)255) + pl.o_bytes;
}

static int attend_common(const lca_layer* L, const uint16_t* q, int32_t n_q, int32_t H,
                         const int32_t* topk, int32_t k, float scale, float* out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (n_q < 1) return set_error(LCA_EINVAL, "n_q must be >= 1 (got %d)", n_q);
  if (H < 1 || H > 128) return set_error(LCA_EUNSUPPORTED, "H must be in 1..128 (got %d)", H);
  if (n_q > L->len_min)
    return set_error(LCA_EINVAL, "n_q (%d) exceeds the shortest row (%lld tokens)", n_q,
                     (long long)L->len_min);
  if ((int64_t)n_q + L->window - 1 > L->ring)
    return set_error(LCA_ECAPACITY, "ring (%d) must be >= n_q + window - 1 = %lld", L->ring,
                     (long long)n_q + L->window - 1);
  if (!(scale == scale) || scale == 0.0f) return set_error(LCA_EINVAL, "scale must be finite and non-zero");
  if ((int64_t)L->batch * n_q > 65535) return set_error(LCA_EUNSUPPORTED, "B * n_q above 65535");
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(out, "out"))) return rc;
  if (topk) {
    if (k < 1 || k > 2048) return set_error(LCA_EUNSUPPORTED, "k must be in 1..2048 (got %d)", k);
    if ((rc = check_ptr(topk, "topk"))) return rc;
  }
  AttendPlan pl = plan_attend(L, n_q, H, k, topk != nullptr);
  const size_t need = pl.splits > 1 ? ((pl.ml_bytes + 255) & ~(size_t)255) + pl.o_bytes : 0;
  if (need && (!ws || ws_bytes < need))
    return set_error(LCA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (need && !aligned16(ws)) return set_error(LCA_EINVAL, "workspace is not 16-byte aligned");
  return launch_attend(L, q, n_q, H, topk, k, scale, out, ws, pl, stream);
}

int lca_csa_attend(const lca_layer* L, const uint16_t* q, int32_t n_q, int32_t H, const int32_t* topk,
                   int32_t k, float scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!topk) return set_error(LCA_EINVAL, "topk is NULL");
  return attend_common(L, q, n_q, H, topk, k, scale, out, ws, ws_bytes, stream);
}

int lca_hca_attend(const lca_layer* L, const uint16_t* q, int32_t n_q, int32_t H, float scale,
                   float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return attend_common(L, q, n_q, H, nullptr, 0, scale, out, ws, ws_bytes, stream);
}

int lca_timing_begin(const char* kernel) {
  if (!kernel) return set_error(LCA_EINVAL, "kernel name is NULL");
  int id = kKernelNone;
  for (int i = 0; i < kKernelCount; i++)
    if (!strcmp(kernel, kKernelNames[i])) id = i;
  if (id == kKernelNone) return set_error(LCA_EINVAL, "unknown kernel name '%s'", kernel);
  std::lock_guard<std::mutex> g(g_timing.mu);
  if (g_timing.kernel != kKernelNone) return set_error(LCA_EINVAL, "a timing session is already open");
  g_timing.kernel = id;
  g_timing.used = 0;
  g_timing.open.store(1, std::memory_order_release);
  return LCA_OK;
}

int lca_timing_end(double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  if (g_timing.kernel == kKernelNone) return set_error(LCA_EINVAL, "no timing session is open");
  double tot = 0.0;
  g_timing.last.clear();
  for (int i = 0; i < g_timing.used; i++) {
    if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess)
      return set_error(LCA_EHIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]) != hipSuccess)
      return set_error(LCA_EHIP, "hipEventElapsedTime failed");
    tot += ms;
    g_timing.last.push_back(ms);
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = g_timing.used;
  g_timing.kernel = kKernelNone;
  g_timing.used = 0;
  g_timing.open.store(0, std::memory_order_release);
  return LCA_OK;
}

int lca_timing_durations(float* ms, int64_t cap, int64_t* launches) {
  std::lock_guard<std::mutex> g(g_timing.mu);
  const int64_t n = (int64_t)g_timing.last.size();
  if (launches) *launches = n;
  if (cap > 0 && !ms) return set_error(LCA_EINVAL, "durations buffer is NULL");
  for (int64_t i = 0; i < n && i < cap; i++) ms[i] = g_timing.last[i];
  return LCA_OK;
}

int lca_set_tuning(const char* name, int32_t value) {
  if (!name) return set_error(LCA_EINVAL, "tuning name is NULL");
  for (int i = 0; i < kTuneCount; i++)
    if (!strcmp(name, kTuneNames[i])) {
      g_tuning.v[i].store(value < 0 ? -1 : value, std::memory_order_relaxed);
      return LCA_OK;
    }
  return set_error(LCA_EINVAL, "unknown tuning name '%s'", name);
}

}  // extern "C"
