// lca_internal.h -- host-side glue shared by the translation units of
// liblca.so: launch entry points, kernel ids for timing, workspace layouts.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lca.h"

namespace lca {

enum KernelId {
  kKernelNone = -1,
  kKernelIndexerScore = 0,
  kKernelTopkSelect = 1,
  kKernelAttend = 2,
  kKernelAttendCombine = 3,
  kKernelCompress = 4,
  kKernelCount = 5
};

// Kernel-choice overrides (lca_set_tuning / the LCA_* environment at load);
// tuning(id) < 0 means automatic.
enum TuneId {
  kTuneScoreTile = 0,
  kTuneTopkCand,
  kTuneTopkSliced,
  kTuneTopkFused,
  kTuneScoreCpw,
  kTuneAttendSplits,
  kTuneCount
};
int tuning(TuneId id);

// The layer's entry placement for the kernels (the PageMap of lca_device.h):
// fills table, max_blocks, pages_per_row, shift, pool_pages.
template <class PM>
inline PM page_map_of(const lca_layer* L) {
  PM pm{};
  pm.table = L->page_table;
  pm.max_blocks = L->max_blocks;
  pm.shift = -1;
  if (L->page_blocks > 0) {
    int sh = 0;
    while ((1 << sh) < L->page_blocks) sh++;
    pm.shift = sh;
    pm.pages_per_row = (int32_t)(L->max_blocks / L->page_blocks);
    pm.pool_pages = (int32_t)L->pool_pages;
  }
  return pm;
}

// Records HIP events around one launch when a timing session for `id` is open.
struct TimedLaunch {
  TimedLaunch(KernelId id, hipStream_t s);
  int done();  // records the stop event; returns LCA_OK or LCA_EHIP
  int slot;
  hipStream_t stream;
};

int set_error(int code, const char* fmt, ...);

int launch_compress(const lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                    const float* igate, int n, hipStream_t stream);

// Indexer workspace (byte offsets in the plan): the fused selection's per-row
// arrival counters and the per-query key histograms [rows][4096] first --
// [0, zero_bytes) is zero on entry and on return -- then the scores: order
// keys [rows][stride], or (key, t) / (key, block) pairs [rows][stride] for
// candidate lists; then, when the selection is split over parts, the
// per-(query, part) listed-key counts, bitmap words and lists; then the
// candidate list lengths.  rows = B * n_q.
struct IndexerPlan {
  int64_t stride;       // key slots per score row (>= visible blocks of any query)
  int chunks;           // score workgroups per row (non-fused decode kernel, tile kernel)
  int cpw;              // chunks of 1024 blocks per workgroup (per half-workgroup when fused)
  int slices;           // selection parts per query on their own workgroups (0: one workgroup)
  int tile;             // 0: one query per score workgroup; 8 or 4: queries per wavefront of the tile kernel
  int qgroups;          // tile kernel: query groups per row
  bool cand;            // tile kernel keeps candidate lists: (key, visit) pairs
  int cand_lists;       // lists per query: chunks x cand_waves x 32
  int cand_waves;       // wavefronts per tile workgroup
  int cand_span;        // blocks per chunk
  bool fused;           // decode scoring selects in its own launch from per-workgroup candidates
  int fused_wgs;        // fused: scoring workgroups per row (candidate segments)
  int fused_span;       // fused: blocks per scoring workgroup
  size_t fused_lds;     // fused: dynamic LDS bytes (keys, then the selection bitmap)
  size_t off_done, off_hist, off_keys, off_part_count, off_part_bits, off_part_cand, off_cand_count;
  size_t zero_bytes;    // [0, zero_bytes): counters and histograms, zero between calls
  size_t total_bytes;
  size_t total() const { return total_bytes; }
};
IndexerPlan plan_indexer(const lca_layer* L, int n_q, int H_I, int k);
// argument checks of lca_indexer_topk (everything but the workspace)
int indexer_validate(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                     const int32_t* topk);
struct CompressArgs;
// append (fused plans only): the launch also appends one token per row with
// these arguments (seq_len then holds the length before the token)
int launch_indexer(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                   int32_t* topk, void* ws, const IndexerPlan& plan, hipStream_t stream,
                   const CompressArgs* append = nullptr);
// lca_decode_append_topk: the append of one token per row to L and the
// selection on `after` (L's host mirrors one token longer), in one launch
// when the plan selects inside the scoring launch and blocks hold at most 8
// tokens, else as the two launches
int launch_decode_append(const lca_layer* L, const lca_layer* after, const uint16_t* kv, const float* gate,
                         const float* ikey, const float* igate, const float* iq, const float* iw, int H_I,
                         int k, int32_t* topk, void* ws, const IndexerPlan& plan, hipStream_t stream);

// Attention: split-K partials (m, l) and unnormalised o per (row, split, head).
struct AttendPlan {
  int splits;
  int head_groups;
  int64_t max_keys;     // upper bound of keys per query
  int chunk;            // keys per split (multiple of the tile)
  size_t ml_bytes, o_bytes;
};
AttendPlan plan_attend(const lca_layer* L, int n_q, int H, int k, bool csa);
int launch_attend(const lca_layer* L, const uint16_t* q, int n_q, int H, const int32_t* topk, int k,
                  float scale, float* out, void* ws, const AttendPlan& plan, hipStream_t stream);

}  // namespace lca
