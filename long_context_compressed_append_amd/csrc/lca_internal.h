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

// Indexer workspace: per-query key histograms [rows][4096] (zero between
// calls), then scores as order-preserving uint32 keys [rows][stride], then,
// when the selection is split over rounds, the per-(query, round) listed-key
// counts, bitmap words and lists.  rows = B * n_q.
struct IndexerPlan {
  int64_t stride;       // keys per score row (>= visible blocks of any query)
  int chunks;           // workgroups per score row
  int cpw;              // chunks of 1024 blocks per workgroup
  int slices;           // selection parts per query on their own workgroups (0: one workgroup)
  int tile;             // 0: one query per score workgroup; 8 or 4: queries per wavefront of the tile kernel
  int qgroups;          // tile kernel: query groups per row
  size_t keys_bytes;
  size_t hist_bytes;    // per-query histograms at the start of the workspace
  size_t part_count_bytes, part_bits_bytes, part_cand_bytes;
  bool cand;            // tile kernel keeps candidate lists: (key, visit) pairs, list lengths at the end
  int cand_lists;       // lists per query: chunks x cand_waves x 32
  int cand_waves;       // wavefronts per tile workgroup
  int cand_span;        // blocks per chunk
  size_t cand_count_bytes;
  bool fused;           // decode scoring selects in its own launch (per-row counters at the end)
  size_t row_done_bytes;
  size_t total() const {
    return hist_bytes + keys_bytes + part_count_bytes + part_bits_bytes + part_cand_bytes + cand_count_bytes +
           row_done_bytes;
  }
};
IndexerPlan plan_indexer(const lca_layer* L, int n_q, int H_I, int k);
int launch_indexer(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                   int32_t* topk, void* ws, const IndexerPlan& plan, hipStream_t stream);

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
