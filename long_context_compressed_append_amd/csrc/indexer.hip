// indexer.hip -- lightning-indexer scores on the FP4 matrix cores, then an
// exact top-k selection.
//
// vibecoco.ai "DeepSeek V4 agent architecture" page, section 混合注意力: an
// FP4 lightning indexer scores compressed blocks with ReLU-scored multi-head
// dot products and the top-k blocks are kept.  agents-report.net
// "DeepSeek-V4：交錯壓縮注意力與低位元 KV 儲存", section 核心技術: the
// indexer picks the top-k compressed blocks for the attention.
//
// Score of block b for one query (H heads):
//   dot_h  = exact dot product of MXFP4(q_h) and the block's MXFP4 key,
//            rounded once to fp32;
//   score  = +0, then score = fma(w_h, max(dot_h, 0), score) for h = 0 .. H-1
//            (one chain in ascending head order); a zero score is +0.
// The selection is bitwise reproducible.
//
// Matrix-core mapping (v_mfma_scale_f32_32x32x64_f8f6f4, both operands e2m1):
// the 32 B columns are 32 consecutive blocks (lanes l and l + 32 give the two
// MX halves of block l%32's key with their E8M0 scales); an A row carries one
// head's whole 64-d MXFP4 query (lanes l and l + 32 give its two halves and
// their scales).  In the 32x32 output layout lane l holds column l%32 and
// rows 8i + 4s + j (s = l/32, i, j < 4), i.e. 16 outputs e = 4i + j per lane.
// The heads are placed so that a lane's outputs are all the heads of one
// block, in order, and its chain needs no other lane:
//   H <= 8 or H <= 16 (decode): outputs e = kHQ g + h of lane half s belong
//     to key tile 2g + s of a group of 32/kHQ tiles.  The group's products
//     accumulate into one output: the A operand of tile t is non-zero only
//     in the rows that map to t, so every other row just adds 0.
//   H <= 32: one tile per product, heads 16s + e; the chain runs over heads
//     0..15 on the low lanes, hops to the high lanes for 16..31, and hops back.
// The hardware adds the two scaled half sums: each half's products are
// multiples of 2^(E-2) below 1152 * 2^E (E = query + key exponent of the
// half), so when both E lie in [-124, 116] and differ by at most 10 every
// partial sum needs at most 24 bits and the result is the exact dot rounded
// once.  Iterations where some block leaves these bounds take the per-half
// layout instead (a row per (head, half), unscaled products, scales applied
// in fp32, double for the far ranges), with the same result.

// While scoring, each workgroup histograms the top 12 bits of its order keys
// and adds them to a per-query histogram; the selection reads that histogram
// to find the bin that holds the k-th key, so it needs a single pass over the
// keys plus an exact ranking of the few keys inside that bin.  For prefill
// chunks the scoring keeps only keys above a running bound derived from its
// own histogram (candidate lists), and the selection passes over those.
//
// Kernels: indexer_score_kernel (one query per row; optionally selecting in
// the same launch), indexer_score_tile_kernel (many queries per row),
// topk_select_kernel / topk_slice_kernel + topk_finish_kernel (selection over
// full key rows), topk_cand_kernel (selection over candidate lists).
#include "compress_ops.h"

namespace lca {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kScoreBlocksPerIter = 32;
constexpr int kScoreItersPerWave = 8;
constexpr int kScoreBlocksPerWG = 4 * kScoreItersPerWave * kScoreBlocksPerIter;  // 1024
constexpr int kScoreTargetWGs = 512;
constexpr int kDepth = 4;          // iterations of key loads in flight per wave
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

// buffer resources: dword 3 of the descriptor selects the raw 32-bit data
// format (gfx9 layout).  Accesses at or past num_records are not performed
// (loads give 0), which stores use to drop a lane without a branch.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kDropOffset = 0x80000000u;   // past every range used here

struct ScoreArgs {
  int n_q, H, m;
  int64_t max_blocks, stride;
  PageMap pm;            // where each block's key lives
  const int32_t* seq_len;
  const uint8_t* idx_code;
  const uint8_t* idx_scale;
  const float* iq;
  const float* iw;
  uint32_t* keys;
  uint32_t* hist;        // [rows][kHistBins], zero on entry
  int cpw;               // chunks of 1024 blocks per workgroup
  int k;                 // blocks selected per query
  // candidate lists (tile kernel): keys holds (key, visit) pairs [rows][stride];
  // list lengths [rows][chunks][kTileWaves][32]
  uint32_t* cand_count;
  uint32_t* row_done;    // fused selection: workgroups of a row done, [rows], zero between calls
  int fused_span;        // fused selection: blocks per scoring workgroup (its candidate segment)
  // fused selection with the decode append (one token per row, blocks of at
  // most 8 tokens): seq_len is the length before the token; the launch
  // appends it (ring, and the block it completes) and advances seq_len
  int append;
  CompressArgs ca;
  uint32_t* status;      // the layer's status word (LCA_STATUS_* bits)
};

// Paged layers: lane l of every wavefront holds the physical page of the
// l-th page from the one holding the workgroup's first block b0 (at most 64
// pages: the plans keep a workgroup's span of blocks within 64 pages), or -1
// past the row's table.
__device__ __forceinline__ int wg_pages(const PageMap& pm, int row, int b0, int lane) {
  const int pg = (b0 >> pm.shift) + lane;
  return pg < pm.pages_per_row ? pm.table[(int64_t)row * pm.pages_per_row + pg] : -1;
}
// The physical entry of block blk (in the workgroup's span) whose 32-block
// group starts at the wavefront-uniform block g0 (a page holds whole
// groups); entry 0 (a harmless in-bounds read) when its page is unmapped.
__device__ __forceinline__ int64_t wg_entry(const PageMap& pm, int lane_pg, int b0, int g0, int blk) {
  const int pg = __builtin_amdgcn_readlane(lane_pg, ((g0 >> pm.shift) - (b0 >> pm.shift)) & 63);
  const int64_t e = phys_entry(pm, pg, blk);
  return e < 0 ? 0 : e;
}
// LCA_STATUS_PAGE when a visible block (below nv) of the workgroup's span
// [b0, b0 + span) lies on an unmapped page (one wavefront reports)
__device__ __forceinline__ void wg_pages_check(const PageMap& pm, int lane_pg, int b0, int span, int nv,
                                               int lane, uint32_t* status) {
  const int first = ((b0 >> pm.shift) + lane) << pm.shift;    // first block of the lane's page
  const int lo = first > b0 ? first : b0;
  const bool bad = first < b0 + span && lo < nv && (uint32_t)lane_pg >= (uint32_t)pm.pool_pages;
  if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) atomicOr(status, LCA_STATUS_PAGE);
}

// max(x, +0) as one integer max on the bit pattern: a negative x (sign bit
// set, a negative int) gives +0, any other x itself.  (fmaxf on a matrix-core
// output would first be canonicalised, a second instruction.)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// exact value of D0 * 2^e0 + D1 * 2^e1 rounded once to fp32, where D0, D1 are
// multiples of 1/4 below 2^11 in magnitude
__device__ __forceinline__ float exact_pair(float D0, int e0, float D1, int e1) {
  if (e0 >= -126 && e0 <= 116 && e1 >= -126 && e1 <= 116) {
    float f0 = __uint_as_float((uint32_t)(e0 + 127) << 23);
    float f1 = __uint_as_float((uint32_t)(e1 + 127) << 23);
    return __builtin_fmaf(D0, f0, __fmul_rn(D1, f1));
  }
  double v = ldexp((double)D0, e0) + ldexp((double)D1, e1);
  return (float)v;
}

// Score of the lane's block (column l % 32) when some exponent sum is out of
// the range where the scaled partials are exact fp32 normals: unscaled MFMA,
// scales in fp32 (double beyond that range).  Rows carry (head, half) pairs:
// lane half s holds heads 16 hg + 8 s .. + 7 of head group hg.  The chain
// extends on the half that holds the next heads and hops across after every
// eight, so it visits the heads in ascending order; the score ends in the
// low half.  Rare; kept out of line.
__device__ __noinline__ float score_unscaled(v8i A0, v8i A1, v8i Bm, int hgroups, int H, int kh,
                                             const int (*q_exp)[2], const float* q_w, int ke0, int ke1) {
  const v16f zero16 = {};
  float c = 0.0f;
  for (int hg = 0; hg < hgroups; hg++) {
    const v16f acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(hg ? A1 : A0, Bm, zero16, 4, 4, 0,
                                                                     127, 0, 127);
    float rl[8], wl[8];
#pragma unroll
    for (int hl = 0; hl < 8; hl++) {
      const int h = 16 * hg + 8 * kh + hl;
      const bool hv = h < H;
      rl[hl] = fmaxf(exact_pair(acc[2 * hl], (hv ? q_exp[h][0] : 0) + ke0, acc[2 * hl + 1],
                                (hv ? q_exp[h][1] : 0) + ke1), 0.0f);
      wl[hl] = hv ? q_w[h] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 2; s++) {
      // the half that holds heads 16 hg + 8 s .. extends the chain, then it hops
#pragma unroll
      for (int hl = 0; hl < 8; hl++) c = __builtin_fmaf(wl[hl], rl[hl], c);
      c = swap_halves(c);
    }
  }
  return c;
}

// inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 within each row of 16 lanes,
// then the total of row 0 (lane 15) is added to row 1, that of row 2 (lane
// 47) to row 3, and that of rows 0-1 (lane 31) to rows 2 and 3.  Lanes whose
// source lies outside the row read 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 1, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 2, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 4, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 8, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xc, 0xf, false);
  return x;
}

// The highest bin b such that the bins above b hold at least k keys of the
// histogram h, found by one wavefront while other wavefronts may still be
// adding to h: every count read was reached, so at least k keys above b
// exist in the end, whatever the interleaving.  `from` is a bin at most one
// above the answer (a previous answer + 1, as counts only grow; 0 at first):
// only bins from there up are read, and from - 1 is returned when they hold
// fewer than k keys (-1 at first).  Lane l sums its share of the range; the
// lanes whose bins all have k keys above them form a prefix 0 .. F-1, and in
// lane F, where the count from the top crosses k, each lane takes one bin
// (from the top down) and a wave scan gives the keys above it.  Wave-uniform.
// kCoherent: h is a histogram in global memory that other workgroups are
// adding to; it is read with agent-scope loads (past this XCD's L2).
// Only bins below `to` (a multiple of 4) are read: keys in higher bins are
// then not counted, so the bin found can only be lower (still a valid bound).
// A range of at most 256 bins (one group per lane) is read once: lane F's
// four counts come from its registers, so the coherent case takes a single
// round trip.
template <bool kCoherent = false>
__device__ __forceinline__ int running_threshold(const uint32_t* h, uint32_t k, int from, int to = kHistBins) {
  const int lane = threadIdx.x & 63;
  const int lo = from & ~3;                           // whole uint4 groups
  const int n4 = (min(to, kHistBins) - lo) >> 2;
  const int per = (n4 + 63) >> 6;                     // groups per lane: <= 16
  const int mine = max(0, min(per, n4 - per * lane));
  const uint4* hv = reinterpret_cast<const uint4*>(h + lo) + per * lane;
  uint32_t s = 0;
  uint4 x1 = make_uint4(0u, 0u, 0u, 0u);            // this lane's group when per == 1
  if (kCoherent) {
    // 16-byte loads that read past this XCD's L2 (buffer cache policy sc1)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(h), (short)0,
                                                                        kHistBins * 4, kBufferWord3);
    for (int i = 0; i < mine; i++) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * lo + 16 * (per * lane + i), 0, 16);
      s += x.x + x.y + x.z + x.w;
      x1 = make_uint4(x.x, x.y, x.z, x.w);
    }
  } else {
    // every LDS read issued before the first is used
    uint4 xs[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      xs[i] = make_uint4(0u, 0u, 0u, 0u);
      if (i < mine) xs[i] = hv[i];
    }
#pragma unroll
    for (int i = 0; i < 16; i++) s += xs[i].x + xs[i].y + xs[i].z + xs[i].w;
    x1 = xs[0];
  }
  const uint32_t incl = wave_inclusive_scan(s);
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;   // keys of higher lanes' bins
  const uint64_t cross = __ballot(above < k && above + s >= k);
  if (cross == 0) return from - 1;                 // fewer than k keys from `from` up
  const int F = __ffsll((long long)cross) - 1;     // lanes 0 .. F-1: every bin qualifies
  const uint32_t aF = (uint32_t)__builtin_amdgcn_readlane((int)above, F);
  const int base = lo + 4 * per * F;
  const int cnt = 4 * __builtin_amdgcn_readlane(mine, F);   // lane F's bins: base .. base + cnt - 1
  uint32_t c;                                      // the lane-th from the top
  if (per == 1) {                                  // cnt == 4: lane F's registers
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)x1.x, F);
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)x1.y, F);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_readlane((int)x1.z, F);
    const uint32_t b3 = (uint32_t)__builtin_amdgcn_readlane((int)x1.w, F);
    c = lane == 0 ? b3 : lane == 1 ? b2 : lane == 2 ? b1 : lane == 3 ? b0 : 0u;
  } else {
    c = lane < cnt ? (kCoherent ? __hip_atomic_load(h + base + cnt - 1 - lane, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : h[base + cnt - 1 - lane])
                   : 0u;
  }
  const uint32_t ci = wave_inclusive_scan(c);
  const uint64_t q = __ballot(lane < cnt && aF + ci - c >= k);   // keys above that bin reach k
  return base + __popcll(q) - 1;
}

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRoundKeys = 64 * kSelThreads;   // blocks per round
constexpr int kCandCap = 4096;
constexpr int kMaxWords = 8192;   // bitmap words of 64 blocks: 524288 blocks
constexpr int kPartKeys = 32 * kSelThreads;   // blocks per workgroup of the sliced path
constexpr int kMaxParts = 64 * kMaxWords / kPartKeys;     // 32
constexpr int kDirectRank = 128;   // lists up to this long are ranked by direct comparison
constexpr int kSliceMaxRows = 256;   // the sliced path is taken below this many queries
constexpr int kSliceMinBlocks = 3 * kRoundKeys / 2;   // ... and above this many blocks per row
constexpr int kMaxCandGroups = 64;   // groups of 32 candidate lists per query (chunks x tile wavefronts)
static_assert(2 * kCandCap >= kMaxWords, "the candidate list doubles as per-word counters");
static_assert(kMaxParts <= 64 && kMaxParts * kSelThreads == 2 * kMaxWords, "part bookkeeping");
static_assert(kDirectRank <= kSelThreads && kDirectRank <= 4096, "one list entry per thread, 12-bit positions");

struct SelectArgs {
  int n_q, m, k;
  int64_t stride;
  const int32_t* seq_len;
  const uint32_t* keys;
  uint32_t* hist;
  int32_t* topk;
  uint32_t* status;      // the layer's status word
  // sliced path: per (query, round) bitmap words [rows][slices][1024], listed
  // key counts [rows][slices] and lists [rows][slices][2][kCandCap]
  int slices;
  uint32_t* part_bits;
  uint32_t* part_count;
  uint32_t* part_cand;
  // candidate lists of the tile kernel: segs = chunks x kTileWavesPerSet
  // groups of 32 lists per query, chunk c starting at block c * span
  const uint32_t* cand_count;
  int segs, span;
};

template <bool kCoherent>
__device__ void select_row(const SelectArgs& a, int srow, uint32_t* hist, uint32_t* tmp, uint32_t* found,
                           uint32_t* cand, uint32_t* bitmap);

// The decode scoring with the selection in the same launch (kFused).
__device__ void fused_tail(const ScoreArgs& a, const SelectArgs& sel, int srow, int nv, uint32_t* lhist,
                           uint32_t* dyn, int wg_b0, int len, int64_t fin_bk, int64_t fin_e);

// kFused: the keys stay in LDS; from its own histogram and the row's
// histogram as it stands the workgroup derives a bin below the row's
// threshold bin and writes only its keys above that bin (candidates, in
// block order) to its segment of the workspace, with agent-scope stores.
// The row's last workgroup to finish (a per-row counter, after every
// thread's stores and histogram atomics have completed) selects from the
// candidates, reading them with agent-scope loads.  No device-scope fence is
// needed: nothing it reads sits only in another XCD's L2.
// kHQ: heads per chain slot (8, 16 or 32 >= H); kTPA key tiles share one
// matrix-core output (4, 2 or 1).  kPaged: the key planes are a page pool
// (a separate instantiation, so that a contiguous layer's workgroups run no
// page lookups and fetch less code).
template <bool kFused, int kHQ, bool kPaged>
__global__ void __launch_bounds__(256) indexer_score_kernel(ScoreArgs a, SelectArgs sel) {
  constexpr int kT = 256;
  constexpr int kTPA = kHQ == 32 ? 1 : 32 / kHQ;
  static_assert(kDepth % kTPA == 0, "a set of loaded iterations holds whole tile groups");
  const int srow = blockIdx.y;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  // This workgroup's chunks of 1024 blocks are [c0, c0 + cpw).  The key loads
  // are issued before the row length arrives: any block below the key row
  // capacity is readable, and blocks past the visible count are masked later.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wh = wave;                           // wavefront of the workgroup
  // Block indices fit 32 bits (a key row holds at most 524 288 blocks).
  const int c0 = (int)blockIdx.x * a.cpw;
  const int cap = (int)(a.stride < a.max_blocks ? a.stride : a.max_blocks);

  __shared__ __attribute__((aligned(16))) uint8_t q_code[32][32];
  __shared__ int q_exp[32][2];
  __shared__ float q_w[32];
  __shared__ __attribute__((aligned(16))) uint32_t lhist[kHistBins];   // read as uint4
  // kFused: the workgroup's keys by block offset (later the selection bitmap)
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  const int wg_b0 = (int)blockIdx.x * a.cpw * kScoreBlocksPerWG;   // kFused: first block of the workgroup
  const int r = lane & 31, kh = lane >> 5;

  // key planes: the row's entries (contiguous), or the page pool (paged)
  constexpr bool paged = kPaged;                 // the launch checked a.pm.shift >= 0
  const int64_t row_base = paged ? 0 : (int64_t)brow * a.max_blocks;
  const uint8_t* kc = a.idx_code + row_base * 32;
  const uint8_t* ks = a.idx_scale + row_base * 2;
  int lane_pg = -1;
  if constexpr (paged) lane_pg = wg_pages(a.pm, brow, wg_b0, lane);
  // The wave walks iterations i = 0 .. n_it-1 of 32 blocks each: iteration i
  // is group i % 8 of this wave's 256 blocks in chunk c0 + i / 8.  Keys are
  // loaded kDepth iterations ahead of their use.
  const int n_it = a.cpw * kScoreItersPerWave;
  auto blk_of = [&](int i) -> int {
    return (c0 + i / kScoreItersPerWave) * kScoreBlocksPerWG +
           wh * (kScoreItersPerWave * kScoreBlocksPerIter) +
           (i % kScoreItersPerWave) * kScoreBlocksPerIter + r;
  };
  // Loads are unconditional (a block past the capacity, or on an unmapped
  // page, reads entry 0) so that no load waits on another; compute() masks
  // what they return.  Each key is read once per launch: non-temporal loads
  // keep the stream from evicting the cache lines that are reused (the
  // kernel's code, the query, the histograms).
  typedef int nt_v4i __attribute__((ext_vector_type(4)));
  auto load = [&](int i, int4& kr, uint32_t& er) {
    const int blk = blk_of(i);
    int64_t b = (i < n_it && blk < cap) ? blk : 0;
    if constexpr (paged) {
      if (i < n_it && blk < cap) b = wg_entry(a.pm, lane_pg, wg_b0, blk - r, blk);
    }
    const nt_v4i v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4i*>(kc + b * 32 + 16 * kh));
    kr = make_int4(v.x, v.y, v.z, v.w);
    er = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(ks + b * 2));
  };
  // query values and weights: all loads in flight before any is used; four
  // consecutive values per thread (16-byte loads), so the 32 values of an MX
  // block are 8 neighbouring lanes
  const float* qsrc = a.iq + (int64_t)srow * a.H * kIdx;
  constexpr int kQv = 2;                          // H_I * 64 <= 2048 values
  float4 qv[kQv];
#pragma unroll
  for (int u = 0; u < kQv; u++) {
    const int e = 4 * (tid + kT * u);
    qv[u] = e < a.H * kIdx ? *reinterpret_cast<const float4*>(qsrc + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float wq = tid < a.H ? a.iw[(int64_t)srow * a.H + tid] : 0.0f;
  // Key loads go out after the query's: the loads complete in issue order, so
  // the query quantisation below does not wait for the keys.
  // two blocks of kDepth iterations in flight
  int4 kA[kDepth], kB[kDepth];
  uint32_t eA[kDepth], eB[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; u++) {
    load(u, kA[u], eA[u]);
    load(kDepth + u, kB[u], eB[u]);
  }
  // the row length through the scalar cache, once every vector load is out
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const int len = *(const_i32p)(a.seq_len + brow);
  const int p = (kFused && a.append ? len : len - a.n_q) + qi;   // append: the new token is at len
  int nv = (p + 1) / a.m;
  if (nv > cap) {                              // more blocks than the plan holds
    if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, LCA_STATUS_INDEXER_CAPACITY);
    nv = cap;
  }
  if constexpr (paged) {
    if (wave == 0) wg_pages_check(a.pm, lane_pg, wg_b0, a.cpw * kScoreBlocksPerWG, nv, lane, a.status);
  }

  for (int i = tid; i < kHistBins; i += kT) lhist[i] = 0;
  // MXFP4 quantisation of the query: an MX block's largest magnitude over
  // its 8 lanes, then four codes per thread (two bytes of q_code)
#pragma unroll
  for (int u = 0; u < kQv; u++) {
    const int e = 4 * (tid + kT * u);
    if (e >= a.H * kIdx) break;                   // uniform per wavefront (H_I * 64: whole 256s)
    const float4 x = qv[u];
    const float amax = octet_max(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    uint32_t c4 = 0;
    int X = -127;
    if (amax > 0.0f) {
      X = floor_log2(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      c4 = f32_e2m1(ldexpf(x.x, -X)) | (f32_e2m1(ldexpf(x.y, -X)) << 4) | (f32_e2m1(ldexpf(x.z, -X)) << 8) |
           (f32_e2m1(ldexpf(x.w, -X)) << 12);
    }
    const int h = e >> 6, el = e & 63;
    *reinterpret_cast<uint16_t*>(&q_code[h][el >> 1]) = (uint16_t)c4;   // values el .. el + 3
    if ((el & 31) == 0) q_exp[h][el >> 5] = X;
  }
  if (tid < a.H) q_w[tid] = wq;
  __syncthreads();

  // Append: the block this token completes (bk, entry e) is finalised by the
  // scoring wavefront whose keys hold it, before that key is scored: its
  // indexer key (group 8) goes to the entry planes and to LDS, and the lane
  // that loaded the block's old bytes takes the new ones (iteration pi, lane
  // pr).  The other groups and the ring copy run after the arrival.
  __shared__ __attribute__((aligned(16))) uint8_t patch[48];
  int pi = -1, pr = 0;
  int4 pk = make_int4(0, 0, 0, 0);
  uint32_t pe = 0;
  int64_t fin_bk = -1, fin_e = -1;
  if constexpr (kFused) {
    if (a.append) {
      const int64_t bk = (int64_t)(len / a.m);
      if ((bk + 1) * a.m == (int64_t)len + 1) {      // this token completes block bk
        if (bk >= a.ca.max_blocks) {
          if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, LCA_STATUS_COMPRESS_CAPACITY);
        } else {
          const int64_t e = entry_index(a.pm, brow, bk);
          if (e < 0) {
            if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, LCA_STATUS_PAGE);
          } else {
            fin_bk = bk;
            fin_e = e;
          }
        }
      }
      const int64_t off = fin_bk - wg_b0;
      if (fin_bk >= 0 && off >= 0 && off < (int64_t)a.cpw * kScoreBlocksPerWG && fin_bk < cap) {
        const int o = (int)off;
        if (wh == (o % kScoreBlocksPerWG) / (kScoreItersPerWave * kScoreBlocksPerIter)) {
          finalize_group(a.ca, brow, fin_bk, len, 8, fin_e, nullptr, lane, patch);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          pi = (o / kScoreBlocksPerWG) * kScoreItersPerWave +
               (o % (kScoreItersPerWave * kScoreBlocksPerIter)) / kScoreBlocksPerIter;
          pr = o % kScoreBlocksPerIter;
          pk = *reinterpret_cast<const int4*>(patch + 16 * kh);
          pe = (uint32_t)patch[32] | ((uint32_t)patch[33] << 8);
        }
      } else if (fin_bk >= cap && wg_b0 == 0 && wh == 0) {
        // past the key row the scoring covers: only the entry (capacity reported above)
        finalize_group(a.ca, brow, fin_bk, len, 8, fin_e, nullptr, lane, nullptr);
      }
    }
  }

  // A operands for the per-half products of the exact fallback (no scales):
  // lane l feeds row l%32 with K-half l/32, row (head, half) holding only that
  // half of the head.
  const int hgroups = (a.H + 15) >> 4;
  v8i A[2];
  int qmin = 1 << 20, qmax = -(1 << 20), qdmin = 0, qdmax = 0;
#pragma unroll
  for (int hg = 0; hg < 2; hg++) {
    A[hg] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    const int G = (r & 7) >> 2, v = 4 * (r >> 3) + (r & 3);
    const int h = 16 * hg + 8 * G + (v >> 1), half = v & 1;
    if (hg < hgroups && half == kh && h < a.H) {
      const int* src = reinterpret_cast<const int*>(&q_code[h][16 * kh]);
      A[hg][0] = src[0];
      A[hg][1] = src[1];
      A[hg][2] = src[2];
      A[hg][3] = src[3];
    }
  }
  // The same query with both MX halves of a head in one A row, for products
  // that add the two halves in hardware.  Row r = 8 i + 4 s + j is output
  // e = 4 i + j of lane half s.  kHQ <= 16: output e is head e % kHQ of tile
  // 2 (e / kHQ) + s of a group of kTPA tiles, and Af[t] holds only the rows
  // of tile t (zero elsewhere); kHQ = 32: one tile, row r carries head 16 s + e.
  v8i Af[kTPA];
  int saf[kTPA];
  {
    const int s_r = (r >> 2) & 1, e_r = 4 * (r >> 3) + (r & 3);
    const int h = kHQ == 32 ? 16 * s_r + e_r : e_r % kHQ;
    const int t_r = kHQ == 32 ? 0 : 2 * (e_r / kHQ) + s_r;
    const bool hv = h < a.H;
    const int* src = reinterpret_cast<const int*>(&q_code[hv ? h : 0][16 * kh]);
    const int d0 = hv ? src[0] : 0, d1 = hv ? src[1] : 0, d2 = hv ? src[2] : 0, d3 = hv ? src[3] : 0;
    const int sc = hv ? q_exp[h][kh] + 127 : 127;
#pragma unroll
    for (int t = 0; t < kTPA; t++) {
      const bool mine = t_r == t;
      Af[t] = (v8i){mine ? d0 : 0, mine ? d1 : 0, mine ? d2 : 0, mine ? d3 : 0, 0, 0, 0, 0};
      saf[t] = mine ? sc : 127;
    }
  }
  // weights of the lane's chain, head order; past H a weight is 0, which
  // leaves the chain unchanged
  float wv[kHQ == 32 ? 16 : kHQ];
#pragma unroll
  for (int e = 0; e < (kHQ == 32 ? 16 : kHQ); e++) {
    const int h = kHQ == 32 ? 16 * kh + e : e;
    wv[e] = h < a.H ? q_w[h] : 0.0f;
  }
  {
    // extremes of the query's 2H block exponents: lane l looks at entry l
    const int e = lane < 2 * a.H ? q_exp[lane >> 1][lane & 1] : 0;
    qmin = wave_minmax<0>(lane < 2 * a.H ? e : (1 << 20));
    qmax = wave_minmax<1>(lane < 2 * a.H ? e : -(1 << 20));
    // range of the heads' half-exponent differences: lane l looks at head l
    const int d = lane < a.H ? q_exp[lane][0] - q_exp[lane][1] : 0;
    qdmin = wave_minmax<0>(lane < a.H ? d : (1 << 20));
    qdmax = wave_minmax<1>(lane < a.H ? d : -(1 << 20));
  }

  // One product adding both halves gives the exactly rounded dot when every
  // half's exponent sum E = query exponent + key exponent lies in [-124, 116]
  // and the two sums of a head differ by at most 10: each half's products are
  // multiples of 2^(E-2) below 1152 * 2^E, so every partial sum then needs at
  // most 24 bits and is an exact fp32 number.  On the key's two E8M0 bytes
  // (exponent + 127) these are the ranges byte in [3 - qmin, 243 - qmax] and
  // byte0 - byte1 in [-10 - qdmin, 10 - qdmax], each checked as one unsigned
  // comparison (an empty range admits nothing).
  int byte_lo = 3 - qmin, diff_lo = -10 - qdmin;
  uint32_t byte_span = (uint32_t)(243 - qmax - byte_lo), diff_span = (uint32_t)(10 - qdmax - diff_lo);
  if (243 - qmax < byte_lo) byte_lo = 1 << 30, byte_span = 0;
  if (10 - qdmax < diff_lo) diff_lo = 1 << 30, diff_span = 0;

  uint32_t* out = a.keys + (int64_t)srow * a.stride;
  const v16f zero16 = {};

  // kDepth iterations at once: their matrix-core products and head chains are
  // independent, so they interleave; one range check covers the block.
  // Lane key kk of the set belongs to iteration it_of(kk) (and column r).
  constexpr int kKeys = kHQ == 32 ? kDepth : kDepth / 2;   // keys per lane per set
  auto it_of = [&](int kk) -> int {
    if (kHQ == 32) return kk;
    const int grp = kk / (kTPA / 2), g = kk % (kTPA / 2);
    return grp * kTPA + 2 * g + kh;
  };
  auto compute = [&](int i0, const int4 (&kr)[kDepth], const uint32_t (&er_in)[kDepth]) {
    int b0[kDepth], b1[kDepth], sb[kDepth];
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      // a block that is not scored takes unit scales (its result is dropped)
      const uint32_t er = blk_of(i0 + u) < nv ? er_in[u] : 0x7F7Fu;
      b0[u] = (int)(er & 0xFF);
      b1[u] = (int)(er >> 8);
      sb[u] = kh ? b1[u] : b0[u];
      ok = ok & ((uint32_t)(b0[u] - byte_lo) <= byte_span) & ((uint32_t)(b1[u] - byte_lo) <= byte_span) &
           ((uint32_t)(b0[u] - b1[u] - diff_lo) <= diff_span);
    }
    float total[kKeys];
    if (__all(ok)) {
      if constexpr (kHQ == 32) {
        v16f acc[kDepth];
#pragma unroll
        for (int u = 0; u < kDepth; u++) {
          const v8i Bm = (v8i){kr[u].x, kr[u].y, kr[u].z, kr[u].w, 0, 0, 0, 0};
          acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Af[0], Bm, zero16, 4, 4, 0, saf[0], 0, sb[u]);
        }
        // heads 0..15 on the low lanes, then 16..31 on the high lanes from
        // there; the score hops back to the low lanes
        float c[kDepth];
#pragma unroll
        for (int u = 0; u < kDepth; u++) {
          c[u] = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; e++) c[u] = __builtin_fmaf(wv[e], relu_bits(acc[u][e]), c[u]);
        }
#pragma unroll
        for (int u = 0; u < kDepth; u++) c[u] = swap_halves(c[u]);
#pragma unroll
        for (int u = 0; u < kDepth; u++) {
#pragma unroll
          for (int e = 0; e < 16; e++) c[u] = __builtin_fmaf(wv[e], relu_bits(acc[u][e]), c[u]);
        }
#pragma unroll
        for (int u = 0; u < kDepth; u++) total[u] = swap_halves(c[u]);
      } else {
#pragma unroll
        for (int grp = 0; grp < kDepth / kTPA; grp++) {
          v16f acc = zero16;
#pragma unroll
          for (int t = 0; t < kTPA; t++) {
            const int u = grp * kTPA + t;
            const v8i Bm = (v8i){kr[u].x, kr[u].y, kr[u].z, kr[u].w, 0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Af[t], Bm, acc, 4, 4, 0, saf[t], 0, sb[u]);
          }
#pragma unroll
          for (int g = 0; g < kTPA / 2; g++) {
            float c = 0.0f;
#pragma unroll
            for (int e = 0; e < kHQ; e++) c = __builtin_fmaf(wv[e], relu_bits(acc[kHQ * g + e]), c);
            total[grp * (kTPA / 2) + g] = c;
          }
        }
      }
    } else {
      float ts[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; u++) {
        const v8i Bm = (v8i){kr[u].x, kr[u].y, kr[u].z, kr[u].w, 0, 0, 0, 0};
        ts[u] = score_unscaled(A[0], A[1], Bm, hgroups, a.H, kh, q_exp, q_w, b0[u] - 127, b1[u] - 127);
      }
      // score of tile u in the low lanes; lane key kk takes iteration it_of(kk)
#pragma unroll
      for (int kk = 0; kk < kKeys; kk++) {
        if (kHQ == 32) {
          total[kk] = ts[kk];
        } else {
          const int grp = kk / (kTPA / 2), g = kk % (kTPA / 2);
          const float hi = swap_halves(ts[grp * kTPA + 2 * g + 1]);
          total[kk] = kh ? hi : ts[grp * kTPA + 2 * g];
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < kKeys; kk++) {
      const int u = it_of(kk);
      const int blk = blk_of(i0 + u);
      if ((kHQ != 32 || kh == 0) & (i0 + u < n_it) & (blk < nv)) {
        const uint32_t key = ord_key(__fadd_rn(total[kk], 0.0f));   // -0 -> +0
        if (kFused)
          dyn_lds[blk - wg_b0] = key;
        else
          out[blk] = key;
        atomicAdd(&lhist[key >> kHistShift], 1u);
      }
    }
  };

  // the appended block's new key replaces what the owning lane loaded
  auto patch_keys = [&](int i0, int4 (&kk)[kDepth], uint32_t (&ee)[kDepth]) {
    if (pi >= i0 && pi < i0 + kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; u++)
        if (i0 + u == pi && r == pr) {
          kk[u] = pk;
          ee[u] = pe;
        }
    }
  };
#pragma unroll 1
  for (int i0 = 0; i0 < n_it; i0 += 2 * kDepth) {
    if (kFused) patch_keys(i0, kA, eA);
    compute(i0, kA, eA);
#pragma unroll
    for (int u = 0; u < kDepth; u++) load(i0 + 2 * kDepth + u, kA[u], eA[u]);
    if (kFused) patch_keys(i0 + kDepth, kB, eB);
    compute(i0 + kDepth, kB, eB);
#pragma unroll
    for (int u = 0; u < kDepth; u++) load(i0 + 3 * kDepth + u, kB[u], eB[u]);
  }
  __syncthreads();
  if constexpr (kFused) {
    fused_tail(a, sel, srow, nv, lhist, dyn_lds, wg_b0, len, fin_bk, fin_e);
  } else {
    uint32_t* gh = a.hist + (int64_t)srow * kHistBins;
    // every count is read before any atomic goes out
    uint32_t hc[kHistBins / kT];
#pragma unroll
    for (int i = 0; i < kHistBins / kT; i++) hc[i] = lhist[tid + kT * i];
#pragma unroll
    for (int i = 0; i < kHistBins / kT; i++)
      if (hc[i]) atomicAdd(&gh[tid + kT * i], hc[i]);
  }
}

// ---------------------------------------------------------------------------
// Scores for many queries per row (prefill chunks): a workgroup takes Qwg
// consecutive queries of one row and a range of blocks, so every key is read
// from memory once per Qwg queries rather than once per query.
//
// One 32x32x64 FP4 product per query pair (H <= 16) or per query (H <= 32)
// and 32 blocks: row r = 8i + 4s + j of the A operand is
//   H <= 16: query 2m + s of the wavefront's set, head 4i + j
//   H <= 32: query m, head 16s + 4i + j
// and carries the head's whole 64-d MXFP4 vector (lanes l and l + 32 give its
// two MX halves with their own E8M0 scales), so lane l's 16 outputs are the
// dot products of its block (column l % 32) with heads 0..15 (16s .. 16s+15)
// of its query, in order.  With both halves in one product the hardware adds
// two scaled partial sums; the result is still the exactly rounded dot when
// every partial sum is an fp32 number: each half's products are multiples of
// 2^(E-2) below 1152 * 2^E (E = query exponent + key exponent of the half),
// so with |E0 - E1| <= 10 and both E in [-124, 116] every partial sum is a
// multiple of 2^(min E - 2) below 2^(max E + 12) and needs at most 24 bits.
// Iterations where some (row, column) leaves these bounds take the per-half
// path (two unscaled products, scales applied exactly per output).
// Each lane runs the head chain of its query in ascending head order; for
// H > 16 the chain runs over heads 0..15 on the low lanes, continues over
// 16..31 on the high lanes and the score hops back (lane l < 32 stores it).
//
// Candidate lists (kCand): instead of one key per block, each lane keeps
// only the keys that can still be among its query's k largest.  From time to
// time (after 4 iterations, then every 8) wavefront w reads the running
// histogram of query w of the workgroup and finds the highest bin b whose
// higher bins already hold k keys; keys in bin b or below cannot reach the
// top k of the row, since the k-th largest key of the row lies above b.
// A lane appends every key in a higher bin, with its iteration index t, as
// a (key, t) pair to its own list, entry j taking the slot of the j-th block
// the lane visits (block b_lo + 32 (w + 8 j) + column; the pair array has
// the layout of the key rows, 8 bytes a slot).  The histogram still counts
// every key, so the selection's threshold bin tb is exact, and every key of
// bin tb and above is in some list.
// ---------------------------------------------------------------------------

constexpr int kTileWaves = 8;
constexpr int kTileMinQueries = 16;                  // rows with at least this many queries
constexpr int kTileTargetWGs = 1024;
constexpr int kTileSets = 1;                         // query sets per workgroup
constexpr int kTileWavesPerSet = kTileWaves / kTileSets;


template <int kQw>   // queries per wavefront: 8 (H <= 16) or 4 (H <= 32)
__device__ __noinline__ v16f tile_dots_unscaled(v8i Am, v8i Bm, int kh, int m, int set,
                                                const int (*q_exp)[32][2], int ke0, int ke1) {
  // per-half products without scales, then each output's exact value
  const v16f zero16 = {};
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const v8i A0 = kh ? zero8 : Am, A1 = kh ? Am : zero8;
  const v16f D0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A0, Bm, zero16, 4, 4, 0, 127, 0, 127);
  const v16f D1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A1, Bm, zero16, 4, 4, 0, 127, 0, 127);
  const int s = (threadIdx.x & 63) >> 5;
  const int q = kQw == 8 ? set * kQw + 2 * m + s : set * kQw + m;
  v16f d;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    const int h = kQw == 8 ? e : 16 * s + e;
    d[e] = exact_pair(D0[e], q_exp[q][h][0] + ke0, D1[e], q_exp[q][h][1] + ke1);
  }
  return d;
}

template <int kQw, bool kCand>
__global__ void __launch_bounds__(64 * kTileWaves) indexer_score_tile_kernel(ScoreArgs a) {
  constexpr int kQwg = kQw * kTileSets;               // queries per workgroup
  constexpr int kNm = 4;                              // products per iteration
  const int brow = blockIdx.z, qg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar bases
  const int set = wave / kTileWavesPerSet, wv = wave % kTileWavesPerSet;
  const int col = lane & 31, kh = lane >> 5;
  const int q0 = qg * kQwg;                           // first query of the workgroup (row-local)

  __shared__ __attribute__((aligned(16))) uint32_t lh[kQwg][kHistBins];
  __shared__ __attribute__((aligned(16))) uint8_t q_code[kQwg][32][32];
  __shared__ int q_exp[kQwg][32][2];
  __shared__ float q_w[kQwg][32];
  __shared__ int thr_s[kQwg];                         // candidate lists: running threshold bins

  // block indices fit int: max_blocks <= 524288
  const int cap = (int)(a.stride < a.max_blocks ? a.stride : a.max_blocks);
  const int b_lo = blockIdx.x * a.cpw * kScoreBlocksPerWG;
  const int b_hi = b_lo + a.cpw * kScoreBlocksPerWG;
  // key planes: the row's entries (contiguous), or the page pool (paged)
  const bool paged = a.pm.shift >= 0;
  const int64_t row_base = paged ? 0 : (int64_t)brow * a.max_blocks;
  const uint8_t* kc = a.idx_code + row_base * 32;
  const uint8_t* ks = a.idx_scale + row_base * 2;
  const int lane_pg = paged ? wg_pages(a.pm, brow, b_lo, lane) : -1;

  // queries: Qwg x H x 64 fp32 values, four consecutive ones per thread and
  // step (16-byte loads, all issued before the first is used), so the 32
  // values of an MX block are 8 neighbouring lanes
  constexpr int kQSteps = kQwg * (kQw == 8 ? 16 : 32) * kIdx / (4 * 64 * kTileWaves);
  static_assert(kQSteps * 4 * 64 * kTileWaves == kQwg * (kQw == 8 ? 16 : 32) * kIdx, "whole steps");
  const int nqv = min(kQwg, a.n_q - q0);              // queries of this workgroup
  const float* qsrc = a.iq + ((int64_t)brow * a.n_q + q0) * a.H * kIdx;
  const int qvals = kQwg * a.H * kIdx;
  float4 qv4[kQSteps];
#pragma unroll
  for (int u = 0; u < kQSteps; u++) {
    const int e = 4 * (tid + 64 * kTileWaves * u);
    const bool ok = e < qvals && e / (a.H * kIdx) < nqv;
    qv4[u] = ok ? *reinterpret_cast<const float4*>(qsrc + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int i = tid; i < kQwg * kHistBins / 4; i += 64 * kTileWaves)
    reinterpret_cast<uint4*>(&lh[0][0])[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < kQSteps; u++) {
    const int e = 4 * (tid + 64 * kTileWaves * u);
    if (e >= qvals) break;                            // whole MX blocks: octets stay whole
    const int q = e / (a.H * kIdx), rem = e % (a.H * kIdx);
    const float4 x = qv4[u];
    const float amax = octet_max(fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    uint32_t c4 = 0;
    int X = -127;
    if (amax > 0.0f) {
      X = floor_log2(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      c4 = f32_e2m1(ldexpf(x.x, -X)) | (f32_e2m1(ldexpf(x.y, -X)) << 4) | (f32_e2m1(ldexpf(x.z, -X)) << 8) |
           (f32_e2m1(ldexpf(x.w, -X)) << 12);
    }
    const int h = rem >> 6, el = rem & 63;
    *reinterpret_cast<uint16_t*>(&q_code[q][h][el >> 1]) = (uint16_t)c4;   // values el .. el + 3
    if ((el & 31) == 0) q_exp[q][h][el >> 5] = X;
  }
  if (kCand && tid < kQwg) thr_s[tid] = -1;
  for (int i = tid; i < kQwg * 32; i += 64 * kTileWaves) {
    const int q = i >> 5, h = i & 31;
    q_w[q][h] = (h < a.H && q < nqv) ? a.iw[((int64_t)brow * a.n_q + q0 + q) * a.H + h] : 0.0f;
  }
  __syncthreads();

  // A operands (row l % 32, K-half l / 32), their scales, the lane's weights
  const int r = col, ri = r >> 3, rs = (r >> 2) & 1, rj = r & 3;
  v8i A[kNm];
  int sa[kNm];
  float wt[kNm][16];
#pragma unroll
  for (int m = 0; m < kNm; m++) {
    const int q = kQw == 8 ? set * kQw + 2 * m + rs : set * kQw + m;
    const int h = kQw == 8 ? 4 * ri + rj : 16 * rs + 4 * ri + rj;
    const bool ok = h < a.H;
    const int* src = reinterpret_cast<const int*>(&q_code[q][ok ? h : 0][16 * kh]);
    A[m] = (v8i){ok ? src[0] : 0, ok ? src[1] : 0, ok ? src[2] : 0, ok ? src[3] : 0, 0, 0, 0, 0};
    sa[m] = ok ? q_exp[q][h][kh] + 127 : 127;
    const int qo = kQw == 8 ? set * kQw + 2 * m + kh : set * kQw + m;
#pragma unroll
    for (int e = 0; e < 16; e++) wt[m][e] = q_w[qo][kQw == 8 ? e : 16 * kh + e];   // 0 past H
  }
  // exponent bounds of this set's query halves: the exact fast path needs
  // |(ea0 + eb0) - (ea1 + eb1)| <= 10 and every ea + eb in [-124, 116]
  int emin = 1 << 20, emax = -(1 << 20), dmin = 1 << 20, dmax = -(1 << 20);
  for (int i = lane; i < kQw * 32; i += 64) {
    const int q = set * kQw + (i >> 5), h = i & 31;
    if (h < a.H && q < nqv) {
      const int e0 = q_exp[q][h][0], e1 = q_exp[q][h][1];
      emin = min(emin, min(e0, e1));
      emax = max(emax, max(e0, e1));
      dmin = min(dmin, e0 - e1);
      dmax = max(dmax, e0 - e1);
    }
  }
  emin = wave_minmax<0>(emin);
  emax = wave_minmax<1>(emax);
  dmin = wave_minmax<0>(dmin);
  dmax = wave_minmax<1>(dmax);

  // visible blocks of the wavefront's queries (query q0 + set * kQw + u)
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const int len = *(const_i32p)(a.seq_len + brow);
  int nvq[kQw];
  int nv_hi = 0;
#pragma unroll
  for (int u = 0; u < kQw; u++) {
    const int q = q0 + set * kQw + u;
    const int p = len - a.n_q + q;
    int nv = q < a.n_q ? (p + 1) / a.m : 0;
    if (nv > cap) {                            // more blocks than the plan holds
      if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, LCA_STATUS_INDEXER_CAPACITY);
      nv = cap;
    }
    nvq[u] = nv;
    nv_hi = nv > nv_hi ? nv : nv_hi;
  }
  const int b_end = b_hi < nv_hi ? b_hi : nv_hi;
  if (paged && wave == 0) wg_pages_check(a.pm, lane_pg, b_lo, b_hi - b_lo, nv_hi, lane, a.status);
  // lane l < 32 stores query 2m (H <= 16) or m of the pair, lane l >= 32 the other
  uint32_t* outq[kNm];
  int nvl[kNm];
  uint32_t* lhq[kNm];
  // candidate lists: the (key, t) pairs of the set's kQw query rows as one
  // buffer; a lane's byte offset of its next list slot, its least key kept
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      a.keys + 2 * ((int64_t)brow * a.n_q + q0 + set * kQw) * a.stride, (short)0, (int)(kQw * a.stride * 8),
      kBufferWord3);
  uint32_t coff[kNm], kmin[kNm];
#pragma unroll
  for (int m = 0; m < kNm; m++) {
    const int u = kQw == 8 ? 2 * m + kh : m;          // H <= 32: both halves hold query m
    const int64_t row = (int64_t)brow * a.n_q + q0 + set * kQw + u;
    outq[m] = a.keys + row * a.stride;
    nvl[m] = (kQw == 8 || kh == 0) ? nvq[u] : 0;     // H <= 32: one store per query
    lhq[m] = &lh[set * kQw + u][0];
    coff[m] = (uint32_t)((u * a.stride + b_lo + 32 * wv + col) * 8);
    kmin[m] = 0;
  }

  const v16f zero16 = {};
  // iteration t covers blocks b_lo + 32 (wv + t * kTileWavesPerSet) + col; the
  // keys of kRing iterations are in flight (a block past the key row reads
  // block 0; what is not scored is masked)
  constexpr int kRing = 4;
  const int n_it = b_end > b_lo ? (b_end - b_lo + 32 * kTileWavesPerSet - 1) / (32 * kTileWavesPerSet) : 0;
  auto blk_of = [&](int t) -> int { return b_lo + 32 * (wv + t * kTileWavesPerSet) + col; };
  int4 kr[kRing];
  uint32_t erw[kRing];
  auto load = [&](int t, int4& k4, uint32_t& e2) {
    const int blk = blk_of(t);
    int64_t bl = (t < n_it && blk < cap) ? blk : 0;
    if (paged && t < n_it && blk < cap) bl = wg_entry(a.pm, lane_pg, b_lo, blk - col, blk);
    k4 = *reinterpret_cast<const int4*>(kc + bl * 32 + 16 * kh);
    e2 = *reinterpret_cast<const uint16_t*>(ks + bl * 2);
  };
#pragma unroll
  for (int u = 0; u < kRing; u++) load(u, kr[u], erw[u]);

  // Guard bounds on the key's raw E8M0 bytes (b = e + 127): both bytes in
  // [blo, bhi] and b0 - b1 in [dlo, dhi] (unsigned range compares).
  const int blo = -124 - emin + 127, bhi = 116 - emax + 127;
  const int dlo = -10 - dmin, dhi = 10 - dmax;
  const bool fast_possible = blo <= bhi && dlo <= dhi;   // else every iteration takes the per-half path
  struct Dots {
    v16f d[kNm];
  };
  // the products of iteration t (matrix cores, or the per-half path)
  auto dots = [&](int t, const int4& k4, uint32_t e2) {
    const int blk = blk_of(t);
    const uint32_t er = blk < b_end ? e2 : 0x7F7Fu;          // unscored blocks: unit scales
    const int b0 = (int)(er & 0xFF), b1 = (int)(er >> 8);
    const bool ok = fast_possible & ((uint32_t)(b0 - blo) <= (uint32_t)(bhi - blo)) &
                    ((uint32_t)(b1 - blo) <= (uint32_t)(bhi - blo)) & ((uint32_t)(b0 - b1 - dlo) <= (uint32_t)(dhi - dlo));
    const v8i Bm = (v8i){k4.x, k4.y, k4.z, k4.w, 0, 0, 0, 0};
    Dots r;
    if (__all(ok)) {
      const int sb = kh ? b1 : b0;
#pragma unroll
      for (int m = 0; m < kNm; m++)
        r.d[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[m], Bm, zero16, 4, 4, 0, sa[m], 0, sb);
    } else {
#pragma unroll
      for (int m = 0; m < kNm; m++)
        r.d[m] = tile_dots_unscaled<kQw>(A[m], Bm, kh, m, set, q_exp, b0 - 127, b1 - 127);
    }
    return r;
  };
  // head chains in ascending head order, keys
  auto finish = [&](int t, const Dots& D) {
    const int blk = blk_of(t);
#pragma unroll
    for (int m = 0; m < kNm; m++) {
      float score = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e++) score = __builtin_fmaf(wt[m][e], relu_bits(D.d[m][e]), score);
      if (kQw == 4) {
        // heads 16..31 continue the chain of 0..15 on the high lanes; the
        // score hops back to the low lanes
        float c = swap_halves(score);
#pragma unroll
        for (int e = 0; e < 16; e++) c = __builtin_fmaf(wt[m][e], relu_bits(D.d[m][e]), c);
        score = swap_halves(c);
      }
      // no -0: every chain starts at +0 and each fma result is exact-rounded
      // from a sum that is -0 only when both terms are
      const uint32_t key = ord_key(score);
      if (blk < nvl[m]) atomicAdd(&lhq[m][key >> kHistShift], 1u);
      if (!kCand) {
        if (blk < nvl[m]) outq[m][blk] = key;
      } else {
        // append (key, t) to the lane's list: the slot of its next visit
        const bool c = blk < nvl[m] && key >= kmin[m];
        __builtin_amdgcn_raw_buffer_store_b64((u32x2_t){key, (uint32_t)t}, crs, (int)(c ? coff[m] : kDropOffset), 0, 0);
        coff[m] += c ? 8u * 32u * kTileWavesPerSet : 0u;
      }
    }
  };
#pragma unroll 1
  for (int t0 = 0; t0 < n_it; t0 += kRing) {
    if (kCand && t0 >= kRing && ((t0 & (t0 - 1)) == 0 || (t0 & 7) == 0)) {
      // wavefront w refreshes the bound of query w, then every lane takes the
      // latest bounds of its queries (another wavefront's may be older: any
      // value it has written is valid)
      if (wv < kQw)
        thr_s[set * kQw + wv] = running_threshold(&lh[set * kQw + wv][0], (uint32_t)a.k, thr_s[set * kQw + wv] + 1);
      // keys above bin b: key >= (b + 1) << 20
#pragma unroll
      for (int m = 0; m < kNm; m++) kmin[m] = (uint32_t)(thr_s[set * kQw + (kQw == 8 ? 2 * m + kh : m)] + 1) << kHistShift;
    }
#pragma unroll
    for (int u = 0; u < kRing; u++) {
      const Dots D = dots(t0 + u, kr[u], erw[u]);
      load(t0 + u + kRing, kr[u], erw[u]);
      finish(t0 + u, D);
    }
  }
  if (kCand) {
    // list lengths, [rows][chunks][kTileWavesPerSet][32 columns]
#pragma unroll
    for (int m = 0; m < kNm; m++) {
      const int u = kQw == 8 ? 2 * m + kh : m;
      const int q = q0 + set * kQw + u;
      const uint32_t first = (uint32_t)((u * a.stride + b_lo + 32 * wv + col) * 8);
      if ((kQw == 8 || kh == 0) && q < a.n_q)
        a.cand_count[((((int64_t)brow * a.n_q + q) * gridDim.x + blockIdx.x) * kTileWavesPerSet + wv) * 32 + col] =
            (coff[m] - first) / (8u * 32u * kTileWavesPerSet);
    }
  }
  __syncthreads();
  // flush the histograms of the workgroup's queries.  With candidate lists
  // only the bins above the query's last bound go out: the row's threshold
  // bin lies above it, and the selection reads exact counts only at and above
  // that bin.
#pragma unroll 1
  for (int q = 0; q < nqv; q++) {
    uint32_t* gh = a.hist + ((int64_t)brow * a.n_q + q0 + q) * kHistBins;
    const int bmin = kCand ? thr_s[q] : -1;
    uint32_t hc[kHistBins / (64 * kTileWaves)];
#pragma unroll
    for (int i = 0; i < kHistBins / (64 * kTileWaves); i++) hc[i] = lh[q][tid + 64 * kTileWaves * i];
#pragma unroll
    for (int i = 0; i < kHistBins / (64 * kTileWaves); i++)
      if (hc[i] && tid + 64 * kTileWaves * i > bmin) atomicAdd(&gh[tid + 64 * kTileWaves * i], hc[i]);
  }
}

// ---------------------------------------------------------------------------
// Exact top-k by (score desc, block asc) for one query, on workgroups of 512
// threads.  Keys are taken in rounds of 32768 blocks; in a round, thread t
// owns the 64 blocks 64t .. 64t+63 (two 32-bit bitmap words).
//   1. The query's histogram of the top 12 key bits (built while scoring)
//      gives the bin tb holding the k-th largest key and the count `above` of
//      keys in higher bins.
//   2. Each thread compares its keys with tb: keys above tb set their bit,
//      keys inside tb are listed in block order (a block-wide scan places
//      every thread's keys).
//   3. Two radix passes of 10 bits over the listed keys give the exact
//      threshold key T and how many keys equal to T are taken; listed keys
//      above T set their bit, and keys equal to T are ranked by block index
//      with a scan over the list, which is in block order.
//   4. The bitmap is compacted into ascending block indices.
// If more than kCandCap keys share tb (many nearly equal scores), a radix
// select over all keys replaces steps 2-3.  The histogram is zeroed for the
// next call.
//
// Short rows or many rows: one workgroup per query does all four steps
// (topk_select_kernel).  Few long rows: step 2 runs on one workgroup per
// (part of 16384 blocks, query) (topk_slice_kernel), which leaves the part's
// bitmap words, its count of listed keys and the list in the workspace; a
// second launch (topk_finish_kernel), one workgroup per query, gathers them
// and does steps 3-4.  The kernel boundary orders the hand-over.  Lists of
// at most 128 keys are ranked in step 3 by direct comparison instead of the
// radix passes.
// ---------------------------------------------------------------------------


// exclusive prefix sum over the kT threads of the workgroup; returns the
// block total in *total (tmp >= kT / 64 words)
template <int kT = kSelThreads>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t before_wave = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kT / 64; w++) {
    const uint32_t t = tmp[w];
    before_wave += w < wave ? t : 0u;
    all += t;
  }
  *total = all;
  __syncthreads();
  return before_wave + x - v;
}

// Over the nb-bin histogram: the bin x where the count from the top reaches
// `need`; found[0] = x, found[1] = keys in bins above x, found[2] = count(x).
__device__ __noinline__ void find_bin(const uint32_t* hist, uint32_t nb, uint32_t need, uint32_t* tmp,
                         uint32_t* found) {
  const int tid = threadIdx.x;
  const uint32_t per = nb >= kSelThreads ? nb / kSelThreads : 1;
  const uint32_t lo = (uint32_t)tid * per;
  const uint32_t hi = lo < nb ? lo + per : lo;
  uint32_t local = 0;
  for (uint32_t j = lo; j < hi; j++) local += hist[j];
  uint32_t total;
  const uint32_t below = block_exclusive_scan(local, tmp, &total);
  uint32_t running = total - below - local;
  for (int j = (int)hi - 1; j >= (int)lo; j--) {
    const uint32_t c = hist[j];
    if (running < need && running + c >= need) {
      found[0] = (uint32_t)j;
      found[1] = running;
      found[2] = c;
    }
    running += c;
  }
  __syncthreads();
}

// Visit the row's keys in 64-key words from word w_start on: wave w takes
// words w_start + w, + 16, ...; the keys of 8 words are loaded before any is
// used, so the loads overlap.
// A key load: plain, or (kCoherent) an agent-scope load that reads past the
// L2 of this XCD, for keys that other workgroups of the same launch wrote
// with agent-scope stores.
template <bool kCoherent>
__device__ __forceinline__ uint32_t load_key(const uint32_t* p) {
  return kCoherent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
}
constexpr int kCoherentAux = 16;   // buffer-load cache policy: sc1 (agent coherent)

template <bool kCoherent = false, typename F>
__device__ __forceinline__ void for_each_word(const uint32_t* keys, int nv, int nwords, F f, int w_start = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kBatch = 8;
#pragma unroll 1
  for (int wb = w_start + wave; wb < nwords; wb += kBatch * (kSelThreads / 64)) {
    uint32_t kk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int j = (wb + u * (kSelThreads / 64)) * 64 + lane;
      kk[u] = load_key<kCoherent>(keys + (j < nv ? j : 0));      // past the count: ignored by f (j >= nv)
    }
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int w = wb + u * (kSelThreads / 64);
      if (w < nwords) f(w, w * 64 + lane, kk[u]);
    }
  }
}

__device__ __forceinline__ void set_bit(uint32_t* bitmap, uint32_t j) {
  atomicOr(&bitmap[j >> 5], 1u << (j & 31));
}

// In a 1024-bin histogram, thread t holding bins 2t and 2t+1 (counts c0,
// c1): the bin where the count from the top reaches `need`: found[0] = bin,
// found[1] = keys in higher bins, found[2] = keys in the bin.  found[] must be
// preset; it is left unchanged when the histogram holds fewer than `need`
// keys.
__device__ __forceinline__ void find_bin_1024(uint32_t c0, uint32_t c1, uint32_t need, uint32_t* tmp,
                                              uint32_t* found) {
  uint32_t total;
  const uint32_t below = block_exclusive_scan(c0 + c1, tmp, &total);
  const uint32_t higher = total - below - c0 - c1;     // keys in bins above 2t + 1
  if (higher < need && higher + c1 >= need) {
    found[0] = 2 * threadIdx.x + 1;
    found[1] = higher;
    found[2] = c1;
  } else if (higher + c1 < need && higher + c1 + c0 >= need) {
    found[0] = 2 * threadIdx.x;
    found[1] = higher + c1;
    found[2] = c0;
  }
  __syncthreads();
}

// The 64 keys of round r of this thread (blocks r * kRoundKeys + 64 t ..),
// loaded unconditionally: a round past the end of the key row reads the
// row's last 64 keys, which are masked at use.  Buffer loads keep each
// 16-byte load whole (no re-split into overlapping pieces) and need no
// per-round address registers; the descriptor's range is the key row.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_row_rsrc(const uint32_t* keys, int64_t stride) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(keys), (short)0, (int)(stride * 4),
                                           kBufferWord3);
}

template <int NV, int kAux = 0>
__device__ __forceinline__ void load_keys(__amdgpu_buffer_rsrc_t row, int64_t stride, int b0, uint4 (&kv)[NV]) {
  b0 = b0 + 4 * NV <= stride ? b0 : (int)stride - 4 * NV;
#pragma unroll
  for (int v = 0; v < NV; v++) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(row, 4 * b0 + 16 * v, 0, kAux);
    kv[v] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

template <int kAux = 0>
__device__ __forceinline__ void load_round(__amdgpu_buffer_rsrc_t row, int64_t stride, int r, uint4 (&kv)[16]) {
  load_keys<16, kAux>(row, stride, r * kRoundKeys + 64 * (int)threadIdx.x, kv);
}

// Step 1 on the histogram held as thread t's bins 8t .. 8t+7 (hv0, hv1):
// found[0] = tb, found[1] = keys in higher bins.  found[] must be preset and
// read after a barrier.
__device__ __forceinline__ void threshold_bin(uint4 hv0, uint4 hv1, uint32_t k, uint32_t* tmp,
                                              uint32_t* found, uint32_t* gh_zero) {
  const int tid = threadIdx.x;
  const uint32_t c8 = hv0.x + hv0.y + hv0.z + hv0.w + hv1.x + hv1.y + hv1.z + hv1.w;
  uint32_t total;
  const uint32_t below = block_exclusive_scan(c8, tmp, &total);
  if (gh_zero) {   // for the next call
    reinterpret_cast<uint4*>(gh_zero)[2 * tid] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(gh_zero)[2 * tid + 1] = make_uint4(0, 0, 0, 0);
  }
  // walk the eight bins from the top (branch-free: at most one hits)
  const uint32_t cs[8] = {hv1.w, hv1.z, hv1.y, hv1.x, hv0.w, hv0.z, hv0.y, hv0.x};
  uint32_t run = total - below - c8;          // keys in bins above this thread's eight
  uint32_t hit = 0, hbin = 0, hrun = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t h = (run < k) & (run + cs[i] >= k);
    hbin = h ? (uint32_t)(8 * tid + 7 - i) : hbin;
    hrun = h ? run : hrun;
    hit |= h;
    run += cs[i];
  }
  if (hit) {
    found[0] = hbin;
    found[1] = hrun;
  }
}

// Step 2 for one thread's 4 NV keys of blocks b0 .. (lim = keys below the
// count): bit e of gt / eq set when key e is above / inside bin tb.  Plain
// integer arithmetic, no per-key lane masks: for bins in [0, 4096),
// tb - bin < 0 iff bin > tb, and (bin ^ tb) - 1 wraps iff they are equal.
template <int NV>
__device__ __forceinline__ void round_bits(const uint4 (&kv)[NV], uint32_t tb, int lim, uint32_t (&gt)[NV / 8],
                                           uint32_t (&eq)[NV / 8]) {
#pragma unroll
  for (int w = 0; w < NV / 8; w++) gt[w] = eq[w] = 0u;
#pragma unroll
  for (int v = 0; v < NV; v++) {
    const uint32_t q[4] = {kv[v].x, kv[v].y, kv[v].z, kv[v].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int e = 4 * v + i;
      const uint32_t bin = q[i] >> kHistShift;
      gt[e >> 5] |= ((tb - bin) >> 31) << (e & 31);
      eq[e >> 5] |= (((bin ^ tb) - 1u) >> 31) << (e & 31);
    }
  }
  // keys past the count are dropped
#pragma unroll
  for (int w = 0; w < NV / 8; w++) {
    const int l = lim - 32 * w;
    const uint32_t m = l >= 32 ? 0xFFFFFFFFu : (l <= 0 ? 0u : (1u << l) - 1u);
    gt[w] &= m;
    eq[w] &= m;
  }
}

// The keys inside bin tb, in block order, from list position pos on: keys to
// ckey[], their blocks to cblk[].
template <int NV>
__device__ __forceinline__ void list_round(const uint4 (&kv)[NV], const uint32_t (&eq)[NV / 8], int b0, uint32_t pos,
                                           uint32_t* ckey, uint32_t* cblk) {
#pragma unroll
  for (int v = 0; v < NV; v++) {
    const uint32_t q[4] = {kv[v].x, kv[v].y, kv[v].z, kv[v].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int e = 4 * v + i;
      if ((eq[e >> 5] >> (e & 31)) & 1u) {
        ckey[pos] = q[i];
        cblk[pos] = (uint32_t)(b0 + e);
        pos++;
      }
    }
  }
}

// Step 3: the nc listed keys (cand[0..nc) keys, cand[kCandCap..) blocks, in
// block order) all lie in bin tb, and `above` keys lie in higher bins.  Sets
// the bits of the listed keys that complete the top k.
__device__ __forceinline__ void rank_listed(const uint32_t* cand, uint32_t nc, uint32_t tb, uint32_t above,
                                            uint32_t k, uint32_t* hist, uint32_t* tmp, uint32_t* found,
                                            uint32_t* bitmap) {
  const int tid = threadIdx.x;
  uint32_t need = k - above;
  if (nc <= (uint32_t)kDirectRank) {
    // Short list: entry i is taken when fewer than `need` listed keys come
    // before it in (key desc, block asc) order.  Every listed key has the
    // bin's 12 high bits and the list is in block order, so the order is
    // that of the 32-bit value (low 20 key bits, 4095 - list position).
    __syncthreads();     // every thread's list entries are in place
    uint32_t* comp = hist;
    if ((uint32_t)tid < nc) comp[tid] = ((cand[tid] & 0xFFFFFu) << 12) | (4095u - (uint32_t)tid);
    __syncthreads();
    if ((uint32_t)tid < nc) {
      const uint32_t ci = comp[tid];
      uint32_t rank = 0;
#pragma unroll 8
      for (uint32_t j = 0; j < nc; j++) rank += comp[j] > ci ? 1u : 0u;
      if (rank < need) set_bit(bitmap, cand[kCandCap + tid]);
    }
    __syncthreads();
    return;
  }
  // exact threshold among the listed keys: bits 19..10, then 9..0.  A pass
  // whose bin holds exactly the keys still needed ends the search: every
  // listed key at or above that bin is taken.
  uint32_t pfx = tb;
  int shift = 20;
  bool exact = false;
#pragma unroll 1
  for (int pass = 0; pass < 2 && !exact; pass++) {
    shift -= 10;
    hist[2 * tid] = 0;
    hist[2 * tid + 1] = 0;
    if (tid == 0) found[0] = found[1] = found[2] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += kSelThreads) {
      const uint32_t key = cand[i];
      if ((key >> (shift + 10)) == pfx) atomicAdd(&hist[(key >> shift) & 1023u], 1u);
    }
    __syncthreads();
    find_bin_1024(hist[2 * tid], hist[2 * tid + 1], need, tmp, found);
    need -= found[1];
    pfx = (pfx << 10) | found[0];
    exact = found[2] == need;      // the bin's keys are exactly the ones needed
    __syncthreads();
  }
  // key >> shift compared with pfx: above -> taken; equal -> taken when the
  // bin is exactly what is needed, else ranked by block (list) order
  constexpr int kPerT = kCandCap / kSelThreads;
  const uint32_t i0 = kPerT * tid;
  uint32_t neq = 0;
#pragma unroll
  for (int i = 0; i < kPerT; i++) {
    const uint32_t j = i0 + i;
    if (j < nc) {
      const uint32_t kp = cand[j] >> shift;
      if (kp > pfx || (exact && kp == pfx)) set_bit(bitmap, cand[kCandCap + j]);
      neq += kp == pfx;
    }
  }
  if (!exact) {
    // shift is 0 here: pfx is the threshold key T, `need` keys equal to it
    uint32_t tot;
    uint32_t rank = block_exclusive_scan(neq, tmp, &tot);
#pragma unroll
    for (int i = 0; i < kPerT; i++) {
      const uint32_t j = i0 + i;
      if (j < nc && cand[j] == pfx) {
        if (rank < need) set_bit(bitmap, cand[kCandCap + j]);
        rank++;
      }
    }
  }
  __syncthreads();
}

// Steps 2-3 when too many keys share bin tb: radix select over every key
// (12 + 12 + 8 bits), then every key above the threshold T and the
// lowest-index keys equal to T.  Writes every bitmap word of the row.
template <bool kCoherent = false>
__device__ __forceinline__ void select_all(const uint32_t* keys, int nv, uint32_t k, uint32_t* hist,
                                           uint32_t* tmp, uint32_t* found, uint32_t* cand, uint32_t* bitmap) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int nwords = (nv + 63) >> 6;
  uint32_t pfx = 0, need = k;
#pragma unroll
  for (int d = 0; d < 3; d++) {
    const int shift = d == 0 ? 20 : (d == 1 ? 8 : 0), width = d == 2 ? 8 : 12;
    const uint32_t nb = 1u << width, mask = nb - 1;
    for (uint32_t j = tid; j < nb; j += kSelThreads) hist[j] = 0;
    __syncthreads();
    for_each_word<kCoherent>(keys, nv, nwords, [&](int w, int j, uint32_t key) {
      if (j < nv && (d == 0 || (key >> (shift + width)) == pfx))
        atomicAdd(&hist[(key >> shift) & mask], 1u);
    });
    __syncthreads();
    find_bin(hist, nb, need, tmp, found);
    need -= found[1];
    pfx = (pfx << width) | found[0];
    __syncthreads();
  }
  const uint32_t T = pfx, need_eq = need;
  // equal keys per 64-block word (the candidate list doubles as the counts)
  uint32_t* eqc = cand;       // 2 * kCandCap >= kMaxWords counters
  for_each_word<kCoherent>(keys, nv, nwords, [&](int w, int j, uint32_t key) {
    const uint64_t gm = __ballot(j < nv && key > T);
    const uint64_t em = __ballot(j < nv && key == T);
    if (lane == 0) {
      bitmap[2 * w] = (uint32_t)gm;
      bitmap[2 * w + 1] = (uint32_t)(gm >> 32);
      eqc[w] = (uint32_t)__popcll(em);
    }
  });
  __syncthreads();
  const int wp = (nwords + kSelThreads - 1) / kSelThreads;
  const int a0 = tid * wp, a1 = min(nwords, a0 + wp);
  uint32_t loc = 0;
  for (int w = a0; w < a1; w++) loc += eqc[w];
  uint32_t tot;
  uint32_t run = block_exclusive_scan(loc, tmp, &tot);
  for (int w = a0; w < a1; w++) {
    const uint32_t c = eqc[w];
    eqc[w] = run;
    run += c;
  }
  __syncthreads();
  for_each_word<kCoherent>(keys, nv, nwords, [&](int w, int j, uint32_t key) {
    const bool eq = j < nv && key == T;
    const uint64_t em = __ballot(eq);
    const uint32_t rank = eqc[w] + (uint32_t)__popcll(em & ((1ull << lane) - 1ull));
    if (eq && rank < need_eq) set_bit(bitmap, (uint32_t)j);
  });
  __syncthreads();
}

// Step 4: ascending block order.  Wave w takes `steps` runs of 64 words,
// from word 64 * steps * w on; in a run, lane l holds word l (consecutive
// lanes read consecutive words, free of bank conflicts).  The words are read
// once into registers; their bit counts and a block scan give each wave its
// first output position, and a wave scan per run places each word's bits.
// Runs without a set bit are skipped, and a wave stops once its positions
// pass k.
__device__ __forceinline__ void compact(const uint32_t* bitmap, int nv, int k, int32_t* out, uint32_t* tmp) {
  constexpr int kMaxSteps = 2 * kMaxWords / (64 * kSelWaves);   // 32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwords32 = (nv + 31) >> 5;
  const int steps = (nwords32 + 64 * kSelWaves - 1) / (64 * kSelWaves);
  const int wbase = wave * steps * 64;
  uint32_t wv[kMaxSteps];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kMaxSteps; j++) {
    const int w = wbase + 64 * j + lane;
    wv[j] = (j < steps && w < nwords32) ? bitmap[w] : 0u;
    c += (uint32_t)__popc(wv[j]);
  }
  uint32_t tot;
  const uint32_t excl = block_exclusive_scan(c, tmp, &tot);
  uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, 0);   // bits in the waves before this one
#pragma unroll
  for (int j = 0; j < kMaxSteps; j++) {
    if (j >= steps || base >= (uint32_t)k) break;
    uint32_t bits = wv[j];
    if (__ballot(bits != 0u) == 0) continue;
    const int w = wbase + 64 * j + lane;
    const uint32_t cw = (uint32_t)__popc(bits);
    const uint32_t incl = wave_inclusive_scan(cw);
    uint32_t pos = base + incl - cw;
    base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = w * 32 + b;
      pos++;
    }
  }
}

// visible blocks of query row srow (row length through the scalar cache)
__device__ __forceinline__ int visible_blocks(const SelectArgs& a, int srow) {
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const int p = *(const_i32p)(a.seq_len + brow) - a.n_q + qi;
  int nv = (p + 1) / a.m;
  if (nv > a.stride) {                         // more blocks than the plan holds
    if (threadIdx.x == 0) atomicOr(a.status, LCA_STATUS_INDEXER_CAPACITY);
    nv = (int)a.stride;
  }
  return nv;
}

// Steps 1-4 for query row srow on one workgroup of kSelThreads threads, with
// the LDS arrays passed in: hist (kHistBins words), tmp (64), found (4),
// cand (2 kCandCap), bitmap (2 kMaxWords).  kCoherent: the histogram and
// keys were written earlier in the same launch (agent-scope stores and
// atomics), so they are read with agent-scope loads.
template <bool kCoherent>
__device__ __forceinline__ void select_row(const SelectArgs& a, int srow, uint32_t* hist, uint32_t* tmp,
                                           uint32_t* found, uint32_t* cand, uint32_t* bitmap) {
  constexpr int kAux = kCoherent ? kCoherentAux : 0;
  const int k = a.k, tid = threadIdx.x;
  int32_t* out = a.topk + (int64_t)srow * k;
  const uint32_t* keys = a.keys + (int64_t)srow * a.stride;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;

  // The histogram loads go out first, then the keys of rounds 0 and 1, so
  // that the histogram phase does not wait for the keys (loads complete in
  // issue order).  Nothing here waits for the row length: the loads are
  // addressed within the key row, and the length comes through the scalar
  // cache after they are issued.  Round r + 2 is loaded while round r + 1
  // is processed (two register sets, no copies).
  uint4 hv[2];
  load_keys<2, kAux>(key_row_rsrc(gh, kHistBins), kHistBins, 8 * tid, hv);
  const __amdgpu_buffer_rsrc_t krow = key_row_rsrc(keys, a.stride);
  uint4 ka[16], kb[16];
  load_round<kAux>(krow, a.stride, 0, ka);
  load_round<kAux>(krow, a.stride, 1, kb);
  const int nv = visible_blocks(a, srow);
  const int rounds = (nv + kRoundKeys - 1) / kRoundKeys;
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;
  threshold_bin(hv[0], hv[1], (uint32_t)k, tmp, found, gh);
  if (nv <= k) {
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
    return;
  }
  __syncthreads();
  const uint32_t tb = found[0], above = found[1];

  uint32_t nc = 0;
  auto one_round = [&](const uint4 (&kv)[16], int r) {
    const int b0 = r * kRoundKeys + 64 * tid;
    const int lim = nv - b0;                    // keys of this thread below the count
    uint32_t gt[2], eq[2];
    round_bits(kv, tb, lim, gt, eq);
    const uint32_t cnt = (uint32_t)(__popc(eq[0]) + __popc(eq[1]));
    if (lim > 0) bitmap[2 * (r * kSelThreads + tid)] = gt[0];
    if (lim > 32) bitmap[2 * (r * kSelThreads + tid) + 1] = gt[1];
    uint32_t tot;
    const uint32_t pos = nc + block_exclusive_scan(cnt, tmp, &tot);
    if (nc + tot <= (uint32_t)kCandCap && cnt) list_round(kv, eq, b0, pos, cand, cand + kCandCap);
    nc += tot;
  };
#pragma unroll 1
  for (int r = 0; r < rounds; r += 2) {
    one_round(ka, r);
    if (r + 1 >= rounds) break;
    load_round<kAux>(krow, a.stride, r + 2, ka);
    one_round(kb, r + 1);
    load_round<kAux>(krow, a.stride, r + 3, kb);
  }

  if (nc <= (uint32_t)kCandCap)
    rank_listed(cand, nc, tb, above, (uint32_t)k, hist, tmp, found, bitmap);
  else
    select_all<kCoherent>(keys, nv, (uint32_t)k, hist, tmp, found, cand, bitmap);
  compact(bitmap, nv, k, out, tmp);
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[4];
  __shared__ uint32_t cand[2 * kCandCap];      // listed keys, then their blocks (block order)
  __shared__ uint32_t bitmap[2 * kMaxWords];   // bit j of word w: block 32 w + j
  select_row<false>(a, blockIdx.x, hist, tmp, found, cand, bitmap);
}

// Step 2 of one part of kPartKeys blocks (blockIdx.x) of one query
// (blockIdx.y); thread t takes the 32 blocks of bitmap word 512 p + t.
__global__ void __launch_bounds__(kSelThreads) topk_slice_kernel(SelectArgs a) {
  const int p = blockIdx.x, srow = blockIdx.y;
  const int tid = threadIdx.x;
  const uint32_t* keys = a.keys + (int64_t)srow * a.stride;
  const uint32_t* gh = a.hist + (int64_t)srow * kHistBins;

  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[4];

  const uint4 hv0 = reinterpret_cast<const uint4*>(gh)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(gh)[2 * tid + 1];
  const int b0 = p * kPartKeys + 32 * tid;
  uint4 kv[8];
  load_keys(key_row_rsrc(keys, a.stride), a.stride, b0, kv);
  const int nv = visible_blocks(a, srow);
  if (nv <= a.k || p * kPartKeys >= nv) return;   // nothing of this part is read
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;
  threshold_bin(hv0, hv1, (uint32_t)a.k, tmp, found, nullptr);
  __syncthreads();
  const uint32_t tb = found[0];
  uint32_t gt[1], eq[1];
  round_bits(kv, tb, nv - b0, gt, eq);
  const int64_t part = (int64_t)srow * a.slices + p;
  a.part_bits[part * kSelThreads + tid] = gt[0];
  const uint32_t cnt = (uint32_t)__popc(eq[0]);
  uint32_t tot;
  const uint32_t pos = block_exclusive_scan(cnt, tmp, &tot);
  if (tid == 0) a.part_count[part] = tot;
  uint32_t* pc = a.part_cand + part * 2 * kCandCap;
  if (tot <= (uint32_t)kCandCap && cnt) list_round(kv, eq, b0, pos, pc, pc + kCandCap);
}

// Steps 3-4 of one query from the parts that topk_slice_kernel left.  The
// first S = kCandCap / slices (rounded down to 8) entries of every part's
// list are loaded with everything else, before the counts are known; only a
// part with more than S listed keys needs a second, dependent gather.
__global__ void __launch_bounds__(kSelThreads) topk_finish_kernel(SelectArgs a) {
  const int srow = blockIdx.x;
  const int k = a.k, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* out = a.topk + (int64_t)srow * k;
  const uint32_t* keys = a.keys + (int64_t)srow * a.stride;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;
  const int nw4 = a.slices * (kSelThreads / 4);   // uint4 words of the row's part bitmaps
  const uint4* pb = reinterpret_cast<const uint4*>(a.part_bits + (int64_t)srow * a.slices * kSelThreads);
  const uint32_t* pn = a.part_count + (int64_t)srow * a.slices;
  const uint32_t* pc = a.part_cand + (int64_t)srow * a.slices * 2 * kCandCap;

  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[4];
  __shared__ uint32_t soff[kMaxParts + 2];     // list offset of each part, the total, a spill flag
  __shared__ uint32_t cand[2 * kCandCap];
  __shared__ uint32_t bitmap[2 * kMaxWords];

  // Everything this query needs goes out before any of it is used, in the
  // order of use: histogram, counts, list entries, bitmap words.
  const uint4 hv0 = reinterpret_cast<const uint4*>(gh)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(gh)[2 * tid + 1];
  const uint32_t my_count = pn[tid < a.slices ? tid : 0];
  const uint32_t S = (uint32_t)(kCandCap / a.slices) & ~7u;
  const uint32_t j0 = 8u * (uint32_t)tid;      // this thread's entry slots j0 .. j0+7
  const uint32_t ss = j0 / S;                  // their part
  const uint32_t si = j0 - ss * S;             // their first entry in that part
  const bool slot_ok = ss < (uint32_t)a.slices;
  const uint4* sk = reinterpret_cast<const uint4*>(pc + (slot_ok ? ss * 2 * kCandCap + si : 0));
  const uint4 sk0 = sk[0], sk1 = sk[1];
  const uint4 sb0 = sk[kCandCap / 4], sb1 = sk[kCandCap / 4 + 1];
  constexpr int kBw = 2 * kMaxWords / 4 / kSelThreads;   // uint4 words per thread: 8
  uint4 bw[kBw];
#pragma unroll
  for (int i = 0; i < kBw; i++) {
    const int j = i * kSelThreads + tid;
    bw[i] = pb[j < nw4 ? j : 0];
  }
  const int nv = visible_blocks(a, srow);
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;
  threshold_bin(hv0, hv1, (uint32_t)k, tmp, found, gh);
  if (nv <= k) {
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const int parts = (nv + kPartKeys - 1) / kPartKeys;
  if (wave == 0) {
    // part offsets by a wave scan over the counts (parts <= kMaxParts <= 64)
    const uint32_t c = lane < parts ? my_count : 0u;
    const uint32_t incl = wave_inclusive_scan(c);
    if (lane < kMaxParts) soff[lane] = incl - c;
    if (lane == 63) soff[kMaxParts] = incl;
    const bool spill = __ballot(c > S) != 0;
    if (lane == 0) soff[kMaxParts + 1] = spill ? 1u : 0u;
  }
#pragma unroll
  for (int i = 0; i < kBw; i++) {
    const int j = i * kSelThreads + tid;
    if (j < nw4) reinterpret_cast<uint4*>(bitmap)[j] = bw[i];
  }
  __syncthreads();
  const uint32_t tb = found[0], above = found[1];
  const uint32_t nc = soff[kMaxParts];
  if (nc <= (uint32_t)kCandCap) {
    if (!soff[kMaxParts + 1]) {
      // every list fits its S slots: place the loaded entries
      if (slot_ok && ss < (uint32_t)parts) {
        const uint32_t b = soff[ss], cnt = soff[ss + 1] - b;
        const uint32_t ks[8] = {sk0.x, sk0.y, sk0.z, sk0.w, sk1.x, sk1.y, sk1.z, sk1.w};
        const uint32_t bs[8] = {sb0.x, sb0.y, sb0.z, sb0.w, sb1.x, sb1.y, sb1.z, sb1.w};
#pragma unroll
        for (int u = 0; u < 8; u++) {
          if (si + u < cnt) {
            cand[b + si + u] = ks[u];
            cand[kCandCap + b + si + u] = bs[u];
          }
        }
      }
    } else {
      // gather the lists: entry i of the row comes from the part r with
      // soff[r] <= i < soff[r + 1]
      uint32_t off[kMaxParts];
#pragma unroll
      for (int r = 0; r < kMaxParts; r++) off[r] = soff[r];
      constexpr int kPerT = kCandCap / kSelThreads;
      uint32_t ck[kPerT], cb[kPerT];
#pragma unroll
      for (int u = 0; u < kPerT; u++) {
        const uint32_t i = (uint32_t)(u * kSelThreads + tid);
        uint32_t r = 0, o = 0;
#pragma unroll
        for (int t = 1; t < kMaxParts; t++) {
          const bool in = t < parts && off[t] <= i;   // parts <= slices
          r += in ? 1u : 0u;
          o = in ? off[t] : o;
        }
        const uint32_t* src = pc + (int64_t)r * 2 * kCandCap;
        const uint32_t e = i < nc ? i - o : 0u;
        ck[u] = src[e];
        cb[u] = src[kCandCap + e];
      }
#pragma unroll
      for (int u = 0; u < kPerT; u++) {
        const uint32_t i = (uint32_t)(u * kSelThreads + tid);
        if (i < nc) {
          cand[i] = ck[u];
          cand[kCandCap + i] = cb[u];
        }
      }
    }
    __syncthreads();
    rank_listed(cand, nc, tb, above, (uint32_t)k, hist, tmp, found, bitmap);
  } else {
    select_all(keys, nv, (uint32_t)k, hist, tmp, found, cand, bitmap);
  }
  compact(bitmap, nv, k, out, tmp);
}

// ---------------------------------------------------------------------------
// Selection from the candidate lists of the tile kernel, one workgroup per
// query.  Step 1 as above (the histogram counts every key).  Step 2 walks the
// lists: keys above bin tb set their bit, keys inside tb are listed in LDS in
// no particular order.  Step 3 ranks the listed keys by (key desc, block asc)
// -- directly for short lists, else by two radix passes over the key bits
// and, when keys equal to the threshold key T must be split, two more over
// the block indices of those keys.  If more than kCandCap keys share bin tb,
// step 3 runs its passes over the lists in memory instead.  Step 4 compacts.
// The bitmap is dynamic LDS of (stride + 31) / 32 words.
// ---------------------------------------------------------------------------

// f(ok, key, block) for every entry of the query's lists, called by all lanes
// of a wavefront together (ok false where there is no entry).  The lists of
// chunk c and tile wavefront v form group r = c * kTileWavesPerSet + v;
// wavefront w takes groups w, w + 8, ...  Entry j of the list of column col
// is the pair (key, t) in slot c * span + 32 (v + kTileWavesPerSet j) + col,
// naming block c * span + 32 (v + kTileWavesPerSet t) + col.  Lanes l and
// l + 32 read column l % 32 at levels j and j + 1.
template <typename F>
__device__ __forceinline__ void for_each_cand(const SelectArgs& a, const uint2* pairs, const uint32_t* cnt, F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  constexpr int kB = 8;
#pragma unroll 1
  for (int r = wave; r < a.segs; r += kSelWaves) {
    const int c = r / kTileWavesPerSet, v = r % kTileWavesPerSet;
    const uint32_t b0 = (uint32_t)(c * a.span + 32 * v + col);
    const uint32_t n = cnt[32 * r + col];
    const uint32_t nmax = (uint32_t)wave_minmax<1>((int)n);
#pragma unroll 1
    for (uint32_t j0 = 0; j0 < nmax; j0 += 2 * kB) {
      uint2 e[kB];
#pragma unroll
      for (int u = 0; u < kB; u++) {
        const uint32_t j = j0 + 2 * u + half;
        e[u] = j < n ? pairs[b0 + 32u * kTileWavesPerSet * j] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kB; u++) {
        const uint32_t j = j0 + 2 * u + half;
        f(j < n, e[u].x, b0 + 32u * kTileWavesPerSet * e[u].y);
      }
    }
  }
}

// Step 3 over unordered entries, all in bin tb: sets the bits of the `need`
// largest by (key desc, block asc).  each(g) calls g(key, block) for every
// entry, from any thread.
template <typename Each>
__device__ __forceinline__ void rank_unordered(Each each, uint32_t tb, uint32_t need, uint32_t* hist1024,
                                               uint32_t* tmp, uint32_t* found, uint32_t* bitmap) {
  const int tid = threadIdx.x;
  // the threshold key T: bits 19..0 below the bin's 12
  uint32_t need_k = need;
  int shift;
  uint32_t pfx = tb;
  {
    shift = 20;
    bool exact = false;
#pragma unroll 1
    for (int pass = 0; pass < 2 && !exact; pass++) {
      shift -= 10;
      hist1024[2 * tid] = 0;
      hist1024[2 * tid + 1] = 0;
      if (tid == 0) found[0] = found[1] = found[2] = 0;
      __syncthreads();
      const int sh = shift;
      const uint32_t pf = pfx;
      each([&](uint32_t key, uint32_t) {
        if ((key >> (sh + 10)) == pf) atomicAdd(&hist1024[(key >> sh) & 1023u], 1u);
      });
      __syncthreads();
      find_bin_1024(hist1024[2 * tid], hist1024[2 * tid + 1], need_k, tmp, found);
      need_k -= found[1];
      pfx = (pfx << 10) | found[0];
      exact = found[2] == need_k;
      __syncthreads();
    }
    if (exact) {
      each([&](uint32_t key, uint32_t blk) {
        if ((key >> shift) >= pfx) set_bit(bitmap, blk);
      });
      __syncthreads();
      return;
    }
  }
  // shift is 0: pfx is T, and need_k of the keys equal to T are taken, those
  // of the lowest blocks: the same passes over 0xFFFFF - block
  const uint32_t T = pfx;
  uint32_t vp = 0;
  int vsh = 20;
  bool vexact = false;
#pragma unroll 1
  for (int pass = 0; pass < 2 && !vexact; pass++) {
    vsh -= 10;
    hist1024[2 * tid] = 0;
    hist1024[2 * tid + 1] = 0;
    if (tid == 0) found[0] = found[1] = found[2] = 0;
    __syncthreads();
    const int sh = vsh;
    const uint32_t pf = vp;
    each([&](uint32_t key, uint32_t blk) {
      const uint32_t x = 0xFFFFFu - blk;
      if (key == T && (x >> (sh + 10)) == pf) atomicAdd(&hist1024[(x >> sh) & 1023u], 1u);
    });
    __syncthreads();
    find_bin_1024(hist1024[2 * tid], hist1024[2 * tid + 1], need_k, tmp, found);
    need_k -= found[1];
    vp = (vp << 10) | found[0];
    vexact = found[2] == need_k;     // block indices are distinct: always true after the second pass
    __syncthreads();
  }
  each([&](uint32_t key, uint32_t blk) {
    if (key > T || (key == T && ((0xFFFFFu - blk) >> vsh) >= vp)) set_bit(bitmap, blk);
  });
  __syncthreads();
}

__global__ void __launch_bounds__(kSelThreads) topk_cand_kernel(SelectArgs a) {
  const int srow = blockIdx.x;
  const int k = a.k, tid = threadIdx.x, lane = tid & 63;
  int32_t* out = a.topk + (int64_t)srow * k;
  const uint2* pairs = reinterpret_cast<const uint2*>(a.keys) + (int64_t)srow * a.stride;
  const uint32_t* cnt = a.cand_count + (int64_t)srow * a.segs * 32;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;

  __shared__ uint32_t hist1024[1024];
  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[4];
  __shared__ uint32_t nlist;
  __shared__ uint32_t cand[2 * kCandCap];      // keys in bin tb, then their blocks
  extern __shared__ uint32_t bitmap[];         // bit j of word w: block 32 w + j

  const uint4 hv0 = reinterpret_cast<const uint4*>(gh)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(gh)[2 * tid + 1];
  const int nv = visible_blocks(a, srow);
  if (tid == 0) {
    found[0] = found[1] = found[2] = found[3] = 0;
    nlist = 0;
  }
  threshold_bin(hv0, hv1, (uint32_t)k, tmp, found, gh);
  if (nv <= k) {
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const int nwords32 = (nv + 31) >> 5;
  for (int w = tid; w < nwords32; w += kSelThreads) bitmap[w] = 0u;
  __syncthreads();
  const uint32_t tb = found[0], above = found[1];
  for_each_cand(a, pairs, cnt, [&](bool ok, uint32_t key, uint32_t blk) {
    const uint32_t bin = key >> kHistShift;
    if (ok && bin > tb) set_bit(bitmap, blk);
    const bool in = ok && bin == tb;
    const uint64_t bm = __ballot(in);
    if (bm) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&nlist, (uint32_t)__popcll(bm));
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
      const uint32_t p = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      if (in && p < (uint32_t)kCandCap) {
        cand[p] = key;
        cand[kCandCap + p] = blk;
      }
    }
  });
  __syncthreads();
  const uint32_t nc = nlist;
  const uint32_t need = (uint32_t)k - above;
  if (nc <= (uint32_t)kDirectRank) {
    // short list: entry i is taken when fewer than `need` entries come before
    // it in (key desc, block asc) order
    if ((uint32_t)tid < nc) {
      const uint32_t ki = cand[tid], bi = cand[kCandCap + tid];
      uint32_t rank = 0;
#pragma unroll 4
      for (uint32_t j = 0; j < nc; j++) {
        const uint32_t kj = cand[j], bj = cand[kCandCap + j];
        rank += (kj > ki || (kj == ki && bj < bi)) ? 1u : 0u;
      }
      if (rank < need) set_bit(bitmap, bi);
    }
    __syncthreads();
  } else if (nc <= (uint32_t)kCandCap) {
    rank_unordered([&](auto g) {
      for (uint32_t i = tid; i < nc; i += kSelThreads) g(cand[i], cand[kCandCap + i]);
    }, tb, need, hist1024, tmp, found, bitmap);
  } else {
    // the lists in memory, keys of bin tb only
    rank_unordered([&](auto g) {
      for_each_cand(a, pairs, cnt, [&](bool ok, uint32_t key, uint32_t blk) {
        if (ok && (key >> kHistShift) == tb) g(key, blk);
      });
    }, tb, need, hist1024, tmp, found, bitmap);
  }
  compact(bitmap, nv, k, out, tmp);
}

// ---------------------------------------------------------------------------
// The selection inside the decode scoring launch (kFused; workgroups of 256
// threads, as the scoring without it).
//
// Each scoring workgroup holds the keys of its blocks in LDS (dyn) and their
// histogram (lhist).  The highest bin b whose higher bins hold at least k of
// its own keys lies below the row's threshold bin tb (the row's counts are at
// least the workgroup's), so only its bins above b go to the row's histogram
// and only its keys above b can be among the row's top k.  The row's
// histogram as it stands (other workgroups' flushes, each count at most its
// final value) often gives a higher such bin; either is valid.  The
// workgroup writes its keys above the bound as (key, block) pairs, in block
// order, to its segment (slot wg_b0 of the row's pair array; capacity: its
// blocks), the count to cand_count[row][workgroup], and arrives at the row's
// counter.  The row's last workgroup to arrive selects:
//   1. the final row histogram gives tb and the count of keys above it (and
//      is zeroed for the next call); the segment counts give the offset of
//      every segment in the row's candidate sequence;
//   2. one pass over the candidates: those above bin tb set their bit in an
//      LDS bitmap of the row's blocks, those inside it go to an LDS list;
//   3. the list is ranked by (key desc, block asc): a histogram of key bits
//      19..10, built during the pass, gives the sub-bin of the last key
//      taken; entries above it are taken and those inside it ranked by
//      direct comparison (more than kFusedTies entries in bin tb: radix
//      passes over the candidates in memory);
//   4. the bitmap is compacted into ascending block indices.
// ---------------------------------------------------------------------------

constexpr int kFT = 256;              // threads of a fused scoring workgroup
constexpr int kFusedTies = 2048;      // bin-tb candidates the selecting workgroup ranks in LDS
constexpr int kMaxFusedSegs = 256;    // scoring workgroups per row
constexpr int kMaxFusedCpw = 4;       // chunks per scoring workgroup: <= 4096 keys in LDS
constexpr int kFusedDirect = 2 * kFT; // bin-tb lists up to this long are ranked directly
constexpr int kBoundWindow = 256;     // histogram bins a scoring workgroup reads for its row bound

// The segments holding candidates i[0..N-1] (each < soff[nseg]): for each,
// the largest s < nseg with soff[s] <= i (soff ascending, soff[0] = 0,
// soff[nseg] = the candidate count), by binary searches run side by side:
// every halving step issues the N LDS reads together, without branches.  The
// steps depend on one another, so they stay a loop (less code to fetch).
template <int N>
__device__ __forceinline__ void segments_of(const uint32_t* soff, int nseg, const uint32_t (&i)[N], int (&s)[N]) {
  static_assert(kMaxFusedSegs <= 256, "eight halving steps");
#pragma unroll
  for (int u = 0; u < N; u++) s[u] = 0;
#pragma unroll 1
  for (int step = 128; step > 0; step >>= 1) {
#pragma unroll
    for (int u = 0; u < N; u++) {
      const int t = min(s[u] + step, nseg);          // soff[nseg] > i: never taken
      s[u] = soff[t] <= i[u] ? t : s[u];
    }
  }
}

// Over the 1024-bin LDS histogram h (thread t holds bins P t .. P t + P - 1,
// P = 1024 / kT): the bin where the count from the top reaches `need`:
// found[0] = bin, found[1] = keys in higher bins, found[2] = keys in the bin.
// found[] must be preset; unchanged when h holds fewer than `need` keys.
template <int kT>
__device__ __forceinline__ void find_bin_1024_t(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* found) {
  constexpr int P = 1024 / kT;
  const int tid = threadIdx.x;
  uint32_t c[P], local = 0;
#pragma unroll
  for (int i = 0; i < P; i++) {
    c[i] = h[P * tid + i];
    local += c[i];
  }
  uint32_t total;
  const uint32_t below = block_exclusive_scan<kT>(local, tmp, &total);
  uint32_t run = total - below - local;           // keys in bins above this thread's
#pragma unroll
  for (int i = P - 1; i >= 0; i--) {
    if (run < need && run + c[i] >= need) {
      found[0] = (uint32_t)(P * tid + i);
      found[1] = run;
      found[2] = c[i];
    }
    run += c[i];
  }
  __syncthreads();
}

// The `need` largest by (key desc, block asc) of n list entries that all lie
// in bin tb (bits 31..20 of the key); entry j is get(j) = (key, block) and
// mark(j) is called for each one taken.  Direct comparison up to
// kFusedDirect entries, else radix passes of 10 bits over the key's low 20
// bits and, for entries equal to the threshold key, over 0xFFFFF - block.
template <int kT, typename Get, typename Mark>
__device__ __forceinline__ void rank_bin_list(int n, Get get, uint32_t tb, uint32_t need, uint32_t* hist1024,
                                              uint32_t* tmp, uint32_t* found, Mark mark) {
  const int tid = threadIdx.x;
  if (n <= kFusedDirect) {
#pragma unroll
    for (int r = 0; r < kFusedDirect / kT; r++) {
      const int i = tid + r * kT;
      if (i < n) {
        const uint2 ei = get(i);
        uint32_t rank = 0;
        for (int j = 0; j < n; j++) {
          const uint2 ej = get(j);
          rank += (ej.x > ei.x || (ej.x == ei.x && ej.y < ei.y)) ? 1u : 0u;
        }
        if (rank < need) mark(i);
      }
    }
    __syncthreads();
    return;
  }
  // threshold key T among the entries: bits 19..10, then 9..0
  uint32_t need_k = need, pfx = tb;
  int shift = 20;
  bool exact = false;
#pragma unroll 1
  for (int pass = 0; pass < 2 && !exact; pass++) {
    shift -= 10;
    for (int i = tid; i < 1024; i += kT) hist1024[i] = 0;
    if (tid == 0) found[0] = found[1] = found[2] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kT) {
      const uint32_t key = get(i).x;
      if ((key >> (shift + 10)) == pfx) atomicAdd(&hist1024[(key >> shift) & 1023u], 1u);
    }
    __syncthreads();
    find_bin_1024_t<kT>(hist1024, need_k, tmp, found);
    need_k -= found[1];
    pfx = (pfx << 10) | found[0];
    exact = found[2] == need_k;
    __syncthreads();
  }
  if (exact) {
    for (int i = tid; i < n; i += kT)
      if ((get(i).x >> shift) >= pfx) mark(i);
    __syncthreads();
    return;
  }
  // shift is 0: pfx is the threshold key T; need_k of the entries equal to
  // it are taken, those of the lowest blocks
  const uint32_t T = pfx;
  uint32_t vp = 0;
  int vsh = 20;
  bool vexact = false;
#pragma unroll 1
  for (int pass = 0; pass < 2 && !vexact; pass++) {
    vsh -= 10;
    for (int i = tid; i < 1024; i += kT) hist1024[i] = 0;
    if (tid == 0) found[0] = found[1] = found[2] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kT) {
      const uint2 e = get(i);
      const uint32_t x = 0xFFFFFu - e.y;
      if (e.x == T && (x >> (vsh + 10)) == vp) atomicAdd(&hist1024[(x >> vsh) & 1023u], 1u);
    }
    __syncthreads();
    find_bin_1024_t<kT>(hist1024, need_k, tmp, found);
    need_k -= found[1];
    vp = (vp << 10) | found[0];
    vexact = found[2] == need_k;     // blocks are distinct: true after the second pass
    __syncthreads();
  }
  for (int i = tid; i < n; i += kT) {
    const uint2 e = get(i);
    if (e.x > T || (e.x == T && ((0xFFFFFu - e.y) >> vsh) >= vp)) mark(i);
  }
  __syncthreads();
}

// The selecting (last) workgroup of row srow.  lhist: 4096 words of LDS
// (free; it takes the sub-bin list); dyn: the dynamic LDS: the row's bitmap
// (nv bits), then up to kFusedTies bin-tb candidates (keys, blocks) and a
// 1024-bin histogram.
__device__ __forceinline__ void fused_select(const ScoreArgs& a, const SelectArgs& sel, int srow, int nv,
                                          uint32_t* lhist, uint32_t* dyn, uint32_t* tmp, uint32_t* found) {
  constexpr int kT = kFT;
  const int k = a.k, tid = threadIdx.x;
  const int nseg = (int)gridDim.x, span = a.fused_span;
  int32_t* out = sel.topk + (int64_t)srow * k;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;
  const uint64_t* row_pairs = reinterpret_cast<const uint64_t*>(a.keys) + (int64_t)srow * a.stride;
  __shared__ uint32_t soff[kMaxFusedSegs + 1];
  __shared__ uint32_t ntie;

  // 1. the row's histogram (16 bins per thread) and segment counts, read
  //    past the caches
  uint4 hv[4];
  load_keys<4, kCoherentAux>(key_row_rsrc(gh, kHistBins), kHistBins, 16 * tid, hv);
  const uint32_t my_count =
      tid < nseg ? __hip_atomic_load(&a.cand_count[(int64_t)srow * nseg + tid], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT)
                 : 0u;
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;
  {
    const uint32_t cs[16] = {hv[3].w, hv[3].z, hv[3].y, hv[3].x, hv[2].w, hv[2].z, hv[2].y, hv[2].x,
                             hv[1].w, hv[1].z, hv[1].y, hv[1].x, hv[0].w, hv[0].z, hv[0].y, hv[0].x};
    uint32_t c16 = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) c16 += cs[i];
    uint32_t total;
    const uint32_t below = block_exclusive_scan<kT>(c16, tmp, &total);
#pragma unroll
    for (int v = 0; v < 4; v++) reinterpret_cast<uint4*>(gh)[4 * tid + v] = make_uint4(0, 0, 0, 0);   // next call
    uint32_t run = total - below - c16;              // keys in bins above this thread's 16
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (run < (uint32_t)k && run + cs[i] >= (uint32_t)k) {
        found[0] = (uint32_t)(16 * tid + 15 - i);
        found[1] = run;
      }
      run += cs[i];
    }
  }
  uint32_t ctot;
  const uint32_t cbase = block_exclusive_scan<kT>(my_count, tmp, &ctot);   // nseg <= kT
  if (tid < nseg) soff[tid] = cbase;
  if (tid == 0) {
    soff[nseg] = ctot;
    ntie = 0;
  }
  if (nv <= k) {
    for (int j = tid; j < k; j += kT) out[j] = j < nv ? j : -1;
    return;
  }
  const int nwords32 = (nv + 31) >> 5;
  uint32_t* bitmap = dyn;
  uint32_t* tkey = dyn + nwords32;
  uint32_t* tblk = tkey + kFusedTies;
  uint32_t* hist1024 = tblk + kFusedTies;
  for (int w = tid; w < nwords32; w += kT) bitmap[w] = 0u;
  for (int i = tid; i < 1024; i += kT) hist1024[i] = 0u;
  __syncthreads();
  const uint32_t tb = found[0], need = (uint32_t)k - found[1];
  const uint32_t C = ctot;
  // 2. one pass over the candidates, kPer per thread in flight: above bin tb
  //    -> bit; inside it -> the LDS list and a histogram of key bits 19..10
  //    (2048 per pass: a decode row has a few thousand candidates at most,
  //    and a wider unrolled pass costs more instruction fetch than it saves)
  constexpr int kPer = 8;
#pragma unroll 1
  for (uint32_t c0 = 0; c0 < C; c0 += kPer * kT) {
    uint64_t e[kPer];
    uint32_t ci[kPer];
    int sg[kPer];                                     // soff[sg] <= i < soff[sg + 1]
#pragma unroll
    for (int u = 0; u < kPer; u++) ci[u] = min(c0 + (uint32_t)(u * kT + tid), C - 1);
    segments_of<kPer>(soff, nseg, ci, sg);
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      const uint32_t i = c0 + (uint32_t)(u * kT + tid);
      e[u] = i < C ? __hip_atomic_load(row_pairs + (int64_t)sg[u] * span + (i - soff[sg[u]]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPer; u++) {
      const uint32_t i = c0 + (uint32_t)(u * kT + tid);
      if (i < C) {
        const uint32_t key = (uint32_t)e[u], blk = (uint32_t)(e[u] >> 32);
        const uint32_t bin = key >> kHistShift;
        if (bin > tb) set_bit(bitmap, blk);
        if (bin == tb) {
          atomicAdd(&hist1024[(key >> 10) & 1023u], 1u);
          const uint32_t t = atomicAdd(&ntie, 1u);
          if (t < (uint32_t)kFusedTies) {
            tkey[t] = key;
            tblk[t] = blk;
          }
        }
      }
    }
  }
  __syncthreads();
  // 3. the bin-tb candidates ranked: from the LDS list, or (more than
  //    kFusedTies of them) from memory, every candidate below bin tb read as
  //    key 0 (below every key of a bin tb > 0; none exist when tb = 0) and
  //    those above it (already set) possibly marked again
  const uint32_t nt = ntie;
  if (nt <= (uint32_t)kFusedTies) {
    // the sub-bin sb of key bits 19..10 that holds the last key taken: list
    // entries above it are taken; those inside it are ranked directly when
    // they do not all fit (few: one 1024th of the bin)
    if (tid == 0) found[0] = found[1] = found[2] = 0;
    __syncthreads();
    find_bin_1024_t<kT>(hist1024, need, tmp, found);
    const uint32_t sb = (tb << 10) | found[0], need2 = need - found[1];
    const bool all_in = found[2] == need2;
    uint32_t* sub = lhist;                            // list positions of the sub-bin's entries (<= nt)
    if (tid == 0) found[3] = 0;
    __syncthreads();
    for (uint32_t j = tid; j < nt; j += kT) {
      const uint32_t kp = tkey[j] >> 10;
      if (kp > sb || (all_in && kp == sb)) set_bit(bitmap, tblk[j]);
      else if (kp == sb) sub[atomicAdd(&found[3], 1u)] = j;
    }
    __syncthreads();
    if (!all_in) {
      const uint32_t ns = found[3];
      for (uint32_t i = tid; i < ns; i += kT) {
        const uint32_t ji = sub[i];
        const uint64_t vi = ((uint64_t)tkey[ji] << 32) | (0xFFFFFFFFu - tblk[ji]);
        uint32_t rank = 0;
#pragma unroll 8
        for (uint32_t q = 0; q < ns; q++) {
          const uint32_t jq = sub[q];
          const uint64_t vq = ((uint64_t)tkey[jq] << 32) | (0xFFFFFFFFu - tblk[jq]);
          rank += vq > vi ? 1u : 0u;
        }
        if (rank < need2) set_bit(bitmap, tblk[ji]);
      }
    }
    __syncthreads();
  } else {
    auto pair_at = [&](int i) -> uint64_t {
      int lo = 0, hi = nseg;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (soff[mid] <= (uint32_t)i) lo = mid; else hi = mid;
      }
      return __hip_atomic_load(row_pairs + (int64_t)lo * span + ((uint32_t)i - soff[lo]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    rank_bin_list<kT>((int)C, [&](int i) {
      const uint64_t v = pair_at(i);
      const uint32_t key = (uint32_t)v;
      return make_uint2((key >> kHistShift) < tb ? 0u : key, (uint32_t)(v >> 32));
    }, tb, need, hist1024, tmp, found, [&](int i) { set_bit(bitmap, (uint32_t)(pair_at(i) >> 32)); });
  }
  // 4. compaction: thread t counts the bits of words t * wq .. t * wq + wq - 1,
  //    a scan gives its first output position
  const int wq = (nwords32 + kT - 1) / kT;
  const int w0 = wq * tid;
  uint32_t cnt = 0;
  for (int w = w0; w < w0 + wq && w < nwords32; w++) cnt += (uint32_t)__popc(bitmap[w]);
  uint32_t tot;
  uint32_t pos = block_exclusive_scan<kT>(cnt, tmp, &tot);
  for (int w = w0; w < w0 + wq && w < nwords32; w++) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = w * 32 + b;
      pos++;
    }
  }
}

__device__ void fused_tail(const ScoreArgs& a, const SelectArgs& sel, int srow, int nv, uint32_t* lhist,
                           uint32_t* dyn, int wg_b0, int len, int64_t fin_bk, int64_t fin_e) {
  constexpr int kT = kFT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int span = a.fused_span;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;
  __shared__ int bnd;
  __shared__ uint32_t tmp[64], found[4];
  __shared__ uint32_t last;
  // 1. the bound from the workgroup's own keys
  if (wave == 0) {
    const int b = running_threshold(lhist, (uint32_t)a.k, 0);
    if (lane == 0) bnd = b;
  }
  __syncthreads();
  const int b_loc = bnd;
  // 2. its counts of the bins above it go to the row's histogram
  for (int i = tid; i < kHistBins; i += kT) {
    const uint32_t c = lhist[i];
    if (c && i > b_loc) atomicAdd(&gh[i], c);
  }
  // 3. a higher bound from the row's histogram as it stands (the flushes of
  //    the workgroups that are done), if it has one, from the kBoundWindow
  //    bins above b_loc (32 octaves of scores: in practice every key above
  //    it; keys beyond the window would only make the bound lower)
  if (wave == 0) {
    const int from = b_loc + 1;
    const int b = running_threshold<true>(gh, (uint32_t)a.k, from, (from & ~3) + kBoundWindow);
    if (lane == 0) bnd = max(b, b_loc);
  }
  __syncthreads();
  const uint32_t kmin = (uint32_t)(bnd + 1) << kHistShift;   // bnd <= 4094
  // 4. the keys above the bound, in block order: thread t takes the blocks
  //    t * per .. t * per + per - 1 of the workgroup
  const int nmine = min(span, nv - wg_b0);
  const int per = span / kT;                                  // <= 16
  constexpr int kMaxPer = kMaxFusedCpw * kScoreBlocksPerWG / kT;
  uint32_t ck[kMaxPer];
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; i++) {
    const int j = tid * per + i;
    const bool ok = i < per && j < nmine;
    ck[i] = ok ? dyn[j] : 0u;
    cnt += (ok && ck[i] >= kmin) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t o = block_exclusive_scan<kT>(cnt, tmp, &tot);
  uint64_t* seg = reinterpret_cast<uint64_t*>(a.keys) + (int64_t)srow * a.stride + wg_b0;
#pragma unroll
  for (int i = 0; i < kMaxPer; i++) {
    const int j = tid * per + i;
    if (i < per && j < nmine && ck[i] >= kmin) {
      __hip_atomic_store(seg + o, ((uint64_t)(uint32_t)(wg_b0 + j) << 32) | ck[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      o++;
    }
  }
  if (tid == 0)
    __hip_atomic_store(&a.cand_count[(int64_t)srow * gridDim.x + blockIdx.x], tot, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  // 5. arrival: this thread's stores and atomics have completed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ uint32_t arrival;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.row_done[srow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    arrival = old;
    last = old == gridDim.x - 1;
  }
  __syncthreads();
  // 6. append: task t < 8 finalises group t of the completed block (if any),
  //    task 8 copies the token into the ring (the indexer key, group 8, was
  //    finalised before it was scored); the workgroup that arrived j-th
  //    takes tasks 4 j .. 4 j + 3 (wavefront w: task 4 j + w), the row's last
  //    one, after its selection, also every task past that (rows of fewer
  //    than three workgroups).  Every task uses the length read at the start.
  const int brow = srow / a.n_q;
  auto task = [&](int t) {
    if (t == 8)
      ring_copy(a.ca, brow, 0, len, lane);
    else if (fin_bk >= 0)
      finalize_group(a.ca, brow, fin_bk, len, t, fin_e, nullptr, lane, nullptr);
  };
  if (!last) {
    if (a.append && 4 * (int)arrival + wave < 9) task(4 * (int)arrival + wave);
    return;
  }
  if (tid == 0) __hip_atomic_store(&a.row_done[srow], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  fused_select(a, sel, srow, nv, lhist, dyn, tmp, found);
  if (a.append) {
    // every workgroup of the row has read the old length
    if (tid == 0) a.ca.seq_len[brow] = len + 1;
    for (int t = 4 * (int)arrival + wave; t < 9; t += 4) task(t);
  }
}

IndexerPlan plan_indexer(const lca_layer* L, int n_q, int H_I, int k) {
  (void)k;
  IndexerPlan pl;
  const int64_t nvmax = L->len_max / L->ratio;   // visible blocks of the last query
  pl.stride = (nvmax + 63) & ~(int64_t)63;
  if (pl.stride < 64) pl.stride = 64;
  int64_t chunks = (nvmax + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG;
  if (chunks < 1) chunks = 1;
  // about kScoreTargetWGs workgroups in all, each with >= 1 chunk of one query
  const int64_t rows = (int64_t)L->batch * n_q;
  int64_t cpw = (rows * chunks + kScoreTargetWGs - 1) / kScoreTargetWGs;
  const int force_cpw = tuning(kTuneScoreCpw);
  if (force_cpw > 0) cpw = force_cpw;
  // paged: a workgroup's blocks span at most 64 pages (its wavefronts hold
  // one page-table entry per lane)
  const int64_t max_cpw = L->page_blocks > 0 ? (int64_t)L->page_blocks * 64 / kScoreBlocksPerWG : chunks;
  if (cpw > max_cpw) cpw = max_cpw;
  if (cpw < 1) cpw = 1;
  if (cpw > chunks) cpw = chunks;
  pl.cpw = (int)cpw;
  pl.chunks = (int)((chunks + cpw - 1) / cpw);
  // many queries per row: the tile kernel (key tiles shared by the queries)
  pl.tile = 0;
  pl.qgroups = 0;
  bool tile = n_q >= kTileMinQueries && H_I <= 32;
  if (tuning(kTuneScoreTile) >= 0) tile = tuning(kTuneScoreTile) != 0 && H_I <= 32;
  if (tile) {
    pl.tile = H_I <= 16 ? 8 : 4;
    pl.qgroups = (n_q + pl.tile * kTileSets - 1) / (pl.tile * kTileSets);
    int64_t tcpw = ((int64_t)L->batch * pl.qgroups * chunks + kTileTargetWGs - 1) / kTileTargetWGs;
    if (force_cpw > 0) tcpw = force_cpw;
    if (tcpw > max_cpw) tcpw = max_cpw;
    if (tcpw < 1) tcpw = 1;
    if (tcpw > chunks) tcpw = chunks;
    pl.cpw = (int)tcpw;
    pl.chunks = (int)((chunks + tcpw - 1) / tcpw);
  }
  // selection: parts of kPartKeys blocks on workgroups of their own when the
  // rows are long and too few to fill the chip
  bool sliced = pl.stride > kSliceMinBlocks && rows < kSliceMaxRows;
  const int force_sliced = tuning(kTuneTopkSliced);
  if (force_sliced >= 0) sliced = force_sliced != 0;
  // tile kernel: candidate lists instead of full key rows, unless a row has
  // too many lists (chunks x wavefronts) to gather
  pl.cand = pl.tile && pl.chunks * kTileWavesPerSet <= kMaxCandGroups;
  if (tuning(kTuneTopkCand) >= 0) pl.cand = pl.tile && tuning(kTuneTopkCand) != 0;
  if (pl.cand) sliced = false;
  // decode (one query per score workgroup, H <= 16): the selection runs in
  // the scoring launch from per-workgroup candidates, unless the sliced or
  // separate selection is asked for
  pl.fused = !pl.tile && H_I <= 16 && force_sliced != 1;
  if (tuning(kTuneTopkFused) >= 0) pl.fused = pl.fused && tuning(kTuneTopkFused) != 0;
  pl.fused_wgs = pl.fused_span = 0;
  pl.fused_lds = 0;
  if (pl.fused) {
    sliced = false;
    int64_t fc = pl.cpw;                             // chunks per workgroup
    const int64_t min_fc = (chunks + kMaxFusedSegs - 1) / kMaxFusedSegs;
    if (fc < min_fc) fc = min_fc;
    if (fc > kMaxFusedCpw) fc = kMaxFusedCpw;        // chunks <= 512: min_fc <= 2
    pl.cpw = (int)fc;
    pl.fused_wgs = (int)((chunks + fc - 1) / fc);
    pl.fused_span = (int)(fc * kScoreBlocksPerWG);
    // dynamic LDS: the workgroup's keys; then, in the selecting workgroup,
    // the row's bitmap, the bin-tb list and a 1024-bin histogram
    size_t words = (size_t)pl.fused_span;
    const size_t sel_words = (size_t)((pl.stride + 31) / 32) + 2 * kFusedTies + 1024;
    if (words < sel_words) words = sel_words;
    pl.fused_lds = 4 * words;
  }
  pl.cand_waves = kTileWavesPerSet;
  pl.cand_lists = pl.cand ? pl.chunks * kTileWavesPerSet * 32 : 0;
  pl.cand_span = pl.cpw * kScoreBlocksPerWG;
  pl.slices = sliced ? (int)((pl.stride + kPartKeys - 1) / kPartKeys) : 0;
  // workspace layout
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  pl.off_done = o;
  o += up(pl.fused ? (size_t)rows * sizeof(uint32_t) : 0);
  pl.off_hist = o;
  o += (size_t)rows * kHistBins * sizeof(uint32_t);
  pl.zero_bytes = o;
  pl.off_keys = o;
  o += up((size_t)rows * pl.stride * ((pl.cand || pl.fused) ? 8 : 4));   // keys, or (key, x) pairs
  pl.off_part_count = o;
  o += up((size_t)rows * pl.slices * sizeof(uint32_t));
  pl.off_part_bits = o;
  o += (size_t)rows * pl.slices * kSelThreads * sizeof(uint32_t);
  pl.off_part_cand = o;
  o += (size_t)rows * pl.slices * 2 * kCandCap * sizeof(uint32_t);
  pl.off_cand_count = o;
  if (pl.cand) o += up((size_t)rows * pl.chunks * kTileWavesPerSet * 32 * sizeof(uint32_t));
  if (pl.fused) o += up((size_t)rows * pl.fused_wgs * sizeof(uint32_t));
  pl.total_bytes = o;
  return pl;
}

// The decode scoring launch (one query per row), contiguous or paged planes.
template <bool kPaged>
static void launch_score(const IndexerPlan& pl, const ScoreArgs& s, const SelectArgs& sa, int H_I, int rows,
                         hipStream_t stream) {
  if (pl.fused) {   // the selection runs in the same launch
    const dim3 g(pl.fused_wgs, rows), b(kFT);
    if (H_I <= 8)
      hipLaunchKernelGGL((indexer_score_kernel<true, 8, kPaged>), g, b, pl.fused_lds, stream, s, sa);
    else
      hipLaunchKernelGGL((indexer_score_kernel<true, 16, kPaged>), g, b, pl.fused_lds, stream, s, sa);
  } else {
    const dim3 g(pl.chunks, rows), b(256);
    if (H_I <= 8)
      hipLaunchKernelGGL((indexer_score_kernel<false, 8, kPaged>), g, b, 0, stream, s, sa);
    else if (H_I <= 16)
      hipLaunchKernelGGL((indexer_score_kernel<false, 16, kPaged>), g, b, 0, stream, s, sa);
    else
      hipLaunchKernelGGL((indexer_score_kernel<false, 32, kPaged>), g, b, 0, stream, s, sa);
  }
}

int launch_indexer(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                   int32_t* topk, void* ws, const IndexerPlan& pl, hipStream_t stream, const CompressArgs* append) {
  const int rows = L->batch * n_q;
  char* base = static_cast<char*>(ws);
  ScoreArgs s;
  s.n_q = n_q;
  s.H = H_I;
  s.m = L->ratio;
  s.max_blocks = L->max_blocks;
  s.pm = page_map_of<PageMap>(L);
  s.stride = pl.stride;
  s.seq_len = L->seq_len;
  s.idx_code = L->idx_code;
  s.idx_scale = L->idx_scale;
  s.iq = iq;
  s.iw = iw;
  s.hist = reinterpret_cast<uint32_t*>(base + pl.off_hist);
  s.cpw = pl.cpw;
  s.keys = reinterpret_cast<uint32_t*>(base + pl.off_keys);
  s.k = k;
  s.cand_count = (pl.cand || pl.fused) ? reinterpret_cast<uint32_t*>(base + pl.off_cand_count) : nullptr;
  s.row_done = pl.fused ? reinterpret_cast<uint32_t*>(base + pl.off_done) : nullptr;
  s.fused_span = pl.fused_span;
  s.append = append != nullptr;
  s.ca = append ? *append : CompressArgs{};
  s.status = L->sync + 1;
  SelectArgs sa;
  sa.n_q = n_q;
  sa.m = L->ratio;
  sa.k = k;
  sa.stride = pl.stride;
  sa.seq_len = L->seq_len;
  sa.keys = s.keys;
  sa.hist = s.hist;
  sa.topk = topk;
  sa.status = s.status;
  sa.slices = pl.slices;
  sa.part_count = reinterpret_cast<uint32_t*>(base + pl.off_part_count);
  sa.part_bits = reinterpret_cast<uint32_t*>(base + pl.off_part_bits);
  sa.part_cand = reinterpret_cast<uint32_t*>(base + pl.off_part_cand);
  sa.cand_count = s.cand_count;
  sa.segs = pl.cand_lists / 32;
  sa.span = pl.cand_span;
  {
    TimedLaunch t(kKernelIndexerScore, stream);
    const dim3 tg(pl.chunks, pl.qgroups, L->batch), tb(64 * kTileWaves);
    if (pl.tile == 8 && pl.cand)
      hipLaunchKernelGGL((indexer_score_tile_kernel<8, true>), tg, tb, 0, stream, s);
    else if (pl.tile == 8)
      hipLaunchKernelGGL((indexer_score_tile_kernel<8, false>), tg, tb, 0, stream, s);
    else if (pl.tile == 4 && pl.cand)
      hipLaunchKernelGGL((indexer_score_tile_kernel<4, true>), tg, tb, 0, stream, s);
    else if (pl.tile == 4)
      hipLaunchKernelGGL((indexer_score_tile_kernel<4, false>), tg, tb, 0, stream, s);
    else if (s.pm.shift >= 0)
      launch_score<true>(pl, s, sa, H_I, rows, stream);
    else
      launch_score<false>(pl, s, sa, H_I, rows, stream);
    int rc = t.done();
    if (rc || pl.fused) return rc;
  }
  // one timed interval covers the selection's one or two launches
  TimedLaunch t(kKernelTopkSelect, stream);
  if (pl.cand) {
    const size_t bitmap_bytes = (size_t)((pl.stride + 31) / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_cand_kernel, dim3(rows), dim3(kSelThreads), bitmap_bytes, stream, sa);
  } else if (pl.slices) {
    hipLaunchKernelGGL(topk_slice_kernel, dim3(pl.slices, rows), dim3(kSelThreads), 0, stream, sa);
    hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(kSelThreads), 0, stream, sa);
  } else {
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelThreads), 0, stream, sa);
  }
  return t.done();
}

int launch_decode_append(const lca_layer* L, const lca_layer* after, const uint16_t* kv, const float* gate,
                         const float* ikey, const float* igate, const float* iq, const float* iw, int H_I,
                         int k, int32_t* topk, void* ws, const IndexerPlan& pl, hipStream_t stream) {
  if (pl.fused && L->has_indexer && L->ratio <= 8) {
    const CompressArgs ca = compress_args(L, kv, gate, ikey, igate, 1);
    return launch_indexer(after, iq, iw, 1, H_I, k, topk, ws, pl, stream, &ca);
  }
  const int rc = launch_compress(L, kv, gate, ikey, igate, 1, stream);
  if (rc) return rc;
  return launch_indexer(after, iq, iw, 1, H_I, k, topk, ws, pl, stream);
}

}  // namespace lca
