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
//   score  = +0, then score = fma(w_h, max(dot_h, 0), score) for h ascending;
//   a zero score is +0.  The selection is bitwise reproducible.
//
// Matrix-core mapping (v_mfma_scale_f32_32x32x64_f8f6f4, both operands e2m1):
// the 32 A rows are (head, half) pairs -- a row carries one head's 32 codes of
// one MX half and zeros in the other half -- and the 32 B columns are 32
// consecutive blocks.  With the 32x32 output layout (lane l holds column l%32
// and rows 8i + 4*(l/32) + j), rows are placed so that lane l < 32 receives
// heads 0..7 and lane l >= 32 heads 8..15 of block l%32, each as its two
// per-half partial dot products.  The hardware applies the E8M0 scales of the
// query half (A) and of the key half (B).  A per-half partial is a sum of 32
// products on one power-of-two grid, below 2^11 grid steps, so it is exact;
// one fp32 add of the two halves then rounds the exact dot once.  Blocks whose
// scaled partials could leave the fp32 normal range take an unscaled MFMA and
// apply the scales in fp32 (double for the far ranges), with the same result.
// The head chain runs on the low lanes for heads 0..7, hops to the high lanes
// for heads 8..15, and hops back for the next group of 16 heads.
//
// While scoring, each workgroup histograms the top 12 bits of its order keys
// and adds them to a per-query histogram; the selection reads that histogram
// to find the bin that holds the k-th key, so it needs a single pass over the
// keys plus an exact ranking of the few keys inside that bin.
#include "lca_device.h"
#include "lca_internal.h"

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

struct ScoreArgs {
  int n_q, H, m;
  int64_t max_blocks, stride;
  const int32_t* seq_len;
  const uint8_t* idx_code;
  const uint8_t* idx_scale;
  const float* iq;
  const float* iw;
  uint32_t* keys;
  uint32_t* hist;        // [rows][kHistBins], zero on entry
  int cpw;               // chunks of 1024 blocks per workgroup
};

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

// Score of the lane's block when some exponent sum is out of the range where
// the scaled partials are exact fp32 normals: unscaled MFMA, scales in fp32
// (double beyond that range).  Rare; kept out of line.
__device__ __noinline__ float score_unscaled(v8i A0, v8i A1, v8i Bm, int hgroups, int H, int kh,
                                             const int (*q_exp)[2], const float* q_w, int ke0, int ke1) {
  const v16f zero16 = {};
  float total = 0.0f;
  for (int hg = 0; hg < hgroups; hg++) {
    const v16f acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(hg ? A1 : A0, Bm, zero16, 4, 4, 0,
                                                                     127, 0, 127);
    float part = 0.0f;
#pragma unroll
    for (int hl = 0; hl < 8; hl++) {
      const int h = 16 * hg + 8 * kh + hl;
      const bool hv = h < H;
      const float rl = fmaxf(exact_pair(acc[2 * hl], (hv ? q_exp[h][0] : 0) + ke0, acc[2 * hl + 1],
                                        (hv ? q_exp[h][1] : 0) + ke1), 0.0f);
      part = __builtin_fmaf(hv ? q_w[h] : 0.0f, rl, part);
    }
    const float upper = __shfl_xor(part, 32, kWave);
    total = (hg == 0) ? part : __fadd_rn(total, part);
    total = __fadd_rn(total, upper);
  }
  return total;
}

__global__ void __launch_bounds__(256) indexer_score_kernel(ScoreArgs a) {
  const int srow = blockIdx.y;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  // This workgroup's chunks of 1024 blocks are [c0, c0 + cpw).  The key loads
  // are issued before the row length arrives: any block below the key row
  // capacity is readable, and blocks past the visible count are masked later.
  const int64_t c0 = (int64_t)blockIdx.x * a.cpw;
  const int64_t cap = a.stride < a.max_blocks ? a.stride : a.max_blocks;

  __shared__ __attribute__((aligned(16))) uint8_t q_code[32][32];
  __shared__ int q_exp[32][2];
  __shared__ float q_w[32];
  __shared__ uint32_t lhist[kHistBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, kh = lane >> 5;

  const uint8_t* kc = a.idx_code + (int64_t)brow * a.max_blocks * 32;
  const uint8_t* ks = a.idx_scale + (int64_t)brow * a.max_blocks * 2;
  // The wave walks iterations i = 0 .. n_it-1 of 32 blocks each: iteration i
  // is group i % 8 of this wave's 256 blocks in chunk c0 + i / 8.  Keys are
  // loaded kDepth iterations ahead of their use.
  const int n_it = a.cpw * kScoreItersPerWave;
  auto blk_of = [&](int i) -> int64_t {
    return (c0 + i / kScoreItersPerWave) * kScoreBlocksPerWG +
           (int64_t)wave * (kScoreItersPerWave * kScoreBlocksPerIter) +
           (i % kScoreItersPerWave) * kScoreBlocksPerIter + r;
  };
  // Loads are unconditional (a block past the capacity reads block 0) so that
  // no load waits on another; compute() masks what they return.
  auto load = [&](int i, int4& kr, uint32_t& er) {
    const int64_t blk = blk_of(i);
    const int64_t b = (i < n_it && blk < cap) ? blk : 0;
    kr = *reinterpret_cast<const int4*>(kc + b * 32 + 16 * kh);
    er = *reinterpret_cast<const uint16_t*>(ks + b * 2);
  };
  // query values and weights: all loads in flight before any is used
  const float* qsrc = a.iq + (int64_t)srow * a.H * kIdx;
  float qv[8];
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int e = tid + 256 * u;
    qv[u] = e < a.H * kIdx ? qsrc[e] : 0.0f;
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
  const int p = *(const_i32p)(a.seq_len + brow) - a.n_q + qi;
  int64_t nv = (int64_t)(p + 1) / a.m;
  if (nv > cap) nv = cap;                      // defensive: never past the key row

  for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0;
  // MXFP4 quantisation of the query, one 32-lane half-wave per MX block.
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const int e = tid + 256 * u;
    if (e >= a.H * kIdx) break;
    const float x = qv[u];
    float amax = half_wave_max(fabsf(x));
    uint32_t code = 0;
    int X = -127;
    if (amax > 0.0f) {
      X = floor_log2(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      code = f32_e2m1(ldexpf(x, -X));
    }
    uint32_t hi = __shfl_xor(code, 1, kWave);
    const int h = e >> 6, el = e & 63;
    if ((el & 1) == 0) q_code[h][el >> 1] = (uint8_t)(code | (hi << 4));
    if ((el & 31) == 0) q_exp[h][el >> 5] = X;
  }
  if (tid < a.H) q_w[tid] = wq;
  __syncthreads();

  // A operands and their E8M0 scales: lane l feeds row l%32 with K-half l/32.
  const int hgroups = (a.H + 15) >> 4;
  v8i A[2];
  int sa[2];
  int qmin = 1 << 20, qmax = -(1 << 20);
#pragma unroll
  for (int hg = 0; hg < 2; hg++) {
    A[hg] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    sa[hg] = 127;
    const int G = (r & 7) >> 2, v = 4 * (r >> 3) + (r & 3);
    const int h = 16 * hg + 8 * G + (v >> 1), half = v & 1;
    if (hg < hgroups && half == kh && h < a.H) {
      const int* src = reinterpret_cast<const int*>(&q_code[h][16 * kh]);
      A[hg][0] = src[0];
      A[hg][1] = src[1];
      A[hg][2] = src[2];
      A[hg][3] = src[3];
      sa[hg] = q_exp[h][kh] + 127;
    }
  }
  // Per-lane epilogue constants for the 8 heads of this lane's set (octet
  // 2*hg + kh); heads past H get weight 0, which leaves the chain unchanged.
  float wv[2][8];
#pragma unroll
  for (int hg = 0; hg < 2; hg++)
#pragma unroll
    for (int hl = 0; hl < 8; hl++) {
      const int h = 16 * hg + 8 * kh + hl;
      wv[hg][hl] = h < a.H ? q_w[h] : 0.0f;
    }
  {
    // extremes of the query's 2H block exponents: lane l looks at entry l
    const int e = lane < 2 * a.H ? q_exp[lane >> 1][lane & 1] : 0;
    int lo = lane < 2 * a.H ? e : (1 << 20), hi = lane < 2 * a.H ? e : -(1 << 20);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      lo = min(lo, __shfl_xor(lo, o, kWave));
      hi = max(hi, __shfl_xor(hi, o, kWave));
    }
    qmin = lo;
    qmax = hi;
  }

  uint32_t* out = a.keys + (int64_t)srow * a.stride;
  const v16f zero16 = {};

  // kDepth iterations at once: their matrix-core products and head chains are
  // independent, so they interleave; one range check covers the block.
  auto compute = [&](int i0, const int4 (&kr)[kDepth], const uint32_t (&er_in)[kDepth]) {
    int ke0[kDepth], ke1[kDepth], sb[kDepth];
    uint32_t er[kDepth];
    bool ok = true;
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      // a block that is not scored takes unit scales (its result is dropped)
      er[u] = blk_of(i0 + u) < nv ? er_in[u] : 0x7F7Fu;
      ke0[u] = (int)(er[u] & 0xFF) - 127;
      ke1[u] = (int)(er[u] >> 8) - 127;
      sb[u] = kh ? (ke1[u] + 127) : (ke0[u] + 127);
      // scaled partials stay normal fp32 when every exponent sum is in range
      ok = ok && (qmin + min(ke0[u], ke1[u]) >= -124) && (qmax + max(ke0[u], ke1[u]) <= 116);
    }
    float total[kDepth];
    if (__all(ok)) {
#pragma unroll
      for (int hg = 0; hg < 2; hg++) {
        if (hg < hgroups) {
          v16f acc[kDepth];
#pragma unroll
          for (int u = 0; u < kDepth; u++) {
            const v8i Bm = (v8i){kr[u].x, kr[u].y, kr[u].z, kr[u].w, 0, 0, 0, 0};
            acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[hg], Bm, zero16, 4, 4, 0, sa[hg],
                                                                     0, sb[u]);
          }
          // both lane sets fold their octet at once; the low set adds the octets
          float part[kDepth], upper[kDepth];
#pragma unroll
          for (int u = 0; u < kDepth; u++) {
            part[u] = 0.0f;
#pragma unroll
            for (int hl = 0; hl < 8; hl++)
              part[u] = __builtin_fmaf(wv[hg][hl],
                                       fmaxf(__fadd_rn(acc[u][2 * hl], acc[u][2 * hl + 1]), 0.0f), part[u]);
          }
#pragma unroll
          for (int u = 0; u < kDepth; u++) upper[u] = __shfl_xor(part[u], 32, kWave);
#pragma unroll
          for (int u = 0; u < kDepth; u++) {
            total[u] = (hg == 0) ? part[u] : __fadd_rn(total[u], part[u]);
            total[u] = __fadd_rn(total[u], upper[u]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kDepth; u++) {
        const v8i Bm = (v8i){kr[u].x, kr[u].y, kr[u].z, kr[u].w, 0, 0, 0, 0};
        total[u] = score_unscaled(A[0], A[1], Bm, hgroups, a.H, kh, q_exp, q_w, ke0[u], ke1[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      const int64_t blk = blk_of(i0 + u);
      if (kh == 0 && i0 + u < n_it && blk < nv) {
        const uint32_t key = ord_key(__fadd_rn(total[u], 0.0f));   // -0 -> +0
        out[blk] = key;
        atomicAdd(&lhist[key >> kHistShift], 1u);
      }
    }
  };

#pragma unroll 1
  for (int i0 = 0; i0 < n_it; i0 += 2 * kDepth) {
    compute(i0, kA, eA);
#pragma unroll
    for (int u = 0; u < kDepth; u++) load(i0 + 2 * kDepth + u, kA[u], eA[u]);
    compute(i0 + kDepth, kB, eB);
#pragma unroll
    for (int u = 0; u < kDepth; u++) load(i0 + 3 * kDepth + u, kB[u], eB[u]);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// ---------------------------------------------------------------------------
// Exact top-k by (score desc, block asc) for one query per workgroup of 512
// threads.  In every round of 32768 blocks, thread t owns the two bitmap
// words of blocks 64t .. 64t+63 of the round.
//   1. The query's histogram of the top 12 key bits (built while scoring)
//      gives the bin tb holding the k-th largest key and the count `above` of
//      keys in higher bins; the histogram is zeroed for the next call.
//   2. Each thread compares its 32 keys with tb: keys above tb set their bit,
//      keys inside tb are listed in LDS in block order (a block-wide scan
//      places every thread's keys).
//   3. Two radix passes of 10 bits over the listed keys give the exact
//      threshold key T and how many keys equal to T are taken; listed keys
//      above T set their bit, and keys equal to T are ranked by block index
//      with a scan over the list, which is in block order.
//   4. The bitmap is compacted into ascending block indices.
// If more than kCandCap keys share tb (many nearly equal scores), a radix
// select over all keys replaces steps 2-3.
// ---------------------------------------------------------------------------

struct SelectArgs {
  int n_q, m, k;
  int64_t stride;
  const int32_t* seq_len;
  const uint32_t* keys;
  uint32_t* hist;
  int32_t* topk;
};

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRoundKeys = 64 * kSelThreads;   // blocks per round
constexpr int kCandCap = 4096;
constexpr int kMaxWords = 8192;   // bitmap words of 64 blocks: 524288 blocks
static_assert(2 * kCandCap >= kMaxWords, "the candidate list doubles as per-word counters");

// exclusive prefix sum over the kSelThreads threads; returns the block total
// in *total (tmp >= 32 words)
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t before_wave = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; w++) {
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
template <typename F>
__device__ __forceinline__ void for_each_word(const uint32_t* keys, int nv, int nwords, F f, int w_start = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kBatch = 8;
#pragma unroll 1
  for (int wb = w_start + wave; wb < nwords; wb += kBatch * (kSelThreads / 64)) {
    uint32_t kk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int j = (wb + u * (kSelThreads / 64)) * 64 + lane;
      kk[u] = keys[j < nv ? j : 0];      // past the count: ignored by f (j >= nv)
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

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(SelectArgs a) {
  const int srow = blockIdx.x;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  const int k = a.k, tid = threadIdx.x, lane = tid & 63;
  int32_t* out = a.topk + (int64_t)srow * k;
  const uint32_t* keys = a.keys + (int64_t)srow * a.stride;
  uint32_t* gh = a.hist + (int64_t)srow * kHistBins;

  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[4];
  __shared__ uint32_t cand[2 * kCandCap];      // listed keys, then their blocks (block order)
  __shared__ uint32_t bitmap[2 * kMaxWords];   // bit j of word w: block 32 w + j

  // The histogram loads go out first, then round 0's keys, so that the
  // histogram phase does not wait for the keys (loads complete in issue
  // order).  Key loads are unconditional: a block past the count reads block
  // 0 of the row and is masked at use.
  // Nothing here waits for the row length: the loads are addressed within
  // the key row (a round past its end reads the row's last 64 keys), and
  // the length comes through the scalar cache after they are issued.
  const uint4 hv0 = reinterpret_cast<const uint4*>(gh)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(gh)[2 * tid + 1];
  uint4 kv[16];
  auto load_round = [&](int r) {
    int b0 = r * kRoundKeys + 64 * tid;
    b0 = b0 + 64 <= a.stride ? b0 : (int)a.stride - 64;
    const uint4* src = reinterpret_cast<const uint4*>(keys + b0);
#pragma unroll
    for (int v = 0; v < 16; v++) kv[v] = src[v];
  };
  load_round(0);
  typedef const int32_t __attribute__((address_space(4)))* const_i32p;
  const int p = *(const_i32p)(a.seq_len + brow) - a.n_q + qi;
  int nv = (p + 1) / a.m;
  if (nv > a.stride) nv = (int)a.stride;       // defensive: never past the key row
  const int rounds = (nv + kRoundKeys - 1) / kRoundKeys;
  if (tid == 0) found[0] = found[1] = found[2] = found[3] = 0;
  // 1. threshold bin tb from the histogram (thread t holds bins 8t .. 8t+7)
  {
    const uint32_t c8 = hv0.x + hv0.y + hv0.z + hv0.w + hv1.x + hv1.y + hv1.z + hv1.w;
    uint32_t total;
    const uint32_t below = block_exclusive_scan(c8, tmp, &total);
    reinterpret_cast<uint4*>(gh)[2 * tid] = make_uint4(0, 0, 0, 0);   // for the next call
    reinterpret_cast<uint4*>(gh)[2 * tid + 1] = make_uint4(0, 0, 0, 0);
    // walk the eight bins from the top (branch-free: at most one hits)
    const uint32_t cs[8] = {hv1.w, hv1.z, hv1.y, hv1.x, hv0.w, hv0.z, hv0.y, hv0.x};
    const uint32_t ku = (uint32_t)k;
    uint32_t run = total - below - c8;          // keys in bins above this thread's eight
    uint32_t hit = 0, hbin = 0, hrun = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t h = (run < ku) & (run + cs[i] >= ku);
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
  if (nv <= k) {
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
    return;
  }
  __syncthreads();
  const uint32_t tb = found[0], above = found[1];
  const int nwords32 = (nv + 31) >> 5;

  // 2. bits above tb, keys inside tb listed in block order
  uint32_t nc = 0;
  for (int r = 0; r < rounds; r++) {
    if (r) load_round(r);
    const int b0 = r * kRoundKeys + 64 * tid;
    const int lim = nv - b0;                    // keys of this thread below the count
    // bits by plain integer arithmetic (no per-key lane masks): for bins in
    // [0, 4096), tb - bin < 0 iff bin > tb, and (bin ^ tb) - 1 wraps iff equal
    uint32_t gt[2] = {0u, 0u}, eq[2] = {0u, 0u};
#pragma unroll
    for (int v = 0; v < 16; v++) {
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
    const uint32_t m0 = lim >= 32 ? 0xFFFFFFFFu : (lim <= 0 ? 0u : (1u << lim) - 1u);
    const uint32_t m1 = lim >= 64 ? 0xFFFFFFFFu : (lim <= 32 ? 0u : (1u << (lim - 32)) - 1u);
    gt[0] &= m0;
    gt[1] &= m1;
    eq[0] &= m0;
    eq[1] &= m1;
    const uint32_t cnt = (uint32_t)(__popc(eq[0]) + __popc(eq[1]));
    if (lim > 0) bitmap[2 * (r * kSelThreads + tid)] = gt[0];
    if (lim > 32) bitmap[2 * (r * kSelThreads + tid) + 1] = gt[1];
    uint32_t tot;
    uint32_t pos = nc + block_exclusive_scan(cnt, tmp, &tot);
    if (nc + tot <= (uint32_t)kCandCap && cnt) {
      // the few listed keys, in block order
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const uint32_t q[4] = {kv[v].x, kv[v].y, kv[v].z, kv[v].w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = 4 * v + i;
          if ((eq[e >> 5] >> (e & 31)) & 1u) {
            cand[pos] = q[i];
            cand[kCandCap + pos] = (uint32_t)(b0 + e);
            pos++;
          }
        }
      }
    }
    nc += tot;
  }

  if (nc <= (uint32_t)kCandCap) {
    // 3. exact threshold among the listed keys: bits 19..10, then 9..0.  A
    // pass whose bin holds exactly the keys still needed ends the search:
    // every listed key at or above that bin is taken.
    uint32_t need = (uint32_t)k - above;
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
  } else {
    const int nwords = (nv + 63) >> 6;
    // Many keys share 24 high bits: radix select over every key (12 + 12 + 8
    // bits), then every key above T and the lowest-index keys equal to T.
    uint32_t pfx = 0, need = (uint32_t)k;
#pragma unroll
    for (int d = 0; d < 3; d++) {
      const int shift = d == 0 ? 20 : (d == 1 ? 8 : 0), width = d == 2 ? 8 : 12;
      const uint32_t nb = 1u << width, mask = nb - 1;
      for (uint32_t j = tid; j < nb; j += kSelThreads) hist[j] = 0;
      __syncthreads();
      for_each_word(keys, nv, nwords, [&](int w, int j, uint32_t key) {
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
    // equal keys per 64-block word (cand_key doubles as the count array)
    uint32_t* eqc = cand;       // 2 * kCandCap = kMaxWords counters
    for_each_word(keys, nv, nwords, [&](int w, int j, uint32_t key) {
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
    for_each_word(keys, nv, nwords, [&](int w, int j, uint32_t key) {
      const bool eq = j < nv && key == T;
      const uint64_t em = __ballot(eq);
      const uint32_t rank = eqc[w] + (uint32_t)__popcll(em & ((1ull << lane) - 1ull));
      if (eq && rank < need_eq) set_bit(bitmap, (uint32_t)j);
    });
    __syncthreads();
  }

  // 4. compaction: ascending block order, thread t owns a run of 32-bit words
  const int wper = (nwords32 + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * wper, w1 = min(nwords32, w0 + wper);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; w++) cnt += __popc(bitmap[w]);
  uint32_t tot;
  uint32_t pos = block_exclusive_scan(cnt, tmp, &tot);
  for (int w = w0; w < w1; w++) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = w * 32 + b;
      pos++;
    }
  }
}

IndexerPlan plan_indexer(const lca_layer* L, int n_q, int H_I, int k) {
  (void)H_I;
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
  const char* env = getenv("LCA_SCORE_CPW");
  if (env && *env) cpw = atoi(env);
  if (cpw < 1) cpw = 1;
  if (cpw > chunks) cpw = chunks;
  pl.cpw = (int)cpw;
  pl.chunks = (int)((chunks + cpw - 1) / cpw);
  pl.keys_bytes = (size_t)L->batch * n_q * pl.stride * sizeof(uint32_t);
  pl.hist_bytes = (size_t)L->batch * n_q * kHistBins * sizeof(uint32_t);
  return pl;
}

int launch_indexer(const lca_layer* L, const float* iq, const float* iw, int n_q, int H_I, int k,
                   int32_t* topk, void* ws, const IndexerPlan& pl, hipStream_t stream) {
  const int rows = L->batch * n_q;
  ScoreArgs s;
  s.n_q = n_q;
  s.H = H_I;
  s.m = L->ratio;
  s.max_blocks = L->max_blocks;
  s.stride = pl.stride;
  s.seq_len = L->seq_len;
  s.idx_code = L->idx_code;
  s.idx_scale = L->idx_scale;
  s.iq = iq;
  s.iw = iw;
  s.hist = static_cast<uint32_t*>(ws);
  s.cpw = pl.cpw;
  s.keys = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + pl.hist_bytes);
  {
    TimedLaunch t(kKernelIndexerScore, stream);
    hipLaunchKernelGGL(indexer_score_kernel, dim3(pl.chunks, rows), dim3(256), 0, stream, s);
    int rc = t.done();
    if (rc) return rc;
  }
  SelectArgs sa;
  sa.n_q = n_q;
  sa.m = L->ratio;
  sa.k = k;
  sa.stride = pl.stride;
  sa.seq_len = L->seq_len;
  sa.keys = s.keys;
  sa.hist = s.hist;
  sa.topk = topk;
  TimedLaunch t(kKernelTopkSelect, stream);
  hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelThreads), 0, stream, sa);
  return t.done();
}

}  // namespace lca
