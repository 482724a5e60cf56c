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
// Matrix-core mapping (v_mfma_scale_f32_32x32x64_f8f6f4, both operands e2m1,
// unit scales): the 32 A rows are (head, half) pairs -- a row carries one
// head's 32 codes of one MX half and zeros in the other half -- and the 32 B
// columns are 32 consecutive blocks.  With the 32x32 output layout (lane l
// holds column l%32 and rows 8i + 4*(l/32) + j), rows are placed so that lane
// l < 32 receives heads 0..7 and lane l >= 32 heads 8..15 of block l%32, each
// as its two per-half partial sums.  A per-half partial sum is a sum of 32
// products on a 1/4 grid below 2^11, so it is exact in fp32 in any order; the
// scales are then applied in fp32 as exact powers of two and the two halves
// added by one fused multiply-add, which rounds the exact dot once.  The head
// chain runs on the low lanes for heads 0..7, hops to the high lanes for
// heads 8..15, and hops back for the next group of 16 heads.
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kScoreBlocksPerIter = 32;
constexpr int kScoreItersPerWave = 8;
constexpr int kScoreBlocksPerWG = 4 * kScoreItersPerWave * kScoreBlocksPerIter;  // 1024

struct ScoreArgs {
  int n_q, H, m;
  int64_t max_blocks, stride;
  const int32_t* seq_len;
  const uint8_t* idx_code;
  const uint8_t* idx_scale;
  const float* iq;
  const float* iw;
  uint32_t* keys;
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

__global__ void __launch_bounds__(256) indexer_score_kernel(ScoreArgs a) {
  const int srow = blockIdx.y;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  const int p = a.seq_len[brow] - a.n_q + qi;
  int64_t nv = (int64_t)(p + 1) / a.m;
  if (nv > a.stride) nv = a.stride;            // defensive: never past the key row
  if (nv > a.max_blocks) nv = a.max_blocks;
  const int64_t base = (int64_t)blockIdx.x * kScoreBlocksPerWG;
  if (base >= nv) return;

  __shared__ __attribute__((aligned(16))) uint8_t q_code[32][32];
  __shared__ int q_exp[32][2];
  __shared__ float q_w[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // MXFP4 quantisation of the query, one 32-lane half-wave per MX block.
  const float* qsrc = a.iq + (int64_t)srow * a.H * kIdx;
  for (int e = tid; e < a.H * kIdx; e += 256) {
    float x = qsrc[e];
    float amax = half_wave_max(fabsf(x));
    uint32_t code = 0;
    int X = 0;
    if (amax > 0.0f) {
      X = floor_log2(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      code = f32_e2m1(ldexpf(x, -X));
    } else {
      X = -127;
    }
    uint32_t hi = __shfl_xor(code, 1, kWave);
    const int h = e >> 6, el = e & 63;
    if ((el & 1) == 0) q_code[h][el >> 1] = (uint8_t)(code | (hi << 4));
    if ((el & 31) == 0) q_exp[h][el >> 5] = X;
  }
  if (tid < a.H) q_w[tid] = a.iw[(int64_t)srow * a.H + tid];
  __syncthreads();

  // A operands: lane l feeds row l%32 with the K-half l/32.
  const int r = lane & 31, kh = lane >> 5;
  const int hgroups = (a.H + 15) >> 4;
  v8i A[2];
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
  // Per-lane epilogue constants for the 8 heads of this lane's set.
  int qe0[2][8], qe1[2][8];
  float wv[2][8];
  bool hv[2][8];
#pragma unroll
  for (int hg = 0; hg < 2; hg++)
#pragma unroll
    for (int hl = 0; hl < 8; hl++) {
      const int h = 16 * hg + 8 * kh + hl;
      hv[hg][hl] = h < a.H;
      qe0[hg][hl] = h < a.H ? q_exp[h][0] : 0;
      qe1[hg][hl] = h < a.H ? q_exp[h][1] : 0;
      wv[hg][hl] = h < a.H ? q_w[h] : 0.0f;
    }

  const uint8_t* kc = a.idx_code + (int64_t)brow * a.max_blocks * 32;
  const uint8_t* ks = a.idx_scale + (int64_t)brow * a.max_blocks * 2;
  uint32_t* out = a.keys + (int64_t)srow * a.stride;
  const v16f zero16 = {};

  for (int it = 0; it < kScoreItersPerWave; it++) {
    const int64_t blk0 = base + (int64_t)wave * (kScoreItersPerWave * kScoreBlocksPerIter) +
                         (int64_t)it * kScoreBlocksPerIter;
    if (blk0 >= nv) break;
    const int64_t blk = blk0 + r;
    const bool valid = blk < nv;
    v8i Bm = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    int ke0 = 0, ke1 = 0;
    if (valid) {
      const int4 kv4 = *reinterpret_cast<const int4*>(kc + blk * 32 + 16 * kh);
      Bm[0] = kv4.x;
      Bm[1] = kv4.y;
      Bm[2] = kv4.z;
      Bm[3] = kv4.w;
      const uint16_t e2 = *reinterpret_cast<const uint16_t*>(ks + blk * 2);
      ke0 = (int)(e2 & 0xFF) - 127;
      ke1 = (int)(e2 >> 8) - 127;
    }
    float part = 0.0f;
#pragma unroll
    for (int hg = 0; hg < 2; hg++) {
      if (hg < hgroups) {
        v16f acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[hg], Bm, zero16, 4, 4, 0, 127,
                                                                   0, 127);
        float rl[8];
#pragma unroll
        for (int hl = 0; hl < 8; hl++) {
          float s = exact_pair(acc[2 * hl], qe0[hg][hl] + ke0, acc[2 * hl + 1], qe1[hg][hl] + ke1);
          rl[hl] = fmaxf(s, 0.0f);
        }
        // low lanes: heads 16hg+0..7
        if (kh == 0) {
#pragma unroll
          for (int hl = 0; hl < 8; hl++)
            if (hv[hg][hl]) part = __builtin_fmaf(wv[hg][hl], rl[hl], part);
        }
        float other = __shfl_xor(part, 32, kWave);
        if (kh == 1) {
          part = other;
#pragma unroll
          for (int hl = 0; hl < 8; hl++)
            if (hv[hg][hl]) part = __builtin_fmaf(wv[hg][hl], rl[hl], part);
        }
        other = __shfl_xor(part, 32, kWave);
        if (kh == 0) part = other;
      }
    }
    if (kh == 0 && valid) {
      const float sc = __fadd_rn(part, 0.0f);   // -0 -> +0
      out[blk] = ord_key(sc);
    }
  }
}

// ---------------------------------------------------------------------------
// Exact top-k by (score desc, block asc) over one score row per workgroup.
// Radix select on the 32-bit order keys (12 + 12 + 8 bits) finds the k-th key
// T and how many keys equal to T are needed; a compaction pass then emits, in
// ascending block order, every block above T and the lowest-index blocks equal
// to T.  Rows with at most k visible blocks emit them all, then -1.
// ---------------------------------------------------------------------------

struct SelectArgs {
  int n_q, m, k;
  int64_t stride;
  const int32_t* seq_len;
  const uint32_t* keys;
  int32_t* topk;
};

constexpr int kSelThreads = 1024;

// exclusive prefix sum over the 1024 threads; returns the block total in *total
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
  if (wave == 0) {
    uint32_t t = lane < 16 ? tmp[lane] : 0u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      uint32_t y = __shfl_up(t, o, kWave);
      if (lane >= o) t += y;
    }
    if (lane < 16) tmp[16 + lane] = t;   // inclusive wave prefix
  }
  __syncthreads();
  const uint32_t before_wave = wave ? tmp[16 + wave - 1] : 0u;
  *total = tmp[16 + 15];
  __syncthreads();
  return before_wave + x - v;
}

__global__ void __launch_bounds__(kSelThreads) topk_select_kernel(SelectArgs a) {
  const int srow = blockIdx.x;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  const int p = a.seq_len[brow] - a.n_q + qi;
  int nv = (p + 1) / a.m;
  if (nv > a.stride) nv = (int)a.stride;       // defensive: never past the key row
  const int k = a.k, tid = threadIdx.x;
  int32_t* out = a.topk + (int64_t)srow * k;
  if (nv <= k) {
    for (int j = tid; j < k; j += kSelThreads) out[j] = j < nv ? j : -1;
    return;
  }
  const uint32_t* keys = a.keys + (int64_t)srow * a.stride;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t tmp[64];
  __shared__ uint32_t found[2];

  uint32_t prefix = 0;
  uint32_t remaining = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int d = 0; d < 3; d++) {
    const int shift = shifts[d], width = widths[d];
    const uint32_t nb = 1u << width, mask = nb - 1;
    for (uint32_t j = tid; j < nb; j += kSelThreads) hist[j] = 0;
    __syncthreads();
    for (int j = tid; j < nv; j += kSelThreads) {
      const uint32_t key = keys[j];
      if (d == 0 || (key >> (shift + width)) == prefix) atomicAdd(&hist[(key >> shift) & mask], 1u);
    }
    __syncthreads();
    // bins owned by this thread: [lo, hi)
    const uint32_t per = nb >= kSelThreads ? nb / kSelThreads : 1;
    const uint32_t lo = (uint32_t)tid * per;
    const uint32_t hi = lo < nb ? lo + per : lo;
    uint32_t local = 0;
    for (uint32_t j = lo; j < hi; j++) local += hist[j];
    uint32_t total;
    const uint32_t below = block_exclusive_scan(local, tmp, &total);
    uint32_t running = total - below - local;   // keys in bins above this thread's range
    for (int j = (int)hi - 1; j >= (int)lo; j--) {
      const uint32_t c = hist[j];
      if (running < remaining && running + c >= remaining) {
        found[0] = (uint32_t)j;
        found[1] = running;
      }
      running += c;
    }
    __syncthreads();
    remaining -= found[1];
    prefix = (prefix << width) | found[0];
    __syncthreads();
  }
  const uint32_t T = prefix, need_eq = remaining;

  // compaction in ascending block order
  const int seg = (nv + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * seg, j1 = min(nv, j0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int j = j0; j < j1; j++) {
    const uint32_t key = keys[j];
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  uint32_t gt_run = block_exclusive_scan(gt, tmp, &tot);
  uint32_t eq_run = block_exclusive_scan(eq, tmp, &tot);
  for (int j = j0; j < j1; j++) {
    const uint32_t key = keys[j];
    if (key > T) {
      const uint32_t pos = gt_run + min(eq_run, need_eq);
      if (pos < (uint32_t)k) out[pos] = j;
      gt_run++;
    } else if (key == T) {
      const uint32_t pos = gt_run + eq_run;
      if (eq_run < need_eq && pos < (uint32_t)k) out[pos] = j;
      eq_run++;
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
  pl.chunks = (int)((nvmax + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG);
  if (pl.chunks < 1) pl.chunks = 1;
  pl.keys_bytes = (size_t)L->batch * n_q * pl.stride * sizeof(uint32_t);
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
  s.keys = static_cast<uint32_t*>(ws);
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
  sa.topk = topk;
  TimedLaunch t(kKernelTopkSelect, stream);
  hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelThreads), 0, stream, sa);
  return t.done();
}

}  // namespace lca
