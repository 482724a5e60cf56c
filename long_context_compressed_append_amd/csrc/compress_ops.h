// compress_ops.h -- device code of the sequence-axis compression shared by
// the compress launch and the decode launch that appends and selects in one
// (ring append, softmax-gated pooling, FP8 / BF16 / MXFP4 quantisation).
// Private to liblca.so.
//
// vibecoco.ai "DeepSeek V4 agent architecture" page, section 混合注意力:
// KV entries are compressed along the sequence by softmax-gated pooling with a
// learned position bias, stored in FP8 with BF16 RoPE dims; the indexer keys
// are FP4.  pnsm.cn "DeepSeek V4 架构深度解析" page, section 2.1: the window
// store keeps raw tokens and overwrites cyclically.
#pragma once

#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

struct CompressArgs {
  int B, m, R, n, has_idx, groups, nfin;   // nfin: block slots per row
  int64_t max_blocks;
  PageMap pm;                              // where each entry lives
  int32_t* seq_len;
  uint32_t* sync;
  uint8_t* nope;
  uint16_t* rope;
  float* kv_scale;
  uint8_t* idx_code;
  uint8_t* idx_scale;
  uint16_t* ring_kv;
  float* ring_gate;
  float* ring_ikey;
  float* ring_igate;
  const float* pos_bias;
  const float* ipos_bias;
  const uint16_t* kv;
  const float* gate;
  const float* ikey;
  const float* igate;
  int64_t ring_tasks, total_tasks;
};

// Token j of this call into the ring of row `row` (length L0 before the call).
__device__ __forceinline__ void ring_copy(const CompressArgs& a, int row, int j, int L0, int lane) {
  const int64_t slot = (int64_t)row * a.R + (int64_t)((L0 + j) % a.R);
  const int64_t src = (int64_t)row * a.n + j;
  // kv: 512 bf16 = 1 KB -> 16 B per lane
  const uint4* skv = reinterpret_cast<const uint4*>(a.kv + src * kKv);
  uint4* dkv = reinterpret_cast<uint4*>(a.ring_kv + slot * kKv);
  dkv[lane] = skv[lane];
  // gate: 512 fp32 = 2 KB -> 32 B per lane
  const uint4* sg = reinterpret_cast<const uint4*>(a.gate + src * kKv);
  uint4* dg = reinterpret_cast<uint4*>(a.ring_gate + slot * kKv);
  dg[lane] = sg[lane];
  dg[lane + 64] = sg[lane + 64];
  if (a.has_idx) {
    const uint4* sk = reinterpret_cast<const uint4*>(a.ikey + src * kIdx);
    const uint4* sgi = reinterpret_cast<const uint4*>(a.igate + src * kIdx);
    uint4* dk = reinterpret_cast<uint4*>(a.ring_ikey + slot * kIdx);
    uint4* dgi = reinterpret_cast<uint4*>(a.ring_igate + slot * kIdx);
    if (lane < 16) dk[lane] = sk[lane];
    else if (lane < 32) dgi[lane - 16] = sgi[lane - 16];
  }
}

// Longer blocks (m = 16 .. 128): the m logits (then weights) of this lane's
// channel go to the wavefront's LDS slice lds[i * 64 + lane] (64 m floats);
// the loads of a batch of NB tokens are all issued before any is used.  NB
// divides m (16 for m = 16, 32 above), so no batch reaches past the block.
template <int NB, typename XF, typename ZF>
__device__ __forceinline__ float pool_long(int m, XF xval, ZF zval, const float* bias, int C, int c,
                                           float* lds, int lane) {
  float mx = -INFINITY;
#pragma unroll 1
  for (int i0 = 0; i0 < m; i0 += NB) {
    float zv[NB], bv[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) zv[i] = zval(i0 + i);
#pragma unroll
    for (int i = 0; i < NB; i++) bv[i] = bias[(i0 + i) * C + c];
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const float ai = __fadd_rn(zv[i], bv[i]);
      lds[(i0 + i) * 64 + lane] = ai;
      mx = ai > mx ? ai : mx;
    }
  }
  float S = 0.0f;
#pragma unroll 8
  for (int i = 0; i < m; i++) {
    const float e = expf(__fsub_rn(lds[i * 64 + lane], mx));
    lds[i * 64 + lane] = e;
    S = __fadd_rn(S, e);
  }
  // the weighted sum in ascending order
  float acc = 0.0f;
#pragma unroll 1
  for (int i0 = 0; i0 < m; i0 += NB) {
    float xv[NB];
#pragma unroll
    for (int i = 0; i < NB; i++) xv[i] = xval(i0 + i);
#pragma unroll
    for (int i = 0; i < NB; i++)
      acc = __fadd_rn(acc, __fmul_rn(__fdiv_rn(lds[(i0 + i) * 64 + lane], S), xv[i]));
  }
  return acc;
}

// Pool channel `c` (of a stream with C channels) over the m tokens of block bk.
// Token t of the block comes from this call's input when t >= L0, else from
// the ring.  Same operation order as the definition: logits, max, exp and
// ascending sum, then the weights times the values in ascending order.
template <bool kBf16>
__device__ __forceinline__ float pool_channel(const CompressArgs& a, int row, int64_t bk, int L0,
                                              int c, int C, const void* in_x, const float* in_z,
                                              const void* ring_x, const float* ring_z,
                                              const float* bias, float* lds, int lane) {
  const int m = a.m;
  const int64_t t0 = bk * m;
  // element index of token t0 + i: the call's input from position L0 on, the
  // ring (slot (t0 + i) % R) before it; branch-free so that loads batch
  const int slot0 = (int)(t0 % a.R);
  auto elem = [&](int i, bool& from_input) -> int64_t {
    const int64_t t = t0 + i;
    from_input = t >= L0;
    int slot = slot0 + i;
    slot = slot >= a.R ? slot - a.R : slot;     // i < m <= R
    return from_input ? ((int64_t)row * a.n + (t - L0)) * C + c : ((int64_t)row * a.R + slot) * C + c;
  };
  auto xval = [&](int i) -> float {
    bool in;
    const int64_t e = elem(i, in);
    if (kBf16) {
      const uint16_t* base = static_cast<const uint16_t*>(in ? in_x : ring_x);
      return bf16_f32(base[e]);
    }
    const float* base = static_cast<const float*>(in ? in_x : ring_x);
    return base[e];
  };
  auto zval = [&](int i) -> float {
    bool in;
    const int64_t e = elem(i, in);
    return (in ? in_z : ring_z)[e];
  };
  if (m <= 8) {
    // short blocks: every token's logit and value in registers, one load pass
    float av[8], xv[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i < m) {
        av[i] = __fadd_rn(zval(i), bias[i * C + c]);
        xv[i] = xval(i);
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (i < m) M = av[i] > M ? av[i] : M;
    float ev[8], S = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (i < m) {
        ev[i] = expf(__fsub_rn(av[i], M));
        S = __fadd_rn(S, ev[i]);
      }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (i < m) acc = __fadd_rn(acc, __fmul_rn(__fdiv_rn(ev[i], S), xv[i]));
    return acc;
  }
  // m = 16 .. 128 (a power of two): batches of 16 tokens for m = 16, else 32
  if (m == 16) return pool_long<16>(m, xval, zval, bias, C, c, lds, lane);
  return pool_long<32>(m, xval, zval, bias, C, c, lds, lane);
}

// Group g of block bk (entry e) of row `row`, whose last tokens come from
// this call (length L0 before it): pooling, then FP8 (groups 0..6, one
// 64-channel group each, lane = channel), BF16 RoPE dims (group 7) or the
// MXFP4 indexer key (group 8, two 32-lane MX blocks).  patch (group 8,
// optional, LDS): also receives the key's 32 code bytes and 2 scale bytes.
__device__ __forceinline__ void finalize_group(const CompressArgs& a, int row, int64_t bk, int L0, int g, int64_t e,
                                               float* lds, int lane, uint8_t* patch) {
  if (g < 8) {
    const int c = g * 64 + lane;
    float y = pool_channel<true>(a, row, bk, L0, c, kKv, a.kv, a.gate, a.ring_kv, a.ring_gate, a.pos_bias, lds, lane);
    if (g < 7) {
      float amax = wave_max(fabsf(y));
      uint32_t code = 0;
      float scale = 0.0f;
      if (amax > 0.0f) {
        float inv = __fdiv_rn(448.0f, amax);
        scale = __fdiv_rn(amax, 448.0f);
        code = f32_e4m3(__fmul_rn(y, inv));
      }
      a.nope[e * kNope + c] = (uint8_t)code;
      if (lane == 0) a.kv_scale[e * kScaleStride + g] = scale;
    } else {
      a.rope[e * kRope + lane] = f32_bf16(y);
      if (lane == 0) a.kv_scale[e * kScaleStride + 7] = 0.0f;
    }
  } else {
    float y = pool_channel<false>(a, row, bk, L0, lane, kIdx, a.ikey, a.igate, a.ring_ikey, a.ring_igate,
                                  a.ipos_bias, lds, lane);
    float amax = half_wave_max(fabsf(y));
    uint32_t code = 0, ebyte = 0;
    if (amax > 0.0f) {
      int X = floor_log2(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      code = f32_e2m1(ldexpf(y, -X));
      ebyte = (uint32_t)(X + 127);
    }
    uint32_t hi = lane_xor1(code);
    if ((lane & 1) == 0) a.idx_code[e * 32 + (lane >> 1)] = (uint8_t)(code | (hi << 4));
    if ((lane & 31) == 0) a.idx_scale[e * 2 + (lane >> 5)] = (uint8_t)ebyte;
    if (patch) {
      if ((lane & 1) == 0) patch[lane >> 1] = (uint8_t)(code | (hi << 4));
      if ((lane & 31) == 0) patch[32 + (lane >> 5)] = (uint8_t)ebyte;
    }
  }
}


// The compression arguments of a call appending n tokens per row.
inline CompressArgs compress_args(const lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                                  const float* igate, int n) {
  CompressArgs a;
  a.B = L->batch;
  a.m = L->ratio;
  a.R = L->ring;
  a.n = n;
  a.has_idx = L->has_indexer;
  a.groups = L->has_indexer ? 9 : 8;
  a.nfin = (n - 1) / L->ratio + 1;
  a.max_blocks = L->max_blocks;
  a.pm = page_map_of<PageMap>(L);
  a.seq_len = L->seq_len;
  a.sync = L->sync;
  a.nope = L->nope;
  a.rope = L->rope;
  a.kv_scale = L->kv_scale;
  a.idx_code = L->idx_code;
  a.idx_scale = L->idx_scale;
  a.ring_kv = L->ring_kv;
  a.ring_gate = L->ring_gate;
  a.ring_ikey = L->ring_ikey;
  a.ring_igate = L->ring_igate;
  a.pos_bias = L->pos_bias;
  a.ipos_bias = L->ipos_bias;
  a.kv = kv;
  a.gate = gate;
  a.ikey = ikey;
  a.igate = igate;
  a.ring_tasks = (int64_t)a.B * n;
  a.total_tasks = a.ring_tasks + (int64_t)a.B * a.nfin * a.groups;
  return a;
}

}  // namespace lca
