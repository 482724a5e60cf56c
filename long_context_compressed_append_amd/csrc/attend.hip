// attend.hip -- attention over compressed entries plus the raw window, on the
// matrix cores, with a split-K online-softmax combine.
//
// pnsm.cn "DeepSeek V4 架构深度解析" page, section 2.1: one attention call over
// the sliding-window KV and the selected compressed KV.  vibecoco.ai "DeepSeek
// V4 agent architecture" page, section 混合注意力 (and agents-report.net
// "DeepSeek-V4：交錯壓縮注意力與低位元 KV 儲存", section 核心技術): CSA keeps
// the top-k compressed blocks, HCA attends densely to all of them; recent
// tokens stay at raw precision; entries are FP8 with BF16 RoPE dims.
//
// All query heads of a row share one 512-d key/value vector per key, so a
// workgroup stages each key once in LDS and 4 wavefronts x 16 heads use it.
//   QK^T  bf16 matrix cores: a staged key holds the exact bf16 value of each
//         e4m3 code (or the raw bf16 window token); the per-64-dim FP8 scale
//         multiplies each 64-dim partial dot in fp32.
//   P V   fp16 matrix cores: the staged value is fp16(code * scale) (or the
//         window token), transposed so that the key index is the contraction
//         dim; P is fp16 in [0, 1].
// Online softmax in base 2 (logits pre-multiplied by log2 e).  Each workgroup
// covers a contiguous chunk of the key list; chunks are merged by the combine
// kernel (or written directly when there is one chunk).
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;          // keys per tile
constexpr int kKst = 520;          // bf16 per staged key row (512 + 8 pad)
constexpr int kVst = 40;           // fp16 per staged value column (32 + 8 pad)
constexpr int kPst = 40;
constexpr int kMaxTopk = 2048;
constexpr int kAttendTargetWGs = 256;

struct AttendArgs {
  int n_q, H, m, W, R, k, splits, chunk, csa;
  int64_t max_blocks;
  float scale_log2;
  const int32_t* seq_len;
  const uint8_t* nope;
  const uint16_t* rope;
  const float* kv_scale;
  const uint16_t* ring_kv;
  const uint16_t* q;
  const int32_t* topk;
  float* out;
  float* ws_ml;
  _Float16* ws_o;
};

__device__ __forceinline__ uint32_t scan_excl_256(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; w++) before += tmp[w];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return before + x - v;
}

__global__ void __launch_bounds__(256) attend_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * kKst];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[kKv * kVst];
  __shared__ float sK[kTile * 8];
  __shared__ int kvalid[kTile];
  __shared__ __attribute__((aligned(16))) _Float16 Ps[4][16 * kPst];
  __shared__ int klist[kMaxTopk];
  __shared__ uint32_t tmp[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int srow = blockIdx.y, split = blockIdx.x, hgrp = blockIdx.z;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  const int p = a.seq_len[brow] - a.n_q + qi;
  int nv = (p + 1) / a.m;
  if (nv > a.max_blocks) nv = (int)a.max_blocks;   // defensive
  const int nw = min(a.W, p + 1);
  const int w0 = p - nw + 1;

  int n_c = nv;
  if (a.csa) {
    // keep listed, visible blocks in list order
    const int32_t* sel = a.topk + (int64_t)srow * a.k;
    const int per = (a.k + 255) / 256;          // <= 8
    const int j0 = tid * per;
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; u++) ev[u] = (u < per && j0 + u < a.k) ? sel[j0 + u] : -1;
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < 8; u++) cnt += (ev[u] >= 0 && ev[u] < nv);
    uint32_t total;
    uint32_t pos = scan_excl_256(cnt, tmp, &total);
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (ev[u] >= 0 && ev[u] < nv && pos < (uint32_t)kMaxTopk) klist[pos++] = ev[u];
    n_c = (int)total;
    __syncthreads();
  }
  const int n_keys = n_c + nw;
  const int kb = split * a.chunk;
  const int ke = min(n_keys, kb + a.chunk);

  const int h0 = hgrp * 64 + wave * 16;
  const bool active = h0 < a.H;
  const int hq = h0 + (lane & 15);            // head of this lane's A-operand row
  const int kq = 8 * (lane >> 4);             // K offset of this lane inside a 32-K step

  v8bf qf[16];
  {
    const uint16_t* qrow = a.q + ((int64_t)srow * a.H + hq) * kKv;
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (active && hq < a.H) v = *reinterpret_cast<const uint4*>(qrow + ks * 32 + kq);
      qf[ks] = __builtin_bit_cast(v8bf, v);
    }
  }
  v4f O[32];
#pragma unroll
  for (int c = 0; c < 32; c++) O[c] = (v4f){0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    mrow[r] = -INFINITY;
    lrow[r] = 0.0f;
  }

  const int sj = tid >> 3, sg = tid & 7;      // staging: key sj, 64-dim group sg
  for (int t0 = kb; t0 < ke; t0 += kTile) {
    __syncthreads();
    {
      const int kk = t0 + sj;
      uint16_t* kdst = Ks + sj * kKst + sg * 64;
      if (kk < ke && kk < n_c) {
        const int e = a.csa ? klist[kk] : kk;
        const int64_t ent = (int64_t)brow * a.max_blocks + e;
        if (sg < 7) {
          const float s = a.kv_scale[ent * kScaleStride + sg];
          const uint4* src = reinterpret_cast<const uint4*>(a.nope + ent * kNope + sg * 64);
          uint4 cv[4];
#pragma unroll
          for (int v = 0; v < 4; v++) cv[v] = src[v];
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const uint4 c16 = cv[v];
            const uint32_t w4[4] = {c16.x, c16.y, c16.z, c16.w};
            uint32_t kb4[8];
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
#pragma unroll
              for (int hw = 0; hw < 2; hw++) {
                // two codes -> exact fp32 (OCP e4m3 on gfx950), bf16 bits for K,
                // fp16(value * scale) for V
                const v2f f = hw ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[q4], true)
                                 : __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[q4], false);
                kb4[q4 * 2 + hw] = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
                const v2f sv = {__fmul_rn(f[0], s), __fmul_rn(f[1], s)};
                const v2h hv = __builtin_convertvector(sv, v2h);
                const int c = v * 16 + q4 * 4 + hw * 2;
                Vt[(sg * 64 + c) * kVst + sj] = hv[0];
                Vt[(sg * 64 + c + 1) * kVst + sj] = hv[1];
              }
            }
            uint4* kd = reinterpret_cast<uint4*>(kdst + v * 16);
            kd[0] = make_uint4(kb4[0], kb4[1], kb4[2], kb4[3]);
            kd[1] = make_uint4(kb4[4], kb4[5], kb4[6], kb4[7]);
          }
          sK[sj * 8 + sg] = s;
        } else {
          const uint4* src = reinterpret_cast<const uint4*>(a.rope + ent * kRope);
          uint4 rv[8];
#pragma unroll
          for (int v = 0; v < 8; v++) rv[v] = src[v];
#pragma unroll
          for (int v = 0; v < 8; v++) {
            const uint4 w = rv[v];
            reinterpret_cast<uint4*>(kdst)[v] = w;
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
              const int c = v * 8 + q4 * 2;
              const v2f f = {__uint_as_float(ww[q4] << 16), __uint_as_float(ww[q4] & 0xFFFF0000u)};
              const v2h hv = __builtin_convertvector(f, v2h);
              Vt[(448 + c) * kVst + sj] = hv[0];
              Vt[(448 + c + 1) * kVst + sj] = hv[1];
            }
          }
          sK[sj * 8 + 7] = 1.0f;
        }
      } else if (kk < ke) {
        const int pos = w0 + (kk - n_c);
        const uint4* src = reinterpret_cast<const uint4*>(
            a.ring_kv + ((int64_t)brow * a.R + pos % a.R) * kKv + sg * 64);
        uint4 rv[8];
#pragma unroll
        for (int v = 0; v < 8; v++) rv[v] = src[v];
#pragma unroll
        for (int v = 0; v < 8; v++) {
          const uint4 w = rv[v];
          reinterpret_cast<uint4*>(kdst)[v] = w;
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int q4 = 0; q4 < 4; q4++) {
            const int c = sg * 64 + v * 8 + q4 * 2;
            const v2f f = {__uint_as_float(ww[q4] << 16), __uint_as_float(ww[q4] & 0xFFFF0000u)};
            const v2h hv = __builtin_convertvector(f, v2h);
            Vt[c * kVst + sj] = hv[0];
            Vt[(c + 1) * kVst + sj] = hv[1];
          }
        }
        sK[sj * 8 + sg] = 1.0f;
      } else {
#pragma unroll 1
        for (int v = 0; v < 8; v++) reinterpret_cast<uint4*>(kdst)[v] = make_uint4(0, 0, 0, 0);
#pragma unroll 1
        for (int c = 0; c < 64; c++) Vt[(sg * 64 + c) * kVst + sj] = (_Float16)0.0f;
        sK[sj * 8 + sg] = 0.0f;
      }
      if (sg == 0) kvalid[sj] = kk < ke;
    }
    __syncthreads();

    if (active) {
      // S = Q K^T for 16 heads x 32 keys, per 64-dim group scaled in fp32
      v4f S[2];
#pragma unroll
      for (int nt = 0; nt < 2; nt++) {
        S[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
        const int key = nt * 16 + (lane & 15);
        const uint16_t* krow = Ks + key * kKst + kq;
#pragma unroll
        for (int g = 0; g < 8; g++) {
          v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < 2; s2++) {
            const int ks = 2 * g + s2;
            const v8bf kb8 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(krow + ks * 32));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kb8, acc, 0, 0, 0);
          }
          const float sc = sK[key * 8 + g];
#pragma unroll
          for (int r = 0; r < 4; r++) S[nt][r] = __builtin_fmaf(sc, acc[r], S[nt][r]);
        }
      }
      // online softmax (base 2); lane holds keys (lane&15)+{0,16}, heads 4*(lane>>4)+r
      const bool v0 = kvalid[lane & 15], v1 = kvalid[16 + (lane & 15)];
      float alpha[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float x0 = v0 ? S[0][r] * a.scale_log2 : -INFINITY;
        const float x1 = v1 ? S[1][r] * a.scale_log2 : -INFINITY;
        float mx = fmaxf(x0, x1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        const float mnew = fmaxf(mrow[r], mx);
        float p0 = 0.f, p1 = 0.f;
        if (mnew == -INFINITY) {
          alpha[r] = 1.0f;
        } else {
          alpha[r] = exp2f(mrow[r] - mnew);
          p0 = exp2f(x0 - mnew);
          p1 = exp2f(x1 - mnew);
        }
        lrow[r] = lrow[r] * alpha[r] + p0 + p1;
        mrow[r] = mnew;
        _Float16* prow = Ps[wave] + (4 * (lane >> 4) + r) * kPst;
        prow[lane & 15] = (_Float16)p0;
        prow[16 + (lane & 15)] = (_Float16)p1;
      }
      const bool rescale = (alpha[0] != 1.0f) | (alpha[1] != 1.0f) | (alpha[2] != 1.0f) | (alpha[3] != 1.0f);
      if (__any(rescale)) {
#pragma unroll
        for (int c = 0; c < 32; c++)
#pragma unroll
          for (int r = 0; r < 4; r++) O[c][r] *= alpha[r];
      }
    }
    __syncthreads();
    if (active) {
      const v8h pa = *reinterpret_cast<const v8h*>(Ps[wave] + (lane & 15) * kPst + kq);
#pragma unroll
      for (int ct = 0; ct < 32; ct++) {
        const v8h vb = *reinterpret_cast<const v8h*>(Vt + (ct * 16 + (lane & 15)) * kVst + kq);
        O[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, O[ct], 0, 0, 0);
      }
    }
  }

  if (!active) return;
#pragma unroll
  for (int r = 0; r < 4; r++)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lrow[r] += __shfl_xor(lrow[r], o, kWave);

  const int hbase = h0 + 4 * (lane >> 4);
  if (a.splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = hbase + r;
      if (h >= a.H) continue;
      const float inv = 1.0f / lrow[r];
      float* dst = a.out + ((int64_t)srow * a.H + h) * kKv;
#pragma unroll
      for (int ct = 0; ct < 32; ct++) dst[ct * 16 + (lane & 15)] = O[ct][r] * inv;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int h = hbase + r;
      if (h >= a.H) continue;
      const int64_t slot = ((int64_t)srow * a.splits + split) * a.H + h;
      if ((lane & 15) == 0) {
        a.ws_ml[slot * 2 + 0] = mrow[r];
        a.ws_ml[slot * 2 + 1] = lrow[r];
      }
      if (lrow[r] > 0.0f) {       // normalised partial output, fp16 (values of V's range)
        const float inv = 1.0f / lrow[r];
        _Float16* dst = a.ws_o + slot * kKv;
#pragma unroll
        for (int ct = 0; ct < 32; ct++) dst[ct * 16 + (lane & 15)] = (_Float16)(O[ct][r] * inv);
      }
    }
  }
}

struct CombineArgs {
  int H, splits;
  const float* ws_ml;
  const _Float16* ws_o;
  float* out;
};

__global__ void __launch_bounds__(128) attend_combine_kernel(CombineArgs a) {
  const int srow = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  float M = -INFINITY;
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // splits in groups of 8: every load of a group in flight before use
  for (int s0 = 0; s0 < a.splits; s0 += 8) {
    float mv[8], lv[8];
    uint2 ov[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int64_t slot = ((int64_t)srow * a.splits + s0 + u) * a.H + h;
      const bool in = s0 + u < a.splits;
      mv[u] = in ? a.ws_ml[slot * 2] : -INFINITY;
      lv[u] = in ? a.ws_ml[slot * 2 + 1] : 0.0f;
      ov[u] = in ? reinterpret_cast<const uint2*>(a.ws_o + slot * kKv)[t] : make_uint2(0, 0);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (lv[u] > 0.0f) Mn = fmaxf(Mn, mv[u]);
    const float rescale = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
    L *= rescale;
    acc.x *= rescale;
    acc.y *= rescale;
    acc.z *= rescale;
    acc.w *= rescale;
    M = Mn;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (!(lv[u] > 0.0f)) continue;
      const float w = lv[u] * exp2f(mv[u] - M);
      L += w;
      const v2h o01 = __builtin_bit_cast(v2h, ov[u].x), o23 = __builtin_bit_cast(v2h, ov[u].y);
      acc.x += w * (float)o01[0];
      acc.y += w * (float)o01[1];
      acc.z += w * (float)o23[0];
      acc.w += w * (float)o23[1];
    }
  }
  const float inv = 1.0f / L;
  reinterpret_cast<float4*>(a.out + ((int64_t)srow * a.H + h) * kKv)[t] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

AttendPlan plan_attend(const lca_layer* L, int n_q, int H, int k, bool csa) {
  AttendPlan pl;
  const int64_t nvmax = L->len_max / L->ratio;
  pl.max_keys = (csa ? (k < nvmax ? k : nvmax) : nvmax) + L->window;
  pl.head_groups = (H + 63) / 64;
  const int64_t rows = (int64_t)L->batch * n_q;
  const int64_t max_tiles = (pl.max_keys + kTile - 1) / kTile;
  int64_t s = (kAttendTargetWGs + rows * pl.head_groups - 1) / (rows * pl.head_groups);
  const int forced = env_int("LCA_ATTEND_SPLITS", 0);
  if (forced > 0) s = forced;
  if (s > max_tiles) s = max_tiles;
  if (s < 1) s = 1;
  const int64_t per = (pl.max_keys + s - 1) / s;
  pl.chunk = (int)(((per + kTile - 1) / kTile) * kTile);
  pl.splits = (int)((pl.max_keys + pl.chunk - 1) / pl.chunk);
  if (pl.splits > 1) {
    pl.ml_bytes = (size_t)rows * pl.splits * H * 2 * sizeof(float);
    pl.o_bytes = (size_t)rows * pl.splits * H * kKv * sizeof(_Float16);
  } else {
    pl.ml_bytes = pl.o_bytes = 0;
  }
  return pl;
}

int launch_attend(const lca_layer* L, const uint16_t* q, int n_q, int H, const int32_t* topk, int k,
                  float scale, float* out, void* ws, const AttendPlan& pl, hipStream_t stream) {
  AttendArgs a;
  a.n_q = n_q;
  a.H = H;
  a.m = L->ratio;
  a.W = L->window;
  a.R = L->ring;
  a.k = k;
  a.splits = pl.splits;
  a.chunk = pl.chunk;
  a.csa = topk != nullptr;
  a.max_blocks = L->max_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.seq_len = L->seq_len;
  a.nope = L->nope;
  a.rope = L->rope;
  a.kv_scale = L->kv_scale;
  a.ring_kv = L->ring_kv;
  a.q = q;
  a.topk = topk;
  a.out = out;
  a.ws_ml = static_cast<float*>(ws);
  a.ws_o = reinterpret_cast<_Float16*>(static_cast<char*>(ws) + ((pl.ml_bytes + 255) & ~(size_t)255));
  const int rows = L->batch * n_q;
  {
    TimedLaunch t(kKernelAttend, stream);
    hipLaunchKernelGGL(attend_kernel, dim3(pl.splits, rows, pl.head_groups), dim3(256), 0, stream, a);
    int rc = t.done();
    if (rc) return rc;
  }
  if (pl.splits > 1) {
    CombineArgs c;
    c.H = H;
    c.splits = pl.splits;
    c.ws_ml = a.ws_ml;
    c.ws_o = a.ws_o;
    c.out = out;
    TimedLaunch t(kKernelAttendCombine, stream);
    hipLaunchKernelGGL(attend_combine_kernel, dim3(rows, H), dim3(128), 0, stream, c);
    return t.done();
  }
  return LCA_OK;
}

}  // namespace lca
