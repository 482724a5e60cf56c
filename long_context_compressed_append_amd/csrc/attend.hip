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
// workgroup stages each key once in LDS and 4 compute wavefronts use it, one
// per SIMD: wavefront w takes heads 16 w .. +15 of its head group over all
// 512 channels, so its scores need no exchange with another wavefront.  Four
// more wavefronts only stage: while the compute wavefronts work on tile t
// from one LDS buffer they load tile t + 2 and convert tile t + 1 into the
// other, so the loads and conversions leave the critical path.
// A staged key is one fp16 image serving as K and as V: the exact value of
// each e4m3 code (e4m3 values are fp16 numbers), or the bf16 RoPE / window
// value (exact in fp16's normal range [2^-14, 65504], below it rounded to
// fp16's subnormal spacing 2^-24).  The query is converted to fp16 the same
// way, so each image is within 2^-11 of its vector's largest magnitude when
// that lies in [2^-14, 65504].  LCA_STATUS_FP16_RANGE in the layer's status
// word reports an input where this may fail: a query head or a 64-channel
// key group (RoPE, or window channels) whose largest magnitude is 65536 or
// more (also inf, NaN) or nonzero and below 2^-14, or an FP8 group scale
// outside [2^-14, 2^8) (where P * scale leaves fp16's normal range).  Every product is computed transposed, keys x heads, so that
// a lane owns one head throughout: lane l holds head l % 16 and key / channel
// quarter l / 16.
//   S^T = K Q^T   fp16 matrix cores over the 512 channels; the per-64-dim
//                 FP8 scale multiplies each 64-dim partial dot in fp32.
//                 Lane l ends with keys 4(l/16)+r and 16+4(l/16)+r of its head.
//   softmax       online, base 2, per lane (one head) plus a max over the four
//                 lanes that share the head; the running maximum is only
//                 moved when it grows by more than 2^8, so rescaling is rare
//                 and P (<= 256) stays in registers.
//   O^T = V^T P^T fp16 matrix cores: the k-slots of the product are the eight
//                 keys the lane already holds, so P^T is the B operand; since
//                 the tile holds code values, the B operand of a 64-dim group
//                 is fp16(p * that group's scale of the key).  The V^T operand
//                 comes from the LDS transpose read ds_read_b64_tr_b16.  Lane
//                 l accumulates channels 16 ct + 4(l/16) + r of its head for
//                 the 32 channel tiles ct.
// Each workgroup covers a contiguous chunk of the key list; chunks are merged
// by the combine kernel (or written directly when there is one chunk).
#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;          // keys per tile
// Row pitch 1056 bytes (32 mod 256): the 8-byte transpose reads of 8 keys x 4
// chunks by 32 lanes cover all banks once.
constexpr int kVst = 528;          // fp16 per staged key row (512 + 16 pad)
constexpr int kMaxChunk = 1024;    // keys per split workgroup (list entries staged in LDS)
constexpr int kAttendTargetWGs = 256;
static_assert(kMaxChunk % (64 * 8) == 0, "whole list entries per thread");

struct AttendArgs {
  int n_q, H, m, W, R, k, splits, chunk, csa, hwaves;
  int64_t max_blocks;
  PageMap pm;             // where each entry lives
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
  uint32_t* status;      // the layer's status word (LCA_STATUS_* bits)
};

// buffer resource word 3: raw 32-bit data (gfx9 layout); an access at or
// past the range reads 0 (loads) or is dropped
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kDropOffset = 0x80000000u;
typedef unsigned int u32x4a __attribute__((ext_vector_type(4)));

constexpr int kComputeWaves = 4;   // 4 head wavefronts of 16 heads, all channels
constexpr int kStageWaves = 4;     // wavefronts that load and convert the next tile
constexpr int kThreads = 64 * (kComputeWaves + kStageWaves);
constexpr float kLazyMax = 8.0f;   // log2 headroom of the running maximum

// Raw data of one staged (key, 32-dim half group) slot, loaded one tile ahead.
struct StageRegs {
  uint4 d[4];       // nope: d[0..1] (32 codes); rope/window: d[0..3] (32 bf16)
  float s;          // FP8 scale of the group (read for every slot, used for nope)
  int kind;         // 0 padding, 1 nope group, 2 rope group of an entry, 3 window group
};

// kCsa: the key list is the top-k list (else every visible entry); kPaged:
// the entry planes are a page pool.  Separate instantiations, so that each
// launch fetches only the code of its own case.
template <bool kCsa, bool kPaged>
__global__ void __launch_bounds__(kThreads) attend_kernel(AttendArgs a) {
  // two tile buffers: the compute wavefronts read tile t from buffer t % 2
  // while the staging wavefronts convert tile t + 1 into the other
  __shared__ __attribute__((aligned(16))) _Float16 Ts[2][kTile * kVst];   // [key][channel]
  __shared__ __attribute__((aligned(16))) float sK[2][8 * kTile];     // [group][key]
  __shared__ __attribute__((aligned(16))) float kbias[2][kTile];      // 0, or -inf for a masked key
  __shared__ int klist[kMaxChunk];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool computes = wave < kComputeWaves;
  const int hw = wave & 3;                    // head wavefront (compute wavefronts)
  const int srow = blockIdx.y, split = blockIdx.x, hgrp = blockIdx.z;
  const int brow = srow / a.n_q, qi = srow % a.n_q;
  const int h0 = hgrp * 64 + hw * 16;
  const bool active = computes && h0 < a.H;
  const int hq = h0 + (lane & 15);            // this lane's head
  const int g = lane >> 4;                    // this lane's key / channel quarter
  const int kq = 8 * g;                       // K offset of this lane inside a 32-K step

  // range_ok turns false on an input the fp16 images may not hold to 2^-11
  // of their vector's largest magnitude (reported through the status word):
  // a query head or a 64-channel key group whose largest magnitude is 65536
  // or more (also inf, NaN), or nonzero and below 2^-14; an FP8 scale
  // outside [2^-14, 2^8)
  bool range_ok = true;
  bool page_ok = true;    // false: a visible entry lay on an unmapped page (staged as masked)
  const int kb = split * a.chunk;
  // Loads go out in the order their data is needed (loads complete in
  // order): the CSA list (for the staging of tile 0), then the query (for
  // the first product); the query is converted only after the list is in
  // LDS, so the staging of tile 0 does not wait for it.
  // Buffer loads, so that no branch separates the loads from their use (a
  // masked lane's offset lies past the range and reads 0) and each wait
  // covers only the loads issued before the ones it needs.
  int e[kMaxChunk / kThreads];
  if (kCsa) {
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.topk + (int64_t)srow * a.k), (short)0, a.k * 4, kRsrcWord3);
#pragma unroll
    for (int u = 0; u < kMaxChunk / kThreads; u++) {
      const int j = tid + u * kThreads, kk = kb + j;
      const bool ok = j < a.chunk && kk < a.k;
      const int v = __builtin_amdgcn_raw_buffer_load_b32(lrs, ok ? 4 * kk : (int)kDropOffset, 0, 0);
      e[u] = ok ? v : -1;
    }
  }
  uint4 qraw[16];  // q of this lane's head (bf16), channels 32 ks + 8 g .. +7
  {
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.q + (int64_t)srow * a.H * kKv), (short)0, a.H * kKv * 2, kRsrcWord3);
    const bool ok = active && hq < a.H;
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      const u32x4a v = __builtin_amdgcn_raw_buffer_load_b128(
          qrs, ok ? (hq * kKv + ks * 32 + kq) * 2 : (int)kDropOffset, 0, 0);
      qraw[ks] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }

  const int p = a.seq_len[brow] - a.n_q + qi;
  int nv = (p + 1) / a.m;
  if (nv > a.max_blocks) nv = (int)a.max_blocks;   // defensive
  const int nw = min(a.W, p + 1);
  const int w0 = p - nw + 1;
  // key list: CSA = the k listed blocks (entries that are -1 or not yet
  // visible are masked), HCA = the visible blocks; then the window tokens
  const int n_c = kCsa ? a.k : nv;
  const int n_keys = n_c + nw;
  const int ke = min(n_keys, kb + a.chunk);
  if (split == a.splits - 1 && n_keys > ke && tid == 0)   // more keys than the plan holds
    atomicOr(a.status, LCA_STATUS_ATTEND_CAPACITY);
  constexpr bool paged = kPaged;               // the launch checked a.pm.shift >= 0
  if (kCsa) {
    // the listed blocks; on a paged layer their physical entries, looked up
    // here all at once (-1: padding or not visible, -2: visible on an
    // unmapped page)
#pragma unroll
    for (int u = 0; u < kMaxChunk / kThreads; u++) {
      const int j = tid + u * kThreads;
      if (j < a.chunk) {
        int v = e[u];
        if (paged) {
          const int64_t pe = e[u] >= 0 && e[u] < nv ? entry_index(a.pm, brow, e[u]) : (int64_t)-1;
          v = pe >= 0 ? (int)pe : (e[u] >= 0 && e[u] < nv ? -2 : -1);
        }
        klist[j] = v;
      }
    }
  }
  // HCA on a paged layer: the split's entries kb .. min(ke, nv) - 1 are
  // consecutive, so klist holds the page-table entries of their pages
  // (pages pg0 ..) and the staging takes each entry's page from LDS
  const int pg0 = paged ? kb >> a.pm.shift : 0;
  const int cend = min(ke, n_c);
  const int npg = paged && cend > kb ? ((cend - 1) >> a.pm.shift) - pg0 + 1 : 0;
  if (!kCsa && paged) {                       // npg <= kMaxChunk: the plan sizes the splits for it
    for (int j = tid; j < npg; j += kThreads)
      klist[j] = a.pm.table[(int64_t)brow * a.pm.pages_per_row + pg0 + j];
  }

  v4f O[32];
#pragma unroll
  for (int c = 0; c < 32; c++) O[c] = (v4f){0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.0f;
  __syncthreads();   // klist

  // staging: key sj, 32-dim part sp; staging wavefront w stages the 64-dim
  // groups w and w + 4 of the 32 keys (a wavefront's slots of one group are
  // all of one kind)
  const int sj = lane & 31, sp = lane >> 5, sw = wave - kComputeWaves;
  // Issue the global loads of this thread's slot of the tile at t0.  Every
  // lane issues the same four 16-byte loads (a masked slot reads a harmless
  // in-bounds address, an FP8 part reads its 32 bytes twice), so the loads
  // of one tile never wait on one another.
  auto stage_load = [&](int t0, int sg, StageRegs& st) {
    const int kk = t0 + sj;
    int kind = 0;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.ring_kv);
    const float* scp = a.kv_scale;
    if (kk < ke) {
      if (kk < n_c) {
        // the entry's place from registers and LDS only: a global load here
        // would make every later data load wait for it (loads complete in
        // order), draining the loads of the tiles in flight
        const int e = kCsa ? klist[kk - kb] : kk;
        int64_t ent = -1;
        if (kCsa && paged) {                      // klist holds physical entries
          ent = e >= 0 ? (int64_t)e : (int64_t)-1;
          page_ok &= e != -2;
        } else if (e >= 0 && e < nv) {
          ent = paged ? phys_entry(a.pm, klist[(e >> a.pm.shift) - pg0], e)   // HCA: the pages in LDS
                      : (int64_t)brow * a.max_blocks + e;
          page_ok &= ent >= 0;                     // a visible entry on an unmapped page
        }
        if (ent >= 0) {
          if (sg < 7) {
            src = a.nope + ent * kNope + sg * 64 + sp * 32;
            scp = a.kv_scale + ent * kScaleStride + sg;
            kind = 1;
          } else {
            src = reinterpret_cast<const uint8_t*>(a.rope + ent * kRope + sp * 32);
            kind = 2;
          }
        }
      } else {
        const int pos = w0 + (kk - n_c);
        src = reinterpret_cast<const uint8_t*>(a.ring_kv + ((int64_t)brow * a.R + pos % a.R) * kKv +
                                               sg * 64 + sp * 32);
        kind = 3;
      }
    }
    const uint4* s0 = reinterpret_cast<const uint4*>(src);
    const uint4* s1 = kind == 1 ? s0 : s0 + 2;
#pragma unroll
    for (int v = 0; v < 2; v++) st.d[v] = s0[v];
#pragma unroll
    for (int v = 0; v < 2; v++) st.d[2 + v] = s1[v];
    st.s = *scp;
    st.kind = kind;
  };
  // Convert the loaded slot into the LDS tile, one fp16 image per key that
  // serves as K and as V: an FP8 code's value exactly (e4m3 values are fp16
  // numbers), a bf16 RoPE or window value exactly when it lies in fp16's
  // normal range; then the group scale and the key mask.
  auto stage_store = [&](const StageRegs& st, int sg, int buf) {
    uint4* tdst = reinterpret_cast<uint4*>(Ts[buf] + sj * kVst + sg * 64 + sp * 32);
    uint32_t gmx = 0;
    if (st.kind == 1) {
      range_ok &= st.s == 0.0f || (st.s >= 6.103515625e-05f && st.s < 256.0f);   // [2^-14, 2^8)
#pragma unroll
      for (int v = 0; v < 2; v++) {
        const uint32_t w4[4] = {st.d[v].x, st.d[v].y, st.d[v].z, st.d[v].w};
        uint32_t hb[8];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            // two codes -> exact fp32 (OCP e4m3 on gfx950) -> exact fp16
            const v2f f = hh ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[q4], true)
                             : __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[q4], false);
            hb[q4 * 2 + hh] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
          }
        }
        tdst[2 * v] = make_uint4(hb[0], hb[1], hb[2], hb[3]);
        tdst[2 * v + 1] = make_uint4(hb[4], hb[5], hb[6], hb[7]);
      }
    } else if (st.kind >= 2) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const v8h h = bf16x8_to_f16(st.d[v]);
        gmx = bf16x8_absmax(st.d[v], gmx);
        tdst[v] = __builtin_bit_cast(uint4, h);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; v++) tdst[v] = make_uint4(0, 0, 0, 0);
    }
    // this lane holds half of a 64-channel group, lane l ^ 32 the other half;
    // a small group is reported by a lane whose half is nonzero (every lane
    // of the wavefront is here, and rarely any lane's half is small)
    range_ok &= gmx < kBf16F16Overflow;
    const bool small = gmx != 0 && gmx < kBf16MinNormalF16;
    if (__builtin_amdgcn_ballot_w64(small)) {
      const uint32_t other = __float_as_uint(swap_halves(__uint_as_float(gmx)));
      range_ok &= !(small && other < kBf16MinNormalF16);
    }
    if (sp == 0) sK[buf][sg * kTile + sj] = st.kind == 1 ? st.s : (st.kind ? 1.0f : 0.0f);
    // a key is valid when its first group is (every group of a key shares it)
    if (sg == 0 && sp == 0) kbias[buf][sj] = st.kind ? 0.0f : -INFINITY;
  };

  // LDS transpose-read addresses of the V^T operand: k-slot j of quarter g is
  // key 4g + j (j < 4) or 16 + 4g + (j - 4).  ds_read_b64_tr_b16 gives lane i
  // of a 16-lane group element i % 4 of the 64-bit rows read by lanes
  // 4j + i / 4, so lane L reads channels 16 ct + 4(L % 4) .. +3 of key
  // 4g + L / 4 (and of key 16 + 4g + L / 4 for the second read).
  const int Lq = lane & 15;
  const int voff = (4 * g + (Lq >> 2)) * kVst + 4 * (Lq & 3);
  const int koff = Lq * kVst + kq;

  // Staging wavefronts: while the compute wavefronts work on tile t they
  // store tile t + 1 (loaded a tile earlier) into the other buffer and load
  // tile t + 2, groups sw and sw + 4.  Every wavefront passes the same
  // barrier before the first tile and once per tile.
  // (Two separate loops, so that the staging registers and the compute
  // registers are never live at once.)
  if (!computes) {
    StageRegs stA, stB;
    if (kb < ke) {
      stage_load(kb, sw, stA);
      stage_load(kb, sw + 4, stB);
    }
    // Pass j stores tile j (loaded one pass earlier) into buffer j % 2, loads
    // tile j + 1 and meets the compute wavefronts' barrier: the one before
    // their first tile (j = 0), then the one after tile j - 1.  One copy of
    // the staging code serves every tile (a launch fetches its code cold).
    int buf = 0;
    for (int t0 = kb;; t0 += kTile, buf ^= 1) {
      if (t0 < ke) {
        stage_store(stA, sw, buf);
        stage_store(stB, sw + 4, buf);
        if (t0 + kTile < ke) {
          stage_load(t0 + kTile, sw, stA);
          stage_load(t0 + kTile, sw + 4, stB);
        }
      }
      __syncthreads();                     // tile j staged, tile j - 1 consumed
      if (t0 >= ke) break;
    }
    if (__any(!range_ok) && lane == 0) atomicOr(a.status, LCA_STATUS_FP16_RANGE);
    if (__any(!page_ok) && lane == 0) atomicOr(a.status, LCA_STATUS_PAGE);
    return;
  }
  // the query's fp16 image, and its range over the head's four lanes l,
  // l ^ 16, l ^ 32, l ^ 48
  v8h qf[16];
  {
    uint32_t qmx = 0;
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
      qf[ks] = bf16x8_to_f16(qraw[ks]);
      qmx = bf16x8_absmax(qraw[ks], qmx);
    }
    qmx = max(qmx, __float_as_uint(swap_rows(__uint_as_float(qmx))));
    qmx = max(qmx, __float_as_uint(swap_halves(__uint_as_float(qmx))));
    range_ok = qmx == 0 || (qmx >= kBf16MinNormalF16 && qmx < kBf16F16Overflow);
  }
  __syncthreads();                         // tile 0 staged
  int cur = 0;
  for (int t0 = kb; t0 < ke; t0 += kTile, cur ^= 1) {
    const _Float16* Kc = Ts[cur] + koff;
    const _Float16* vrow0 = Ts[cur] + voff;
    const _Float16* vrow1 = vrow0 + 16 * kVst;

    // S^T = K Q^T over the 512 channels, 32 keys x 16 heads, per 64-dim
    // group scaled in fp32
    // (groups outer, the two key tiles inner: two independent product
    // chains side by side)
    v4f S[2];
    S[0] = S[1] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gl = 0; gl < 8; gl++) {
#pragma unroll
      for (int nt = 0; nt < 2; nt++) {
        const _Float16* krow = Kc + nt * 16 * kVst;
        v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
          const int ks = 2 * gl + s2;
          const v8h kh8 = *reinterpret_cast<const v8h*>(krow + ks * 32);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh8, qf[ks], acc, 0, 0, 0);
        }
        const v4f sc = *reinterpret_cast<const v4f*>(sK[cur] + gl * kTile + nt * 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; r++) S[nt][r] = __builtin_fmaf(sc[r], acc[r], S[nt][r]);
      }
    }
    // online softmax (base 2) of this lane's head over its eight keys
    const v4f kb0 = *reinterpret_cast<const v4f*>(kbias[cur] + 4 * g);
    const v4f kb1 = *reinterpret_cast<const v4f*>(kbias[cur] + 16 + 4 * g);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      x[r] = S[0][r] * a.scale_log2 + kb0[r];
      x[4 + r] = S[1][r] * a.scale_log2 + kb1[r];
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; j++) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, swap_rows(mx));
    mx = fmaxf(mx, swap_halves(mx));
    // move the reference only when the tile's maximum exceeds it by more
    // than the headroom (always on the first key seen)
    if (__any(mx > mrow + kLazyMax)) {
      const float mnew = fmaxf(mrow, mx);
      // first key seen: 0 (O and l are still 0); unchanged reference: 1
      const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int c = 0; c < 32; c++)
#pragma unroll
        for (int r = 0; r < 4; r++) O[c][r] *= alpha;
      mrow = mnew;
    }
    const float mref = mrow == -INFINITY ? 0.0f : mrow;          // no key seen yet
    float pj[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      pj[j] = __builtin_amdgcn_exp2f(x[j] - mref);
      lrow += pj[j];
    }
    // O^T += V^T P^T over the 32 channel tiles.  The tile holds code values,
    // so each 64-dim group's FP8 scale goes into P: B operand of group gl =
    // fp16(p_j * scale of key j's group), for the group's four channel tiles.
    // Software-pipelined by hand: the transpose reads of tile c + 2 and the
    // scales of the next group go out before the product of tile c, so each
    // product waits only for reads issued two steps earlier (LDS reads
    // complete in order); scheduling barriers keep that order.
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    auto tr_pair = [&](int c, v4s& lo, v4s& hi) {
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vrow0 + 16 * c));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vrow1 + 16 * c));
    };
    auto scales = [&](int gl, v4f& s0, v4f& s1) {
      const float* sg0 = sK[cur] + gl * kTile + 4 * g;
      s0 = *reinterpret_cast<const v4f*>(sg0);
      s1 = *reinterpret_cast<const v4f*>(sg0 + 16);
    };
    constexpr int kTrDepth = 2;        // channel tiles of transpose reads in flight
    v4s lo_r[kTrDepth], hi_r[kTrDepth];
    v4f s0, s1;
    scales(0, s0, s1);
#pragma unroll
    for (int d = 0; d < kTrDepth; d++) tr_pair(d, lo_r[d], hi_r[d]);
    v8h pb;
#pragma unroll
    for (int c = 0; c < 32; c++) {
      if ((c & 3) == 0) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
          pb[r] = (_Float16)__fmul_rn(pj[r], s0[r]);
          pb[4 + r] = (_Float16)__fmul_rn(pj[4 + r], s1[r]);
        }
      }
      if ((c & 3) == 2 && c + 2 < 32) scales((c + 2) >> 2, s0, s1);
      v4s lo_n, hi_n;
      if (c + kTrDepth < 32) tr_pair(c + kTrDepth, lo_n, hi_n);
      __builtin_amdgcn_sched_barrier(0);
      const v4h lo_h = __builtin_bit_cast(v4h, lo_r[c % kTrDepth]), hi_h = __builtin_bit_cast(v4h, hi_r[c % kTrDepth]);
      const v8h va = {lo_h[0], lo_h[1], lo_h[2], lo_h[3], hi_h[0], hi_h[1], hi_h[2], hi_h[3]};
      O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, O[c], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (c + kTrDepth < 32) {
        lo_r[c % kTrDepth] = lo_n;
        hi_r[c % kTrDepth] = hi_n;
      }
    }
    __syncthreads();                       // tile t + 1 staged, tile t consumed
  }

  if (__any(!range_ok) && lane == 0) atomicOr(a.status, LCA_STATUS_FP16_RANGE);
  if (!active) return;
  lrow += swap_rows(lrow);
  lrow += swap_halves(lrow);
  if (a.splits == 1) {
    if (hq < a.H) {
      const float inv = 1.0f / lrow;
      float4* dst = reinterpret_cast<float4*>(a.out + ((int64_t)srow * a.H + hq) * kKv + 4 * g);
#pragma unroll
      for (int c = 0; c < 32; c++)
        dst[c * 4] = make_float4(O[c][0] * inv, O[c][1] * inv, O[c][2] * inv, O[c][3] * inv);
    }
  } else {
    // partials: (m, l) per head, and this lane's normalised outputs in fp16:
    // value index ct * 4 + r of the head's 128 per lane, as 16 uint4 per lane
    // interleaved across the wave
    if (hq < a.H && g == 0) {
      const int64_t slot = ((int64_t)srow * a.splits + split) * a.H + hq;
      reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(mrow, lrow);
    }
    const float inv = lrow > 0.0f ? 1.0f / lrow : 0.0f;
    const int64_t rec = ((int64_t)srow * a.splits + split) * a.hwaves + (hgrp * 4 + hw);
    uint4* dst = reinterpret_cast<uint4*>(a.ws_o + rec * 8192) + lane;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i0 = q * 8 + 2 * e;   // values i0, i0 + 1: (c, r) = (i0 / 4, i0 % 4)
        const v2f f = {O[i0 >> 2][i0 & 3] * inv, O[(i0 + 1) >> 2][(i0 + 1) & 3] * inv};
        w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2h));
      }
      dst[q * 64] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

struct CombineArgs {
  int H, splits, hwaves;
  const float* ws_ml;
  const _Float16* ws_o;
  float* out;
};

// Grid (row, wavefront of 16 heads, quarter): thread (q, lane) merges uint4 q
// of the record that `lane` of every split wrote -- 8 values of head
// hw * 16 + lane % 16, channels 16(2q + j / 4) + 4(lane / 16) + j % 4 -- with
// an online rescale over batches of eight splits.
__global__ void __launch_bounds__(256) attend_combine_kernel(CombineArgs a) {
  const int srow = blockIdx.x, hw = blockIdx.y;
  const int lane = threadIdx.x & 63, q = blockIdx.z * 4 + (threadIdx.x >> 6);
  const int h = hw * 16 + (lane & 15), g = lane >> 4;
  if (h >= a.H) return;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (int64_t)srow * a.splits * a.H + h;
  const uint4* rec0 = reinterpret_cast<const uint4*>(a.ws_o) + (int64_t)srow * a.splits * a.hwaves * 1024 +
                      (int64_t)hw * 1024 + q * 64 + lane;
  const int64_t rstride = (int64_t)a.hwaves * 1024;
  float M = -INFINITY, L = 0.0f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = 0.0f;
  for (int s0 = 0; s0 < a.splits; s0 += 8) {
    float2 mlu[8];
    uint4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int s = s0 + u;
      mlu[u] = make_float2(-INFINITY, 0.0f);
      raw[u] = make_uint4(0, 0, 0, 0);
      if (s < a.splits) {
        mlu[u] = ml[(int64_t)s * a.H];
        raw[u] = rec0[s * rstride];
      }
    }
    float bm = M;
#pragma unroll
    for (int u = 0; u < 8; u++)
      if (mlu[u].y > 0.0f) bm = fmaxf(bm, mlu[u].x);
    if (bm == -INFINITY) continue;             // no split of this batch saw a key
    const float c = __builtin_amdgcn_exp2f(M - bm);   // M = -inf -> 0
    L *= c;
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] *= c;
    M = bm;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const float w = mlu[u].y > 0.0f ? mlu[u].y * __builtin_amdgcn_exp2f(mlu[u].x - M) : 0.0f;
      L += w;
      const uint32_t ww[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const v2h v = __builtin_bit_cast(v2h, ww[e]);
        acc[2 * e] += w * (float)v[0];
        acc[2 * e + 1] += w * (float)v[1];
      }
    }
  }
  const float inv = 1.0f / L;
  float* dst = a.out + ((int64_t)srow * a.H + h) * kKv + 32 * q + 4 * g;
  *reinterpret_cast<float4*>(dst) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<float4*>(dst + 16) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
}

AttendPlan plan_attend(const lca_layer* L, int n_q, int H, int k, bool csa) {
  AttendPlan pl;
  const int64_t nvmax = L->len_max / L->ratio;
  pl.max_keys = (csa ? (int64_t)k : nvmax) + L->window;
  pl.head_groups = (H + 63) / 64;
  const int64_t rows = (int64_t)L->batch * n_q;
  const int64_t max_tiles = (pl.max_keys + kTile - 1) / kTile;
  int64_t s = (kAttendTargetWGs + rows * pl.head_groups - 1) / (rows * pl.head_groups);
  const int forced = tuning(kTuneAttendSplits);
  if (forced > 0) s = forced;
  if (s > max_tiles) s = max_tiles;
  if (s < 1) s = 1;
  int64_t per = (pl.max_keys + s - 1) / s;
  if (csa && per > kMaxChunk) per = kMaxChunk;
  // paged HCA: a split's pages (at most per / PB + 2) fit the LDS list
  if (!csa && L->page_blocks > 0 && per > (int64_t)(kMaxChunk - 2) * L->page_blocks)
    per = (int64_t)(kMaxChunk - 2) * L->page_blocks;
  pl.chunk = (int)(((per + kTile - 1) / kTile) * kTile);
  pl.splits = (int)((pl.max_keys + pl.chunk - 1) / pl.chunk);
  if (pl.splits > 1) {
    pl.ml_bytes = (size_t)rows * pl.splits * H * 2 * sizeof(float);
    // one 128-value fp16 record per lane of every (split, wavefront of 16 heads)
    pl.o_bytes = (size_t)rows * pl.splits * (pl.head_groups * 4) * 8192 * sizeof(_Float16);
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
  a.hwaves = pl.head_groups * 4;
  a.max_blocks = L->max_blocks;
  a.pm = page_map_of<PageMap>(L);
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
  a.status = L->sync + 1;
  const int rows = L->batch * n_q;
  {
    TimedLaunch t(kKernelAttend, stream);
    const dim3 g(pl.splits, rows, pl.head_groups), b(kThreads);
    const bool paged = a.pm.shift >= 0;
    if (a.csa && paged)
      hipLaunchKernelGGL((attend_kernel<true, true>), g, b, 0, stream, a);
    else if (a.csa)
      hipLaunchKernelGGL((attend_kernel<true, false>), g, b, 0, stream, a);
    else if (paged)
      hipLaunchKernelGGL((attend_kernel<false, true>), g, b, 0, stream, a);
    else
      hipLaunchKernelGGL((attend_kernel<false, false>), g, b, 0, stream, a);
    int rc = t.done();
    if (rc) return rc;
  }
  if (pl.splits > 1) {
    CombineArgs c;
    c.H = H;
    c.splits = pl.splits;
    c.hwaves = a.hwaves;   // record stride: every wavefront slot of the attention grid
    c.ws_ml = a.ws_ml;
    c.ws_o = a.ws_o;
    c.out = out;
    TimedLaunch t(kKernelAttendCombine, stream);
    hipLaunchKernelGGL(attend_combine_kernel, dim3(rows, (H + 15) / 16, 4), dim3(256), 0, stream, c);
    return t.done();
  }
  return LCA_OK;
}

}  // namespace lca
