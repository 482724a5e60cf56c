// lca_device.h -- device-side number formats and wave helpers for the gfx950
// kernels.  Private to liblca.so.
//
// Formats (fixed by the workload definitions and the OCP FP8 / MX documents):
//   bf16     upper half of binary32, round to nearest even;
//   e4m3fn   1/4/3 bits, bias 7, max 448, no infinities, saturating encode;
//   e2m1     1/2/1 bits, values 0, .5, 1, 1.5, 2, 3, 4, 6, saturating encode;
//   E8M0     2^(e-127) block exponent of an MX block of 32 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lca {

constexpr int kKv = 512;
constexpr int kNope = 448;
constexpr int kRope = 64;
constexpr int kIdx = 64;
constexpr int kScaleStride = 8;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (finite inputs; +-inf stay infinite).
__device__ __forceinline__ uint16_t f32_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// e4m3fn code -> fp32 value (exact).
__device__ __forceinline__ float e4m3_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// e4m3fn code -> bf16 bits of the same value (exact: 4 significant bits).
__device__ __forceinline__ uint32_t e4m3_bf16(uint32_t c) {
  return __float_as_uint(e4m3_f32(c)) >> 16;
}

// fp32 -> e4m3fn code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t f32_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                 // below the smallest normal 2^-6
    code = (uint32_t)rintf(a * 512.0f);       // multiples of 2^-9, ties to even
  } else {
    uint32_t ua = __float_as_uint(a);
    uint32_t e = (ua >> 23) - 127u + 7u;      // 1..15
    uint32_t mant = ua & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    code = (e << 3) + keep + up;              // a carry moves into the exponent
  }
  return sign | code;
}

// fp32 (already divided by the block scale) -> e2m1 code, RNE, saturating.
__device__ __forceinline__ uint32_t f32_e2m1(float x) {
  float a = fabsf(x);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return (__float_as_uint(x) >> 28 & 8u) | c;
}

// floor(log2(a)) for finite a > 0 (normal or subnormal), exact.
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)(u >> 23);
  if (e) return e - 127;
  return (31 - __clz((int)(u & 0x7FFFFFu))) - 149;
}

// Lane reductions on DPP moves (no LDS round trips).  A step combines each
// lane with the lane `ctrl` names; a lane whose source lies outside its row,
// or whose row is masked off, combines with itself.  Shifts by 1, 2, 4 and 8
// leave in lane 15 of every 16-lane row the reduction of the row; the
// broadcast of lane 15 into the next row (rows 1 and 3) then leaves that of
// lanes 0-31 in lane 31 and of lanes 32-63 in lane 63, and the broadcast of
// lane 31 into rows 2 and 3 that of the wave in lane 63.
constexpr int kDppRowShr = 0x110, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_max(float x) {
  const int xi = __float_as_int(x);
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, kCtrl, kRowMask, 0xf, false)));
}

template <int kOp, int kCtrl, int kRowMask>   // kOp 0: min, 1: max
__device__ __forceinline__ int dpp_minmax(int x) {
  const int y = __builtin_amdgcn_update_dpp(x, x, kCtrl, kRowMask, 0xf, false);
  return kOp ? max(x, y) : min(x, y);
}

__device__ __forceinline__ float row_max_steps(float v) {
  v = dpp_max<kDppRowShr + 1, 0xf>(v);
  v = dpp_max<kDppRowShr + 2, 0xf>(v);
  v = dpp_max<kDppRowShr + 4, 0xf>(v);
  v = dpp_max<kDppRowShr + 8, 0xf>(v);
  return dpp_max<kDppRowBcast15, 0xa>(v);
}

// max over the wave, in every lane
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<kDppRowBcast31, 0xc>(row_max_steps(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// max over the 32-lane half of the wave that the caller is in
__device__ __forceinline__ float half_wave_max(float v) {
  v = row_max_steps(v);
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (threadIdx.x & 32) ? hi : lo;
}

// max over the caller's aligned group of 8 lanes, in every lane of it: two
// quad permutations (lanes 1, 0, 3, 2, then 2, 3, 0, 1) give each lane its
// quad's maximum, the half-row mirror (lane i with lane 7 - i) joins the two
// quads
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141;
__device__ __forceinline__ float octet_max(float v) {
  v = dpp_max<kDppQuadXor1, 0xf>(v);
  v = dpp_max<kDppQuadXor2, 0xf>(v);
  return dpp_max<kDppRowHalfMirror, 0xf>(v);
}

// min (kOp 0) or max (kOp 1) over the wave, in every lane
template <int kOp>
__device__ __forceinline__ int wave_minmax(int v) {
  v = dpp_minmax<kOp, kDppRowShr + 1, 0xf>(v);
  v = dpp_minmax<kOp, kDppRowShr + 2, 0xf>(v);
  v = dpp_minmax<kOp, kDppRowShr + 4, 0xf>(v);
  v = dpp_minmax<kOp, kDppRowShr + 8, 0xf>(v);
  v = dpp_minmax<kOp, kDppRowBcast15, 0xa>(v);
  v = dpp_minmax<kOp, kDppRowBcast31, 0xc>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// the value of lane l ^ 32 (gfx950 permlane32 swap: a VALU op)
__device__ __forceinline__ float swap_halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// the value of lane l ^ 16 (gfx950 permlane16 swap: odd rows with even rows)
__device__ __forceinline__ float swap_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// the value of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2)
__device__ __forceinline__ uint32_t lane_xor1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xf, 0xf, false);
}

// eight bf16 values (uint4) as fp16: exact for values in fp16's normal
// range (bf16 keeps 8 significant bits, fp16 11)
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8h_t bf16x8_to_f16(uint4 w) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  v8h_t r;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const v2f_t f = {__uint_as_float(ww[i] << 16), __uint_as_float(ww[i] & 0xFFFF0000u)};
    const v2h_t h = __builtin_convertvector(f, v2h_t);
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// Largest magnitude of eight bf16 values w folded into mx, as bf16
// magnitude bits (ordered like the magnitudes; inf and NaN above every
// finite value).  fp16 holds a vector of bf16 values to 2^-11 of its largest
// magnitude when that lies in [2^-14, 65504]: values in fp16's normal range
// convert exactly, smaller ones lose at most 2^-25 to fp16's subnormal
// spacing 2^-24.
__device__ __forceinline__ uint32_t bf16x8_absmax(uint4 w, uint32_t mx) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; i++) mx = max(mx, max(ww[i] & 0x7FFFu, (ww[i] >> 16) & 0x7FFFu));
  return mx;
}
constexpr uint32_t kBf16F16Overflow = 0x4780u;    // 65536: the first bf16 magnitude above 65504
constexpr uint32_t kBf16MinNormalF16 = 0x3880u;   // 2^-14

// Where entry b of a row lives in the entry planes (nope, rope, kv_scale,
// idx_code, idx_scale).  Contiguous layers (shift < 0): row * max_blocks + b.
// Paged layers: the row's page-table entry for page b >> shift, times the
// page size, plus b's offset in its page; -1 when that page is unmapped
// (entry negative or not below pool_pages).
struct PageMap {
  const int32_t* table;     // [B][pages_per_row], null when contiguous
  int64_t max_blocks;
  int32_t pages_per_row;
  int32_t shift;            // log2(page_blocks), or -1
  int32_t pool_pages;
  int32_t pad;
};
__device__ __forceinline__ int64_t phys_entry(const PageMap& pm, int page, int64_t b) {
  return (uint32_t)page < (uint32_t)pm.pool_pages ? ((int64_t)page << pm.shift) + (b & ((1 << pm.shift) - 1))
                                                   : (int64_t)-1;
}
__device__ __forceinline__ int64_t entry_index(const PageMap& pm, int row, int64_t b) {
  if (pm.shift < 0) return (int64_t)row * pm.max_blocks + b;
  return phys_entry(pm, pm.table[(int64_t)row * pm.pages_per_row + (b >> pm.shift)], b);
}

__device__ __forceinline__ uint32_t ord_key(float s) {
  // negative: every bit flipped; otherwise the sign bit set (one xor with
  // the sign spread over the word, sign bit forced)
  const uint32_t u = __float_as_uint(s);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

}  // namespace lca
