// peak.hip -- measured ceilings of the chip, for the benchmark's roofline
// denominators (libpeak.so, separate from the library's ABI).
//
// Matrix cores: every wavefront runs `iters` rounds of kChains independent
// accumulator chains of one matrix instruction with register operands and no
// memory traffic, so with several wavefronts per SIMD the issue rate of that
// instruction is the only limit:
//   kind 0  v_mfma_f32_32x32x16_f16            2*32*32*16 = 32768 flops
//   kind 1  v_mfma_scale_f32_32x32x64_f8f6f4   fp8 e4m3 operands, 131072 flops
//   kind 2  v_mfma_scale_f32_32x32x64_f8f6f4   fp4 e2m1 operands, 131072 flops
// HBM: a grid-stride copy and a grid-stride read of 16-byte words over
// buffers far larger than the 256 MB Infinity Cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;

template <int kKind>
__global__ void __launch_bounds__(256) mfma_peak_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  v16f_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; c++) acc[c] = (v16f_t){};
  // small operands that depend on the lane (no constant folding): sums stay
  // far from overflow over any number of rounds used here
  const _Float16 h = (_Float16)(0.0009765625f * (float)(lane & 3));
  const v8h_t a16 = {h, h, h, h, h, h, h, h};
  const int w8 = 0x08080808 * (lane & 1);       // e4m3 2^-6 bytes, or zeros
  const int w4 = 0x11111111 * (lane & 1);       // e2m1 0.5 nibbles, or zeros
  const v8i_t a8 = {w8, w8, w8, w8, w8, w8, w8, w8};
  const v8i_t a4 = {w4, w4, w4, w4, 0, 0, 0, 0};
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int c = 0; c < kChains; c++) {
      if (kKind == 0) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a16, a16, acc[c], 0, 0, 0);
      if (kKind == 1) acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, acc[c], 0, 0, 0, 127, 0, 127);
      if (kKind == 2) acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a4, a4, acc[c], 4, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; c++)
#pragma unroll
    for (int e = 0; e < 16; e++) s += acc[c][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride loops with four independent 16-byte accesses in flight per
// thread (then a tail of single ones).
__global__ void __launch_bounds__(256) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) read_kernel(const uint4* __restrict__ src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// Matrix-instruction rounds: `blocks` workgroups of 256 threads, `iters`
// rounds of 4 instructions per wavefront; out holds blocks * 256 floats.
// Returns 0, or -1 on a bad argument, -5 when the launch failed.
int peak_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !out || kind < 0 || kind > 2) return -1;
  if (kind == 0) hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(256), 0, stream, out, iters);
  if (kind == 1) hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(256), 0, stream, out, iters);
  if (kind == 2) hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Copy of `bytes` (a multiple of 16, both pointers 16-byte aligned).
int peak_copy(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || bytes < 16 || (bytes & 15) || blocks < 1) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Read of `bytes` (a multiple of 16); out holds blocks * 256 words.
int peak_read(const void* src, int64_t bytes, int blocks, uint32_t* out, hipStream_t stream) {
  if (!src || !out || bytes < 16 || (bytes & 15) || blocks < 1) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint4*>(src), bytes / 16,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
