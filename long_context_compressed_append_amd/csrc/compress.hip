// compress.hip -- ring append + block finalisation (softmax-gated pooling and
// FP8 / BF16 / MXFP4 quantisation) in one launch.
//
// vibecoco.ai "DeepSeek V4 agent architecture" page, section 混合注意力:
// KV entries are compressed along the sequence by softmax-gated pooling with a
// learned position bias (4x for CSA, 128x for HCA), stored in FP8 with BF16
// RoPE dims; the indexer keys are FP4.  pnsm.cn "DeepSeek V4 架构深度解析"
// page, section 2.1: the window store keeps raw tokens and overwrites
// cyclically.
//
// Work decomposition: every wavefront takes one task.
//   ring task      (row, token)        copies the raw token into slot pos % R
//   finalise task  (row, block, group) pools one 64-channel group of one
//                  newly completed block: lane = channel.  Groups 0..6 are
//                  the FP8 groups (wave-wide amax), group 7 the BF16 RoPE dims,
//                  group 8 the indexer stream (two 32-lane MXFP4 blocks).
// Finalise tasks read the tokens of the current call from the inputs and the
// older tokens of a straddling block from the ring; ring tasks only write
// slots of the current call's tokens, which never alias those older tokens
// while R >= n + m - 1.  The last workgroup to finish advances seq_len.
#include "compress_ops.h"

namespace lca {

__global__ void __launch_bounds__(256) compress_kernel(CompressArgs a) {
  // per-wavefront LDS slices of 64 x m floats for blocks of m >= 16 tokens
  // (dynamic shared memory, sized at launch; empty for shorter blocks)
  extern __shared__ float pool_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* lds = pool_lds + (a.m > 8 ? wave * 64 * a.m : 0);
  const int64_t task = (int64_t)blockIdx.x * 4 + wave;
  if (task < a.ring_tasks) {
    const int row = (int)(task / a.n);
    ring_copy(a, row, (int)(task % a.n), a.seq_len[row], lane);
  } else if (task < a.total_tasks) {
    int64_t f = task - a.ring_tasks;
    const int g = (int)(f % a.groups);
    f /= a.groups;
    const int s = (int)(f % a.nfin);
    const int row = (int)(f / a.nfin);
    const int L0 = a.seq_len[row];
    const int64_t bk = (int64_t)(L0 / a.m) + s;
    const bool completes = (bk + 1) * a.m <= (int64_t)L0 + a.n;
    // (row and block are uniform over the wavefront: so is every branch here)
    const int64_t e = completes && bk < a.max_blocks ? entry_index(a.pm, row, bk) : -1;
    if (completes && bk >= a.max_blocks) {           // past the cache (a replay beyond its plan)
      if (lane == 0) atomicOr(a.sync + 1, LCA_STATUS_COMPRESS_CAPACITY);
    } else if (completes && e < 0) {                 // its page is not mapped
      if (lane == 0) atomicOr(a.sync + 1, LCA_STATUS_PAGE);
    } else if (completes) {                          // block completes in this call
      finalize_group(a, row, bk, L0, g, e, lds, lane, nullptr);
    }
  }
  // The last workgroup to finish advances every row's length.  The barrier
  // completes every load of this workgroup (seq_len included) before its
  // counter increment, so no workgroup reads a length after it was advanced.
  // Nothing else written here is read by another workgroup of this launch,
  // so no memory fence is needed (a device-scope fence would write back and
  // invalidate a whole L2); the next launch sees every write.
  __shared__ uint32_t is_last;
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(a.sync, 1u) == gridDim.x - 1;
  __syncthreads();
  if (is_last) {
    for (int r = threadIdx.x; r < a.B; r += blockDim.x) a.seq_len[r] += a.n;
    if (threadIdx.x == 0) atomicExch(a.sync, 0u);
  }
}

int launch_compress(const lca_layer* L, const uint16_t* kv, const float* gate, const float* ikey,
                    const float* igate, int n, hipStream_t stream) {
  CompressArgs a = compress_args(L, kv, gate, ikey, igate, n);
  int64_t blocks = (a.total_tasks + 3) / 4;
  if (blocks > 0x7FFFFFFF) return LCA_EUNSUPPORTED;
  TimedLaunch t(kKernelCompress, stream);
  const size_t lds_bytes = a.m > 8 ? (size_t)4 * 64 * a.m * sizeof(float) : 0;   // <= 128 KB
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)blocks), dim3(256), lds_bytes, stream, a);
  return t.done();
}

}  // namespace lca
