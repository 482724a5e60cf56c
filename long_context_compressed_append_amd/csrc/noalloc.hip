// noalloc.hip -- lca_indexer_topk_noalloc: the indexer's top-k with its
// workspace in a file-scope device array instead of caller memory, for
// callers that cannot allocate (code under HIP graph capture, serving loops
// that forbid hipMalloc).
//
// The array holds the histograms, score keys and selection lists of one
// call.  Each GPU the library runs on holds its own copy until the process
// ends; its address is looked up once per device (hipGetSymbolAddress, with
// that device current) and passed to the kernels as a pointer.  Every call
// on a GPU shares that copy, so calls that overlap on one GPU race; the
// counters and histograms are cleared by a fill kernel at the start of every
// call (a kernel, not a memset, so the call stays capturable).
#include <mutex>

#include "lca_device.h"
#include "lca_internal.h"

namespace lca {

static __device__ __align__(256) uint8_t scratch[LCA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// the scratch array's device address on the current device (looked up once)
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(LCA_EHIP, "hipGetDevice failed or device id out of range (%d)", dev);
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(LCA_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return LCA_OK;
}
}  // namespace

__global__ void __launch_bounds__(256) zero_fill_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace lca

using namespace lca;

extern "C" int lca_indexer_topk_noalloc(const lca_layer* L, const float* iq, const float* iw, int32_t n_q,
                                        int32_t H_I, int32_t k, int32_t* topk, hipStream_t stream) {
  // the same checks as lca_indexer_topk, then the scratch array as workspace
  if (!L) return set_error(LCA_EINVAL, "layer is NULL");
  if (n_q < 1 || L->batch < 1 || L->ratio < 1) return set_error(LCA_EINVAL, "invalid layer or n_q");
  const IndexerPlan pl = plan_indexer(L, n_q, H_I, k);
  const size_t need = pl.total();
  if (need > (size_t)LCA_NOALLOC_SCRATCH_BYTES)
    return set_error(LCA_EWORKSPACE, "the call needs %zu bytes of workspace; the static scratch holds %zu",
                     need, (size_t)LCA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  rc = indexer_validate(L, iq, iw, n_q, H_I, k, topk);
  if (rc) return rc;
  // counters and histograms start at zero: clear the first zero_bytes (a
  // multiple of 16)
  const int64_t n16 = (int64_t)(pl.zero_bytes / 16);
  const int blocks = (int)(n16 / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<uint4*>(ws), n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LCA_EHIP, "zero-fill launch failed: %s", hipGetErrorString(e));
  return launch_indexer(L, iq, iw, n_q, H_I, k, topk, ws, pl, stream);
}
