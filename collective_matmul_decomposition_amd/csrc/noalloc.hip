// cm_gemm_rs_noalloc: cm_gemm_rs with its workspace in a static device array,
// for callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "collmm.h"
#include "internal.h"

// One array per GPU, allocated by the runtime when the library's code object
// is loaded on that GPU and held until the process ends.  On the host the name
// stands for the device symbol, not for an address: host code uses only the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[CM_NOALLOC_WS_BYTES];

namespace {

// Device address of `scratch` on device `dev` (the current device), looked up
// once per device.
cm_status scratch_address(int dev, char **out) {
  static std::mutex mu;
  static std::unordered_map<int, char *> addr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      collmm::set_error("hipGetSymbolAddress (the static workspace): %s", hipGetErrorString(e));
      return CM_ERR_HIP;
    }
    it = addr.emplace(dev, static_cast<char *>(ptr)).first;
  }
  *out = it->second;
  return CM_OK;
}

}  // namespace

extern "C" cm_status cm_gemm_rs_noalloc(const cm_plan *plan, const void *x, const void *w, void *y, void *compute,
                                        void *const *comm, int n_comm) {
  if (!plan) {
    collmm::set_error("null plan");
    return CM_ERR_INVALID_ARG;
  }
  if (plan->ws_bytes > CM_NOALLOC_WS_BYTES) {
    collmm::set_error("cm_gemm_rs_noalloc: the plan needs a workspace of %zu bytes; the static one holds %zu",
                      plan->ws_bytes, (size_t)CM_NOALLOC_WS_BYTES);
    return CM_ERR_WORKSPACE;
  }
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    collmm::set_error("hipGetDevice: %s", hipGetErrorString(e));
    return CM_ERR_HIP;
  }
  char *ws = nullptr;
  const cm_status st = scratch_address(dev, &ws);
  if (st != CM_OK) return st;
  // The program is enqueued op by op: instantiating a graph may allocate
  // device memory.
  cm_plan eager = *plan;
  eager.desc.exec_mode = CM_EXEC_EAGER;
  return cm_gemm_rs(&eager, x, w, y, ws, CM_NOALLOC_WS_BYTES, compute, comm, n_comm, nullptr);
}
