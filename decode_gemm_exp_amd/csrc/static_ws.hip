// static_ws.hip -- the GEMM stage with its scratch memory in a static device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch of the GEMM stage is the split-K partial sums (and, for the
// register-fed kernel, the packed copy of x); uw_matmul_stage takes it from
// the caller's workspace.  Here it lives in `scratch`, one array per GPU that
// the library runs on, held until the process ends.  Its device address is
// looked up once per device with hipGetSymbolAddress on the first call made
// with that device current, and that address (never the array's host-side
// name) is what the kernels receive.  Every call on one GPU shares the array
// and it keeps the last call's contents; nothing in it has to start at zero
// (every partial slice is written in full before the reduction reads it, and
// the packed x before the kernel that reads it), but calls that overlap on
// one GPU race on it.
#include <mutex>

#include "uw_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[UW_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device.
uw_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return UW_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return UW_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return UW_OK;
}

}  // namespace

extern "C" uw_status uw_matmul_stage_static(const uw_matrix* m, uw_pipeline p, const void* prep_dev,
                                            const uint16_t* x_dev, int64_t batch, float* y_dev,
                                            const uw_kernel_cfg* cfg, void* stream) {
  void* ws = nullptr;
  const uw_status st = scratch_address(&ws);
  if (st != UW_OK) return st;
  size_t need = 0;
  return uw::matmul_stage_into(m, p, prep_dev, x_dev, batch, y_dev, ws, UW_STATIC_SCRATCH_BYTES, cfg,
                               static_cast<hipStream_t>(stream), &need);
}
