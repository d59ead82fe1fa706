// Allocation-free residual-add + RMSNorm backward: the parameter-gradient
// partial rows go to a library-held device array instead of a caller
// workspace, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation). The kernels are
// the ones fr_add_rmsnorm_bwd launches; they take the array's device address
// as their workspace argument.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends. In host code the
// name is a host-side stand-in, never a device address: its address on the
// current device is looked up once per device with hipGetSymbolAddress and
// only that pointer is used. Every call on a GPU shares that GPU's array;
// each call overwrites the partial rows it reads (nothing has to start at
// zero), and calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fr_kernels.hpp"

namespace fr {

static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The array's address on the current device (looked up on the first call
// made with that device current).
hipError_t scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_rmsnorm_bwd_noalloc(const RmsNormBwdVariant* v, const void* h, const void* dy,
                                      const void* dres, const void* w, void* dh, float* dweight,
                                      int64_t rows, int cols, float eps, hipStream_t s) {
  const int grid = bwd_grid(*v, rows);
  if ((int64_t)grid * cols * (int64_t)sizeof(float) > kNoallocScratchBytes)
    return hipErrorInvalidValue;  // the entry point rejects such calls first
  float* ws = nullptr;
  hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return e;
  e = v->launch(h, dy, dres, w, dh, ws, grid, rows, cols, eps, s);
  if (e != hipSuccess) return e;
  return launch_colsum(ws, grid, cols, dweight, nullptr, s);
}

}  // namespace fr
