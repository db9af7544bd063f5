// engram_device.hip -- the library's single device translation unit: the
// per-device status word and every kernel of the Engram hot path (gfx950).
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.h"

namespace engram {

// First device-detected status since the last engram_get_error() on this
// device (0 = none).  Written only with a vector-memory compare-and-swap.
__device__ int g_device_status;

__device__ __forceinline__ void latch_error(int status) { atomicCAS(&g_device_status, 0, status); }

// Raises a kernel's dynamic-LDS limit on the current device, once per device
// (bit d of `done` records device d; two threads that both see the bit clear both
// set the same value, which is harmless).
static hipError_t ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

hipError_t read_and_clear_device_error(hipStream_t stream, int* status) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_device_status), sizeof(int), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  if (v != 0) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_device_status), &zero, sizeof(int), 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
  }
  *status = v;
  return hipSuccess;
}

}  // namespace engram

#include "kernels/hash.hip"
#include "kernels/gather.hip"
#include "kernels/lookup.hip"
#include "kernels/gemm.hip"
#include "kernels/gemm_packed.hip"
#include "kernels/gemm_gather.hip"
#include "kernels/gate.hip"
