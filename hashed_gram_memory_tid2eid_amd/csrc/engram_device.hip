// engram_device.hip -- the library's single device translation unit: the
// per-device status word and every kernel of the Engram hot path (gfx950).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace engram {

// First device-detected status since the last engram_get_error() on this
// device (0 = none).  Written only with a vector-memory compare-and-swap.
__device__ int g_device_status;

__device__ __forceinline__ void latch_error(int status) { atomicCAS(&g_device_status, 0, status); }

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
#include "kernels/gemm.hip"
#include "kernels/gemm_gather.hip"
#include "kernels/gate.hip"
