// noalloc.cpp -- engram_gated_residual_noalloc: the gated residual of
// engram_gated_residual for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).  Its scratch
// -- v [T][hidden] and, for the split-K plan, the slices [splits][T][hidden] --
// lives in one file-scope device array instead of caller or handle memory.
//
// In host code the array's name only stands in for the device symbol: the array's
// device address on a device comes from hipGetSymbolAddress, taken once per
// device with that device current and kept here; kernels get that address as an
// argument.  Each device holds its own copy of the array until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchFloats = ENGRAM_NOALLOC_SCRATCH_BYTES / sizeof(float);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchFloats];

std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's scratch array (looked up on first use).
int scratch_on_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return engram::hip_error_status(e);
  if (dev < 0 || dev >= kMaxDevices) return ENGRAM_E_UNSUPPORTED;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return engram::hip_error_status(e);
      p = static_cast<float*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ENGRAM_OK;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

extern "C" int engram_gated_residual_noalloc(const engram_layout* L, const void* d_rows,
                                             int64_t rows_ld, const engram_wkv* W, int32_t hc_mult,
                                             const uint8_t* d_keep, void* d_streams, int32_t T,
                                             hipStream_t stream) {
  int rc = engram::wkv_check(W, L, T);
  if (rc != ENGRAM_OK) return rc;
  if (T == 0) return ENGRAM_OK;
  if (!d_rows || !d_streams) return ENGRAM_E_ARG;
  // v first, the split-K slices after it on a 256-byte boundary; every element the
  // kernels read is written by this call before it is read, so nothing is cleared
  const engram_proj_plan p = engram::wkv_plan_for(W, T);
  const int64_t v_elems = round_up((int64_t)T * W->hidden, 64);
  const int64_t part_elems = p.kernel == ENGRAM_PROJ_SPLITK ? (int64_t)p.splits * T * W->hidden : 0;
  if (v_elems + part_elems > (int64_t)kScratchFloats) return ENGRAM_E_SCRATCH;
  float* base = nullptr;
  rc = scratch_on_current_device(&base);
  if (rc != ENGRAM_OK) return rc;
  float* d_v = base;
  float* d_partials = base + v_elems;
  rc = engram::wkv_project_to(L, d_rows, rows_ld, W, d_v, d_partials, T, stream);
  if (rc != ENGRAM_OK) return rc;
  return engram::wkv_gate_from(L, W, d_v, d_partials, hc_mult, d_keep, d_streams, T, stream);
}
