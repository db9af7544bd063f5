// mfma_ceiling.hip -- a measurement program, not part of the library: the bf16
// matrix-core rate of this part with no data movement.  Every CU runs two workgroups
// of 8 waves; each wave keeps 16 accumulators of v_mfma_f32_16x16x32_bf16 (the
// projection's instruction) busy on operands held in registers (seeded pseudo-random
// bf16, so the multipliers switch as on real data), either each product into the next
// accumulator or in chains of 2 or 4 products into one.  The only memory access is one
// store of each lane's accumulators at the end, into a buffer sized for the grid.
// Prints one line per run: "mfma chain <c>: <ms> ms, <TFLOP/s> TFLOP/s".
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;

template <int CHAIN>
__global__ __launch_bounds__(kThreads) void mfma_probe(float* out, int iters, uint32_t seed) {
  bf16x8 a[4], b[4];
  uint32_t s = seed ^ (blockIdx.x * 977u + threadIdx.x * 131u);
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 8; ++e) {
      s = s * 1664525u + 1013904223u;
      a[i][e] = (__bf16)((float)((int)(s >> 9) - (1 << 22)) * (1.0f / (1 << 22)));
      s = s * 1664525u + 1013904223u;
      b[i][e] = (__bf16)((float)((int)(s >> 9) - (1 << 22)) * (1.0f / (1 << 22)));
    }
  f32x4 acc[16];
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    // 64 products per iteration: 16 accumulators x 4 k-steps
#pragma unroll
    for (int k0 = 0; k0 < 4; k0 += CHAIN)
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int k = k0; k < k0 + CHAIN; ++k)
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i >> 2) ^ k], b[(i & 3) ^ k], acc[i], 0, 0, 0);
  }
  float* o = out + ((size_t)blockIdx.x * kThreads + threadIdx.x) * 64;
  for (int i = 0; i < 16; ++i) *reinterpret_cast<f32x4*>(o + 4 * i) = acc[i];
}

template <int CHAIN>
static int run(float* out, int blocks, int iters) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL(mfma_probe<CHAIN>, dim3(blocks), dim3(kThreads), 0, 0, out, iters / 10, 1u);
  if (hipEventRecord(e0) != hipSuccess) return 1;
  hipLaunchKernelGGL(mfma_probe<CHAIN>, dim3(blocks), dim3(kThreads), 0, 0, out, iters, 7u);
  if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return 1;
  if (hipGetLastError() != hipSuccess) return 1;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
  const double flops = (double)blocks * (kThreads / 64) * iters * 64 * (2.0 * 16 * 16 * 32);
  printf("mfma chain %d: %.3f ms, %.1f TFLOP/s\n", CHAIN, ms, flops / (ms * 1e-3) / 1e12);
  fflush(stdout);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

int main() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 1;
  const int blocks = 2 * cus, iters = 20000;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * kThreads * 64 * sizeof(float)) != hipSuccess) return 1;
  int rc = 0;
  for (int r = 0; r < 3 && rc == 0; ++r) rc = run<1>(out, blocks, iters) | run<2>(out, blocks, iters) |
                                               run<4>(out, blocks, iters);
  (void)hipFree(out);
  return rc;
}
