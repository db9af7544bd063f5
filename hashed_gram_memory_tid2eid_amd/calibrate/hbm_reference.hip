// hbm_reference.hip -- a measurement program, not part of the library: what plain
// streaming kernels reach in HBM on this part, as references for the hot path's
// HBM-bound kernels.  Every workgroup of 256 threads moves one contiguous 4 KB block per
// operand in one pass (a grid of one workgroup per block, no grid-stride loop: on this
// part a grid-stride copy over 8,192 workgroups ran 20% slower), over buffers far
// larger than the caches:
//   read    2 GiB read (nontemporal 16-byte loads), nothing written;
//   write   2 GiB written, nothing read;
//   copy    2 GiB read, 2 GiB written;
//   expand  1 GiB read, 2 GiB written, each 4 KB read block to 8 KB of consecutive
//           output (the row gather's 1 : 2 ratio of fp8 bytes read to bf16 written);
//   gate    the gated residual's traffic at 65,536 tokens and hidden 4,096: per token
//           16 KB of fp32 read and 4 x 8 KB of bf16 read and written back in place, one
//           workgroup per token, with none of its arithmetic; each store waits only for
//           its own loads;
//   gate_phased  the same with a workgroup barrier after the loads (a read phase, then
//           a write phase per workgroup, as the gate's cross-wave sum imposes).
// Prints one line per run: "hbm <name>: <ms> ms, <GB/s> GB/s".
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

// one 16-byte chunk per thread, block b owning chunks [256 b, 256 b + 256)
__global__ __launch_bounds__(256) void read_kernel(const u32x4* p, u32x4* sink) {
  const u32x4 r = __builtin_nontemporal_load(p + blockIdx.x * 256L + threadIdx.x);
  if (r[0] == 0x9E3779B9u && r[1] == 0x7F4A7C15u) sink[0] = r;  // keeps the loads
}

__global__ __launch_bounds__(256) void write_kernel(u32x4* q) {
  q[blockIdx.x * 256L + threadIdx.x] = u32x4{blockIdx.x, threadIdx.x, 1u, 2u};
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* p, u32x4* q) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  q[i] = __builtin_nontemporal_load(p + i);
}

// block b reads chunks [256 b, +256) and writes output chunks [512 b, +512)
__global__ __launch_bounds__(256) void expand_kernel(const u32x4* p, u32x4* q) {
  const u32x4 a = __builtin_nontemporal_load(p + blockIdx.x * 256L + threadIdx.x);
  u32x4* out = q + blockIdx.x * 512L;
  out[threadIdx.x] = a;
  out[256 + threadIdx.x] = a ^ 0x5A5A5A5Au;
}

template <bool PHASED>
__global__ __launch_bounds__(512) void gate_kernel(const float* v, unsigned short* x, int hidden) {
  const int t = blockIdx.x, c = threadIdx.x;
  const bool active = c < (hidden >> 3);  // 512 chunks of 8 at hidden 4,096: every thread
  const float* vr = v + (long)t * hidden + c * 8;
  unsigned short* xr = x + (long)t * 4 * hidden + c * 8;
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
  u32x4 s[4] = {};
  if (active) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vr));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vr + 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + (long)k * hidden));
  }
  const unsigned int bit = __float_as_uint(a[0] + a[1] + a[2] + a[3] + b[0] + b[1] + b[2] + b[3]) & 1u;
  if (PHASED) {
    // a value that depends on every load of the lane goes into LDS before the barrier,
    // so all of the workgroup's loads land before any of its stores
    __shared__ unsigned int seen;
    if (c == 0) seen = 0u;
    __syncthreads();
    atomicOr(&seen, (s[0][0] ^ s[1][1] ^ s[2][2] ^ s[3][3] ^ bit) & 0x80000000u);
    __syncthreads();
    if (seen == 0x12345678u) return;  // never true (bit 31 only); keeps the value live
  }
  if (active)
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(xr + (long)k * hidden) = s[k] ^ bit;
}

int main() {
  const long gib = 1L << 30;
  const int T = 65536, H = 4096;
  u32x4 *a, *b, *sink;
  float* v;
  unsigned short* x;
  CHECK(hipMalloc(&a, 2 * gib));
  CHECK(hipMalloc(&b, 2 * gib));
  CHECK(hipMalloc(&sink, 16));
  CHECK(hipMalloc(&v, (size_t)T * H * 4));
  CHECK(hipMalloc(&x, (size_t)T * 4 * H * 2));
  CHECK(hipMemset(a, 0x3C, 2 * gib));
  CHECK(hipMemset(b, 0, 2 * gib));
  CHECK(hipMemset(v, 0, (size_t)T * H * 4));
  CHECK(hipMemset(x, 0x3F, (size_t)T * 4 * H * 2));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const int reps = 10;
  const dim3 block(256);
  auto time = [&](const char* name, double bytes, auto launch) {
    launch();
    CHECK(hipEventRecord(e0));
    for (int i = 0; i < reps; ++i) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipGetLastError());
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= reps;
    std::printf("hbm %s: %.4f ms, %.0f GB/s\n", name, ms, bytes / (ms * 1e6));
  };
  const unsigned blocks2g = (unsigned)(2 * gib / 4096), blocks1g = (unsigned)(gib / 4096);
  for (int run = 0; run < 3; ++run) {
    time("read", 2.0 * gib, [&] { hipLaunchKernelGGL(read_kernel, dim3(blocks2g), block, 0, 0, a, sink); });
    time("write", 2.0 * gib, [&] { hipLaunchKernelGGL(write_kernel, dim3(blocks2g), block, 0, 0, b); });
    time("copy", 4.0 * gib, [&] { hipLaunchKernelGGL(copy_kernel, dim3(blocks2g), block, 0, 0, a, b); });
    time("expand", 3.0 * gib, [&] { hipLaunchKernelGGL(expand_kernel, dim3(blocks1g), block, 0, 0, a, b); });
    time("gate", (double)T * H * (4 + 2 * 4 * 2), [&] { hipLaunchKernelGGL((gate_kernel<false>), dim3(T), dim3(512), 0, 0, v, x, H); });
    time("gate_phased", (double)T * H * (4 + 2 * 4 * 2), [&] { hipLaunchKernelGGL((gate_kernel<true>), dim3(T), dim3(512), 0, 0, v, x, H); });
  }
  CHECK(hipDeviceSynchronize());
  return 0;
}
