// gate.hip -- sigmoid-gated residual add of the projected memory into the hc
// residual streams ([NeMo-V41] "nemo_automodel.components.models.deepseek_v41.
// model", forward contract: Engram writes into the streams before its layer;
// [vLLM-V41] "vllm/models/deepseek_v41/nvidia/model", DeepseekV4Model.forward:
// the gate of an image-span token is zeroed).  Included into engram_device.hip.
//
// One workgroup per token (256 or 512 threads).  Each thread holds CPT chunks of 8
// elements of v (fp32) and of each of the hc = 4 streams (bf16) in registers,
// so every byte is read once and written once: partial dot products per
// stream -> wave reduction (xor shuffles) -> cross-wave sum in LDS in a fixed
// order (deterministic) -> g = sigmoid(z) -> x + g v rounded once to bf16.
// A token with keep = 0 returns before touching its streams: they stay
// bit for bit.  After a split-K projection, v arrives as partial slices that
// are summed here in slice order (deterministic), optionally written out.

namespace engram {

typedef unsigned int g_u32x4 __attribute__((ext_vector_type(4)));
typedef float g_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHc = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(unsigned short, a) |
         ((uint32_t)__builtin_bit_cast(unsigned short, b) << 16);
}

template <int CPT, int THREADS>
__global__ __launch_bounds__(THREADS) void gate_add_kernel(GateArgs a) {
  const int t = blockIdx.x;
  const bool kept = a.keep == nullptr || a.keep[t] != 0;
  if (!kept && a.v_out == nullptr) return;  // uniform per workgroup
  const int tid = threadIdx.x;
  const int nchunks = a.hidden >> 3;
  const float* vrow = a.v + (int64_t)t * a.hidden;
  unsigned short* xrow = reinterpret_cast<unsigned short*>(a.streams) + (int64_t)t * kHc * a.hidden;

  float v[CPT][8];
  g_u32x4 x[kHc][CPT];
  float dot[kHc] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * THREADS;
    if (ch < nchunks) {
      // v and the stream rows are read once: nontemporal loads (5% faster at
      // 65,536 tokens than ordinary ones, measured)
      g_f32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const g_f32x4*>(vrow + ch * 8));
      g_f32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const g_f32x4*>(vrow + ch * 8 + 4));
      for (int sp = 1; sp < a.splits; ++sp) {  // split-K slices, summed in slice order
        const float* pr = vrow + (int64_t)sp * a.split_stride + ch * 8;
        v0 += *reinterpret_cast<const g_f32x4*>(pr);
        v1 += *reinterpret_cast<const g_f32x4*>(pr + 4);
      }
      if (a.v_out != nullptr) {
        float* vo = a.v_out + (int64_t)t * a.hidden + ch * 8;
        *reinterpret_cast<g_f32x4*>(vo) = v0;
        *reinterpret_cast<g_f32x4*>(vo + 4) = v1;
      }
      v[c][0] = v0[0]; v[c][1] = v0[1]; v[c][2] = v0[2]; v[c][3] = v0[3];
      v[c][4] = v1[0]; v[c][5] = v1[1]; v[c][6] = v1[2]; v[c][7] = v1[3];
#pragma unroll
      for (int s = 0; s < kHc; ++s)
        x[s][c] = __builtin_nontemporal_load(
            reinterpret_cast<const g_u32x4*>(xrow + (int64_t)s * a.hidden + ch * 8));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
#pragma unroll
      for (int s = 0; s < kHc; ++s) x[s][c] = g_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < kHc; ++s) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dot[s] = fmaf(bf16_lo(x[s][c][w]), v[c][2 * w], dot[s]);
        dot[s] = fmaf(bf16_hi(x[s][c][w]), v[c][2 * w + 1], dot[s]);
      }
    }
  }

  if (!kept) return;  // v_out written; the streams of a dead token stay bit for bit

  __shared__ float part[THREADS / 64][kHc];
#pragma unroll
  for (int s = 0; s < kHc; ++s) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot[s] += __shfl_xor(dot[s], off, 64);
  }
  if ((tid & 63) == 0) {
#pragma unroll
    for (int s = 0; s < kHc; ++s) part[tid >> 6][s] = dot[s];
  }
  __syncthreads();
  float g[kHc];
#pragma unroll
  for (int s = 0; s < kHc; ++s) {
    float z = part[0][s];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w) z += part[w][s];
    z *= a.inv_sqrt_hidden;
    g[s] = 1.0f / (1.0f + expf(-z));
  }

#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = tid + c * THREADS;
    if (ch >= nchunks) continue;
#pragma unroll
    for (int s = 0; s < kHc; ++s) {
      g_u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o[w] = pack_bf16(fmaf(g[s], v[c][2 * w], bf16_lo(x[s][c][w])),
                         fmaf(g[s], v[c][2 * w + 1], bf16_hi(x[s][c][w])));
      *reinterpret_cast<g_u32x4*>(xrow + (int64_t)s * a.hidden + ch * 8) = o;
    }
  }
}

hipError_t launch_gate_add(const GateArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  if (a.T == 0) return hipSuccess;
  const int nchunks = a.hidden / 8;
  const dim3 grid((unsigned)a.T);
  // one chunk of 8 elements per thread where the row allows it: 512 threads for
  // hidden 4,096 keeps the register count low enough for 8 waves per SIMD
  if (nchunks <= 256)
    hipLaunchKernelGGL((gate_add_kernel<1, 256>), grid, dim3(256), 0, stream, a);
  else if (nchunks <= 512)
    hipLaunchKernelGGL((gate_add_kernel<1, 512>), grid, dim3(512), 0, stream, a);
  else if (nchunks <= 1024)
    hipLaunchKernelGGL((gate_add_kernel<2, 512>), grid, dim3(512), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace engram
