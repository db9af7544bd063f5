// gather.hip -- row gather + row-wise dequant ([VeOmni#1370] "feat: support
// DeepSeek-V4.1-Flash in SeedOmni", PR summary: the FP8 rows are
// dequantised with their row scale when they are looked up).  Included into engram_device.hip.
//
// The output of one call is T token rows of k_pad elements, each the 3*H
// segments (order-major, then head) of seg_pitch elements; a segment holds the
// D dequantised elements of one looked-up table row followed by zeros.  The
// work is a flat list of 16-element output chunks (T * 3H * seg_pitch/16 of
// them).  Consecutive lanes take consecutive chunks, so one wave-wide 16-byte
// load reads 1 KB of consecutive table bytes (fp8).  A lane's 16 dequantised
// elements are 32 B of bf16; the wave stages its 2 KB of output in LDS and reads
// it back transposed, so each of its two wave-wide 16-byte stores writes 1 KB
// of consecutive output (whole cache lines; without the staging each store
// instruction would leave 16-byte holes and the memory system would write
// partial lines).  Each lane keeps UNROLL chunks in flight: two, or one for
// small calls (decode steps), which then spread over twice as many workgroups.
//
// Dequant of a chunk: 16 e4m3fn bytes -> 16 fp32 (hardware conversion,
// v_cvt_pk_f32_fp8), times the scale (one v_mul_f32 each: exactly the IEEE
// product), then round-to-nearest-even to bf16 (v_cvt_pk_bf16_f32) or kept as
// fp32.  The scale is the row's fp32 scale, or, for (1, 32)-blocked tables
// ([VeOmni#1370] per-row-scale commit: each row carries an exponent for every block of 32
// columns),
// the e8m0 byte b of the chunk's block as the float 2^(b-127) (b = 0 is the
// subnormal 2^-127, b = 255 NaN); a 16-element chunk never straddles a block.
// BF16 tables are copied (or widened to fp32).
//
// Several Engram sites share one row-id array [T][sites][3][H]; a call gathers
// one site's columns (row_ids points at them, tokens rid_ld ints apart).  A
// site's buckets live in three per-order tables or in one table for the site.

namespace engram {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 2;  // chunks in flight per lane (measured: 2 beats 4 and 8)
// below this many workgroups at kGatherUnroll, a call runs with one chunk per lane
constexpr uint64_t kGatherSmallBlocks = 512;

// q = n / d for 0 <= n < 2^31 via a 64-bit multiply: m = ceil(2^s / d) with
// s = 31 + ceil(log2 d) is exact on that range (round-up multiplier method).
struct FastDiv {
  uint64_t m;
  uint32_t s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

struct GatherKArgs {
  const uint8_t* t0;
  const uint8_t* t1;
  const uint8_t* t2;
  const void* s0;
  const void* s1;
  const void* s2;
  int32_t r0, r1, r2;  // rows per table
  const int32_t* row_ids;
  int32_t rid_extra;   // rid_ld - cols: extra ints between consecutive tokens' row ids
  uint32_t split;      // heads (per-order tables) or 2^30 (one table: every segment is n = 0)
  uint32_t nblk;       // e8m0 bytes per row (row_dim / 32)
  void* out;
  int64_t out_ld;
  int64_t pitch;
  uint32_t total;      // chunks
  uint32_t chunks;     // per segment = seg_pitch / 16
  uint32_t cols;       // 3 * heads
  uint32_t heads;
  uint32_t row_dim;
  uint32_t seg_pitch;
  FastDiv div_chunks;
  FastDiv div_cols;
  int32_t linear_out;  // out_ld == cols * seg_pitch: chunk g starts at element 16 g
};

__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(unsigned short, b);
}

__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : (b == 255 ? 0x7FC00000u : b << 23));
}

template <bool kBf16Table, bool kF32Out, bool kBlockScale, int UNROLL>
__global__ __launch_bounds__(kGatherThreads) void gather_dequant_kernel(GatherKArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Per-wave LDS staging for the bf16 path: a lane converts 16 elements (32 B),
  // the wave's 64 chunks (2 KB) go to LDS and come back transposed so that each
  // of the two wave-wide 16-byte stores writes 1 KB of consecutive output.
  __shared__ u32x4 stage[kGatherThreads / 64][2][128];
  const bool staged = !kF32Out && a.linear_out;
  // Grid-stride over blocks of kGatherThreads * UNROLL chunks: one block per
  // workgroup normally; a capped grid (tables in host memory) walks several.
  const uint32_t per_block = kGatherThreads * UNROLL;
  for (uint32_t base = blockIdx.x * per_block; base < a.total; base += gridDim.x * per_block) {
    const uint32_t first = base + threadIdx.x;

    u32x4 raw[UNROLL][kBf16Table ? 2 : 1];
    float scale[UNROLL];
    uint32_t tok[UNROLL], seg[UNROLL], chunk[UNROLL];
    bool live[UNROLL], any[UNROLL];

    // Issue every load first so that UNROLL row reads are in flight per lane.
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t g = first + (uint32_t)u * kGatherThreads;
      live[u] = g < a.total;
      any[u] = false;
      scale[u] = 1.0f;
#pragma unroll
      for (int h = 0; h < (kBf16Table ? 2 : 1); ++h) raw[u][h] = u32x4{0u, 0u, 0u, 0u};
      tok[u] = seg[u] = chunk[u] = 0;
      if (!live[u]) continue;
      const uint32_t rowidx = fdiv(g, a.div_chunks);  // token * cols + seg
      chunk[u] = g - rowidx * a.chunks;
      tok[u] = fdiv(rowidx, a.div_cols);
      seg[u] = rowidx - tok[u] * a.cols;
      const uint32_t n = (seg[u] >= a.split) + (seg[u] >= 2 * a.split);
      if (chunk[u] * 16 >= a.row_dim) continue;  // pure padding: zeros
      const int32_t row = a.row_ids[(int64_t)rowidx + (int64_t)tok[u] * a.rid_extra];
      const int32_t rows = n == 0 ? a.r0 : (n == 1 ? a.r1 : a.r2);
      if (row < 0 || row >= rows) {
        latch_error(ENGRAM_E_ROW_RANGE);
        continue;
      }
      const uint8_t* tb = n == 0 ? a.t0 : (n == 1 ? a.t1 : a.t2);
      const uint8_t* src = tb + (int64_t)row * a.pitch + (int64_t)chunk[u] * 16 * (kBf16Table ? 2 : 1);
      raw[u][0] = *reinterpret_cast<const u32x4*>(src);
      if (kBf16Table) {
        raw[u][kBf16Table ? 1 : 0] = *reinterpret_cast<const u32x4*>(src + 16);
      } else if (kBlockScale) {
        const uint8_t* sc = static_cast<const uint8_t*>(n == 0 ? a.s0 : (n == 1 ? a.s1 : a.s2));
        scale[u] = e8m0_value(sc[(int64_t)row * a.nblk + (chunk[u] >> 1)]);
      } else {
        const float* sc = static_cast<const float*>(n == 0 ? a.s0 : (n == 1 ? a.s1 : a.s2));
        scale[u] = sc[row];
      }
      any[u] = true;
    }

#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t e0 = chunk[u] * 16;
      const uint32_t valid = e0 >= a.row_dim ? 0u : (a.row_dim - e0 >= 16 ? 16u : a.row_dim - e0);
      const int64_t obase = (int64_t)tok[u] * a.out_ld + (int64_t)seg[u] * a.seg_pitch + e0;

      float f[16];
      if (kBf16Table) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const uint32_t word = raw[u][w >> 2][w & 3];
          f[2 * w] = __uint_as_float(word << 16);
          f[2 * w + 1] = __uint_as_float(word & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = raw[u][0][w];
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
          f[4 * w + 0] = lo[0] * scale[u];
          f[4 * w + 1] = lo[1] * scale[u];
          f[4 * w + 2] = hi[0] * scale[u];
          f[4 * w + 3] = hi[1] * scale[u];
        }
      }
      if (!any[u]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = 0.0f;
      } else if (valid < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((uint32_t)i >= valid) f[i] = 0.0f;
      }

      if (kF32Out) {
        if (!live[u]) continue;
        float* dst = reinterpret_cast<float*>(a.out) + obase;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst) + q);
        }
        continue;
      }
      u32x4 o[2];
      if (kBf16Table && any[u] && valid == 16) {
        o[0] = raw[u][0];
        o[1] = raw[u][kBf16Table ? 1 : 0];
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w)
          o[w >> 2][w & 3] = bf16_bits_rne(f[2 * w]) | (bf16_bits_rne(f[2 * w + 1]) << 16);
      }
      if (staged) {
        // chunk g sits at element 16 g of the output (rows are back to back), so the
        // wave's chunks g0..g0+63 are 2 KB of consecutive output
        u32x4* buf = stage[wave][u & 1];
        buf[2 * lane] = o[0];
        buf[2 * lane + 1] = o[1];
        const u32x4 s0 = buf[lane], s1 = buf[64 + lane];
        const uint32_t g0 = first - (uint32_t)lane + (uint32_t)u * kGatherThreads;
        unsigned short* dst = reinterpret_cast<unsigned short*>(a.out) + (int64_t)g0 * 16;
        if (g0 + (uint32_t)(lane >> 1) < a.total)
          __builtin_nontemporal_store(s0, reinterpret_cast<u32x4*>(dst) + lane);
        if (g0 + 32u + (uint32_t)(lane >> 1) < a.total)
          __builtin_nontemporal_store(s1, reinterpret_cast<u32x4*>(dst) + 64 + lane);
      } else if (live[u]) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(a.out) + obase;
        __builtin_nontemporal_store(o[0], reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(o[1], reinterpret_cast<u32x4*>(dst) + 1);
      }
    }
  }
}

static FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;  // ceil(log2 d)
  FastDiv f;
  f.s = 31 + l;
  f.m = (uint64_t)(((unsigned __int128)1 << f.s) + d - 1) / d;
  return f;
}

template <int UNROLL>
static void launch_gather_variant(const GatherArgs& g, const GatherKArgs& a, uint64_t total,
                                  hipStream_t stream) {
  const uint32_t per_block = kGatherThreads * UNROLL;
  uint64_t blocks = (total + per_block - 1) / per_block;
  if (g.max_blocks > 0 && blocks > (uint64_t)g.max_blocks) blocks = (uint64_t)g.max_blocks;
  const dim3 grid((unsigned)blocks);
  const dim3 block(kGatherThreads);
  if (g.bf16_table) {
    if (g.f32_out)
      hipLaunchKernelGGL((gather_dequant_kernel<true, true, false, UNROLL>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gather_dequant_kernel<true, false, false, UNROLL>), grid, block, 0, stream, a);
  } else if (g.scale_block == 32) {
    if (g.f32_out)
      hipLaunchKernelGGL((gather_dequant_kernel<false, true, true, UNROLL>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gather_dequant_kernel<false, false, true, UNROLL>), grid, block, 0, stream, a);
  } else {
    if (g.f32_out)
      hipLaunchKernelGGL((gather_dequant_kernel<false, true, false, UNROLL>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gather_dequant_kernel<false, false, false, UNROLL>), grid, block, 0, stream, a);
  }
}

hipError_t launch_gather_dequant(const GatherArgs& g, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  GatherKArgs a;
  a.t0 = g.table[0];
  a.t1 = g.table[1];
  a.t2 = g.table[2];
  a.s0 = g.scale[0];
  a.s1 = g.scale[1];
  a.s2 = g.scale[2];
  a.r0 = (int32_t)g.rows[0];
  a.r1 = (int32_t)g.rows[1];
  a.r2 = (int32_t)g.rows[2];
  a.row_ids = g.row_ids;
  a.rid_extra = g.rid_ld - g.cols;
  a.split = g.per_site_table ? (1u << 30) : (uint32_t)g.heads;
  a.nblk = (uint32_t)(g.row_dim / 32);
  a.out = g.out;
  a.out_ld = g.out_ld;
  a.pitch = g.pitch;
  a.chunks = (uint32_t)(g.seg_pitch / 16);
  a.linear_out = g.out_ld == (int64_t)g.cols * g.seg_pitch ? 1 : 0;
  a.cols = (uint32_t)g.cols;
  a.heads = (uint32_t)g.heads;
  a.row_dim = (uint32_t)g.row_dim;
  a.seg_pitch = (uint32_t)g.seg_pitch;
  const uint64_t total = (uint64_t)g.T * a.cols * a.chunks;
  if (total == 0) return hipSuccess;
  if (total >= (1ull << 31)) return hipErrorInvalidValue;  // host splits larger calls
  a.total = (uint32_t)total;
  a.div_chunks = make_fastdiv(a.chunks);
  a.div_cols = make_fastdiv(a.cols);
  const uint64_t blocks2 = (total + kGatherThreads * kGatherUnroll - 1) / (kGatherThreads * kGatherUnroll);
  if (g.max_blocks == 0 && blocks2 < kGatherSmallBlocks)
    launch_gather_variant<1>(g, a, total, stream);
  else
    launch_gather_variant<kGatherUnroll>(g, a, total, stream);
  return hipGetLastError();
}

}  // namespace engram
