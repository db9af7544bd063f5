// gemm.hip -- the wkv down-projection v = E W^T on the CDNA4 matrix cores.
// Included into engram_device.hip.
//
// C[M][N] (fp32) = A[M][K] (bf16, row-major) * B[N][K]^T (bf16, row-major):
// both operands are K-contiguous, which is the layout the gathered token rows
// and the projection weight already have.  K is a multiple of 64 (k_pad).
//
// Tile: a 256-thread workgroup (4 waves, 2 x 2) owns a BM x BN block of C and
// walks K in steps of 64.  Each wave owns a (BM/2) x (BN/2) sub-block made of
// 32 x 32 tiles computed by v_mfma_f32_32x32x16_bf16 (gfx950): per lane 8 bf16
// of A (row lane%32, k 8*(lane/32)..+8) and 8 of B, 16 fp32 accumulators.
// Operand tiles are staged through LDS, double buffered: while the waves run
// the MFMAs on one K step, the next step's global loads are in flight in
// registers; they are written to the other LDS buffer before the single
// barrier of the step.  LDS rows are 64 elements (128 B) stored with an XOR
// swizzle of the 16-byte chunks (chunk ^ (row & 7)), so the 16-byte reads of
// 8 consecutive rows land on distinct banks.
//
// Tile order: workgroup ids are dealt round-robin to the 8 XCDs, each with its
// own L2.  The id is remapped so that each XCD gets a contiguous run of tiles,
// walked in groups of GROUP_M row blocks: the concurrently running workgroups
// of one XCD share A row blocks and B column blocks in that XCD's L2.

namespace engram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;  // K elements per step; 8 chunks of 16 B per LDS row

template <int BM, int BN>
struct GemmShape {
  static constexpr int WM = BM / 2;          // wave sub-block rows
  static constexpr int WN = BN / 2;          // wave sub-block cols
  static constexpr int TM = WM / 32;         // 32x32 tiles per wave, rows
  static constexpr int TN = WN / 32;         // 32x32 tiles per wave, cols
  static constexpr int A_LOADS = BM * 8 / kGemmThreads;  // 16-B chunks per thread
  static constexpr int B_LOADS = BN * 8 / kGemmThreads;
  static constexpr int LDS_ELEMS = (BM + BN) * kBK;      // one buffer
};

struct GemmKArgs {
  const __bf16* A;
  const __bf16* B;
  float* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

template <int BM, int BN>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_nt_kernel(GemmKArgs a) {
  using S = GemmShape<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds[];

  // ---- tile id: XCD-contiguous runs, then GROUP_M swizzle ------------------
  const int ntiles = a.tiles_m * a.tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) {
    const int per_xcd = ntiles >> 3;
    bid = (bid & 7) * per_xcd + (bid >> 3);
  }
  const int group = a.group_m * a.tiles_n;
  const int gid = bid / group;
  const int first_m = gid * a.group_m;
  const int gm = min(a.tiles_m - first_m, a.group_m);
  const int in_group = bid - gid * group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> register staging -----------------------------------------
  bf16x8 ra[S::A_LOADS], rb[S::B_LOADS];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
      const int idx = tid + i * kGemmThreads;
      const int row = idx >> 3, ch = idx & 7;
      const int m = m0 + row;
      if (m < a.M)
        ra[i] = *reinterpret_cast<const bf16x8*>(a.A + (int64_t)m * a.lda + k0 + ch * 8);
      else
        ra[i] = bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) {
      const int idx = tid + i * kGemmThreads;
      const int row = idx >> 3, ch = idx & 7;
      const int n = n0 + row;
      if (n < a.N)
        rb[i] = *reinterpret_cast<const bf16x8*>(a.B + (int64_t)n * a.ldb + k0 + ch * 8);
      else
        rb[i] = bf16x8{};
    }
  };
  auto store_tiles = [&](int buf) {
    __bf16* la = lds + buf * S::LDS_ELEMS;
    __bf16* lb = la + BM * kBK;
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
      const int idx = tid + i * kGemmThreads;
      *reinterpret_cast<bf16x8*>(la + swz(idx >> 3, idx & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) {
      const int idx = tid + i * kGemmThreads;
      *reinterpret_cast<bf16x8*>(lb + swz(idx >> 3, idx & 7)) = rb[i];
    }
  };

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j) acc[i][j] = f32x16{};

  const int nk = a.K / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int lrow = lane & 31;   // row of the 32x32 operand tile this lane feeds
  const int lk = lane >> 5;     // which 8-element half of a 16-wide k step
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * kBK);
    const __bf16* la = lds + buf * S::LDS_ELEMS;
    const __bf16* lb = la + BM * kBK;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = ks * 2 + lk;
      bf16x8 fa[S::TM], fb[S::TN];
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(la + swz(wm * S::WM + i * 32 + lrow, ch));
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(lb + swz(wn * S::WN + j * 32 + lrow, ch));
#pragma unroll
      for (int i = 0; i < S::TM; ++i)
#pragma unroll
        for (int j = 0; j < S::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2),
  //      accumulator (i%4) + 4*(i/8) --------------------------------------------
#pragma unroll
  for (int i = 0; i < S::TM; ++i) {
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int n = n0 + wn * S::WN + j * 32 + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * S::WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < a.M) a.C[(int64_t)m * a.ldc + n] = acc[i][j][v];
      }
    }
  }
}

template <int BM, int BN>
static hipError_t launch_gemm_tile(const GemmArgs& g, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  using S = GemmShape<BM, BN>;
  GemmKArgs a;
  a.A = reinterpret_cast<const __bf16*>(g.A);
  a.B = reinterpret_cast<const __bf16*>(g.B);
  a.C = g.C;
  a.lda = g.lda;
  a.ldb = g.ldb;
  a.ldc = g.ldc;
  a.M = g.M;
  a.N = g.N;
  a.K = g.K;
  a.tiles_m = (g.M + BM - 1) / BM;
  a.tiles_n = (g.N + BN - 1) / BN;
  a.group_m = 4;
  const size_t lds_bytes = 2 * (size_t)S::LDS_ELEMS * sizeof(__bf16);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_nt_kernel<BM, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN>), dim3(grid), dim3(kGemmThreads), lds_bytes,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_nt(const GemmArgs& g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  // Large M: 256 x 256 tiles (128 KB of LDS, one workgroup per CU).
  // Small M: 128 x 128 tiles so that more CUs get work.
  if ((int64_t)g.M * g.N >= (int64_t)64 * 256 * 256)
    return launch_gemm_tile<256, 256>(g, stream);
  return launch_gemm_tile<128, 128>(g, stream);
}

}  // namespace engram
