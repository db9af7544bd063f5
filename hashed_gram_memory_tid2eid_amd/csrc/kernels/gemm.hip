// gemm.hip -- the wkv down-projection v = E W^T on the CDNA4 matrix cores
// ([VeOmni#1370] "feat: support DeepSeek-V4.1-Flash in SeedOmni", config commit:
// the Engram connection projects the concatenated retrieved rows to the hidden
// size before its gate).  Included into engram_device.hip.
//
// C[M][N] (fp32) = A[M][K] (bf16, row-major) * B[N][K]^T (bf16, row-major):
// both operands are K-contiguous, the layout the gathered token rows and the
// projection weight already have.  K is a multiple of 32 (k_pad is of 64).
//
// Tile: a workgroup of WM_WAVES x WN_WAVES waves owns a BM x BN block of C; each
// wave owns a (BM/WM_WAVES) x (BN/WN_WAVES) sub-block of 32 x 32 tiles computed
// with v_mfma_f32_32x32x16_bf16 (per lane 8 bf16 of A: row lane%32, k
// 8*(lane/32)..+8; 8 of B; 16 fp32 accumulators).  Large M uses 256 x 256 tiles
// with 8 waves (2 x 4, 128 x 64 each, two waves per SIMD): while one wave of a
// SIMD waits on a stage barrier or its loads, the other keeps the matrix core
// busy (measured 1.45 PFLOP/s against 1.21 for 4 waves of 128 x 128).
//
// Operands reach LDS by direct global->LDS loads (global_load_lds_dwordx4, no
// register staging) in stages of 64 k: one whole 128-byte line of every operand
// row, so each line is fetched once and every cache request is a full line.  Two
// stages (2 x 64 KB for a 256 x 256 tile) form a ring: stage kt+1 streams in
// while stage kt multiplies; one barrier per stage.  128 x 128 tiles (few tokens)
// use a ring of 4 stages of 32 KB, so three stages stay in flight.  A wave writes 1 KB of
// consecutive LDS per load, so the XOR swizzle of the 16-byte chunks
// (chunk ^ ((row >> 1) & 7), rows of 128 B) is applied by choosing which global
// chunk each lane fetches; with it the fragment reads are free of LDS bank
// conflicts (measured with the bank-conflict counter).
//
// Inside a stage the four k16 steps are software pipelined: the fragments of
// step ks+1 are read while step ks's MFMAs run, and the next stage's first step
// is read while the last step multiplies.  At most one step of fragments is
// outstanding at any wait, so the compiler's lgkmcnt tracking stays exact and
// each explicit wait falls on data requested a whole MFMA phase earlier.

// Tile order: workgroup ids are dealt round-robin to the 8 XCDs (each with its
// own L2); the id is remapped so that each XCD gets a contiguous run of tiles,
// walked in groups of GROUP_M = 2 row blocks (measured best of 1/2/4/8/16), so the
// concurrently running
// workgroups of one XCD share A row blocks and B column blocks in its L2.

namespace engram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define ENGRAM_LDS_AS __attribute__((address_space(3)))

constexpr int kGemmBK = 64;      // k per stage: one 128-byte line of every operand row
// LDS ring depth: 2 stages of 64 KB for 256 x 256 tiles (all the LDS allows); 4 stages
// of 32 KB for 128 x 128 tiles, whose few-token calls are bound by load latency
constexpr int kSmallTileStages = 4;

struct GemmKArgs {
  const __bf16* A;
  const __bf16* B;
  float* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
  int32_t vec_store;  // C 16-byte aligned and ldc % 4 == 0: whole-tile stores may be 16-byte
  int32_t k_chunk;          // split-K: k per split (blockIdx.y picks the split)
  int64_t c_split_stride;   // split-K: elements between the splits' partial C slices
};

// physical 16-byte chunk of logical chunk c in a 128-byte LDS row: c ^ ((row >> 1) & 7).
// Measured on gfx950 with the bank-conflict counter: fragment reads (32 rows x 2
// chunks per ds_read_b128) see no conflicts with this swizzle.
__device__ __forceinline__ int gemm_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt with vmcnt <= N and no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int BM, int BN, int WM_WAVES, int WN_WAVES, int STAGES>
__global__ __launch_bounds__(64 * WM_WAVES * WN_WAVES, 1)
void gemm_bf16_nt_kernel(GemmKArgs a) {
  constexpr int BK = kGemmBK;
  constexpr int NWAVES = WM_WAVES * WN_WAVES;
  constexpr int WM = BM / WM_WAVES, WN = BN / WN_WAVES, TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int AI = BM / 8 / NWAVES, BI = BN / 8 / NWAVES;  // 1 KB direct loads per wave per stage
  static_assert(AI * 8 * NWAVES == BM && BI * 8 * NWAVES == BN, "tile must fill whole load rounds");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- split-K: split y multiplies k in [y k_chunk, (y+1) k_chunk) into its own
  //      partial slice of C (the consumer sums the slices in split order)
  if (gridDim.y > 1) {
    const int sp = blockIdx.y;
    a.A += (int64_t)sp * a.k_chunk;
    a.B += (int64_t)sp * a.k_chunk;
    a.C += (int64_t)sp * a.c_split_stride;
    a.K = a.k_chunk;
  }

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
  const int m0 = (first_m + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN_WAVES, wn = wave % WN_WAVES;

  // ---- direct global->LDS loads: wave w, load i fills LDS bytes
  //      [(NWAVES i + w) KB, +1 KB) of the A (or B) region; lane l writes 16 B at
  //      l*16, i.e. row P/8, physical chunk P%8 with P = 64(NWAVES i + w) + l, so 8 lanes
  //      fetch one whole 128-byte line.  Rows past M (N) read a valid row; their
  //      results are never stored.
  const __bf16* ap[AI];
  const __bf16* bp[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int P = 64 * (i * NWAVES + wave) + lane, row = P >> 3, c = (P & 7) ^ gemm_swz(row);
    ap[i] = a.A + (int64_t)min(m0 + row, a.M - 1) * a.lda + 8 * c;
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int P = 64 * (i * NWAVES + wave) + lane, row = P >> 3, c = (P & 7) ^ gemm_swz(row);
    bp[i] = a.B + (int64_t)min(n0 + row, a.N - 1) * a.ldb + 8 * c;
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(ap[i] + kt * BK),
                                       (ENGRAM_LDS_AS void*)(st + (i * NWAVES + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bp[i] + kt * BK),
                                       (ENGRAM_LDS_AS void*)(st + A_BYTES + (i * NWAVES + wave) * 1024), 16, 0, 0);
  };

  // ---- fragment row offsets (elements) and swizzles inside a stage -----------
  const int lrow = lane & 31, lk = lane >> 5;
  int arow[TM], brow[TN], aswz[TM], bswz[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * WM + i * 32 + lrow;
    arow[i] = r * BK;
    aswz[i] = gemm_swz(r);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int r = wn * WN + j * 32 + lrow;
    brow[j] = BM * BK + r * BK;
    bswz[j] = gemm_swz(r);
  }
  // fragments of k16 step ks (0..3) of stage kt
  auto load_frags = [&](int kt, int ks, bf16x8* fa, bf16x8* fb) {
    const __bf16* base = reinterpret_cast<const __bf16*>(smem + (kt % STAGES) * STAGE);
    const int c = ks * 2 + lk;
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(base + brow[j] + 8 * (c ^ bswz[j]));
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(base + arow[i] + 8 * (c ^ aswz[i]));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // ---- pipeline: stage kt+1 streams in while stage kt multiplies; inside a stage
  //      the fragments of k16 step ks+1 are read while step ks multiplies, and the
  //      next stage's first step is read while the last step multiplies.  At most
  //      one step of fragments (TM + TN reads) is outstanding at any wait.
  const int nk = a.K / BK;
  constexpr int LOADS = AI + BI;  // direct loads per wave per stage
  // prologue: every slot of the ring is free; wait for stage 0 only
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s);
  if (nk >= STAGES) wait_vmcnt<(STAGES - 1) * LOADS>(); else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  load_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 2, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 3, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    // this wave is done reading stage kt once step 3 has landed; the barrier makes
    // that true for every wave and publishes stage kt+1 (stages kt+2 .. kt+STAGES-1
    // may still be in flight), then slot kt%STAGES is refilled with stage
    // kt+STAGES (the last iteration re-reads its own stage to keep the counts fixed)
    wait_lgkmcnt0();
    if (kt + 1 < nk) {
      if (kt + STAGES - 1 < nk) wait_vmcnt<(STAGES - 2) * LOADS>(); else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES < nk) issue(kt + STAGES);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt + 1 < nk ? kt + 1 : kt, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: D[r][c] of a 32x32 tile sits in lane c + 32*((r/4)%2),
  //      accumulator (r%4) + 4*(r/8).  Each wave stages one 32-row slab of its
  //      sub-block (32 x WN fp32) in its own LDS area, then writes the slab back
  //      row by row with 16-byte stores, so every store instruction covers whole
  //      row segments of C instead of scattering 4-byte values.
  constexpr int SLAB = 32 * WN;                 // floats per staged slab
  constexpr int PITCH = WN + 4;                 // LDS row pitch (floats), breaks bank aliasing
  static_assert(NWAVES * 32 * PITCH * 4 <= STAGES * STAGE, "epilogue staging must fit in the ring");
  (void)SLAB;
  __builtin_amdgcn_s_barrier();                 // every wave is done with the operand ring
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * PITCH;
  const bool full = (m0 + BM <= a.M) && (n0 + BN <= a.N) && a.vec_store;
  constexpr int LANES_PER_ROW = WN / 4;         // 16-byte pieces per staged row
  constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        slab[r * PITCH + j * 32 + (lane & 31)] = acc[i][j][v];
      }
    }
    const int gm0 = m0 + wm * WM + i * 32;
    const int gn = n0 + wn * WN + (lane % LANES_PER_ROW) * 4;
#pragma unroll
    for (int q = 0; q < 32 / ROWS_PER_PASS; ++q) {
      const int r = q * ROWS_PER_PASS + lane / LANES_PER_ROW;
      const f32x4 val = *reinterpret_cast<const f32x4*>(slab + r * PITCH + (lane % LANES_PER_ROW) * 4);
      const int m = gm0 + r;
      float* dst = a.C + (int64_t)m * a.ldc + gn;
      if (full) {
        *reinterpret_cast<f32x4*>(dst) = val;
      } else if (m < a.M) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gn + e < a.N) dst[e] = val[e];
      }
    }
  }
}

template <int BM, int BN, int WMW, int WNW, int STAGES>
static hipError_t launch_gemm_tile(const GemmArgs& g, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  constexpr int STAGE = (BM + BN) * kGemmBK * 2;
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
  a.group_m = 2;
  a.vec_store = (g.ldc % 4 == 0 && ((uintptr_t)g.C & 15) == 0) ? 1 : 0;
  const int splits = g.splits > 1 ? g.splits : 1;
  a.k_chunk = g.K / splits;
  a.c_split_stride = g.c_split_stride;
  const size_t lds_bytes = (size_t)STAGES * STAGE;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(
      reinterpret_cast<const void*>(&gemm_bf16_nt_kernel<BM, BN, WMW, WNW, STAGES>), (int)lds_bytes, lds_set);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, BN, WMW, WNW, STAGES>), dim3(grid, (unsigned)splits),
                     dim3(64 * WMW * WNW), lds_bytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_nt(const GemmArgs& g, hipStream_t stream) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.K % kGemmBK != 0 || g.K <= 0) return hipErrorInvalidValue;
  if (g.splits > 1 && (g.K % (kGemmBK * g.splits) != 0)) return hipErrorInvalidValue;
  // Large M: 256 x 256 tiles, 8 waves (2 stages x 64 KB of LDS, one workgroup per CU).
  // Small M: 128 x 128 tiles, 4 waves, so that more CUs get work.
  if ((int64_t)g.M * g.N >= (int64_t)64 * 256 * 256)
    return launch_gemm_tile<256, 256, 2, 4, 2>(g, stream);
  return launch_gemm_tile<128, 128, 2, 2, kSmallTileStages>(g, stream);
}

}  // namespace engram
