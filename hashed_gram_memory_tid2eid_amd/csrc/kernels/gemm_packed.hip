// gemm_packed.hip -- the wkv down-projection v = E W^T with W held in matrix-core
// fragment order ([VeOmni#1370] "feat: support DeepSeek-V4.1-Flash in SeedOmni",
// config commit: the Engram connection projects the concatenated retrieved rows to
// the hidden size before its gate).  Included into engram_device.hip after gemm.hip.
//
// The weight is static, so it is rearranged once (pack_weight_kernel) into
//   Wp[N/16][K/32][64 lanes][8 bf16]:
// the 16 bytes lane l needs as the B operand of v_mfma_f32_16x16x32_bf16 for column
// tile j and k32 step s (column 16 j + l % 16, k 32 s + 8 (l / 16) .. +8) sit at
// chunk (j K/32 + s) 64 + l.  A wave then fetches a whole B fragment with one
// 16-byte-per-lane load of 1 KB of consecutive bytes (8 full cache lines) straight
// into registers, and B takes no LDS at all: no direct-load writes and no
// fragment reads.  The LDS keeps only the gathered rows (operand A), in a deeper
// ring than the two-operand kernel can afford.
//
// Tile: 256 x 256 per workgroup, 8 waves as 1 (M) x 8 (N), 256 x 32 per wave (16 x 2
// tiles of 16 x 16, two waves per SIMD).  Every wave reads the whole A stage from LDS
// and fetches only its own 32 columns of B, so no B fragment is fetched twice: with
// 2 x 4 waves of 128 x 64 the two waves of a column block each fetched it, a third
// more vector-memory traffic per CU, and the kernel was 3-4% slower although it read
// half as much from LDS.  Calls with a short K take 128 x 256 tiles of 4 waves (1 x 4,
// 128 x 64 per wave) instead, two workgroups per CU: one workgroup's prologue and
// epilogue then overlap the other's main loop, and each stage barrier holds only one
// wave per SIMD.
// The 16 x 16 x 32 shape instead of 32 x 32 x 16 (the two-operand kernel's): the
// same flops per cycle with a quarter of the accumulator per instruction, so the
// matrix core reads and writes a third fewer register bytes per flop; measured 2-4%
// faster at every K here, with C bit-identical to gemm_bf16_nt_kernel's (the matrix
// core sums each output's products in the same k order under both shapes).
// A: direct loads into LDS of one 128-byte line per row per 64-k stage, in a ring
// of A_STAGES stages, XOR-swizzled as in gemm.hip.
// Inside a stage four sub-steps run: k32 step 0 on the first half of the wave tile's
// rows, step 0 on the second half, then step 1 on each half.
// B: a ring of the two k32 steps in registers; step s of stage kt+1 is requested right
// after the last sub-step of stage kt that multiplies step s.
//
// Schedules.  The 128-row kernel runs every wave through the same sequence: the A
// fragments of the next sub-step are read from LDS while this one multiplies, one
// barrier per stage, and each wave raises its issue priority over its MFMA runs
// (s_setprio 1), so a SIMD keeps issuing the wave whose products are ready while the
// other issues loads (about 2% at k_pad 19,584 before the ping-pong below).
// The 256-row kernel ping-pongs instead: waves 0-3 (one per SIMD) and waves 4-7 take
// turns on the matrix cores.  A stage runs in four phases separated by barriers; in each
// phase one group multiplies two sub-steps while the other reads the A fragments of its
// next two sub-steps from LDS, and the second group runs the same loop one phase behind
// the first.  With every wave on the same sequence both waves of a SIMD tended to wait
// at the same moments; taking turns raised the matrix cores' busy share from 71% to 76%
// of the cycles at k_pad 19,584 (the clock under load fell from ~1.80 to ~1.75 GHz with
// it) and the kernel ran 1.3-2.1% faster, with C bit-identical (same products in the same
// k order for every output).
//
// Every iteration issues the same loads (the last stages re-read clamped, in-bounds
// addresses into slots nothing reads again), so the explicit vector-memory counter
// wait of each schedule is a fixed number.

namespace engram {

constexpr int kPackedAStages = 4;  // A ring: 4 stages of 64 k (32 KB each at 256 rows, 16 KB at 128)
// calls with k_pad up to this take 128 x 256 tiles (against 256 x 256 at 65,536 tokens:
// 5-6% faster at k_pad 3,072 and 6,144, 2% at 9,792, level at 13,056, 2% slower at
// 16,320 and 3-4% at 19,584)
constexpr int kPackedShortK = 12288;
// dword 3 of a buffer resource on gfx9-family parts: 32-bit data format, no swizzle
constexpr int kBufferRsrcFlags = 0x00020000;

struct GemmPackedKArgs {
  const __bf16* A;     // bf16 [M][lda]
  const bf16x8* Bp;    // packed weight, [N16][K32][64] chunks of 8 bf16
  float* C;            // f32 [M][ldc]
  int64_t lda, ldc;
  int32_t M, N, K;     // K multiple of 64
  int32_t tiles_m, tiles_n, group_m;
  int32_t vec_store;
};

__global__ __launch_bounds__(256)
void pack_weight_kernel(const __bf16* __restrict__ W, int64_t ldw, int32_t N, int32_t K,
                        int64_t total_chunks, bf16x8* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_chunks) return;
  const int k32 = K >> 5;
  const int lane = (int)(c & 63);
  const int64_t t = c >> 6;
  const int s = (int)(t % k32);
  const int j = (int)(t / k32);
  const int n = j * 16 + (lane & 15);
  const int k = s * 32 + 8 * (lane >> 4);
  bf16x8 v = {};
  if (n < N) v = *reinterpret_cast<const bf16x8*>(W + (int64_t)n * ldw + k);
  out[c] = v;
}

template <int A_STAGES, int BM, int WM_WAVES, int WN_WAVES, bool PINGPONG>
__device__ __forceinline__ void packed_gemm_tile(const GemmPackedKArgs& a) {
  constexpr int BN = 256, NWAVES = WM_WAVES * WN_WAVES;
  constexpr int BK = kGemmBK;
  constexpr int WM = BM / WM_WAVES, WN = BN / WN_WAVES, TM = WM / 16, TN = WN / 16;
  constexpr int HM = TM / 2;                   // 16-row blocks per half
  constexpr int STAGE = BM * BK * 2;           // bytes of A per stage
  constexpr int AI = BM / 8 / NWAVES;          // 1 KB direct loads per wave per stage
  constexpr int BL = TN;                       // B loads per k32 step
  constexpr int PER_ITER = 2 * BL + AI;        // vector-memory loads per iteration
  static_assert(A_STAGES >= 2, "ring needs two stages");
  static_assert(AI * 8 * NWAVES == BM, "A tile must fill whole load rounds");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- tile id: XCD-contiguous runs, then GROUP_M swizzle (as gemm.hip) -------
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
  const int nk = a.K / BK;
  const int k32 = a.K >> 5;

  // Both operands are read through buffer resources (MUBUF): the compiler counts
  // direct-to-LDS buffer loads and register buffer loads on one in-order vector
  // memory counter, so its waits for the B registers stay exact (mixing global
  // direct-to-LDS loads with register loads makes it wait for everything).  Each
  // resource starts at this tile's first row (column tile) so byte offsets fit
  // 32 bits; its record count covers exactly the rows (tiles) the tile may read.
  const int rows_here = min(a.M - m0, BM);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.A + (int64_t)m0 * a.lda), (short)0, (int)((int64_t)rows_here * a.lda * 2), kBufferRsrcFlags);
  const int n16 = (a.N + 15) / 16;
  const int jt0 = n0 / 16;
  const int tiles_here = min(n16 - jt0, BN / 16);
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.Bp + (int64_t)jt0 * k32 * 64), (short)0, tiles_here * k32 * 1024, kBufferRsrcFlags);

  // ---- A: direct loads into LDS (wave w, load i fills LDS bytes
  //      [(NWAVES i + w) KB, +1 KB) of the stage; 8 lanes fetch one whole line).
  //      Rows past M read row M-1 (never stored).
  int aoff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int P = 64 * (i * NWAVES + wave) + lane, row = P >> 3, c = (P & 7) ^ gemm_swz(row);
    aoff[i] = (min(row, rows_here - 1) * (int)a.lda + 8 * c) * 2;
  }
  auto issue_a = [&](int kt) {
    char* st = smem + (kt % A_STAGES) * STAGE;
    const int ks = min(kt, nk - 1);  // past the end: an in-bounds stage into a slot no one reads
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (ENGRAM_LDS_AS void*)(st + (i * NWAVES + wave) * 1024), 16,
                                               aoff[i] + ks * BK * 2, 0, 0, 0);
  };

  // ---- B: packed fragments; column tiles past N read the last tile (never stored)
  int boff[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int jt = min(wn * TN + j, tiles_here - 1);
    boff[j] = (jt * k32 * 64 + lane) * 16;
  }
  bf16x8 bfr[2][TN];
  auto issue_b = [&](int kt, int ks) {
    const int s = min(kt, nk - 1) * 2 + ks;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[ks][j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(brsrc, boff[j] + s * 1024, 0, 0));
  };

  // rows 16 apart share the swizzle ((row >> 1) & 7), so one base and one swizzle
  // serve every block; the blocks are immediate offsets of 16 rows
  const int lrow = lane & 15, lk = lane >> 4;
  const int r0 = wm * WM + lrow;
  const int arow0 = r0 * BK, aswz0 = gemm_swz(r0);
  // fragments of rows half h (16-row blocks h HM .. +HM) for k32 step ks
  auto load_a = [&](int kt, int ks, int h, bf16x8* fa) {
    const __bf16* base = reinterpret_cast<const __bf16*>(smem + (kt % A_STAGES) * STAGE) + arow0 +
                         8 * ((ks * 4 + lk) ^ aswz0);
#pragma unroll
    for (int i = 0; i < HM; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(base + (h * HM + i) * 16 * BK);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{};
  auto mma = [&](const bf16x8* fa, const bf16x8* fb, int h) {
    if constexpr (!PINGPONG) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < HM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[h * HM + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[h * HM + i][j], 0, 0, 0);
    if constexpr (!PINGPONG) __builtin_amdgcn_s_setprio(0);
  };

  if constexpr (PINGPONG) {
    // Group 0 = waves 0 .. NWAVES/2-1, group 1 = the rest; one wave of each per SIMD.
    // Loop body per stage kt, phases ending at a barrier:
    //   Q0 multiply k32 step 0 (both row halves), then request B(kt+1, 0)
    //   Q1 read the fragments of step 1; wait for this wave's parts of A(kt+1)
    //   Q2 multiply step 1, then request B(kt+1, 1)
    //   Q3 request A(kt+A_STAGES) into the slot of stage kt (every wave read its last
    //      fragments of stage kt in its Q1, before a barrier both groups have passed),
    //      then read the fragments of step 0 of stage kt+1
    // Group 1 runs phase Q of the body while group 0 runs the next one, so by the start
    // of group 0's Q3(kt) both groups have waited for their parts of A(kt+1).
    static_assert(NWAVES % 2 == 0, "two groups of waves");
    const bool group1 = wave >= NWAVES / 2;  // uniform per wave
    issue_b(0, 0);
    issue_b(0, 1);
#pragma unroll
    for (int s = 0; s < A_STAGES; ++s) issue_a(s);
    wait_vmcnt<(A_STAGES - 1) * AI>();
    __builtin_amdgcn_s_barrier();
    // Loads a wave has issued after A(kt+1) when it waits in Q1(kt): fewest at kt = 0
    // (A stages 2 .. A_STAGES-1 of the prologue and B(1, 0)); later stages have issued
    // more, so the count also waits for later A stages, requested stages earlier.
    constexpr int WAIT = (A_STAGES - 2) * AI + BL;
    static_assert(WAIT <= 63, "vmcnt field holds 6 bits");
    bf16x8 fa0[HM], fa1[HM];
    load_a(0, 0, 0, fa0);
    load_a(0, 0, 1, fa1);
    wait_lgkmcnt0();
    if (group1) __builtin_amdgcn_s_barrier();  // group 1's first phase: beside group 0's Q0(0)
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < nk; ++kt) {
      mma(fa0, bfr[0], 0);  // Q0
      mma(fa1, bfr[0], 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(kt + 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      load_a(kt, 1, 0, fa0);  // Q1
      load_a(kt, 1, 1, fa1);
      wait_lgkmcnt0();
      wait_vmcnt<WAIT>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      mma(fa0, bfr[1], 0);  // Q2
      mma(fa1, bfr[1], 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(kt + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      issue_a(kt + A_STAGES);  // Q3
      const int kn = kt + 1 < nk ? kt + 1 : kt;
      load_a(kn, 0, 0, fa0);
      load_a(kn, 0, 1, fa1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    }
    if (!group1) __builtin_amdgcn_s_barrier();  // beside group 1's last phase
  } else {
  // ---- prologue: B of stage 0, then A stages 0 .. A_STAGES-1; wait for A stage 0
    issue_b(0, 0);
    issue_b(0, 1);
  #pragma unroll
    for (int s = 0; s < A_STAGES; ++s) issue_a(s);
    wait_vmcnt<(A_STAGES - 1) * AI>();
    __builtin_amdgcn_s_barrier();
  
    // Loads issued after A stage kt+1 when iteration kt waits for it: fewest at kt = 0,
    // where the stage came from the prologue and only A stages 2 .. A_STAGES-1 and B
    // step 0 of stage 1 follow it.  That count serves every iteration: later ones have
    // more loads after the stage (in steady state (A_STAGES-2) whole iterations plus two
    // B steps), so the wait also covers A stage kt+2, requested two iterations earlier.
    // One count keeps the loop a single body; with an exact count per iteration the
    // compiler peels the first iterations and runs out of registers there.
    constexpr int WAIT = (A_STAGES - 2) * AI + BL;
    static_assert(WAIT <= (A_STAGES - 2) * PER_ITER + 2 * BL && WAIT <= 63, "vmcnt field holds 6 bits");
  
    bf16x8 fa0[HM], fa1[HM];
    load_a(0, 0, 0, fa0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      load_a(kt, 0, 1, fa1);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa0, bfr[0], 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      load_a(kt, 1, 0, fa0);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa1, bfr[0], 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(kt + 1, 0);
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      load_a(kt, 1, 1, fa1);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa0, bfr[1], 0);
      __builtin_amdgcn_sched_barrier(0);
      // this wave has read all of A stage kt once the last sub-step's fragments have
      // landed; the barrier makes that true for every wave and publishes A stage kt+1,
      // then slot kt % A_STAGES is refilled with stage kt + A_STAGES
      wait_lgkmcnt0();
      wait_vmcnt<WAIT>();
      __builtin_amdgcn_s_barrier();
      issue_a(kt + A_STAGES);
      __builtin_amdgcn_sched_barrier(0);
      load_a(kt + 1 < nk ? kt + 1 : kt, 0, 0, fa0);
      __builtin_amdgcn_sched_barrier(0);
      mma(fa1, bfr[1], 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(kt + 1, 1);
    }
  }

  // ---- epilogue (as gemm.hip): stage one 16-row slab per wave in LDS, write whole
  //      row segments of C with 16-byte stores.  The clamped loads and fragment reads
  //      of the last iterations may still be in flight: drain them first.
  constexpr int PITCH = WN + 4;
  static_assert(NWAVES * 16 * PITCH * 4 <= A_STAGES * STAGE, "epilogue staging must fit in the ring");
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  float* slab = reinterpret_cast<float*>(smem) + wave * 16 * PITCH;
  const bool full = (m0 + BM <= a.M) && (n0 + BN <= a.N) && a.vec_store;
  constexpr int LANES_PER_ROW = WN / 4;
  constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * (lane >> 4) + v;
        slab[r * PITCH + j * 16 + (lane & 15)] = acc[i][j][v];
      }
    }
    const int gm0 = m0 + wm * WM + i * 16;
    const int gn = n0 + wn * WN + (lane % LANES_PER_ROW) * 4;
#pragma unroll
    for (int q = 0; q < 16 / ROWS_PER_PASS; ++q) {
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

// 256 x 256 tiles, one workgroup of 8 waves (1 x 8) per CU (calls with a long K)
__global__ __launch_bounds__(512, 1) void gemm_bf16_nt_packed_kernel(GemmPackedKArgs a) {
  packed_gemm_tile<kPackedAStages, 256, 1, 8, true>(a);
}
// 128 x 256 tiles, two workgroups of 4 waves per CU (short K)
__global__ __launch_bounds__(256, 2) void gemm_bf16_nt_packed128_kernel(GemmPackedKArgs a) {
  packed_gemm_tile<kPackedAStages, 128, 1, 4, false>(a);
}

hipError_t launch_pack_weight(const PackWeightArgs& g, hipStream_t stream) {
  (void)hipGetLastError();
  if (g.N <= 0 || g.K <= 0 || g.K % 32 != 0) return hipErrorInvalidValue;
  const int64_t total = (int64_t)((g.N + 15) / 16) * (g.K / 32) * 64;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const __bf16*>(g.W), g.ldw, g.N, g.K, total,
                     reinterpret_cast<bf16x8*>(g.out));
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_nt_packed(const GemmPackedArgs& g, hipStream_t stream) {
  (void)hipGetLastError();
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (g.K % kGemmBK != 0 || g.K <= 0) return hipErrorInvalidValue;
  GemmPackedKArgs a;
  a.A = reinterpret_cast<const __bf16*>(g.A);
  a.Bp = reinterpret_cast<const bf16x8*>(g.Bp);
  a.C = g.C;
  a.lda = g.lda;
  a.ldc = g.ldc;
  a.M = g.M;
  a.N = g.N;
  a.K = g.K;
  a.tiles_n = (g.N + 255) / 256;
  a.vec_store = (g.ldc % 4 == 0 && ((uintptr_t)g.C & 15) == 0) ? 1 : 0;
  // short K: two 128-row workgroups per CU, in tile groups of 8 row blocks up to k_pad
  // 4,096 and of 4 above (measured at 3,072: 8 is 2-4% faster than 4, 16 is 3-5% slower;
  // at 6,144: 4 is 1.3% faster than 8); long K: one 256-row workgroup per CU, groups of 4
  // (at k_pad 19,584 as fast as groups of 2, 7.645 against 7.648 ms, with a third less
  // traffic beyond L2: an XCD's 32 concurrent tiles then re-read W per 4 row blocks)
  const bool short_k = g.K <= kPackedShortK;
  const int bm = short_k ? 128 : 256;
  a.tiles_m = (g.M + bm - 1) / bm;
  a.group_m = short_k && g.K <= 4096 ? 8 : 4;
  const size_t lds_bytes = (size_t)kPackedAStages * bm * kGemmBK * 2;
  static std::atomic<uint64_t> lds_set256{0}, lds_set128{0};
  const hipError_t e =
      short_k ? ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_bf16_nt_packed128_kernel), (int)lds_bytes,
                                   lds_set128)
              : ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_bf16_nt_packed_kernel), (int)lds_bytes,
                                   lds_set256);
  if (e != hipSuccess) return e;
  // per-tile byte offsets are 32-bit: one tile's rows of A and 8 column tiles of B
  if ((int64_t)256 * g.lda * 2 > 0x7FFFFFFF || (int64_t)16 * (g.K / 32) * 1024 > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (short_k)
    hipLaunchKernelGGL(gemm_bf16_nt_packed128_kernel, dim3((unsigned)grid), dim3(256), lds_bytes, stream, a);
  else
    hipLaunchKernelGGL(gemm_bf16_nt_packed_kernel, dim3((unsigned)grid), dim3(512), lds_bytes, stream, a);
  return hipGetLastError();
}

}  // namespace engram
