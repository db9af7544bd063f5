// gemm_gather.hip -- fused gather + row-wise dequant + wkv projection:
//   v[t][o] = sum_k W[o][k] * bf16(fp32(e4m3(table[row_ids[t][seg]][k_in_seg])) * scale)
// without writing the gathered rows to HBM ([VeOmni#1370] "feat: support
// DeepSeek-V4.1-Flash in SeedOmni": the PR summary's row-wise FP8 dequant on
// lookup and the config commit's wkv projection, done in one kernel).  Included
// into engram_device.hip after gemm.hip (shares its swizzle and wait helpers).
//
// Same tile and wave layout as gemm_bf16_nt_kernel (256 x 256, 8 waves of
// 128 x 64, v_mfma_f32_32x32x16_bf16, stages of 64 k), with the A operand taken
// straight from the tables:
//  - direct global->LDS loads bring 64 fp8 bytes of each of the tile's 256
//    table rows per stage (16 KB, two stages ahead);
//  - during the MFMA phases of stage kt every thread dequantises its share of
//    stage kt+1 (8 elements per phase: v_cvt_pk_f32_fp8, one fp32 multiply by
//    the row scale, round-to-nearest-even to bf16) into a bf16 buffer laid out
//    like the plain kernel's A stage, so each element is converted once, not
//    once per reading wave;
//  - B (the weight) streams as in the plain kernel, one stage ahead.
// LDS: B ring 2 x 32 KB, converted A ring 2 x 32 KB, fp8 A ring 2 x 16 KB = 160 KB.
// A stage never straddles two segments (seg_pitch is a multiple of 64), so a
// stage reads one table row per token; a thread converts the same four tile rows
// in every stage and keeps their scales in registers, refreshed when the
// segment changes: one fp32 scale per row, or, for (1, 32)-blocked tables, the
// row's e8m0 bytes (at most 8: rows of up to 256 elements, the released layout)
// from which each stage picks its block's exponent.

namespace engram {

struct GatherGemmKArgs {
  const uint8_t* t0;
  const uint8_t* t1;
  const uint8_t* t2;
  const void* s0;           // float [rows], or uint8 e8m0 [rows][nblk]
  const void* s1;
  const void* s2;
  int32_t nblk;             // e8m0 bytes per row (block scales)
  int32_t r0, r1, r2;       // rows per table
  const int32_t* row_ids;   // the site's first column; tokens rid_ld ints apart
  int32_t rid_ld;
  int32_t split;            // heads (per-order tables) or 2^29 (one table per site)
  int64_t pitch;            // table row pitch, bytes (>= seg_pitch)
  int32_t row_dim, seg_pitch, cols, heads;
  const __bf16* B;          // [N][ldb]
  int64_t ldb;
  float* C;                 // [M][ldc]
  int64_t ldc;
  int32_t M, N, K;          // K = cols * seg_pitch
  int32_t tiles_m, tiles_n, group_m, vec_store;
};

constexpr int kGgBM = 256, kGgBN = 256, kGgBK = 64;
constexpr int kGgWM = 2, kGgWN = 4, kGgWaves = kGgWM * kGgWN, kGgThreads = 64 * kGgWaves;
constexpr int kGgB_BYTES = kGgBN * kGgBK * 2;    // 32 KB
constexpr int kGgA16_BYTES = kGgBM * kGgBK * 2;  // 32 KB
constexpr int kGgA8_BYTES = kGgBM * kGgBK;       // 16 KB
constexpr int kGgB_OFF = 0, kGgA16_OFF = 2 * kGgB_BYTES, kGgA8_OFF = kGgA16_OFF + 2 * kGgA16_BYTES;
constexpr int kGgLDS = kGgA8_OFF + 2 * kGgA8_BYTES;  // 160 KB

__device__ __forceinline__ int gg_order(const GatherGemmKArgs& a, int seg) {
  return (seg >= a.split) + (seg >= 2 * a.split);
}
__device__ __forceinline__ const uint8_t* gg_table(const GatherGemmKArgs& a, int n) {
  return n == 0 ? a.t0 : (n == 1 ? a.t1 : a.t2);
}
__device__ __forceinline__ const void* gg_scale(const GatherGemmKArgs& a, int n) {
  return n == 0 ? a.s0 : (n == 1 ? a.s1 : a.s2);
}
constexpr int kGgMaxBlocks = 8;  // e8m0 bytes a converting thread keeps per row
__device__ __forceinline__ int gg_rows(const GatherGemmKArgs& a, int n) {
  return n == 0 ? a.r0 : (n == 1 ? a.r1 : a.r2);
}

template <bool kBlockScale>
__global__ __launch_bounds__(kGgThreads, 1) void gemm_gather_fp8_kernel(GatherGemmKArgs a) {
  constexpr int BK = kGgBK;
  constexpr int WM = kGgBM / kGgWM, WN = kGgBN / kGgWN, TM = WM / 32, TN = WN / 32;
  constexpr int BI = kGgBN / 8 / kGgWaves;   // 1 KB B loads per wave per stage (4)
  constexpr int AI = kGgA8_BYTES / 1024 / kGgWaves;  // 1 KB fp8 A loads per wave per stage (2)
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- tile id (as in the plain kernel) -----------------------------------
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
  const int m0 = (first_m + in_group % gm) * kGgBM;
  const int n0 = (in_group / gm) * kGgBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kGgWN, wn = wave % kGgWN;

  // ---- B: direct loads exactly as in the plain kernel -----------------------
  const __bf16* bp[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int P = 64 * (i * kGgWaves + wave) + lane, row = P >> 3, c = (P & 7) ^ gemm_swz(row);
    bp[i] = a.B + (int64_t)min(n0 + row, a.N - 1) * a.ldb + 8 * c;
  }
  auto issue_b = [&](int kt) {
    char* st = smem + kGgB_OFF + (kt & 1) * kGgB_BYTES;
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bp[i] + kt * BK),
                                       (ENGRAM_LDS_AS void*)(st + (i * kGgWaves + wave) * 1024), 16, 0, 0);
  };

  // ---- A fp8: wave w, load i fills bytes [(8i + w) KB, +1 KB) of the fp8 stage;
  //      lane l writes 16 B at l*16: tile row P/4, 16-byte piece P%4 of the row's
  //      64 bytes, P = 64(8i + w) + l.  The row pointer is refreshed per segment.
  int a_row[AI], a_piece[AI];
  const uint8_t* ap[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int P = 64 * (i * kGgWaves + wave) + lane;
    a_row[i] = P >> 2;
    a_piece[i] = P & 3;
    ap[i] = a.t0;
  }
  int dma_seg = -1;
  auto set_dma_segment = [&](int seg) {
    const int n = gg_order(a, seg);
    const uint8_t* tb = gg_table(a, n);
    const int rows = gg_rows(a, n);
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int m = m0 + a_row[i];
      int r = m < a.M ? a.row_ids[(int64_t)m * a.rid_ld + seg] : 0;
      if (r < 0 || r >= rows) r = 0;  // reported by the converting thread; keep the read in bounds
      ap[i] = tb + (int64_t)r * a.pitch + 16 * a_piece[i];
    }
    dma_seg = seg;
  };
  auto issue_a8 = [&](int kt) {
    const int k0 = kt * BK, seg = k0 / a.seg_pitch;
    if (seg != dma_seg) set_dma_segment(seg);
    const int off = k0 - seg * a.seg_pitch;
    char* st = smem + kGgA8_OFF + (kt & 1) * kGgA8_BYTES;
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(ap[i] + off),
                                       (ENGRAM_LDS_AS void*)(st + (i * kGgWaves + wave) * 1024), 16, 0, 0);
  };

  // ---- dequant: in phase q of a stage, thread tid converts the 8 elements at
  //      bytes [8(tid%8), +8) of tile row 64q + tid/8; consecutive lanes read
  //      consecutive 8-byte words of the fp8 stage ----------------------------------
  const int cpiece = tid & 7;
  int conv_seg = -1;
  float cscale[4];  // per phase row; 0 for rows past M and bad row ids (they convert to zeros)
  uint32_t cblk[4][kBlockScale ? 2 : 1];  // block scales: the row's e8m0 bytes, little-endian
  auto set_conv_segment = [&](int seg) {
    const int n = gg_order(a, seg);
    const int rows = gg_rows(a, n);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + 64 * q + (tid >> 3);
      cscale[q] = 0.f;
      if (kBlockScale) cblk[q][0] = cblk[q][kBlockScale ? 1 : 0] = 0u;
      if (m < a.M) {
        const int r = a.row_ids[(int64_t)m * a.rid_ld + seg];
        if (r < 0 || r >= rows) {
          latch_error(ENGRAM_E_ROW_RANGE);
        } else if (kBlockScale) {
          const uint8_t* sb = static_cast<const uint8_t*>(gg_scale(a, n)) + (int64_t)r * a.nblk;
          if (a.nblk == kGgMaxBlocks) {  // 8-byte aligned: one load
            typedef unsigned int u32x2s __attribute__((ext_vector_type(2)));
            const u32x2s w = *reinterpret_cast<const u32x2s*>(sb);
            cblk[q][0] = w[0];
            cblk[q][kBlockScale ? 1 : 0] = w[1];
          } else {
            for (int b = 0; b < a.nblk; ++b)
              cblk[q][b >> 2] |= (uint32_t)sb[b] << (8 * (b & 3));
          }
          cscale[q] = 1.f;  // marks a valid row
        } else {
          cscale[q] = static_cast<const float*>(gg_scale(a, n))[r];
        }
      }
    }
    conv_seg = seg;
  };
  auto convert = [&](int kt, int q) {  // stage kt, phase q (0..3)
    const int k0 = kt * BK, seg = k0 / a.seg_pitch;
    if (seg != conv_seg) set_conv_segment(seg);
    const int crow = 64 * q + (tid >> 3);
    const int e0 = k0 - seg * a.seg_pitch + 8 * cpiece;  // element index inside the segment
    const char* src = smem + kGgA8_OFF + (kt & 1) * kGgA8_BYTES + crow * 64 + 8 * cpiece;
    typedef unsigned int u32x2g __attribute__((ext_vector_type(2)));
    typedef float f32x2g __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4g __attribute__((ext_vector_type(4)));
    const u32x2g w = *reinterpret_cast<const u32x2g*>(src);
    float s = cscale[q];
    if (kBlockScale && s != 0.f) {  // the exponent of this piece's 32-element block
      const int blk = (e0 >> 5) & (kGgMaxBlocks - 1);  // padding pieces are zeroed below
      s = e8m0_value((cblk[q][blk >> 2] >> (8 * (blk & 3))) & 0xFFu);
    }
    float f[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2g lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], false);
      const f32x2g hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], true);
      f[4 * h + 0] = lo[0] * s;
      f[4 * h + 1] = lo[1] * s;
      f[4 * h + 2] = hi[0] * s;
      f[4 * h + 3] = hi[1] * s;
    }
    if (e0 + 8 > a.row_dim) {  // only the last stage of a segment reaches its padding
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (e0 + j >= a.row_dim) f[j] = 0.f;  // segment padding (also drops a NaN pad byte)
    }
    u32x4g o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 lo = (__bf16)f[2 * j], hi = (__bf16)f[2 * j + 1];
      o[j] = (uint32_t)__builtin_bit_cast(unsigned short, lo) |
             ((uint32_t)__builtin_bit_cast(unsigned short, hi) << 16);
    }
    char* dst = smem + kGgA16_OFF + (kt & 1) * kGgA16_BYTES + crow * 128 + 16 * (cpiece ^ gemm_swz(crow));
    *reinterpret_cast<u32x4g*>(dst) = o;
  };

  // ---- fragment reads (A from the converted buffer, B from its ring) ----------
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
    brow[j] = r * BK;
    bswz[j] = gemm_swz(r);
  }
  auto load_frags = [&](int kt, int ks, bf16x8* fa, bf16x8* fb) {
    const __bf16* abase = reinterpret_cast<const __bf16*>(smem + kGgA16_OFF + (kt & 1) * kGgA16_BYTES);
    const __bf16* bbase = reinterpret_cast<const __bf16*>(smem + kGgB_OFF + (kt & 1) * kGgB_BYTES);
    const int c = ks * 2 + lk;
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(bbase + brow[j] + 8 * (c ^ bswz[j]));
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(abase + arow[i] + 8 * (c ^ aswz[i]));
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

  // ---- prologue: B(0), fp8 A(0), fp8 A(1) in; A(0) converted -----------------
  const int nk = a.K / BK;
  issue_b(0);
  issue_a8(0);
  if (nk > 1) issue_a8(1);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) convert(0, q);
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();

  // ---- main loop: at the top of iteration kt, converted A(kt) and B(kt) are in
  //      LDS and fp8 A(kt+1) has landed.  The iteration streams B(kt+1) and fp8
  //      A(kt+2) in, converts A(kt+1) a quarter per MFMA phase, multiplies
  //      stage kt, then waits for its loads and meets the other waves.
  bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    load_frags(kt, 0, fa0, fb0);
    if (more) issue_b(kt + 1);
    if (kt + 2 < nk) issue_a8(kt + 2);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    if (more) convert(kt + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 2, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1);
    if (more) convert(kt + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(kt, 3, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    if (more) convert(kt + 1, 2);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1);
    if (more) convert(kt + 1, 3);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  }

  // ---- epilogue (as in the plain kernel) -----------------------------------------
  constexpr int PITCH = WN + 4;
  static_assert(kGgWaves * 32 * PITCH * 4 <= kGgLDS, "epilogue staging must fit");
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * PITCH;
  const bool full = (m0 + kGgBM <= a.M) && (n0 + kGgBN <= a.N) && a.vec_store;
  constexpr int LANES_PER_ROW = WN / 4;
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

hipError_t launch_gemm_gather_fp8(const GatherGemmArgs& g, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  if (g.M == 0 || g.N == 0) return hipSuccess;
  GatherGemmKArgs a;
  a.t0 = g.table[0];
  a.t1 = g.table[1];
  a.t2 = g.table[2];
  a.s0 = g.scale[0];
  a.s1 = g.scale[1];
  a.s2 = g.scale[2];
  a.nblk = g.scale_block ? g.row_dim / g.scale_block : 0;
  a.r0 = (int32_t)g.rows[0];
  a.r1 = (int32_t)g.rows[1];
  a.r2 = (int32_t)g.rows[2];
  a.row_ids = g.row_ids;
  a.rid_ld = g.rid_ld;
  a.split = g.per_site_table ? (1 << 29) : g.heads;  // 2 * split stays below 2^31
  a.pitch = g.pitch;
  a.row_dim = g.row_dim;
  a.seg_pitch = g.seg_pitch;
  a.cols = g.cols;
  a.heads = g.heads;
  a.B = reinterpret_cast<const __bf16*>(g.B);
  a.ldb = g.ldb;
  a.C = g.C;
  a.ldc = g.ldc;
  a.M = g.M;
  a.N = g.N;
  a.K = g.cols * g.seg_pitch;
  a.tiles_m = (g.M + kGgBM - 1) / kGgBM;
  a.tiles_n = (g.N + kGgBN - 1) / kGgBN;
  a.group_m = 2;
  a.vec_store = (g.ldc % 4 == 0 && ((uintptr_t)g.C & 15) == 0) ? 1 : 0;
  if (g.scale_block != 0 && (g.scale_block != 32 || a.nblk < 1 || a.nblk > kGgMaxBlocks))
    return hipErrorInvalidValue;  // the entry point refuses these first
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (g.scale_block) {
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_gather_fp8_kernel<true>),
                                            kGgLDS, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_gather_fp8_kernel<true>, dim3(grid), dim3(kGgThreads), kGgLDS, stream, a);
  } else {
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&gemm_gather_fp8_kernel<false>),
                                            kGgLDS, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_gather_fp8_kernel<false>, dim3(grid), dim3(kGgThreads), kGgLDS, stream, a);
  }
  return hipGetLastError();
}

}  // namespace engram
