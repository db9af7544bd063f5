// lookup.hip -- steps 1 and 2 of a decode step in one launch: compress, rolling hash
// with the store, and the row gather + dequant, for calls in which every sequence is
// one token continuing from its store slot ([VeOmni#1370] "feat: support
// DeepSeek-V4.1-Flash in SeedOmni", n-gram incremental decode cache commit: each decode
// step hashes the new token against the three ids kept per sequence; PR summary: the
// FP8 rows are dequantised with their row scale on lookup).  Included into
// engram_device.hip after hash.hip and gather.hip, whose helpers it uses.
//
// One workgroup per token.  Lanes c < 3H of wave 0 each build the token's window (its
// own compressed id and the slot's three ids) and the row id of hash column c; lane 0
// writes the eid, and the new tail after the workgroup barrier, by which every lane's
// read of the old tail has been used.
// The row ids go to LDS, and the whole workgroup then gathers the token's 3H segments
// in 16-element chunks as gather_dequant_kernel does (e4m3fn codes times the row's fp32
// scale, rounded once to bf16, zeros past the row; each wave's 2 KB of output staged in
// LDS so that its stores write whole lines).  The results equal engram_compress_hash
// (each token its own sequence, seq_start 0 where it has a slot) followed by
// engram_gather_dequant, bit for bit: the same operations on the same values.

namespace engram {

constexpr int kLookupThreads = 256;

__global__ __launch_bounds__(kLookupThreads) void lookup_decode_kernel(LookupArgs a) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cols = 3 * a.heads;
  __shared__ int32_t rid[ENGRAM_MAX_COLUMNS];
  __shared__ u32x4 stage[kLookupThreads / 64][128];

  int slot = -1;
  uint32_t w0 = 0, w1 = 0, w2 = 0;
  if (wave == 0 && lane < cols) {
    // the per-token inputs first, all at once; then the loads that depend on them, at
    // once too: addresses are clamped in bounds and the values selected afterwards, so
    // no load waits on a branch (two dependent rounds instead of three or four)
    const int32_t tok = a.tokens[t];
    const bool dead = a.dead != nullptr && a.dead[t] != 0;
    const int32_t slot_in = a.slots != nullptr ? a.slots[t] : -1;
    const bool tok_ok = tok >= 0 && tok < a.vocab;
    const bool slot_ok = slot_in >= -1 && slot_in < a.num_slots && (slot_in < 0 || a.store != nullptr);
    const uint32_t pad = (uint32_t)a.tid2eid[a.pad_token_id] & kIdMask;
    const uint32_t e = (uint32_t)a.tid2eid[tok_ok ? tok : 0] & kIdMask;
    int32_t s0 = 0, s1 = 0, s2 = 0;
    if (a.store != nullptr) {  // uniform
      const int32_t* st = a.store + 3 * (slot_ok && slot_in >= 0 ? slot_in : 0);
      s0 = st[0];
      s1 = st[1];
      s2 = st[2];
    }
    if (!dead && !tok_ok && lane == 0) latch_error(ENGRAM_E_TOKEN_RANGE);
    if (!slot_ok && lane == 0) latch_error(ENGRAM_E_SLOT_RANGE);
    slot = slot_ok ? slot_in : -1;
    w0 = dead || !tok_ok ? pad : e;
    // the window: a dead token's is all PAD; a token without a slot starts its
    // sequence, so its lookback is PAD; otherwise the slot holds the three earlier ids,
    // oldest first
    const bool back = !dead && slot >= 0;
    w1 = back ? (uint32_t)s2 : pad;
    w2 = back ? (uint32_t)s1 : pad;
    const uint32_t w3 = back ? (uint32_t)s0 : pad;
    const uint64_t k2 = (uint64_t)w0 + (uint64_t)w1 * a.vc1;
    const uint64_t k3 = k2 + (uint64_t)w2 * a.vc2;
    const uint64_t k4 = k3 + (uint64_t)w3 * a.vc3;
    const int order = lane / a.heads;
    const uint64_t key = order == 0 ? k2 : (order == 1 ? k3 : k4);
    const int32_t row = (int32_t)(a.offset[lane] + mod_barrett(key, a.prime[lane], a.barrett[lane]));
    rid[lane] = row;
    a.row_ids[(int64_t)t * cols + lane] = row;
    if (lane == 0) a.eids[t] = (int32_t)w0;
  }
  __syncthreads();
  // the new tail (w2, w1, w0), oldest first: every read of the old one went into a row
  // id in LDS before the barrier
  if (tid == 0 && slot >= 0) {
    int32_t* st = a.store + 3 * slot;
    st[0] = (int32_t)w2;
    st[1] = (int32_t)w1;
    st[2] = (int32_t)w0;
  }

  // the token's 3H segments of seg_pitch elements, chunk g at element 16 g of its row
  const uint32_t total = (uint32_t)cols * a.chunks;
  unsigned short* out = reinterpret_cast<unsigned short*>(a.out) + (int64_t)t * a.out_ld;
  for (uint32_t base = 0; base < total; base += kLookupThreads) {
    const uint32_t g = base + (uint32_t)tid;
    u32x4 o[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (g < total) {
      const uint32_t seg = g / a.chunks, chunk = g - seg * a.chunks;
      const uint32_t e0 = chunk * 16;
      if (e0 < (uint32_t)a.row_dim) {
        const uint32_t n = a.per_site_table ? 0u : seg / (uint32_t)a.heads;
        const int32_t row = rid[seg];
        const int32_t rows = n == 0 ? a.r0 : (n == 1 ? a.r1 : a.r2);
        if (row < 0 || row >= rows) {
          latch_error(ENGRAM_E_ROW_RANGE);
        } else {
          const uint8_t* tb = n == 0 ? a.t0 : (n == 1 ? a.t1 : a.t2);
          const float* sc = n == 0 ? a.s0 : (n == 1 ? a.s1 : a.s2);
          const u32x4 raw = *reinterpret_cast<const u32x4*>(tb + (int64_t)row * a.pitch + e0);
          const float scale = sc[row];
          const uint32_t valid = (uint32_t)a.row_dim - e0 >= 16 ? 16u : (uint32_t)a.row_dim - e0;
          float f[16];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], true);
            f[4 * w + 0] = lo[0] * scale;
            f[4 * w + 1] = lo[1] * scale;
            f[4 * w + 2] = hi[0] * scale;
            f[4 * w + 3] = hi[1] * scale;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((uint32_t)i >= valid) f[i] = 0.0f;
#pragma unroll
          for (int w = 0; w < 8; ++w)
            o[w >> 2][w & 3] = bf16_bits_rne(f[2 * w]) | (bf16_bits_rne(f[2 * w + 1]) << 16);
        }
      }
    }
    // the wave's 64 chunks are 2 KB of consecutive output: stage them and write back
    // transposed, so that each 16-byte store instruction writes 1 KB of whole lines
    u32x4* buf = stage[wave];
    buf[2 * lane] = o[0];
    buf[2 * lane + 1] = o[1];
    const u32x4 s0 = buf[lane], s1 = buf[64 + lane];
    const uint32_t g0 = base + (uint32_t)wave * 64;
    if (g0 + (uint32_t)(lane >> 1) < total)
      __builtin_nontemporal_store(s0, reinterpret_cast<u32x4*>(out + (int64_t)g0 * 16) + lane);
    if (g0 + 32u + (uint32_t)(lane >> 1) < total)
      __builtin_nontemporal_store(s1, reinterpret_cast<u32x4*>(out + (int64_t)g0 * 16) + 64 + lane);
  }
}

hipError_t launch_lookup_decode(const LookupArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  if (a.T == 0) return hipSuccess;
  if (3 * a.heads > 64 || a.chunks < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lookup_decode_kernel, dim3((unsigned)a.T), dim3(kLookupThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace engram
