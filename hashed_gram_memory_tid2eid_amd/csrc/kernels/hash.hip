// hash.hip -- compress + rolling n-gram hash, the slot store, and the tid2eid
// set-up check.  Included into engram_device.hip (one device translation unit
// so that every kernel can latch the device status word).
//
// One lane per token.  A wave covers 64 consecutive tokens of the flattened
// batch; the three lookback ids of every lane come from its neighbours through
// cross-lane shuffles, and lanes 0..2 additionally fetch the three tokens in
// front of the wave (the halo).  Blocking (sequence starts, dead positions) is
// decided per lane from the shuffled dead bits and the lane's sequence start,
// found by a binary search over cu_seqlens.
//
// Hash ([VeOmni#1370] "feat: support DeepSeek-V4.1-Flash in SeedOmni", n-gram
// memory lookup commit: hash multipliers derive from the compressed vocab
// size): key_n = sum_{j<n} w_j V_c^j, exact in 64 bits since V_c <= 2^16, then
// key mod p by Barrett reduction with the host-computed m = floor((2^64-1)/p):
// q' = mulhi(key, m) is q or q-1, so one conditional subtraction finishes it.

namespace engram {

constexpr uint32_t kDeadBit = 1u << 30;
constexpr uint32_t kIdMask = kDeadBit - 1;

__device__ __forceinline__ uint32_t mod_barrett(uint64_t key, uint32_t p, uint64_t m) {
  const uint64_t q = __umul64hi(key, m);
  uint64_t r = key - q * (uint64_t)p;
  if (r >= p) r -= p;
  return (uint32_t)r;
}

// Compressed id of position q packed with its dead bit.  Only the owning lane
// reports an out-of-range token (`report`), the halo copies stay silent.
__device__ __forceinline__ uint32_t packed_eid(const HashArgs& a, int q, uint32_t pad,
                                               bool report) {
  const bool dead = a.dead != nullptr && a.dead[q] != 0;
  if (dead) return pad | kDeadBit;
  const int32_t tok = a.tokens[q];
  if (tok < 0 || tok >= a.vocab) {
    if (report) latch_error(ENGRAM_E_TOKEN_RANGE);
    return pad;
  }
  return (uint32_t)a.tid2eid[tok] & kIdMask;
}

// Largest s in [0, S) with cu[s] <= t (cu[0] = 0 <= t < T = cu[S]).  The first probe
// is the sequence an even split of the T tokens over the S sequences puts t in: exact
// for decode steps (one token per sequence) and equal-length batches, where the
// search is one pair of independent loads instead of a chain of log2(S); otherwise
// it narrows a binary search.  The result stays in [0, S) even for malformed
// cu_seqlens (which the kernel latches).
__device__ __forceinline__ int find_sequence(const int32_t* cu, int S, int T, int t, int* next) {
  int lo = 0, hi = S - 1;
  int g = (int)((int64_t)t * S / (T > 0 ? T : 1));
  g = g < S - 1 ? g : S - 1;
  const int cg = cu[g], cg1 = cu[g + 1];
  if (cg <= t) {
    if (cg1 > t) {
      *next = cg1;
      return g;
    }
    lo = g + 1 < S - 1 ? g + 1 : S - 1;
  } else {
    hi = g - 1 > 0 ? g - 1 : 0;
  }
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  *next = cu[lo + 1];
  return lo;
}

// The workgroup of 256 tokens that updates sequence s's store slot inside the hash
// kernel: the one holding both its first and its last position (an empty sequence:
// its start, or the call's last token when it starts at T).  -1 when the sequence
// spans two workgroups or its bounds are malformed; store_update_kernel then does it.
__device__ __forceinline__ int store_owner(int b0, int b1, int T) {
  if (b0 < 0 || b1 < b0 || b1 > T) return -1;
  int lo, hi;
  if (b1 > b0) {
    lo = b0;
    hi = b1 - 1;
  } else {
    lo = b0 < T ? b0 : (T > 0 ? T - 1 : 0);
    hi = lo;
  }
  return (lo >> 8) == (hi >> 8) ? (lo >> 8) : -1;
}

// An empty sequence q of the call leaves its slot as it was, or PAD when it starts
// here.
__device__ __forceinline__ void empty_slot(const HashArgs& a, int q, int32_t pad) {
  const int slot = a.slots[q];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    latch_error(ENGRAM_E_SLOT_RANGE);
    return;
  }
  if (a.seq_start == nullptr || a.seq_start[q] != 0) {
    int32_t* st = a.store + 3 * slot;
    st[0] = pad;
    st[1] = pad;
    st[2] = pad;
  }
}

// One lane's token t: window with lookback blocking, keys, row ids of every site.
// With the store updated in this kernel: the window of a sequence's last position
// holds the sequence's new tail (its three newest ids, oldest first: w3 is dropped,
// and a dead position's all-PAD window is the PAD tail); when the whole sequence
// lies in this workgroup its last lane returns that slot in *pending and the ids in
// tail[], to be written after the workgroup barrier.  The lane of a sequence's last
// position also settles the empty sequences right after it, and lane 0 those before
// the first position (an empty sequence's slot is read by no lane).
__device__ __forceinline__ void hash_lane(const HashArgs& a, int t, uint32_t own,
                                          const uint32_t prev[4], uint32_t pad, int* pending,
                                          int32_t tail[3]) {
  int b1 = 0;
  const int s = find_sequence(a.cu_seqlens, a.S, a.T, t, &b1);
  int start = a.cu_seqlens[s];
  if (start > t) {  // only when cu_seqlens[0] > 0, already latched above
    start = t;
  }
  const bool starts = a.seq_start == nullptr || a.seq_start[s] != 0;
  int slot = a.slots != nullptr ? a.slots[s] : -1;
  if (slot < -1 || slot >= a.num_slots || (slot >= 0 && a.store == nullptr)) {
    latch_error(ENGRAM_E_SLOT_RANGE);
    slot = -1;
  }

  uint32_t w[4];
  bool blocked = (own & kDeadBit) != 0;
  w[0] = own & kIdMask;  // pad when dead
#pragma unroll
  for (int j = 1; j <= 3; ++j) {
    const int q = t - j;
    uint32_t val = pad;
    if (!blocked) {
      if (q >= start) {
        if (prev[j] & kDeadBit)
          blocked = true;
        else
          val = prev[j] & kIdMask;
      } else if (starts) {
        blocked = true;
      } else if (slot < 0) {
        latch_error(ENGRAM_E_NEED_STORE);
        blocked = true;
      } else {
        val = (uint32_t)a.store[3 * slot + 3 - (start - q)];
      }
    }
    w[j] = blocked ? pad : val;
  }

  const uint64_t k2 = (uint64_t)w[0] + (uint64_t)w[1] * a.vc1;
  const uint64_t k3 = k2 + (uint64_t)w[2] * a.vc2;
  const uint64_t k4 = k3 + (uint64_t)w[3] * a.vc3;
  a.eids[t] = (int32_t)w[0];
  if (a.store_in_kernel && t == b1 - 1) {
    if (slot >= 0 && store_owner(start, b1, a.T) == (t >> 8)) {
      *pending = slot;
      tail[0] = (int32_t)w[2];
      tail[1] = (int32_t)w[1];
      tail[2] = (int32_t)w[0];
    }
    for (int q = s + 1; q < a.S && a.cu_seqlens[q + 1] == b1; ++q) empty_slot(a, q, (int32_t)pad);
  }
  if (a.store_in_kernel && t == 0)
    for (int q = 0; q < s; ++q) empty_slot(a, q, (int32_t)pad);
  // every site from the same keys: [site][order][head]
  const int cols = 3 * a.heads;
  int32_t* out = a.row_ids + (int64_t)t * (cols * a.num_sites);
  for (int st = 0; st < a.num_sites; ++st) {
    const int base = st * cols;
    for (int h = 0; h < a.heads; ++h) {
      const int c2 = base + h;
      out[c2] = (int32_t)(a.offset[c2] + mod_barrett(k2, a.prime[c2], a.barrett[c2]));
      const int c3 = base + a.heads + h;
      out[c3] = (int32_t)(a.offset[c3] + mod_barrett(k3, a.prime[c3], a.barrett[c3]));
      const int c4 = base + 2 * a.heads + h;
      out[c4] = (int32_t)(a.offset[c4] + mod_barrett(k4, a.prime[c4], a.barrett[c4]));
    }
  }
}

// The three window ids that follow position `last` of a sequence whose
// positions in this call start at b0, oldest first in out[0..2]: walking back
// from `last`, a dead position reads PAD and blocks everything before it; the
// walk continues into the ids before the call (prev, oldest first) unless the
// sequence starts in this call, which blocks.  last < b0 means no position of
// the call is kept: the ids before the call (or PAD) stand.
__device__ __forceinline__ void tail_after(const int32_t* eids, const uint8_t* dead, int b0, int last,
                                           bool starts, const int32_t* prev, int32_t pad,
                                           int32_t out[3]) {
  int32_t w[3];
  bool blocked = false;
  for (int j = 0; j <= 2; ++j) {
    const int q = last - j;
    int32_t val = pad;
    if (!blocked) {
      if (q >= b0) {
        if (dead != nullptr && dead[q] != 0)
          blocked = true;
        else
          val = eids[q];
      } else if (starts) {
        blocked = true;
      } else {
        val = prev[3 - (b0 - q)];
      }
    }
    w[j] = blocked ? pad : val;
  }
  out[0] = w[2];
  out[1] = w[1];
  out[2] = w[0];
}

// Sequence s (well-formed bounds b0 <= b1 in its call) leaves its last three
// window ids, oldest first, in its slot.
__device__ void update_slot(const HashArgs& a, int s, int b0, int b1) {
  const int slot = a.slots[s];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    latch_error(ENGRAM_E_SLOT_RANGE);
    return;
  }
  const int32_t pad = a.tid2eid[a.pad_token_id];
  const bool starts = a.seq_start == nullptr || a.seq_start[s] != 0;
  int32_t* st = a.store + 3 * slot;
  int32_t w[3];
  tail_after(a.eids, a.dead, b0, b1 - 1, starts, st, pad, w);
  st[0] = w[0];
  st[1] = w[1];
  st[2] = w[2];
}

__global__ __launch_bounds__(256) void compress_hash_kernel(HashArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const bool valid = t < a.T;
  const uint32_t pad = (uint32_t)a.tid2eid[a.pad_token_id] & kIdMask;

  // cu_seqlens must be 0 = c0 <= c1 <= ... <= cS = T.
  if (t < a.S && a.cu_seqlens[t] > a.cu_seqlens[t + 1]) latch_error(ENGRAM_E_SEQLENS);
  if (t == 0 && (a.cu_seqlens[0] != 0 || a.cu_seqlens[a.S] != a.T)) latch_error(ENGRAM_E_SEQLENS);

  const uint32_t own = valid ? packed_eid(a, t, pad, true) : 0u;
  uint32_t halo = 0u;
  if (lane < 3) {
    const int q = (t - lane) - 3 + lane;  // the three positions before the wave
    if (q >= 0 && q < a.T) halo = packed_eid(a, q, pad, false);
  }
  // prev[j] = packed id of position t - j (all lanes take part in the shuffles)
  uint32_t prev[4];
#pragma unroll
  for (int j = 1; j <= 3; ++j) {
    const uint32_t from_wave = __shfl_up(own, (unsigned)j, 64);
    const uint32_t from_halo = __shfl(halo, (lane - j + 3) & 63, 64);
    prev[j] = lane >= j ? from_wave : from_halo;
  }
  int pending = -1;
  int32_t tail[3];
  if (valid) hash_lane(a, t, own, prev, pad, &pending, tail);
  if (!a.store_in_kernel) return;

  // the new tails of the sequences that lie in this workgroup: every read of their
  // old slot content (by their first three positions, all in this workgroup) happens
  // before the barrier
  __syncthreads();
  if (pending >= 0) {
    int32_t* st = a.store + 3 * pending;
    st[0] = tail[0];
    st[1] = tail[1];
    st[2] = tail[2];
  }
}

// One thread per sequence, for the slots the hash kernel did not update: sequences
// that span two of its workgroups (or every sequence of a call without tokens).
// Runs after compress_hash_kernel on the same stream, so every read of the old slot
// content has happened.
__global__ __launch_bounds__(256) void store_update_kernel(HashArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.S) return;
  const int b0 = a.cu_seqlens[s], b1 = a.cu_seqlens[s + 1];
  if (b0 < 0 || b1 > a.T || b1 < b0) return;  // malformed: latched by the hash kernel
  if (a.store_in_kernel && (b1 == b0 || store_owner(b0, b1, a.T) >= 0)) return;  // done there
  update_slot(a, s, b0, b1);
}

// Speculative rollback: each slot is set to the tail it would hold had the last
// call covered only the first keep_len[s] tokens of sequence s.  The tail
// before that call is the caller's snapshot (read with engram_store_read before
// the call); the call's compressed ids and dead mask supply the rest.  A tail is
// three ids, so the snapshot is the state itself and the replay touches at most
// the last three kept positions.
__global__ __launch_bounds__(256) void store_rollback_kernel(RollbackArgs a) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= a.S) return;
  const int slot = a.slots[s];
  if (slot < 0) return;
  if (slot >= a.num_slots) {
    latch_error(ENGRAM_E_SLOT_RANGE);
    return;
  }
  const int b0 = a.cu_seqlens[s], b1 = a.cu_seqlens[s + 1];
  const int keep = a.keep_len[s];
  if (b0 < 0 || b1 > a.T || b1 < b0 || keep < 0 || keep > b1 - b0) {
    latch_error(ENGRAM_E_SEQLENS);
    return;
  }
  const int32_t pad = a.tid2eid[a.pad_token_id];
  const bool starts = a.seq_start == nullptr || a.seq_start[s] != 0;
  int32_t w[3];
  tail_after(a.eids, a.dead, b0, b0 + keep - 1, starts, a.snapshot + 3 * (int64_t)s, pad, w);
  int32_t* st = a.store + 3 * (int64_t)slot;
  st[0] = w[0];
  st[1] = w[1];
  st[2] = w[2];
}

hipError_t launch_store_rollback(const RollbackArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  if (a.S == 0) return hipSuccess;
  hipLaunchKernelGGL(store_rollback_kernel, dim3((a.S + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_compress_hash(const HashArgs& args, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  HashArgs a = args;
  const bool with_store = a.slots != nullptr && a.store != nullptr && a.S > 0;
  a.store_in_kernel = (with_store && a.T > 0) ? 1 : 0;
  const int work = a.T > a.S + 1 ? a.T : a.S + 1;
  const int blocks = (work + 255) / 256;
  hipLaunchKernelGGL(compress_hash_kernel, dim3(blocks), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // with 1..256 tokens one workgroup holds every position, so every slot was settled
  // inside the hash kernel; otherwise the sequences that span two workgroups (or, with
  // no tokens, all of them) are left to a second kernel
  if (with_store && (a.T > 256 || a.T == 0)) {
    hipLaunchKernelGGL(store_update_kernel, dim3((a.S + 255) / 256), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// tid2eid set-up check: count ids outside [0, V_c), find the largest id, and
// report the pad id.
__global__ __launch_bounds__(256) void map_check_kernel(MapCheckArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) a.result[2] = a.tid2eid[a.pad_token_id];
  if (i >= a.vocab) return;
  const int32_t e = a.tid2eid[i];
  if (e < 0 || e >= a.vc) atomicAdd(&a.result[0], 1);
  atomicMax(&a.result[1], e);
}

hipError_t launch_map_check(const MapCheckArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  hipLaunchKernelGGL(map_check_kernel, dim3((a.vocab + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Store helpers (reset / write / read by slot), one thread per (slot, column).
__global__ __launch_bounds__(256) void store_op_kernel(StoreArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = (a.slots == nullptr ? (int64_t)a.num_slots : (int64_t)a.n) * 3;
  if (i >= count) return;
  const int64_t r = i / 3, c = i - r * 3;
  const int32_t slot = a.slots == nullptr ? (int32_t)r : a.slots[r];
  if (slot < 0 || slot >= a.num_slots) {
    latch_error(ENGRAM_E_SLOT_RANGE);
    return;
  }
  int32_t* cell = a.store + 3 * (int64_t)slot + c;
  if (a.op == STORE_RESET) {
    *cell = a.pad_eid;
  } else if (a.op == STORE_WRITE) {
    // a row with any id outside [0, vc) is not written at all
    const int32_t* row = a.ids + 3 * r;
    bool ok = true;
    for (int j = 0; j < 3; ++j) ok = ok && row[j] >= 0 && row[j] < a.vc;
    if (!ok) {
      if (c == 0) latch_error(ENGRAM_E_ID_RANGE);
      return;
    }
    *cell = row[c];
  } else {
    a.ids[i] = *cell;
  }
}

hipError_t launch_store_op(const StoreArgs& a, hipStream_t stream) {
  (void)hipGetLastError();  // drop a stale error another library left on this thread
  const int64_t count = (a.slots == nullptr ? (int64_t)a.num_slots : (int64_t)a.n) * 3;
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(store_op_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace engram
