// abi.cpp -- the extern "C" entry points of include/engram.h: argument checks
// that the host can make without touching device memory, then kernel launches
// on the caller's stream.  Hot calls allocate nothing and never synchronise.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <new>

#include "internal.h"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

thread_local hipError_t g_last_hip = hipSuccess;

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return ENGRAM_OK;
  g_last_hip = e;
  return ENGRAM_E_HIP;
}

}  // namespace

extern "C" int engram_tid2eid_check(const engram_layout* L, const int32_t* d_tid2eid,
                                    int32_t* pad_eid, hipStream_t stream) {
  if (!L || !d_tid2eid || !pad_eid) return ENGRAM_E_ARG;
  int32_t* d_res = nullptr;
  hipError_t me = hipMalloc(&d_res, 3 * sizeof(int32_t));
  if (me != hipSuccess) return hip_status(me);
  int32_t h_res[3] = {0, 0, 0};
  hipError_t e = hipMemcpyAsync(d_res, h_res, sizeof h_res, hipMemcpyHostToDevice, stream);
  engram::MapCheckArgs a;
  a.tid2eid = d_tid2eid;
  a.vocab = (int32_t)L->desc.vocab_size;
  a.vc = (int32_t)L->desc.compressed_vocab;
  a.pad_token_id = (int32_t)L->desc.pad_token_id;
  a.result = d_res;
  if (e == hipSuccess) e = engram::launch_map_check(a, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(h_res, d_res, sizeof h_res, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(d_res);
  if (e != hipSuccess) return hip_status(e);
  if (h_res[0] != 0 || h_res[1] != a.vc - 1) return ENGRAM_E_MAP_RANGE;
  *pad_eid = h_res[2];
  return ENGRAM_OK;
}

// ---- store ------------------------------------------------------------------

static int current_device(int32_t* dev) {
  int d = 0;
  const hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return hip_status(e);
  *dev = d;
  return ENGRAM_OK;
}

// The store belongs to the device that is current now, and was made for a layout
// with the same compressed vocabulary and pad token.
static int store_usable(const engram_store* st, const engram_layout* L) {
  if (!st) return ENGRAM_E_ARG;
  if (L && (st->vc != L->desc.compressed_vocab || st->pad_token_id != L->desc.pad_token_id))
    return ENGRAM_E_ARG;
  int32_t dev = 0;
  const int rc = current_device(&dev);
  if (rc != ENGRAM_OK) return rc;
  return dev == st->device ? ENGRAM_OK : ENGRAM_E_ARG;
}

static int store_op(const engram_store* st, const int32_t* d_slots, int32_t n, int32_t* d_ids,
                    int op, hipStream_t stream) {
  int rc = store_usable(st, nullptr);
  if (rc != ENGRAM_OK) return rc;
  if (d_slots && n < 0) return ENGRAM_E_ARG;
  const int32_t count = d_slots ? n : st->num_slots;
  if (op != engram::STORE_RESET && count > 0 && !d_ids) return ENGRAM_E_ARG;
  engram::StoreArgs a;
  a.store = st->ids;
  a.num_slots = st->num_slots;
  a.slots = d_slots;
  a.n = count;
  a.ids = d_ids;
  a.pad_eid = st->pad_eid;
  a.vc = (int32_t)st->vc;
  a.op = op;
  return hip_status(engram::launch_store_op(a, stream));
}

extern "C" int engram_store_create(const engram_layout* L, int32_t pad_eid, int32_t num_slots,
                                   hipStream_t stream, engram_store** out) {
  if (!L || !out || num_slots < 1) return ENGRAM_E_ARG;
  *out = nullptr;
  if (pad_eid < 0 || pad_eid >= L->desc.compressed_vocab) return ENGRAM_E_ARG;
  engram_store* st = new (std::nothrow) engram_store();
  if (!st) return ENGRAM_E_ARG;
  int rc = current_device(&st->device);
  if (rc != ENGRAM_OK) {
    delete st;
    return rc;
  }
  const hipError_t e = hipMalloc(&st->ids, (size_t)num_slots * 3 * sizeof(int32_t));
  if (e != hipSuccess) {
    delete st;
    return hip_status(e);
  }
  st->num_slots = num_slots;
  st->pad_eid = pad_eid;
  st->vc = L->desc.compressed_vocab;
  st->pad_token_id = L->desc.pad_token_id;
  rc = store_op(st, nullptr, 0, nullptr, engram::STORE_RESET, stream);
  if (rc != ENGRAM_OK) {
    engram_store_destroy(st);
    return rc;
  }
  *out = st;
  return ENGRAM_OK;
}

extern "C" void engram_store_destroy(engram_store* st) {
  if (!st) return;
  (void)hipFree(st->ids);
  delete st;
}

extern "C" int engram_store_query(const engram_store* st, int32_t* num_slots, int32_t* pad_eid) {
  if (!st) return ENGRAM_E_ARG;
  if (num_slots) *num_slots = st->num_slots;
  if (pad_eid) *pad_eid = st->pad_eid;
  return ENGRAM_OK;
}

extern "C" int engram_store_reset(engram_store* st, const int32_t* d_slots, int32_t n,
                                  hipStream_t stream) {
  return store_op(st, d_slots, n, nullptr, engram::STORE_RESET, stream);
}

extern "C" int engram_store_write(engram_store* st, const int32_t* d_slots, int32_t n,
                                  const int32_t* d_ids, hipStream_t stream) {
  return store_op(st, d_slots, n, const_cast<int32_t*>(d_ids), engram::STORE_WRITE, stream);
}

extern "C" int engram_store_read(const engram_store* st, const int32_t* d_slots, int32_t n,
                                 int32_t* d_ids, hipStream_t stream) {
  return store_op(st, d_slots, n, d_ids, engram::STORE_READ, stream);
}

extern "C" int engram_store_rollback(const engram_layout* L, const int32_t* d_tid2eid,
                                    engram_store* st, const int32_t* d_slots, int32_t S,
                                    const int32_t* d_cu_seqlens, int32_t T, const int32_t* d_eids,
                                    const uint8_t* d_dead, const uint8_t* d_seq_start,
                                    const int32_t* d_snapshot, const int32_t* d_keep_len,
                                    hipStream_t stream) {
  if (!L || S < 0 || T < 0) return ENGRAM_E_ARG;
  if (S == 0) return ENGRAM_OK;
  if (!d_tid2eid || !d_slots || !d_cu_seqlens || !d_keep_len) return ENGRAM_E_ARG;
  const int rc = store_usable(st, L);
  if (rc != ENGRAM_OK) return rc;
  if (T > 0 && !d_eids) return ENGRAM_E_ARG;
  if (d_seq_start && !d_snapshot) return ENGRAM_E_ARG;  // continuing sequences need their tails
  engram::RollbackArgs a;
  a.store = st->ids;
  a.num_slots = st->num_slots;
  a.slots = d_slots;
  a.S = S;
  a.T = T;
  a.cu_seqlens = d_cu_seqlens;
  a.eids = d_eids;
  a.dead = d_dead;
  a.seq_start = d_seq_start;
  a.snapshot = d_snapshot;
  a.keep_len = d_keep_len;
  a.tid2eid = d_tid2eid;
  a.pad_token_id = (int32_t)L->desc.pad_token_id;
  return hip_status(engram::launch_store_rollback(a, stream));
}

// ---- 1. compress + hash -------------------------------------------------------

extern "C" int engram_compress_hash(const engram_layout* L, const int32_t* d_tid2eid,
                                    const int32_t* d_tokens, int32_t T,
                                    const int32_t* d_cu_seqlens, int32_t S,
                                    const uint8_t* d_seq_start, const int32_t* d_slots,
                                    engram_store* store, const uint8_t* d_dead, int32_t* d_eids,
                                    int32_t* d_row_ids, hipStream_t stream) {
  if (!L || T < 0 || S < 0 || !d_tid2eid) return ENGRAM_E_ARG;
  if (T > 0 && (S < 1 || !d_tokens || !d_eids || !d_row_ids)) return ENGRAM_E_ARG;
  if (S > 0 && !d_cu_seqlens) return ENGRAM_E_ARG;
  if (store) {
    const int rc = store_usable(store, L);
    if (rc != ENGRAM_OK) return rc;
  }
  int32_t* d_store = store ? store->ids : nullptr;
  const int32_t num_slots = store ? store->num_slots : 0;
  if (T == 0 && S == 0) return ENGRAM_OK;
  engram::HashArgs a;
  a.tid2eid = d_tid2eid;
  a.tokens = d_tokens;
  a.cu_seqlens = d_cu_seqlens;
  a.seq_start = d_seq_start;
  a.slots = d_slots;
  a.store = d_store;
  a.dead = d_dead;
  a.eids = d_eids;
  a.row_ids = d_row_ids;
  a.T = T;
  a.S = S;
  a.num_slots = num_slots;
  a.heads = L->heads;
  a.num_sites = L->num_sites;
  a.vocab = (int32_t)L->desc.vocab_size;
  a.pad_token_id = (int32_t)L->desc.pad_token_id;
  a.vc1 = L->vc_pow[1];
  a.vc2 = L->vc_pow[2];
  a.vc3 = L->vc_pow[3];
  memcpy(a.prime, L->prime, sizeof a.prime);
  memcpy(a.offset, L->offset, sizeof a.offset);
  memcpy(a.barrett, L->barrett, sizeof a.barrett);
  return hip_status(engram::launch_compress_hash(a, stream));
}

// ---- 2. gather + dequant -------------------------------------------------------

// Workgroups of a gather whose tables live in host memory: enough requests in
// flight to fill the host link (~64 KB per workgroup), few enough CUs to leave the
// others free.
constexpr int kHostGatherBlocks = 64;

static bool in_host_memory(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // unknown to HIP: not pinned host memory
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

// in_host_memory for the gather's launch shape, remembered per thread for the last few
// table pointers: a hot call then makes no runtime query.  The answer only chooses
// between the full grid and the grid-stride launch on a few workgroups, which write
// the same output, so a stale entry (memory freed and reallocated elsewhere at the
// same address) can cost speed but never change a result.
static bool in_host_memory_cached(const void* p) {
  constexpr int kEntries = 8;
  thread_local const void* keys[kEntries] = {};
  thread_local bool vals[kEntries] = {};
  thread_local int next = 0;
  for (int i = 0; i < kEntries; ++i)
    if (keys[i] == p) return vals[i];
  const bool v = in_host_memory(p);
  keys[next] = p;
  vals[next] = v;
  next = (next + 1) % kEntries;
  return v;
}

// Resolves the tables and scales one gather reads: the site's three order
// tables, or its one table (entry 0) repeated for every order.
static int site_tables(const engram_layout* L, const void* const* d_tables,
                       const void* const* d_scales, const uint8_t* table[3], const void* scale[3],
                       int64_t rows[3]) {
  const bool bf16_table = L->desc.table_dtype == ENGRAM_DTYPE_BF16;
  const int used = L->per_site_table ? 1 : 3;
  for (int n = 0; n < 3; ++n) {
    const int src = n < used ? n : 0;
    if (!d_tables[src]) return ENGRAM_E_ARG;
    if (!aligned(d_tables[src], 16)) return ENGRAM_E_ALIGN;
    table[n] = static_cast<const uint8_t*>(d_tables[src]);
    scale[n] = nullptr;
    if (!bf16_table) {
      if (!d_scales[src]) return ENGRAM_E_ARG;
      if (L->scale_block == 0 && !aligned(d_scales[src], 4)) return ENGRAM_E_ALIGN;
      scale[n] = d_scales[src];
    }
    rows[n] = L->desc.rows[src];
  }
  return ENGRAM_OK;
}

extern "C" int engram_gather_dequant(const engram_layout* L, const void* const* d_tables,
                                     const void* const* d_scales, const int32_t* d_row_ids,
                                     int32_t site, int32_t T, int32_t out_dtype, void* d_out,
                                     int64_t out_ld, hipStream_t stream) {
  if (!L || T < 0 || !d_tables) return ENGRAM_E_ARG;
  if (site < 0 || site >= L->num_sites) return ENGRAM_E_ARG;
  if (out_dtype != ENGRAM_DTYPE_BF16 && out_dtype != ENGRAM_DTYPE_F32) return ENGRAM_E_ARG;
  const bool bf16_table = L->desc.table_dtype == ENGRAM_DTYPE_BF16;
  if (!bf16_table && !d_scales) return ENGRAM_E_ARG;
  if (T == 0) return ENGRAM_OK;
  if (!d_row_ids || !d_out) return ENGRAM_E_ARG;
  if (out_ld < L->k_pad || out_ld % 8 != 0) return ENGRAM_E_ALIGN;
  if (!aligned(d_out, 16)) return ENGRAM_E_ALIGN;
  engram::GatherArgs g;
  const int rc = site_tables(L, d_tables, d_scales, g.table, g.scale, g.rows);
  if (rc != ENGRAM_OK) return rc;
  g.rid_ld = L->all_cols;
  g.per_site_table = L->per_site_table;
  g.scale_block = L->scale_block;
  g.pitch = L->desc.row_pitch_bytes;
  g.heads = L->heads;
  g.cols = L->cols;
  g.row_dim = L->desc.row_dim;
  g.seg_pitch = (int32_t)L->seg_pitch;
  g.bf16_table = bf16_table ? 1 : 0;
  g.f32_out = out_dtype == ENGRAM_DTYPE_F32 ? 1 : 0;
  // Tables in host memory: the host link bounds the gather long before the CUs do,
  // so it runs as a grid-stride kernel on a few workgroups and leaves the rest of the
  // chip to work overlapping it (the next projection, on another stream).
  g.max_blocks = 0;
  for (int n = 0; n < 3; ++n)
    if (in_host_memory_cached(g.table[n])) g.max_blocks = kHostGatherBlocks;
  const size_t out_elt = out_dtype == ENGRAM_DTYPE_F32 ? 4 : 2;
  g.out_ld = out_ld;
  // one launch covers fewer than 2^31 output chunks; split bigger calls by tokens
  const int64_t chunks_per_token = (int64_t)L->cols * (L->seg_pitch / 16);
  const int64_t max_tokens = ((int64_t)1 << 31) / chunks_per_token - 1;
  const int32_t* site_rows = d_row_ids + (int64_t)site * L->cols;
  for (int64_t t0 = 0; t0 < T; t0 += max_tokens) {
    const int64_t tn = (T - t0 < max_tokens) ? T - t0 : max_tokens;
    g.row_ids = site_rows + t0 * L->all_cols;
    g.out = static_cast<char*>(d_out) + (size_t)t0 * out_ld * out_elt;
    g.T = (int32_t)tn;
    hipError_t e = engram::launch_gather_dequant(g, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  return ENGRAM_OK;
}

// ---- 1 + 2 for a decode step: compress, hash and gather in one launch -------------

extern "C" int engram_lookup_decode(const engram_layout* L, const int32_t* d_tid2eid,
                                    const int32_t* d_tokens, int32_t T, const int32_t* d_slots,
                                    engram_store* store, const uint8_t* d_dead, int32_t* d_eids,
                                    int32_t* d_row_ids, const void* const* d_tables,
                                    const void* const* d_scales, void* d_rows, int64_t rows_ld,
                                    hipStream_t stream) {
  if (!L) return ENGRAM_E_ARG;
  if (L->num_sites != 1 || L->desc.table_dtype != ENGRAM_DTYPE_FP8_E4M3FN || L->scale_block != 0)
    return ENGRAM_E_UNSUPPORTED;
  if (T < 0 || !d_tid2eid || !d_tables || !d_scales) return ENGRAM_E_ARG;
  if (d_slots && !store) return ENGRAM_E_NEED_STORE;
  if (store) {
    const int rc = store_usable(store, L);
    if (rc != ENGRAM_OK) return rc;
  }
  if (T == 0) return ENGRAM_OK;
  if (!d_tokens || !d_eids || !d_row_ids || !d_rows) return ENGRAM_E_ARG;
  if (rows_ld < L->k_pad || rows_ld % 8 != 0) return ENGRAM_E_ALIGN;
  if (!aligned(d_rows, 16)) return ENGRAM_E_ALIGN;
  const uint8_t* table[3];
  const void* scale[3];
  int64_t rows[3];
  const int rc = site_tables(L, d_tables, d_scales, table, scale, rows);
  if (rc != ENGRAM_OK) return rc;
  engram::LookupArgs a;
  a.tid2eid = d_tid2eid;
  a.tokens = d_tokens;
  a.slots = d_slots;
  a.store = store ? store->ids : nullptr;
  a.dead = d_dead;
  a.eids = d_eids;
  a.row_ids = d_row_ids;
  a.T = T;
  a.num_slots = store ? store->num_slots : 0;
  a.heads = L->heads;
  a.vocab = (int32_t)L->desc.vocab_size;
  a.pad_token_id = (int32_t)L->desc.pad_token_id;
  a.vc1 = L->vc_pow[1];
  a.vc2 = L->vc_pow[2];
  a.vc3 = L->vc_pow[3];
  for (int c = 0; c < 3 * L->heads; ++c) {  // site 0's columns come first
    a.prime[c] = L->prime[c];
    a.offset[c] = L->offset[c];
    a.barrett[c] = L->barrett[c];
  }
  a.t0 = table[0];
  a.t1 = table[1];
  a.t2 = table[2];
  a.s0 = static_cast<const float*>(scale[0]);
  a.s1 = static_cast<const float*>(scale[1]);
  a.s2 = static_cast<const float*>(scale[2]);
  a.r0 = (int32_t)rows[0];
  a.r1 = (int32_t)rows[1];
  a.r2 = (int32_t)rows[2];
  a.per_site_table = L->per_site_table;
  a.pitch = L->desc.row_pitch_bytes;
  a.row_dim = L->desc.row_dim;
  a.chunks = (uint32_t)(L->seg_pitch / 16);
  a.out = d_rows;
  a.out_ld = rows_ld;
  return hip_status(engram::launch_lookup_decode(a, stream));
}

// ---- 3. projection + gated residual ---------------------------------------------

extern "C" int engram_project(const engram_layout* L, const void* d_rows, int64_t rows_ld,
                              const void* d_w, int64_t w_ld, int32_t hidden, float* d_v,
                              int32_t T, hipStream_t stream) {
  if (!L || T < 0 || hidden < 1) return ENGRAM_E_ARG;
  if (T == 0) return ENGRAM_OK;
  if (!d_rows || !d_w || !d_v) return ENGRAM_E_ARG;
  if (rows_ld < L->k_pad || w_ld < L->k_pad || rows_ld % 8 || w_ld % 8) return ENGRAM_E_ALIGN;
  if (!aligned(d_rows, 16) || !aligned(d_w, 16) || !aligned(d_v, 4)) return ENGRAM_E_ALIGN;
  engram::GemmArgs g;
  g.A = d_rows;
  g.B = d_w;
  g.C = d_v;
  g.lda = rows_ld;
  g.ldb = w_ld;
  g.ldc = hidden;
  g.M = T;
  g.N = hidden;
  g.K = (int32_t)L->k_pad;
  g.splits = 1;
  g.c_split_stride = 0;
  return hip_status(engram::launch_gemm_bf16_nt(g, stream));
}

extern "C" int engram_packed_weight_bytes(const engram_layout* L, int32_t hidden, int64_t* bytes) {
  if (!L || hidden < 1 || !bytes) return ENGRAM_E_ARG;
  *bytes = (int64_t)((hidden + 31) / 32) * 32 * L->k_pad * 2;
  return ENGRAM_OK;
}

extern "C" int engram_pack_weight(const engram_layout* L, const void* d_w, int64_t w_ld,
                                  int32_t hidden, void* d_packed, hipStream_t stream) {
  if (!L || hidden < 1 || !d_w || !d_packed) return ENGRAM_E_ARG;
  if (w_ld < L->k_pad || w_ld % 8) return ENGRAM_E_ALIGN;
  if (!aligned(d_w, 16) || !aligned(d_packed, 16)) return ENGRAM_E_ALIGN;
  engram::PackWeightArgs g;
  g.W = d_w;
  g.ldw = w_ld;
  g.N = hidden;
  g.K = (int32_t)L->k_pad;
  g.out = d_packed;
  return hip_status(engram::launch_pack_weight(g, stream));
}

extern "C" int engram_project_packed(const engram_layout* L, const void* d_rows, int64_t rows_ld,
                                     const void* d_packed, int32_t hidden, float* d_v, int32_t T,
                                     hipStream_t stream) {
  if (!L || T < 0 || hidden < 1) return ENGRAM_E_ARG;
  if (T == 0) return ENGRAM_OK;
  if (!d_rows || !d_packed || !d_v) return ENGRAM_E_ARG;
  if (rows_ld < L->k_pad || rows_ld % 8) return ENGRAM_E_ALIGN;
  if (!aligned(d_rows, 16) || !aligned(d_packed, 16) || !aligned(d_v, 4)) return ENGRAM_E_ALIGN;
  // the kernel addresses one 256-row tile of rows and the 256 columns of the packed
  // weight one tile reads (16 column tiles of 16) with 32-bit byte offsets
  if ((int64_t)256 * rows_ld * 2 > INT32_MAX || (int64_t)8 * L->k_pad * 64 > INT32_MAX)
    return ENGRAM_E_UNSUPPORTED;
  engram::GemmPackedArgs g;
  g.A = d_rows;
  g.Bp = d_packed;
  g.C = d_v;
  g.lda = rows_ld;
  g.ldc = hidden;
  g.M = T;
  g.N = hidden;
  g.K = (int32_t)L->k_pad;
  return hip_status(engram::launch_gemm_bf16_nt_packed(g, stream));
}

extern "C" int engram_project_splitk(const engram_layout* L, const void* d_rows, int64_t rows_ld,
                                     const void* d_w, int64_t w_ld, int32_t hidden,
                                     float* d_partials, int32_t splits, int32_t T,
                                     hipStream_t stream) {
  if (!L || T < 0 || hidden < 1 || splits < 1) return ENGRAM_E_ARG;
  if (L->k_pad % (64 * (int64_t)splits) != 0) return ENGRAM_E_ALIGN;
  if (T == 0) return ENGRAM_OK;
  if (!d_rows || !d_w || !d_partials) return ENGRAM_E_ARG;
  if (rows_ld < L->k_pad || w_ld < L->k_pad || rows_ld % 8 || w_ld % 8) return ENGRAM_E_ALIGN;
  if (!aligned(d_rows, 16) || !aligned(d_w, 16) || !aligned(d_partials, 4)) return ENGRAM_E_ALIGN;
  engram::GemmArgs g;
  g.A = d_rows;
  g.B = d_w;
  g.C = d_partials;
  g.lda = rows_ld;
  g.ldb = w_ld;
  g.ldc = hidden;
  g.M = T;
  g.N = hidden;
  g.K = (int32_t)L->k_pad;
  g.splits = splits;
  g.c_split_stride = (int64_t)T * hidden;
  return hip_status(engram::launch_gemm_bf16_nt(g, stream));
}

extern "C" int engram_gather_project(const engram_layout* L, const void* const* d_tables,
                                     const void* const* d_scales, const int32_t* d_row_ids,
                                     int32_t site, int32_t T, const void* d_w, int64_t w_ld,
                                     int32_t hidden, float* d_v, hipStream_t stream) {
  if (!L || T < 0 || hidden < 1 || !d_tables || !d_scales) return ENGRAM_E_ARG;
  if (site < 0 || site >= L->num_sites) return ENGRAM_E_ARG;
  if (L->desc.table_dtype != ENGRAM_DTYPE_FP8_E4M3FN) return ENGRAM_E_UNSUPPORTED;
  // (1, 32) block scales: a converting thread keeps a row's e8m0 bytes in registers,
  // at most 8 of them (rows of up to 256 elements, the released layout)
  if (L->scale_block != 0 && L->desc.row_dim > 8 * 32) return ENGRAM_E_UNSUPPORTED;
  if (T == 0) return ENGRAM_OK;
  if (!d_row_ids || !d_w || !d_v) return ENGRAM_E_ARG;
  const int64_t pitch = L->desc.row_pitch_bytes;
  if (pitch < L->seg_pitch || pitch % 16 != 0) return ENGRAM_E_ALIGN;
  if (w_ld < L->k_pad || w_ld % 8 != 0) return ENGRAM_E_ALIGN;
  if (!aligned(d_w, 16) || !aligned(d_v, 4)) return ENGRAM_E_ALIGN;
  engram::GatherGemmArgs g;
  const void* scale[3];
  const int rc = site_tables(L, d_tables, d_scales, g.table, scale, g.rows);
  if (rc != ENGRAM_OK) return rc;
  for (int n = 0; n < 3; ++n)  // rows stream through direct-to-LDS loads: HBM tables only
    if (in_host_memory(g.table[n]) || in_host_memory(scale[n])) return ENGRAM_E_UNSUPPORTED;
  for (int n = 0; n < 3; ++n) {
    // a row's 8 e8m0 bytes are read with one 8-byte load
    if (L->scale_block != 0 && L->desc.row_dim == 8 * 32 && !aligned(scale[n], 8)) return ENGRAM_E_ALIGN;
    g.scale[n] = scale[n];
  }
  g.scale_block = L->scale_block;
  g.row_ids = d_row_ids + (int64_t)site * L->cols;
  g.rid_ld = L->all_cols;
  g.per_site_table = L->per_site_table;
  g.pitch = pitch;
  g.row_dim = L->desc.row_dim;
  g.seg_pitch = (int32_t)L->seg_pitch;
  g.cols = L->cols;
  g.heads = L->heads;
  g.B = d_w;
  g.ldb = w_ld;
  g.C = d_v;
  g.ldc = hidden;
  g.M = T;
  g.N = hidden;
  return hip_status(engram::launch_gemm_gather_fp8(g, stream));
}

extern "C" int engram_gate_add(const engram_layout* L, const float* d_v, int32_t hidden,
                               int32_t hc_mult, const uint8_t* d_keep, void* d_streams,
                               int32_t T, hipStream_t stream) {
  if (!L || T < 0) return ENGRAM_E_ARG;
  if (hc_mult != 4) return ENGRAM_E_UNSUPPORTED;
  if (hidden < 8 || hidden % 8 != 0) return ENGRAM_E_ALIGN;
  if (hidden > 8192) return ENGRAM_E_UNSUPPORTED;
  if (T == 0) return ENGRAM_OK;
  if (!d_v || !d_streams) return ENGRAM_E_ARG;
  if (!aligned(d_v, 16) || !aligned(d_streams, 16)) return ENGRAM_E_ALIGN;
  engram::GateArgs a;
  a.v = d_v;
  a.splits = 1;
  a.split_stride = 0;
  a.v_out = nullptr;
  a.keep = d_keep;
  a.streams = d_streams;
  a.T = T;
  a.hidden = hidden;
  a.hc = hc_mult;
  a.inv_sqrt_hidden = (float)(1.0 / sqrt((double)hidden));
  return hip_status(engram::launch_gate_add(a, stream));
}

extern "C" int engram_gate_add_partials(const engram_layout* L, const float* d_partials,
                                        int32_t splits, int32_t hidden, int32_t hc_mult,
                                        const uint8_t* d_keep, void* d_streams, float* d_v,
                                        int32_t T, hipStream_t stream) {
  if (!L || T < 0 || splits < 1) return ENGRAM_E_ARG;
  if (hc_mult != 4) return ENGRAM_E_UNSUPPORTED;
  if (hidden < 8 || hidden % 8 != 0) return ENGRAM_E_ALIGN;
  if (hidden > 8192) return ENGRAM_E_UNSUPPORTED;
  if (T == 0) return ENGRAM_OK;
  if (!d_partials || !d_streams) return ENGRAM_E_ARG;
  if (!aligned(d_partials, 16) || !aligned(d_streams, 16) || (d_v && !aligned(d_v, 16)))
    return ENGRAM_E_ALIGN;
  engram::GateArgs a;
  a.v = d_partials;
  a.splits = splits;
  a.split_stride = (int64_t)T * hidden;
  a.v_out = d_v;
  a.keep = d_keep;
  a.streams = d_streams;
  a.T = T;
  a.hidden = hidden;
  a.hc = hc_mult;
  a.inv_sqrt_hidden = (float)(1.0 / sqrt((double)hidden));
  return hip_status(engram::launch_gate_add(a, stream));
}

// ---- 3'. the wkv handle: the projection kernel chosen per call ------------------

namespace {

// Calls with at least this many outputs (tokens x hidden), i.e. 64 tiles of
// 256 x 256, take the packed kernel's 256-row tiles.
constexpr int64_t kBigProjection = 64 * 256 * 256;
constexpr int kCUs = 256;

// Split-K factor chosen for a call: the largest of 2, 4, 8 that keeps the 128 x 128
// tiles times the splits within one workgroup per CU, at least 4 k-steps of 64 per
// split, and k_pad a multiple of 64 x splits; 1 when none does.  (Decode, 256 tokens
// x 4,096 outputs: 64 tiles -> 4 splits, measured 24 us against 42 us unsplit.)
int choose_splits(int64_t T, int64_t hidden, int64_t k_pad) {
  const int64_t tiles = ((T + 127) / 128) * ((hidden + 127) / 128);
  int best = 1;
  for (int s = 2; s <= 8; s *= 2)
    if (tiles * s <= kCUs && k_pad % (64 * s) == 0 && k_pad / s >= 256) best = s;
  return best;
}

engram_proj_plan plan_for(int64_t T, int64_t hidden, int64_t k_pad, bool packed, int forced) {
  engram_proj_plan p;
  p.kernel = ENGRAM_PROJ_PLAIN;
  p.splits = 1;
  if (packed && T * hidden >= kBigProjection) {
    p.kernel = ENGRAM_PROJ_PACKED;
    return p;
  }
  const int s = forced > 0 ? forced : (T * hidden >= kBigProjection ? 1 : choose_splits(T, hidden, k_pad));
  if (s > 1) {
    p.kernel = ENGRAM_PROJ_SPLITK;
    p.splits = s;
  }
  return p;
}

// The packed kernel addresses 256 columns of the packed weight with 32-bit offsets.
bool packed_weight_addressable(int64_t k_pad) { return (int64_t)8 * k_pad * 64 <= INT32_MAX; }

int wkv_usable(const engram_wkv* W, const engram_layout* L, int32_t T) {
  if (!W || !L || T < 0 || T > W->max_tokens || W->k_pad != L->k_pad) return ENGRAM_E_ARG;
  int d = 0;
  const hipError_t e = hipGetDevice(&d);
  if (e != hipSuccess) return hip_status(e);
  return d == W->device ? ENGRAM_OK : ENGRAM_E_ARG;
}

int gate_shape(int32_t hidden, int32_t hc_mult) {
  if (hc_mult != 4) return ENGRAM_E_UNSUPPORTED;
  if (hidden < 8 || hidden % 8 != 0) return ENGRAM_E_ALIGN;
  if (hidden > 8192) return ENGRAM_E_UNSUPPORTED;
  return ENGRAM_OK;
}

}  // namespace

extern "C" int engram_projection_plan(const engram_layout* L, int32_t hidden, int32_t T,
                                      int32_t packed, int32_t splits, engram_proj_plan* plan) {
  if (!L || hidden < 1 || T < 0 || splits < 0 || !plan) return ENGRAM_E_ARG;
  *plan = plan_for(T, hidden, L->k_pad, packed != 0 && packed_weight_addressable(L->k_pad), splits);
  return ENGRAM_OK;
}

extern "C" int engram_wkv_create(const engram_layout* L, const void* d_w, int64_t w_ld,
                                 int32_t hidden, int32_t max_tokens, int32_t splits,
                                 hipStream_t stream, engram_wkv** out) {
  if (!L || !d_w || !out || hidden < 1 || max_tokens < 1 || splits < 0 || splits > 64)
    return ENGRAM_E_ARG;
  *out = nullptr;
  if (w_ld < L->k_pad || w_ld % 8 || !aligned(d_w, 16)) return ENGRAM_E_ALIGN;
  if (splits > 1 && L->k_pad % (64 * (int64_t)splits) != 0) return ENGRAM_E_ALIGN;
  engram_wkv* W = new (std::nothrow) engram_wkv();
  if (!W) return ENGRAM_E_ARG;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    delete W;
    return hip_status(e);
  }
  W->device = dev;
  W->w = d_w;
  W->w_ld = w_ld;
  W->hidden = hidden;
  W->max_tokens = max_tokens;
  W->forced_splits = splits;
  W->k_pad = L->k_pad;
  // packed copy: only if some call of up to max_tokens tokens takes the packed kernel
  const bool can_pack = packed_weight_addressable(L->k_pad);
  if (can_pack && (int64_t)max_tokens * hidden >= kBigProjection) {
    int64_t bytes = 0;
    (void)engram_packed_weight_bytes(L, hidden, &bytes);
    e = hipMalloc(&W->packed, (size_t)bytes);
    int rc = e == hipSuccess ? ENGRAM_OK : hip_status(e);
    if (rc == ENGRAM_OK) rc = engram_pack_weight(L, d_w, w_ld, hidden, W->packed, stream);
    if (rc != ENGRAM_OK) {
      engram_wkv_destroy(W);
      return rc;
    }
  }
  // split-K workspace: the largest splits x T x hidden any call will need
  int64_t need = 0;
  for (int64_t T = 1; T <= max_tokens; ++T) {
    const engram_proj_plan p = plan_for(T, hidden, L->k_pad, W->packed != nullptr, splits);
    if (p.kernel == ENGRAM_PROJ_SPLITK && (int64_t)p.splits * T * hidden > need)
      need = (int64_t)p.splits * T * hidden;
    if (p.kernel == ENGRAM_PROJ_PACKED) break;  // every larger call is packed too
  }
  if (need > 0) {
    e = hipMalloc(&W->partials, (size_t)need * sizeof(float));
    if (e != hipSuccess) {
      engram_wkv_destroy(W);
      return hip_status(e);
    }
    W->partial_elems = need;
  }
  *out = W;
  return ENGRAM_OK;
}

extern "C" void engram_wkv_destroy(engram_wkv* W) {
  if (!W) return;
  if (W->packed) (void)hipFree(W->packed);
  if (W->partials) (void)hipFree(W->partials);
  delete W;
}

extern "C" int engram_wkv_plan(const engram_wkv* W, int32_t T, engram_proj_plan* plan) {
  if (!W || !plan || T < 0 || T > W->max_tokens) return ENGRAM_E_ARG;
  *plan = plan_for(T, W->hidden, W->k_pad, W->packed != nullptr, W->forced_splits);
  return ENGRAM_OK;
}

namespace engram {

int wkv_check(const engram_wkv* W, const engram_layout* L, int32_t T) { return wkv_usable(W, L, T); }

engram_proj_plan wkv_plan_for(const engram_wkv* W, int32_t T) {
  return plan_for(T, W->hidden, W->k_pad, W->packed != nullptr, W->forced_splits);
}

// The planned projection of a T-token call into d_v, or (split-K) into the slices
// at d_partials ([splits][T][hidden]; capacity checked by the caller).
int wkv_project_to(const engram_layout* L, const void* d_rows, int64_t rows_ld, const engram_wkv* W,
                   float* d_v, float* d_partials, int32_t T, hipStream_t stream) {
  if (T == 0) return ENGRAM_OK;
  if (!d_v) return ENGRAM_E_ARG;
  const engram_proj_plan p = wkv_plan_for(W, T);
  if (p.kernel == ENGRAM_PROJ_PACKED) {
    const int rc = engram_project_packed(L, d_rows, rows_ld, W->packed, W->hidden, d_v, T, stream);
    if (rc != ENGRAM_E_UNSUPPORTED) return rc;
    // rows too wide for the packed kernel's 32-bit tile offsets: the plain kernel
  } else if (p.kernel == ENGRAM_PROJ_SPLITK) {
    return engram_project_splitk(L, d_rows, rows_ld, W->w, W->w_ld, W->hidden, d_partials,
                                 p.splits, T, stream);
  }
  return engram_project(L, d_rows, rows_ld, W->w, W->w_ld, W->hidden, d_v, T, stream);
}

// The gated add of a T-token call from d_v, or (split-K) from the slices at
// d_partials, summed into d_v first.
int wkv_gate_from(const engram_layout* L, const engram_wkv* W, float* d_v, const float* d_partials,
                  int32_t hc_mult, const uint8_t* d_keep, void* d_streams, int32_t T,
                  hipStream_t stream) {
  const int rc = gate_shape(W->hidden, hc_mult);
  if (rc != ENGRAM_OK) return rc;
  if (T == 0) return ENGRAM_OK;
  const engram_proj_plan p = wkv_plan_for(W, T);
  if (p.kernel == ENGRAM_PROJ_SPLITK)
    return engram_gate_add_partials(L, d_partials, p.splits, W->hidden, hc_mult, d_keep, d_streams,
                                    d_v, T, stream);
  return engram_gate_add(L, d_v, W->hidden, hc_mult, d_keep, d_streams, T, stream);
}

int hip_error_status(hipError_t e) { return hip_status(e); }

}  // namespace engram

extern "C" int engram_wkv_project(const engram_layout* L, const void* d_rows, int64_t rows_ld,
                                  const engram_wkv* W, float* d_v, int32_t T, hipStream_t stream) {
  const int rc = wkv_usable(W, L, T);
  if (rc != ENGRAM_OK) return rc;
  const engram_proj_plan p = engram::wkv_plan_for(W, T);
  if (p.kernel == ENGRAM_PROJ_SPLITK && (int64_t)p.splits * T * W->hidden > W->partial_elems)
    return ENGRAM_E_ARG;
  return engram::wkv_project_to(L, d_rows, rows_ld, W, d_v, W->partials, T, stream);
}

extern "C" int engram_wkv_gate_add(const engram_layout* L, const engram_wkv* W, float* d_v,
                                   int32_t hc_mult, const uint8_t* d_keep, void* d_streams,
                                   int32_t T, hipStream_t stream) {
  const int rc = wkv_usable(W, L, T);
  if (rc != ENGRAM_OK) return rc;
  return engram::wkv_gate_from(L, W, d_v, W->partials, hc_mult, d_keep, d_streams, T, stream);
}

extern "C" int engram_gated_residual(const engram_layout* L, const void* d_rows, int64_t rows_ld,
                                     const engram_wkv* W, int32_t hc_mult, const uint8_t* d_keep,
                                     void* d_streams, float* d_v, int32_t T, hipStream_t stream) {
  int rc = wkv_usable(W, L, T);
  if (rc != ENGRAM_OK) return rc;
  rc = gate_shape(W->hidden, hc_mult);
  if (rc != ENGRAM_OK) return rc;
  if (T == 0) return ENGRAM_OK;
  if (!d_rows || !d_streams || !d_v) return ENGRAM_E_ARG;
  if (!aligned(d_v, 16) || !aligned(d_streams, 16)) return ENGRAM_E_ALIGN;
  rc = engram_wkv_project(L, d_rows, rows_ld, W, d_v, T, stream);
  if (rc != ENGRAM_OK) return rc;
  return engram_wkv_gate_add(L, W, d_v, hc_mult, d_keep, d_streams, T, stream);
}

extern "C" int engram_get_error(hipStream_t stream) {
  int status = 0;
  hipError_t e = engram::read_and_clear_device_error(stream, &status);
  if (e != hipSuccess) return hip_status(e);
  return status;
}

extern "C" const char* engram_last_hip_error(void) { return hipGetErrorName(g_last_hip); }

#ifndef ENGRAM_BUILD_ID
#define ENGRAM_BUILD_ID "engram-src-sha256:unknown"
#endif
extern "C" const char* engram_build_id(void) { return ENGRAM_BUILD_ID; }

extern "C" int engram_host_device_pointer(const void* host, void** dev) {
  if (!host || !dev) return ENGRAM_E_ARG;
  *dev = nullptr;
  return hip_status(hipHostGetDevicePointer(dev, const_cast<void*>(host), 0));
}
