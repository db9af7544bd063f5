// internal.h -- declarations shared by the library's host and device translation
// units (not part of the public ABI in include/engram.h).
#pragma once

#include <stdint.h>

#include "../../include/engram.h"

struct engram_layout {
  engram_layout_desc desc;
  int64_t floor;
  int32_t heads;
  int32_t cols;                          // 3 * heads: hash columns of one site
  int32_t num_sites;
  int32_t all_cols;                      // num_sites * cols: ints per token of row_ids
  int32_t per_site_table;                // ENGRAM_TABLE_PER_SITE
  int32_t scale_block;                   // 0 (fp32 per row) or 32 (e8m0 per 32 elements)
  uint32_t prime[ENGRAM_MAX_COLUMNS];    // [site][order][head]
  uint32_t offset[ENGRAM_MAX_COLUMNS];
  uint64_t barrett[ENGRAM_MAX_COLUMNS];  // floor((2^64 - 1) / prime)
  int64_t prime_sum[ENGRAM_MAX_SITES][3];
  int64_t seg_pitch;                     // round_up(D, 64) elements
  int64_t k_pad;                         // cols * seg_pitch
  uint64_t vc_pow[4];                    // V_c^0 .. V_c^3
};

// A rolling store: device int32 [num_slots][3] owned by the handle, bound to the
// compressed vocabulary and pad id of the layout it was made for.
struct engram_store {
  int32_t* ids;
  int32_t num_slots;
  int32_t pad_eid;
  int64_t vc;
  int64_t pad_token_id;
  int32_t device;
};

// A site's projection weight: the caller's bf16 [hidden][w_ld] matrix, its packed
// copy (or null) and the split-K workspace (or null), owned by the handle.
struct engram_wkv {
  const void* w;
  int64_t w_ld;
  int32_t hidden;
  int32_t max_tokens;
  int32_t forced_splits;   // 0: chosen per call
  int64_t k_pad;
  void* packed;            // packed weight, or null
  float* partials;         // float [splits][T][hidden] workspace, or null
  int64_t partial_elems;   // capacity of partials
  int32_t device;
};

namespace engram {

// Device-side status word (one per device, see engram_get_error).
hipError_t read_and_clear_device_error(hipStream_t stream, int* status);

struct HashArgs {
  const int32_t* tid2eid;
  const int32_t* tokens;
  const int32_t* cu_seqlens;
  const uint8_t* seq_start;
  const int32_t* slots;
  int32_t* store;
  const uint8_t* dead;
  int32_t* eids;
  int32_t* row_ids;
  int32_t T, S, num_slots, heads;
  int32_t num_sites;
  int32_t vocab, pad_token_id;
  uint64_t vc1, vc2, vc3;
  uint32_t prime[ENGRAM_MAX_COLUMNS];
  uint32_t offset[ENGRAM_MAX_COLUMNS];
  uint64_t barrett[ENGRAM_MAX_COLUMNS];
  int32_t store_in_kernel;  // set by the launcher: slots inside one workgroup updated in the hash kernel
};
hipError_t launch_compress_hash(const HashArgs& a, hipStream_t stream);

// One decode step's compress + hash + gather in one launch (every sequence one token
// continuing from its slot; one site; e4m3fn tables with fp32 row scales; bf16 rows).
struct LookupArgs {
  const int32_t* tid2eid;
  const int32_t* tokens;
  const int32_t* slots;   // [T] or NULL (= every token starts its sequence)
  int32_t* store;         // [num_slots][3] or NULL
  const uint8_t* dead;    // [T] or NULL
  int32_t* eids;          // [T]
  int32_t* row_ids;       // [T][3H]
  int32_t T, num_slots, heads, vocab, pad_token_id;
  uint64_t vc1, vc2, vc3;
  uint32_t prime[3 * ENGRAM_MAX_HEADS];  // site 0's columns, [order][head]
  uint32_t offset[3 * ENGRAM_MAX_HEADS];
  uint64_t barrett[3 * ENGRAM_MAX_HEADS];
  const uint8_t* t0;
  const uint8_t* t1;
  const uint8_t* t2;
  const float* s0;
  const float* s1;
  const float* s2;
  int32_t r0, r1, r2;     // rows per table
  int32_t per_site_table; // every segment reads t0
  int64_t pitch;          // bytes per table row
  int32_t row_dim;
  uint32_t chunks;        // seg_pitch / 16
  void* out;              // bf16 [T][out_ld]
  int64_t out_ld;
};
hipError_t launch_lookup_decode(const LookupArgs& a, hipStream_t stream);

struct MapCheckArgs {
  const int32_t* tid2eid;
  int32_t vocab, vc, pad_token_id;
  int32_t* result;  // device int32[3]: {bad count, max id, pad id}
};
hipError_t launch_map_check(const MapCheckArgs& a, hipStream_t stream);

struct RollbackArgs {
  int32_t* store;
  int32_t num_slots;
  const int32_t* slots;       // [S]
  int32_t S, T;
  const int32_t* cu_seqlens;  // [S+1] of the call being rolled back
  const int32_t* eids;        // [T] of that call
  const uint8_t* dead;        // [T] or NULL
  const uint8_t* seq_start;   // [S] or NULL (= every sequence started in that call)
  const int32_t* snapshot;    // [S][3] tails before that call
  const int32_t* keep_len;    // [S]
  const int32_t* tid2eid;
  int32_t pad_token_id;
};
hipError_t launch_store_rollback(const RollbackArgs& a, hipStream_t stream);

enum StoreOp { STORE_RESET = 0, STORE_WRITE = 1, STORE_READ = 2 };
struct StoreArgs {
  int32_t* store;
  int32_t num_slots;
  const int32_t* slots;  // NULL = all slots (reset only)
  int32_t n;
  int32_t* ids;          // [n][3]
  int32_t pad_eid;
  int32_t vc;            // STORE_WRITE: ids must lie in [0, vc)
  int32_t op;
};
hipError_t launch_store_op(const StoreArgs& a, hipStream_t stream);

struct GatherArgs {
  const uint8_t* table[3];
  const void* scale[3];    // float [rows] or uint8 e8m0 [rows][D/32]
  int64_t rows[3];
  const int32_t* row_ids;  // the site's first column; tokens rid_ld ints apart
  int32_t rid_ld;
  int32_t per_site_table;  // every segment reads table[0]
  int32_t scale_block;     // 0 or 32
  void* out;
  int64_t out_ld;          // elements
  int64_t pitch;           // bytes
  int32_t T, heads, cols, row_dim, seg_pitch;
  int32_t bf16_table;      // 0: e4m3fn + fp32 scale, 1: bf16
  int32_t f32_out;         // 0: bf16 out, 1: fp32 out
  int32_t max_blocks;      // > 0: at most this many workgroups (grid-stride), 0: one per block
};
hipError_t launch_gather_dequant(const GatherArgs& a, hipStream_t stream);

struct GemmArgs {
  const void* A;   // bf16 [M][lda]
  const void* B;   // bf16 [N][ldb]
  float* C;        // f32 [M][ldc]
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t splits;          // 1: C = A B^T; > 1: split-K partial slices of C
  int64_t c_split_stride;  // elements between partial slices
};
hipError_t launch_gemm_bf16_nt(const GemmArgs& a, hipStream_t stream);

// The projection weight in matrix-core fragment order (see kernels/gemm_packed.hip):
// out[N16][K32][64][8] bf16, N16 = ceil(N / 16), K32 = K / 32, rows past N zero.
struct PackWeightArgs {
  const void* W;   // bf16 [N][ldw]
  int64_t ldw;
  int32_t N, K;    // K multiple of 32
  void* out;
};
hipError_t launch_pack_weight(const PackWeightArgs& a, hipStream_t stream);

struct GemmPackedArgs {
  const void* A;   // bf16 [M][lda]
  const void* Bp;  // packed weight of [N][K]
  float* C;        // f32 [M][ldc]
  int64_t lda, ldc;
  int32_t M, N, K;
};
hipError_t launch_gemm_bf16_nt_packed(const GemmPackedArgs& a, hipStream_t stream);

// Fused gather + dequant + projection for e4m3fn tables: C = A B^T where row t of
// A is the dequantised concatenation of the rows that row_ids[t] names.
struct GatherGemmArgs {
  const uint8_t* table[3];
  const void* scale[3];    // float [rows] or uint8 e8m0 [rows][D/32]
  int32_t scale_block;     // 0 or 32
  int64_t rows[3];
  const int32_t* row_ids;  // the site's first column; tokens rid_ld ints apart
  int32_t rid_ld;
  int32_t per_site_table;  // every segment reads table[0]
  int64_t pitch;           // bytes, >= seg_pitch, multiple of 16
  int32_t row_dim, seg_pitch, cols, heads;
  const void* B;           // bf16 [N][ldb], ldb >= cols * seg_pitch
  int64_t ldb;
  float* C;                // f32 [M][ldc]
  int64_t ldc;
  int32_t M, N;
};
hipError_t launch_gemm_gather_fp8(const GatherGemmArgs& a, hipStream_t stream);

struct GateArgs {
  const float* v;         // [T][hidden], or [splits][T][hidden] partial slices
  int32_t splits;         // >= 1: v is the sum of the slices, in slice order
  int64_t split_stride;   // elements between slices
  float* v_out;           // optional: the summed v is written here
  const uint8_t* keep;    // [T] or NULL
  void* streams;          // bf16 [T][hc][hidden]
  int32_t T, hidden, hc;
  float inv_sqrt_hidden;
};
hipError_t launch_gate_add(const GateArgs& a, hipStream_t stream);

// The wkv handle's dispatch (abi.cpp), shared by the entry points that bring their
// own scratch: the argument check of a T-token call, its plan, the planned
// projection into d_v or the split-K slices at d_partials, and the gated add from
// them; and the status of a failed HIP call (recorded for engram_last_hip_error).
int wkv_check(const engram_wkv* W, const engram_layout* L, int32_t T);
engram_proj_plan wkv_plan_for(const engram_wkv* W, int32_t T);
int wkv_project_to(const engram_layout* L, const void* d_rows, int64_t rows_ld, const engram_wkv* W,
                   float* d_v, float* d_partials, int32_t T, hipStream_t stream);
int wkv_gate_from(const engram_layout* L, const engram_wkv* W, float* d_v, const float* d_partials,
                  int32_t hc_mult, const uint8_t* d_keep, void* d_streams, int32_t T,
                  hipStream_t stream);
int hip_error_status(hipError_t e);

}  // namespace engram
