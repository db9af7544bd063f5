/*
 * engram.h -- C ABI of the MI355X (gfx950) Engram n-gram memory hot path.
 *
 * The path, in the order the calls run:
 *   1. engram_compress_hash   token ids -> compressed ids (tid2eid) -> rolling
 *                             2/3/4-gram windows -> hashed row ids, with a
 *                             slot-keyed store of the last three ids for decode;
 *   2. engram_gather_dequant  row ids -> e4m3fn (or bf16) table rows from HBM ->
 *                             row-wise dequantised bf16 (or fp32) rows;
 *   3. engram_gated_residual  rows -> wkv down-projection (MFMA) -> per-stream
 *                             sigmoid gate -> residual add into the hc streams,
 *                             from a weight handle (engram_wkv_create) that picks
 *                             the projection kernel per call; engram_wkv_project +
 *                             engram_wkv_gate_add are its two halves, and
 *                             engram_project* / engram_gate_add* the single
 *                             kernels it dispatches to.
 *   engram_gather_project     steps 2 and the projection in one kernel for
 *                             e4m3fn tables (rows stay on chip).
 *   engram_project_splitk +   the projection split over K for few tokens
 *   engram_gate_add_partials  (decode), summed deterministically in the gate.
 *   engram_lookup_decode      steps 1 and 2 of a decode step (one token per
 *                             sequence, continuing from the store) in one launch.
 *   engram_store_*            the rolling store: reset, write, read (snapshot)
 *                             and rollback to accepted lengths.
 *   One layout may describe several Engram sites sharing one hash pass; the
 *   gathers then take a site index.  Tables may live in HBM or in pinned host
 *   memory (engram_host_device_pointer).
 *
 * Pages defining the operations (titles; sections named):
 *  [VeOmni#1370] GitHub PR "feat: support DeepSeek-V4.1-Flash in SeedOmni"
 *                (ByteDance-Seed/VeOmni #1370).
 *  [NeMo-V41]    NeMo AutoModel API page
 *                "nemo_automodel.components.models.deepseek_v41.model".
 *  [vLLM-V41]    vLLM docs page "vllm/models/deepseek_v41/nvidia/model".
 *
 * Conventions for every call:
 *  - Return value: ENGRAM_OK (0) or a negative ENGRAM_E_* status.  Argument
 *    errors that the host can see are returned at once and nothing is launched.
 *  - Device pointers ("d_" prefix) are caller-owned device memory on the
 *    current HIP device; the library never frees or keeps them.  Host pointers
 *    have no prefix.  Sizes are element counts unless the name says bytes.
 *  - Hot calls (compress_hash, gather_dequant, gather_project, project*,
 *    gate_add*, gated_residual, wkv_project, wkv_gate_add, store_reset / write /
 *    read / rollback) allocate nothing, never synchronise, and only enqueue
 *    kernels on `stream`; none records a memset, so a caller may capture them in
 *    a HIP graph.  Set-up calls (*_create, tid2eid_check) may allocate and
 *    synchronise.
 *  - Faults that only the device can see (a token id outside the vocabulary,
 *    a row id outside its table, a bad slot, malformed cu_seqlens, a continuing
 *    sequence without a store) latch the first such status in a per-device
 *    error word; the affected outputs are unspecified.  engram_get_error()
 *    synchronises, returns that status and clears it.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define ENGRAM_OK 0
#define ENGRAM_E_ARG (-1)          /* malformed argument (null, negative size, bad enum)   */
#define ENGRAM_E_LAYOUT_ROWS (-2)  /* a table has fewer rows than its bucket prime sum      */
#define ENGRAM_E_VC_RANGE (-3)     /* compressed vocab^4 exceeds 2^64 (key not exact)      */
#define ENGRAM_E_NEED_STORE (-4)   /* a continuing sequence (seq_start 0) has no store slot */
#define ENGRAM_E_TOKEN_RANGE (-5)  /* device: a live token id outside [0, vocab_size)       */
#define ENGRAM_E_ROW_RANGE (-6)    /* device: a row id outside [0, rows of its table)        */
#define ENGRAM_E_SEQLENS (-7)      /* device: cu_seqlens not 0 = c0 <= c1 <= ... <= cS = T    */
#define ENGRAM_E_SLOT_RANGE (-8)   /* device: a slot outside [-1, num_slots)                 */
#define ENGRAM_E_MAP_RANGE (-9)    /* tid2eid has an id outside [0, V_c) or its size != V_c  */
#define ENGRAM_E_ALIGN (-10)       /* pointer / leading dimension / pitch misaligned        */
#define ENGRAM_E_HIP (-11)         /* a HIP runtime call failed                             */
#define ENGRAM_E_NOFIT (-12)       /* no bucket floor fits the requested table rows         */
#define ENGRAM_E_UNSUPPORTED (-13) /* a valid but unimplemented shape (e.g. hc_mult != 4)   */
#define ENGRAM_E_ID_RANGE (-14)    /* device: a compressed id written to the store is outside [0, V_c) */
#define ENGRAM_E_SCRATCH (-15)     /* the call needs more scratch than engram_gated_residual_noalloc holds */

/* ---- element types ------------------------------------------------------ */
typedef enum engram_dtype {
  ENGRAM_DTYPE_FP8_E4M3FN = 1, /* OCP e4m3fn: bias 7, max 448, 0x7F/0xFF NaN, no inf */
  ENGRAM_DTYPE_BF16 = 2,
  ENGRAM_DTYPE_F32 = 3
} engram_dtype;

#define ENGRAM_MAX_HEADS 8 /* hash heads per n-gram order */
#define ENGRAM_MAX_SITES 4 /* Engram sites sharing one hash pass */

/* How a site's buckets are laid out in memory. */
typedef enum engram_table_split {
  /* one table per n-gram order (PR summary: 3-table lookup over 2-/3-/4-gram
     tables); bucket offsets restart at 0 in each order's table */
  ENGRAM_TABLES_PER_ORDER = 0,
  /* one table per site holding all 3*H buckets back to back (order-major, then
     head), as the released checkpoint stores one embedding per Engram layer
     ([VeOmni#1370] n-gram memory lookup commit: 384,006,168 / 384,016,682 rows) */
  ENGRAM_TABLE_PER_SITE = 1
} engram_table_split;

/* Scales of e4m3fn tables. */
typedef enum engram_scale_layout {
  ENGRAM_SCALE_ROW_F32 = 0,      /* one fp32 scale per row                        */
  ENGRAM_SCALE_BLOCK32_E8M0 = 32 /* one e8m0 exponent byte per 32 elements of a row
                                    ([VeOmni#1370] per-row-scale commit: the tables
                                    are blocked (1, 32)); value 2^(b - 127), 0xFF NaN */
} engram_scale_layout;

/* ---- layout ------------------------------------------------------------- */
/* Description of the Engram sites that share one hash pass ([vLLM-V41]
 * DeepseekV4Model.forward: one gather of hashes feeds every layer, each taking
 * its columns through layer_hash_index).  Each site has 3 n-gram orders 2, 3, 4
 * with `heads_per_order` prime-sized hash buckets each. */
typedef struct engram_layout_desc {
  int64_t vocab_size;       /* tokenizer vocabulary = length of tid2eid ([VeOmni#1370]
                               vocab_size / engram_vocab_size commit: 129,280)        */
  int64_t compressed_vocab; /* V_c, size of the compressed id space (<= 65,536)       */
  int64_t pad_token_id;     /* its compressed id is the pad id of blocked lookbacks    */
  int32_t max_ngram;        /* must be 4 (orders 2, 3, 4)                              */
  int32_t heads_per_order;  /* H, 1..ENGRAM_MAX_HEADS                                  */
  int64_t rows[3];          /* TABLES_PER_ORDER: rows of each site's 2-, 3-, 4-gram
                               tables.  TABLE_PER_SITE: rows[0] = rows of each site's
                               table; rows[1], rows[2] ignored                         */
  int64_t hash_floor;       /* primes are drawn at and above this floor (the pages'
                               hash_vocab_size); 0 = fit the largest floor whose
                               primes fit every table                                  */
  int32_t row_dim;          /* D, elements per table row                                */
  int32_t table_dtype;      /* ENGRAM_DTYPE_FP8_E4M3FN (+ scales) or BF16               */
  int64_t row_pitch_bytes;  /* bytes between rows: multiple of 16 and at least
                               round_up(D, 16) * element size                           */
  int32_t num_sites;        /* sites sharing the hash pass, 1..ENGRAM_MAX_SITES (0 = 1);
                               site s draws its primes after sites 0..s-1            */
  int32_t table_split;      /* engram_table_split                                      */
  int32_t scale_layout;     /* engram_scale_layout (fp8 tables; BLOCK32 needs D % 32 == 0) */
  int32_t reserved;         /* 0 */
} engram_layout_desc;

typedef struct engram_layout engram_layout; /* opaque, immutable after creation */

#define ENGRAM_MAX_COLUMNS (ENGRAM_MAX_SITES * 3 * ENGRAM_MAX_HEADS)

/* Read-back of a created layout. */
typedef struct engram_layout_info {
  int64_t hash_floor;                       /* the floor used (given or fitted)          */
  int32_t heads_per_order;
  int32_t row_dim;
  int64_t rows[3];
  int64_t primes[ENGRAM_MAX_COLUMNS];       /* [site][order][head]; first num_sites*3*H
                                               entries used                             */
  int64_t offsets[ENGRAM_MAX_COLUMNS];      /* bucket start inside its table (the order's
                                               table, or the site's table)              */
  int64_t prime_sum[ENGRAM_MAX_SITES][3];   /* bucket rows per (site, order)            */
  int64_t seg_pitch;                        /* elements between the (order, head)
                                               segments of one gathered token row:
                                               round_up(D, 64); the tail is zero        */
  int64_t k_pad;                            /* 3 * H * seg_pitch: width of a gathered
                                               token row and of the projection's K      */
  int32_t num_sites;
  int32_t table_split;
  int32_t scale_layout;
  int32_t reserved;
} engram_layout_info;

/* Creates the layout: draws the bucket primes (site by site, for each order,
 * for each head, the smallest prime at or above the floor not yet drawn,
 * [VeOmni#1370] n-gram memory lookup commit and the validate_bucket_layout
 * review thread), fixes offsets as prefix sums inside each table, and checks
 * every table against its prime sum (fewer rows -> ENGRAM_E_LAYOUT_ROWS, more
 * rows allowed, as that review thread proposes).  Host only: no HIP call.
 * Errors: ENGRAM_E_ARG, ENGRAM_E_LAYOUT_ROWS, ENGRAM_E_VC_RANGE, ENGRAM_E_NOFIT,
 * ENGRAM_E_ALIGN (pitch; D not a multiple of 32 with block scales).  On success
 * *out owns host memory freed by destroy. */
int engram_layout_create(const engram_layout_desc* desc, engram_layout** out);
void engram_layout_destroy(engram_layout* layout);
int engram_layout_query(const engram_layout* layout, engram_layout_info* info);

/* Set-up check of the compression map (not a hot call; synchronises `stream`):
 * every entry of d_tid2eid[vocab_size] must lie in [0, V_c) and the largest
 * must be V_c - 1 ([VeOmni#1370] checkpoint-splitter commit: the compressed
 * vocabulary size the map produces is checked against the config, because a
 * different map silently rehashes the tables).  Writes the pad id
 * tid2eid[pad_token_id] to *pad_eid.  Errors: ENGRAM_E_MAP_RANGE, ENGRAM_E_HIP. */
int engram_tid2eid_check(const engram_layout* layout, const int32_t* d_tid2eid,
                         int32_t* pad_eid, hipStream_t stream);

/* ---- rolling store ------------------------------------------------------ */
/* The store keeps, per slot, the last three window ids of its sequence, oldest
 * first ([VeOmni#1370] n-gram incremental decode cache commit: the whole cache
 * is a fixed-width tail of max_ngram_size - 1 ids, which leaves no way to
 * express a history that is missing while the position is past the start;
 * [vLLM-V41] DeepseekV4Model.__init__: compressed ids are kept per KV-cache
 * slot so chunked prefill and decode can look back).  A slot holding pad ids
 * behaves exactly like a sequence start.
 *
 * The handle owns device memory int32 [num_slots][3] on the device that was
 * current at creation, bound to the layout it was made for (its compressed
 * vocabulary and pad id): every id it holds lies in [0, V_c).  Calls that use
 * it must run on that device. */
typedef struct engram_store engram_store; /* opaque */

/* Set-up call (allocates; not a hot call): a store of num_slots >= 1 slots, every
 * slot (pad_eid, pad_eid, pad_eid), the fill enqueued on `stream`.  pad_eid is
 * tid2eid[pad_token_id] as engram_tid2eid_check returns it, in [0, V_c).
 * Errors: ENGRAM_E_ARG, ENGRAM_E_HIP (allocation).  On success *out owns the
 * memory; engram_store_destroy frees it (the caller first makes sure no work
 * that uses the store is still pending). */
int engram_store_create(const engram_layout* layout, int32_t pad_eid, int32_t num_slots,
                        hipStream_t stream, engram_store** out);
void engram_store_destroy(engram_store* store);
/* Slot count and pad id of a store. */
int engram_store_query(const engram_store* store, int32_t* num_slots, int32_t* pad_eid);

/* Hot calls on the store (enqueue one kernel on `stream`, allocate nothing).
 * d_slots: int32 [n] slot indices, or NULL for every slot in order (n is then
 * ignored); d_ids: int32 [n][3] (or [num_slots][3]).
 *   reset: the slots <- (pad, pad, pad);
 *   write: store[d_slots[i]] <- d_ids[i][0..2]; a row holding an id outside
 *          [0, V_c) is not written and latches ENGRAM_E_ID_RANGE;
 *   read:  d_ids[i][0..2] <- store[d_slots[i]] (a snapshot before a
 *          speculative call, or a check).
 * Host errors: ENGRAM_E_ARG.  Device errors: ENGRAM_E_SLOT_RANGE (that slot is
 * skipped), ENGRAM_E_ID_RANGE. */
int engram_store_reset(engram_store* store, const int32_t* d_slots, int32_t n, hipStream_t stream);
int engram_store_write(engram_store* store, const int32_t* d_slots, int32_t n, const int32_t* d_ids,
                       hipStream_t stream);
int engram_store_read(const engram_store* store, const int32_t* d_slots, int32_t n, int32_t* d_ids,
                      hipStream_t stream);

/* Speculative rollback.  After an engram_compress_hash call that updated the
 * store for S sequences (a verify pass over draft tokens), sets each slot
 * d_slots[s] >= 0 to the tail it would hold had that call covered only the
 * first d_keep_len[s] tokens of sequence s (0 <= keep_len <= its length).
 * Snapshot = the slots' tails read with engram_store_read (same d_slots order)
 * before the call; only continuing sequences (d_seq_start[s] == 0) read it.
 * The other arguments are the call's own: d_cu_seqlens [S+1], T, d_eids [T]
 * (as the call wrote them), d_dead [T] or NULL, d_seq_start [S] or NULL (= all
 * started in the call; then d_snapshot may be NULL).
 * ([VeOmni#1370] n-gram incremental decode cache commit: the cache is a
 * fixed-width tail of the last three ids; review of the decode-cache
 * snapshot: state that only grows is rolled back by length, bounded state is
 * copied.  The tail is bounded, so its snapshot is the 3-id copy and rolling
 * back to a length replays at most the last three kept ids onto it.)
 * Host errors: ENGRAM_E_ARG (also a store made for another layout).  Device
 * errors: ENGRAM_E_SLOT_RANGE, ENGRAM_E_SEQLENS (keep_len outside [0, length]
 * or malformed cu_seqlens; that slot is left unchanged). */
int engram_store_rollback(const engram_layout* layout, const int32_t* d_tid2eid, engram_store* store,
                          const int32_t* d_slots, int32_t S, const int32_t* d_cu_seqlens, int32_t T,
                          const int32_t* d_eids, const uint8_t* d_dead, const uint8_t* d_seq_start,
                          const int32_t* d_snapshot, const int32_t* d_keep_len, hipStream_t stream);

/* ---- 1. compress + hash -------------------------------------------------- */
/* For each token t of each sequence s (tokens cu_seqlens[s] .. cu_seqlens[s+1]-1):
 *   e_t   = dead_t ? PAD : tid2eid[token_t],  PAD = tid2eid[pad_token_id]
 *           ([VeOmni#1370] pack_ngram_inputs commit: dead image-span positions
 *           compress to pad, the id a blocked lookback already reads);
 *   window (w0..w3) = (e_t, e_{t-1}, e_{t-2}, e_{t-3}) where a lookback stops
 *           (reads PAD from there on) at a dead position or before a sequence
 *           that starts here ([VeOmni#1370] n-gram memory lookup commit: no
 *           n-gram crosses an image span or reaches before the first
 *           position); a dead token's own window is all PAD; positions before
 *           a continuing sequence are read from its store slot;
 *   key_n = sum_{j<n} w_j * V_c^j (exact in 64 bits), n = 2, 3, 4;
 *   row_ids[t][site][n-2][h] = offsets[site][n][h] + key_n mod primes[site][n][h]
 *           for every site of the layout in the same pass ([NeMo-V41]
 *           DeepseekV41Block.forward: logical memory rows [batch, sequence,
 *           hash_heads]; [vLLM-V41] forward: one hash pass over the flattened
 *           batch, each layer reading its columns through layer_hash_index).
 * After the call, each sequence with a slot leaves its last three window ids
 * (oldest first) in the store; an empty sequence that starts here leaves PAD.
 * Arguments:
 *   d_tid2eid   int32 [vocab_size]
 *   d_tokens    int32 [T], T >= 0
 *   d_cu_seqlens int32 [S+1], S >= 1 if T > 0
 *   d_seq_start uint8 [S] or NULL (= every sequence starts here)
 *   d_slots     int32 [S] or NULL; -1 = no slot.  Slots of one call must be
 *               distinct (two sequences updating one slot race).
 *   store       a store made for this layout (engram_store_create), or NULL
 *   d_dead      uint8 [T] or NULL (= no dead position)
 *   d_eids      int32 [T] out: e_t
 *   d_row_ids   int32 [T][num_sites][3][H] out
 * Host errors: ENGRAM_E_ARG (also a store made for another layout).  Device
 * errors: ENGRAM_E_TOKEN_RANGE, ENGRAM_E_SEQLENS, ENGRAM_E_SLOT_RANGE,
 * ENGRAM_E_NEED_STORE. */
int engram_compress_hash(const engram_layout* layout, const int32_t* d_tid2eid,
                         const int32_t* d_tokens, int32_t T, const int32_t* d_cu_seqlens,
                         int32_t S, const uint8_t* d_seq_start, const int32_t* d_slots,
                         engram_store* store, const uint8_t* d_dead, int32_t* d_eids,
                         int32_t* d_row_ids, hipStream_t stream);

/* ---- 2. gather + dequant -------------------------------------------------- */
/* For each token t, order n, head h, element d < D of site `site`:
 *   out[t][(n*H + h)*seg_pitch + d] = fp32(q * scale) rounded to out_dtype,
 *   q = e4m3fn value of table[row][d], row = row_ids[t][site][n][h], scale =
 *   the row's fp32 scale or the e8m0 exponent of its block d / 32 ([VeOmni#1370]
 *   PR summary: FP8 rows are dequantised with their row scale at lookup time;
 *   per-row-scale
 *   commit: (1, 32) blocks).  BF16 tables carry no scale and are copied (or
 *   widened to fp32).  Elements d in [D, seg_pitch) of every segment are
 *   written as zero.
 * Arguments:
 *   d_tables   host array of 3 device pointers (TABLES_PER_ORDER: the site's
 *              order-n table uint8 [rows[n]][pitch]; TABLE_PER_SITE: entry 0 is
 *              the site's table [rows[0]][pitch], entries 1, 2 ignored), 16-byte
 *              aligned
 *   d_scales   host array of 3 device pointers, same tables: float [rows] for
 *              ROW_F32 scales, uint8 [rows][D/32] e8m0 bytes for BLOCK32 scales;
 *              NULL for bf16 tables
 *   d_row_ids  int32 [T][num_sites][3][H], as written by engram_compress_hash
 *   site       0 .. num_sites-1: whose columns (and tables) this call gathers
 *   out_dtype  ENGRAM_DTYPE_BF16 (hot path) or ENGRAM_DTYPE_F32 (exact check)
 *   d_out      [T][out_ld] of out_dtype, 16-byte aligned; out_ld >= k_pad and a
 *              multiple of 8
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN.  Device error: ENGRAM_E_ROW_RANGE
 * (that segment is written as zero). */
int engram_gather_dequant(const engram_layout* layout, const void* const* d_tables,
                          const void* const* d_scales, const int32_t* d_row_ids, int32_t site,
                          int32_t T, int32_t out_dtype, void* d_out, int64_t out_ld,
                          hipStream_t stream);

/* ---- 1 + 2 for a decode step ------------------------------------------------- */
/* A decode step's compress, hash and gather in one launch, for calls in which every
 * sequence is one token that continues from its store slot ([VeOmni#1370] n-gram
 * incremental decode cache commit: each step hashes the new token against the three
 * ids kept per sequence; PR summary: FP8 rows dequantised with their row scale on
 * lookup).  Token t is sequence t: with a slot (d_slots[t] >= 0) its window's three
 * earlier ids come from the store, and its new tail goes back into the slot; without
 * one (d_slots NULL, or d_slots[t] = -1) it starts its sequence (lookback PAD).
 * Writes exactly what engram_compress_hash (cu_seqlens = 0, 1, ..., T; seq_start 0
 * where the token has a slot, else 1) followed by engram_gather_dequant (site 0,
 * bf16 rows) write: d_eids [T], d_row_ids [T][3][H], the store, and d_rows bf16
 * [T][rows_ld] (rows_ld >= k_pad, a multiple of 8; 16-byte aligned).  Slots must
 * be distinct within a call.  d_tables / d_scales as for engram_gather_dequant.
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN, ENGRAM_E_NEED_STORE (slots without a
 * store), ENGRAM_E_UNSUPPORTED (several sites, bf16 tables, BLOCK32 scales).
 * Device errors: ENGRAM_E_TOKEN_RANGE, ENGRAM_E_SLOT_RANGE (that token starts its
 * sequence), ENGRAM_E_ROW_RANGE. */
int engram_lookup_decode(const engram_layout* layout, const int32_t* d_tid2eid,
                         const int32_t* d_tokens, int32_t T, const int32_t* d_slots,
                         engram_store* store, const uint8_t* d_dead, int32_t* d_eids,
                         int32_t* d_row_ids, const void* const* d_tables,
                         const void* const* d_scales, void* d_rows, int64_t rows_ld,
                         hipStream_t stream);

/* ---- 3. projection + gated residual ---------------------------------------- */
/* v[t][o] = sum_{k < k_pad} rows[t][k] * W[o][k], bf16 x bf16 accumulated in
 * fp32 on the matrix cores: the Engram connection's wkv projection
 * ([VeOmni#1370] config commit: the Engram connection is wkv plus a gate that
 * reads the mHC residual stream).
 *   d_rows bf16 [T][rows_ld], d_w bf16 [hidden][w_ld] (columns k_pad.. ignored;
 *   columns of W facing segment padding must be zero), d_v float [T][hidden].
 *   rows_ld, w_ld >= k_pad and multiples of 8; pointers 16-byte aligned;
 *   hidden a multiple of 8.
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN. */
int engram_project(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                   const void* d_w, int64_t w_ld, int32_t hidden, float* d_v, int32_t T,
                   hipStream_t stream);

/* The projection weight rearranged once into matrix-core fragment order, so that
 * engram_project_packed reads it with whole-line loads straight into registers
 * and keeps only the rows in on-chip memory (same wkv projection as
 * engram_project, [VeOmni#1370] config commit).
 * engram_packed_weight_bytes: size of the packed form of a [hidden][k_pad] weight,
 *   ceil(hidden / 32) * 32 * k_pad * 2 bytes.
 * engram_pack_weight: d_w bf16 [hidden][w_ld] as for engram_project (columns
 *   k_pad.. ignored) -> d_packed (caller-owned, that many bytes, 16-byte aligned):
 *   for column tile j = o / 16, k32 step s = k / 32 and lane l = o % 16 + 16 ((k % 32) / 8),
 *   element W[o][k] sits at bf16 index ((j (k_pad / 32) + s) 64 + l) 8 + k % 8 (the B
 *   operand of the 16 x 16 x 32 bf16 matrix-core instruction); rows past hidden up to
 *   the next multiple of 16 are zero, the rest of the buffer is not written.  Enqueued
 *   on `stream`; d_w may be freed once it ran.
 * engram_project_packed: v = rows W^T as engram_project, from the packed weight,
 *   bit-identical to engram_project (the same products summed in the same order).
 *   Meant for many tokens (tiles of 128 x 256 for k_pad up to 12,288, else 256 x 256);
 *   d_rows, rows_ld, d_v, T as for engram_project.
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN; ENGRAM_E_UNSUPPORTED when 256 rows of
 * rows_ld elements or k_pad * 64 bytes pass 2^31 - 1 (32-bit per-tile offsets). */
int engram_packed_weight_bytes(const engram_layout* layout, int32_t hidden, int64_t* bytes);
int engram_pack_weight(const engram_layout* layout, const void* d_w, int64_t w_ld, int32_t hidden,
                       void* d_packed, hipStream_t stream);
int engram_project_packed(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                          const void* d_packed, int32_t hidden, float* d_v, int32_t T,
                          hipStream_t stream);

/* Split-K form of engram_project for few tokens (decode): K is cut into `splits`
 * equal chunks (k_pad must be a multiple of 64 * splits) that run as separate
 * workgroups, so a small token count still fills the chip; chunk s writes
 *   d_partials[s][t][o] = sum over its k of rows[t][k] * W[o][k]
 * (float [splits][T][hidden], caller-owned workspace).  engram_gate_add_partials
 * sums the slices in slice order, so the result is deterministic.
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN. */
int engram_project_splitk(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                          const void* d_w, int64_t w_ld, int32_t hidden, float* d_partials,
                          int32_t splits, int32_t T, hipStream_t stream);

/* Steps 2 and the projection half of step 3 in one kernel, for e4m3fn tables:
 *   v[t][o] = sum_{k < k_pad} rows[t][k] * W[o][k]
 * with rows[t] exactly the bf16 rows engram_gather_dequant would write (row-wise
 * dequant on lookup, [VeOmni#1370] PR summary; wkv projection, [VeOmni#1370]
 * config commit), built tile by tile in on-chip memory and never stored.
 * Same accumulation order as engram_project, so v matches the two-call path bit
 * for bit.
 *   d_tables, d_scales, d_row_ids, site as for engram_gather_dequant; the
 *   layout's row_pitch_bytes must be >= seg_pitch and a multiple of 16 (a row is
 *   read in 64-byte pieces up to seg_pitch; bytes past D are ignored).
 *   d_w, w_ld, hidden, d_v as for engram_project.
 *   Scales: one fp32 per row, or BLOCK32 e8m0 bytes for rows of at most 256
 *   elements (the released layout's width); with 256-element rows each scale
 *   array must be 8-byte aligned.
 * Host errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN, ENGRAM_E_UNSUPPORTED (bf16 tables,
 * BLOCK32 scales on rows wider than 256, tables in host memory).  Device error:
 * ENGRAM_E_ROW_RANGE (that segment contributes zero). */
int engram_gather_project(const engram_layout* layout, const void* const* d_tables,
                          const void* const* d_scales, const int32_t* d_row_ids, int32_t site,
                          int32_t T, const void* d_w, int64_t w_ld, int32_t hidden, float* d_v,
                          hipStream_t stream);

/* For each token t and stream s < hc_mult:
 *   z = <x[t][s][:], v[t][:]> / sqrt(hidden),  g = keep_t * sigmoid(z),
 *   x[t][s][:] <- bf16(x[t][s][:] + g * v[t][:])   (in place; keep_t = 0 leaves
 *   the stream bit for bit)
 * ([NeMo-V41] forward contract: Engram writes into the hc residual streams
 * before its layer; [vLLM-V41] forward: image-span tokens have their gate
 * zeroed).  d_v float [T][hidden]; d_keep uint8 [T] or NULL (= all kept);
 * d_streams bf16 [T][hc_mult][hidden], 16-byte aligned; hidden a multiple of 8,
 * at most 8192.  hc_mult must be 4 (ENGRAM_E_UNSUPPORTED otherwise). */
int engram_gate_add(const engram_layout* layout, const float* d_v, int32_t hidden,
                    int32_t hc_mult, const uint8_t* d_keep, void* d_streams, int32_t T,
                    hipStream_t stream);

/* engram_gate_add with v given as the split-K slices of engram_project_splitk:
 * v[t][o] = sum_{s < splits} d_partials[s][t][o], summed in slice order; d_v
 * (float [T][hidden], 16-byte aligned) receives that v when not NULL.  Otherwise
 * as engram_gate_add. */
int engram_gate_add_partials(const engram_layout* layout, const float* d_partials, int32_t splits,
                             int32_t hidden, int32_t hc_mult, const uint8_t* d_keep,
                             void* d_streams, float* d_v, int32_t T, hipStream_t stream);

/* ---- 3'. the projection weight of a site, and the gated residual ------------ */
/* A site's wkv weight bound once, at set-up, to the layout and to the largest call
 * it will serve ([VeOmni#1370] config commit: the Engram connection is wkv plus a
 * gate reading the mHC residual stream).  The handle decides, per call, which
 * projection kernel runs (engram_projection_plan), and owns what that needs:
 *   - the weight packed in fragment order (engram_pack_weight), when some call of
 *     up to max_tokens tokens reaches the packed kernel;
 *   - the split-K workspace float [splits][T][hidden], when some call takes the
 *     split-K form.
 * d_w (bf16 [hidden][w_ld], as for engram_project) stays caller-owned and must
 * outlive the handle: calls that take the plain or split-K kernel read it. */
typedef struct engram_wkv engram_wkv; /* opaque */

/* Projection kernels a call can run. */
typedef enum engram_proj_kernel {
  ENGRAM_PROJ_PLAIN = 0,  /* engram_project: 256 x 256 or 128 x 128 tiles, both operands via LDS */
  ENGRAM_PROJ_PACKED = 1, /* engram_project_packed: many tokens, weight in fragment order */
  ENGRAM_PROJ_SPLITK = 2  /* engram_project_splitk + the slice sum in the gate: few tokens */
} engram_proj_kernel;

typedef struct engram_proj_plan {
  int32_t kernel; /* engram_proj_kernel */
  int32_t splits; /* split-K factor (1 unless kernel == ENGRAM_PROJ_SPLITK) */
} engram_proj_plan;

/* The kernel a T-token projection of a [hidden][k_pad] weight runs (host only,
 * no HIP call):
 *   PACKED when `packed` (a packed weight exists) and T * hidden >= 64 * 256 * 256
 *     (enough 256 x 256 tiles to fill the chip);
 *   else SPLITK with s splits when s > 1, where s = `splits` if given (> 0),
 *     otherwise the largest of 2, 4, 8 such that the call's 128 x 128 tiles times s
 *     stay within one workgroup per CU (256), each split keeps at least 4 k-steps
 *     of 64, and k_pad is a multiple of 64 s (none: s = 1);
 *   else PLAIN.
 * Errors: ENGRAM_E_ARG. */
int engram_projection_plan(const engram_layout* layout, int32_t hidden, int32_t T, int32_t packed,
                           int32_t splits, engram_proj_plan* plan);

/* Set-up call (allocates; packs on `stream`): the handle for calls of up to
 * max_tokens tokens.  splits: 0 = chosen per call as engram_projection_plan says,
 * s >= 1 = every call below the packed size takes s splits (1: never split).
 * Errors: ENGRAM_E_ARG, ENGRAM_E_ALIGN (as engram_project; k_pad not a multiple
 * of 64 s for a forced s), ENGRAM_E_HIP (allocation). */
int engram_wkv_create(const engram_layout* layout, const void* d_w, int64_t w_ld, int32_t hidden,
                      int32_t max_tokens, int32_t splits, hipStream_t stream, engram_wkv** out);
void engram_wkv_destroy(engram_wkv* wkv);
/* The plan a T-token call of this handle follows (T <= max_tokens). */
int engram_wkv_plan(const engram_wkv* wkv, int32_t T, engram_proj_plan* plan);

/* Step 3 of the path: v = W rows^T by the planned kernel, then for each token and
 * stream the gated add of engram_gate_add, in place, on one stream:
 *   z = <x[t][s][:], v[t][:]> / sqrt(hidden),  g = keep_t * sigmoid(z),
 *   x[t][s][:] <- bf16(x[t][s][:] + g * v[t][:]).
 * d_rows bf16 [T][rows_ld] (rows_ld >= k_pad, multiple of 8, 16-byte aligned),
 * d_keep uint8 [T] or NULL, d_streams bf16 [T][hc_mult][hidden] in/out, d_v
 * float [T][hidden] (caller-owned workspace; receives v), T <= max_tokens.
 * Every planned kernel sums the same products of each k-step of 16 in the same
 * order within its slice, so v is the fp32 accumulation the plain kernel makes,
 * except that split-K sums s slices (each in that order), deterministically.
 * Calls sharing one handle must not overlap (the split-K workspace is the
 * handle's).  There is no variant without rows: a site that has Engram and no
 * looked-up rows is a caller error, never a skip ([VeOmni#1370] decode-stack
 * commit: a missing n-gram embedding raises).
 * Host errors: ENGRAM_E_ARG (also T > max_tokens, or a handle made for another
 * layout), ENGRAM_E_ALIGN, ENGRAM_E_UNSUPPORTED (hc_mult != 4, hidden > 8192). */
int engram_gated_residual(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                          const engram_wkv* wkv, int32_t hc_mult, const uint8_t* d_keep,
                          void* d_streams, float* d_v, int32_t T, hipStream_t stream);

/* The two halves of engram_gated_residual, for callers that put other work
 * between them (the next call's gather, for example): engram_wkv_project runs
 * the planned projection (for split-K it leaves the slices in the handle's
 * workspace and d_v is written by the second half); engram_wkv_gate_add runs the
 * gated add (summing the slices into d_v first for split-K).  Same T, d_v and
 * handle in both; nothing else may use the handle in between. */
int engram_wkv_project(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                       const engram_wkv* wkv, float* d_v, int32_t T, hipStream_t stream);
int engram_wkv_gate_add(const engram_layout* layout, const engram_wkv* wkv, float* d_v,
                        int32_t hc_mult, const uint8_t* d_keep, void* d_streams, int32_t T,
                        hipStream_t stream);

/* ---- the gated residual without allocation --------------------------------- */
/* For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same result as
 * engram_gated_residual (the same planned kernels in the same order, so the
 * streams are bit for bit the same), with its scratch -- v float [T][hidden],
 * and for the split-K plan the slices float [splits][T][hidden] -- in a
 * library-owned device array of ENGRAM_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the first call on that GPU until the process ends.  v is not returned.
 * The call allocates nothing and never synchronises.  Calls on one GPU share its
 * array: calls that overlap on one GPU (two streams, two threads) race, and must
 * be ordered by the caller.  Nothing in the array needs clearing between calls.
 * Errors: as engram_gated_residual, and ENGRAM_E_SCRATCH when
 * round_up(T * hidden, 64) (+ splits * T * hidden for split-K) floats exceed the
 * array (at hidden 4,096: up to 2,048 tokens, or 409 with 4 splits). */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (32u << 20)
int engram_gated_residual_noalloc(const engram_layout* layout, const void* d_rows, int64_t rows_ld,
                                  const engram_wkv* wkv, int32_t hc_mult, const uint8_t* d_keep,
                                  void* d_streams, int32_t T, hipStream_t stream);

/* ---- errors ------------------------------------------------------------- */
const char* engram_strerror(int status);
/* Synchronises `stream`, returns the first device-detected status latched on
 * the current device since the last call (ENGRAM_OK if none) and clears it.
 * Returns ENGRAM_E_HIP if the synchronisation itself fails. */
int engram_get_error(hipStream_t stream);
/* Name of the last HIP runtime error behind an ENGRAM_E_HIP status returned on
 * this thread ("hipSuccess" if none); a static string. */
const char* engram_last_hip_error(void);

/* Identity of the build: "engram-src-sha256:" followed by 16 hex digits of a
 * SHA-256 over the library's sources and compiler flags; a static string. */
const char* engram_build_id(void);

/* ---- host-resident tables -------------------------------------------------- */
/* Tables too large for HBM may live in pinned host memory (hipHostMalloc); the
 * gather kernels then read their rows over the host link ([vLLM-V41]
 * DeepseekV4Model.__init__: Engram tables offloaded to the CPU get a prefetch
 * stream of their own).  Writes to *dev the device-side address of pinned host
 * memory `host`, to be passed as a table or scale pointer.  Not a hot call.
 * Errors: ENGRAM_E_ARG, ENGRAM_E_HIP (memory that is not pinned). */
int engram_host_device_pointer(const void* host, void** dev);

#ifdef __cplusplus
}
#endif
#endif /* ENGRAM_H */
