/*
 * engram_oracle.h -- the oracle: a plain, slow, single-threaded CPU statement of
 * what the Engram n-gram memory computes.  TEST INFRASTRUCTURE ONLY: only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * Pages followed (titles; sections named, no line numbers):
 *  [VeOmni#1370]  GitHub PR "feat: support DeepSeek-V4.1-Flash in SeedOmni"
 *                 (ByteDance-Seed/VeOmni #1370): PR summary (deepseek_v41_ngram
 *                 entry), the "n-gram memory lookup" commit note, the
 *                 pack_ngram_inputs commit note, the "n-gram incremental decode
 *                 cache" commit note, the vocab_size / engram_vocab_size commit
 *                 note, the per-row (1,32) scale commit note, and the review
 *                 thread proposing a row-count guard for validate_bucket_layout.
 *  [NeMo-V41]     NeMo AutoModel API page
 *                 "nemo_automodel.components.models.deepseek_v41.model":
 *                 forward contract; DeepseekV41Block.forward parameters.
 *  [vLLM-V41]     vLLM docs page "vllm/models/deepseek_v41/nvidia/model":
 *                 DeepseekV4Model.__init__ (NgramHashState) and
 *                 DeepseekV4Model.forward (Engram hash block).
 *
 * Where the pages leave a step open the reading taken is stated at the function.
 * Every function returns 0 on success or a negative ORC_E* code.
 */
#ifndef ENGRAM_ORACLE_H
#define ENGRAM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORC_OK = 0,
  ORC_E_ARG = -1,          /* malformed argument                                */
  ORC_E_ROWS = -2,         /* a table has fewer rows than its prime sum        */
  ORC_E_VC = -3,           /* compressed vocab too large for an exact 64-bit key */
  ORC_E_NEED_STORE = -4,   /* continuation sequence without a rolling store     */
  ORC_E_TOKEN = -5,        /* token id outside [0, vocab)                       */
  ORC_E_NAN = -6,          /* an e4m3fn NaN byte in a table row                 */
  ORC_E_NOFIT = -7         /* no bucket floor fits the requested rows           */
};

/* Prime draw of the bucket layout ([VeOmni#1370] n-gram lookup commit: trial
 * division reproduces the released draw; review thread on validate_bucket_layout
 * shows the draw).  For each layer, for each order 2..max_ngram, for each head:
 * the smallest prime >= floor not already drawn (search restarts at the floor
 * for every order).  Output order: [layer][order][head]. */
int oracle_draw_primes(int n_layers, int max_ngram, int n_heads, uint64_t floor_,
                       uint64_t *primes_out);

/* Floor fit for three per-order tables of rows[0..2] rows (one Engram site,
 * orders 2,3,4, H heads each): the largest floor F <= min(rows)/H whose draw
 * gives every order a prime sum <= that order's rows.  Writes F, the primes
 * [3][H] and the per-table offsets [3][H] (prefix sums within each table). */
int oracle_fit_layout(const uint64_t rows[3], int n_heads, uint64_t *floor_out,
                      uint64_t *primes_out, uint64_t *offsets_out);

/* Layout for a given floor (the pages' hash_vocab_size): draws the primes and
 * rejects any table whose rows are below its prime sum (review thread's guard:
 * fewer rows is an error, more rows is allowed). */
int oracle_layout_at_floor(const uint64_t rows[3], int n_heads, uint64_t floor_,
                           uint64_t *primes_out, uint64_t *offsets_out);

/* Compress + rolling n-gram hash, token by token.
 *   tid2eid [vocab]          compressed id of every token id
 *   tokens  [T]              token ids
 *   cu_seqlens [S+1]         sequence boundaries, cu[0]=0, cu[S]=T
 *   seq_start [S] or NULL    1 = the sequence starts here (history is PAD);
 *                            0 = it continues the slot's stored history.  NULL = all 1.
 *   slots [S] or NULL        rolling-store slot of each sequence, -1 = none
 *   store [num_slots][3] or NULL   last three window ids, oldest first; updated
 *   dead [T] or NULL         1 = dead position (image span)
 *   primes/offsets [3][H]    layout
 * Outputs eids[T] and row_ids[T][3][H] (order-major, then head). */
int oracle_compress_hash(int64_t vocab, int64_t vc, int64_t pad_token_id, int n_heads,
                         const uint64_t *primes, const uint64_t *offsets,
                         const int32_t *tid2eid, const int32_t *tokens, int64_t T,
                         const int32_t *cu_seqlens, int64_t S, const uint8_t *seq_start,
                         const int32_t *slots, int32_t *store, int64_t num_slots,
                         const uint8_t *dead, int32_t *eids, int32_t *row_ids);

/* Primes [site][order][head] and bucket offsets of n_sites sites sharing one hash
 * pass (site s draws after sites 0..s-1); per_site_table selects one table per
 * site (offsets run across its orders) or one table per order (offsets restart). */
int oracle_site_layout(int n_sites, int n_heads, uint64_t floor_, int per_site_table,
                       uint64_t *primes_out, uint64_t *offsets_out);

/* Decode one OCP e4m3fn byte to its exact value (NaN for 0x7F / 0xFF). */
float oracle_e4m3fn_decode(uint8_t b);

/* Round a double to the nearest bfloat16 (ties to even); returns the bf16 bits. */
uint16_t oracle_bf16_rne(double x);

/* Dequantize n rows of D e4m3fn bytes, each with its fp32 scale:
 *   out_f32 = fp32(q * scale) (one IEEE multiply), out_bf16 = RNE_bf16(out_f32).
 * Either output may be NULL.  If scales is NULL the rows are bf16 bit patterns
 * (2 bytes each, little endian) and are widened exactly. */
int oracle_dequant_rows(const uint8_t *rows, const float *scales, int64_t n, int64_t D,
                        int is_bf16_table, float *out_f32, uint16_t *out_bf16);

/* Value of an OCP MX e8m0 scale byte: 2^(b - 127), NaN for 0xFF. */
double oracle_e8m0_decode(uint8_t b);

/* Dequantize n rows of D e4m3fn bytes with (1, 32) e8m0 block scales
 * (scales [n][D/32]): out_f32 = fp32(q * 2^(b-127)), out_bf16 = RNE_bf16(out_f32). */
int oracle_dequant_rows_block32(const uint8_t *rows, const uint8_t *scales, int64_t n, int64_t D,
                                float *out_f32, uint16_t *out_bf16);

/* Down-projection v[t][o] = sum_k E[t][k] * W[o][k] in fp64 (E, W given as bf16). */
int oracle_project(const uint16_t *E, const uint16_t *W, int64_t T, int64_t K,
                   int64_t hidden, double *v);

/* Gated residual add into hc streams of one token set:
 *   z_s = <x_s, v> / sqrt(hidden)   (fp64),
 *   g_s = keep ? 1/(1+exp(-z_s)) : 0,
 *   y_s = keep ? RNE_bf16(x_s + g_s v) : x_s  (bit for bit).
 * x, y: bf16 [T][hc][hidden]; v: fp64 [T][hidden]; keep: [T] or NULL (= all 1). */
int oracle_gate_add(const uint16_t *x, const double *v, const uint8_t *keep, int64_t T,
                    int64_t hc, int64_t hidden, uint16_t *y, double *gates_out);

#ifdef __cplusplus
}
#endif
#endif
