/*
 * engram_oracle.c -- the oracle for the Engram n-gram memory hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  A plain, slow, single-threaded statement of what
 * the path computes, written from the pages (see engram_oracle.h for the page
 * list).  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it; the HIP library never does, and the two share no code.
 *
 * Floating point: IEEE fp32 where the method fixes it (the dequant multiply),
 * fp64 everywhere else.  Built with -ffp-contract=off so that no multiply-add is
 * fused behind the source's back.
 */
#include "engram_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Layout: prime draw, floor fit, row-count guard                           */
/* ------------------------------------------------------------------------ */

/* Primality of every integer in [lo, lo + len), by a segmented sieve of
 * Eratosthenes: the base primes up to sqrt(lo + len - 1) come from a plain sieve,
 * and each strikes out its multiples inside the window.  out[i] = 1 iff lo + i
 * is prime.  Returns ORC_E_ARG if a buffer cannot be allocated. */
static int sieve_window(uint64_t lo, uint64_t len, uint8_t *out) {
  const uint64_t hi = lo + len - 1;
  uint64_t r = 1;
  while ((r + 1) * (r + 1) <= hi) ++r;
  uint8_t *base = (uint8_t *)malloc((size_t)r + 1);
  if (!base) return ORC_E_ARG;
  memset(base, 1, (size_t)r + 1);
  base[0] = 0;
  if (r >= 1) base[1] = 0;
  for (uint64_t p = 2; p * p <= r; ++p)
    if (base[p])
      for (uint64_t m = p * p; m <= r; m += p) base[m] = 0;
  memset(out, 1, (size_t)len);
  for (uint64_t i = 0; i < len && lo + i < 2; ++i) out[i] = 0; /* 0 and 1 are not prime */
  for (uint64_t p = 2; p <= r; ++p) {
    if (!base[p]) continue;
    uint64_t m = (lo + p - 1) / p * p; /* first multiple of p at or above lo */
    if (m < p * p) m = p * p;          /* p itself stays prime */
    for (; m <= hi; m += p) out[m - lo] = 0;
  }
  free(base);
  return ORC_OK;
}

/* [VeOmni#1370] n-gram memory lookup commit and the validate_bucket_layout
 * review thread: layer after layer, order after order (2 .. max_ngram), head
 * after head, each bucket takes the smallest prime at or above the floor that
 * no earlier bucket took.  So the buckets receive the consecutive primes from
 * the floor upward, in (layer, order, head) order; they are read off a sieved
 * window above the floor, widened until it holds enough primes. */
int oracle_draw_primes(int n_layers, int max_ngram, int n_heads, uint64_t floor_,
                       uint64_t *primes_out) {
  if (n_layers < 1 || max_ngram < 2 || n_heads < 1 || floor_ < 1 || !primes_out)
    return ORC_E_ARG;
  const int need = n_layers * (max_ngram - 1) * n_heads;
  uint64_t len = 4096;
  for (;;) {
    uint8_t *flag = (uint8_t *)malloc((size_t)len);
    if (!flag) return ORC_E_ARG;
    if (sieve_window(floor_, len, flag) != ORC_OK) {
      free(flag);
      return ORC_E_ARG;
    }
    int count = 0;
    for (uint64_t i = 0; i < len && count < need; ++i)
      if (flag[i]) primes_out[count++] = floor_ + i;
    free(flag);
    if (count == need) return ORC_OK;
    len *= 2;
  }
}

static void offsets_from_primes(const uint64_t *primes, int n_heads, uint64_t *offsets) {
  for (int t = 0; t < 3; ++t) {
    uint64_t acc = 0;
    for (int h = 0; h < n_heads; ++h) {
      offsets[t * n_heads + h] = acc;
      acc += primes[t * n_heads + h];
    }
  }
}

static int sums_fit(const uint64_t *primes, int n_heads, const uint64_t rows[3]) {
  for (int t = 0; t < 3; ++t) {
    uint64_t s = 0;
    for (int h = 0; h < n_heads; ++h) s += primes[t * n_heads + h];
    if (s > rows[t]) return 0;
  }
  return 1;
}

/* Row-count guard from the validate_bucket_layout review thread: a table
 * smaller than its prime sum is rejected, a larger one is allowed.  Here each
 * order has its own table, so the guard applies per order. */
int oracle_layout_at_floor(const uint64_t rows[3], int n_heads, uint64_t floor_,
                           uint64_t *primes_out, uint64_t *offsets_out) {
  if (!rows || n_heads < 1 || !primes_out || !offsets_out) return ORC_E_ARG;
  int rc = oracle_draw_primes(1, 4, n_heads, floor_, primes_out);
  if (rc) return rc;
  offsets_from_primes(primes_out, n_heads, offsets_out);
  return sums_fit(primes_out, n_heads, rows) ? ORC_OK : ORC_E_ROWS;
}

/* Layout of the Engram sites that share one hash pass: site s takes the 3H
 * primes drawn after sites 0..s-1 ([vLLM-V41] DeepseekV4Model.forward: one
 * gather of hashes feeds every layer, each reading its columns through
 * layer_hash_index; [VeOmni#1370] n-gram memory lookup commit: the two
 * layers' tables hold 384,006,168 and 384,016,682 rows).  per_site_table = 1:
 * one table per site, each bucket starting where the previous (order, head)
 * bucket of the site ended; 0: one table per order, offsets restarting at 0. */
int oracle_site_layout(int n_sites, int n_heads, uint64_t floor_, int per_site_table,
                       uint64_t *primes_out, uint64_t *offsets_out) {
  if (n_sites < 1 || n_heads < 1 || !primes_out || !offsets_out) return ORC_E_ARG;
  int rc = oracle_draw_primes(n_sites, 4, n_heads, floor_, primes_out);
  if (rc) return rc;
  for (int s = 0; s < n_sites; ++s) {
    uint64_t acc = 0;
    for (int t = 0; t < 3; ++t) {
      if (!per_site_table) acc = 0;
      for (int h = 0; h < n_heads; ++h) {
        const int c = (s * 3 + t) * n_heads + h;
        offsets_out[c] = acc;
        acc += primes_out[c];
      }
    }
  }
  return ORC_OK;
}

/* Three per-order tables of given row counts: the largest floor whose draw fits
 * every table (reading of the pages' one-table-per-layer layout split at the
 * order boundaries). */
int oracle_fit_layout(const uint64_t rows[3], int n_heads, uint64_t *floor_out,
                      uint64_t *primes_out, uint64_t *offsets_out) {
  if (!rows || n_heads < 1 || !floor_out || !primes_out || !offsets_out) return ORC_E_ARG;
  uint64_t rmin = rows[0];
  if (rows[1] < rmin) rmin = rows[1];
  if (rows[2] < rmin) rmin = rows[2];
  for (uint64_t f = rmin / (uint64_t)n_heads; f >= 2; --f) {
    if (oracle_draw_primes(1, 4, n_heads, f, primes_out) != ORC_OK) return ORC_E_ARG;
    if (sums_fit(primes_out, n_heads, rows)) {
      offsets_from_primes(primes_out, n_heads, offsets_out);
      *floor_out = f;
      return ORC_OK;
    }
  }
  return ORC_E_NOFIT;
}

/* ------------------------------------------------------------------------ */
/* Compress + rolling n-gram hash                                           */
/* ------------------------------------------------------------------------ */

/* Token by token, in sequence order, carrying a three-id tail as the n-gram
 * incremental decode cache commit describes: the longest n-gram (order 4) at a
 * position looks back over at most the 3 ids before it, so those 3 ids are all
 * the state a sequence needs.
 *
 *  - compress: e = tid2eid[token]; a dead position (image span) compresses to
 *    the pad id ([VeOmni#1370] pack_ngram_inputs commit: a dead position takes
 *    the same pad id that a cut-off lookback reads).  PAD = tid2eid[pad_token_id].
 *  - a sequence that starts here has an all-PAD history (lookback never reaches
 *    past position 0; packed samples restart); a continuing sequence reads the
 *    slot's stored tail ([vLLM-V41] NgramHashState, a slot-keyed rolling store).
 *  - the window of position t is (w0,w1,w2,w3) = (e_t, tail[2], tail[1],
 *    tail[0]); a dead position's own window is all PAD (no n-gram crosses an
 *    image span).
 *  - after t: tail = dead ? (PAD,PAD,PAD) : (tail[1], tail[2], e_t), so nothing
 *    before a dead position is ever read again.
 *  - hash (reading of the pages' statement that the hash multipliers are
 *    functions of the compressed vocabulary size): key_n = sum_{j<n} w_j * vc^j as an exact integer; the row of head h
 *    is offsets[n][h] + key_n mod primes[n][h].
 */
int oracle_compress_hash(int64_t vocab, int64_t vc, int64_t pad_token_id, int n_heads,
                         const uint64_t *primes, const uint64_t *offsets,
                         const int32_t *tid2eid, const int32_t *tokens, int64_t T,
                         const int32_t *cu_seqlens, int64_t S, const uint8_t *seq_start,
                         const int32_t *slots, int32_t *store, int64_t num_slots,
                         const uint8_t *dead, int32_t *eids, int32_t *row_ids) {
  if (vocab < 1 || n_heads < 1 || !primes || !offsets || !tid2eid || !cu_seqlens ||
      S < 0 || T < 0 || (T > 0 && (!tokens || !eids || !row_ids)))
    return ORC_E_ARG;
  if (vc < 1 || vc > 65536) return ORC_E_VC; /* vc^4 must not exceed 2^64 */
  if (pad_token_id < 0 || pad_token_id >= vocab) return ORC_E_ARG;
  const int32_t pad = tid2eid[pad_token_id];
  if (pad < 0 || pad >= vc) return ORC_E_ARG;
  if (cu_seqlens[0] != 0 || cu_seqlens[S] != T) return ORC_E_ARG;
  for (int64_t s = 0; s < S; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return ORC_E_ARG;

  uint64_t vpow[4];
  vpow[0] = 1;
  for (int j = 1; j < 4; ++j) vpow[j] = vpow[j - 1] * (uint64_t)vc;

  for (int64_t s = 0; s < S; ++s) {
    const int starts = seq_start ? (seq_start[s] != 0) : 1;
    const int32_t slot = slots ? slots[s] : -1;
    if (slot >= 0 && (!store || slot >= num_slots)) return ORC_E_ARG;
    if (slot < -1) return ORC_E_ARG;

    int32_t tail[3];
    if (starts) {
      tail[0] = tail[1] = tail[2] = pad;
    } else {
      if (slot < 0) return ORC_E_NEED_STORE;
      memcpy(tail, store + 3 * (int64_t)slot, sizeof tail);
    }

    for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
      const int is_dead = dead ? (dead[t] != 0) : 0;
      int32_t e;
      if (is_dead) {
        e = pad;
      } else {
        if (tokens[t] < 0 || tokens[t] >= vocab) return ORC_E_TOKEN;
        e = tid2eid[tokens[t]];
        if (e < 0 || e >= vc) return ORC_E_ARG;
      }
      eids[t] = e;

      int64_t w[4];
      if (is_dead) {
        w[0] = w[1] = w[2] = w[3] = pad;
      } else {
        w[0] = e;
        w[1] = tail[2];
        w[2] = tail[1];
        w[3] = tail[0];
      }

      for (int order = 2; order <= 4; ++order) {
        unsigned __int128 key = 0;
        for (int j = 0; j < order; ++j)
          key += (unsigned __int128)(uint64_t)w[j] * (unsigned __int128)vpow[j];
        for (int h = 0; h < n_heads; ++h) {
          const int col = (order - 2) * n_heads + h;
          const uint64_t p = primes[col];
          const uint64_t row = offsets[col] + (uint64_t)(key % p);
          if (row > 0x7FFFFFFFull) return ORC_E_ARG;
          row_ids[t * 3 * n_heads + col] = (int32_t)row;
        }
      }

      if (is_dead) {
        tail[0] = tail[1] = tail[2] = pad;
      } else {
        tail[0] = tail[1];
        tail[1] = tail[2];
        tail[2] = e;
      }
    }
    if (slot >= 0) memcpy(store + 3 * (int64_t)slot, tail, sizeof tail);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequant                                                                  */
/* ------------------------------------------------------------------------ */

/* OCP e4m3fn ("fn": finite, no infinities): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is
 * NaN.  [VeOmni#1370] PR summary: the tables are e4m3fn with a row-wise scale. */
float oracle_e4m3fn_decode(uint8_t b) {
  const int sign = (b >> 7) & 1;
  const int ex = (b >> 3) & 0xF;
  const int man = b & 0x7;
  if (ex == 0xF && man == 0x7) return NAN;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -9);
  else
    v = ldexp(1.0 + (double)man / 8.0, ex - 7);
  return (float)(sign ? -v : v); /* exact: at most 4 significant bits */
}

static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Nearest bfloat16 to x, ties to even, computed from the value (not from a
 * float's bit pattern): scale x so its last kept bit is the units digit, round
 * to an integer with nearbyint (ties-to-even in the default rounding mode),
 * scale back.  bf16 keeps 8 significant bits; its quantum never drops below
 * 2^-133 (the smallest subnormal). */
uint16_t oracle_bf16_rne(double x) {
  if (isnan(x)) return 0x7FC0;
  const int neg = signbit(x) ? 1 : 0;
  const double ax = fabs(x);
  uint16_t mag;
  if (ax == 0.0) {
    mag = 0;
  } else if (isinf(ax)) {
    mag = 0x7F80;
  } else {
    int e;
    (void)frexp(ax, &e); /* ax = m * 2^e with m in [0.5, 1) */
    int q = (e - 1) - 7;
    if (q < -133) q = -133;
    const double r = nearbyint(ldexp(ax, -q));
    const float f = (float)ldexp(r, q); /* exact, or +inf past the bf16 range */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    mag = (uint16_t)(u >> 16);
  }
  return (uint16_t)(mag | (neg ? 0x8000 : 0));
}

/* Dequant of one gathered row: fp32(q * scale) with a single IEEE multiply, then
 * one round to bf16.  BF16 tables carry no scale and widen exactly. */
int oracle_dequant_rows(const uint8_t *rows, const float *scales, int64_t n, int64_t D,
                        int is_bf16_table, float *out_f32, uint16_t *out_bf16) {
  if (n < 0 || D < 0 || (n > 0 && D > 0 && !rows)) return ORC_E_ARG;
  if (!is_bf16_table && n > 0 && !scales) return ORC_E_ARG;
  int rc = ORC_OK;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t d = 0; d < D; ++d) {
      float e;
      if (is_bf16_table) {
        const uint8_t *p = rows + 2 * (r * D + d);
        e = bf16_bits_to_float((uint16_t)(p[0] | (p[1] << 8)));
      } else {
        const float q = oracle_e4m3fn_decode(rows[r * D + d]);
        if (isnan(q)) rc = ORC_E_NAN;
        const float s = scales[r];
        e = q * s;
      }
      if (out_f32) out_f32[r * D + d] = e;
      if (out_bf16) out_bf16[r * D + d] = oracle_bf16_rne((double)e);
    }
  }
  return rc;
}

/* OCP MX E8M0 scale byte: an unsigned exponent with bias 127, value
 * 2^(b - 127); 0xFF is NaN; there is no zero and no sign.  [VeOmni#1370]
 * per-row-scale commit: in the released tables every row has such an exponent
 * for each block of 32 columns. */
double oracle_e8m0_decode(uint8_t b) {
  if (b == 0xFF) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* Dequant with (1, 32) blocks: element d of row r is fp32(q * s) with s the
 * fp32 value of the e8m0 byte scales[r][d / 32] (2^-127 is an fp32 subnormal,
 * so every byte but 0xFF is exact) and one IEEE multiply, then one round to
 * bf16. */
int oracle_dequant_rows_block32(const uint8_t *rows, const uint8_t *scales, int64_t n, int64_t D,
                                float *out_f32, uint16_t *out_bf16) {
  if (n < 0 || D < 0 || D % 32 != 0 || (n > 0 && D > 0 && (!rows || !scales))) return ORC_E_ARG;
  const int64_t nblk = D / 32;
  int rc = ORC_OK;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t d = 0; d < D; ++d) {
      const float q = oracle_e4m3fn_decode(rows[r * D + d]);
      if (isnan(q)) rc = ORC_E_NAN;
      const float s = (float)oracle_e8m0_decode(scales[r * nblk + d / 32]);
      const float e = q * s;
      if (out_f32) out_f32[r * D + d] = e;
      if (out_bf16) out_bf16[r * D + d] = oracle_bf16_rne((double)e);
    }
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Projection and gated residual                                            */
/* ------------------------------------------------------------------------ */

/* v = W E for each token, the Engram connection's wkv projection ([VeOmni#1370]
 * config commit: the connection is wkv plus a gate reading the mHC stream),
 * accumulated in fp64 in k order. */
int oracle_project(const uint16_t *E, const uint16_t *W, int64_t T, int64_t K,
                   int64_t hidden, double *v) {
  if (T < 0 || K < 0 || hidden < 0 || (T > 0 && hidden > 0 && (!E || !W || !v)))
    return ORC_E_ARG;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t o = 0; o < hidden; ++o) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += (double)bf16_bits_to_float(E[t * K + k]) *
               (double)bf16_bits_to_float(W[o * K + k]);
      v[t * hidden + o] = acc;
    }
  }
  return ORC_OK;
}

/* Gated residual into the hc streams, before the Engram layer ([NeMo-V41]
 * forward contract: Engram writes into the streams before its layer).  Gate
 * reading: one scalar per (token, stream), sigmoid of the stream's scaled dot
 * product with v, zeroed on dead positions ([vLLM-V41] forward: the gate is
 * zeroed for image-span tokens). */
int oracle_gate_add(const uint16_t *x, const double *v, const uint8_t *keep, int64_t T,
                    int64_t hc, int64_t hidden, uint16_t *y, double *gates_out) {
  if (T < 0 || hc < 1 || hidden < 1 || (T > 0 && (!x || !v || !y))) return ORC_E_ARG;
  for (int64_t t = 0; t < T; ++t) {
    const int k = keep ? (keep[t] != 0) : 1;
    for (int64_t s = 0; s < hc; ++s) {
      const uint16_t *xs = x + (t * hc + s) * hidden;
      uint16_t *ys = y + (t * hc + s) * hidden;
      const double *vt = v + t * hidden;
      double g = 0.0;
      if (k) {
        double dot = 0.0;
        for (int64_t o = 0; o < hidden; ++o) dot += (double)bf16_bits_to_float(xs[o]) * vt[o];
        const double z = dot / sqrt((double)hidden);
        g = 1.0 / (1.0 + exp(-z));
      }
      if (gates_out) gates_out[t * hc + s] = g;
      for (int64_t o = 0; o < hidden; ++o) {
        if (k)
          ys[o] = oracle_bf16_rne((double)bf16_bits_to_float(xs[o]) + g * vt[o]);
        else
          ys[o] = xs[o];
      }
    }
  }
  return ORC_OK;
}
