// layout.cpp -- host-side bucket layout of the Engram sites sharing one hash
// pass (no HIP calls).
//
// Bucket primes ([VeOmni#1370] "feat: support DeepSeek-V4.1-Flash in SeedOmni",
// n-gram memory lookup commit and the validate_bucket_layout review thread):
// for each site (layer), each order 2..4 and each head, the smallest prime at
// or above the floor that no earlier (site, order, head) drew.  That is the
// first num_sites*3*H primes at or above the floor, dealt out site-major, then
// order, then head; that is how it is computed here (Miller-Rabin on a walk
// upward from the floor).
//
// Table split: one table per order (PR summary: 3-table lookup over 2-/3-/4-gram
// tables), so each order's buckets start at offset 0 of its own table; or one
// table per site (the released checkpoint's one embedding per Engram layer),
// with offsets running across the orders.  The row-count guard of the review
// thread (fewer rows than the prime sum is an error, more is allowed) applies
// per table.  With no floor given, the floor is the largest one whose primes
// fit every table; it is found by walking the floor down from an upper bound
// while keeping the window of the first num_sites*3*H primes at or above it.
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "internal.h"

namespace {

uint64_t mulmod(uint64_t a, uint64_t b, uint64_t m) {
  return (uint64_t)((unsigned __int128)a * b % m);
}

uint64_t powmod(uint64_t b, uint64_t e, uint64_t m) {
  uint64_t r = 1 % m;
  b %= m;
  while (e) {
    if (e & 1) r = mulmod(r, b, m);
    b = mulmod(b, b, m);
    e >>= 1;
  }
  return r;
}

// Deterministic Miller-Rabin for 64-bit n (the first twelve prime bases suffice).
bool is_prime(uint64_t n) {
  static const uint64_t bases[] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
  if (n < 2) return false;
  for (uint64_t p : bases) {
    if (n % p == 0) return n == p;
  }
  uint64_t d = n - 1;
  int s = 0;
  while ((d & 1) == 0) {
    d >>= 1;
    ++s;
  }
  for (uint64_t a : bases) {
    uint64_t x = powmod(a, d, n);
    if (x == 1 || x == n - 1) continue;
    bool composite = true;
    for (int r = 1; r < s; ++r) {
      x = mulmod(x, x, n);
      if (x == n - 1) {
        composite = false;
        break;
      }
    }
    if (composite) return false;
  }
  return true;
}

// The first `count` primes >= floor, in increasing order.
std::vector<uint64_t> primes_from(uint64_t floor_, int count) {
  std::vector<uint64_t> out;
  for (uint64_t x = floor_; (int)out.size() < count; ++x)
    if (is_prime(x)) out.push_back(x);
  return out;
}

// Bucket rows per (site, order) of a draw; does every table hold its buckets?
bool window_fits(const std::vector<uint64_t>& p, int sites, int heads, bool per_site,
                 const int64_t rows[3], int64_t sums[ENGRAM_MAX_SITES][3]) {
  bool ok = true;
  for (int st = 0; st < sites; ++st) {
    int64_t site_total = 0;
    for (int n = 0; n < 3; ++n) {
      int64_t s = 0;
      for (int h = 0; h < heads; ++h) s += (int64_t)p[(st * 3 + n) * heads + h];
      sums[st][n] = s;
      site_total += s;
      if (!per_site && s > rows[n]) ok = false;
    }
    if (per_site && site_total > rows[0]) ok = false;
  }
  return ok;
}

}  // namespace

extern "C" int engram_layout_create(const engram_layout_desc* d, engram_layout** out) {
  if (!d || !out) return ENGRAM_E_ARG;
  *out = nullptr;
  const int H = d->heads_per_order;
  if (d->max_ngram != 4 || H < 1 || H > ENGRAM_MAX_HEADS) return ENGRAM_E_ARG;
  if (d->vocab_size < 1 || d->vocab_size > INT32_MAX) return ENGRAM_E_ARG;
  if (d->compressed_vocab < 1) return ENGRAM_E_ARG;
  if (d->compressed_vocab > 65536) return ENGRAM_E_VC_RANGE;  // V_c^4 <= 2^64
  if (d->pad_token_id < 0 || d->pad_token_id >= d->vocab_size) return ENGRAM_E_ARG;
  if (d->row_dim < 1) return ENGRAM_E_ARG;
  if (d->hash_floor < 0) return ENGRAM_E_ARG;
  const int S = d->num_sites == 0 ? 1 : d->num_sites;
  if (S < 1 || S > ENGRAM_MAX_SITES) return ENGRAM_E_ARG;
  if (d->table_split != ENGRAM_TABLES_PER_ORDER && d->table_split != ENGRAM_TABLE_PER_SITE)
    return ENGRAM_E_ARG;
  const bool per_site = d->table_split == ENGRAM_TABLE_PER_SITE;
  for (int n = 0; n < (per_site ? 1 : 3); ++n)
    if (d->rows[n] < 1 || d->rows[n] > INT32_MAX) return ENGRAM_E_ARG;
  int elt;
  if (d->table_dtype == ENGRAM_DTYPE_FP8_E4M3FN)
    elt = 1;
  else if (d->table_dtype == ENGRAM_DTYPE_BF16)
    elt = 2;
  else
    return ENGRAM_E_ARG;
  if (d->scale_layout != ENGRAM_SCALE_ROW_F32 && d->scale_layout != ENGRAM_SCALE_BLOCK32_E8M0)
    return ENGRAM_E_ARG;
  if (d->scale_layout == ENGRAM_SCALE_BLOCK32_E8M0) {
    if (d->table_dtype != ENGRAM_DTYPE_FP8_E4M3FN) return ENGRAM_E_ARG;
    if (d->row_dim % 32 != 0) return ENGRAM_E_ALIGN;
  }
  const int64_t min_pitch = ((int64_t)(d->row_dim + 15) / 16) * 16 * elt;
  if (d->row_pitch_bytes % 16 != 0 || d->row_pitch_bytes < min_pitch) return ENGRAM_E_ALIGN;

  const int cols = 3 * H;
  const int count = S * cols;
  int64_t rows[3] = {d->rows[0], d->rows[1], d->rows[2]};
  std::vector<uint64_t> p;
  int64_t sums[ENGRAM_MAX_SITES][3];
  uint64_t floor_;
  if (d->hash_floor > 0) {
    floor_ = (uint64_t)d->hash_floor;
    p = primes_from(floor_, count);
    if (!window_fits(p, S, H, per_site, rows, sums)) return ENGRAM_E_LAYOUT_ROWS;
  } else {
    int64_t start;
    if (per_site) {
      start = rows[0] / cols;
    } else {
      start = rows[0];
      if (rows[1] < start) start = rows[1];
      if (rows[2] < start) start = rows[2];
      start /= H;
    }
    floor_ = (uint64_t)start;
    if (floor_ < 2) return ENGRAM_E_NOFIT;
    p = primes_from(floor_, count);
    while (!window_fits(p, S, H, per_site, rows, sums)) {
      if (floor_ <= 2) return ENGRAM_E_NOFIT;
      --floor_;
      if (is_prime(floor_)) {  // it joins the window at the front, the largest leaves
        p.insert(p.begin(), floor_);
        p.pop_back();
      }
    }
  }

  engram_layout* L = (engram_layout*)calloc(1, sizeof(engram_layout));
  if (!L) return ENGRAM_E_ARG;
  L->desc = *d;
  L->desc.num_sites = S;
  L->floor = (int64_t)floor_;
  L->heads = H;
  L->cols = cols;
  L->num_sites = S;
  L->all_cols = count;
  L->per_site_table = per_site ? 1 : 0;
  L->scale_block = d->scale_layout == ENGRAM_SCALE_BLOCK32_E8M0 ? 32 : 0;
  for (int st = 0; st < S; ++st) {
    uint64_t acc = 0;  // a site's table: offsets run across its orders
    for (int n = 0; n < 3; ++n) {
      if (!per_site) acc = 0;  // an order's table: offsets restart
      for (int h = 0; h < H; ++h) {
        const int c = (st * 3 + n) * H + h;
        L->prime[c] = (uint32_t)p[c];
        L->offset[c] = (uint32_t)acc;
        L->barrett[c] = UINT64_MAX / p[c];
        acc += p[c];
      }
      L->prime_sum[st][n] = sums[st][n];
    }
  }
  L->seg_pitch = ((int64_t)d->row_dim + 63) / 64 * 64;
  L->k_pad = (int64_t)cols * L->seg_pitch;
  const uint64_t vc = (uint64_t)d->compressed_vocab;
  L->vc_pow[0] = 1;
  L->vc_pow[1] = vc;
  L->vc_pow[2] = vc * vc;
  L->vc_pow[3] = vc * vc * vc;
  *out = L;
  return ENGRAM_OK;
}

extern "C" void engram_layout_destroy(engram_layout* L) { free(L); }

extern "C" int engram_layout_query(const engram_layout* L, engram_layout_info* info) {
  if (!L || !info) return ENGRAM_E_ARG;
  memset(info, 0, sizeof *info);
  info->hash_floor = L->floor;
  info->heads_per_order = L->heads;
  info->row_dim = L->desc.row_dim;
  for (int n = 0; n < 3; ++n) info->rows[n] = L->desc.rows[n];
  for (int st = 0; st < L->num_sites; ++st)
    for (int n = 0; n < 3; ++n) info->prime_sum[st][n] = L->prime_sum[st][n];
  for (int c = 0; c < L->all_cols; ++c) {
    info->primes[c] = L->prime[c];
    info->offsets[c] = L->offset[c];
  }
  info->seg_pitch = L->seg_pitch;
  info->k_pad = L->k_pad;
  info->num_sites = L->num_sites;
  info->table_split = L->per_site_table ? ENGRAM_TABLE_PER_SITE : ENGRAM_TABLES_PER_ORDER;
  info->scale_layout = L->scale_block == 32 ? ENGRAM_SCALE_BLOCK32_E8M0 : ENGRAM_SCALE_ROW_F32;
  return ENGRAM_OK;
}

extern "C" const char* engram_strerror(int s) {
  switch (s) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_E_ARG: return "malformed argument";
    case ENGRAM_E_LAYOUT_ROWS: return "a table has fewer rows than its bucket prime sum";
    case ENGRAM_E_VC_RANGE: return "compressed vocabulary too large for an exact 64-bit key";
    case ENGRAM_E_NEED_STORE: return "a continuing sequence has no rolling-store slot";
    case ENGRAM_E_TOKEN_RANGE: return "token id outside the vocabulary";
    case ENGRAM_E_ROW_RANGE: return "row id outside its table";
    case ENGRAM_E_SEQLENS: return "cu_seqlens is not a non-decreasing 0..T sequence";
    case ENGRAM_E_SLOT_RANGE: return "store slot out of range";
    case ENGRAM_E_MAP_RANGE: return "tid2eid does not map onto [0, compressed_vocab)";
    case ENGRAM_E_ALIGN: return "misaligned pointer, pitch or leading dimension";
    case ENGRAM_E_HIP: return "HIP runtime error";
    case ENGRAM_E_NOFIT: return "no bucket floor fits the table rows";
    case ENGRAM_E_UNSUPPORTED: return "unsupported shape";
    case ENGRAM_E_ID_RANGE: return "compressed id written to the store outside [0, compressed_vocab)";
    case ENGRAM_E_SCRATCH: return "call needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}
