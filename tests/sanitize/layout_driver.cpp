// Host driver for the library's layout code under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_sanitizers.py, no GPU).
// It creates, queries and destroys layouts for the workload shapes and for a few
// thousand random descriptions (valid and invalid), and checks each created
// layout's invariants on its own: every bucket size is prime, at or above the
// floor, drawn once; offsets are prefix sums inside each table; every table holds
// its buckets; the segment geometry is D rounded up to 64.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <set>

#include "engram.h"

static bool is_prime(int64_t n) {
  if (n < 2) return false;
  for (int64_t d = 2; d * d <= n; ++d)
    if (n % d == 0) return false;
  return true;
}

static int fail(const char* what, int64_t a, int64_t b) {
  fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, (long long)a, (long long)b);
  return 1;
}

static int check(const engram_layout_desc& d, const engram_layout_info& in) {
  const int H = in.heads_per_order, S = in.num_sites;
  if (H != d.heads_per_order) return fail("heads", H, d.heads_per_order);
  if (in.seg_pitch != (d.row_dim + 63) / 64 * 64) return fail("seg_pitch", in.seg_pitch, d.row_dim);
  if (in.k_pad != 3 * H * in.seg_pitch) return fail("k_pad", in.k_pad, in.seg_pitch);
  if (d.hash_floor && in.hash_floor != d.hash_floor) return fail("floor", in.hash_floor, d.hash_floor);
  std::set<int64_t> seen;
  for (int s = 0; s < S; ++s) {
    int64_t acc = 0;
    for (int n = 0; n < 3; ++n) {
      if (in.table_split == ENGRAM_TABLES_PER_ORDER) acc = 0;
      int64_t sum = 0;
      for (int h = 0; h < H; ++h) {
        const int c = (s * 3 + n) * H + h;
        const int64_t p = in.primes[c];
        if (!is_prime(p)) return fail("not prime", p, c);
        if (p < in.hash_floor) return fail("below floor", p, in.hash_floor);
        if (!seen.insert(p).second) return fail("drawn twice", p, c);
        if (in.offsets[c] != acc) return fail("offset", in.offsets[c], acc);
        acc += p;
        sum += p;
      }
      if (in.prime_sum[s][n] != sum) return fail("prime_sum", in.prime_sum[s][n], sum);
      const int64_t rows = in.table_split == ENGRAM_TABLE_PER_SITE ? d.rows[0] : d.rows[n];
      if (acc > rows) return fail("table too small", acc, rows);
    }
  }
  return 0;
}

int main() {
  std::mt19937_64 rng(20261203);
  int created = 0, refused = 0, bad = 0;
  // the workload shapes first, then random descriptions
  const int64_t shapes[][5] = {  // rows, heads, D, floor, sites
      {4096, 2, 128, 0, 1},     {1048576, 2, 512, 0, 1}, {4194304, 1, 1024, 0, 1},
      {5040000, 1, 6500, 0, 1}, {1024, 2, 64, 64, 1},    {384016682, 8, 256, 16000000, 2},
      {500000, 8, 256, 20000, 2}};
  for (int i = 0; i < 3000; ++i) {
    engram_layout_desc d = {};
    d.vocab_size = 129280;
    d.compressed_vocab = 65536;
    d.pad_token_id = 129279;
    d.max_ngram = 4;
    d.table_dtype = ENGRAM_DTYPE_FP8_E4M3FN;
    d.table_split = ENGRAM_TABLES_PER_ORDER;
    d.scale_layout = ENGRAM_SCALE_ROW_F32;
    if (i < (int)(sizeof shapes / sizeof shapes[0])) {
      const int64_t* s = shapes[i];
      d.rows[0] = d.rows[1] = d.rows[2] = s[0];
      d.heads_per_order = (int32_t)s[1];
      d.row_dim = (int32_t)s[2];
      d.hash_floor = s[3];
      d.num_sites = (int32_t)s[4];
      if (d.num_sites > 1) {
        d.table_split = ENGRAM_TABLE_PER_SITE;
        d.scale_layout = ENGRAM_SCALE_BLOCK32_E8M0;
      }
    } else {
      auto r = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); };
      // a valid description, then (one time in three) one field made invalid
      d.heads_per_order = (int32_t)r(1, 8);
      d.num_sites = (int32_t)r(0, 4);
      d.table_split = (int32_t)r(0, 1);
      const int64_t base = r(2000, 3000000);
      for (int n = 0; n < 3; ++n) d.rows[n] = base + r(0, 5000);
      d.hash_floor = r(0, 2) == 0 ? 0 : r(2, base / 40 + 2);
      d.row_dim = (int32_t)(r(1, 280) * 32);
      d.table_dtype = r(0, 3) == 0 ? ENGRAM_DTYPE_BF16 : ENGRAM_DTYPE_FP8_E4M3FN;
      d.scale_layout = r(0, 1) ? ENGRAM_SCALE_BLOCK32_E8M0 : ENGRAM_SCALE_ROW_F32;
      d.compressed_vocab = r(2, 65536);
      if (r(0, 2) == 0) {
        switch (r(0, 9)) {
          case 0: d.heads_per_order = (int32_t)r(-1, 0) + 9 * (int32_t)r(0, 1); break;
          case 1: d.num_sites = (int32_t)r(5, 7); break;
          case 2: d.rows[r(0, 2)] = r(-3, 40); break;
          case 3: d.row_dim = (int32_t)r(-2, 0); break;
          case 4: d.table_dtype = (int32_t)r(3, 9); break;
          case 5: d.compressed_vocab = r(0, 1) ? r(-2, 1) : r(65537, 1 << 20); break;
          case 6: d.pad_token_id = r(0, 1) ? -1 : d.vocab_size; break;
          case 7: d.max_ngram = (int32_t)r(2, 3); break;
          case 8: d.reserved = 1; break;
          default: d.table_split = (int32_t)r(2, 5); break;
        }
      }
    }
    const int64_t elt = d.table_dtype == ENGRAM_DTYPE_BF16 ? 2 : 1;
    const int64_t want = ((int64_t)(d.row_dim > 0 ? d.row_dim : 0) + 15) / 16 * 16 * elt;
    d.row_pitch_bytes = (rng() % 8 == 0) ? want + (int64_t)(rng() % 40) - 20 : (want + 127) / 128 * 128;
    engram_layout* L = nullptr;
    const int rc = engram_layout_create(&d, &L);
    if (rc != ENGRAM_OK) {
      if (L) return fail("handle on error", rc, 0);
      if (engram_strerror(rc) == nullptr) return fail("strerror", rc, 0);
      ++refused;
      continue;
    }
    engram_layout_info in;
    if (engram_layout_query(L, &in) != ENGRAM_OK) return fail("query", i, 0);
    bad += check(d, in);
    engram_layout_destroy(L);
    ++created;
  }
  if (engram_layout_create(nullptr, nullptr) == ENGRAM_OK) return fail("null desc", 0, 0);
  engram_layout_destroy(nullptr);
  for (int s = -30; s <= 5; ++s)
    if (engram_strerror(s) == nullptr) return fail("strerror", s, 0);
  if (bad) return 1;
  printf("layout driver ok: %d layouts created and checked, %d refused\n", created, refused);
  return 0;
}
