/* Exhaustive host check of the span partition (dcp_partition.h), which the partial-
 * attention kernels and the split-K merge share.  Built with gcc (optionally with
 * -fsanitize=address,undefined) by tests/test_partition.py; prints the number of failures.
 *
 * 1. span_of is the inverse of span_start: for every weighted position x < WT,
 *    span_start(w) <= x < span_start(w + 1) with w = span_of(x), plain and XCD-weighted.
 * 2. For random batches (tile counts including empty requests, per-request charge A,
 *    P spans), a brute-force walk that assigns every tile to the span whose weighted
 *    range holds its position gives, per span, the first and one-past-last tile and the
 *    pieces (request runs) in order; the kernels' span location (dcp_span_cut over the
 *    request holding the span's start / end) must give the same tile range, and the
 *    split-K merge's slot choice (dcp_piece_slot over each request's spans) must name
 *    the slot the walk gives the piece (2w for a span's first piece, 2w+1 for its last). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dcp_partition.h"

static long failures = 0;
#define CHECK(c, ...)                                        \
  do {                                                       \
    if (!(c)) {                                              \
      if (failures < 20) { printf("FAIL: " __VA_ARGS__); printf("\n"); } \
      ++failures;                                            \
    }                                                        \
  } while (0)

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint64_t rnd(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12; rng_state ^= rng_state << 25; rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}

static void check_inverse(int64_t WT, int64_t P, int weighted) {
  for (int64_t x = 0; x < WT; ++x) {
    const int64_t w = dcp_span_of(x, WT, P, weighted);
    CHECK(w >= 0 && w < P, "span_of out of range WT=%lld P=%lld x=%lld", (long long)WT, (long long)P, (long long)x);
    if (w < 0 || w >= P) continue;
    CHECK(dcp_span_start(w, WT, P, weighted) <= x && x < dcp_span_start(w + 1, WT, P, weighted),
          "span_of(%lld) = %lld, WT=%lld P=%lld weighted=%d", (long long)x, (long long)w,
          (long long)WT, (long long)P, weighted);
  }
}

static void check_inverse_sampled(int64_t WT, int64_t P, int weighted) {
  /* every span boundary and its neighbours, plus random positions */
  for (int64_t w = 0; w <= P; ++w) {
    const int64_t s = dcp_span_start(w, WT, P, weighted);
    for (int64_t d = -2; d <= 2; ++d) {
      const int64_t x = s + d;
      if (x < 0 || x >= WT) continue;
      const int64_t v = dcp_span_of(x, WT, P, weighted);
      CHECK(v >= 0 && v < P && dcp_span_start(v, WT, P, weighted) <= x &&
            x < dcp_span_start(v + 1, WT, P, weighted), "sampled WT=%lld P=%lld x=%lld", (long long)WT,
            (long long)P, (long long)x);
    }
  }
  for (int k = 0; k < 2000; ++k) {
    const int64_t x = (int64_t)(rnd() % (uint64_t)WT);
    const int64_t v = dcp_span_of(x, WT, P, weighted);
    CHECK(v >= 0 && v < P && dcp_span_start(v, WT, P, weighted) <= x &&
          x < dcp_span_start(v + 1, WT, P, weighted), "random WT=%lld P=%lld x=%lld", (long long)WT,
          (long long)P, (long long)x);
  }
}

#define MAXB 64
#define MAXP 300

static void check_batch(int B, const int64_t* n, int64_t A, int64_t P, int weighted) {
  int64_t WP[MAXB + 1], F[MAXB + 1];
  WP[0] = 0; F[0] = 0;
  for (int b = 0; b < B; ++b) {
    WP[b + 1] = WP[b] + (n[b] > 0 ? A + n[b] : 0);
    F[b + 1] = F[b] + n[b];
  }
  const int64_t WT = WP[B], TT = F[B];
  if (WT == 0) return;
  /* brute force: span of every tile by scanning the span starts */
  static int64_t first_tile[MAXP], end_tile[MAXP];
  static int piece_req[MAXP][MAXB + 2], piece_cnt[MAXP];
  for (int64_t w = 0; w < P; ++w) { first_tile[w] = -1; end_tile[w] = -1; piece_cnt[w] = 0; }
  int64_t w = 0; /* tiles come in increasing weighted position: the span only moves up */
  for (int b = 0; b < B; ++b)
    for (int64_t k = 0; k < n[b]; ++k) {
      const int64_t pos = WP[b] + A + k;
      while (w + 1 < P && dcp_span_start(w + 1, WT, P, weighted) <= pos) ++w;
      const int64_t tile = F[b] + k;
      if (first_tile[w] < 0) first_tile[w] = tile;
      end_tile[w] = tile + 1;
      if (piece_cnt[w] == 0 || piece_req[w][piece_cnt[w] - 1] != b) piece_req[w][piece_cnt[w]++] = b;
    }
  /* the kernels' span location */
  for (int64_t w = 0; w < P; ++w) {
    const int64_t x0 = dcp_span_start(w, WT, P, weighted), x1 = dcp_span_start(w + 1, WT, P, weighted);
    int64_t start = 0, end = 0;
    if (x0 < x1) {
      for (int b = 0; b < B; ++b) {
        if (n[b] == 0) continue;
        const int64_t wend = WP[b] + A + n[b];
        if (WP[b] <= x0 && x0 < wend) start = dcp_span_cut(x0, WP[b], A, F[b]);
        if (WP[b] <= x1 && x1 < wend) end = dcp_span_cut(x1, WP[b], A, F[b]);
      }
      if (x1 >= WT) end = TT;
    }
    const int64_t bs = first_tile[w] < 0 ? 0 : first_tile[w], be = first_tile[w] < 0 ? 0 : end_tile[w];
    CHECK((start >= end && first_tile[w] < 0) || (start == bs && end == be),
          "span %lld tiles [%lld,%lld) vs brute [%lld,%lld) (P=%lld WT=%lld)", (long long)w, (long long)start,
          (long long)end, (long long)bs, (long long)be, (long long)P, (long long)WT);
  }
  /* slots: a span's first piece takes 2w, its last 2w+1 (a span holds at most two
   * pieces of requests it does not hold whole) */
  for (int b = 0; b < B; ++b) {
    if (n[b] == 0) continue;
    const int64_t wf = dcp_span_of(WP[b] + A, WT, P, weighted);
    const int64_t wl = dcp_span_of(WP[b] + A + n[b] - 1, WT, P, weighted);
    for (int64_t w = 0; w < P; ++w) {
      int idx = -1;
      for (int i = 0; i < piece_cnt[w]; ++i)
        if (piece_req[w][i] == b) idx = i;
      const int inside = w >= wf && w <= wl;
      if (!inside) { CHECK(idx < 0, "request %d has a tile in span %lld outside [%lld,%lld]", b, (long long)w, (long long)wf, (long long)wl); continue; }
      if (dcp_span_empty(w, WT, P, weighted)) { CHECK(idx < 0, "empty span %lld holds a tile", (long long)w); continue; }
      CHECK(idx >= 0, "span %lld in [%lld,%lld] holds no tile of request %d", (long long)w, (long long)wf, (long long)wl, b);
      if (idx < 0 || wf == wl) continue;
      CHECK(idx == 0 || idx == piece_cnt[w] - 1, "split piece in the middle of span %lld", (long long)w);
      const int64_t brute = 2 * w + (idx == 0 ? 0 : 1);
      CHECK(dcp_piece_slot(w, wf, dcp_span_start(w, WT, P, weighted), WP[b]) == brute,
            "slot of request %d in span %lld: %lld vs %lld", b, (long long)w,
            (long long)dcp_piece_slot(w, wf, dcp_span_start(w, WT, P, weighted), WP[b]), (long long)brute);
    }
  }
}

int main(void) {
  /* 1. exhaustive inverse for small totals, sampled for large ones */
  for (int64_t P = 1; P <= 264; P += (P < 40 ? 1 : 8)) {
    for (int weighted = 0; weighted <= (P % 8 == 0 ? 1 : 0); ++weighted) {
      for (int64_t WT = 1; WT <= 700; ++WT) check_inverse(WT, P, weighted);
      const int64_t big[] = {4095, 65536, 131079, 1000003, 10000019, 123456789};
      for (int i = 0; i < 6; ++i) check_inverse_sampled(big[i], P, weighted);
    }
  }
  /* 2. random batches */
  for (int iter = 0; iter < 3000; ++iter) {
    const int B = 1 + (int)(rnd() % MAXB);
    int64_t n[MAXB];
    const int mode = (int)(rnd() % 4);
    for (int b = 0; b < B; ++b) {
      const uint64_t r = rnd();
      n[b] = (r % 7 == 0) ? 0 : (mode == 0 ? (int64_t)(r % 4) : mode == 1 ? (int64_t)(r % 40) :
                                 mode == 2 ? (int64_t)(r % 3000) : (int64_t)((r % 5 == 0) ? r % 40000 : r % 300));
    }
    const int64_t Ps[] = {1, 2, 3, 7, 8, 16, 33, 64, 128, 200, 256};
    const int64_t P = Ps[rnd() % 11];
    const int64_t A = (int64_t)(rnd() % 6);
    const int weighted = (P % 8 == 0) ? (int)(rnd() % 2) : 0;
    check_batch(B, n, A, P, weighted);
  }
  printf("%ld failures\n", failures);
  return failures != 0;
}
