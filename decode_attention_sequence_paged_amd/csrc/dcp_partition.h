/* Work partition of one rank's tiles into spans (host and device; plain C as well).
 *
 * A rank's local tokens of the whole batch are cut into tiles of T tokens (a tile never
 * crosses a request), and the tiles are laid out on a weighted line: request b occupies
 * the weighted range [WP_b, WP_(b+1)) with WP_(b+1) = WP_b + A + n_b, where n_b is its
 * tile count and A the extra work charged to every request with tiles (its query slice
 * and output row); its tile k sits at weighted position WP_b + A + k.  Span w covers
 * the weighted range [span_start(w), span_start(w+1)) of the total WT, i.e. exactly the
 * tiles whose weighted positions fall into it (a boundary inside a request's charge
 * therefore moves to the request's first tile).  A request whose tiles fall into
 * several spans is computed piecewise; span w owns workspace slots 2w (its first
 * request piece) and 2w+1 (its last).
 *
 * The partial-attention kernels, the split-K merge and the host tests use these same
 * functions. */
#ifndef DCP_PARTITION_H_
#define DCP_PARTITION_H_

#include <stdint.h>

#include "dcp_shard.h" /* DCP_HD */

/* XCD-weighted spans: when span w runs on XCD w % 8 (one head group, P % 8 == 0), the
 * work-groups of the odd XCDs stream 5-7% slower than those of the even ones (measured
 * in every call, on every box tried), so an odd-XCD span gets DCP_SPAN_ODD /
 * DCP_SPAN_EVEN of an even one's work.  Span w then starts at unit U(w) of U(P). */
#define DCP_SPAN_EVEN 17
#define DCP_SPAN_ODD 16
#define DCP_SPAN_GROUP (4 * (DCP_SPAN_EVEN + DCP_SPAN_ODD))

/* U(w): units of work before span w (w itself unless XCD-weighted). */
DCP_HD int64_t dcp_span_units(int64_t w, int weighted) {
  if (!weighted) return w;
  const int64_t j = w & 7;
  return (w >> 3) * DCP_SPAN_GROUP + DCP_SPAN_EVEN * ((j + 1) >> 1) + DCP_SPAN_ODD * (j >> 1);
}

/* Weighted start of span w (0 <= w <= P; span_start(P) = WT). */
DCP_HD int64_t dcp_span_start(int64_t w, int64_t WT, int64_t P, int weighted) {
  return dcp_span_units(w, weighted) * WT / dcp_span_units(P, weighted);
}

/* The span that holds weighted position x (0 <= x < WT): the last w with
 * span_start(w) <= x, i.e. with U(w) <= ((x + 1) U(P) - 1) / WT. */
DCP_HD int64_t dcp_span_of(int64_t x, int64_t WT, int64_t P, int weighted) {
  const int64_t umax = ((x + 1) * dcp_span_units(P, weighted) - 1) / WT;
  if (!weighted) return umax;
  const int64_t g = umax / DCP_SPAN_GROUP, r = umax - g * DCP_SPAN_GROUP;
  int64_t j = 0;
  for (int k = 1; k < 8; ++k)
    if (DCP_SPAN_EVEN * ((k + 1) >> 1) + DCP_SPAN_ODD * (k >> 1) <= r) j = k;
  const int64_t w = g * 8 + j;
  return w < P ? w : P - 1;
}

/* A span with an empty weighted range holds no tile. */
DCP_HD int dcp_span_empty(int64_t w, int64_t WT, int64_t P, int weighted) {
  return dcp_span_start(w, WT, P, weighted) == dcp_span_start(w + 1, WT, P, weighted);
}

/* First tile (in the rank's global tile order) at or after weighted position x, for x
 * inside the weighted range of the request whose first tile is F and whose range
 * starts at WP (x inside its charge maps to its first tile). */
DCP_HD int64_t dcp_span_cut(int64_t x, int64_t WP, int64_t A, int64_t F) {
  const int64_t k = x - WP - A;
  return F + (k > 0 ? k : 0);
}

/* Workspace slot of the piece of a request (weighted start WP, tiles in spans w_first ..
 * w_last) that span w computes: the first span may start before the request (the piece
 * is then that span's last, slot 2w+1); every later span starts inside it (its first
 * piece, slot 2w). */
DCP_HD int64_t dcp_piece_slot(int64_t w, int64_t w_first, int64_t span_x0, int64_t WP) {
  return 2 * w + ((w == w_first && span_x0 < WP) ? 1 : 0);
}

#endif /* DCP_PARTITION_H_ */
