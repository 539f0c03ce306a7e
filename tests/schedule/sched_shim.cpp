// C entry points over the kernels' tile-schedule header, built by the host
// compiler for the brute-force schedule test.  Each one composes the header's
// functions the way the kernels do: a key tile's query-block range and its
// split over jobs (dK/dV kernels), a query tile's key-block range (dQ and
// forward kernels), the per-element windows of partial tiles, and the
// full-tile test.
#include "../../flashattention_backward_fa_amd/csrc/fa_bwd_schedule.h"

using namespace fa_sched;

extern "C" {

int sched_visible(int i, int j, int s1, int s2, int left, int right) {
  return visible(i, j, s1, s2, s2 - s1, left, right);
}

// Query blocks [out[0], out[1]) of size br for the key tile at j0 (size bc),
// split part p of `parts`.
void sched_key_tile_blocks(int s1, int s2, int j0, int bc, int br, int p, int parts, int left, int right, int* out) {
  const int j1 = imin(j0 + bc, s2);
  const Span r = split_part(blocks_covering(rows_seeing(s1, j0, j1, s2 - s1, left, right), br), p, parts);
  out[0] = r.lo;
  out[1] = r.hi;
}

// Query rows [out[0], out[1]) that see a key of [j0, j1).
void sched_rows_seeing(int s1, int s2, int j0, int j1, int left, int right, int* out) {
  const Span r = rows_seeing(s1, j0, j1, s2 - s1, left, right);
  out[0] = r.lo;
  out[1] = r.hi;
}

// Key blocks [out[0], out[1]) of size bk for the query tile at i0 (size bq).
void sched_query_tile_blocks(int s1, int s2, int i0, int bq, int bk, int left, int right, int* out) {
  const int i1 = imin(i0 + bq, s1);
  const Span r = blocks_covering(keys_seen(s2, i0, i1, s2 - s1, left, right), bk);
  out[0] = r.lo;
  out[1] = r.hi;
}

void sched_keys_seen(int s1, int s2, int i0, int i1, int left, int right, int* out) {
  const Span r = keys_seen(s2, i0, i1, s2 - s1, left, right);
  out[0] = r.lo;
  out[1] = r.hi;
}

int sched_tile_full(int i0, int bi, int j0, int bj, int s1, int s2, int left, int right) {
  return tile_full(i0, bi, j0, bj, s1, s2, s2 - s1, left, right);
}

// Membership of offsets 0..n-1 from `origin` in the window of row i's keys
// (by_row != 0) or of key j's rows (by_row == 0).
void sched_window_mask(int by_row, int idx, int origin, int n, int s1, int s2, int left, int right,
                       unsigned char* out) {
  const Span s = by_row ? keys_of_row(idx, s1, s2, s2 - s1, left, right) : rows_of_key(idx, s1, s2, s2 - s1, left, right);
  const Window w = window(s, origin);
  for (int x = 0; x < n; ++x) out[x] = in_window(w, x) ? 1 : 0;
}

}  // extern "C"
