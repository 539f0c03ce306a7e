// Tile-schedule arithmetic shared by every attention kernel of the library:
// which keys a query row sees under the band mask, which query rows a key tile
// needs, which keys a query tile needs, the block cover of such a range, the
// balanced split of a block range over jobs, and whether a (query tile, key
// tile) pair is visible everywhere (so that the element mask can be skipped).
//
// The mask is the sparse-mode band of page "CANN ops-transformer FlashAttnGrad
// 算子详解", section 四 4.3, read with bottom-right alignment: with
// off = s2 - s1, key j is visible to query row i iff
//   (left < 0 || j >= i + off - left)  and  (right < 0 || j <= i + off + right),
// where a negative bound means unbounded.  Causal is (left, 0).  The host
// normalises every mask mode to (left, right) with left, right >= -1, and the
// ranges below are exact (neither too wide nor too narrow) under that rule.
//
// Plain constexpr functions with no HIP dependence: HIP compiles them for the
// device as well as the host, and a host compiler builds them into the
// brute-force check of the schedule.
#pragma once

namespace fa_sched {

constexpr int imin(int a, int b) { return a < b ? a : b; }
constexpr int imax(int a, int b) { return a > b ? a : b; }

// Half-open index range [lo, hi); empty when hi <= lo.
struct Span {
  int lo, hi;
};

// The band rule for one (row, key) pair; rows and keys past the sequence
// ends are never visible.
constexpr bool visible(int i, int j, int s1, int s2, int off, int left, int right) {
  return i >= 0 && i < s1 && j >= 0 && j < s2 && (left < 0 || j >= i + off - left) &&
         (right < 0 || j <= i + off + right);
}

// Query rows of [0, s1) that see at least one key of [j0, j1), for
// 0 <= j0 < j1 <= s2.
constexpr Span rows_seeing(int s1, int j0, int j1, int off, int left, int right) {
  return Span{right >= 0 ? imax(0, j0 - off - right) : 0, left >= 0 ? imin(s1, j1 - off + left) : s1};
}

// Keys of [0, s2) that at least one row of [i0, i1) sees, for 0 <= i0 < i1 <= s1.
constexpr Span keys_seen(int s2, int i0, int i1, int off, int left, int right) {
  return Span{left >= 0 ? imax(0, i0 + off - left) : 0, right >= 0 ? imin(s2, i1 + off + right) : s2};
}

// Keys visible to row i (empty when i is past the end).
constexpr Span keys_of_row(int i, int s1, int s2, int off, int left, int right) {
  return i < s1 ? keys_seen(s2, i, i + 1, off, left, right) : Span{0, 0};
}

// Rows that see key j (empty when j is past the end).
constexpr Span rows_of_key(int j, int s1, int s2, int off, int left, int right) {
  return j < s2 ? rows_seeing(s1, j, j + 1, off, left, right) : Span{0, 0};
}

// Rows of a sequence that take part: the first `used` of its `alloc` rows when a
// per-sequence used length is given (seqused_q / seqused_kv), clamped to
// [0, alloc]; the rest are padding that nothing attends and whose gradients are
// zero.
constexpr int used_len(int alloc, int used) { return used < 0 ? 0 : (used < alloc ? used : alloc); }

// Blocks of `bs` indices that cover r: block indices [lo, hi) (empty when r is).
constexpr Span blocks_covering(Span r, int bs) {
  return r.hi > r.lo ? Span{r.lo / bs, (r.hi + bs - 1) / bs} : Span{r.lo / bs, r.lo / bs};
}

// Part p of `parts` contiguous, balanced parts of the block range r.
constexpr Span split_part(Span r, int p, int parts) {
  return Span{r.lo + (int)((long long)(r.hi - r.lo) * p / parts),
              r.lo + (int)((long long)(r.hi - r.lo) * (p + 1) / parts)};
}

// True when every row of [i0, i0 + bi) and every key of [j0, j0 + bj) lie in
// the sequence and every pair of them is visible: the tile needs no mask.
constexpr bool tile_full(int i0, int bi, int j0, int bj, int s1, int s2, int off, int left, int right) {
  return i0 + bi <= s1 && j0 + bj <= s2 && (right < 0 || j0 + bj - 1 <= i0 + off + right) &&
         (left < 0 || j0 >= i0 + bi - 1 + off - left);
}

// A span as one unsigned compare relative to an origin: x (an offset from
// `origin`) is inside iff (unsigned)x - base <= span.  An empty span gets a
// base that no offset in [0, 2^31 - 1) reaches.
struct Window {
  unsigned base, span;
};
constexpr Window window(Span s, int origin) {
  return s.hi > s.lo ? Window{(unsigned)(s.lo - origin), (unsigned)(s.hi - 1 - s.lo)} : Window{0x7fffffffu, 0u};
}
constexpr bool in_window(Window w, int x) { return (unsigned)x - w.base <= w.span; }

}  // namespace fa_sched
