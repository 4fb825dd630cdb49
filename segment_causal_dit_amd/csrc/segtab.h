// Device-side walks over the packed segment table (segments s = 0..n_seg-1
// span rows [seg_start[s], seg_start[s+1]), the first seg_text_len[s] rows
// text, the first seg_text_valid[s] of those unpadded).
//
// The table sits in the kernel arguments; indexing it with a run-time index
// is a scalar memory load, and the wait for one shares the counter of the
// wave's LDS reads. The walks below are for loops that visit tiles in
// ascending row order: they touch the table only when the walk crosses into
// another segment, instead of scanning it for every tile.
#pragma once

#include <climits>

namespace segc {

// Segment of a row, for rows visited in ascending order.
struct SegWalk {
  int s;      // segment of the last row asked about
  int next;   // first row of segment s + 1
  template <class P>
  __device__ void init(const P& p, int row) {
    s = 0;
    for (int i = 1; i < p.n_seg; ++i) s += (row >= p.seg_start[i]) ? 1 : 0;
    next = p.seg_start[s + 1];
  }
  template <class P>
  __device__ int at(const P& p, int row) {
    while (row >= next) {
      ++s;
      next = p.seg_start[s + 1];
    }
    return s;
  }
};

// Tiles of `bn` rows that lie wholly inside the video rows of one segment no
// later than `last`: every query of segment >= `last` sees every key in them.
// Tiles are asked about in ascending order.
struct FreeRuns {
  int s;        // segment whose video run is being walked
  int lo, hi;   // tiles [lo, hi) of that run
  template <class P>
  __device__ void set(const P& p, int bn, int last) {
    if (s > last) {
      lo = hi = INT_MAX;
      return;
    }
    const int a = p.seg_start[s] + p.seg_text_len[s];
    lo = (a + bn - 1) / bn;
    hi = p.seg_start[s + 1] / bn;
  }
  template <class P>
  __device__ void init(const P& p, int bn, int last) {
    s = 0;
    set(p, bn, last);
  }
  template <class P>
  __device__ bool free(const P& p, int bn, int last, int tile) {
    while (tile >= hi) {
      ++s;
      set(p, bn, last);
    }
    return tile >= lo;
  }
};

// Visibility of key row j inside a tile of rows [j0, j0 + rows) whose first
// row is in segment sg: the range [lo, hi] of query segments that see it,
// packed lo | hi << 16 (lo > hi: nobody). Video rows of segment s are seen
// by segments >= s, unpadded text rows only by s, padded text by nobody.
// The loop runs over the segments that overlap the tile (uniform bounds).
template <class P>
__device__ inline int key_visibility(const P& p, int sg, int j0, int rows, int j, bool valid) {
  int lo = 0xFFFF, hi = 0;
  for (int s = sg; s < p.n_seg && p.seg_start[s] < j0 + rows; ++s) {
    const int st = p.seg_start[s], en = p.seg_start[s + 1];
    const int ti = j - st;
    if (valid && j >= st && j < en) {
      if (ti >= p.seg_text_len[s]) {
        lo = s;
        hi = 0xFFFF;
      } else if (ti < p.seg_text_valid[s]) {
        lo = s;
        hi = s;
      }
    }
  }
  return lo | (hi << 16);
}

// Segment of row r inside a tile of rows [r0, r0 + rows) whose first row is
// in segment sg (uniform loop over the boundaries inside the tile).
template <class P>
__device__ inline int row_segment(const P& p, int sg, int r0, int rows, int r) {
  int s = sg;
  for (int i = sg + 1; i < p.n_seg && p.seg_start[i] < r0 + rows; ++i) s += (r >= p.seg_start[i]) ? 1 : 0;
  return s;
}

}  // namespace segc
