// Layout maps and the causal ring schedule, shared by the host API and the
// kernels (host + device inline functions).
//
// Every chunk is one or two row segments on which the global token position
// is an arithmetic progression pos = base + step * (row - row0):
//   contiguous: one segment, base c*L, step 1
//   striped:    one segment, base c,   step N
//   zig-zag:    rows [0, s): base c*s; rows [s, 2s): base (2N-1-c)*s; step 1
// For a query segment and a KV segment with the same step g the causal rule
// "key position <= query position" (lecture 013 notes; the diagonal is kept
// as with triu(diagonal=1) in ring_attention_causal_step) becomes
//   key row k visible to query row p  <=>  k - p <= delta,
//   delta = floor((base_q - base_k) / g),
// with rows counted from each segment's start.  One integer per segment pair
// therefore covers all three layouts.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define RA_HD __host__ __device__ __forceinline__
#else
#define RA_HD inline
#endif

namespace ra {

enum Layout : int32_t { CONTIGUOUS = 0, STRIPED = 1, ZIGZAG = 2 };
enum Kind : int32_t { FULL = 0, MASKED = 1, SKIP = 2 };

struct Segment {
  int32_t row0;   // first row inside the chunk
  int32_t len;    // number of rows
  int64_t base;   // global position of row0
  int64_t step;   // position increment per row
};

RA_HD int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

RA_HD int num_segments(int32_t layout) { return layout == ZIGZAG ? 2 : 1; }

// Segment sidx of chunk c; L = seq / n is passed in so that device code needs no division.
RA_HD Segment segment_l(int32_t layout, int64_t L, int32_t n, int32_t c, int sidx) {
  Segment g;
  if (layout == CONTIGUOUS) {
    g.row0 = 0; g.len = (int32_t)L; g.base = (int64_t)c * L; g.step = 1;
  } else if (layout == STRIPED) {
    g.row0 = 0; g.len = (int32_t)L; g.base = c; g.step = n;
  } else {
    const int64_t s = L / 2;
    g.row0 = sidx == 0 ? 0 : (int32_t)s;
    g.len = (int32_t)s;
    g.base = (sidx == 0 ? (int64_t)c : (int64_t)(2 * n - 1 - c)) * s;
    g.step = 1;
  }
  return g;
}

RA_HD Segment segment(int32_t layout, int64_t seq, int32_t n, int32_t c, int sidx) {
  return segment_l(layout, seq / n, n, c, sidx);
}

RA_HD int64_t position(int32_t layout, int64_t seq, int32_t n, int32_t c, int64_t row) {
  const int64_t L = seq / n;
  if (layout == CONTIGUOUS) return (int64_t)c * L + row;
  if (layout == STRIPED) return row * n + c;
  const int64_t s = L / 2;
  return row < s ? (int64_t)c * s + row : (int64_t)(2 * n - 1 - c) * s + (row - s);
}

RA_HD int64_t pair_delta(const Segment& q, const Segment& k) {
  return q.step == 1 ? q.base - k.base : floor_div(q.base - k.base, q.step);
}

// FULL when every key row is visible to every query row, SKIP when none is.
RA_HD int32_t pair_kind(int64_t delta, int64_t q_len, int64_t k_len) {
  if (delta >= k_len - 1) return FULL;
  if (delta < -(q_len - 1)) return SKIP;
  return MASKED;
}

RA_HD int32_t ring_kv_chunk(int32_t q_chunk, int32_t step, int32_t n) {
  int32_t j = (q_chunk - step) % n;
  return j < 0 ? j + n : j;
}

}  // namespace ra
