// Work decomposition of the REINFORCE Zero loss's token pass, as plain
// functions the kernel calls and a host program can check (no GPU needed).
//
// A response [s, e) is cut into segments of kSegTokens tokens counted from
// s: segment j is [s + j kSeg, min(e, s + (j + 1) kSeg)). The token pass's
// workgroup b owns the segments whose first token lies in the window
// [b kSeg, (b + 1) kSeg). Its span [p, q) runs from the first segment start
// at or after b kSeg to the first at or after (b + 1) kSeg (or the end of the
// batch). The segment holding token b kSeg ends at most kSeg tokens after its
// start, so p <= (b + 1) kSeg, and q < (b + 2) kSeg: a span is shorter than
// 2 kSeg tokens. Every segment start in a span lies in its window (q is the
// first start at or after the window's end), so a span holds at most one
// segment start of any one response.
#pragma once

#include "itl_config.h"

namespace itl {

__host__ __device__ inline long long plan_clamp(long long x, long long lo, long long hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// The first segment start at or after t of the response [s, e) (e if none).
__host__ __device__ inline long long seg_at_or_after(long long s, long long e, long long t) {
  if (t <= s) return s;
  const long long c = s + ((t - s + kSegTokens - 1) / kSegTokens) * kSegTokens;
  return c < e ? c : e;
}

struct Span {
  long long p, q;
};

// Span of window [w0, w0 + kSeg): (sa, ea) is the response holding token w0,
// (sb, eb) the one holding token w0 + kSeg (ignored when that is past the
// batch). Clamped so that p <= q, q - p <= 2 kSeg and q <= n_tok whatever the
// offsets (bad offsets give unspecified values, never an out-of-bounds index).
__host__ __device__ inline Span window_span(long long w0, long long n_tok, long long sa, long long ea, long long sb,
                                            long long eb) {
  const long long w1 = w0 + kSegTokens;
  long long p = seg_at_or_after(sa, ea, w0);
  long long q = w1 < n_tok ? seg_at_or_after(sb, eb, w1) : n_tok;
  p = plan_clamp(p, w0, w1 < n_tok ? w1 : n_tok);
  q = plan_clamp(q, p, w0 + 2 * kSegTokens < n_tok ? w0 + 2 * kSegTokens : n_tok);
  return Span{p, q};
}

// Windows whose first token w kSeg the response [s, e) holds: w0 .. w1 - 1
// (none for an empty range). The window map of large batches is written
// from these, one response per thread, each window by the one response
// holding its first token.
__host__ __device__ inline long long first_window(long long s) { return (s + kSegTokens - 1) / kSegTokens; }
__host__ __device__ inline long long end_window(long long e) { return (e + kSegTokens - 1) / kSegTokens; }

// The segment start of the response [s, e) that lies in the span [p, q),
// if any (there is at most one).
__host__ __device__ inline bool segment_in_span(long long s, long long e, long long p, long long q, long long& c) {
  if (s >= q) return false;
  c = s >= p ? s : seg_at_or_after(s, e, p);
  return c < e && c < q;
}

// Length of the segment starting at c of the response [s, e), cut at the
// span's end q (a no-op for valid offsets: a span ends at a segment start).
__host__ __device__ inline long long segment_len(long long e, long long c, long long q) {
  long long end = c + kSegTokens < e ? c + kSegTokens : e;
  end = end < q ? end : q;
  return end - c;
}

// The tree that sums a segment: 0 = one lane, 1 = one wavefront, 2 = the
// workgroup.
__host__ __device__ inline int segment_class(long long len) { return len <= kLaneSeg ? 0 : (len <= kWaveSeg ? 1 : 2); }

// Slot of a segment sum of a response longer than one segment: responses of
// more than kSeg tokens start at least kSeg + 1 tokens apart, so slots
// 2 floor(s / kSeg) + j of different responses never meet (a response of q
// full segments and a partial one spans at most q + 1 slots before the next
// such response's first slot, at least 2 q further).
__host__ __device__ inline long long segment_slot(long long s, long long c) {
  return 2 * (s / kSegTokens) + (c - s) / kSegTokens;
}
__host__ __device__ inline long long n_segment_slots(long long n_tok) {
  return 2 * ((n_tok + kSegTokens - 1) / kSegTokens + 1);
}

}  // namespace itl
