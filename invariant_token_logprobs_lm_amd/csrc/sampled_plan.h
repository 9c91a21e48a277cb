// Work decomposition of the backward's sampled term, as plain functions the
// kernels call and a host program can check (no GPU needed).
//
// The sampled entry of each token's dlogits row adds coef[t] H[t] to row
// y_t of dW. The tokens are stably sorted by id (a counting sort, one 8-bit
// digit per pass, least significant first: sort_passes(vocab) passes over
// keys sort_key(y, vocab)), so each id's tokens form one run in ascending
// token order. A run of L tokens is summed by a fixed tree that depends on
// L alone:
//   - segments: kRunSeg consecutive tokens of the run, counted from its
//     start, each summed in token order;
//   - groups: kRunGroup consecutive segments, their sums added in order;
//   - the row: the group sums added in order.
// A run of at most kRunSeg tokens is one segment (its sum is the row); one
// of at most kRunSeg * kRunGroup tokens is one group.
//
// Segment and group sums of runs longer than one segment / one group go to
// slots run_slot(s, j, len) (s = the run's first sorted position, j = the
// segment / group index, len = kRunSeg / kRunSeg * kRunGroup). Runs longer
// than len start at least len + 1 positions apart, so the slots
// 2 floor(s / len) + j of different runs never meet (a run of q full pieces
// and a partial one reaches slot 2 floor(s / len) + q; the next such run's
// first slot is at least 2 (floor(s / len) + q)).
#pragma once

#include <stdint.h>

#include "itl_config.h"

namespace itl {

constexpr int kSortDigitBits = 8;
constexpr int kSortBins = 1 << kSortDigitBits;
constexpr int kSortThreads = 256;
constexpr int kSortPerThread = 8;
constexpr int kSortTile = kSortThreads * kSortPerThread;  // tokens per workgroup of a pass
constexpr int kRunSeg = 64;
constexpr int kRunGroup = 64;
constexpr long long kRunGroupTokens = (long long)kRunSeg * kRunGroup;

// Sort key of a token id: the id, or vocab (after every valid id) for an id
// outside [0, vocab), whose token then adds nothing.
__host__ __device__ inline uint32_t sort_key(int32_t y, int vocab) {
  return (uint32_t)y < (uint32_t)vocab ? (uint32_t)y : (uint32_t)vocab;
}

// Digit passes that cover every key 0 .. vocab.
__host__ __device__ inline int sort_passes(int vocab) {
  int bits = 0;
  while (bits < 32 && ((uint32_t)vocab >> bits) != 0u) ++bits;
  return bits == 0 ? 1 : (bits + kSortDigitBits - 1) / kSortDigitBits;
}

__host__ __device__ inline long long sort_blocks(long long n_tok) { return (n_tok + kSortTile - 1) / kSortTile; }

__host__ __device__ inline long long run_slot(long long s, long long j, long long len) { return 2 * (s / len) + j; }
__host__ __device__ inline long long n_run_slots(long long n_tok, long long len) {
  return 2 * ((n_tok + len - 1) / len + 1);
}

__host__ __device__ inline long long n_pieces(long long L, long long len) { return (L + len - 1) / len; }

}  // namespace itl
