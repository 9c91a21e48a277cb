// Host-side check of the logprob kernels' work decomposition (the same
// inline functions the kernels call, from itl_config.h): for each (n_tok,
// vocab) given on the command line, every (token block, slice) pair is
// computed by exactly one workgroup of the wide grid, slices tile the
// vocabulary contiguously, and the narrow grid covers every (64-token block,
// slice) once. Prints "ok <cases>" or the first violation and exits 1.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "itl_config.h"

using namespace itl;

static int check(long long n_tok, long long vocab) {
  const int S = n_slices(vocab), n_vt = n_vocab_tiles(vocab);
  if (S < 1 || S > kMaxSlices || S > n_vt) return printf("bad S=%d for V=%lld\n", S, vocab), 1;
  // slices tile [0, n_vt) contiguously, each non-empty
  for (int s = 0; s < S; ++s)
    if (slice_tile(s + 1, n_vt, S) <= slice_tile(s, n_vt, S)) return printf("empty slice %d V=%lld\n", s, vocab), 1;
  if (slice_tile(0, n_vt, S) != 0 || slice_tile(S, n_vt, S) != n_vt) return printf("slices do not tile V=%lld\n", vocab), 1;
  // wide grid
  const int n_tb = (int)ceil_div(n_tok, kBT);
  const int G = slices_per_group(n_tok, vocab);
  const long long grid = (long long)n_tb * n_slice_groups(n_tok, vocab);
  std::vector<unsigned char> seen((size_t)n_tb * S, 0);
  for (long long b = 0; b < grid; ++b) {
    const WideWork w = wide_work((int)b, n_tb, S, G);
    if (w.tb < 0 || w.tb >= n_tb || w.slice_first < 0 || w.slice_end > S || w.slice_end <= w.slice_first)
      return printf("bad work b=%lld n=%lld V=%lld: tb=%d slices [%d,%d)\n", b, n_tok, vocab, w.tb, w.slice_first,
                    w.slice_end), 1;
    for (int s = w.slice_first; s < w.slice_end; ++s) {
      unsigned char& c = seen[(size_t)w.tb * S + s];
      if (c) return printf("pair (%d,%d) twice n=%lld V=%lld\n", w.tb, s, n_tok, vocab), 1;
      c = 1;
    }
  }
  for (unsigned char c : seen)
    if (!c) return printf("pair missed n=%lld V=%lld\n", n_tok, vocab), 1;
  // narrow grid: blockIdx -> (slice = b % S, token block = b / S)
  if (n_tok <= kNarrowMaxTokens) {
    const long long nb = ceil_div(n_tok, kNarrowBRows) * S;
    std::vector<unsigned char> s2((size_t)nb, 0);
    for (long long b = 0; b < nb; ++b) {
      const long long t0 = (b / S) * kNarrowBRows;
      if (t0 >= n_tok) return printf("narrow block past the tokens n=%lld\n", n_tok), 1;
      s2[(size_t)((b / S) * S + b % S)]++;
    }
    for (unsigned char c : s2)
      if (c != 1) return printf("narrow coverage n=%lld V=%lld\n", n_tok, vocab), 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  int cases = 0;
  for (int i = 1; i + 1 < argc; i += 2) {
    if (check(atoll(argv[i]), atoll(argv[i + 1]))) return 1;
    ++cases;
  }
  printf("ok %d\n", cases);
  return 0;
}
