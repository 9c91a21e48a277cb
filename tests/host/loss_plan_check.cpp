// Host-side check of the loss token pass's work decomposition (the same
// inline functions the kernel calls, from loss_plan.h), on seeded response
// layouts: the windows' spans tile the batch, every token lies in exactly one
// segment, owned by exactly one window, each segment starts at a multiple of
// kSegTokens from its response's start and lies inside its span, a span is
// shorter than 2 kSegTokens and holds at most one start of a response, the
// kernel's enumeration rounds reach every response that overlaps a span, and
// the segment-sum slots of different responses never meet, and the window
// map names each window's holder.
// Usage: loss_plan_check <seed> <n_layouts>. Prints "ok <layouts>" or the
// first violation and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "loss_plan.h"

using namespace itl;

static uint64_t rng_state;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static long long uniform(long long lo, long long hi) { return lo + (long long)(next_u64() % (uint64_t)(hi - lo + 1)); }

static std::vector<long long> draw_lengths(int kind) {
  std::vector<long long> T;
  const int n = (int)uniform(1, 3000);
  for (int i = 0; i < n; ++i) {
    switch (kind) {
      case 0: T.push_back(uniform(1, 8)); break;
      case 1: T.push_back(uniform(1, 300)); break;
      case 2: T.push_back(uniform(kSegTokens - 2, kSegTokens + 2)); break;
      case 3: T.push_back(uniform(1, 5 * kSegTokens)); break;
      case 4: T.push_back(next_u64() % 50 == 0 ? uniform(kSegTokens, 20 * kSegTokens) : uniform(1, 40)); break;
      default: T.push_back(uniform(1, 3)); break;
    }
  }
  if (kind == 5) T.assign(1, uniform(1, 50 * kSegTokens));  // one long response
  return T;
}

static int check(const std::vector<long long>& T) {
  const int n_resp = (int)T.size();
  std::vector<long long> off(n_resp + 1, 0);
  for (int i = 0; i < n_resp; ++i) off[i + 1] = off[i] + T[i];
  const long long n_tok = off[n_resp];
  std::vector<unsigned char> covered(n_tok, 0);
  const long long n_win = (n_tok + kSegTokens - 1) / kSegTokens;
  long long prev_q = 0;
  auto holder = [&](long long t) {  // largest i with off[i] <= t
    return (int)(std::upper_bound(off.begin(), off.begin() + n_resp, t) - off.begin()) - 1;
  };
  for (long long b = 0; b < n_win; ++b) {
    const long long w0 = b * kSegTokens, w1 = w0 + kSegTokens;
    const int ia = holder(w0), ib = holder(w1 < n_tok ? w1 : w0);
    const Span sp = window_span(w0, n_tok, off[ia], off[ia + 1], off[ib], off[ib + 1]);
    if (sp.p != prev_q) return printf("spans do not tile: window %lld starts at %lld, previous ended %lld\n", b, sp.p, prev_q), 1;
    if (sp.q < sp.p || sp.q - sp.p > 2 * kSegTokens || sp.p < w0) return printf("bad span [%lld, %lld) window %lld\n", sp.p, sp.q, b), 1;
    prev_q = sp.q;
    // the kernel's enumeration: rounds of kLossThreads responses from the
    // holder of p, continuing while the next response starts before q
    const int i0 = (sp.p < off[ia + 1] || ia + 1 >= n_resp) ? ia : ia + 1;
    int last = i0 - 1;
    for (int base = i0; base < n_resp; base += kLossThreads) {
      last = std::min(n_resp, base + kLossThreads) - 1;
      const int nxt = base + kLossThreads;
      if (nxt >= n_resp || off[nxt] >= sp.q) break;
    }
    for (int i = std::max(0, i0 - 2); i <= std::min(n_resp - 1, last + 2); ++i) {
      long long c[1];
      const int n = segment_in_span(off[i], off[i + 1], sp.p, sp.q, c[0]) ? 1 : 0;
      if (n > 0 && (i < i0 || i > last)) return printf("response %d overlaps window %lld but is not enumerated\n", i, b), 1;
      if (i < i0 || i > last) continue;  // (a response the kernel does not visit adds nothing)
      for (int k = 0; k < n; ++k) {
        if ((c[k] - off[i]) % kSegTokens != 0) return printf("segment start off the grid\n"), 1;
        if (c[k] < w0 || c[k] >= w1) return printf("segment start %lld outside window %lld\n", c[k], b), 1;
        const long long len = segment_len(off[i + 1], c[k], sp.q);
        const long long full = std::min(off[i + 1], c[k] + kSegTokens) - c[k];
        if (len != full || len < 1) return printf("segment cut by the span end\n"), 1;
        if (segment_class(len) < 0 || segment_class(len) > 2) return 1;
        for (long long t = c[k]; t < c[k] + len; ++t) {
          if (t < sp.p || t >= sp.q) return printf("token %lld outside its span\n", t), 1;
          covered[t]++;
        }
      }
    }
  }
  // the window map: each window written once, by the holder of its first token
  {
    std::vector<int> writer(n_win, -1);
    for (int i = 0; i < n_resp; ++i)
      for (long long w = first_window(off[i]); w < std::min(end_window(off[i + 1]), n_win); ++w) {
        if (writer[w] != -1) return printf("window %lld written by responses %d and %d\n", w, writer[w], i), 1;
        writer[w] = i;
      }
    for (long long w = 0; w < n_win; ++w)
      if (writer[w] != holder(w * kSegTokens)) return printf("window %lld mapped to %d, held by %d\n", w, writer[w], holder(w * kSegTokens)), 1;
  }
  // (tokens of a response never visited stay uncovered and fail below)
  if (prev_q != n_tok) return printf("spans end at %lld, batch at %lld\n", prev_q, n_tok), 1;
  for (long long t = 0; t < n_tok; ++t)
    if (covered[t] != 1) return printf("token %lld covered %d times\n", t, covered[t]), 1;
  // segment-sum slots of the responses longer than one segment
  const long long n_slots = n_segment_slots(n_tok);
  std::vector<int> owner(n_slots, -1);
  for (int i = 0; i < n_resp; ++i) {
    if (T[i] <= kSegTokens) continue;
    for (long long c = off[i]; c < off[i + 1]; c += kSegTokens) {
      const long long slot = segment_slot(off[i], c);
      if (slot < 0 || slot >= n_slots) return printf("slot %lld out of range\n", slot), 1;
      if (owner[slot] != -1) return printf("slot %lld shared by responses %d and %d\n", slot, owner[slot], i), 1;
      owner[slot] = i;
    }
  }
  return 0;
}

int main(int argc, char** argv) {
  rng_state = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
  const int n = argc > 2 ? atoi(argv[2]) : 100;
  for (int k = 0; k < n; ++k)
    if (check(draw_lengths(k % 6))) return 1;
  printf("ok %d\n", n);
  return 0;
}
