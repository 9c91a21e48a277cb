// Host-side check of the backward's sampled term decomposition
// (sampled_plan.h, the same inline functions the kernels call) on seeded
// token-id arrays (flat, Zipf-like with one id taking a large share, all
// one id, ids out of range):
//   - the digit passes cover every key, and the counting sort's steps as
//     the kernels take them (per-block digit counts of kSortTile keys, a
//     digit-major exclusive scan, in-order placement per block) give the
//     stable sort (std::stable_sort by key) after every pass's composition;
//   - every token of a valid id lies in exactly one segment and, for runs
//     longer than one segment, every segment in exactly one group;
//   - segment and group slots of different runs never meet and stay below
//     n_run_slots.
// Usage: sampled_plan_check <seed> <n_cases>. Prints "ok <cases>" or the
// first violation and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "sampled_plan.h"

using namespace itl;

static uint64_t rng_state;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static long long uniform(long long lo, long long hi) { return lo + (long long)(next_u64() % (uint64_t)(hi - lo + 1)); }

struct Case {
  int vocab;
  std::vector<int32_t> y;
};

static Case draw(int kind) {
  Case c;
  const int vocabs[] = {1, 7, 255, 256, 257, 65535, 65536, 151936, 129280, 1 << 20};
  c.vocab = vocabs[uniform(0, 9)];
  const int n = (int)(kind == 4 ? uniform(0, 3) : uniform(1, 30000));
  c.y.resize(n);
  for (int i = 0; i < n; ++i) {
    switch (kind) {
      case 0: c.y[i] = (int32_t)uniform(0, c.vocab - 1); break;  // flat
      case 1: {                                                   // one id takes about 40 %, the rest Zipf-like
        const uint64_t r = next_u64() % 1000;
        c.y[i] = r < 400 ? (int32_t)(c.vocab / 3) : (int32_t)std::min<long long>(c.vocab - 1, (long long)(1.0 / (1e-4 + (double)(next_u64() % 10000) / 10000.0)));
        break;
      }
      case 2: c.y[i] = (int32_t)(c.vocab - 1); break;  // one id
      case 3: {                                        // some ids out of range
        const uint64_t r = next_u64() % 10;
        c.y[i] = r == 0 ? -(int32_t)uniform(1, 5) : (r == 1 ? c.vocab + (int32_t)uniform(0, 5) : (int32_t)uniform(0, c.vocab - 1));
        break;
      }
      default: c.y[i] = (int32_t)uniform(0, c.vocab - 1); break;
    }
  }
  return c;
}

// The counting sort as the kernels take it, on the host.
static void counting_sort(const Case& c, std::vector<uint32_t>& keys, std::vector<uint32_t>& vals) {
  const long long n = (long long)c.y.size();
  keys.resize(n);
  vals.resize(n);
  for (long long i = 0; i < n; ++i) {
    keys[i] = sort_key(c.y[i], c.vocab);
    vals[i] = (uint32_t)i;
  }
  const long long nb = sort_blocks(n);
  for (int p = 0; p < sort_passes(c.vocab); ++p) {
    const int shift = p * kSortDigitBits;
    std::vector<uint32_t> hist((size_t)kSortBins * nb, 0);
    for (long long i = 0; i < n; ++i) hist[((keys[i] >> shift) & (kSortBins - 1)) * nb + i / kSortTile]++;
    uint32_t run = 0;
    for (auto& h : hist) {
      const uint32_t x = h;
      h = run;
      run += x;
    }
    std::vector<uint32_t> ko(n), vo(n);
    for (long long i = 0; i < n; ++i) {  // in order within each block: the placement's rounds, waves and lanes
      const uint32_t dg = (keys[i] >> shift) & (kSortBins - 1);
      const uint32_t pos = hist[dg * nb + i / kSortTile]++;
      ko[pos] = keys[i];
      vo[pos] = vals[i];
    }
    keys.swap(ko);
    vals.swap(vo);
  }
}

static int check(const Case& c) {
  const long long n = (long long)c.y.size();
  const int passes = sort_passes(c.vocab);
  if (passes * kSortDigitBits < 32 && ((uint64_t)c.vocab >> (passes * kSortDigitBits)) != 0)
    return printf("passes %d do not cover key %d\n", passes, c.vocab), 1;
  std::vector<uint32_t> keys, vals;
  counting_sort(c, keys, vals);
  std::vector<uint32_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0u);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](uint32_t a, uint32_t b) { return sort_key(c.y[a], c.vocab) < sort_key(c.y[b], c.vocab); });
  for (long long i = 0; i < n; ++i)
    if (vals[i] != idx[i] || keys[i] != sort_key(c.y[idx[i]], c.vocab))
      return printf("sorted position %lld: token %u, the stable sort has %u\n", i, vals[i], idx[i]), 1;
  // runs, pieces and slots
  const long long seg_slots = n_run_slots(n, kRunSeg), grp_slots = n_run_slots(n, kRunGroupTokens);
  std::vector<int> seg_owner(seg_slots, -1), grp_owner(grp_slots, -1);
  std::vector<unsigned char> covered(n, 0);
  for (long long s = 0; s < n;) {
    long long e = s + 1;
    while (e < n && keys[e] == keys[s]) ++e;
    const long long L = e - s;
    if (keys[s] < (uint32_t)c.vocab) {
      if (L <= kRunSeg) {
        for (long long i = s; i < e; ++i) covered[i]++;
      } else {
        const long long nseg = n_pieces(L, kRunSeg);
        for (long long j = 0; j < nseg; ++j) {
          const long long slot = run_slot(s, j, kRunSeg);
          if (slot < 0 || slot >= seg_slots) return printf("segment slot %lld out of range\n", slot), 1;
          if (seg_owner[slot] != -1) return printf("segment slot %lld shared by runs at %d and %lld\n", slot, seg_owner[slot], s), 1;
          seg_owner[slot] = (int)s;
          const long long cnt = std::min<long long>(kRunSeg, L - j * kRunSeg);
          for (long long i = s + j * kRunSeg; i < s + j * kRunSeg + cnt; ++i) covered[i]++;
        }
        const long long ngrp = n_pieces(L, kRunGroupTokens);
        long long segs_in_groups = 0;
        for (long long g = 0; g < ngrp; ++g) {
          segs_in_groups += std::min<long long>(kRunGroup, nseg - g * kRunGroup);
          if (L > kRunGroupTokens) {
            const long long slot = run_slot(s, g, kRunGroupTokens);
            if (slot < 0 || slot >= grp_slots) return printf("group slot %lld out of range\n", slot), 1;
            if (grp_owner[slot] != -1) return printf("group slot %lld shared\n", slot), 1;
            grp_owner[slot] = (int)s;
          }
        }
        if (segs_in_groups != nseg) return printf("groups hold %lld of %lld segments\n", segs_in_groups, nseg), 1;
      }
    }
    s = e;
  }
  for (long long i = 0; i < n; ++i) {
    const bool valid = keys[i] < (uint32_t)c.vocab;
    if (covered[i] != (valid ? 1 : 0)) return printf("sorted position %lld covered %d times\n", i, covered[i]), 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  rng_state = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
  const int n = argc > 2 ? atoi(argv[2]) : 50;
  for (int k = 0; k < n; ++k)
    if (check(draw(k % 5))) return 1;
  printf("ok %d\n", n);
  return 0;
}
