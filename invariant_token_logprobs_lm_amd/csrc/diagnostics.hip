// Train/inference mismatch diagnostics over sampled-token logprobs.
//
// "vLLM says aligned kernels make asynchronous RL stable at lag 64", section
// "Asynchronous training has two different gaps": the learner/rollout
// logprob gap splits into weight lag (different weights, same computation)
// and kernel mismatch (same weights and tokens, different engines), and the
// importance-weight deviation is judged by its peak over its median. The
// "vLLM Train-Inference Consistency Release Notes", section "The Technical
// Challenge: Train-Inference Mismatch", track the train-inference KL.
//
// Per token, in fp64 from the fp32 inputs (exact conversions):
//   delta = lp - lp_rollout, w = exp(delta), dev = |expm1(delta)| = |w - 1|
//   KL(rollout || learner) estimators k1 = -delta, k2 = delta^2 / 2,
//   k3 = expm1(delta) - delta (J. Schulman, "Approximating KL Divergence")
//   split: lag = lp - lp_same, kernel = lp_same - lp_rollout (lp_same = the
//   learner's computation at the rollout's weights), |.| and k3 of each, and
//   the count of tokens whose lp_same and lp_rollout differ in any bit.
//
// One HBM pass over the inputs, then an exact median by radix selection:
//   1. mismatch_clear: zeroes the prefix histogram and the selection state
//      (a kernel, not a memset, so the call can be captured in a graph).
//   2. mismatch_terms: 2048 tokens per workgroup; per-thread fp64 sums, maxima
//      and minima over 8 tokens, a fixed reduction per workgroup, one record
//      per workgroup; dev written out as its fp64 bit pattern (non-negative
//      doubles order like their bits as unsigned integers), and counted in a
//      histogram of its top 16 bits (per workgroup in LDS, then added to the
//      global one: integer counts, so the order of the additions is moot).
//   3. mismatch_select_prefix: one workgroup finds the 16-bit prefixes that
//      hold ranks (n - 1) / 2 and n / 2, and each rank within its prefix.
//   4. mismatch_gather: the keys with those prefixes are copied out (in any
//      order: only their values matter).
//   5. mismatch_select: one workgroup finds each rank's key among them, 8 bits
//      at a time (6 histogram passes over the low 48 bits).
//   6. mismatch_finalize: one workgroup folds the records in workgroup order
//      (fixed per n_tok, so the result is run-to-run deterministic) and
//      writes the statistics with the median of the two selected keys.

#include <math.h>

#include <algorithm>

#include "itl.h"
#include "itl_launch.h"

namespace itl {

namespace {

constexpr int kDiagThreads = 256;
constexpr int kDiagPerThread = 8;
constexpr int kDiagTokensPerBlock = kDiagThreads * kDiagPerThread;

// Fields of a workgroup record: sums first, then maxima, the minimum, the
// count (carried as a double: exact below 2^53).
enum Rec {
  kSumK1, kSumK2, kSumK3, kSumW, kSumLag, kSumLagK3, kSumKer, kSumKerK3,
  kMaxW, kMaxDev, kMaxLag, kMaxKer,
  kMinW,
  kCountKer,
  kRecFields
};
constexpr int kFirstMax = kMaxW, kFirstMin = kMinW, kFirstCount = kCountKer;

__device__ __forceinline__ double combine(int f, double a, double b) {
  if (f < kFirstMax || f >= kFirstCount) return a + b;
  if (f < kFirstMin) return fmax(a, b);
  return fmin(a, b);
}

__device__ __forceinline__ double identity(int f) {
  if (f < kFirstMax || f >= kFirstCount) return 0.0;
  if (f < kFirstMin) return -INFINITY;
  return INFINITY;
}

// Fixed-shape reduction of the workgroup's 256 values of field f: an xor
// butterfly within each wavefront (every lane ends with the same value:
// each step combines the same two operands on both partners, and the
// combines are commutative), then the 4 wavefront results in wavefront
// order. Every thread returns the result.
__device__ __forceinline__ double block_reduce(double* sh, int f, double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = combine(f, v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < kDiagThreads / 64; ++i) r = combine(f, r, sh[i]);
  __syncthreads();
  return r;
}

constexpr int kPrefixBits = 16;
constexpr int kPrefixBins = 1 << (kPrefixBits - 1);  // dev >= 0: the sign bit is 0
constexpr int kPrefixShift = 64 - kPrefixBits;
constexpr int kSelThreads = 1024;                    // the one-workgroup selection kernels
constexpr int kGatherBlocks = kSelThreads;           // candidate segments, one per selection thread
constexpr int kSelLdsKeys = 15 * 1024;               // candidates kept in LDS (120 KiB); more are re-read
static_assert(kPrefixBins % (4 * kSelThreads) == 0, "bins per thread");

// Selection state: the two target ranks' prefixes and ranks within them,
// then their keys.
struct SelectState {
  unsigned int rank_in[2];
  unsigned int prefix[2];
  unsigned long long key[2];
};

// Exclusive scan of one unsigned value per thread over groups of kGroup
// consecutive threads (a multiple of 64), with each group's total. Every
// thread of the workgroup must call it; wsum holds one entry per wavefront.
template <int kGroup>
__device__ __forceinline__ unsigned int group_excl_scan(unsigned int v, unsigned int* wsum, unsigned int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  constexpr int kWaves = kGroup / 64;
  const int g0 = (w / kWaves) * kWaves;
  unsigned int before = 0;
  total = 0;
  for (int i = 0; i < kWaves; ++i) {
    const unsigned int s = wsum[g0 + i];
    if (g0 + i < w) before += s;
    total += s;
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kDiagThreads) void mismatch_clear_kernel(unsigned int* __restrict__ hist,
                                                                      SelectState* __restrict__ st) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int i = blockIdx.x * kDiagThreads + threadIdx.x; i < kPrefixBins / 4; i += gridDim.x * kDiagThreads)
    h4[i] = uint4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x == 0) *st = SelectState{};
}

__global__ __launch_bounds__(kDiagThreads) void mismatch_terms_kernel(const float* __restrict__ lp,
                                                                      const float* __restrict__ lpr,
                                                                      const float* __restrict__ lps, long long n,
                                                                      unsigned long long* __restrict__ dev_bits,
                                                                      double* __restrict__ rec,
                                                                      unsigned int* __restrict__ hist) {
  __shared__ double sh[kDiagThreads];
  __shared__ __align__(16) unsigned int lh[kPrefixBins];
  __shared__ unsigned int pmin, pmax;  // the range of prefixes this workgroup saw
  {
    uint4* l4 = reinterpret_cast<uint4*>(lh);
    for (int i = threadIdx.x; i < kPrefixBins / 4; i += kDiagThreads) l4[i] = uint4{0u, 0u, 0u, 0u};
    if (threadIdx.x == 0) {
      pmin = kPrefixBins;
      pmax = 0u;
    }
  }
  __syncthreads();
  double acc[kRecFields];
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) acc[f] = identity(f);
  unsigned int my_min = kPrefixBins, my_max = 0u;
  const long long base = (long long)blockIdx.x * kDiagTokensPerBlock + threadIdx.x;
  for (int i = 0; i < kDiagPerThread; ++i) {
    const long long t = base + (long long)i * kDiagThreads;  // coalesced: consecutive threads, consecutive tokens
    if (t >= n) break;
    const float a = lp[t], r = lpr[t];
    const double d = (double)a - (double)r;
    const double em1 = expm1(d);
    const double w = exp(d);
    const double dev = fabs(em1);
    acc[kSumK1] += -d;
    acc[kSumK2] += d * d * 0.5;
    acc[kSumK3] += em1 - d;
    acc[kSumW] += w;
    acc[kMaxW] = fmax(acc[kMaxW], w);
    acc[kMinW] = fmin(acc[kMinW], w);
    acc[kMaxDev] = fmax(acc[kMaxDev], dev);
    const unsigned long long key = (unsigned long long)__double_as_longlong(dev);
    dev_bits[t] = key;
    const unsigned int p = (unsigned int)(key >> kPrefixShift);
    atomicAdd(&lh[p], 1u);
    my_min = min(my_min, p);
    my_max = max(my_max, p);
    if (lps) {
      const float s = lps[t];
      const double lag = (double)a - (double)s, ker = (double)s - (double)r;
      acc[kSumLag] += fabs(lag);
      acc[kSumLagK3] += expm1(lag) - lag;
      acc[kMaxLag] = fmax(acc[kMaxLag], fabs(lag));
      acc[kSumKer] += fabs(ker);
      acc[kSumKerK3] += expm1(ker) - ker;
      acc[kMaxKer] = fmax(acc[kMaxKer], fabs(ker));
      acc[kCountKer] += __float_as_uint(s) != __float_as_uint(r) ? 1.0 : 0.0;
    }
  }
  if (my_min <= my_max) {
    atomicMin(&pmin, my_min);
    atomicMax(&pmax, my_max);
  }
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) {
    const double r = block_reduce(sh, f, acc[f]);
    if (threadIdx.x == 0) rec[(size_t)blockIdx.x * kRecFields + f] = r;
  }
  // (block_reduce ends with a barrier: every LDS count and the range are in)
  for (unsigned int i = pmin + threadIdx.x; i <= pmax && i < (unsigned int)kPrefixBins; i += kDiagThreads)
    if (lh[i]) atomicAdd(&hist[i], lh[i]);
}

// Ranks (n - 1) / 2 and n / 2: the prefix that holds each and the rank
// within it, from the prefix histogram (each of 1024 threads owns 32
// consecutive bins; an exclusive scan of the per-thread sums).
__global__ __launch_bounds__(kSelThreads) void mismatch_select_prefix_kernel(const unsigned int* __restrict__ hist,
                                                                             long long n,
                                                                             SelectState* __restrict__ st) {
  constexpr int kPer = kPrefixBins / kSelThreads;  // 32
  // LDS copy with one pad word after every 32 bins, so that the 64 lanes
  // reading bin j of their own 32 hit different banks
  __shared__ unsigned int lh[kPrefixBins + kPrefixBins / kPer];
  __shared__ unsigned int wsum[kSelThreads / 64];
  const int t = threadIdx.x;
  auto at = [](int i) { return i + i / kPer; };
  {
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
#pragma unroll
    for (int i = t; i < kPrefixBins / 4; i += kSelThreads) {  // coalesced
      const uint4 v = h4[i];
      lh[at(4 * i)] = v.x;
      lh[at(4 * i + 1)] = v.y;
      lh[at(4 * i + 2)] = v.z;
      lh[at(4 * i + 3)] = v.w;
    }
  }
  __syncthreads();
  unsigned int sum = 0;
  for (int i = 0; i < kPer; ++i) sum += lh[at(t * kPer + i)];
  unsigned int total;
  unsigned int before = group_excl_scan<kSelThreads>(sum, wsum, total);
  const unsigned int rank[2] = {(unsigned int)((n - 1) / 2), (unsigned int)(n / 2)};
  for (int i = 0; i < kPer; ++i) {
    const unsigned int c = lh[at(t * kPer + i)];
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (rank[r] >= before && rank[r] < before + c) {
        st->prefix[r] = (unsigned int)(t * kPer + i);
        st->rank_in[r] = rank[r] - before;
      }
    before += c;
  }
}

// The keys with either target prefix, gathered per segment of cap
// consecutive tokens (segment b at cand[b cap ...], its count in counts[b];
// the order within a segment does not matter).
__global__ __launch_bounds__(kDiagThreads) void mismatch_gather_kernel(const unsigned long long* __restrict__ keys,
                                                                       long long n, long long cap,
                                                                       const SelectState* __restrict__ st,
                                                                       unsigned long long* __restrict__ cand,
                                                                       unsigned int* __restrict__ counts) {
  __shared__ unsigned int cnt;
  if (threadIdx.x == 0) cnt = 0u;
  __syncthreads();
  const unsigned int p0 = st->prefix[0], p1 = st->prefix[1];
  const long long t0 = (long long)blockIdx.x * cap;
  const long long t1 = min(n, t0 + cap);
  unsigned long long* seg = cand + t0;
  for (long long t = t0 + threadIdx.x; t < t1; t += kDiagThreads) {
    const unsigned long long k = keys[t];
    const unsigned int p = (unsigned int)(k >> kPrefixShift);
    if (p == p0 || p == p1) seg[atomicAdd(&cnt, 1u)] = k;
  }
  __syncthreads();
  if (threadIdx.x == 0) counts[blockIdx.x] = cnt;
}

// Each target: the key with the target's prefix whose rank among the keys
// with that prefix is rank_in, found 8 bits at a time from bit 47 down: a
// 256-bin histogram of the candidates that match the bits fixed so far picks
// the next byte (the bin holding the rank, by a scan over the 256 bins).
__global__ __launch_bounds__(kSelThreads) void mismatch_select_kernel(const unsigned long long* __restrict__ cand,
                                                                      const unsigned int* __restrict__ counts,
                                                                      long long cap,
                                                                      SelectState* __restrict__ st) {
  __shared__ unsigned long long lc[kSelLdsKeys];
  __shared__ unsigned int h[2][256];
  __shared__ unsigned int wsum[kSelThreads / 64];
  __shared__ unsigned long long fixed[2];
  __shared__ unsigned int want[2];
  const int t = threadIdx.x;
  // segment t (kGatherBlocks == kSelThreads)
  const unsigned int c = counts[t];
  const unsigned long long* seg = cand + (long long)t * cap;
  unsigned int m;
  const unsigned int off = group_excl_scan<kSelThreads>(c, wsum, m);
  const bool in_lds = m <= (unsigned int)kSelLdsKeys;
  if (in_lds) {
    // eight loads in flight per round trip
    for (unsigned int j0 = 0; j0 < c; j0 += 8) {
      unsigned long long v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = j0 + j < c ? seg[j0 + j] : 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < c) lc[off + j0 + j] = v[j];
    }
  }
  if (t < 2) {
    fixed[t] = (unsigned long long)st->prefix[t] << kPrefixShift;
    want[t] = st->rank_in[t];
  }
  for (int shift = kPrefixShift - 8; shift >= 0; shift -= 8) {
    if (t < 512) h[t >> 8][t & 255] = 0u;
    __syncthreads();
    const unsigned long long mask_hi = ~0ull << (shift + 8);  // the bits fixed so far
    const unsigned long long f0 = fixed[0], f1 = fixed[1];
    auto count = [&](unsigned long long k) {
      const unsigned int b = (unsigned int)((k >> shift) & 255u);
      if ((k & mask_hi) == f0) atomicAdd(&h[0][b], 1u);
      if ((k & mask_hi) == f1) atomicAdd(&h[1][b], 1u);
    };
    if (in_lds) {
      for (unsigned int i = t; i < m; i += kSelThreads) count(lc[i]);
    } else {
      for (unsigned int j = 0; j < c; ++j) count(seg[j]);
    }
    __syncthreads();
    // threads 256 r + b (r = 0, 1): bin b of target r
    const int r = (t >> 8) & 1;
    const unsigned int v = t < 512 ? h[r][t & 255] : 0u;
    const unsigned int w = want[r];
    unsigned int group_total;
    const unsigned int below = group_excl_scan<256>(v, wsum, group_total);
    if (t < 512 && w >= below && w < below + v) {
      fixed[r] |= (unsigned long long)(t & 255) << shift;
      want[r] = w - below;
    }
    __syncthreads();
  }
  if (t < 2) st->key[t] = fixed[t];
}

__device__ __forceinline__ double bits_to_double(unsigned long long b) { return __longlong_as_double((long long)b); }

__global__ __launch_bounds__(kDiagThreads) void mismatch_finalize_kernel(const double* __restrict__ rec, int n_blocks,
                                                                         const SelectState* __restrict__ sel,
                                                                         long long n, int has_split,
                                                                         double* __restrict__ stats) {
  __shared__ double sh[kDiagThreads];
  double acc[kRecFields];
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) acc[f] = identity(f);
  for (int b = threadIdx.x; b < n_blocks; b += kDiagThreads)
#pragma unroll
    for (int f = 0; f < kRecFields; ++f) acc[f] = combine(f, acc[f], rec[(size_t)b * kRecFields + f]);
  double tot[kRecFields];
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) tot[f] = block_reduce(sh, f, acc[f]);
  if (threadIdx.x != 0) return;
  const double nan = __longlong_as_double(0x7ff8000000000000LL);
  for (int i = 0; i < ITL_STAT_COUNT; ++i) stats[i] = nan;
  stats[ITL_STAT_N_TOK] = (double)n;
  if (n == 0) return;
  const double inv = 1.0 / (double)n;
  stats[ITL_STAT_KL_K1] = tot[kSumK1] * inv;
  stats[ITL_STAT_KL_K2] = tot[kSumK2] * inv;
  stats[ITL_STAT_KL_K3] = tot[kSumK3] * inv;
  stats[ITL_STAT_WEIGHT_MEAN] = tot[kSumW] * inv;
  stats[ITL_STAT_WEIGHT_MAX] = tot[kMaxW];
  stats[ITL_STAT_WEIGHT_MIN] = tot[kMinW];
  const double peak = tot[kMaxDev];
  const double med = (n & 1) ? bits_to_double(sel->key[1])
                             : (bits_to_double(sel->key[0]) + bits_to_double(sel->key[1])) * 0.5;
  stats[ITL_STAT_DEVIATION_MAX] = peak;
  stats[ITL_STAT_DEVIATION_MEDIAN] = med;
  stats[ITL_STAT_DEVIATION_PEAK_OVER_MEDIAN] = med > 0.0 ? peak / med : (peak == 0.0 ? 1.0 : INFINITY);
  if (has_split) {
    stats[ITL_STAT_LAG_ABS_MEAN] = tot[kSumLag] * inv;
    stats[ITL_STAT_LAG_ABS_MAX] = tot[kMaxLag];
    stats[ITL_STAT_LAG_KL_K3] = tot[kSumLagK3] * inv;
    stats[ITL_STAT_KERNEL_ABS_MEAN] = tot[kSumKer] * inv;
    stats[ITL_STAT_KERNEL_ABS_MAX] = tot[kMaxKer];
    stats[ITL_STAT_KERNEL_KL_K3] = tot[kSumKerK3] * inv;
    stats[ITL_STAT_KERNEL_NONZERO] = tot[kCountKer];
  }
}

// Workspace: dev bits, candidates, the workgroup records, the prefix
// histogram, the selection state.
struct DiagLayout {
  size_t keys, cand, counts, rec, hist, sel, total;
  long long cap;  // tokens per candidate segment
};

DiagLayout diag_layout(long long n) {
  DiagLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const long long nb = (n + kDiagTokensPerBlock - 1) / kDiagTokensPerBlock;
  L.cap = (n + kGatherBlocks - 1) / kGatherBlocks;
  L.keys = take((size_t)n * 8);
  L.cand = take((size_t)(L.cap * kGatherBlocks) * 8);
  L.counts = take((size_t)kGatherBlocks * 4);
  L.rec = take((size_t)nb * kRecFields * 8);
  L.hist = take((size_t)kPrefixBins * 4);
  L.sel = take(sizeof(SelectState));
  L.total = off;
  return L;
}

}  // namespace

size_t mismatch_stats_workspace_bytes(long long n_tok) { return diag_layout(n_tok).total; }

hipError_t launch_mismatch_stats(const float* lp, const float* lpr, const float* lps, long long n, double* stats,
                                 void* workspace, hipStream_t stream) {
  const DiagLayout L = diag_layout(n);
  char* ws = static_cast<char*>(workspace);
  auto* keys = reinterpret_cast<unsigned long long*>(ws + L.keys);
  auto* cand = reinterpret_cast<unsigned long long*>(ws + L.cand);
  auto* counts = reinterpret_cast<unsigned int*>(ws + L.counts);
  auto* rec = reinterpret_cast<double*>(ws + L.rec);
  auto* hist = reinterpret_cast<unsigned int*>(ws + L.hist);
  auto* sel = reinterpret_cast<SelectState*>(ws + L.sel);
  const int nb = (int)((n + kDiagTokensPerBlock - 1) / kDiagTokensPerBlock);
  if (n > 0) {
    hipLaunchKernelGGL(mismatch_clear_kernel, dim3(kPrefixBins / 4 / kDiagThreads), dim3(kDiagThreads), 0, stream,
                       hist, sel);
    hipLaunchKernelGGL(mismatch_terms_kernel, dim3((unsigned)nb), dim3(kDiagThreads), 0, stream, lp, lpr, lps, n,
                       keys, rec, hist);
    hipLaunchKernelGGL(mismatch_select_prefix_kernel, dim3(1), dim3(kSelThreads), 0, stream, hist, n, sel);
    hipLaunchKernelGGL(mismatch_gather_kernel, dim3(kGatherBlocks), dim3(kDiagThreads), 0, stream, keys, n, L.cap,
                       sel, cand, counts);
    hipLaunchKernelGGL(mismatch_select_kernel, dim3(1), dim3(kSelThreads), 0, stream, cand, counts, L.cap, sel);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mismatch_finalize_kernel, dim3(1), dim3(kDiagThreads), 0, stream, rec, nb, sel, n,
                     lps != nullptr ? 1 : 0, stats);
  return hipGetLastError();
}

}  // namespace itl
