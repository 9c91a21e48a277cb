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
// Three launches, one HBM pass over the inputs:
//   1. mismatch_terms: 2048 tokens per workgroup; per-thread fp64 sums, maxima
//      and minima over 8 tokens, a fixed LDS tree per workgroup, one record
//      per workgroup; dev written out as its fp64 bit pattern (non-negative
//      doubles order like their bits as unsigned integers).
//   2. hipCUB radix sort of the dev bits (for the exact median).
//   3. mismatch_finalize: one workgroup folds the records in workgroup order
//      (fixed per n_tok, so the result is run-to-run deterministic) and
//      writes the statistics.

#include <math.h>

#include <algorithm>

#include <hipcub/hipcub.hpp>

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

// Fixed-shape tree over the workgroup's 256 values of field f (stride
// halving); thread 0 returns the result.
__device__ __forceinline__ double block_reduce(double* sh, int f, double v) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int s = kDiagThreads / 2; s > 0; s >>= 1) {
    if (t < s) sh[t] = combine(f, sh[t], sh[t + s]);
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kDiagThreads) void mismatch_terms_kernel(const float* __restrict__ lp,
                                                                      const float* __restrict__ lpr,
                                                                      const float* __restrict__ lps, long long n,
                                                                      unsigned long long* __restrict__ dev_bits,
                                                                      double* __restrict__ rec) {
  __shared__ double sh[kDiagThreads];
  double acc[kRecFields];
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) acc[f] = identity(f);
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
    dev_bits[t] = (unsigned long long)__double_as_longlong(dev);
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
#pragma unroll
  for (int f = 0; f < kRecFields; ++f) {
    const double r = block_reduce(sh, f, acc[f]);
    if (threadIdx.x == 0) rec[(size_t)blockIdx.x * kRecFields + f] = r;
  }
}

__device__ __forceinline__ double bits_to_double(unsigned long long b) { return __longlong_as_double((long long)b); }

__global__ __launch_bounds__(kDiagThreads) void mismatch_finalize_kernel(const double* __restrict__ rec, int n_blocks,
                                                                         const unsigned long long* __restrict__ sorted,
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
  const double med = (n & 1) ? bits_to_double(sorted[n / 2])
                             : (bits_to_double(sorted[n / 2 - 1]) + bits_to_double(sorted[n / 2])) * 0.5;
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

// Workspace: dev bits, sorted dev bits, the workgroup records, sort scratch.
struct DiagLayout {
  size_t keys, sorted, rec, tmp, tmp_bytes, total;
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
  L.keys = take((size_t)n * 8);
  L.sorted = take((size_t)n * 8);
  L.rec = take((size_t)nb * kRecFields * 8);
  size_t tmp = 0;
  // A size query (null temp storage): computes `tmp`, launches nothing.
  (void)hipcub::DeviceRadixSort::SortKeys(nullptr, tmp, (const unsigned long long*)nullptr,
                                          (unsigned long long*)nullptr, (int)std::max<long long>(n, 1), 0, 64,
                                          nullptr);
  L.tmp = take(tmp);
  L.tmp_bytes = tmp;
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
  auto* sorted = reinterpret_cast<unsigned long long*>(ws + L.sorted);
  auto* rec = reinterpret_cast<double*>(ws + L.rec);
  const int nb = (int)((n + kDiagTokensPerBlock - 1) / kDiagTokensPerBlock);
  if (n > 0) {
    hipLaunchKernelGGL(mismatch_terms_kernel, dim3((unsigned)nb), dim3(kDiagThreads), 0, stream, lp, lpr, lps, n,
                       keys, rec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    size_t tmp = L.tmp_bytes;
    e = hipcub::DeviceRadixSort::SortKeys(ws + L.tmp, tmp, keys, sorted, (int)n, 0, 64, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mismatch_finalize_kernel, dim3(1), dim3(kDiagThreads), 0, stream, rec, nb, sorted, n,
                     lps != nullptr ? 1 : 0, stats);
  return hipGetLastError();
}

}  // namespace itl
