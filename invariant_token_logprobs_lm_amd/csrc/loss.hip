// Group advantage and REINFORCE Zero loss ("vLLM says aligned kernels make
// asynchronous RL stable at lag 64", section "REINFORCE Zero removes the
// mismatch first"):
//
//   A_i          = r_i - mean of the rewards of i's group
//   ratio_t      = exp(logprob_t - rollout_logprob_t)      (no clipping)
//   resp_loss[i] = -A_i * (sum_{t in i} ratio_t) / T_i       (tokens averaged in a response)
//   loss         = (1/N) sum_i resp_loss[i]                  (then over responses)
//   coef[t]      = -ratio_t * A_i / (N * T_i)                (dloss/dlogprob_t, plain REINFORCE)
//
// Every sum runs over a segment-relative index with a tree fixed by the
// segment's length: a group's advantages and a response's loss are the same
// bits wherever the group or response sits in the batch. These kernels move
// a few bytes per token and are bound by HBM bandwidth (or launch latency at
// small sizes); lanes read consecutive elements.

#include <algorithm>

#include "device_common.h"
#include "itl_config.h"
#include "itl_launch.h"

namespace itl {

constexpr int kLongLossBlocks = 4096;    // workgroups of the long-response kernel (grid shape only)
constexpr int kShortLossBlocks = 16384;  // workgroups of the short-response kernel (grid shape only)

namespace {

// One wavefront per group (four per workgroup): lane j adds elements j,
// j+64, ... of the group in ascending order, then a fixed xor butterfly
// combines the lanes.
__global__ __launch_bounds__(256) void group_advantage_kernel(const float* __restrict__ rewards,
                                                              const int32_t* __restrict__ goff, int n_groups,
                                                              int n_resp, float* __restrict__ adv) {
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= n_groups) return;
  const int s = min(max(goff[g], 0), n_resp);
  const int e = min(max(goff[g + 1], s), n_resp);
  const int n = e - s;
  if (n <= 0) return;
  float acc = 0.0f;
  for (int i = s + lane; i < e; i += 64) acc += rewards[i];
  const float mean = wave_sum(acc) / (float)n;
  for (int i = s + lane; i < e; i += 64) adv[i] = rewards[i] - mean;
}

// Sum over a 256-thread block: wavefront butterflies, then the four wave
// sums in a fixed tree. Every thread gets the same bits.
__device__ __forceinline__ float block_sum256(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float ratio_of(float lp, float lpr) { return fast_exp2((lp - lpr) * kLog2e); }

// A response's tokens are summed by one of three fixed trees, chosen by its
// length alone (so the bits still depend on nothing but the response): up
// to kTinyResponse tokens, eight lanes (lane j holds token j; an xor
// butterfly over the eight); up to kShortResponse tokens, one wavefront
// (lane j adds tokens j, j+64, ... in ascending order, then the xor
// butterfly); longer ones, one 256-thread workgroup (thread j adds tokens j,
// j+256, ..., then the wavefront butterflies and the four wave sums in a
// fixed tree).
__device__ __forceinline__ void finish_response(int i, long long s, long long e, float S, const float* lp,
                                                const float* lpr, const float* adv, int n_resp, int tid, int stride,
                                                float* resp_loss, float* coef) {
  const long long T = e - s;
  if (T <= 0) return;
  const float A = adv[i];
  if (tid == 0) resp_loss[i] = -A * (S / (float)T);
  if (coef) {
    const float k = (float)(-(double)A / ((double)n_resp * (double)T));
    for (long long t = s + tid; t < e; t += stride) coef[t] = ratio_of(lp[t], lpr[t]) * k;
  }
}

// Tiny responses: eight per wavefront, eight lanes each.
__global__ __launch_bounds__(256) void response_loss_tiny_kernel(
    const float* __restrict__ lp, const float* __restrict__ lpr, const float* __restrict__ adv,
    const int64_t* __restrict__ off, int n_resp, long long n_tok, float* __restrict__ resp_loss,
    float* __restrict__ coef) {
  const int i = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int j = threadIdx.x & 7;
  long long s = 0, e = 0;
  if (i < n_resp) {
    s = min(max(off[i], 0LL), n_tok);
    e = min(max(off[i + 1], s), n_tok);
  }
  const long long T = e - s;
  const bool mine = T >= 1 && T <= kTinyResponse;
  const float r = mine && j < T ? ratio_of(lp[s + j], lpr[s + j]) : 0.0f;
  // every lane takes part in the shuffles; xor offsets below 8 stay in the
  // eight-lane segment
  float S = r;
  S += __shfl_xor(S, 4, 64);
  S += __shfl_xor(S, 2, 64);
  S += __shfl_xor(S, 1, 64);
  if (!mine) return;
  const float A = adv[i];
  if (j == 0) resp_loss[i] = -A * (S / (float)T);
  if (coef && j < T) coef[s + j] = r * (float)(-(double)A / ((double)n_resp * (double)T));
}

// Short responses: each wavefront owns a contiguous run of responses, reads
// their lengths 64 at a time and sums the short ones in order, one at a time.
__global__ __launch_bounds__(256) void response_loss_short_kernel(
    const float* __restrict__ lp, const float* __restrict__ lpr, const float* __restrict__ adv,
    const int64_t* __restrict__ off, int n_resp, long long n_tok, float* __restrict__ resp_loss,
    float* __restrict__ coef) {
  const int lane = threadIdx.x & 63;
  const int n_waves = (int)gridDim.x * 4;
  const int wv = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int per = (n_resp + n_waves - 1) / n_waves;
  const int r0 = min(wv * per, n_resp), r1 = min(r0 + per, n_resp);
  for (int c0 = r0; c0 < r1; c0 += 64) {
    bool mine = false;
    if (c0 + lane < r1) {
      const long long s = min(max(off[c0 + lane], 0LL), n_tok);
      const long long e = min(max(off[c0 + lane + 1], s), n_tok);
      mine = e - s > kTinyResponse && e - s <= kShortResponse;
    }
    uint64_t todo = __builtin_amdgcn_ballot_w64(mine);
    while (todo) {  // ascending response order
      const int k = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int i = c0 + k;
      const long long s = min(max(off[i], 0LL), n_tok);
      const long long e = min(max(off[i + 1], s), n_tok);
      float acc = 0.0f;
      for (long long t = s + lane; t < e; t += 64) acc += ratio_of(lp[t], lpr[t]);
      finish_response(i, s, e, wave_sum(acc), lp, lpr, adv, n_resp, lane, 64, resp_loss, coef);
    }
  }
}

// Long responses: one workgroup each. Workgroup b owns a contiguous run of
// responses (one response per workgroup up to kLongLossBlocks responses);
// its threads read the run's lengths 256 at a time and the workgroup then
// sums the long ones in order (the short kernel has the others).
__global__ __launch_bounds__(kLossThreads) void response_loss_long_kernel(
    const float* __restrict__ lp, const float* __restrict__ lpr, const float* __restrict__ adv,
    const int64_t* __restrict__ off, int n_resp, long long n_tok, float* __restrict__ resp_loss,
    float* __restrict__ coef) {
  __shared__ float red[4];
  __shared__ int is_long[kLossThreads];
  const int per = (n_resp + (int)gridDim.x - 1) / (int)gridDim.x;
  const int r0 = min((int)blockIdx.x * per, n_resp), r1 = min(r0 + per, n_resp);
  for (int c0 = r0; c0 < r1; c0 += kLossThreads) {
    const int i = c0 + (int)threadIdx.x;
    int lg = 0;
    if (i < r1) {
      const long long s = min(max(off[i], 0LL), n_tok);
      const long long e = min(max(off[i + 1], s), n_tok);
      lg = e - s > kShortResponse;
    }
    is_long[threadIdx.x] = lg;
    __syncthreads();
    const int m = min(kLossThreads, r1 - c0);
    for (int j = 0; j < m; ++j) {
      if (!is_long[j]) continue;  // the same value in every thread
      const int r = c0 + j;
      const long long s = min(max(off[r], 0LL), n_tok);
      const long long e = min(max(off[r + 1], s), n_tok);
      float acc = 0.0f;
      for (long long t = s + threadIdx.x; t < e; t += kLossThreads) acc += ratio_of(lp[t], lpr[t]);
      finish_response(r, s, e, block_sum256(acc, red), lp, lpr, adv, n_resp, threadIdx.x, kLossThreads, resp_loss,
                      coef);
    }
    __syncthreads();  // every thread is done with is_long before it is refilled
  }
}

// Single workgroup: mean of the per-response losses in a fixed order. The
// array is read as 16-byte groups of four, thread j taking groups j, j +
// kMeanThreads, ... (each pass of the workgroup reads one contiguous 16 KiB
// run) into four accumulators, one per position in the group, combined in a
// fixed order; the last n_resp mod 4 values go to thread 0's accumulators;
// then the wavefront butterflies and the wave sums in order. A fixed
// function of n_resp.
__global__ __launch_bounds__(kMeanThreads) void loss_mean_kernel(const float* __restrict__ resp_loss, int n_resp,
                                                                 float* __restrict__ loss) {
  __shared__ float red[kMeanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n4 = n_resp / 4;
  const bool vec = (reinterpret_cast<uintptr_t>(resp_loss) & 15) == 0;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  auto group = [&](int g) {
    return vec ? reinterpret_cast<const float4*>(resp_loss)[g]
               : make_float4(resp_loss[4 * g], resp_loss[4 * g + 1], resp_loss[4 * g + 2], resp_loss[4 * g + 3]);
  };
  auto add = [&](float4 v) {
    a0 += v.x;
    a1 += v.y;
    a2 += v.z;
    a3 += v.w;
  };
  int g = threadIdx.x;
  // Four groups loaded before any is added (the same additions in the same
  // order as one group at a time): four loads in flight per thread.
  for (; g + 3 * kMeanThreads < n4; g += 4 * kMeanThreads) {
    const float4 v0 = group(g), v1 = group(g + kMeanThreads), v2 = group(g + 2 * kMeanThreads),
                 v3 = group(g + 3 * kMeanThreads);
    add(v0);
    add(v1);
    add(v2);
    add(v3);
  }
  for (; g < n4; g += kMeanThreads) add(group(g));
  if (threadIdx.x == 0) {
    const int r = 4 * n4;
    if (r < n_resp) a0 += resp_loss[r];
    if (r + 1 < n_resp) a1 += resp_loss[r + 1];
    if (r + 2 < n_resp) a2 += resp_loss[r + 2];
  }
  float acc = (a0 + a1) + (a2 + a3);
  acc = wave_sum(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float total = 0.0f;
    for (int w = 0; w < kMeanThreads / 64; ++w) total += red[w];
    loss[0] = total / (float)n_resp;
  }
}

__global__ void check_tokens_kernel(const int32_t* __restrict__ tokens, long long n_tok, int vocab, int* flag) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t < n_tok) {
    const int y = tokens[t];
    if (y < 0 || y >= vocab) flag[0] = 1;
  }
}

__global__ void check_offsets_kernel(const int64_t* __restrict__ off, int n_resp, long long n_tok, int* flag) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0 && (off[0] != 0 || off[n_resp] != n_tok)) flag[0] = 2;
  if (i < n_resp && off[i + 1] <= off[i]) flag[0] = 2;
}

}  // namespace

hipError_t launch_group_advantage(const float* rewards, const int32_t* group_offsets, int n_groups, int n_resp,
                                  float* advantages, hipStream_t stream) {
  hipLaunchKernelGGL(group_advantage_kernel, dim3((unsigned)ceil_div(n_groups, 4)), dim3(256), 0, stream, rewards,
                     group_offsets, n_groups, n_resp, advantages);
  return hipGetLastError();
}

hipError_t launch_reinforce_zero_loss(const float* logprob, const float* rollout_logprob, const float* advantages,
                                      const int64_t* resp_offsets, int n_resp, long long n_tok, float* resp_loss,
                                      float* loss, float* coef, hipStream_t stream) {
  hipLaunchKernelGGL(response_loss_tiny_kernel, dim3((unsigned)ceil_div(n_resp, 32)), dim3(256), 0, stream, logprob,
                     rollout_logprob, advantages, resp_offsets, n_resp, n_tok, resp_loss, coef);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(response_loss_short_kernel, dim3((unsigned)std::min<long long>(ceil_div(n_resp, 4), kShortLossBlocks)),
                     dim3(256), 0, stream, logprob, rollout_logprob, advantages, resp_offsets, n_resp, n_tok, resp_loss,
                     coef);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(response_loss_long_kernel, dim3((unsigned)std::min(n_resp, kLongLossBlocks)), dim3(kLossThreads),
                     0, stream, logprob, rollout_logprob, advantages, resp_offsets, n_resp, n_tok, resp_loss, coef);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(kMeanThreads), 0, stream, resp_loss, n_resp, loss);
  return hipGetLastError();
}

hipError_t launch_check_inputs(const int32_t* tokens, long long n_tok, int vocab, const int64_t* resp_offsets,
                               int n_resp, int* flag, hipStream_t stream) {
  if (tokens && n_tok > 0) {
    hipLaunchKernelGGL(check_tokens_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, tokens,
                       n_tok, vocab, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (resp_offsets && n_resp > 0) {
    hipLaunchKernelGGL(check_offsets_kernel, dim3((unsigned)ceil_div(n_resp, 256)), dim3(256), 0, stream,
                       resp_offsets, n_resp, n_tok, flag);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace itl
