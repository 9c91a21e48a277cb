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

#include "device_common.h"
#include "itl_config.h"
#include "itl_launch.h"

namespace itl {

namespace {

// One wavefront per group: lane j adds elements j, j+64, ... of the group in
// ascending order, then a fixed xor butterfly combines the lanes.
__global__ __launch_bounds__(64) void group_advantage_kernel(const float* __restrict__ rewards,
                                                             const int32_t* __restrict__ goff, int n_resp,
                                                             float* __restrict__ adv) {
  const int g = blockIdx.x;
  const int lane = threadIdx.x;
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

// One workgroup per response: thread j handles tokens j, j+256, ... of the
// response in ascending order.
__global__ __launch_bounds__(kLossThreads) void response_loss_kernel(
    const float* __restrict__ lp, const float* __restrict__ lpr, const float* __restrict__ adv,
    const int64_t* __restrict__ off, int n_resp, long long n_tok, float* __restrict__ resp_loss,
    float* __restrict__ coef) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const long long s = min(max(off[i], 0LL), n_tok);
  const long long e = min(max(off[i + 1], s), n_tok);
  const long long T = e - s;
  float acc = 0.0f;
  for (long long t = s + threadIdx.x; t < e; t += kLossThreads) acc += ratio_of(lp[t], lpr[t]);
  const float S = block_sum256(acc, red);
  if (T <= 0) return;
  const float A = adv[i];
  if (threadIdx.x == 0) resp_loss[i] = -A * (S / (float)T);
  if (coef) {
    const float k = (float)(-(double)A / ((double)n_resp * (double)T));
    for (long long t = s + threadIdx.x; t < e; t += kLossThreads) coef[t] = ratio_of(lp[t], lpr[t]) * k;
  }
}

// Single workgroup: mean of the per-response losses in a fixed order.
__global__ __launch_bounds__(kMeanThreads) void loss_mean_kernel(const float* __restrict__ resp_loss, int n_resp,
                                                                 float* __restrict__ loss) {
  __shared__ float red[kMeanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc = 0.0f;
  for (int i = threadIdx.x; i < n_resp; i += kMeanThreads) acc += resp_loss[i];
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
  hipLaunchKernelGGL(group_advantage_kernel, dim3(n_groups), dim3(64), 0, stream, rewards, group_offsets, n_resp,
                     advantages);
  return hipGetLastError();
}

hipError_t launch_reinforce_zero_loss(const float* logprob, const float* rollout_logprob, const float* advantages,
                                      const int64_t* resp_offsets, int n_resp, long long n_tok, float* resp_loss,
                                      float* loss, float* coef, hipStream_t stream) {
  hipLaunchKernelGGL(response_loss_kernel, dim3(n_resp), dim3(kLossThreads), 0, stream, logprob, rollout_logprob,
                     advantages, resp_offsets, n_resp, n_tok, resp_loss, coef);
  hipError_t e = hipGetLastError();
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
