// Host-side launchers of the library's kernels. Arguments are already
// validated by the C ABI layer (api.hip); these only size grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace itl {

// Workspace layout of the forward: per-(slice, token) partial (max, sumexp)
// pairs, then the per-token sampled logit.
size_t lmhead_workspace_bytes(long long n_tok, long long vocab);

// logits (nullable): also write z[t, v] at logits[t * ld + v] for v < vocab.
hipError_t launch_lmhead_logprob(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                 const int32_t* tokens, float* logprob, float* lse, float* logits, long long ld,
                                 void* workspace, hipStream_t stream);

// Merge each token's n_parts (max, sumexp) partials (slice-major) into its
// logprob (z_y - lse) and lse (nullable).
hipError_t launch_lse_combine(const float2* part, const float* zy, int n_tok, int n_parts, float* logprob, float* lse,
                              hipStream_t stream);

hipError_t launch_group_advantage(const float* rewards, const int32_t* group_offsets, int n_groups,
                                  int n_resp, float* advantages, hipStream_t stream);

// Workspace of the loss: the fp64 per-response losses, the fp64 segment sums
// of responses longer than one segment, and the fp64 partial sums of the mean.
size_t loss_workspace_bytes(long long n_tok, long long n_resp);

hipError_t launch_reinforce_zero_loss(const float* logprob, const float* rollout_logprob,
                                      const float* advantages, const int64_t* resp_offsets, int n_resp,
                                      long long n_tok, float* resp_loss, float* loss, float* coef,
                                      void* workspace, hipStream_t stream);

size_t backward_workspace_bytes(long long n_tok, long long d, long long vocab, int dtype);

// Tokens per chunk of the backward (a multiple of the token block). dW's sum
// over tokens is carried across chunks in this order, so it is part of dW's
// bits; the build info reports it.
constexpr int kBwdChunkTokens = 16384;

// Largest vocabulary the backward handles (its padded rows must be
// addressable by 32-bit buffer offsets over 256-row tiles).
constexpr long long kBwdMaxVocab = (1LL << 31) / (256LL * 4) - 256;

// The backward's sampled term: dW[v] = sum over tokens t with y_t = v of
// coef[t] H[t] for every row v (zeros where no token samples v), in the
// fixed order of sampled_plan.h.
size_t sampled_dw_workspace_bytes(long long n_tok, long long d, long long vocab);
hipError_t launch_sampled_dw(const void* H, int dtype, int n_tok, int d, int vocab, const int32_t* tokens,
                             const float* coef, float* dW, void* workspace, hipStream_t stream);

// logits (nullable): the forward's z[t, v] at logits[t * ld + v]; the dlogits
// are then formed from them instead of recomputing the contraction (same bits).
hipError_t launch_reinforce_zero_backward(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                          const int32_t* tokens, const float* lse, const float* coef,
                                          const float* logits, long long ld, float* dH, float* dW, void* workspace,
                                          hipStream_t stream);

hipError_t launch_quantize_rows_fp8(const void* X, int dtype, long long n_rows, int d, uint8_t* Xq, float* scale,
                                    hipStream_t stream);

hipError_t launch_lmhead_logprob_fp8(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq, const float* w_scale,
                                     int n_tok, int d, int vocab, const int32_t* tokens, float* logprob, float* lse,
                                     void* workspace, hipStream_t stream);

hipError_t launch_quantize_rows_mxfp4(const void* X, int dtype, long long n_rows, int d, uint8_t* Xq, uint8_t* sc,
                                      hipStream_t stream);

hipError_t launch_lmhead_logprob_mxfp4(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq4,
                                       const uint8_t* w_sc, int n_tok, int d, int vocab, const int32_t* tokens,
                                       float* logprob, float* lse, void* workspace, hipStream_t stream);

size_t mismatch_stats_workspace_bytes(long long n_tok);

hipError_t launch_mismatch_stats(const float* lp, const float* lpr, const float* lps, long long n, double* stats,
                                 void* workspace, hipStream_t stream);

// Device-side validation; writes a nonzero value to *flag on a violation.
hipError_t launch_check_inputs(const int32_t* tokens, long long n_tok, int vocab, const int64_t* resp_offsets,
                               int n_resp, int* flag, hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace itl
