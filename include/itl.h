/*
 * itl.h -- C ABI of the invariant token-logprob library (MI355X / gfx950).
 *
 * The library computes, on one GPU, each sampled token's log-probability
 * from final hidden states (an LM-head contraction, a log-softmax over the
 * vocabulary and a gather of the sampled token), the REINFORCE Zero loss on
 * top of it, and the loss's gradient with respect to the hidden states and
 * the head weights.
 *
 * Sources (web pages, cited by title and section):
 *  [RZ] "vLLM says aligned kernels make asynchronous RL stable at lag 64",
 *       section "REINFORCE Zero removes the mismatch first": the rollout
 *       records each sampled token's logprob; the learner divides its own
 *       probability by that record, at token level and without clipping;
 *       the advantage is the response's reward minus its group's mean
 *       reward; tokens are averaged within a response; plain REINFORCE.
 *  [BC] "vLLM Train-Inference Consistency Release Notes", section
 *       "Achieving Bitwise Consistency": kernel determinism, batch
 *       independence and prefill/decode phase consistency; section
 *       "Overview": bitwise-identical sampled-token logprobs (diff = 0)
 *       between rollout and training.
 *  [FP8] "vLLM says aligned kernels make asynchronous RL stable at lag 64",
 *       section "Zero mismatch expands to newer models": the consistent path
 *       of the newest model runs FP8 (and MXFP4) weights.
 *  [GAP] "vLLM says aligned kernels make asynchronous RL stable at lag 64",
 *       section "Asynchronous training has two different gaps": the
 *       learner/rollout logprob gap splits into weight lag and kernel
 *       mismatch; the importance-weight deviation is judged by its peak over
 *       its median. "vLLM Train-Inference Consistency Release Notes", section
 *       "The Technical Challenge: Train-Inference Mismatch": the
 *       train-inference KL divergence.
 *
 * Determinism contract [BC]. For one build of this library (see
 * itl_build_info) and one (vocab, d, dtype):
 *  - each token's logprob and lse are bitwise identical whatever n_tok,
 *    the token's row position, its batch-mates, the stream, or concurrent
 *    load. A decode step (n_tok = 1) and a prefill over many tokens give the
 *    same bits for the same hidden state: calls of at most 64 tokens run a
 *    narrow kernel that performs, per token, the same matrix-core
 *    instructions on the same operand fragments and the same fold sequence
 *    as the kernel for larger calls.
 *  - each resp_loss[i] is a bitwise function of response i's own
 *    (logprob, rollout_logprob, advantage, T_i) only;
 *  - loss, coef, advantages, dH and dW are run-to-run deterministic (no
 *    atomics, no split-K, fixed reduction orders).
 *
 * Conventions shared by every entry point.
 *  - All array pointers are DEVICE memory owned by the caller. The library
 *    never allocates, frees or synchronises (itl_check_inputs excepted).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *  - Layouts are dense row-major: H [n_tok, d], W [vocab, d] (the usual
 *    `lm_head.weight` layout), dH [n_tok, d], dW [vocab, d].
 *  - dtype selects the element type of H and W: ITL_BF16 (bfloat16 bits)
 *    or ITL_F32. Accumulation is always fp32. d must be a positive
 *    multiple of 64 (otherwise ITL_ERR_UNSUPPORTED); vocab is any value in
 *    [1, 2^31 - 256].
 *  - n_tok == 0 (or n_resp / n_groups == 0) is a no-op returning ITL_OK.
 *  - Host-detectable errors return before anything is launched.
 *    A failed launch returns ITL_ERR_HIP; itl_last_error() describes it.
 *  - Preconditions on device-resident values (0 <= tokens[t] < vocab,
 *    increasing offsets, no empty response or group) are NOT checked by
 *    the compute entry points; itl_check_inputs checks them on request.
 *    Violating them gives unspecified values, never an out-of-bounds
 *    access.
 *  - No C++ exception crosses this interface; nothing aborts.
 */
#ifndef ITL_H_
#define ITL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype codes are plain int32_t values (an enum would make an
 * unknown dtype code passed from C undefined behaviour in the C++ library;
 * as an int32_t it is a value like any other, answered with
 * ITL_ERR_UNSUPPORTED). */
typedef int32_t itl_status;
enum {
  ITL_OK = 0,
  ITL_ERR_INVALID_ARG = 1, /* null pointer, negative size, size overflow */
  ITL_ERR_UNSUPPORTED = 2, /* a shape or dtype this build does not handle */
  ITL_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  ITL_ERR_HIP = 4,         /* a HIP runtime call or launch failed */
  ITL_ERR_BAD_INPUT = 5    /* itl_check_inputs found an invalid value */
};

typedef int32_t itl_dtype;
enum { ITL_BF16 = 0, ITL_F32 = 1 };

/* Bytes of device workspace itl_lmhead_logprob needs for (n_tok, vocab):
 * about (16 S + 4) n_tok with S = min(ceil(vocab / 256), 256) vocabulary
 * slices (one fp32 (max, sum of exp) pair per token, slice and wavefront,
 * then the sampled logits). Returns 0 for n_tok == 0 and SIZE_MAX for
 * invalid sizes. */
size_t itl_lmhead_logprob_workspace_bytes(int64_t n_tok, int64_t vocab);

/* Sampled-token logprob [RZ][BC]:
 *   z[t, v]  = sum_k H[t, k] * W[v, k]           (fp32 accumulate, ascending k)
 *   lse[t]   = log sum_v exp(z[t, v])
 *   logprob[t] = z[t, tokens[t]] - lse[t]
 * H [n_tok, d], W [vocab, d] of `dtype`, both 16-byte aligned
 * (ITL_ERR_INVALID_ARG otherwise); tokens int32 [n_tok] with
 * 0 <= tokens[t] < vocab. Outputs fp32: logprob [n_tok]; lse [n_tok] may be
 * NULL. workspace: >= itl_lmhead_logprob_workspace_bytes(n_tok, vocab)
 * bytes, 256-byte aligned; its contents on entry do not matter.
 * The logits never leave the chip: the contraction is fused with an online
 * log-sum-exp over fixed vocabulary slices and the sampled-token gather.
 * Because the sampled logit and the normaliser come from the same fp32
 * accumulators, logprob <= 0 holds in fp32. */
itl_status itl_lmhead_logprob(const void* H, const void* W, itl_dtype dtype,
                              int64_t n_tok, int64_t d, int64_t vocab,
                              const int32_t* tokens, float* logprob, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* itl_lmhead_logprob for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. It takes no workspace: its scratch is a static 64 MiB device
 * array inside this library (one copy per GPU, held until the process ends;
 * its device address is looked up once per device on the first call). The
 * call itself allocates and frees nothing. Same arguments (minus the
 * workspace), same kernels, same logprob and lse bits as itl_lmhead_logprob.
 * Limit: itl_lmhead_logprob_workspace_bytes(n_tok, vocab) <= 64 MiB, i.e.
 * at most 16,368 tokens per call for vocab >= 65,281 (more for smaller
 * vocabularies); larger calls return ITL_ERR_UNSUPPORTED before anything is
 * launched. Every call on one GPU uses that GPU's one scratch array: calls
 * that may overlap on one GPU (different streams, different host threads
 * without ordering) race and give unspecified values; calls ordered on one
 * stream are safe. The scratch needs no clearing (every value read is
 * written earlier in the same call). */
itl_status itl_lmhead_logprob_noalloc(const void* H, const void* W, itl_dtype dtype,
                                      int64_t n_tok, int64_t d, int64_t vocab,
                                      const int32_t* tokens, float* logprob, float* lse, void* stream);

/* The same call as itl_lmhead_logprob, with the same logprob and lse bits,
 * that also keeps the head's logits for the backward [RZ] (the gradient of
 * the loss through the log-softmax needs every z[t, v] once more):
 *   logits[t * ld_logits + v] = z[t, v]     fp32, 0 <= t < n_tok, 0 <= v < vocab
 * the exact fp32 accumulator values the log-sum-exp folds. logits is a
 * caller-owned device buffer of n_tok * ld_logits floats, 16-byte aligned,
 * with ld_logits >= vocab and a multiple of 4 (else ITL_ERR_INVALID_ARG)
 * and at most 8,388,607 (else ITL_ERR_UNSUPPORTED); entries v >= vocab of a
 * row are left untouched. It is large (about
 * 4 n_tok vocab bytes: 159 GB for 308,010 tokens of a 129,280-row head), a
 * trade of HBM for the contraction itl_reinforce_zero_backward would
 * otherwise repeat; workspace as for itl_lmhead_logprob. */
itl_status itl_lmhead_logprob_keep_logits(const void* H, const void* W, itl_dtype dtype,
                                          int64_t n_tok, int64_t d, int64_t vocab,
                                          const int32_t* tokens, float* logprob, float* lse,
                                          float* logits, int64_t ld_logits,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Group-mean baseline [RZ]: advantages[i] = rewards[i] - mean of the
 * rewards of i's group. Group g owns responses group_offsets[g] ..
 * group_offsets[g+1]-1; group_offsets int32 [n_groups+1], starting at 0 and
 * ending at n_resp. rewards and advantages fp32 [n_resp] (device offsets
 * are clamped to [0, n_resp], so bad offsets cannot index out of bounds).
 * The fp32 summation tree depends only on the group's size (eight lanes for
 * groups of up to 8, a wavefront for larger ones, with the same bits where
 * both apply), so a group's advantages do not depend on where it sits in the
 * batch. */
itl_status itl_group_advantage(const float* rewards, const int32_t* group_offsets,
                               int32_t n_groups, int32_t n_resp, float* advantages, void* stream);

/* Bytes of device workspace itl_reinforce_zero_loss needs for (n_tok,
 * n_resp): about 8 n_resp + n_tok / 128 bytes (fp64 per-response losses,
 * fp64 sums of 2048-token segments of long responses, fp64 partial sums of
 * the mean), plus 24 bytes per 2048 tokens for more than 512 responses (the
 * response holding each 2048-token window's first token). Returns 0 for
 * n_resp == 0 and SIZE_MAX for invalid sizes. */
size_t itl_reinforce_zero_loss_workspace_bytes(int64_t n_tok, int32_t n_resp);

/* REINFORCE Zero loss [RZ]. Response i owns tokens resp_offsets[i] ..
 * resp_offsets[i+1]-1 (int64 [n_resp+1], starting at 0, ending at n_tok),
 * T_i of them. With ratio_t = exp(logprob[t] - rollout_logprob[t])
 * (unclipped, fp32):
 *   resp_loss[i] = -advantages[i] * (sum_{t in i} ratio_t) / T_i
 *   loss[0]      = (1/n_resp) * sum_i resp_loss[i]
 *   coef[t]      = dloss/dlogprob[t] = -ratio_t * advantages[i] / (n_resp * T_i)
 * Outputs fp32; coef may be NULL. resp_loss[i] excludes 1/n_resp, so it is
 * batch-invariant: its sum of ratios is accumulated in fp64 by a tree fixed
 * by T_i alone (2048-token segments counted from the response's first token,
 * each summed by a tree chosen by its length, added in order). loss[0] is
 * the mean of the fp64 per-response values (before their rounding to fp32)
 * by a fixed tree that depends only on n_resp (chunks of 1024 consecutive
 * responses, then the chunks in order): the mean of group-centred terms
 * nearly cancels, and this keeps its rounding error far below 1e-3 of itself
 * (about 1e-5 of it on the workloads tested). loss and
 * coef depend on n_resp by definition. workspace: >=
 * itl_reinforce_zero_loss_workspace_bytes(n_tok, n_resp) bytes, 256-byte
 * aligned; its contents on entry do not matter. */
itl_status itl_reinforce_zero_loss(const float* logprob, const float* rollout_logprob,
                                   const float* advantages, const int64_t* resp_offsets,
                                   int32_t n_resp, int64_t n_tok,
                                   float* resp_loss, float* loss, float* coef,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace itl_reinforce_zero_backward needs for (n_tok,
 * d, vocab, dtype). Returns SIZE_MAX for invalid sizes or dtype. */
size_t itl_reinforce_zero_backward_workspace_bytes(int64_t n_tok, int64_t d, int64_t vocab, itl_dtype dtype);

/* Gradient of the REINFORCE Zero loss through the head [RZ]:
 *   G[t, v] = coef[t] * (onehot(tokens[t])[v] - exp(z[t, v] - lse[t]))
 *   dH = G W   (fp32 [n_tok, d], overwritten)
 *   dW = G^T H (fp32 [vocab, d], overwritten; all zeros when n_tok == 0)
 * H, W, tokens as for itl_lmhead_logprob; lse and coef fp32 [n_tok] as
 * produced by itl_lmhead_logprob / itl_reinforce_zero_loss. The logits are
 * recomputed with the forward's contraction. The sampled-token entries
 * (+coef[t]) are applied exactly in fp32; the dense part -coef[t] p[t, v] is
 * rounded to the head's dtype before its contractions (for bf16 heads a
 * relative error of about 2^-9 per element). Every sum has a fixed order and
 * there are no atomics, so dH and dW are run-to-run deterministic; dW's sum
 * over tokens runs in ascending token order in chunks of a fixed size. A
 * row dH[t] involves token t alone and has the same bits whatever its
 * batch-mates and position (given the same lse[t] and coef[t]).
 * The sampled entries' sum into dW[v] is fixed by the tokens sampling v
 * alone: in ascending token order (a stable counting sort by id), in
 * segments of 64 tokens, groups of 64 segments, then the groups, each in
 * order, every product and sum rounded to fp32.
 * workspace: >= itl_reinforce_zero_backward_workspace_bytes(n_tok, d,
 * vocab, dtype) bytes, 256-byte aligned (it holds transposed copies of W
 * and of a chunk of H, two copies of the chunk's dense dlogits, the sorted
 * token ids and the sampled term's segment and group sums). H, W, dH and
 * dW must be 16-byte aligned (ITL_ERR_INVALID_ARG otherwise). vocab above
 * about 2.1e6 returns ITL_ERR_UNSUPPORTED.
 * Out-of-range token ids give unspecified values, never an out-of-bounds
 * access. */
itl_status itl_reinforce_zero_backward(const void* H, const void* W, itl_dtype dtype,
                                       int64_t n_tok, int64_t d, int64_t vocab,
                                       const int32_t* tokens, const float* lse, const float* coef,
                                       float* dH, float* dW,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* itl_reinforce_zero_backward with the dlogits formed from kept logits
 * (written by itl_lmhead_logprob_keep_logits for the same H, W, tokens)
 * instead of recomputing the contraction [RZ]: G, dH and dW have the same
 * bits as itl_reinforce_zero_backward's, since the kept values are the
 * recompute's values. logits / ld_logits as there (not read when n_tok is
 * 0); every other argument, the workspace size and the errors as for
 * itl_reinforce_zero_backward. */
itl_status itl_reinforce_zero_backward_from_logits(const void* H, const void* W, itl_dtype dtype,
                                                   int64_t n_tok, int64_t d, int64_t vocab,
                                                   const int32_t* tokens, const float* lse, const float* coef,
                                                   const float* logits, int64_t ld_logits,
                                                   float* dH, float* dW,
                                                   void* workspace, size_t workspace_bytes, void* stream);

/* Per-row FP8 quantisation [FP8] (OCP E4M3: bias 7, no infinities, largest
 * finite value 448). For each row r of X [n_rows, d] (dtype bf16 or fp32):
 *   scale[r] = amax_r / 448 in fp32 (correctly rounded; 1 for an all-zero row)
 *   Xq[r, k] = E4M3 code of X[r, k] / scale[r] (fp32 division, correctly
 *              rounded; round to nearest, ties to even; saturating at +-448)
 * so the codes and scales are a fixed function of the input bits (rows of W
 * are quantised once; rows of H, per call, are batch-independent). X must
 * be finite. Xq uint8 [n_rows, d] (4-byte aligned), scale fp32 [n_rows]. d
 * must be a multiple of 128 (ITL_ERR_UNSUPPORTED otherwise). */
itl_status itl_quantize_rows_fp8(const void* X, itl_dtype dtype, int64_t n_rows, int64_t d,
                                 uint8_t* Xq, float* scale, void* stream);

/* Sampled-token logprob from an FP8 head [FP8][RZ][BC]: Hq [n_tok, d] and Wq
 * [vocab, d] E4M3 codes with per-row scales h_scale [n_tok], w_scale [vocab]
 * (as written by itl_quantize_rows_fp8), on the FP8 matrix cores:
 *   z[t, v]    = (acc[t, v] * w_scale[v]) * h_scale[t],
 *   acc[t, v]  = sum_k e4m3(Hq[t, k]) e4m3(Wq[v, k])   (fp32, fixed K order)
 *   logprob[t] = z[t, tokens[t]] - log sum_v exp(z[t, v])
 * with the same fused log-sum-exp, vocabulary slices and combine as
 * itl_lmhead_logprob, and the same determinism contract (calls of at most
 * 128 tokens run a narrow kernel with the same per-token arithmetic). d must
 * be a multiple of 128; Hq, Wq 16-byte aligned.
 * workspace: >= itl_lmhead_logprob_workspace_bytes(n_tok, vocab) bytes,
 * 256-byte aligned. lse may be NULL. */
itl_status itl_lmhead_logprob_fp8(const uint8_t* Hq, const float* h_scale,
                                  const uint8_t* Wq, const float* w_scale,
                                  int64_t n_tok, int64_t d, int64_t vocab,
                                  const int32_t* tokens, float* logprob, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* MXFP4 quantisation [FP8] (OCP Microscaling: blocks of 32 consecutive
 * values of a row share an E8M0 power-of-two scale 2^e, e = floor(log2
 * amax) - 2 clamped to [-127, 127] (-127 for an all-zero block); elements are
 * E2M1 codes of x / 2^e, round to nearest even, saturating at +-6, two per
 * byte (even element in the low nibble)). X [n_rows, d] bf16 or fp32, d a
 * multiple of 128 (ITL_ERR_UNSUPPORTED otherwise); Xq uint8 [n_rows, d / 2]
 * (16-byte aligned); scale_codes uint8 [n_rows, d / 32] holding e + 127.
 * Codes and scales are a fixed function of the input bits. X must be
 * finite. */
itl_status itl_quantize_rows_mxfp4(const void* X, itl_dtype dtype, int64_t n_rows, int64_t d,
                                   uint8_t* Xq, uint8_t* scale_codes, void* stream);

/* Sampled-token logprob from an MXFP4 head [FP8][RZ][BC]: Wq4 / w_scale_codes
 * as written by itl_quantize_rows_mxfp4 (vocab rows), Hq / h_scale E4M3
 * token rows as written by itl_quantize_rows_fp8, on the FP4 x FP8 matrix
 * cores (v_mfma_scale_f32_32x32x64_f8f6f4 applies the W block scales):
 *   z[t, v] = acc[t, v] * h_scale[t],
 *   acc[t, v] = sum_k e2m1(W)[v, k] 2^(e[v, k / 32]) e4m3(Hq[t, k]) (fp32)
 * then as itl_lmhead_logprob_fp8 (same slices, fold, combine and
 * determinism; calls of at most 128 tokens run a narrow kernel with the same
 * per-token arithmetic). d a multiple of 128; Hq, Wq4 16-byte aligned; workspace >=
 * itl_lmhead_logprob_workspace_bytes(n_tok, vocab), 256-byte aligned. */
itl_status itl_lmhead_logprob_mxfp4(const uint8_t* Hq, const float* h_scale,
                                    const uint8_t* Wq4, const uint8_t* w_scale_codes,
                                    int64_t n_tok, int64_t d, int64_t vocab,
                                    const int32_t* tokens, float* logprob, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Statistics written by itl_mismatch_stats (fp64, indices into `stats`). */
typedef enum itl_stat {
  ITL_STAT_N_TOK = 0,
  ITL_STAT_KL_K1,                      /* mean of -delta                   */
  ITL_STAT_KL_K2,                      /* mean of delta^2 / 2              */
  ITL_STAT_KL_K3,                      /* mean of expm1(delta) - delta     */
  ITL_STAT_WEIGHT_MEAN,                /* mean of w = exp(delta)           */
  ITL_STAT_WEIGHT_MAX,
  ITL_STAT_WEIGHT_MIN,
  ITL_STAT_DEVIATION_MAX,              /* max of |w - 1|                   */
  ITL_STAT_DEVIATION_MEDIAN,           /* median of |w - 1|                */
  ITL_STAT_DEVIATION_PEAK_OVER_MEDIAN, /* max / median (1 if both 0, +inf if only the median is) */
  ITL_STAT_LAG_ABS_MEAN,               /* lag = logprob - same_weights     */
  ITL_STAT_LAG_ABS_MAX,
  ITL_STAT_LAG_KL_K3,
  ITL_STAT_KERNEL_ABS_MEAN,            /* kernel = same_weights - rollout  */
  ITL_STAT_KERNEL_ABS_MAX,
  ITL_STAT_KERNEL_KL_K3,
  ITL_STAT_KERNEL_NONZERO,             /* tokens whose two fp32 values differ in any bit */
  ITL_STAT_COUNT
} itl_stat;

/* Bytes of device workspace itl_mismatch_stats needs for n_tok tokens
 * (about 16 n_tok plus 140 KiB). SIZE_MAX for invalid sizes. */
size_t itl_mismatch_stats_workspace_bytes(int64_t n_tok);

/* Train/inference mismatch diagnostics of one batch of sampled tokens [GAP].
 * logprob: the learner's fp32 [n_tok]; rollout_logprob: the rollout's
 * record fp32 [n_tok]; same_weights_logprob (nullable): the learner's
 * computation at the rollout's weights, which splits the gap into weight lag
 * (logprob - same_weights) and kernel mismatch (same_weights - rollout). Per
 * token, in fp64 from the exact fp32 values: delta = logprob -
 * rollout_logprob, w = exp(delta); KL(rollout || learner) by the sample
 * estimators k1, k2, k3 of J. Schulman's "Approximating KL Divergence"
 * (tokens are drawn from the rollout policy). The median is exact (radix
 * selection of the middle value(s) of |w - 1| by their fp64 bits; the mean
 * of the two middle values for even n_tok).
 * stats: DEVICE fp64 [ITL_STAT_COUNT], written on `stream`; the split
 * fields are NaN without same_weights_logprob, every field but N_TOK is
 * NaN when n_tok == 0. Run-to-run deterministic (fixed reduction order for
 * a given n_tok; the selection's integer counts do not depend on the order
 * their atomic additions land in). workspace: >= itl_mismatch_stats_workspace_bytes(n_tok)
 * bytes, 256-byte aligned. n_tok above 2^31 - 1 returns
 * ITL_ERR_UNSUPPORTED. */
itl_status itl_mismatch_stats(const float* logprob, const float* rollout_logprob,
                              const float* same_weights_logprob, int64_t n_tok, double* stats,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Opt-in validation of device-resident inputs (synchronises `stream`):
 * 0 <= tokens[t] < vocab for all t (tokens may be NULL to skip), and, when
 * resp_offsets is not NULL, resp_offsets[0] == 0, resp_offsets[n_resp] ==
 * n_tok and T_i >= 1. Returns ITL_OK or ITL_ERR_BAD_INPUT. */
itl_status itl_check_inputs(const int32_t* tokens, int64_t n_tok, int64_t vocab,
                            const int64_t* resp_offsets, int32_t n_resp, void* stream);

/* Static description of a status code. */
const char* itl_status_string(itl_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char* itl_last_error(void);

/* Compile-time tile, slice and chunk constants and the target arch, so a
 * rollout process and a learner process can assert they run the same
 * arithmetic. */
const char* itl_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* ITL_H_ */
