// C ABI of the library (declared in include/itl.h): argument validation,
// workspace sizing, status codes. Every host-detectable error returns before
// anything is enqueued; nothing here allocates, frees or synchronises except
// itl_check_inputs.

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "itl.h"
#include "itl_config.h"
#include "itl_launch.h"
#include "sampled_plan.h"

namespace {

thread_local std::string g_last_error;

itl_status fail(itl_status s, const char* what) {
  g_last_error = what;
  return s;
}

itl_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return ITL_ERR_HIP;
}

constexpr int64_t kMaxTok = (int64_t)INT32_MAX - itl::kBT;
constexpr int64_t kMaxVocab = (int64_t)INT32_MAX - itl::kBV;
constexpr int64_t kFp8DMultiple = 128;  // one 128-byte K step = 128 E4M3 values
// the loss's token pass has one workgroup per 2048-token window
constexpr int64_t kMaxLossTok = (int64_t)INT32_MAX * itl::kSegTokens;

int elem_size(itl_dtype dt) { return dt == ITL_BF16 ? 2 : 4; }

// Shared shape checks of the head entry points.
itl_status check_head(itl_dtype dtype, int64_t n_tok, int64_t d, int64_t vocab) {
  if (n_tok < 0 || d <= 0 || vocab <= 0) return fail(ITL_ERR_INVALID_ARG, "n_tok must be >= 0, d and vocab > 0");
  if (dtype != ITL_BF16 && dtype != ITL_F32) return fail(ITL_ERR_UNSUPPORTED, "dtype must be ITL_BF16 or ITL_F32");
  if (d % itl::kDMultiple != 0) return fail(ITL_ERR_UNSUPPORTED, "d must be a multiple of 64");
  if (n_tok > kMaxTok) return fail(ITL_ERR_UNSUPPORTED, "n_tok too large for one call");
  if (vocab > kMaxVocab) return fail(ITL_ERR_UNSUPPORTED, "vocab too large");
  // a 256-row operand block must be addressable with 32-bit buffer offsets
  if (d >= ((int64_t)1 << 31) / (elem_size(dtype) * (int64_t)itl::kBT)) return fail(ITL_ERR_UNSUPPORTED, "d too large");
  const int64_t grid = itl::ceil_div(n_tok, itl::kBT) * itl::n_slice_groups(n_tok, vocab);
  if (grid > INT32_MAX) return fail(ITL_ERR_UNSUPPORTED, "problem too large for one launch");
  return ITL_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) != 0; }

// The head kernels move H and W rows in 16-byte pieces per lane.
bool misaligned16(const void* a, const void* b) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15) != 0;
}

// Scratch of itl_lmhead_logprob_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. Host code never uses its name
// as an address: the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

__device__ __align__(256) unsigned char itl_noalloc_scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on the device `stream` belongs to (the
// current device for the null stream).
itl_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "itl_lmhead_logprob_noalloc: device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(ITL_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "itl_lmhead_logprob_noalloc: current device");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "itl_lmhead_logprob_noalloc: set device");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(itl_noalloc_scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "itl_lmhead_logprob_noalloc: scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ITL_OK;
}

}  // namespace

extern "C" {

size_t itl_lmhead_logprob_workspace_bytes(int64_t n_tok, int64_t vocab) {
  if (n_tok < 0 || vocab <= 0 || n_tok > kMaxTok || vocab > kMaxVocab) return SIZE_MAX;
  return itl::lmhead_workspace_bytes(n_tok, vocab);
}

itl_status itl_lmhead_logprob(const void* H, const void* W, itl_dtype dtype, int64_t n_tok, int64_t d, int64_t vocab,
                              const int32_t* tokens, float* logprob, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  itl_status st = check_head(dtype, n_tok, d, vocab);
  if (st != ITL_OK) return st;
  if (n_tok == 0) return ITL_OK;
  if (!H || !W || !tokens || !logprob) return fail(ITL_ERR_INVALID_ARG, "null H, W, tokens or logprob");
  if (misaligned16(H, W)) return fail(ITL_ERR_INVALID_ARG, "H and W must be 16-byte aligned");
  if (!workspace || workspace_bytes < itl::lmhead_workspace_bytes(n_tok, vocab))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_lmhead_logprob_workspace_bytes()");
  if (misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_lmhead_logprob(H, W, (int)dtype, (int)n_tok, (int)d, (int)vocab, tokens, logprob, lse,
                                            nullptr, 0, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_lmhead_logprob");
}

itl_status itl_lmhead_logprob_noalloc(const void* H, const void* W, itl_dtype dtype, int64_t n_tok, int64_t d,
                                      int64_t vocab, const int32_t* tokens, float* logprob, float* lse, void* stream) {
  g_last_error.clear();
  itl_status st = check_head(dtype, n_tok, d, vocab);
  if (st != ITL_OK) return st;
  if (n_tok == 0) return ITL_OK;
  if (!H || !W || !tokens || !logprob) return fail(ITL_ERR_INVALID_ARG, "null H, W, tokens or logprob");
  if (misaligned16(H, W)) return fail(ITL_ERR_INVALID_ARG, "H and W must be 16-byte aligned");
  if (itl::lmhead_workspace_bytes(n_tok, vocab) > kNoAllocScratchBytes)
    return fail(ITL_ERR_UNSUPPORTED,
                "n_tok too large for itl_lmhead_logprob_noalloc's 64 MiB scratch (at most 16,368 tokens for "
                "vocab >= 65,281; use itl_lmhead_logprob with a workspace)");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  st = noalloc_scratch(s, &scratch);
  if (st != ITL_OK) return st;
  hipError_t e = itl::launch_lmhead_logprob(H, W, (int)dtype, (int)n_tok, (int)d, (int)vocab, tokens, logprob, lse,
                                            nullptr, 0, scratch, s);
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_lmhead_logprob_noalloc");
}

namespace {

// The kept-logits buffer: [n_tok, ld] fp32, ld >= vocab and a multiple of 4,
// 16-byte aligned, every offset t * ld + v addressable.
itl_status check_logits(const float* logits, int64_t ld, int64_t n_tok, int64_t vocab) {
  if (!logits) return fail(ITL_ERR_INVALID_ARG, "null logits");
  if (ld < vocab || ld % 4 != 0) return fail(ITL_ERR_INVALID_ARG, "ld_logits must be >= vocab and a multiple of 4");
  // 128 token rows of the buffer must be addressable with 32-bit offsets
  if (ld > (int64_t)(UINT32_MAX / (4u * 128u))) return fail(ITL_ERR_UNSUPPORTED, "ld_logits too large");
  if ((reinterpret_cast<uintptr_t>(logits) & 15) != 0) return fail(ITL_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  if (n_tok > 0 && ld > (INT64_MAX / 8) / n_tok) return fail(ITL_ERR_INVALID_ARG, "n_tok * ld_logits overflows");
  return ITL_OK;
}

}  // namespace

itl_status itl_lmhead_logprob_keep_logits(const void* H, const void* W, itl_dtype dtype, int64_t n_tok, int64_t d,
                                          int64_t vocab, const int32_t* tokens, float* logprob, float* lse,
                                          float* logits, int64_t ld_logits, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  g_last_error.clear();
  itl_status st = check_head(dtype, n_tok, d, vocab);
  if (st != ITL_OK) return st;
  if (n_tok == 0) return ITL_OK;
  if (!H || !W || !tokens || !logprob) return fail(ITL_ERR_INVALID_ARG, "null H, W, tokens or logprob");
  if (misaligned16(H, W)) return fail(ITL_ERR_INVALID_ARG, "H and W must be 16-byte aligned");
  st = check_logits(logits, ld_logits, n_tok, vocab);
  if (st != ITL_OK) return st;
  if (!workspace || workspace_bytes < itl::lmhead_workspace_bytes(n_tok, vocab))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_lmhead_logprob_workspace_bytes()");
  if (misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_lmhead_logprob(H, W, (int)dtype, (int)n_tok, (int)d, (int)vocab, tokens, logprob, lse,
                                            logits, (long long)ld_logits, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_lmhead_logprob_keep_logits");
}

itl_status itl_group_advantage(const float* rewards, const int32_t* group_offsets, int32_t n_groups, int32_t n_resp,
                               float* advantages, void* stream) {
  g_last_error.clear();
  if (n_groups < 0 || n_resp < 0) return fail(ITL_ERR_INVALID_ARG, "n_groups and n_resp must be >= 0");
  if (n_groups == 0 || n_resp == 0) return ITL_OK;
  if (!rewards || !group_offsets || !advantages) return fail(ITL_ERR_INVALID_ARG, "null rewards, offsets or output");
  hipError_t e = itl::launch_group_advantage(rewards, group_offsets, n_groups, n_resp, advantages,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_group_advantage");
}

size_t itl_reinforce_zero_loss_workspace_bytes(int64_t n_tok, int32_t n_resp) {
  if (n_tok < 0 || n_resp < 0 || n_tok > kMaxLossTok) return SIZE_MAX;
  return itl::loss_workspace_bytes(n_tok, n_resp);
}

itl_status itl_reinforce_zero_loss(const float* logprob, const float* rollout_logprob, const float* advantages,
                                   const int64_t* resp_offsets, int32_t n_resp, int64_t n_tok, float* resp_loss,
                                   float* loss, float* coef, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (n_resp < 0 || n_tok < 0) return fail(ITL_ERR_INVALID_ARG, "n_resp and n_tok must be >= 0");
  if (n_tok > kMaxLossTok) return fail(ITL_ERR_UNSUPPORTED, "n_tok too large for one call");
  if (n_resp == 0) return ITL_OK;
  if (!resp_offsets || !advantages || !resp_loss || !loss)
    return fail(ITL_ERR_INVALID_ARG, "null offsets, advantages or outputs");
  if (n_tok > 0 && (!logprob || !rollout_logprob)) return fail(ITL_ERR_INVALID_ARG, "null logprob arrays");
  if (!workspace || workspace_bytes < itl::loss_workspace_bytes(n_tok, n_resp))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_reinforce_zero_loss_workspace_bytes()");
  if (misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_reinforce_zero_loss(logprob, rollout_logprob, advantages, resp_offsets, n_resp, n_tok,
                                                 resp_loss, loss, coef, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_reinforce_zero_loss");
}

size_t itl_reinforce_zero_backward_workspace_bytes(int64_t n_tok, int64_t d, int64_t vocab, itl_dtype dtype) {
  if (n_tok < 0 || d <= 0 || vocab <= 0 || n_tok > kMaxTok || vocab > kMaxVocab) return SIZE_MAX;
  if (dtype != ITL_BF16 && dtype != ITL_F32) return SIZE_MAX;
  // shapes the backward refuses get no size either (and no wrapped product)
  if (d % itl::kDMultiple != 0 || d >= ((int64_t)1 << 31) / (elem_size(dtype) * (int64_t)itl::kBT)) return SIZE_MAX;
  return itl::backward_workspace_bytes(n_tok, d, vocab, (int)dtype);
}

namespace {

itl_status backward(const void* H, const void* W, itl_dtype dtype, int64_t n_tok, int64_t d, int64_t vocab,
                    const int32_t* tokens, const float* lse, const float* coef, const float* logits, int64_t ld,
                    float* dH, float* dW, void* workspace, size_t workspace_bytes, void* stream, const char* name) {
  itl_status st = check_head(dtype, n_tok, d, vocab);
  if (st != ITL_OK) return st;
  if (!W || !dW) return fail(ITL_ERR_INVALID_ARG, "null W or dW");
  if (n_tok > 0 && (!H || !tokens || !lse || !coef || !dH))
    return fail(ITL_ERR_INVALID_ARG, "null H, tokens, lse, coef or dH");
  if (vocab > itl::kBwdMaxVocab) return fail(ITL_ERR_UNSUPPORTED, "vocab too large for the backward");
  if (((reinterpret_cast<uintptr_t>(H) | reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(dH) |
        reinterpret_cast<uintptr_t>(dW)) & 15) != 0)
    return fail(ITL_ERR_INVALID_ARG, "H, W, dH and dW must be 16-byte aligned");
  const size_t need = itl::backward_workspace_bytes(n_tok, d, vocab, (int)dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_reinforce_zero_backward_workspace_bytes()");
  if (need > 0 && misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_reinforce_zero_backward(H, W, (int)dtype, (int)n_tok, (int)d, (int)vocab, tokens, lse,
                                                     coef, logits, (long long)ld, dH, dW, workspace,
                                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, name);
}

}  // namespace

itl_status itl_reinforce_zero_backward_from_logits(const void* H, const void* W, itl_dtype dtype, int64_t n_tok,
                                                   int64_t d, int64_t vocab, const int32_t* tokens, const float* lse,
                                                   const float* coef, const float* logits, int64_t ld_logits,
                                                   float* dH, float* dW, void* workspace, size_t workspace_bytes,
                                                   void* stream) {
  g_last_error.clear();
  if (n_tok > 0) {
    itl_status st = check_logits(logits, ld_logits, n_tok, vocab);
    if (st != ITL_OK) return st;
  }
  return backward(H, W, dtype, n_tok, d, vocab, tokens, lse, coef, n_tok > 0 ? logits : nullptr, ld_logits, dH, dW,
                  workspace, workspace_bytes, stream, "itl_reinforce_zero_backward_from_logits");
}

itl_status itl_reinforce_zero_backward(const void* H, const void* W, itl_dtype dtype, int64_t n_tok, int64_t d,
                                       int64_t vocab, const int32_t* tokens, const float* lse, const float* coef,
                                       float* dH, float* dW, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return backward(H, W, dtype, n_tok, d, vocab, tokens, lse, coef, nullptr, 0, dH, dW, workspace, workspace_bytes,
                  stream, "itl_reinforce_zero_backward");
}

itl_status itl_quantize_rows_fp8(const void* X, itl_dtype dtype, int64_t n_rows, int64_t d, uint8_t* Xq, float* scale,
                                 void* stream) {
  g_last_error.clear();
  if (n_rows < 0 || d <= 0) return fail(ITL_ERR_INVALID_ARG, "n_rows must be >= 0 and d > 0");
  if (dtype != ITL_BF16 && dtype != ITL_F32) return fail(ITL_ERR_UNSUPPORTED, "dtype must be ITL_BF16 or ITL_F32");
  if (d % kFp8DMultiple != 0) return fail(ITL_ERR_UNSUPPORTED, "d must be a multiple of 128");
  if (n_rows > (int64_t)INT32_MAX * 4 || d > INT32_MAX) return fail(ITL_ERR_UNSUPPORTED, "too many rows or columns");
  if (n_rows == 0) return ITL_OK;
  if (!X || !Xq || !scale) return fail(ITL_ERR_INVALID_ARG, "null X, Xq or scale");
  if ((reinterpret_cast<uintptr_t>(Xq) & 3) != 0) return fail(ITL_ERR_INVALID_ARG, "Xq must be 4-byte aligned");
  hipError_t e = itl::launch_quantize_rows_fp8(X, (int)dtype, n_rows, (int)d, Xq, scale,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_quantize_rows_fp8");
}

itl_status itl_lmhead_logprob_fp8(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq, const float* w_scale,
                                  int64_t n_tok, int64_t d, int64_t vocab, const int32_t* tokens, float* logprob,
                                  float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (n_tok < 0 || d <= 0 || vocab <= 0) return fail(ITL_ERR_INVALID_ARG, "n_tok must be >= 0, d and vocab > 0");
  if (d % kFp8DMultiple != 0) return fail(ITL_ERR_UNSUPPORTED, "d must be a multiple of 128");
  if (n_tok > kMaxTok) return fail(ITL_ERR_UNSUPPORTED, "n_tok too large for one call");
  if (vocab > kMaxVocab) return fail(ITL_ERR_UNSUPPORTED, "vocab too large");
  if (d >= ((int64_t)1 << 31) / (int64_t)itl::kBT) return fail(ITL_ERR_UNSUPPORTED, "d too large");
  if (vocab > (int64_t)(UINT32_MAX / 4)) return fail(ITL_ERR_UNSUPPORTED, "vocab too large");
  // the grid of the kernel that runs: narrow for few tokens
  const bool narrow = n_tok <= itl::kNarrowMaxTokens;
  const int64_t grid = narrow ? itl::ceil_div(n_tok, itl::kNarrowBRows) * itl::n_slices(vocab)
                              : itl::ceil_div(n_tok, itl::kBT) * itl::n_slice_groups(n_tok, vocab);
  if (grid > INT32_MAX) return fail(ITL_ERR_UNSUPPORTED, "problem too large for one launch");
  if (n_tok == 0) return ITL_OK;
  if (!Hq || !h_scale || !Wq || !w_scale || !tokens || !logprob)
    return fail(ITL_ERR_INVALID_ARG, "null Hq, h_scale, Wq, w_scale, tokens or logprob");
  if (((reinterpret_cast<uintptr_t>(Hq) | reinterpret_cast<uintptr_t>(Wq)) & 15) != 0)
    return fail(ITL_ERR_INVALID_ARG, "Hq and Wq must be 16-byte aligned");
  if (!workspace || workspace_bytes < itl::lmhead_workspace_bytes(n_tok, vocab))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_lmhead_logprob_workspace_bytes()");
  if (misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_lmhead_logprob_fp8(Hq, h_scale, Wq, w_scale, (int)n_tok, (int)d, (int)vocab, tokens,
                                                logprob, lse, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_lmhead_logprob_fp8");
}

itl_status itl_quantize_rows_mxfp4(const void* X, itl_dtype dtype, int64_t n_rows, int64_t d, uint8_t* Xq,
                                   uint8_t* scale_codes, void* stream) {
  g_last_error.clear();
  if (n_rows < 0 || d <= 0) return fail(ITL_ERR_INVALID_ARG, "n_rows must be >= 0 and d > 0");
  if (dtype != ITL_BF16 && dtype != ITL_F32) return fail(ITL_ERR_UNSUPPORTED, "dtype must be ITL_BF16 or ITL_F32");
  if (d % kFp8DMultiple != 0) return fail(ITL_ERR_UNSUPPORTED, "d must be a multiple of 128");
  if (d > INT32_MAX || n_rows > ((int64_t)INT32_MAX * 256) / (d / 32)) return fail(ITL_ERR_UNSUPPORTED, "too many rows");
  if (n_rows == 0) return ITL_OK;
  if (!X || !Xq || !scale_codes) return fail(ITL_ERR_INVALID_ARG, "null X, Xq or scale_codes");
  if ((reinterpret_cast<uintptr_t>(Xq) & 15) != 0) return fail(ITL_ERR_INVALID_ARG, "Xq must be 16-byte aligned");
  hipError_t e = itl::launch_quantize_rows_mxfp4(X, (int)dtype, n_rows, (int)d, Xq, scale_codes,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_quantize_rows_mxfp4");
}

itl_status itl_lmhead_logprob_mxfp4(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq4,
                                    const uint8_t* w_scale_codes, int64_t n_tok, int64_t d, int64_t vocab,
                                    const int32_t* tokens, float* logprob, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (n_tok < 0 || d <= 0 || vocab <= 0) return fail(ITL_ERR_INVALID_ARG, "n_tok must be >= 0, d and vocab > 0");
  if (d % kFp8DMultiple != 0) return fail(ITL_ERR_UNSUPPORTED, "d must be a multiple of 128");
  if (n_tok > kMaxTok) return fail(ITL_ERR_UNSUPPORTED, "n_tok too large for one call");
  if (vocab > kMaxVocab) return fail(ITL_ERR_UNSUPPORTED, "vocab too large");
  if (d >= ((int64_t)1 << 31) / (int64_t)itl::kBT) return fail(ITL_ERR_UNSUPPORTED, "d too large");
  const int64_t grid = itl::ceil_div(n_tok, itl::kBT) * itl::n_slice_groups(n_tok, vocab);
  if (grid > INT32_MAX) return fail(ITL_ERR_UNSUPPORTED, "problem too large for one launch");
  if (n_tok == 0) return ITL_OK;
  if (!Hq || !h_scale || !Wq4 || !w_scale_codes || !tokens || !logprob)
    return fail(ITL_ERR_INVALID_ARG, "null Hq, h_scale, Wq4, w_scale_codes, tokens or logprob");
  if (((reinterpret_cast<uintptr_t>(Hq) | reinterpret_cast<uintptr_t>(Wq4)) & 15) != 0)
    return fail(ITL_ERR_INVALID_ARG, "Hq and Wq4 must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(w_scale_codes) & 3) != 0)
    return fail(ITL_ERR_INVALID_ARG, "w_scale_codes must be 4-byte aligned");
  if (!workspace || workspace_bytes < itl::lmhead_workspace_bytes(n_tok, vocab))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_lmhead_logprob_workspace_bytes()");
  if (misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_lmhead_logprob_mxfp4(Hq, h_scale, Wq4, w_scale_codes, (int)n_tok, (int)d, (int)vocab,
                                                  tokens, logprob, lse, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_lmhead_logprob_mxfp4");
}

size_t itl_mismatch_stats_workspace_bytes(int64_t n_tok) {
  if (n_tok < 0 || n_tok > INT32_MAX) return SIZE_MAX;
  return n_tok == 0 ? 0 : itl::mismatch_stats_workspace_bytes(n_tok);
}

itl_status itl_mismatch_stats(const float* logprob, const float* rollout_logprob, const float* same_weights_logprob,
                              int64_t n_tok, double* stats, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (n_tok < 0) return fail(ITL_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (n_tok > INT32_MAX) return fail(ITL_ERR_UNSUPPORTED, "n_tok too large for one call");
  if (!stats) return fail(ITL_ERR_INVALID_ARG, "null stats");
  if (n_tok > 0 && (!logprob || !rollout_logprob)) return fail(ITL_ERR_INVALID_ARG, "null logprob arrays");
  const size_t need = n_tok == 0 ? 0 : itl::mismatch_stats_workspace_bytes(n_tok);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(ITL_ERR_WORKSPACE, "workspace missing or smaller than itl_mismatch_stats_workspace_bytes()");
  if (need > 0 && misaligned(workspace)) return fail(ITL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipError_t e = itl::launch_mismatch_stats(logprob, rollout_logprob, same_weights_logprob, n_tok, stats, workspace,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ITL_OK : hip_fail(e, "itl_mismatch_stats");
}

itl_status itl_check_inputs(const int32_t* tokens, int64_t n_tok, int64_t vocab, const int64_t* resp_offsets,
                            int32_t n_resp, void* stream) {
  g_last_error.clear();
  if (n_tok < 0 || n_resp < 0 || vocab <= 0 || vocab > kMaxVocab)
    return fail(ITL_ERR_INVALID_ARG, "bad sizes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* flag = nullptr;
  hipError_t e = hipMalloc(&flag, sizeof(int));
  if (e != hipSuccess) return hip_fail(e, "itl_check_inputs");
  int host = 0;
  e = hipMemcpyAsync(flag, &host, sizeof(int), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = itl::launch_check_inputs(tokens, n_tok, (int)vocab, resp_offsets, n_resp, flag, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipFree(flag);
  if (e != hipSuccess) return hip_fail(e, "itl_check_inputs");
  if (host == 1) return fail(ITL_ERR_BAD_INPUT, "a token id is outside [0, vocab)");
  if (host == 2) return fail(ITL_ERR_BAD_INPUT, "response offsets must start at 0, end at n_tok and increase");
  return ITL_OK;
}

const char* itl_status_string(itl_status status) {
  switch (status) {
    case ITL_OK: return "ITL_OK";
    case ITL_ERR_INVALID_ARG: return "ITL_ERR_INVALID_ARG: invalid argument";
    case ITL_ERR_UNSUPPORTED: return "ITL_ERR_UNSUPPORTED: shape or dtype not supported by this build";
    case ITL_ERR_WORKSPACE: return "ITL_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case ITL_ERR_HIP: return "ITL_ERR_HIP: HIP runtime error";
    case ITL_ERR_BAD_INPUT: return "ITL_ERR_BAD_INPUT: invalid device-resident input";
  }
  return "unknown itl_status";
}

const char* itl_last_error(void) { return g_last_error.c_str(); }

const char* itl_build_info(void) {
  static const std::string info = [] {
    char buf[768];
    snprintf(buf, sizeof buf,
             "itl 0.3 arch=gfx950 threads=%d wide_threads=%d token_block=%d vocab_tile=%d k_step_bytes=%d w_slots=%d h_slots=%d "
             "swap_slots_over_k_steps=%d max_slices=%d slices=balanced narrow_max_tokens=%d narrow_token_block=%d narrow128_max_tokens=%d "
             "mfma_bf16=16x16x32 mfma_f32=16x16x4 fp8=e4m3_row_scaled mfma_fp8=16x16x128 mxfp4=e2m1_e8m0_32 mfma_mxfp4=32x32x64 "
             "bwd_chunk_tokens=%d loss_segment_tokens=%d loss_lane_segment=%d loss_wave_segment=%d loss_threads=%d "
             "loss_mean_chunk=%d loss_sums=f64 bwd_sampled_sort=stable_counting bwd_sampled_segment=%d "
             "bwd_sampled_group=%d",
             itl::kThreads, itl::kThreads8, itl::kBT, itl::kBV, itl::kStepBytes, itl::kWSlots, itl::kHSlots, itl::kNearBMaxSteps,
             itl::kMaxSlices, itl::kNarrowMaxTokens, itl::kNarrowBRows, itl::kNarrow128MaxTokens, itl::kBwdChunkTokens, itl::kSegTokens,
             itl::kLaneSeg, itl::kWaveSeg, itl::kLossThreads, itl::kFinishChunk, itl::kRunSeg, itl::kRunGroup);
    return std::string(buf);
  }();
  return info.c_str();
}

}  // extern "C"
