// Fused LM-head contraction + online log-sum-exp + sampled-token gather.
//
// What is computed ("vLLM says aligned kernels make asynchronous RL stable at
// lag 64", section "REINFORCE Zero removes the mismatch first": the logprob
// of each sampled token; "vLLM Train-Inference Consistency Release Notes",
// section "Achieving Bitwise Consistency": deterministic, batch-independent
// and phase-consistent):
//
//   z[t, v]    = sum_k H[t, k] W[v, k]         fp32 accumulate, ascending k
//   lse[t]     = log sum_v exp(z[t, v])
//   logprob[t] = z[t, y_t] - lse[t]
//
// Kernel 1 (lmhead_lse_partial8, or the narrow kernel for calls of at most
// 64 tokens) computes z^T tiles on the matrix cores: the MFMA A operand is a
// 256-row tile of W, the B operand a 256-token block of H, both read
// K-contiguous, on the eight-wavefront engine (tile_engine8.h). The
// vocabulary is cut into S = min(tiles, 256) balanced slices, a function of V
// alone. A workgroup owns one token block and a run of consecutive slices
// and walks their tiles in ascending order; after each tile its lanes fold
// the tile into a running (max, sum of exp) per token (fold_column16) and
// pick out z[t, y_t] if y_t falls in the tile. The logits never leave
// registers. At each slice end the four lane quarters that share a token
// are merged and each wavefront writes one (max, sumexp) pair per token, then
// starts the next slice afresh, so the 2 S partials of a token are the same
// whether a workgroup walks one slice (small batches: every CU streams W) or
// several (large batches: fewer, longer workgroups).
// Kernel 2 (lse_combine) merges a token's 2 S partials in a fixed order.
// With kKeep the same kernels also write every logit z[t, v] (fp32, row
// stride ld) from the accumulators the fold reads, for a backward that
// forms the dlogits from them instead of recomputing the contraction; the
// arithmetic, and so every partial and logprob, is unchanged.
//
// Why the bits do not depend on the batch: the tile shapes, K order, slice
// width and every reduction tree are compile-time constants; a token's
// column is computed by the same instruction sequence whatever its position
// in the block, and rows beyond n_tok are loaded as zeros and never written.
// There is no split-K and no atomic.
//
// MFMA layouts used (16 x 16 blocks: v_mfma_f32_16x16x32_bf16, and
// v_mfma_f32_16x16x4f32 for fp32 heads): lane l supplies row (l mod 16) of
// an A block and column (l mod 16) of a B block, with the k range chosen by
// l / 16; accumulator register i of lane l holds row 4*(l/16) + i, column
// (l mod 16).

#include "itl_launch.h"
#include "lse_fold.h"
#include "tile_engine.h"
#include "tile_engine8.h"

namespace itl {

namespace {

// Kept logits are written with buffer stores against a range that ends at
// the wavefront's last valid token row, so rows past n_tok are dropped by
// the hardware instead of a branch. LogitRows: the range (SGPRs) and this
// lane's row offset in bytes, (c16 * ld + 4 quad) * 4 (ld * 4 * 128 < 2^32).
struct LogitRows {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;
  uint32_t bn_stride;  // bytes between the token columns of blocks bn and bn + 1 (16 rows)
};

// Built in each epilogue, not once per kernel: kept live across the K loop,
// these registers would push the loop's operands into scratch. The empty asm
// makes the inputs opaque, so the compiler cannot hoist the build out of
// the tile loop.
__device__ __forceinline__ LogitRows logit_rows(float* logits, long long ld, int tok_first, int n_rows, int n_tok,
                                                int c16, int quad) {
  asm volatile("" : "+s"(tok_first));
  LogitRows r;
  const int valid = max(0, min(n_rows, n_tok - tok_first));
  // Raw buffer (stride 0), 32-bit data format: the same descriptor word 3 as
  // the engine's operand loads. The fields are wave-uniform by construction;
  // readfirstlane tells the compiler so (a descriptor it takes for divergent
  // would turn every store into a loop over the lanes' distinct values).
  const uint64_t base = reinterpret_cast<uint64_t>(logits + (size_t)tok_first * (size_t)ld);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int nbytes = __builtin_amdgcn_readfirstlane((int)((uint32_t)valid * (uint32_t)ld * 4u));
  r.rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0, nbytes,
                                             0x00020000);
  r.voff = ((uint32_t)c16 * (uint32_t)ld + 4u * (uint32_t)quad) * 4u;
  r.bn_stride = __builtin_amdgcn_readfirstlane(16u * (uint32_t)ld * 4u);
  return r;
}

// Write this lane's 4 logits of a 16 x 16 block: token column bn of the
// rows, vocabulary rows v0 + 4 quad + r (r < 4) from register r (v0 = the
// block's first row, the same for the whole wavefront): 16 contiguous bytes
// of the token's row. In the vocabulary's last tile, rows at or past the
// vocabulary are not written.
template <class kPartial>
__device__ __forceinline__ void store_logits(const LogitRows& rows, int bn, int v0, int quad, int vocab,
                                             const floatx4& z, kPartial) {
  const uint32_t voff = rows.voff + (uint32_t)bn * rows.bn_stride;
  const uint32_t so = (uint32_t)v0 * 4u;
  if constexpr (!kPartial::value) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4v, z), rows.rsrc, voff, so, kLogitStorePolicy);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (v0 + 4 * quad + r < vocab)
        __builtin_amdgcn_raw_buffer_store_b32((int)__float_as_uint(z[r]), rows.rsrc, voff + 4u * r, so,
                                              kLogitStorePolicy);
  }
}

// Kernel 1 for calls of more than 64 tokens, on the eight-wavefront engine
// (run_tiles8): a 512-thread workgroup per (256-token block, slice group).
// Wavefront (wv, tq) holds W rows 128 wv .. + 127 of each tile against
// tokens t0 + 64 tq .. + 63; lane l holds tokens t0 + 64 tq + 16 bn +
// (l mod 16) (bn < 4), 32 of the wavefront's 128 rows each. After each tile
// each token column's 32 logits are folded in one step (fold_column16),
// tiles in order, and at the slice's end the four lane quarters are merged,
// as in the narrow kernel, so a token's partials have the same bits in
// both. With kKeep the tile's logits are stored first (one 16-byte store per
// block).
template <int kDtype, bool kKeep, bool kBFar>
__global__ __launch_bounds__(kThreads8, 1) void lmhead_lse_partial8_kernel(
    const char* __restrict__ H, const char* __restrict__ W, const int32_t* __restrict__ tokens, int n_tok,
    int row_bytes, int vocab, int n_tb, int n_slices, int group, float2* __restrict__ part,
    float* __restrict__ zy_out, float* __restrict__ logits, long long ld) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes8 L = lanes8();
  const int wv = L.wv, tq = L.tq, quad = L.quad, c16 = L.c16;

  const int S = n_slices;
  const WideWork work = wide_work(blockIdx.x, n_tb, S, group);
  const int t0 = work.tb * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(work.slice_first, n_vt, S);
  const int tile_end = slice_tile(work.slice_end, n_vt, S);
  const int nks = row_bytes / kStepBytes;

  Col16 c[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int tok = t0 + tq * 64 + bn * 16 + c16;
    c[bn] = Col16{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f};
  }
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(W + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  const int4v hr = rsrc_words(H + (size_t)t0 * row_bytes, (uint32_t)min(kBT, n_tok - t0) * row_bytes);

  int slice = work.slice_first;
  int slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
  auto epilogue = [&](int tile, floatx4 (&acc)[8][4]) {
    const int vw = tile * kBV + wv * 128;
    // This lane's token offset, made opaque here so that the per-lane
    // addresses below are formed in each epilogue: hoisted out of the tile
    // loop they would be live across the K loop and push values into scratch.
    int lt = L.lane;
    asm volatile("" : "+v"(lt));
    lt = tq * 64 + (lt & 15);
    auto fold_tile = [&](auto partial, auto pick) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        if constexpr (kKeep) {
          const LogitRows rows = logit_rows(logits, ld, t0 + tq * 64, 64, n_tok, c16, quad);
#pragma unroll
          for (int bm = 0; bm < 8; ++bm) store_logits(rows, bn, vw + bm * 16, quad, vocab, acc[bm][bn], partial);
        }
        floatx4 z[8];
#pragma unroll
        for (int bm = 0; bm < 8; ++bm) z[bm] = acc[bm][bn];
        if constexpr (decltype(pick)::value) pick_sampled(c[bn], z, vw, quad, zy_out + (t0 + lt + bn * 16));
        fold_column16(c[bn], z, vw, quad, vocab, partial);
        __builtin_amdgcn_sched_barrier(0);  // one token column at a time (register pressure)
      }
    };
    // A lane's sampled row lies in this wavefront's 128 rows of a given tile
    // for about one tile in V / 128, so most tiles skip the pick (a uniform
    // branch: the picked values are the same either way).
    bool mine = false;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      int y = c[bn].y;
      asm volatile("" : "+v"(y));  // (no test hoisted out of the tile loop)
      mine = mine || (unsigned)(y - vw) < 128u;
    }
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{}, std::true_type{});  // only the vocabulary's last tile
    else if (__builtin_amdgcn_ballot_w64(mine) != 0) fold_tile(std::false_type{}, std::true_type{});
    else fold_tile(std::false_type{}, std::false_type{});
    if (tile == slice_last_tile) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const int tok = t0 + lt + bn * 16;
        flush_slice16(c[bn], tok, n_tok, quad, ((size_t)slice * 2 + wv) * n_tok + tok, part);
      }
      ++slice;
      int Sx = S;
      asm volatile("" : "+s"(Sx));  // (the division's set-up stays here, not live across the K loop)
      slice_last_tile = slice_tile(slice + 1, n_vt, Sx) - 1;
    }
  };
  run_tiles8<kDtype, kBFar>(smem, L, row_bytes, tile_begin, tile_end, nks, w_rsrc, hr, epilogue);
}

// The same partials for few tokens: kBRows-token blocks (64, or 128 for
// calls of 65 to 128 tokens, where one wide 256-token block would do twice
// the contraction work), one workgroup per (token block, slice), the
// workgroup's slice walked by run_tiles_narrow. Lane l of wavefront (wv, wt)
// holds tokens t0 + (kBRows / 2) wt + 16 bn + (l mod 16) (bn < kBRows / 32)
// against the same W rows, with the same fold, as in
// lmhead_lse_partial8_kernel, so the partials (and the logprobs) have the
// same bits.
template <int kDtype, bool kKeep, int kBRows>
__global__ __launch_bounds__(kThreads, 1) void lmhead_lse_partial_narrow_kernel(
    const char* __restrict__ H, const char* __restrict__ W, const int32_t* __restrict__ tokens, int n_tok,
    int row_bytes, int vocab, int n_slices, float2* __restrict__ part, float* __restrict__ zy_out,
    float* __restrict__ logits, long long ld) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes L = lanes();
  const int wv = L.wv, wt = L.wt, quad = L.lane >> 4, c16 = L.lane & 15;
  // Token block fastest-varying after the slice: with 256 slices the token
  // blocks of a slice share an XCD (blockIdx mod 8) and its L2.
  const int S = n_slices;
  const int slice = blockIdx.x % S;
  constexpr int kBN = kBRows / 32;  // token columns per lane
  constexpr int kWaveToks = kBRows / 2;
  const int t0 = (blockIdx.x / S) * kBRows;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(slice, n_vt, S);
  const int tile_end = slice_tile(slice + 1, n_vt, S);
  const int nks = row_bytes / kStepBytes;
  Col16 c[kBN];
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * kWaveToks + bn * 16 + c16;
    c[bn] = Col16{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f};
  }

  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(W + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  const int4v hr = rsrc_words(H + (size_t)t0 * row_bytes, (uint32_t)min(kBRows, n_tok - t0) * row_bytes);
  const LogitRows rows = logit_rows(logits, ld, t0 + wt * kWaveToks, kWaveToks, n_tok, c16, quad);
  auto epilogue = [&](int tile, floatx4 (&acc)[8][kBN]) {
    const int vw = tile * kBV + wv * 128;
    auto fold_tile = [&](auto partial) {
      if constexpr (kKeep) {
#pragma unroll
        for (int bn = 0; bn < kBN; ++bn)
#pragma unroll
          for (int bm = 0; bm < 8; ++bm) store_logits(rows, bn, vw + bm * 16, quad, vocab, acc[bm][bn], partial);
      }
#pragma unroll
      for (int bn = 0; bn < kBN; ++bn) {
        floatx4 z[8];
#pragma unroll
        for (int bm = 0; bm < 8; ++bm) z[bm] = acc[bm][bn];
        pick_sampled(c[bn], z, vw, quad, zy_out + (t0 + wt * kWaveToks + bn * 16 + c16));
        fold_column16(c[bn], z, vw, quad, vocab, partial);
      }
    };
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{});
    else fold_tile(std::false_type{});
  };
  run_tiles_narrow<kDtype, kBRows>(smem, L, row_bytes, tile_begin, tile_end, nks, w_rsrc, hr, epilogue);
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * kWaveToks + bn * 16 + c16;
    flush_slice16(c[bn], tok, n_tok, quad, ((size_t)slice * 2 + wv) * n_tok + tok, part);
  }
}

}  // namespace

// Per token: merge the 2 S partials (slice-major, then wavefront). A
// 1024-thread workgroup takes 64 tokens (lane = token, so every load is one
// coalesced 512-byte row of the partial table); its 16 wavefronts split the
// partials into 16 fixed consecutive runs, fold each run in order, and the
// 16 run states are merged in run order. The run boundaries depend on S only,
// so a token's result has the same bits whatever n_tok. A run is at most 32
// partials; all of a run's loads are issued before its first merge, so a
// call waits on one memory round trip, not one per partial (a decode call's
// combine is latency-bound).
constexpr int kCombineWaves = 16;
constexpr int kCombineMaxRun = 32;
static_assert(2 * kMaxSlices <= kCombineWaves * kCombineMaxRun, "a run must fit the register buffer");

namespace {

__global__ __launch_bounds__(64 * kCombineWaves) void lse_combine_kernel(const float2* __restrict__ part,
                                                                         const float* __restrict__ zy, int n_tok,
                                                                         int n_parts, float* __restrict__ logprob,
                                                                         float* __restrict__ lse) {
  __shared__ float2 run_state[kCombineWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const int run = (n_parts + kCombineWaves - 1) / kCombineWaves;
  const int p0 = min(w * run, n_parts), p1 = min(p0 + run, n_parts);
  float m = -INFINITY, s = 0.0f;
  if (t < n_tok) {
    float2 v[kCombineMaxRun];
#pragma unroll
    for (int i = 0; i < kCombineMaxRun; ++i)
      if (p0 + i < p1) v[i] = part[(size_t)(p0 + i) * n_tok + t];
#pragma unroll
    for (int i = 0; i < kCombineMaxRun; ++i)
      if (p0 + i < p1) lse_merge(m, s, v[i].x, v[i].y);
  }
  run_state[w][lane] = make_float2(m, s);
  __syncthreads();
  if (w != 0 || t >= n_tok) return;
#pragma unroll
  for (int r = 1; r < kCombineWaves; ++r) lse_merge(m, s, run_state[r][lane].x, run_state[r][lane].y);
  // lse >= the largest logit holds mathematically; the fold's shared
  // exponent offset can leave the sum a rounding below 1 when one logit
  // dominates, so it is kept explicitly (and with it logprob <= 0)
  const float l = fmaxf(m + fast_log2(s) * kLn2, m);
  logprob[t] = zy[t] - l;
  if (lse) lse[t] = l;
}

}  // namespace

hipError_t launch_lse_combine(const float2* part, const float* zy, int n_tok, int n_parts, float* logprob, float* lse,
                              hipStream_t stream) {
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)ceil_div(n_tok, 64)), dim3(64 * kCombineWaves), 0, stream,
                     part, zy, n_tok, n_parts, logprob, lse);
  return hipGetLastError();
}

size_t lmhead_workspace_bytes(long long n_tok, long long vocab) {
  if (n_tok <= 0) return 0;
  return align256((size_t)2 * n_slices(vocab) * (size_t)n_tok * sizeof(float2)) + align256((size_t)n_tok * sizeof(float));
}

namespace {

template <int kDtype, bool kKeep>
void launch_partials(const char* H, const char* W, const int32_t* tokens, int n_tok, int row_bytes, int vocab,
                     float2* part, float* zy, float* logits, long long ld, hipStream_t stream) {
  const int S = n_slices(vocab);
  if (n_tok <= kNarrowMaxTokens) {
    const dim3 grid((unsigned)ceil_div(n_tok, kNarrowBRows) * (unsigned)S);
    hipLaunchKernelGGL((lmhead_lse_partial_narrow_kernel<kDtype, kKeep, kNarrowBRows>), grid, dim3(kThreads), 0,
                       stream, H, W, tokens, n_tok, row_bytes, vocab, S, part, zy, logits, ld);
  } else if (n_tok <= kNarrow128MaxTokens) {
    const dim3 grid((unsigned)S);
    hipLaunchKernelGGL((lmhead_lse_partial_narrow_kernel<kDtype, kKeep, kNarrow128MaxTokens>), grid, dim3(kThreads), 0,
                       stream, H, W, tokens, n_tok, row_bytes, vocab, S, part, zy, logits, ld);
  } else {
    const int G = slices_per_group(n_tok, vocab);
    const int ntb = (int)ceil_div(n_tok, kBT);
    const dim3 grid((unsigned)ntb * (unsigned)n_slice_groups(n_tok, vocab));
    // Long K loops stage the token block two K steps ahead (see run_tiles8).
    // The fp32 head's kept-logits kernel always does (the other load order
    // needs one register more than it has): the load order changes no
    // arithmetic, so the bits are the same either way.
    constexpr bool kFarOnly = kDtype == 1 && kKeep;
    if (kFarOnly || row_bytes / kStepBytes > kNearBMaxSteps)
      hipLaunchKernelGGL((lmhead_lse_partial8_kernel<kDtype, kKeep, true>), grid, dim3(kThreads8), 0, stream, H, W,
                         tokens, n_tok, row_bytes, vocab, ntb, S, G, part, zy, logits, ld);
    else if constexpr (!kFarOnly)
      hipLaunchKernelGGL((lmhead_lse_partial8_kernel<kDtype, kKeep, false>), grid, dim3(kThreads8), 0, stream, H, W,
                         tokens, n_tok, row_bytes, vocab, ntb, S, G, part, zy, logits, ld);
  }
}

}  // namespace

hipError_t launch_lmhead_logprob(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                 const int32_t* tokens, float* logprob, float* lse, float* logits, long long ld,
                                 void* workspace, hipStream_t stream) {
  const int es = dtype == 0 ? 2 : 4;
  const int row_bytes = d * es;
  const int S = n_slices(vocab);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)2 * S * (size_t)n_tok * sizeof(float2)));
  const char* Hc = static_cast<const char*>(H);
  const char* Wc = static_cast<const char*>(W);
  if (dtype == 0) {
    if (logits) launch_partials<0, true>(Hc, Wc, tokens, n_tok, row_bytes, vocab, part, zy, logits, ld, stream);
    else launch_partials<0, false>(Hc, Wc, tokens, n_tok, row_bytes, vocab, part, zy, nullptr, 0, stream);
  } else {
    if (logits) launch_partials<1, true>(Hc, Wc, tokens, n_tok, row_bytes, vocab, part, zy, logits, ld, stream);
    else launch_partials<1, false>(Hc, Wc, tokens, n_tok, row_bytes, vocab, part, zy, nullptr, 0, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lse_combine(part, zy, n_tok, 2 * S, logprob, lse, stream);
}

}  // namespace itl
