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
// Kernel 1 (lmhead_lse_partial) computes z^T tiles on the matrix cores: the
// MFMA A operand is a 256-row tile of W, the B operand a 256-token block of
// H, both read K-contiguous. The vocabulary is cut into S = min(tiles, 256)
// balanced slices, a function of V alone. A workgroup owns one token block
// and a run of consecutive slices and walks their tiles in ascending order;
// after each tile its lanes fold the tile into a running (max, sum of exp)
// per token and pick out z[t, y_t] if y_t falls in the tile. The logits never
// leave registers. At each slice end the two lane halves that share a token
// are merged and each wavefront writes one (max, sumexp) pair per token, then
// starts the next slice afresh, so the 2 S partials of a token are the same
// whether a workgroup walks one slice (small batches: every CU streams W) or
// several (large batches: fewer, longer workgroups).
// Kernel 2 (lse_combine) merges a token's 2 S partials in a fixed order.
//
// Why the bits do not depend on the batch: the tile shapes, K order, slice
// width and every reduction tree are compile-time constants; a token's
// column is computed by the same instruction sequence whatever its position
// in the block, and rows beyond n_tok are loaded as zeros and never written.
// There is no split-K and no atomic.
//
// MFMA layouts used (v_mfma_f32_32x32x16_bf16, and v_mfma_f32_32x32x2f32 for
// fp32 heads): lane l supplies row (l mod 32) of A and column (l mod 32) of
// B, with the k range chosen by l / 32; accumulator register i of lane l
// holds row 8*(i/4) + 4*(l/32) + (i mod 4), column (l mod 32).

#include "itl_launch.h"
#include "tile_engine.h"

namespace itl {

namespace {

template <int kDtype>
__global__ __launch_bounds__(kThreads, 1) void lmhead_lse_partial_kernel(
    const char* __restrict__ H, const char* __restrict__ W, const int32_t* __restrict__ tokens, int n_tok,
    int row_bytes, int vocab, int n_tb, int n_slices, int group, float2* __restrict__ part,
    float* __restrict__ zy_out) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes L = lanes();
  const int wv = L.wv, wt = L.wt, half = L.half, col = L.col;

  // Workgroup order: super-bands of kSuperBand token blocks, walked slice
  // group by slice group with the token block fastest. Workgroups are
  // dispatched to the 8 XCDs round-robin, so the 32 workgroups an XCD runs
  // at once hold 4 token blocks x 8 slice groups (each H block read by 8 of
  // them, each W tile by 4, through the XCD's L2), and all XCDs walk the same
  // slices at the same time (W shared through the Infinity Cache). The order
  // and the grouping change only which workgroup computes a slice when,
  // never any arithmetic.
  const int S = n_slices;
  const int n_groups = (S + group - 1) / group;
  const int b = blockIdx.x;
  const int band = b / (kSuperBand * n_groups);
  const int tb_first = band * kSuperBand;
  const int nb = min(kSuperBand, n_tb - tb_first);
  const int rem = b - band * kSuperBand * n_groups;
  const int grp = rem / nb;
  const int t0 = (tb_first + rem % nb) * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int slice_first = grp * group;
  const int slice_end = min(slice_first + group, S);
  const int tile_begin = slice_tile(slice_first, n_vt, S);
  const int tile_end = slice_tile(slice_end, n_vt, S);
  const int nks = row_bytes / kStepBytes;

  // The engine's A operand is the W tile (vocabulary rows), its B operand
  // the H block (tokens): lane l's accumulators are vocabulary rows of token
  // t0 + 128 wt + 32 bn + (l mod 32).
  int y[4];
  float mrun[4], srun[4], zy[4];
  bool found[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int tok = t0 + wt * 128 + bn * 32 + col;
    y[bn] = tok < n_tok ? tokens[tok] : -1;
    mrun[bn] = -INFINITY;
    srun[bn] = 0.0f;
    zy[bn] = 0.0f;
    found[bn] = false;
  }

  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(W + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  const int4v hr = rsrc_words(H + (size_t)t0 * row_bytes, (uint32_t)min(kBT, n_tok - t0) * row_bytes);

  // Tile epilogue: fold the tile's logits into the running state. Each lane
  // folds its 16 logits of one 32x32 block at a time into the running (max,
  // sum of exp) of that token column; the logits are copied out of the
  // matrix-core registers 16 at a time, where they are used (acc_read), so
  // the epilogue needs few VGPRs next to the 256 accumulators. The sampled
  // logit is picked with a select tree keyed on the bits of its row,
  // without a branch.
  int slice = slice_first;                              // slice of the tiles being folded
  int slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
  auto epilogue = [&](int tile, floatx16 (&acc)[4][4]) {
    const int vw = tile * kBV + wv * 128;
    const bool partial = tile * kBV + kBV > vocab;  // only the vocabulary's last tile
    mfma_result_wait();
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int o = y[bn] - vw;  // sampled row relative to this wavefront's 128 rows
      // Register i of a lane holds row 32 bm + 8 (i / 4) + 4 half + (i % 4):
      // bits 0, 1, 3, 4 of the row pick i, bit 2 picks the lane half.
      const bool b0 = (o & 1) != 0, b1 = (o & 2) != 0, b2 = (o & 8) != 0, b3 = (o & 16) != 0;
      const bool mine = (unsigned)o < 128u && ((o >> 2) & 1) == half;
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        floatx16 z;  // a vector, not an array: it must stay in registers
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = acc_read(acc[bm][bn], i);
        if (partial) {
          const int lim = vocab - (vw + bm * 32 + 4 * half);  // rows at or past this offset do not exist
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = (8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : z[i];
        }
        const float pick = select16(z, b0, b1, b2, b3);
        const bool here = mine && (o >> 5) == bm;
        zy[bn] = here ? pick : zy[bn];
        found[bn] = found[bn] || here;

        float bmax = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) bmax = fmaxf(bmax, z[i]);
        const float mnew = fmaxf(mrun[bn], bmax);
        // A lane whose rows so far are all absent has mnew = -inf; it then
        // scales by exp2(-inf) = 0 around 0 and keeps (m, s) = (-inf, 0).
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        // (z - m) is exactly 0 for the running maximum, so its term is
        // exactly 1 and stays 1 (later rescales by exp2(0)): the final sum
        // is >= 1 and logprob <= 0 holds in fp32.
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          s0 += fast_exp2((z[i] - mref) * kLog2e);
          s1 += fast_exp2((z[i + 1] - mref) * kLog2e);
        }
        srun[bn] = srun[bn] * fast_exp2((mrun[bn] - mref) * kLog2e) + (s0 + s1);
        mrun[bn] = mnew;
      }
    }
    if (tile == slice_last_tile) {
      // Slice end: lanes l and l^32 hold the same tokens (different rows);
      // each wavefront writes its own partial (wv = 0, 1) and starts over.
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const float m2 = __shfl_xor(mrun[bn], 32, 64);
        const float s2 = __shfl_xor(srun[bn], 32, 64);
        lse_merge(mrun[bn], srun[bn], m2, s2);
        const int tok = t0 + wt * 128 + bn * 32 + col;
        if (half == 0 && tok < n_tok) part[((size_t)slice * 2 + wv) * n_tok + tok] = make_float2(mrun[bn], srun[bn]);
        mrun[bn] = -INFINITY;
        srun[bn] = 0.0f;
      }
      ++slice;
      slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
    }
  };
  run_tiles<kDtype>(smem, L, row_bytes, tile_begin, tile_end, nks, w_rsrc, hr, epilogue);

#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
    if (found[bn]) zy_out[t0 + wt * 128 + bn * 32 + col] = zy[bn];
}

// Per token: merge the 2 S partials (slice-major, then wavefront) in order.
__global__ __launch_bounds__(256) void lse_combine_kernel(const float2* __restrict__ part,
                                                          const float* __restrict__ zy, int n_tok,
                                                          int n_parts, float* __restrict__ logprob,
                                                          float* __restrict__ lse) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float M = -INFINITY;
  for (int s = 0; s < n_parts; ++s) M = fmaxf(M, part[(size_t)s * n_tok + t].x);
  float S = 0.0f;
  for (int s = 0; s < n_parts; ++s) {
    const float2 p = part[(size_t)s * n_tok + t];
    S += p.y * fast_exp2((p.x - M) * kLog2e);
  }
  const float l = M + fast_log2(S) * kLn2;
  logprob[t] = zy[t] - l;
  if (lse) lse[t] = l;
}

}  // namespace

size_t lmhead_workspace_bytes(long long n_tok, long long vocab) {
  if (n_tok <= 0) return 0;
  return align256((size_t)2 * n_slices(vocab) * (size_t)n_tok * sizeof(float2)) + align256((size_t)n_tok * sizeof(float));
}

hipError_t launch_lmhead_logprob(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                 const int32_t* tokens, float* logprob, float* lse, void* workspace,
                                 hipStream_t stream) {
  const int es = dtype == 0 ? 2 : 4;
  const int row_bytes = d * es;
  const int S = n_slices(vocab);
  const int G = slices_per_group(n_tok, vocab);
  const int ntb = (int)ceil_div(n_tok, kBT);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)2 * S * (size_t)n_tok * sizeof(float2)));
  const dim3 grid((unsigned)ntb * (unsigned)n_slice_groups(n_tok, vocab));
  if (dtype == 0)
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<0>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, ntb, S, G, part, zy);
  else
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<1>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, ntb, S, G, part, zy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, part, zy, n_tok,
                     2 * S, logprob, lse);
  return hipGetLastError();
}

}  // namespace itl
