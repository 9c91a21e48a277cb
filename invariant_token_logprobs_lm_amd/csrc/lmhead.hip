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
// H, both read K-contiguous. A workgroup owns one token block and one
// vocabulary slice of kTilesPerSlice tiles and walks the slice's tiles in
// ascending order; after each tile its lanes fold the tile into a running
// (max, sum of exp) per token and pick out z[t, y_t] if y_t falls in the
// tile. The logits never leave registers. At the end of the slice the two
// lane halves and the two wavefronts that share a token are merged in a
// fixed order and one (max, sumexp) pair per (slice, token) is written.
// Kernel 2 (lse_combine) merges a token's slice partials in slice order.
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

#include "device_common.h"
#include "itl_config.h"
#include "itl_launch.h"

namespace itl {

namespace {

// One 16-byte fragment per lane and operand feeds one K sub-step.
template <int kDtype>
struct Mma;

template <>
struct Mma<0> {  // bf16: 8 elements per lane, k16 per instruction
  __device__ static __forceinline__ void step(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

template <>
struct Mma<1> {  // fp32: 4 elements per lane; instruction j takes element j (k2 each)
  __device__ static __forceinline__ void step(floatx16& acc, uint4 a, uint4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// LDS tile: 256 rows x 8 chunks of 16 bytes. Chunk c of row r is stored at
// position c ^ (r & 7), so the eight lanes that read one logical chunk of
// eight consecutive rows hit eight different bank groups.
constexpr int kTileChunks = kBV * (kRowBytes / 16);

template <int kDtype>
__global__ __launch_bounds__(kThreads, 1) void lmhead_lse_partial_kernel(
    const char* __restrict__ H, const char* __restrict__ W, const int32_t* __restrict__ tokens, int n_tok,
    int row_bytes, int vocab, int n_slices, float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 lds[2][2][kTileChunks];  // [stage][0 = W tile, 1 = H block][chunk]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave & 1;   // which 128 vocabulary rows of the tile
  const int wt = wave >> 1;  // which 128 tokens of the block
  const int half = lane >> 5;
  const int col = lane & 31;

  const int slice = blockIdx.x % n_slices;
  const int tb = blockIdx.x / n_slices;
  const int t0 = tb * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice * kTilesPerSlice;
  const int tile_end = min(tile_begin + kTilesPerSlice, n_vt);
  const int nks = row_bytes / kRowBytes;

  // Loader mapping: thread -> (row = tid/8 + 32 j, chunk = tid % 8), j < 8.
  const int ld_row = tid >> 3;
  const int ld_col = tid & 7;
  const int st_base = ld_row * 8 + (ld_col ^ (ld_row & 7));
  uint32_t voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) voff[j] = (uint32_t)(ld_row + 32 * j) * (uint32_t)row_bytes + ld_col * 16;

  const int h_rows = min(kBT, n_tok - t0);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(H + (size_t)t0 * row_bytes, (uint32_t)h_rows * row_bytes);
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return make_rsrc(W + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };

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

  // Prologue: the slice's first K step into stage 0.
  __amdgpu_buffer_rsrc_t wr = w_rsrc(tile_begin);
  uint4 ra[8], rb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ra[j] = buffer_load16(wr, voff[j], 0);
    rb[j] = buffer_load16(hr, voff[j], 0);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lds[0][0][st_base + 256 * j] = ra[j];
    lds[0][1][st_base + 256 * j] = rb[j];
  }
  __syncthreads();

  int stage = 0;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const bool more_tiles = tile + 1 < tile_end;
    const __amdgpu_buffer_rsrc_t wr_next = more_tiles ? w_rsrc(tile + 1) : wr;

    floatx16 acc[4][4];
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = floatx16{};

    for (int ks = 0; ks < nks; ++ks) {
      // Prefetch the next K step (the next tile's first after the last one).
      // The loads and stores are unconditional: after the slice's last step
      // they re-read a valid step into the idle stage, which nobody reads.
      const bool in_tile = ks + 1 < nks;
      const __amdgpu_buffer_rsrc_t wn = in_tile ? wr : wr_next;
      const uint32_t koff = in_tile ? (uint32_t)(ks + 1) * kRowBytes : 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ra[j] = buffer_load16(wn, voff[j] + koff, 0);
        rb[j] = buffer_load16(hr, voff[j] + koff, 0);
      }

      // 4 K sub-steps of 32 bytes per row from the current stage.
      const uint4* sw = lds[stage][0];
      const uint4* sh = lds[stage][1];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int pc = (kk * 2 + half) ^ (lane & 7);
        uint4 a[4], b[4];
#pragma unroll
        for (int bm = 0; bm < 4; ++bm) a[bm] = sw[(wv * 128 + bm * 32 + col) * 8 + pc];
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) b[bn] = sh[(wt * 128 + bn * 32 + col) * 8 + pc];
#pragma unroll
        for (int bm = 0; bm < 4; ++bm)
#pragma unroll
          for (int bn = 0; bn < 4; ++bn) Mma<kDtype>::step(acc[bm][bn], a[bm], b[bn]);
      }

      {
        uint4* dw = lds[stage ^ 1][0];
        uint4* dh = lds[stage ^ 1][1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          dw[st_base + 256 * j] = ra[j];
          dh[st_base + 256 * j] = rb[j];
        }
      }
      __syncthreads();
      stage ^= 1;
    }

    // Tile epilogue: fold this tile's logits into the running state, one
    // token column (64 logits per lane) at a time.
    const int vw = tile * kBV + wv * 128;  // first vocabulary row of this wavefront
    const bool partial = tile * kBV + kBV > vocab;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      float z[64];
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[bm * 16 + i] = acc[bm][bn][i];

      // Register q = 16 bm + i of this lane holds vocabulary row
      // vw + 32 bm + 8 (i / 4) + 4 half + (i % 4).
      const int o = y[bn] - vw;
      if (o >= 0 && o < 128) {
        const int r = o & 31;
        if (((r >> 2) & 1) == half) {
          const int idx = (o >> 5) * 16 + ((r >> 3) << 2) + (r & 3);
          float v = 0.0f;
#pragma unroll
          for (int q = 0; q < 64; ++q) v = (q == idx) ? z[q] : v;
          zy[bn] = v;
          found[bn] = true;
        }
      }
      if (partial) {
#pragma unroll
        for (int q = 0; q < 64; ++q) {
          const int v = vw + (q >> 4) * 32 + ((q & 15) >> 2) * 8 + half * 4 + (q & 3);
          if (v >= vocab) z[q] = -INFINITY;
        }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int q = 0; q < 64; ++q) tmax = fmaxf(tmax, z[q]);
      const float mnew = fmaxf(mrun[bn], tmax);
      if (mnew != -INFINITY) {
        // (z - m) is exactly 0 for the maximum, so its term is exactly 1
        // and the final sum is >= 1: logprob <= 0 holds in fp32.
        float s[4];
#pragma unroll
        for (int bm = 0; bm < 4; ++bm) {
          s[bm] = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) s[bm] += fast_exp2((z[bm * 16 + i] - mnew) * kLog2e);
        }
        const float tsum = (s[0] + s[1]) + (s[2] + s[3]);
        srun[bn] = srun[bn] * fast_exp2((mrun[bn] - mnew) * kLog2e) + tsum;
        mrun[bn] = mnew;
      }
    }
    wr = wr_next;
  }

  // Slice end. Lanes l and l^32 hold the same tokens (different rows).
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const float m2 = __shfl_xor(mrun[bn], 32, 64);
    const float s2 = __shfl_xor(srun[bn], 32, 64);
    lse_merge(mrun[bn], srun[bn], m2, s2);
    if (found[bn]) zy_out[t0 + wt * 128 + bn * 32 + col] = zy[bn];
  }
  // Wavefronts wv = 0 and wv = 1 hold the same tokens; merge through LDS.
  float2* xch = reinterpret_cast<float2*>(&lds[0][0][0]);
  if (wv == 1 && half == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) xch[wt * 128 + bn * 32 + col] = make_float2(mrun[bn], srun[bn]);
  }
  __syncthreads();
  if (wv == 0 && half == 0) {
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int tok = t0 + wt * 128 + bn * 32 + col;
      const float2 o = xch[wt * 128 + bn * 32 + col];
      float m = mrun[bn], s = srun[bn];
      lse_merge(m, s, o.x, o.y);
      if (tok < n_tok) part[(size_t)slice * n_tok + tok] = make_float2(m, s);
    }
  }
}

// Per token: merge the slice partials in ascending slice order.
__global__ __launch_bounds__(256) void lse_combine_kernel(const float2* __restrict__ part,
                                                          const float* __restrict__ zy, int n_tok,
                                                          int n_slices, float* __restrict__ logprob,
                                                          float* __restrict__ lse) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float M = -INFINITY;
  for (int s = 0; s < n_slices; ++s) M = fmaxf(M, part[(size_t)s * n_tok + t].x);
  float S = 0.0f;
  for (int s = 0; s < n_slices; ++s) {
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
  return align256((size_t)n_slices(vocab) * (size_t)n_tok * sizeof(float2)) + align256((size_t)n_tok * sizeof(float));
}

hipError_t launch_lmhead_logprob(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                 const int32_t* tokens, float* logprob, float* lse, void* workspace,
                                 hipStream_t stream) {
  const int es = dtype == 0 ? 2 : 4;
  const int row_bytes = d * es;
  const int S = n_slices(vocab);
  const int ntb = (int)ceil_div(n_tok, kBT);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)S * (size_t)n_tok * sizeof(float2)));
  const dim3 grid((unsigned)ntb * (unsigned)S);
  if (dtype == 0)
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<0>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, S, part, zy);
  else
    hipLaunchKernelGGL(lmhead_lse_partial_kernel<1>, grid, dim3(kThreads), 0, stream, static_cast<const char*>(H),
                       static_cast<const char*>(W), tokens, n_tok, row_bytes, vocab, S, part, zy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)ceil_div(n_tok, 256)), dim3(256), 0, stream, part, zy, n_tok,
                     S, logprob, lse);
  return hipGetLastError();
}

}  // namespace itl
