// Gradient of the REINFORCE Zero loss through the LM head ("vLLM says aligned
// kernels make asynchronous RL stable at lag 64", section "REINFORCE Zero
// removes the mismatch first": plain REINFORCE, so dloss/dlogprob_t = coef[t]
// and the logprob is a log-softmax of the head's logits):
//
//   G[t, v] = dloss/dz[t, v] = coef[t] (onehot(y_t)[v] - p[t, v]),
//   p[t, v] = exp(z[t, v] - lse[t])
//   dH = G W,   dW = G^T H
//
// G splits into a dense part -coef[t] p[t, v] and one sampled entry
// +coef[t] per token. The sampled entries are applied exactly, in fp32:
//   dH[t]    += coef[t] W[y_t]
//   dW[v]     = sum over tokens t with y_t = v of coef[t] H[t]
// the latter (sampled.hip) in an order fixed by the tokens of id v alone,
// before any dense part is added.
// The dense part g[t, v] = -coef[t] p[t, v] is formed in the head's dtype
// (bf16 for bf16 heads: the MFMA operand) and contracted on the matrix cores
// with the eight-wavefront tile engine (tile_engine8.h), one chunk of
// kBwdChunk tokens at a time:
//   1. dlogits: z recomputed by the forward's contraction, g written twice:
//      token-major Gd [chunk, Vpad] (for dH) and vocabulary-major GdT
//      [Vpad, chunk] (for dW); padding rows and columns hold zeros.
//      When the caller kept the forward's logits (fp32, the same bits the
//      recompute gives), g is formed from them instead: one pass over HBM in
//      place of a full contraction, with g's arithmetic unchanged, so dH and
//      dW have the same bits either way.
//   2. dH rows of the chunk = Gd W^T-rows (K = Vpad ascending) + sampled term.
//   3. dW += GdT H^T-rows of the chunk (K = the chunk's tokens ascending).
// dW starts as zeros plus the sampled term; chunks are added in token order.
// Every sum has a fixed order (no atomics, no split-K): run-to-run bitwise
// deterministic. The transposed copies W^T [d, Vpad] and H^T [d, chunk] make
// every contraction "both operands K-contiguous", the form the engine runs.

#include <algorithm>

#include "itl_launch.h"
#include "tile_engine.h"
#include "tile_engine8.h"

namespace itl {

namespace {

constexpr int kBwdChunk = kBwdChunkTokens;  // tokens per chunk (a multiple of kBT)
static_assert(kBwdChunk % kBT == 0, "chunks hold whole token blocks");

template <int kDtype>
struct Elem;
template <>
struct Elem<0> {
  using T = uint16_t;  // bf16 bits
  static constexpr int kSize = 2;
  __device__ static __forceinline__ float to_f(T x) { return __uint_as_float((uint32_t)x << 16); }
  // Round to nearest even (inputs here are finite).
  __device__ static __forceinline__ T from_f(float f) {
    const uint32_t u = __float_as_uint(f);
    return (T)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
};
template <>
struct Elem<1> {
  using T = float;
  static constexpr int kSize = 4;
  __device__ static __forceinline__ float to_f(T x) { return x; }
  __device__ static __forceinline__ T from_f(float f) { return f; }
};

long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

// out[c, r] = in[r, c] for r < rows, 0 for rows <= r < out_cols; c < cols.
// in: [rows, cols] row-major (row stride in_stride elements); out: [cols,
// out_cols] row-major. 64 x 64 element tiles through LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, long long in_stride, int rows,
                                                        int cols, T* __restrict__ out, int out_cols) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? in[(size_t)r * in_stride + c] : T(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < out_cols) out[(size_t)c * out_cols + r] = tile[tx][i];
  }
}

// Workgroup order shared by the three contractions: the grid is n_fast x
// n_slow blocks; super-bands of kBwdSuperBand fast indices are walked with the
// slow index outer, so the workgroups an XCD runs together share operands.
__device__ __forceinline__ void band_order(int b, int n_fast, int n_slow, int& fast, int& slow) {
  const int band = b / (kBwdSuperBand * n_slow);
  const int first = band * kBwdSuperBand;
  const int nb = min(kBwdSuperBand, n_fast - first);
  const int rem = b - band * kBwdSuperBand * n_slow;
  slow = rem / nb;
  fast = first + rem % nb;
}

// 1. dlogits. A = W tiles (vocabulary), B = the chunk's H block (tokens); as
// in the forward, on the eight-wavefront engine. Grid: token blocks (fast) x
// vocabulary slices (slow). Lane l of wavefront (wv, tq) holds vocabulary
// rows 128 wv + 16 bm + 4 (l / 16) .. + 3 of each tile at tokens t0 + 64 tq +
// 16 bn + (l mod 16).
template <int kDtype, bool kBFar>
__global__ __launch_bounds__(kThreads8, 1) void dlogits_kernel(
    const char* __restrict__ Hc, int len, const char* __restrict__ W, int row_bytes, int vocab, int vpad,
    int n_tb, int n_slices, int group, const int32_t* __restrict__ y, const float* __restrict__ lse,
    const float* __restrict__ coef, typename Elem<kDtype>::T* __restrict__ Gd, typename Elem<kDtype>::T* __restrict__ GdT) {
  using E = Elem<kDtype>;
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes8 L = lanes8();
  int tb, grp;
  band_order(blockIdx.x, n_tb, (n_slices + group - 1) / group, tb, grp);
  const int t0 = tb * kBT;
  const int n_vt = vpad / kBV;
  const int tile_begin = slice_tile(grp * group, n_vt, n_slices);
  const int tile_end = slice_tile(min(grp * group + group, n_slices), n_vt, n_slices);
  float l2e_lse[4], negc[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int t = t0 + L.tq * 64 + bn * 16 + L.c16;
    const bool ok = t < len;
    l2e_lse[bn] = ok ? lse[t] * kLog2e : 0.0f;
    negc[bn] = ok ? -coef[t] : 0.0f;  // padding tokens get g = 0
  }
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(W + (size_t)v0 * row_bytes, (uint32_t)max(0, min(kBV, vocab - v0)) * row_bytes);
  };
  const int4v hr = rsrc_words(Hc + (size_t)t0 * row_bytes, (uint32_t)min(kBT, len - t0) * row_bytes);
  auto epilogue = [&](int tile, floatx4 (&acc)[8][4]) {
    const int vw = tile * kBV + L.wv * 128 + 4 * L.quad;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int t = t0 + L.tq * 64 + bn * 16 + L.c16;  // < chunk's padded length
#pragma unroll
      for (int bm = 0; bm < 8; ++bm) {
        const int v = vw + bm * 16;  // rows v .. v + 3
        typename E::T g[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = acc[bm][bn][r];
          const float p = fast_exp2(z * kLog2e - l2e_lse[bn]);
          g[r] = E::from_f(v + r < vocab ? negc[bn] * p : 0.0f);
          GdT[(size_t)(v + r) * kBwdChunk + t] = g[r];
        }
        if constexpr (kDtype == 0) {
          uint2 pk;
          pk.x = (uint32_t)g[0] | ((uint32_t)g[1] << 16);
          pk.y = (uint32_t)g[2] | ((uint32_t)g[3] << 16);
          *reinterpret_cast<uint2*>(Gd + (size_t)t * vpad + v) = pk;
        } else {
          *reinterpret_cast<float4*>(Gd + (size_t)t * vpad + v) = make_float4(g[0], g[1], g[2], g[3]);
        }
        if ((bm & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  run_tiles8<kDtype, kBFar>(smem, L, row_bytes, tile_begin, tile_end, row_bytes / kStepBytes, w_rsrc, hr, epilogue);
}

// 1'. dlogits from kept logits: the same g as dlogits_kernel, for a tile of
// 128 tokens x 128 vocabulary rows. z is read token-major (16 bytes per
// lane, a token row's 512 contiguous bytes per 32 lanes), g is written to
// Gd directly and to GdT through an LDS transpose (each of GdT's rows gets
// the tile's 128 tokens contiguously). Tokens at or past len and rows at or
// past vocab get g = 0, as in dlogits_kernel (their z is never read).
constexpr int kGTile = 128;

template <int kDtype>
__global__ __launch_bounds__(256) void dlogits_from_logits_kernel(
    const float* __restrict__ logits, long long ld, int len, int vocab, int vpad, const float* __restrict__ lse,
    const float* __restrict__ coef, typename Elem<kDtype>::T* __restrict__ Gd,
    typename Elem<kDtype>::T* __restrict__ GdT) {
  using E = Elem<kDtype>;
  using T = typename E::T;
  // The transposed tile: element (v, t) at row v; bf16 packs tokens 2 j and
  // 2 j + 1 into word j. One pad word per row spreads a column over banks.
  constexpr int kPack = 4 / (int)sizeof(T);  // tokens per 32-bit word
  constexpr int kRowWords = kGTile / kPack + 1;
  __shared__ uint32_t tile[kGTile * kRowWords];
  const int v0 = blockIdx.x * kGTile;
  const int t0 = blockIdx.y * kGTile;
  const int vq = threadIdx.x & 31;  // vocabulary rows v0 + 4 vq .. + 3
  const int tr = threadIdx.x >> 5;  // 0..7
  const int v = v0 + 4 * vq;
  for (int p = 0; p < kGTile / (8 * kPack); ++p) {
    T g[kPack][4];
#pragma unroll
    for (int k = 0; k < kPack; ++k) {
      const int tl = (tr + 8 * p) * kPack + k;  // token within the tile
      const int t = t0 + tl;
      if (t < len) {
        const float l2e_lse = lse[t] * kLog2e;
        const float negc = -coef[t];
        const float* row = logits + (size_t)t * (size_t)ld;
        floatx4 z;
        if (v + 3 < vocab) {
          z = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(row + v));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) z[r] = v + r < vocab ? row[v + r] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = fast_exp2(z[r] * kLog2e - l2e_lse);
          g[k][r] = E::from_f(v + r < vocab ? negc * pr : 0.0f);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) g[k][r] = E::from_f(0.0f);
      }
      if constexpr (kDtype == 0) {
        uint2 pk;
        pk.x = (uint32_t)g[k][0] | ((uint32_t)g[k][1] << 16);
        pk.y = (uint32_t)g[k][2] | ((uint32_t)g[k][3] << 16);
        *reinterpret_cast<uint2*>(Gd + (size_t)t * vpad + v) = pk;
      } else {
        *reinterpret_cast<float4*>(Gd + (size_t)t * vpad + v) = make_float4(g[k][0], g[k][1], g[k][2], g[k][3]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t w;
      if constexpr (kDtype == 0) w = (uint32_t)g[0][r] | ((uint32_t)g[1][r] << 16);
      else w = __float_as_uint(g[0][r]);
      tile[(4 * vq + r) * kRowWords + tr + 8 * p] = w;
    }
  }
  __syncthreads();
  // GdT rows v0 .. v0 + 127, tokens t0 .. t0 + 127: 16 bytes per lane.
  constexpr int kLanesPerRow = kGTile / kPack / 4;  // 16 (bf16) or 32 (fp32)
  constexpr int kRowsPerPass = 256 / kLanesPerRow;
  const int j = threadIdx.x % kLanesPerRow;
  for (int vr = threadIdx.x / kLanesPerRow; vr < kGTile; vr += kRowsPerPass) {
    const uint32_t* src = tile + vr * kRowWords + 4 * j;
    const uint4 w = make_uint4(src[0], src[1], src[2], src[3]);
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(GdT + (size_t)(v0 + vr) * kBwdChunk + t0) + 16 * j) = w;
  }
}

// 2. dH for the chunk. A = W^T tile (d rows, K = Vpad), B = Gd token block,
// on the eight-wavefront engine. Grid: token blocks (fast) x d tiles (slow).
// Lane l of wavefront (wv, tq) holds d rows 128 wv + 16 bm + 4 (l / 16) ..
// + 3 of the tile for tokens t0 + 64 tq + 16 bn + (l mod 16).
template <int kDtype, bool kBFar>
__global__ __launch_bounds__(kThreads8, 1) void dh_kernel(const char* __restrict__ WT, const char* __restrict__ Gd,
                                                         int vpad, int d, int vocab, int len, int n_tb, int n_dt,
                                                         const int32_t* __restrict__ y, const float* __restrict__ coef,
                                                         const typename Elem<kDtype>::T* __restrict__ W,
                                                         float* __restrict__ dH) {
  using E = Elem<kDtype>;
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes8 L = lanes8();
  int tb, dt;
  band_order(blockIdx.x, n_tb, n_dt, tb, dt);
  const int t0 = tb * kBT;
  const int row_bytes = vpad * E::kSize;
  auto a_rsrc = [&](int tile) {
    const int k0 = tile * kBV;
    return rsrc_words(WT + (size_t)k0 * row_bytes, (uint32_t)min(kBV, d - k0) * row_bytes);
  };
  const int4v br = rsrc_words(Gd + (size_t)t0 * row_bytes, (uint32_t)min(kBT, len - t0) * row_bytes);
  auto epilogue = [&](int tile, floatx4 (&acc)[8][4]) {
    const int kw = tile * kBV + L.wv * 128 + 4 * L.quad;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int t = t0 + L.tq * 64 + bn * 16 + L.c16;
      const bool ok = t < len;
      const int yr = ok ? y[t] : 0;
      const bool yok = (unsigned)yr < (unsigned)vocab;  // an invalid id contributes no sampled term
      const float c = ok && yok ? coef[t] : 0.0f;
      const int yt = yok ? yr : 0;
#pragma unroll
      for (int bh = 0; bh < 2; ++bh) {
        // Four blocks' groups of 4 W[y] values, loaded together.
        float wyv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = kw + (4 * bh + j) * 16;  // d rows k .. k + 3 (d is a multiple of 64)
          const typename E::T* wy = W + (size_t)yt * d + (k < d ? k : 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) wyv[j][r] = E::to_f(wy[r]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int bm = 4 * bh + j;
          const int k = kw + bm * 16;
          if (ok && k < d) {
            const floatx4& o = acc[bm][bn];
            float4 out;
            out.x = o[0] + c * wyv[j][0];
            out.y = o[1] + c * wyv[j][1];
            out.z = o[2] + c * wyv[j][2];
            out.w = o[3] + c * wyv[j][3];
            *reinterpret_cast<float4*>(dH + (size_t)t * d + k) = out;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  run_tiles8<kDtype, kBFar>(smem, L, row_bytes, dt, dt + 1, row_bytes / kStepBytes, a_rsrc, br, epilogue);
}

// 3. dW += the chunk's part. A = GdT vocabulary tile (K = chunk tokens), B =
// H^T d block, on the eight-wavefront engine. Grid: vocabulary tiles (fast)
// x d tiles (slow). Lane l of wavefront (wv, tq) holds vocabulary rows
// 128 wv + 16 bm + 4 (l / 16) .. + 3 of the tile at d column k0 + 64 tq +
// 16 bn + (l mod 16).
template <int kDtype, bool kBFar>
__global__ __launch_bounds__(kThreads8, 1) void dw_kernel(const char* __restrict__ GdT, const char* __restrict__ HT,
                                                         int kpad, int vocab, int d, int n_vt, int n_dt,
                                                         float* __restrict__ dW) {
  using E = Elem<kDtype>;
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes8 L = lanes8();
  int vt, dt;
  band_order(blockIdx.x, n_vt, n_dt, vt, dt);
  const int row_bytes = kBwdChunk * E::kSize;
  const int k0 = dt * kBT;
  auto a_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(GdT + (size_t)v0 * row_bytes, (uint32_t)kBV * row_bytes);
  };
  const int4v br = rsrc_words(HT + (size_t)k0 * row_bytes, (uint32_t)min(kBT, d - k0) * row_bytes);
  auto epilogue = [&](int tile, floatx4 (&acc)[8][4]) {
    const int vw = tile * kBV + L.wv * 128 + 4 * L.quad;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int k = k0 + L.tq * 64 + bn * 16 + L.c16;
#pragma unroll
      for (int bh = 0; bh < 2; ++bh) {
        // Four blocks' 16 dW values of this lane's column k, read together,
        // then updated and written back.
        float old[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = vw + (4 * bh + j) * 16 + r;
            old[j][r] = v < vocab && k < d ? dW[(size_t)v * d + k] : 0.0f;
          }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = vw + (4 * bh + j) * 16 + r;
            if (v < vocab && k < d) dW[(size_t)v * d + k] = old[j][r] + acc[4 * bh + j][bn][r];
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  run_tiles8<kDtype, kBFar>(smem, L, row_bytes, vt, vt + 1, kpad * E::kSize / kStepBytes, a_rsrc, br, epilogue);
}

// Workspace layout of the backward (each region 256-byte aligned).
struct BwdLayout {
  size_t wt, ht, gd, gdt, sampled, total;
};

BwdLayout bwd_layout(long long n_tok, long long d, long long vocab, int es) {
  BwdLayout L{};
  const long long vpad = round_up(vocab, kBV);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.wt = take((size_t)d * vpad * es);
  L.ht = take((size_t)d * kBwdChunk * es);
  L.gd = take((size_t)kBwdChunk * vpad * es);
  L.gdt = take((size_t)vpad * kBwdChunk * es);
  L.sampled = take(sampled_dw_workspace_bytes(n_tok, d, vocab));
  L.total = off;
  return L;
}

template <int kDtype>
hipError_t run_backward(const void* H, const void* W, int n_tok, int d, int vocab, const int32_t* tokens,
                        const float* lse, const float* coef, const float* logits, long long ld, float* dH,
                        float* dW, void* workspace, hipStream_t stream) {
  using E = Elem<kDtype>;
  using T = typename E::T;
  const int es = E::kSize;
  const int vpad = (int)round_up(vocab, kBV);
  const BwdLayout Ly = bwd_layout(n_tok, d, vocab, es);
  char* ws = static_cast<char*>(workspace);
  T* WT = reinterpret_cast<T*>(ws + Ly.wt);
  T* HT = reinterpret_cast<T*>(ws + Ly.ht);
  T* Gd = reinterpret_cast<T*>(ws + Ly.gd);
  T* GdT = reinterpret_cast<T*>(ws + Ly.gdt);
  const T* Hp = static_cast<const T*>(H);
  const T* Wp = static_cast<const T*>(W);
  hipError_t e;
#define ITL_CHECK_LAUNCH()           \
  do {                               \
    e = hipGetLastError();           \
    if (e != hipSuccess) return e;   \
  } while (0)

  // dW = the sampled term (zeros in rows no token samples).
  e = launch_sampled_dw(H, kDtype, n_tok, d, vocab, tokens, coef, dW, ws + Ly.sampled, stream);
  if (e != hipSuccess) return e;
  if (n_tok == 0) return hipSuccess;

  // W^T [d, Vpad], zero-padded.
  hipLaunchKernelGGL(transpose_kernel<T>, dim3((unsigned)ceil_div(vpad, 64), (unsigned)ceil_div(d, 64)), dim3(256), 0,
                     stream, Wp, (long long)d, vocab, d, WT, vpad);
  ITL_CHECK_LAUNCH();

  const int S = n_slices(vpad);
  const int G = std::max(1, kTilesPerGroup * S / (vpad / kBV));  // about kTilesPerGroup tiles per workgroup
  const int n_groups = (S + G - 1) / G;
  const int n_dt = (int)ceil_div(d, kBT);
  const int n_vt = vpad / kBV;
  const int row_bytes = d * es;
  // Load schedule (no effect on the arithmetic): the recomputing dlogits
  // kernel follows the forward's rule (its token block two K steps ahead
  // once the K loop is long); dH stages its dlogits block two ahead on long
  // loops too (measured 1.5 % faster at 2020 K steps); dW keeps its
  // vocabulary tile two ahead (the other way measured 3 % slower).
  const bool dl_far = row_bytes / kStepBytes > kNearBMaxSteps;
  const bool dh_far = vpad * es / kStepBytes > kNearBMaxSteps;
  for (int c0 = 0; c0 < n_tok; c0 += kBwdChunk) {
    const int len = std::min(kBwdChunk, n_tok - c0);
    const int kpad = (int)round_up(len, kBT);
    const int n_tb = kpad / kBT;
    const char* Hc = static_cast<const char*>(H) + (size_t)c0 * row_bytes;
    if (logits)
      hipLaunchKernelGGL(dlogits_from_logits_kernel<kDtype>, dim3((unsigned)(vpad / kGTile), (unsigned)(kpad / kGTile)),
                         dim3(256), 0, stream, logits + (size_t)c0 * (size_t)ld, ld, len, vocab, vpad, lse + c0,
                         coef + c0, Gd, GdT);
    else
      hipLaunchKernelGGL((dl_far ? dlogits_kernel<kDtype, true> : dlogits_kernel<kDtype, false>),
                         dim3((unsigned)(n_tb * n_groups)), dim3(kThreads8), 0, stream, Hc,
                         len, static_cast<const char*>(W), row_bytes, vocab, vpad, n_tb, S, G, tokens + c0, lse + c0,
                         coef + c0, Gd, GdT);
    ITL_CHECK_LAUNCH();
    hipLaunchKernelGGL((dh_far ? dh_kernel<kDtype, true> : dh_kernel<kDtype, false>),
                       dim3((unsigned)(n_tb * n_dt)), dim3(kThreads8), 0, stream,
                       reinterpret_cast<const char*>(WT), reinterpret_cast<const char*>(Gd), vpad, d, vocab, len, n_tb, n_dt,
                       tokens + c0, coef + c0, Wp, dH + (size_t)c0 * d);
    ITL_CHECK_LAUNCH();
    // H^T of the chunk [d, kBwdChunk], tokens past len zero.
    hipLaunchKernelGGL(transpose_kernel<T>, dim3((unsigned)(kBwdChunk / 64), (unsigned)ceil_div(d, 64)), dim3(256), 0,
                       stream, Hp + (size_t)c0 * d, (long long)d, len, d, HT, kBwdChunk);
    ITL_CHECK_LAUNCH();
    hipLaunchKernelGGL((dw_kernel<kDtype, false>),
                       dim3((unsigned)(n_vt * n_dt)), dim3(kThreads8), 0, stream,
                       reinterpret_cast<const char*>(GdT), reinterpret_cast<const char*>(HT), kpad, vocab, d, n_vt,
                       n_dt, dW);
    ITL_CHECK_LAUNCH();
  }
#undef ITL_CHECK_LAUNCH
  return hipSuccess;
}

}  // namespace

size_t backward_workspace_bytes(long long n_tok, long long d, long long vocab, int dtype) {
  return bwd_layout(n_tok, d, vocab, dtype == 0 ? 2 : 4).total;
}

hipError_t launch_reinforce_zero_backward(const void* H, const void* W, int dtype, int n_tok, int d, int vocab,
                                          const int32_t* tokens, const float* lse, const float* coef,
                                          const float* logits, long long ld, float* dH, float* dW, void* workspace,
                                          hipStream_t stream) {
  if (dtype == 0)
    return run_backward<0>(H, W, n_tok, d, vocab, tokens, lse, coef, logits, ld, dH, dW, workspace, stream);
  return run_backward<1>(H, W, n_tok, d, vocab, tokens, lse, coef, logits, ld, dH, dW, workspace, stream);
}

}  // namespace itl
