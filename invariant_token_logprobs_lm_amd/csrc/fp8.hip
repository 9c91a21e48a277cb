// FP8 (E4M3) head: per-row quantisation and the sampled-token logprob from
// E4M3 operands on the FP8 matrix cores.
//
// "vLLM says aligned kernels make asynchronous RL stable at lag 64", section
// "Zero mismatch expands to newer models": the consistent path of the newest
// model runs FP8 (and MXFP4) weights; the aligned logprob must then come from
// the low-precision head with the same invariance. Readings (the pages give
// no format details): OCP E4M3 ("E4M3FN": bias 7, no infinities, max 448),
// one float32 scale per row (a vocabulary row of W, a token row of H):
//   scale[r] = amax_r / 448 (1 for an all-zero row), code = E4M3(x / scale)
// with the division in float32 (correctly rounded) and the conversion
// rounding to nearest, ties to even, saturating at +-448. The conversion is
// written out from the format's fields (exact power-of-two scaling and a
// round-to-nearest-even to 3 mantissa bits), not left to a conversion
// instruction, so the codes are a fixed function of the input bits.
//   z[t, v] = (acc[t, v] * w_scale[v]) * h_scale[t],
//   acc[t, v] = sum_k E4M3(Hq[t, k]) E4M3(Wq[v, k]) (fp32, fixed K order)
// then the same online log-sum-exp, slice partials and combine as the bf16
// head (shared fold, lse_fold.h). Calls of at most 64 tokens run narrow
// kernels that perform, per token, the same matrix-core instructions on the
// same fragments and the same fold, so a token's logprob does not depend on
// the batch.

#include "itl_launch.h"
#include "lse_fold.h"
#include "tile_engine.h"
#include "tile_engine8.h"

namespace itl {

namespace {

// E4M3 code of a finite float32, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 512.0f);  // subnormal multiples of 2^-9; 8 is the smallest normal (0x08)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // a >= 2^-6 is a normal float32
    float r = rintf(ldexpf(a, 3 - e));                       // 1.mmm x 8, in [8, 16]
    if (r == 16.0f) {
      e += 1;
      r = 8.0f;
    }
    if (e > 8 || (e == 8 && r > 14.0f)) code = 0x7Eu;  // beyond 448 = 1.75 x 2^8: saturate
    else code = ((uint32_t)(e + 7) << 3) | ((uint32_t)r - 8u);
  }
  return sign | code;
}

template <int kDtype>
__device__ __forceinline__ float load_elem(const void* X, size_t i) {
  if constexpr (kDtype == 0) return __uint_as_float((uint32_t)static_cast<const uint16_t*>(X)[i] << 16);
  else return static_cast<const float*>(X)[i];
}

// One wavefront per row: amax by a butterfly of maxima (exact, so any tree
// gives the same value), then the codes. Rows of up to 512 16-byte chunks
// (4096 bf16 / 2048 fp32 values) are read once, 16 bytes per lane per load,
// and kept in registers for the second pass (when X is 16-byte and Xq
// 8-byte aligned); other rows are read twice, 4 values per lane per step.
// Both paths compute every code the same way.
template <int kDtype>
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const void* __restrict__ X, long long n_rows, int d,
                                                                uint8_t* __restrict__ Xq, float* __restrict__ scale) {
  constexpr int kPerChunk = kDtype == 0 ? 8 : 4;  // values per 16-byte chunk
  constexpr int kMaxChunks = 8;                   // chunks a lane keeps in registers
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const size_t base = (size_t)row * d;
  const int n_chunks = d / kPerChunk;  // d is a multiple of 128
  auto value = [&](const uint4& v, int j) {
    const uint32_t w = (&v.x)[kDtype == 0 ? j >> 1 : j];
    if constexpr (kDtype == 0) return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
    else return __uint_as_float(w);
  };
  const bool aligned = ((reinterpret_cast<uintptr_t>(X) & 15) | (reinterpret_cast<uintptr_t>(Xq) & 7)) == 0;
  if (aligned && n_chunks <= 64 * kMaxChunks) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(X) + base * (kDtype == 0 ? 2 : 4));
    uint4 v[kMaxChunks];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int idx = lane + 64 * c;
      v[c] = idx < n_chunks ? src[idx] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kPerChunk; ++j) amax = fmaxf(amax, fabsf(value(v[c], j)));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (lane == 0) scale[row] = s;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int idx = lane + 64 * c;
      if (idx >= n_chunks) break;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < kPerChunk; ++j) {
        const uint32_t code = e4m3_rne(__fdiv_rn(value(v[c], j), s));
        if (j < 4) lo |= code << (8 * j);
        else hi |= code << (8 * (j - 4));
      }
      if constexpr (kDtype == 0) *reinterpret_cast<uint2*>(Xq + base + (size_t)idx * 8) = make_uint2(lo, hi);
      else *reinterpret_cast<uint32_t*>(Xq + base + (size_t)idx * 4) = lo;
    }
    return;
  }
  float amax = 0.0f;
  for (int k = lane * 4; k < d; k += 256)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(load_elem<kDtype>(X, base + k + j)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (lane == 0) scale[row] = s;
  for (int k = lane * 4; k < d; k += 256) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) packed |= e4m3_rne(__fdiv_rn(load_elem<kDtype>(X, base + k + j), s)) << (8 * j);
    *reinterpret_cast<uint32_t*>(Xq + base + k) = packed;
  }
}

// z = (z * w) * h, element by element, each product rounded to fp32: the
// logits of four rows of one token from their accumulators, the rows'
// scales w and the token's scale h (the wide and the narrow kernels both use
// it, so their logits have the same bits).
__device__ __forceinline__ void scale_logits(floatx4& z, const float4& w, float h) {
  const floatx4 wv = {w.x, w.y, w.z, w.w};
  z = (z * wv) * h;
}

// The bf16 head's wide partial kernel with E4M3 operands, on the
// eight-wavefront engine's FP8 schedule (run_tiles8<2>): the same workgroup
// order, slices, lane layout and fold (fold_column16); the epilogue scales
// each accumulator by its vocabulary row's and its token's scale,
//   z = (acc * w_scale[v]) * h_scale[t],
// before folding. The wavefront's 128 row scales of a tile come into LDS by
// the engine's side load (two 4-byte-per-lane loads into the wavefront's own
// rows of a free slot), so the epilogue reads them without waiting on the
// operand loads in flight.
template <bool kBFar>
__global__ __launch_bounds__(kThreads8, 1) void lmhead_fp8_partial8_kernel(
    const uint8_t* __restrict__ Hq, const float* __restrict__ h_scale, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const int32_t* __restrict__ tokens, int n_tok, int d, int vocab, int n_tb,
    int n_slices, int group, float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes8 L = lanes8();
  const int wv = L.wv, tq = L.tq, quad = L.quad, c16 = L.c16;
  const int S = n_slices;
  const WideWork work = wide_work(blockIdx.x, n_tb, S, group);
  const int t0 = work.tb * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(work.slice_first, n_vt, S);
  const int tile_end = slice_tile(work.slice_end, n_vt, S);
  const int row_bytes = d;
  const int nks = row_bytes / kStepBytes;

  Col16 c[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int tok = t0 + tq * 64 + bn * 16 + c16;
    c[bn] = Col16{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f};
  }
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(Wq + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  const int4v hr = rsrc_words(Hq + (size_t)t0 * row_bytes, (uint32_t)min(kBT, n_tok - t0) * row_bytes);
  // Side load: lane l fetches the scales of rows vw + l and vw + 64 + l (vw
  // = the wavefront's first row of the tile) to bytes 4 l and 256 + 4 l of
  // its LDS rows, so that row r of the 128 sits at float r, and the scale of
  // token t0 + 64 tq + l to byte 512 + 4 l (kept in registers across the K
  // loop, the token scales would push the loop's operands out of them).
  // Rows past the vocabulary and tokens past n_tok read 0 through the
  // buffers' ranges.
  const int4v ws_words = rsrc_words(w_scale, (uint32_t)vocab * 4u);
  const int4v hs_words = rsrc_words(h_scale + t0, (uint32_t)min(kBT, n_tok - t0) * 4u);
  int scale_chunk = 0;
  auto side = [&](int tile, uint32_t lds, int chunk) {
    const uint32_t off = (uint32_t)(tile * kBV + wv * 128 + L.lane) * 4u;
    dma4(ws_words, off, 0u, lds);
    dma4(ws_words, off + 256u, 0u, lds + 256u);
    dma4(hs_words, (uint32_t)(tq * 64 + L.lane) * 4u, 0u, lds + 512u);
    scale_chunk = chunk;
  };

  int slice = work.slice_first;
  int slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
  auto epilogue = [&](int tile, floatx4 (&acc)[8][4]) {
    const int vw = tile * kBV + wv * 128;
    // the side load landed (the engine issued kDma8PerWave loads after it)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDma8PerWave) : "memory");
    // The logits, in place: acc[bm][bn] row 16 bm + 4 quad + i, token
    // 64 tq + 16 bn + c16 (scales at floats 16 bm + 4 quad + i and
    // 128 + 16 bn + c16 of the side rows).
    {
      const float4* sw = reinterpret_cast<const float4*>(smem) + scale_chunk + quad;
      const float* sh = reinterpret_cast<const float*>(smem) + scale_chunk * 4 + 128 + c16;
      float hs[4];
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) hs[bn] = sh[bn * 16];
#pragma unroll
      for (int bm = 0; bm < 8; ++bm) {
        const float4 w = sw[4 * bm];
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) scale_logits(acc[bm][bn], w, hs[bn]);
      }
    }
    int lt = L.lane;
    asm volatile("" : "+v"(lt));  // (per-lane addresses formed here, not kept across the K loop)
    lt = tq * 64 + (lt & 15);
    auto fold_tile = [&](auto partial, auto pick) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        floatx4 z[8];
#pragma unroll
        for (int bm = 0; bm < 8; ++bm) z[bm] = acc[bm][bn];
        if constexpr (decltype(pick)::value) pick_sampled(c[bn], z, vw, quad, zy_out + (t0 + lt + bn * 16));
        fold_column16(c[bn], z, vw, quad, vocab, partial);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    bool mine = false;
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      int y = c[bn].y;
      asm volatile("" : "+v"(y));
      mine = mine || (unsigned)(y - vw) < 128u;
    }
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{}, std::true_type{});
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
      asm volatile("" : "+s"(Sx));
      slice_last_tile = slice_tile(slice + 1, n_vt, Sx) - 1;
    }
  };
  run_tiles8<2, kBFar>(smem, L, row_bytes, tile_begin, tile_end, nks, w_rsrc, hr, epilogue, side);
}

// Decode-shaped FP8 calls (at most kNarrow128MaxTokens tokens): kBRows-token
// blocks (64, or one block of 128 for calls of 65 to 128 tokens), one
// workgroup per (token block, slice), the narrow engine's FP8 steps
// (run_tiles_narrow<2, kBRows>). Lane l of wavefront (wv, wt) holds tokens
// t0 + (kBRows / 2) wt + 16 bn + (l mod 16) (bn < kBRows / 32) against the
// same W rows, with the same MFMA sequence, scales and fold as
// lmhead_fp8_partial8_kernel, so the partials and logprobs have the same
// bits. The row scales of up to kNarrowScaleTiles tiles are fetched at a
// time into two registers per tile (lane l: rows vw + l, vw + 64 + l) and
// spread to the lanes that need them with ds_bpermute; the first group
// before the first operand load, so that waiting for them waits for nothing
// else.
constexpr int kNarrowScaleTiles = 4;

template <int kBRows>
__global__ __launch_bounds__(kThreads, 1) void lmhead_fp8_partial_narrow_kernel(
    const uint8_t* __restrict__ Hq, const float* __restrict__ h_scale, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, const int32_t* __restrict__ tokens, int n_tok, int d, int vocab, int n_slices,
    float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes L = lanes();
  const int wv = L.wv, wt = L.wt, quad = L.lane >> 4, c16 = L.lane & 15;
  const int S = n_slices;
  const int slice = blockIdx.x % S;
  constexpr int kBN = kBRows / 32;  // token columns per lane
  constexpr int kWaveToks = kBRows / 2;
  const int t0 = (blockIdx.x / S) * kBRows;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(slice, n_vt, S);
  const int tile_end = slice_tile(slice + 1, n_vt, S);
  const int row_bytes = d;
  const int nks = row_bytes / kStepBytes;
  Col16 c[kBN];
  float hs[kBN];
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * kWaveToks + bn * 16 + c16;
    c[bn] = Col16{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f};
    hs[bn] = tok < n_tok ? h_scale[tok] : 0.0f;
  }
  float g_lo[kNarrowScaleTiles], g_hi[kNarrowScaleTiles];
  // Scales of tiles first .. first + kNarrowScaleTiles - 1 (0 past the
  // slice or the vocabulary), waited for here.
  auto load_scales = [&](int first) {
#pragma unroll
    for (int j = 0; j < kNarrowScaleTiles; ++j) {
      const int row = (first + j) * kBV + wv * 128 + L.lane;
      const bool in = first + j < tile_end;
      g_lo[j] = in && row < vocab ? w_scale[row] : 0.0f;
      g_hi[j] = in && row + 64 < vocab ? w_scale[row + 64] : 0.0f;
    }
    asm volatile("" ::"v"(g_lo[0]), "v"(g_lo[1]), "v"(g_lo[2]), "v"(g_lo[3]), "v"(g_hi[0]), "v"(g_hi[1]),
                 "v"(g_hi[2]), "v"(g_hi[3]));
#pragma unroll
    for (int bn = 0; bn < kBN; ++bn) asm volatile("" ::"v"(c[bn].y), "v"(hs[bn]));
  };
  static_assert(kNarrowScaleTiles == 4, "load_scales waits for four tiles' scales");
  load_scales(tile_begin);

  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(Wq + (size_t)v0 * row_bytes, (uint32_t)min(kBV, vocab - v0) * row_bytes);
  };
  const int4v hr = rsrc_words(Hq + (size_t)t0 * row_bytes, (uint32_t)min(kBRows, n_tok - t0) * row_bytes);
  auto epilogue = [&](int tile, floatx4 (&acc)[8][kBN]) {
    const int vw = tile * kBV + wv * 128;
    const int j = (tile - tile_begin) % kNarrowScaleTiles;
    const float lo = j == 0 ? g_lo[0] : j == 1 ? g_lo[1] : j == 2 ? g_lo[2] : g_lo[3];
    const float hi = j == 0 ? g_hi[0] : j == 1 ? g_hi[1] : j == 2 ? g_hi[2] : g_hi[3];
    // Scales of rows 16 bm + 4 quad + i: row r of the 128 sits in lane r of
    // lo (r < 64) or lane r - 64 of hi.
    float4 wsc[8];
#pragma unroll
    for (int bm = 0; bm < 8; ++bm) {
      const int src = __float_as_int(bm < 4 ? lo : hi);
      const int base = (16 * (bm & 3) + 4 * quad) * 4;
      wsc[bm].x = __int_as_float(__builtin_amdgcn_ds_bpermute(base, src));
      wsc[bm].y = __int_as_float(__builtin_amdgcn_ds_bpermute(base + 4, src));
      wsc[bm].z = __int_as_float(__builtin_amdgcn_ds_bpermute(base + 8, src));
      wsc[bm].w = __int_as_float(__builtin_amdgcn_ds_bpermute(base + 12, src));
    }
    auto fold_tile = [&](auto partial) {
#pragma unroll
      for (int bn = 0; bn < kBN; ++bn) {
        floatx4 z[8];
#pragma unroll
        for (int bm = 0; bm < 8; ++bm) {
          z[bm] = acc[bm][bn];
          scale_logits(z[bm], wsc[bm], hs[bn]);
        }
        pick_sampled(c[bn], z, vw, quad, zy_out + (t0 + wt * kWaveToks + bn * 16 + c16));
        fold_column16(c[bn], z, vw, quad, vocab, partial);
      }
    };
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{});
    else fold_tile(std::false_type{});
    // more than kNarrowScaleTiles tiles in the slice (vocabularies above
    // 256 kNarrowScaleTiles tiles): the next group
    if (j == kNarrowScaleTiles - 1 && tile + 1 < tile_end) load_scales(tile + 1);
  };
  run_tiles_narrow<2, kBRows>(smem, L, row_bytes, tile_begin, tile_end, nks, w_rsrc, hr, epilogue);
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * kWaveToks + bn * 16 + c16;
    flush_slice16(c[bn], tok, n_tok, quad, ((size_t)slice * 2 + wv) * n_tok + tok, part);
  }
}

// ---- MXFP4 weights ("FP8 and MXFP4 weights", same section) ----
// OCP MX: blocks of 32 consecutive values along d share a power-of-two scale
// 2^e, e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an all-zero
// block), stored as the E8M0 byte e + 127; elements are E2M1 (values 0, 0.5,
// 1, 1.5, 2, 3, 4, 6) of x / 2^e, round to nearest even, saturating at 6,
// packed two per byte (even element in the low nibble).

// E2M1 code of a finite float32, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e2m1_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float a = fabsf(x);
  if (a < 1.0f) return sign | (uint32_t)rintf(a * 2.0f);  // 0, 0.5 or (rounded up) 1.0 = code 2
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
  float r = rintf(ldexpf(a, 1 - e));  // 1.m x 2, in [2, 4]
  if (r == 4.0f) {
    e += 1;
    r = 2.0f;
  }
  if (e > 2 || (e == 2 && r > 3.0f)) return sign | 7u;
  return sign | ((uint32_t)(e + 1) << 1) | ((uint32_t)r - 2u);
}

// One lane per 32-value block: amax, the block exponent, 32 codes packed
// into 16 bytes, one scale byte.
template <int kDtype>
__global__ __launch_bounds__(256) void quantize_rows_mxfp4_kernel(const void* __restrict__ X, long long n_rows, int d,
                                                                  uint8_t* __restrict__ Xq, uint8_t* __restrict__ sc) {
  const long long nb = (long long)n_rows * (d / 32);
  const long long blk = (long long)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nb) return;
  const size_t base = (size_t)blk * 32;  // rows are whole blocks: block b of the matrix starts at element 32 b
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = load_elem<kDtype>(X, base + i);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  int e = -127;
  if (amax > 0.0f) {
    const int fl = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;  // floor(log2 amax); <= -127 when subnormal
    e = fl - 2 < -127 ? -127 : (fl - 2 > 127 ? 127 : fl - 2);
  }
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i >> 3] |= e2m1_rne(ldexpf(v[i], -e)) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(Xq + (size_t)blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  sc[blk] = (uint8_t)(e + 127);
}

// The fp8 head's partial kernel with MXFP4 weights: the W block scales are
// applied by the matrix cores; the epilogue scales by the token's scale.
__global__ __launch_bounds__(kThreads, 1) void lmhead_mxfp4_partial_kernel(
    const uint8_t* __restrict__ Hq, const float* __restrict__ h_scale, const uint8_t* __restrict__ Wq4,
    const uint8_t* __restrict__ w_sc, const int32_t* __restrict__ tokens, int n_tok, int d, int vocab, int n_tb,
    int n_slices, int group, float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes L = lanes();
  const int wv = L.wv, wt = L.wt, half = L.half, col = L.col;
  const int S = n_slices;
  const WideWork work = wide_work(blockIdx.x, n_tb, S, group);
  const int t0 = work.tb * kBT;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int slice_first = work.slice_first;
  const int tile_begin = slice_tile(work.slice_first, n_vt, S);
  const int tile_end = slice_tile(work.slice_end, n_vt, S);
  const int w_row_bytes = d / 2, s_row_bytes = d / 32, h_row_bytes = d;
  const int nks = d / 128;

  Col c[4];
  float hs[4];
#pragma unroll
  for (int bn = 0; bn < 4; ++bn) {
    const int tok = t0 + wt * 128 + bn * 32 + col;
    c[bn] = Col{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f, 0.0f, false};
    hs[bn] = tok < n_tok ? h_scale[tok] : 0.0f;
  }
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(Wq4 + (size_t)v0 * w_row_bytes, (uint32_t)min(kBV, vocab - v0) * w_row_bytes);
  };
  auto s_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(w_sc + (size_t)v0 * s_row_bytes, (uint32_t)min(kBV, vocab - v0) * s_row_bytes);
  };
  const int4v hr = rsrc_words(Hq + (size_t)t0 * h_row_bytes, (uint32_t)min(kBT, n_tok - t0) * h_row_bytes);

  int slice = slice_first;
  int slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
  auto epilogue = [&](int tile, floatx16 (&acc)[4][4]) {
    const int vw = tile * kBV + wv * 128;
    mfma_result_wait();
    auto fold_tile = [&](auto partial) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
#pragma unroll
        for (int bm = 0; bm < 4; ++bm) {
          floatx16 z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = acc_read(acc[bm][bn], i) * hs[bn];
          fold_values(c[bn], z, bm, vw, half, vocab, partial);
        }
      }
    };
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{});
    else fold_tile(std::false_type{});
    if (tile == slice_last_tile) {
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        const int tok = t0 + wt * 128 + bn * 32 + col;
        flush_slice(c[bn], tok, n_tok, half, ((size_t)slice * 2 + wv) * n_tok + tok, part);
      }
      ++slice;
      slice_last_tile = slice_tile(slice + 1, n_vt, S) - 1;
    }
  };
  run_tiles_mx4(smem, L, w_row_bytes, s_row_bytes, h_row_bytes, tile_begin, tile_end, nks, w_rsrc, s_rsrc, hr,
                epilogue);

#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
    if (c[bn].found) zy_out[t0 + wt * 128 + bn * 32 + col] = c[bn].zy;
}

// Decode-shaped MXFP4 calls (at most kNarrow128MaxTokens tokens): kBRows-token
// blocks (64, or one block of 128 for calls of 65 to 128 tokens), one
// workgroup per (token block, slice), run_tiles_narrow_mx4<kBRows>. Lane l
// of wavefront (wv, wt) holds tokens t0 + (kBRows / 2) wt + 32 bn + (l mod 32)
// (bn < kBRows / 64) against the same W rows, with the same MFMA fragments,
// scales and fold, as in lmhead_mxfp4_partial_kernel, so the partials and
// logprobs have the same bits.
template <int kBRows>
__global__ __launch_bounds__(kThreads, 1) void lmhead_mxfp4_partial_narrow_kernel(
    const uint8_t* __restrict__ Hq, const float* __restrict__ h_scale, const uint8_t* __restrict__ Wq4,
    const uint8_t* __restrict__ w_sc, const int32_t* __restrict__ tokens, int n_tok, int d, int vocab, int n_slices,
    float2* __restrict__ part, float* __restrict__ zy_out) {
  __shared__ uint4 smem[kEngineSmemChunks];
  const Lanes L = lanes();
  const int wv = L.wv, wt = L.wt, half = L.half, col = L.col;
  const int S = n_slices;
  const int slice = blockIdx.x % S;
  constexpr int kBN = kBRows / 64;
  const int t0 = (blockIdx.x / S) * kBRows;
  const int n_vt = (vocab + kBV - 1) / kBV;
  const int tile_begin = slice_tile(slice, n_vt, S);
  const int tile_end = slice_tile(slice + 1, n_vt, S);
  const int w_row_bytes = d / 2, s_row_bytes = d / 32, h_row_bytes = d;
  const int nks = d / 128;
  Col c[kBN];
  float hs[kBN];
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * (kBRows / 2) + bn * 32 + col;
    c[bn] = Col{tok < n_tok ? tokens[tok] : -1, -INFINITY, 0.0f, 0.0f, false};
    hs[bn] = tok < n_tok ? h_scale[tok] : 0.0f;
  }
  auto w_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(Wq4 + (size_t)v0 * w_row_bytes, (uint32_t)min(kBV, vocab - v0) * w_row_bytes);
  };
  auto s_rsrc = [&](int tile) {
    const int v0 = tile * kBV;
    return rsrc_words(w_sc + (size_t)v0 * s_row_bytes, (uint32_t)min(kBV, vocab - v0) * s_row_bytes);
  };
  const int4v hr = rsrc_words(Hq + (size_t)t0 * h_row_bytes, (uint32_t)min(kBRows, n_tok - t0) * h_row_bytes);
  auto epilogue = [&](int tile, floatx16 (&acc)[4][kBN]) {
    const int vw = tile * kBV + wv * 128;
    mfma_result_wait();
    auto fold_tile = [&](auto partial) {
#pragma unroll
      for (int bn = 0; bn < kBN; ++bn)
#pragma unroll
        for (int bm = 0; bm < 4; ++bm) {
          floatx16 z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = acc_read(acc[bm][bn], i) * hs[bn];
          fold_values(c[bn], z, bm, vw, half, vocab, partial);
        }
    };
    if (tile * kBV + kBV > vocab) fold_tile(std::true_type{});
    else fold_tile(std::false_type{});
  };
  run_tiles_narrow_mx4<kBRows>(smem, L, w_row_bytes, s_row_bytes, h_row_bytes, tile_begin, tile_end, nks, w_rsrc,
                               s_rsrc, hr, epilogue);
#pragma unroll
  for (int bn = 0; bn < kBN; ++bn) {
    const int tok = t0 + wt * (kBRows / 2) + bn * 32 + col;
    flush_slice(c[bn], tok, n_tok, half, ((size_t)slice * 2 + wv) * n_tok + tok, part);
    if (c[bn].found) zy_out[tok] = c[bn].zy;
  }
}

}  // namespace

hipError_t launch_quantize_rows_fp8(const void* X, int dtype, long long n_rows, int d, uint8_t* Xq, float* scale,
                                    hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(n_rows, 4));
  if (dtype == 0)
    hipLaunchKernelGGL(quantize_rows_fp8_kernel<0>, grid, dim3(256), 0, stream, X, n_rows, d, Xq, scale);
  else
    hipLaunchKernelGGL(quantize_rows_fp8_kernel<1>, grid, dim3(256), 0, stream, X, n_rows, d, Xq, scale);
  return hipGetLastError();
}

hipError_t launch_lmhead_logprob_fp8(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq, const float* w_scale,
                                     int n_tok, int d, int vocab, const int32_t* tokens, float* logprob, float* lse,
                                     void* workspace, hipStream_t stream) {
  const int S = n_slices(vocab);
  const int G = slices_per_group(n_tok, vocab);
  const int ntb = (int)ceil_div(n_tok, kBT);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)2 * S * (size_t)n_tok * sizeof(float2)));
  if (n_tok <= kNarrowMaxTokens) {
    const dim3 grid((unsigned)ceil_div(n_tok, kNarrowBRows) * (unsigned)S);
    hipLaunchKernelGGL((lmhead_fp8_partial_narrow_kernel<kNarrowBRows>), grid, dim3(kThreads), 0, stream, Hq, h_scale,
                       Wq, w_scale, tokens, n_tok, d, vocab, S, part, zy);
  } else if (n_tok <= kNarrow128MaxTokens) {
    hipLaunchKernelGGL((lmhead_fp8_partial_narrow_kernel<kNarrow128MaxTokens>), dim3((unsigned)S), dim3(kThreads), 0,
                       stream, Hq, h_scale, Wq, w_scale, tokens, n_tok, d, vocab, S, part, zy);
  } else {
    const dim3 grid((unsigned)ntb * (unsigned)n_slice_groups(n_tok, vocab));
    // Long K loops stage the token block two K steps ahead, as in the bf16
    // head (the load order changes no arithmetic).
    if (d / kStepBytes > kNearBMaxSteps)
      hipLaunchKernelGGL((lmhead_fp8_partial8_kernel<true>), grid, dim3(kThreads8), 0, stream, Hq, h_scale, Wq,
                         w_scale, tokens, n_tok, d, vocab, ntb, S, G, part, zy);
    else
      hipLaunchKernelGGL((lmhead_fp8_partial8_kernel<false>), grid, dim3(kThreads8), 0, stream, Hq, h_scale, Wq,
                         w_scale, tokens, n_tok, d, vocab, ntb, S, G, part, zy);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lse_combine(part, zy, n_tok, 2 * S, logprob, lse, stream);
}

}  // namespace itl

namespace itl {

hipError_t launch_quantize_rows_mxfp4(const void* X, int dtype, long long n_rows, int d, uint8_t* Xq, uint8_t* sc,
                                      hipStream_t stream) {
  const long long nb = n_rows * (d / 32);
  const dim3 grid((unsigned)ceil_div(nb, 256));
  if (dtype == 0)
    hipLaunchKernelGGL(quantize_rows_mxfp4_kernel<0>, grid, dim3(256), 0, stream, X, n_rows, d, Xq, sc);
  else
    hipLaunchKernelGGL(quantize_rows_mxfp4_kernel<1>, grid, dim3(256), 0, stream, X, n_rows, d, Xq, sc);
  return hipGetLastError();
}

hipError_t launch_lmhead_logprob_mxfp4(const uint8_t* Hq, const float* h_scale, const uint8_t* Wq4,
                                       const uint8_t* w_sc, int n_tok, int d, int vocab, const int32_t* tokens,
                                       float* logprob, float* lse, void* workspace, hipStream_t stream) {
  const int S = n_slices(vocab);
  const int G = slices_per_group(n_tok, vocab);
  const int ntb = (int)ceil_div(n_tok, kBT);
  float2* part = static_cast<float2*>(workspace);
  float* zy = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256((size_t)2 * S * (size_t)n_tok * sizeof(float2)));
  if (n_tok <= kNarrowMaxTokens) {
    const dim3 grid((unsigned)ceil_div(n_tok, kNarrowBRows) * (unsigned)S);
    hipLaunchKernelGGL((lmhead_mxfp4_partial_narrow_kernel<kNarrowBRows>), grid, dim3(kThreads), 0, stream, Hq,
                       h_scale, Wq4, w_sc, tokens, n_tok, d, vocab, S, part, zy);
  } else if (n_tok <= kNarrow128MaxTokens) {
    hipLaunchKernelGGL((lmhead_mxfp4_partial_narrow_kernel<kNarrow128MaxTokens>), dim3((unsigned)S), dim3(kThreads), 0,
                       stream, Hq, h_scale, Wq4, w_sc, tokens, n_tok, d, vocab, S, part, zy);
  } else {
    const dim3 grid((unsigned)ntb * (unsigned)n_slice_groups(n_tok, vocab));
    hipLaunchKernelGGL(lmhead_mxfp4_partial_kernel, grid, dim3(kThreads), 0, stream, Hq, h_scale, Wq4, w_sc, tokens,
                       n_tok, d, vocab, ntb, S, G, part, zy);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lse_combine(part, zy, n_tok, 2 * S, logprob, lse, stream);
}

}  // namespace itl
