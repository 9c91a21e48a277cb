// Per-lane online log-sum-exp folds of the head's logits: fold_column16 for
// the bf16 / fp32 / FP8 heads (wide and narrow kernels, 16 x 16 blocks),
// fold_values for the MXFP4 head (32 x 32 blocks, block by block).
// Kernels that share a fold and feed it the same logit values in the same
// order give a token the same partials, and so the same logprob, bit for
// bit.
#pragma once

#include "device_common.h"
#include "tile_engine.h"

namespace itl {

// Online log-sum-exp state of one token column in one lane: the running
// (max, sum of exp) of the slice so far, and the sampled logit once seen.
struct Col {
  int y;          // sampled row, -1 past the last token
  float m, s;     // running max and sum of exp(z - m)
  float zy;       // the sampled logit
  bool found;
};

// The same state for the 16 x 16 fold: the sampled logit is not carried
// (pick_sampled writes it out from the tile that holds it).
struct Col16 {
  int y;       // sampled row, -1 past the last token
  float m, s;  // running max and sum of exp(z - m)
};

// Fold one 32 x 32 block of logits (rows vw + 32 bm + ..., this lane's
// token column; z[i] = row 32 bm + 8 (i / 4) + 4 half + (i % 4)) into the
// state (the MXFP4 kernels' fold). The sampled logit is picked with a
// select tree keyed on the bits of its row, without a branch. Their wide and
// narrow kernels fold with this one function, in the same block order, so a
// token's state has the same bits whichever of them computed it.
//
// kPartial (a std::bool_constant): the block may hold rows past the
// vocabulary, which are masked. Callers choose it once per tile, so that a
// full tile's epilogue has no masking and no branches.
//
// kPick = std::false_type: the caller knows that no lane's sampled row lies
// in this wavefront's 128 rows of the tile, so the pick is skipped (it would
// leave zy and found unchanged).
template <class kPartial, class kPick = std::true_type>
__device__ __forceinline__ void fold_values(Col& c, floatx16 z, int bm, int vw, int half, int vocab, kPartial,
                                            kPick = kPick{}) {
  if constexpr (kPartial::value) {
    const int lim = vocab - (vw + bm * 32 + 4 * half);  // rows at or past this offset do not exist
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = (8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : z[i];
  }
  if constexpr (kPick::value) {
    const int o = c.y - vw;  // sampled row relative to this wavefront's 128 rows
    // Register i of a lane holds row 32 bm + 8 (i / 4) + 4 half + (i % 4):
    // bits 0, 1, 3, 4 of the row pick i, bit 2 picks the lane half.
    const bool b0 = (o & 1) != 0, b1 = (o & 2) != 0, b2 = (o & 8) != 0, b3 = (o & 16) != 0;
    const bool here = (unsigned)o < 128u && ((o >> 2) & 1) == half && (o >> 5) == bm;
    const float pick = select16(z, b0, b1, b2, b3);
    c.zy = here ? pick : c.zy;
    c.found = c.found || here;
  }

  float bmax = z[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) bmax = fmaxf(bmax, z[i]);
  const float mnew = fmaxf(c.m, bmax);
  // A lane whose rows so far are all absent has mnew = -inf; it then scales
  // by exp2(-inf) = 0 around 0 and keeps (m, s) = (-inf, 0).
  const float mref = mnew == -INFINITY ? 0.0f : mnew;
  // (z - m) is exactly 0 for the running maximum, so its term is exactly 1
  // and stays 1 (later rescales by exp2(0)): the final sum is >= 1 and
  // logprob <= 0 holds in fp32.
  // Two interleaved sums, even and odd registers, each in register order
  // (the first term starts the sum: 0 + t = t exactly).
  floatx16 t;
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = fast_exp2((z[i] - mref) * kLog2e);
  float s0 = t[0], s1 = t[1];
#pragma unroll
  for (int i = 2; i < 16; i += 2) {
    s0 += t[i];
    s1 += t[i + 1];
  }
  c.s = __builtin_fmaf(c.s, fast_exp2((c.m - mref) * kLog2e), s0 + s1);
  c.m = mnew;
}

// Of a lane's 32 values of one token (block bm register i: row offset
// 16 bm + 4 quad + i), the one at row offset o: block bits 4-6 of o,
// register bits 0-1 (bits 2-3 name the lane quarter), by a tree of selects.
__device__ __forceinline__ float select32(const floatx4 (&z)[8], int o) {
  const bool b0 = (o & 1) != 0, b1 = (o & 2) != 0, b4 = (o & 16) != 0, b5 = (o & 32) != 0, b6 = (o & 64) != 0;
  float v[8];
#pragma unroll
  for (int bm = 0; bm < 8; ++bm) v[bm] = b1 ? (b0 ? z[bm][3] : z[bm][2]) : (b0 ? z[bm][1] : z[bm][0]);
  const float w0 = b4 ? v[1] : v[0], w1 = b4 ? v[3] : v[2], w2 = b4 ? v[5] : v[4], w3 = b4 ? v[7] : v[6];
  const float x0 = b5 ? w1 : w0, x1 = b5 ? w3 : w2;
  return b6 ? x1 : x0;
}

// The lane of a wavefront that holds token column c's sampled row in this
// tile (row offset o = y - vw in [0, 128), lane quarter (o / 4) mod 4)
// writes that logit to *zy. It is read from the same accumulators the fold
// reads, before any masking (a sampled row lies inside the vocabulary).
__device__ __forceinline__ void pick_sampled(const Col16& c, const floatx4 (&z)[8], int vw, int quad, float* zy) {
  // y made opaque here: otherwise the compiler forms the select bits of the
  // row (loop-invariant) once, ahead of the K loop, and keeps them live
  // across it.
  int y = c.y;
  asm volatile("" : "+v"(y));
  const int o = y - vw;
  if ((unsigned)o < 128u && ((o >> 2) & 3) == quad) *zy = select32(z, o);
}

// Fold one tile's logits of one token column (this lane's 32 of the
// wavefront's 128 rows: block bm register i holds row 16 bm + 4 quad + i)
// into the state, as one step: the bf16, fp32 and FP8 heads' fold, shared by
// their wide and narrow kernels (the MXFP4 kernels fold block by block with
// fold_values). The 32 logits' maximum M (exact in any order) moves the
// running maximum to m' = max(m, M); every term of the tile is then
// exp2(z log2e + b) with one rounded offset b = -m' log2e (a fused
// multiply-add per logit), summed into eight partial sums in a fixed order
// and added to the old sum rescaled by exp2(m log2e + b). The shared offset
// moves every term of the tile by the same factor, within |m'| 2^-24 of 1
// (the maximum's own term is not exactly 1: the combine keeps lse >= the
// largest logit, so logprob <= 0 still holds in fp32).
//
// kPartial (a std::bool_constant): the tile may hold rows past the
// vocabulary, which are masked. Callers choose it once per tile, so that a
// full tile's epilogue has no masking and no branches.
template <class kPartial>
__device__ __forceinline__ void fold_column16(Col16& c, floatx4 (&z)[8], int vw, int quad, int vocab, kPartial) {
  if constexpr (kPartial::value) {
    const int lim = vocab - (vw + 4 * quad);  // row offsets 16 bm + i at or past this do not exist
#pragma unroll
    for (int bm = 0; bm < 8; ++bm)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[bm][i] = (16 * bm + i >= lim) ? -INFINITY : z[bm][i];
  }
  // (a chain: the compiler pairs it into three-operand maxima)
  float mnew = c.m;
#pragma unroll
  for (int k = 0; k < 32; ++k) mnew = fmaxf(mnew, z[k >> 2][k & 3]);
  // A lane whose rows so far are all absent has mnew = -inf; it then works
  // around 0 and keeps (m, s) = (-inf, 0).
  const float mref = mnew == -INFINITY ? 0.0f : mnew;
  const float b = -mref * kLog2e;
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = fast_exp2(__builtin_fmaf(z[k >> 2][k & 3], kLog2e, b));
#pragma unroll
  for (int k = 8; k < 32; ++k) s[k & 7] += fast_exp2(__builtin_fmaf(z[k >> 2][k & 3], kLog2e, b));
  const float sum = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  c.s = __builtin_fmaf(c.s, fast_exp2(__builtin_fmaf(c.m, kLog2e, b)), sum);
  c.m = mnew;
}

// Slice end of fold_column16's states: lanes l, l ^ 16, l ^ 32 and l ^ 48
// hold the same token (different rows); they are merged as (q0 q1)(q2 q3)
// (lane quarters l / 16), the lowest lane writes the wavefront's partial of
// the slice, and every lane starts the next slice afresh.
__device__ __forceinline__ void flush_slice16(Col16& c, int tok, int n_tok, int quad, size_t part_index,
                                              float2* __restrict__ part) {
  float m2 = __shfl_xor(c.m, 16, 64);
  float s2 = __shfl_xor(c.s, 16, 64);
  lse_merge(c.m, c.s, m2, s2);
  m2 = __shfl_xor(c.m, 32, 64);
  s2 = __shfl_xor(c.s, 32, 64);
  lse_merge(c.m, c.s, m2, s2);
  if (quad == 0 && tok < n_tok) part[part_index] = make_float2(c.m, c.s);
  c.m = -INFINITY;
  c.s = 0.0f;
}

// Slice end of fold_values's states: lanes l and l ^ 32 hold the same token
// (different rows); the lower lane merges the upper lane's state into its own and writes the
// wavefront's partial of the slice; every lane starts the next slice afresh.
__device__ __forceinline__ void flush_slice(Col& c, int tok, int n_tok, int half, size_t part_index,
                                            float2* __restrict__ part) {
  const float m2 = __shfl_xor(c.m, 32, 64);
  const float s2 = __shfl_xor(c.s, 32, 64);
  lse_merge(c.m, c.s, m2, s2);
  if (half == 0 && tok < n_tok) part[part_index] = make_float2(c.m, c.s);
  c.m = -INFINITY;
  c.s = 0.0f;
}

}  // namespace itl
