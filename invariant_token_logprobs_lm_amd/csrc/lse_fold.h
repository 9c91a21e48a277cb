// Per-lane online log-sum-exp folds of the head's logits: fold_column for
// the bf16 / fp32 heads (wide and narrow kernels), fold_values for the FP8 /
// MXFP4 heads (block by block). Kernels that share a fold and feed it the
// same logit values in the same order give a token the same partials, and
// so the same logprob, bit for bit.
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

// Fold one 32 x 32 block of logits (rows vw + 32 bm + ..., this lane's
// token column; z[i] = row 32 bm + 8 (i / 4) + 4 half + (i % 4)) into the
// state (the FP8 / MXFP4 kernels' fold). The sampled logit is picked with a
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

// Fold one tile's four 32 x 32 blocks of one token column (block bm holds
// rows 32 bm + 8 (i / 4) + 4 half + (i % 4) of the wavefront's 128 rows) into
// the state, as one step: the bf16 and fp32 heads' fold, shared by their
// wide and narrow kernels (the FP8 kernels fold block by block with
// fold_values). The 64 logits' maximum M (exact in any order) moves the
// running maximum to m' = max(m, M); every term of the tile is then
// exp2(z log2e + b) with one rounded offset b = -m' log2e (a fused
// multiply-add per logit), summed into eight partial sums in a fixed order
// and added to the old sum rescaled by exp2(m log2e + b). The shared offset
// moves every term of the tile by the same factor, within |m'| 2^-24 of 1
// (the maximum's own term is not exactly 1: the combine keeps lse >= the
// largest logit, so logprob <= 0 still holds in fp32).
template <class kPartial, class kPick>
__device__ __forceinline__ void fold_column(Col& c, floatx16 z0, floatx16 z1, floatx16 z2, floatx16 z3, int vw,
                                            int half, int vocab, kPartial, kPick) {
  floatx16 z[4] = {z0, z1, z2, z3};
  if constexpr (kPartial::value) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      const int lim = vocab - (vw + bm * 32 + 4 * half);  // rows at or past this offset do not exist
#pragma unroll
      for (int i = 0; i < 16; ++i) z[bm][i] = (8 * (i >> 2) + (i & 3) >= lim) ? -INFINITY : z[bm][i];
    }
  }
  if constexpr (kPick::value) {
    const int o = c.y - vw;  // sampled row relative to this wavefront's 128 rows
    const bool b0 = (o & 1) != 0, b1 = (o & 2) != 0, b2 = (o & 8) != 0, b3 = (o & 16) != 0;
    const bool here = (unsigned)o < 128u && ((o >> 2) & 1) == half;
    const int bm = (o >> 5) & 3;
    const float pick = select16(bm == 0 ? z[0] : bm == 1 ? z[1] : bm == 2 ? z[2] : z[3], b0, b1, b2, b3);
    c.zy = here ? pick : c.zy;
    c.found = c.found || here;
  }
  float mx[4];
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    float a = fmaxf(z[bm][0], z[bm][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) a = fmaxf(a, z[bm][i]);
    mx[bm] = a;
  }
  const float mnew = fmaxf(c.m, fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
  // A lane whose rows so far are all absent has mnew = -inf; it then works
  // around 0 and keeps (m, s) = (-inf, 0).
  const float mref = mnew == -INFINITY ? 0.0f : mnew;
  const float b = -mref * kLog2e;
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = fast_exp2(__builtin_fmaf(z[0][k], kLog2e, b));
#pragma unroll
  for (int k = 8; k < 64; ++k) s[k & 7] += fast_exp2(__builtin_fmaf(z[k >> 4][k & 15], kLog2e, b));
  const float sum = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  c.s = __builtin_fmaf(c.s, fast_exp2(__builtin_fmaf(c.m, kLog2e, b)), sum);
  c.m = mnew;
}

// Slice end: lanes l and l ^ 32 hold the same token (different rows); the
// lower lane merges the upper lane's state into its own and writes the
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
