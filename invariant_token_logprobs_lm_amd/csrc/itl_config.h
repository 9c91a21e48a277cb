// Compile-time shape constants of the library's arithmetic.
//
// Everything that fixes a reduction order lives here and nowhere else: the
// vocabulary tile and the vocabulary slice width (the order in which a
// token's logits are folded), the K step, and the token block, which only
// shapes the schedule (the narrow kernels' 64- and 128-token blocks give
// the 256-token block's bits). None of them depends on the number of tokens
// in a call, which is what makes a token's result independent of its
// batch-mates and of the prefill/decode split ("vLLM Train-Inference
// Consistency Release Notes", section "Achieving Bitwise Consistency": batch
// independence and phase consistency). They are part of itl_build_info(),
// since a change to the tile or the slices changes result bits.
#pragma once

#include <hip/hip_runtime.h>

namespace itl {

constexpr int kThreads = 256;        // 4 wavefronts of 64 lanes (narrow and MXFP4 engines)
constexpr int kThreads8 = 512;       // 8 wavefronts (the bf16 / fp32 / FP8 wide engine)
constexpr int kBT = 256;             // tokens per block (MFMA B operand)
constexpr int kBV = 256;             // vocabulary rows per tile (MFMA A operand)
constexpr int kStepBytes = 128;      // bytes of one operand row per K step (64 bf16 / 32 fp32)
constexpr int kWSlots = 3;           // LDS slots of the W-tile ring (loads two K steps ahead)
constexpr int kHSlots = 2;           // LDS slots of the H-block ring (loads one K step ahead)
constexpr int kMaxSlices = 256;      // vocabulary slices: min(tiles, this), a function of the vocabulary only
constexpr int kTilesPerGroup = 16;   // grid shape only (backward dlogits): a workgroup walks about this many
                                     // tiles of consecutive slices (the arithmetic per slice is the same)
constexpr int kWideTilesPerGroup = 4;  // the same for the forward kernels: with the vocabularies of interest
                                       // (>= 512 tiles) one slice per workgroup, the fastest order measured
constexpr int kNarrowBRows = 64;      // tokens per block of the narrow (few-token) kernel
constexpr int kNarrowMaxTokens = 64;   // calls with at most this many tokens use the narrow kernel
constexpr int kNarrow128MaxTokens = 128;  // calls of 65 to this many tokens: the narrow kernel on one 128-token block
constexpr int kSuperBand = 64;       // token blocks walked together, slice group by slice group (workgroup order)
constexpr int kBwdSuperBand = 32;    // the same for the backward kernels' walk (64 measured 3 % slower there)
constexpr int kNearBMaxSteps = 48;   // load schedule only: K loops longer than this stage the fixed operand
                                     // two K steps ahead (eight-wavefront forward at 65,536 tokens, same bits:
                                     // 64 steps (d = 4096) 2-3 % faster; 112 and 40 steps within 1 % either way)
constexpr int kDMultiple = 64;       // d must be a multiple of this

// REINFORCE Zero loss. A response is cut into segments of kSegTokens tokens
// counted from its first token; a segment is summed by one of three trees
// chosen by its length alone (up to kLaneSeg tokens: one lane in token order;
// up to kWaveSeg: one wavefront, lane j adding tokens j, j + 64, ...; longer:
// the token pass's workgroup, thread j adding tokens j, j + kLossThreads, ...);
// the segments are added in order. The mean over responses is taken over
// chunks of kFinishChunk consecutive responses, then over the chunks in
// order. All of it is part of the loss's bits.
constexpr int kSegTokens = 2048;
constexpr int kLaneSeg = 32;
constexpr int kWaveSeg = 256;
constexpr int kLossThreads = 512;    // threads of a token-pass workgroup
constexpr int kFinishChunk = 1024;   // responses per workgroup of the finishing pass (4 per thread)

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

inline int n_vocab_tiles(long long vocab) { return (int)ceil_div(vocab, kBV); }
inline int n_slices(long long vocab) {
  const long long nvt = n_vocab_tiles(vocab);
  return (int)(nvt < kMaxSlices ? nvt : kMaxSlices);
}

// Slices per workgroup: 1 while the grid is small (decode-shaped calls keep
// one workgroup per slice, so every CU streams W), else the largest power of
// two g with g slices holding at most 1.5 kWideTilesPerGroup tiles (a power
// of two divides S = 256 evenly). Changes which workgroup computes a slice,
// never how: each slice's partial is the same instruction sequence. (Walking
// 2 to 4 slices per workgroup measured 1-3 % slower than 1 on the bf16
// heads: workgroups that share operands through an XCD's L2 drift apart
// over long walks.)
inline int slices_per_group(long long n_tok, long long vocab) {
  const long long ntb = ceil_div(n_tok, kBT);
  const long long S = n_slices(vocab), nvt = n_vocab_tiles(vocab);
  if (ntb * S <= 2048) return 1;
  long long g = 1;
  while (2 * g <= S && 2 * g * nvt * 2 <= 3LL * kWideTilesPerGroup * S) g *= 2;
  return (int)g;
}
inline int n_slice_groups(long long n_tok, long long vocab) {
  return (int)ceil_div(n_slices(vocab), slices_per_group(n_tok, vocab));
}

// Slice s covers vocabulary tiles [slice_tile(s), slice_tile(s + 1)): the
// tiles are split as evenly as possible, so a slice holds floor(n_vt / S)
// or ceil(n_vt / S) tiles. This is a pure function of the vocabulary size.
__host__ __device__ inline int slice_tile(int s, int n_vt, int S) { return (int)(((long long)s * n_vt) / S); }

// Work of workgroup b of the wide logprob kernels (grid = n_tb x
// ceil(S / group)): super-bands of kSuperBand token blocks walked slice group
// by slice group with the token block fastest. Workgroups are dispatched to
// the 8 XCDs round-robin, so the 32 workgroups an XCD runs at once hold 8
// token blocks x 4 slice groups (each W tile read by 8 of them, each H block
// by 4, through the XCD's L2), and all XCDs walk the same slices at the same
// time (W shared through the Infinity Cache). Measured against 4 x 8: 0.5-2 %
// faster; 16 x 2 and 32 x 1 are slower. Only which workgroup computes a
// slice when depends on this order, never any arithmetic.
struct WideWork {
  int tb;           // token block
  int slice_first;  // slices [slice_first, slice_end)
  int slice_end;
};

__host__ __device__ inline WideWork wide_work(int b, int n_tb, int S, int group) {
  const int n_groups = (S + group - 1) / group;
  const int band = b / (kSuperBand * n_groups);
  const int tb_first = band * kSuperBand;
  const int nb = n_tb - tb_first < kSuperBand ? n_tb - tb_first : kSuperBand;
  const int rem = b - band * kSuperBand * n_groups;
  const int grp = rem / nb;
  WideWork w;
  w.tb = tb_first + rem % nb;
  w.slice_first = grp * group;
  w.slice_end = w.slice_first + group < S ? w.slice_first + group : S;
  return w;
}

}  // namespace itl
