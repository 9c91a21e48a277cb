// Compile-time shape constants of the library's arithmetic.
//
// Everything that fixes a reduction order lives here and nowhere else: the
// token block, the vocabulary tile, the K step, and the vocabulary slice
// width. None of them depends on the number of tokens in a call, which is
// what makes a token's result independent of its batch-mates and of the
// prefill/decode split ("vLLM Train-Inference Consistency Release Notes",
// section "Achieving Bitwise Consistency": batch independence and phase
// consistency). Changing any of them changes result bits, so they are part
// of itl_build_info().
#pragma once

#include <hip/hip_runtime.h>

namespace itl {

constexpr int kThreads = 256;        // 4 wavefronts of 64 lanes
constexpr int kBT = 256;             // tokens per block (MFMA B operand)
constexpr int kBV = 256;             // vocabulary rows per tile (MFMA A operand)
constexpr int kStepBytes = 128;      // bytes of one operand row per K step (64 bf16 / 32 fp32)
constexpr int kWSlots = 3;           // LDS slots of the W-tile ring (loads two K steps ahead)
constexpr int kHSlots = 2;           // LDS slots of the H-block ring (loads one K step ahead)
constexpr int kTilesPerSlice = 16;   // at most this many vocabulary tiles per slice
constexpr int kSuperBand = 32;       // token blocks walked together, slice by slice (workgroup order)
constexpr int kDMultiple = 64;       // d must be a multiple of this

constexpr int kLossThreads = 256;    // threads per response in the loss kernel
constexpr int kMeanThreads = 1024;   // threads of the single-block mean

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

inline int n_vocab_tiles(long long vocab) { return (int)ceil_div(vocab, kBV); }
inline int n_slices(long long vocab) { return (int)ceil_div(n_vocab_tiles(vocab), kTilesPerSlice); }

// Slice s covers vocabulary tiles [slice_tile(s), slice_tile(s + 1)): the
// tiles are split as evenly as possible, so a slice holds
// floor(n_vt / S) or ceil(n_vt / S) <= kTilesPerSlice tiles. This is a pure
// function of the vocabulary size.
__host__ __device__ inline int slice_tile(int s, int n_vt, int S) { return (int)(((long long)s * n_vt) / S); }

}  // namespace itl
