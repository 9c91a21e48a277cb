// Device-side helpers shared by the library's kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace itl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

// Cache policy of the kept-logits buffer stores: the default (write-back
// through L2). Each store instruction writes 64-byte pieces of 16 tokens'
// rows (four lanes each) and the L2 merges neighbouring blocks' pieces into
// whole 128-byte lines. On the large-moe head's forward (65,536 tokens) the
// non-temporal bit and the sc0 bit measured equal, sc0 with sc1 2 % slower.
constexpr int kLogitStorePolicy = 0;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge two partial log-sum-exp states (m = running max, s = sum of
// exp(z - m)) as s exp(m - M) + s2 exp(m2 - M), the first product fused
// into the add. The result is a fixed function of the two states in this
// argument order, so callers fix the merge tree and get fixed bits.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {  // both sides empty
    m = -INFINITY;
    s = 0.0f;
    return;
  }
  s = __builtin_fmaf(s, fast_exp2((m - M) * kLog2e), s2 * fast_exp2((m2 - M) * kLog2e));
  m = M;
}

// Sum over the 64 lanes of a wavefront with a fixed xor butterfly. Every lane
// ends with the same bits: each step adds the same two operands on both
// partner lanes, and fp addition is commutative.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// The same butterfly in fp64.
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace itl
