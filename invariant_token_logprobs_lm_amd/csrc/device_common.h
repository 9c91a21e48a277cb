// Device-side helpers shared by the library's kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace itl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw buffer resource over [base, base + nbytes). Loads whose VGPR offset is
// past nbytes return zeros instead of faulting (callers keep the scalar
// offset at 0: only the VGPR offset is range-checked), which is how tile rows beyond the last token or
// vocabulary row are read safely. Word 3 is the gfx9-family raw-buffer
// configuration (32-bit data format, no swizzle, no index stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  int4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return uint4{(unsigned)v[0], (unsigned)v[1], (unsigned)v[2], (unsigned)v[3]};
}

__device__ __forceinline__ float buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}

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

}  // namespace itl
