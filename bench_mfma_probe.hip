// Sustained-throughput probe of the bf16 matrix cores (gfx950), for the
// benchmark's roofline: what the bf16 MFMA instructions sustain on this chip
// with operand data that changes every instruction, as in a real
// contraction, and no memory traffic at all. Benchmark infrastructure, not
// part of the library: built into libitl_bench_probe.so beside bench.py,
// which calls it through ctypes.
//
// Two shapes, each in the tiling the library's kernels give it:
//   shape 0: v_mfma_f32_32x32x16_bf16, 256-thread workgroups (one wavefront
//            per SIMD), a 4 x 4 block tile per wavefront (16 accumulators);
//   shape 1: v_mfma_f32_16x16x32_bf16, 512-thread workgroups (two
//            wavefronts per SIMD), an 8 x 4 block tile per wavefront (32
//            accumulators), the bf16 forward's wavefront tile.
// Each round issues one MFMA per block of the tile, block (i, j) taking A
// fragment i and B fragment j of the lane's fragments, read once from
// `operands`. One float per thread is written so the work is not optimised
// away.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kLanesOfOperands = 4096;  // operands holds 4096 lanes x 16 fragments of 16 bytes
constexpr int kFragsPerLane = 16;

__global__ __launch_bounds__(256, 1) void mfma_probe32_kernel(const uint4* __restrict__ operands,
                                                              float* __restrict__ out, int iters) {
  const int t = (blockIdx.x * 256 + threadIdx.x) & (kLanesOfOperands - 1);
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, operands[t * kFragsPerLane + i]);
    b[i] = __builtin_bit_cast(bf16x8_t, operands[t * kFragsPerLane + 8 + i]);
  }
  floatx16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = floatx16{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j >> 2], b[j & 3], acc[j], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(512, 1) void mfma_probe16_kernel(const uint4* __restrict__ operands,
                                                              float* __restrict__ out, int iters) {
  const int t = (blockIdx.x * 512 + threadIdx.x) & (kLanesOfOperands - 1);
  bf16x8_t a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = __builtin_bit_cast(bf16x8_t, operands[t * kFragsPerLane + i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8_t, operands[t * kFragsPerLane + 8 + i]);
  floatx4 acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = floatx4{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j >> 2], b[j & 3], acc[j], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[j][i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Bytes of `operands` the probe reads (random bf16 bit patterns, caller-owned
// device memory).
size_t itl_probe_operand_bytes(void) { return (size_t)kLanesOfOperands * kFragsPerLane * 16; }

// Threads per workgroup of a shape (0 or 1, see above); `out` of a launch
// holds blocks times this many floats. 0 for an unknown shape.
int itl_probe_threads(int shape) { return shape == 0 ? 256 : shape == 1 ? 512 : 0; }

// Flops of one probe launch of a shape: per wavefront and round, 16 MFMAs of
// 32 x 32 x 16 (shape 0) or 32 of 16 x 16 x 32 (shape 1), both 2^19 flops.
double itl_probe_flops(int shape, int blocks, int iters) {
  return 524288.0 * iters * (double)blocks * (itl_probe_threads(shape) / 64);
}

// Enqueue one probe launch of a shape: `blocks` workgroups, `out` holds
// blocks * itl_probe_threads(shape) floats (device). Returns 0 or the HIP
// error code.
int itl_probe_mfma_bf16(int shape, const void* operands, float* out, int blocks, int iters, void* stream) {
  if ((shape != 0 && shape != 1) || !operands || !out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  const uint4* ops = static_cast<const uint4*>(operands);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_probe32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ops, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe16_kernel, dim3((unsigned)blocks), dim3(512), 0, st, ops, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
