// Sustained-throughput probe of the bf16 matrix cores (gfx950), for the
// benchmark's roofline: what v_mfma_f32_32x32x16_bf16 sustains on this chip
// with operand data that changes every instruction, as in a real contraction,
// and no memory traffic at all. Benchmark infrastructure, not part of the
// library: built into libitl_bench_probe.so beside bench.py, which calls it
// through ctypes.
//
// Each 256-thread workgroup (one wavefront per SIMD) runs `iters` rounds of
// 16 MFMAs into 16 accumulators; MFMA j of a round takes A fragment j / 4 and
// B fragment j % 4 of the lane's 8 fragments (a 4 x 4 block tile, the
// library's wavefront tile), read once from `operands`. One float per thread
// is written so the work is not optimised away.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kLanesOfOperands = 4096;  // operands holds 4096 lanes x 8 fragments of 16 bytes

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint4* __restrict__ operands, float* __restrict__ out,
                                                            int iters) {
  const int t = (blockIdx.x * 256 + threadIdx.x) & (kLanesOfOperands - 1);
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, operands[t * 8 + i]);
    b[i] = __builtin_bit_cast(bf16x8_t, operands[t * 8 + 4 + i]);
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

}  // namespace

extern "C" {

// Bytes of `operands` the probe reads (random bf16 bit patterns, caller-owned
// device memory).
size_t itl_probe_operand_bytes(void) { return (size_t)kLanesOfOperands * 8 * 16; }

// Flops of one probe launch.
double itl_probe_flops(int blocks, int iters) { return 32768.0 * 16.0 * iters * (double)blocks * 4.0; }

// Enqueue one probe launch: `blocks` workgroups of 256 threads, `out` holds
// blocks * 256 floats (device). Returns 0 or the HIP error code.
int itl_probe_mfma_bf16(const void* operands, float* out, int blocks, int iters, void* stream) {
  if (!operands || !out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(operands), out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
