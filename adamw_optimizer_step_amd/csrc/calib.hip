// Calibration kernel: the MFMA rate this part sustains with no memory
// traffic, the practical ceiling against which the Newton-Schulz GEMMs are
// read. Not part of the optimizer step.
//
// Each wave keeps 16 independent 32x32 fp32 accumulator blocks (the same
// shape as one wave of the GEMM kernel) and issues `iters` rounds of one
// 32x32x16 bf16 MFMA per block, operands in registers; at the end one value
// per lane is stored so that nothing is optimised away. Work per launch:
// blocks x 4 waves x iters x 16 x 32768 flops.
#include "calib.hpp"

namespace ma {

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_calib_mfma(int iters, float* sink) {
  f32x16_t acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
  // small operands so that the sums stay finite whatever iters is
  const uint32_t lane = threadIdx.x & 63;
  const u32x4_t a = {0x3C003C00u ^ lane, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  const u32x4_t b = {0x3A003A00u, 0x3A003A00u ^ lane, 0x3A003A00u, 0x3A003A00u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc[k][k];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_calib_mfma(int blocks, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_calib_mfma, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace ma
