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

// A bf16 pair with a random sign and mantissa and exponent 2^-1, from a hash
// (finite sums whatever iters is).
__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ uint32_t calib_pair(uint32_t h) {
  return (0x3F00u | (h & 0x807Fu)) | ((0x3F00u | ((h >> 16) & 0x807Fu)) << 16);
}

// CHANGING = false: near-constant operands (a few bits differ by lane), the
// least switching activity; true: four sets of random operands that change
// from one MFMA to the next, as the operands of a real product do. The MFMA
// datapath draws more power on the second, and under the part's power limit
// its clock, and with it the sustained rate, drops.
template <bool CHANGING>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_calib_mfma(int iters, float* sink) {
  f32x16_t acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
  const uint32_t lane = threadIdx.x & 63;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (CHANGING) {
        a[s][w] = calib_pair(calib_hash(lane * 131u + s * 17u + w + 1u + blockIdx.x * 7919u));
        b[s][w] = calib_pair(calib_hash(lane * 257u + s * 29u + w + 1000003u + blockIdx.x * 104729u));
      } else {
        a[s][w] = w == 0 ? 0x3C003C00u ^ lane : 0x3C003C00u;
        b[s][w] = w == 1 ? 0x3A003A00u ^ lane : 0x3A003A00u;
      }
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[k & 3]),
                                                       __builtin_bit_cast(bf16x8_t, b[(k >> 2) & 3]), acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc[k][k];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_calib_mfma(int blocks, int iters, int changing, float* sink, hipStream_t s) {
  if (changing) hipLaunchKernelGGL(k_calib_mfma<true>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else hipLaunchKernelGGL(k_calib_mfma<false>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace ma
