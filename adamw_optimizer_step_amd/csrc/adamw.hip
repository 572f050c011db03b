// AdamW step over many flat fp32 buffers in one launch (gfx950).
//
// Rule ("3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo",
// section "Implementing AdamW from scratch"; "Chapter 4: The MuonAdamW
// Optimizer", section "The AdamW Step"), per element, binary32, one rounding
// per operation, no contraction (built with -ffp-contract=off):
//     p = p * cd                         (cd = 1 - lr*wd, only when wd != 0)
//     m = b1*m + c1*g                    (c1 = 1 - b1)
//     v = b2*v + c2*(g*g)                (c2 = 1 - b2)
//     p = p - ss * (m / (sqrt(v)/s2 + eps))
// with ss = lr/(1 - b1^t) and s2 = sqrt(1 - b2^t) formed on the host in fp64.
//
// 28 bytes of HBM traffic per element (p, g, m, v read; p, m, v written).
// Each block streams 4096 consecutive elements of one segment with 16-byte
// non-temporal loads and stores (all loads of a thread issued before its
// arithmetic; the state is touched once per step); a table of
// segments in the kernel arguments lets one launch cover every buffer, the
// multi-tensor ("fused"/"foreach") form the pages mention.
#include "adamw.hpp"

namespace ma {

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v, const AdamSeg& S) {
  if (S.decay) p = __fmul_rn(p, S.cd);
  m = __fadd_rn(__fmul_rn(S.b1, m), __fmul_rn(S.c1, g));
  v = __fadd_rn(__fmul_rn(S.b2, v), __fmul_rn(S.c2, __fmul_rn(g, g)));
  const float den = __fadd_rn(__fdiv_rn(__builtin_sqrtf(v), S.s2), S.eps);
  p = __fsub_rn(p, __fmul_rn(S.ss, __fdiv_rn(m, den)));
}

// Segment of block b (blocks of kAdamBlockElems elements, numbered across
// the segments in order).
__device__ __forceinline__ const AdamSeg& adam_segment(const AdamArgs& a, int64_t b) {
  int si = 0;
#pragma unroll
  for (int q = 1; q < kMaxAdamSegs; ++q)
    if (q < a.nseg && b >= a.s[q].block_begin) si = q;
  return a.s[si];
}

// One block of elements. LEAN: one 4-element chunk of each buffer per thread
// at a time (a small register footprint); otherwise all of the thread's
// chunks are loaded before any arithmetic.
template <bool LEAN>
__device__ __forceinline__ void adamw_block(const AdamSeg& S, int64_t e0, int tid) {
  if (S.vec) {
    constexpr int U = kAdamBlockElems / (256 * 4);
    constexpr int W = LEAN ? 1 : U;   // chunks in flight per thread
#pragma unroll 1
    for (int u0 = 0; u0 < U; u0 += W) {
      float4 p[W], g[W], m[W], v[W];
      bool full[W];
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const int64_t i = e0 + (int64_t)((u0 + u) * 256 + tid) * 4;
        full[u] = i + 4 <= S.n;
        if (full[u]) {
          p[u] = ld16f<true>(S.p + i);
          g[u] = ld16f<true>(S.g + i);
          m[u] = ld16f<true>(S.m + i);
          v[u] = ld16f<true>(S.v + i);
        }
      }
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const int64_t i = e0 + (int64_t)((u0 + u) * 256 + tid) * 4;
        if (full[u]) {
          adamw_elem(p[u].x, g[u].x, m[u].x, v[u].x, S);
          adamw_elem(p[u].y, g[u].y, m[u].y, v[u].y, S);
          adamw_elem(p[u].z, g[u].z, m[u].z, v[u].z, S);
          adamw_elem(p[u].w, g[u].w, m[u].w, v[u].w, S);
          st16f<true>(S.p + i, p[u]);
          st16f<true>(S.m + i, m[u]);
          st16f<true>(S.v + i, v[u]);
        } else {
          for (int64_t j = i; j < S.n && j < i + 4; ++j) {
            float pp = S.p[j], mm = S.m[j], vv = S.v[j];
            adamw_elem(pp, S.g[j], mm, vv, S);
            S.p[j] = pp; S.m[j] = mm; S.v[j] = vv;
          }
        }
      }
    }
  } else {
    for (int64_t j = e0 + tid; j < S.n && j < e0 + kAdamBlockElems; j += 256) {
      float pp = S.p[j], mm = S.m[j], vv = S.v[j];
      adamw_elem(pp, S.g[j], mm, vv, S);
      S.p[j] = pp; S.m[j] = mm; S.v[j] = vv;
    }
  }
}

__global__ void __launch_bounds__(256) k_adamw(const AdamArgs a) {
  const int64_t b = blockIdx.x;
  const AdamSeg& S = adam_segment(a, b);
  adamw_block<false>(S, (b - S.block_begin) * kAdamBlockElems, threadIdx.x);
}

// The same update by a fixed grid that strides over the blocks, LEAN: few
// registers per wave, so that a workgroup fits on a CU beside a Newton-Schulz
// GEMM workgroup (two waves of about 216 registers per SIMD) and the update
// can run on another stream while the GEMMs run.
__global__ void __launch_bounds__(256) k_adamw_lean(const AdamArgs a) {
  int si = 0;   // b only grows, so the segment index only advances
#pragma unroll 1
  for (int64_t b = blockIdx.x; b < a.total_blocks; b += gridDim.x) {
#pragma unroll 1
    while (si + 1 < a.nseg && b >= a.s[si + 1].block_begin) ++si;
    const AdamSeg& S = a.s[si];
    adamw_block<true>(S, (b - S.block_begin) * kAdamBlockElems, threadIdx.x);
  }
}

hipError_t launch_adamw(const AdamArgs& a, hipStream_t s) {
  if (a.total_blocks <= 0) return hipSuccess;
  if (a.lean_blocks > 0) {
    const int grid = a.lean_blocks < a.total_blocks ? a.lean_blocks : a.total_blocks;
    hipLaunchKernelGGL(k_adamw_lean, dim3((unsigned)grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_adamw, dim3((unsigned)a.total_blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ma
