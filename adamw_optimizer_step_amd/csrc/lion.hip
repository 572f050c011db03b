// Lion step over many flat fp32 buffers in one launch (gfx950).
//
// Rule ("3.9 Optimizers: SGD, Adam, Adafactor, Lion, Muon & Shampoo", section
// "Lion: Learning the Sign of the Update" and exercise 5; "Muon vs AdamW,
// Lion and Sophia: a fair race", section "Lion"), per element, binary32, one
// rounding per operation, no contraction (built with -ffp-contract=off):
//     p = p * cd                         (cd = 1 - lr*wd, only when wd != 0)
//     c = b1*m + c1*g                    (c1 = 1 - b1; not stored)
//     p = p - lr*sign(c)                 (sign(+-0) = +0, sign(NaN) = NaN)
//     m = b2*m + c2*g                    (c2 = 1 - b2)
// so each weight moves by exactly lr (before rounding of p - lr) whatever the
// gradient's size, and a weight whose blend is zero keeps its bits.
//
// 20 bytes of HBM traffic per element (p, g, m read; p, m written). Each
// block streams 4096 consecutive elements of one segment with 16-byte loads,
// all loads of a thread issued before its arithmetic; one launch covers
// every segment through the table in the kernel arguments.
#include "lion.hpp"

namespace ma {

__device__ __forceinline__ void lion_elem(float& p, float g, float& m, const LionSeg& S) {
  if (S.decay) p = __fmul_rn(p, S.cd);
  const float c = __fadd_rn(__fmul_rn(S.b1, m), __fmul_rn(S.c1, g));
  const float s = c > 0.f ? 1.f : (c < 0.f ? -1.f : (c == c ? 0.f : c));
  p = __fsub_rn(p, __fmul_rn(S.lr, s));
  m = __fadd_rn(__fmul_rn(S.b2, m), __fmul_rn(S.c2, g));
}

__global__ void __launch_bounds__(256) k_lion(const LionArgs a) {
  const int64_t b = blockIdx.x;
  int si = 0;
#pragma unroll
  for (int q = 1; q < kMaxLionSegs; ++q)
    if (q < a.nseg && b >= a.s[q].block_begin) si = q;
  const LionSeg& S = a.s[si];
  const int64_t e0 = (b - S.block_begin) * kLionBlockElems;
  const int tid = threadIdx.x;
  if (S.vec) {
    constexpr int U = kLionBlockElems / (256 * 4);
    float4 p[U], g[U], m[U];
    bool full[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = e0 + (int64_t)(u * 256 + tid) * 4;
      full[u] = i + 4 <= S.n;
      if (full[u]) {
        p[u] = ld16f<true>(S.p + i);
        g[u] = ld16f<true>(S.g + i);
        m[u] = ld16f<true>(S.m + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = e0 + (int64_t)(u * 256 + tid) * 4;
      if (full[u]) {
        lion_elem(p[u].x, g[u].x, m[u].x, S);
        lion_elem(p[u].y, g[u].y, m[u].y, S);
        lion_elem(p[u].z, g[u].z, m[u].z, S);
        lion_elem(p[u].w, g[u].w, m[u].w, S);
        st16f<true>(S.p + i, p[u]);
        st16f<true>(S.m + i, m[u]);
      } else {
        for (int64_t j = i; j < S.n && j < i + 4; ++j) {
          float pp = S.p[j], mm = S.m[j];
          lion_elem(pp, S.g[j], mm, S);
          S.p[j] = pp; S.m[j] = mm;
        }
      }
    }
  } else {
    for (int64_t j = e0 + tid; j < S.n && j < e0 + kLionBlockElems; j += 256) {
      float pp = S.p[j], mm = S.m[j];
      lion_elem(pp, S.g[j], mm, S);
      S.p[j] = pp; S.m[j] = mm;
    }
  }
}

hipError_t launch_lion(const LionArgs& a, hipStream_t s) {
  if (a.total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_lion, dim3((unsigned)a.total_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ma
