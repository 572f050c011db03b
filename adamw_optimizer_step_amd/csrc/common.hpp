// Shared device helpers and launch descriptors of the Muon + AdamW library.
// Target: AMD Instinct MI355X (gfx950, CDNA4), 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace ma {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kPad = 256;          // workspace matrices are padded to multiples of this
constexpr int kMaxMatsPerLaunch = 64;

// storage codes (match ma_dtype)
constexpr int DT_F32 = 0;
constexpr int DT_BF16 = 1;

__host__ __device__ constexpr int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ----------------------------------------------------------------------------
// bf16 <-> fp32
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round-to-nearest-even fp32 -> bf16 of two values, packed low|high<<16
// (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// 16-byte loads and stores, optionally non-temporal (`nt`): for data a step
// touches once (gradients, optimizer state, parameters, the final update), so
// that it neither displaces the iteration's operands in the caches nor leaves
// dirty lines for the next kernel's traffic to wait behind.
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (NT) {
    const u32x4_nt_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, const uint4& x) {
  if constexpr (NT) {
    const u32x4_nt_t y = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(y, reinterpret_cast<u32x4_nt_t*>(p));
  } else {
    *reinterpret_cast<uint4*>(p) = x;
  }
}
template <bool NT>
__device__ __forceinline__ float4 ld16f(const void* p) {
  const uint4 u = ld16<NT>(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
template <bool NT>
__device__ __forceinline__ void st16f(void* p, const float4& x) {
  st16<NT>(p, make_uint4(__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)));
}

// Non-temporal access for the data the Muon elementwise kernels touch once.
constexpr bool kNT = true;

// load / store n consecutive elements of storage type DT as fp32 (n = 8: one
// 16-byte vector for bf16, two for fp32). Pointers must be 16-byte aligned.
template <int DT, bool NT = false>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    uint4 u = ld16<NT>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    float4 a = ld16f<NT>(p);
    float4 b = ld16f<NT>(reinterpret_cast<const float4*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int DT, bool NT = false>
__device__ __forceinline__ void store8(void* p, const float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    st16<NT>(p, u);
  } else {
    st16f<NT>(p, make_float4(v[0], v[1], v[2], v[3]));
    st16f<NT>(reinterpret_cast<float4*>(p) + 1, make_float4(v[4], v[5], v[6], v[7]));
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if constexpr (DT == DT_BF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}

template <int DT>
__device__ __forceinline__ void store1(void* p, int64_t i, float x) {
  if constexpr (DT == DT_BF16) reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  else reinterpret_cast<float*>(p)[i] = x;
}

template <int DT> constexpr int elem_bytes() { return DT == DT_BF16 ? 2 : 4; }

// ----------------------------------------------------------------------------
// The Muon update of one weight (cautious decoupled decay, then the step):
//   mask = cautious ? (u*w >= 0) : true
//   w1 = (decay && mask) ? w - c_wd*w : w;   return w1 - c_lr*u
// one binary32 rounding per operation, no contraction (cautious weight decay
// of the nanochat discussion "Stuck at the optimizer after figuring out
// backward()", reply by mira687; decay and step both read the weight before
// the update, "Chapter 4: The MuonAdamW Optimizer", section "The Full Muon
// Step"). Shared by the update kernels and the fused update of the last
// Newton-Schulz product, so that both give the same bits.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float muon_update(float w, float u, float c_lr, float c_wd, bool cautious, bool decay) {
  const bool mask = cautious ? (__fmul_rn(u, w) >= 0.0f) : true;
  const float w1 = (decay && mask) ? __fsub_rn(w, __fmul_rn(c_wd, w)) : w;
  return __fsub_rn(w1, __fmul_rn(c_lr, u));
}

// ----------------------------------------------------------------------------
// wavefront reduction (fixed order: butterfly over the 64 lanes)
// ----------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

}  // namespace ma
