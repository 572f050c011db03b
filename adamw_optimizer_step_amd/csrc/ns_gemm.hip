// Batched Newton-Schulz GEMMs on MFMA (gfx950).
//
// One quintic Newton-Schulz step X <- a X + (b A + c A A) X, A = X X^T, is
// three products ("Chapter 4: The MuonAdamW Optimizer", section "Polar
// Express: Newton-Schulz Orthogonalization"; "3.9 Optimizers ...", section
// "Muon: Orthogonalizing the Update"). Every iterate X (m x n, m <= n) is kept
// in two layouts, X and X^T, so that all three are of one form,
//     C[i][j] = sum_k P[i][k] * Q[j][k]        (both operands K-contiguous):
//   GRAM  A  = X X^T        P = Q = X       K = n   A symmetric: tiles bi <= bj
//   POLY  B  = b A + c A A  P = Q = A       K = m   A A = A A^T; B symmetric
//   AXPY  X' = a X + B X    P = B, Q = X^T  K = m   writes X' and X'^T
// The epilogues fuse the a/b/c combination and the mirrored or dual-layout
// stores, staged through LDS so that global stores are 16-byte coalesced.
//
// Kernel shape: 256 threads = 4 waves in a 2x2 grid; each wave owns a
// (BM/2) x (BN/2) sub-tile made of 32x32 MFMA blocks (bf16:
// v_mfma_f32_32x32x16_bf16, fp32: v_mfma_f32_32x32x2_f32). P and Q tiles of
// BM x BK and BN x BK are double-buffered in LDS with a 16-byte row pad
// (conflict-free 16-byte fragment reads); global loads of the next K tile
// are issued before the MFMAs of the current one. The block index is
// remapped so that each of the 8 XCDs walks a contiguous run of tiles (tiles
// of one matrix share its L2).
#include "ns_gemm.hpp"

namespace ma {

template <int DT> struct MfmaTraits;
template <> struct MfmaTraits<DT_BF16> {
  using T = uint16_t;
  static constexpr int kElem = 2;
  static constexpr int kFragK = 16;   // K covered by one fragment read (two lane halves)
  static constexpr int kLaneK = 8;    // elements per lane per fragment read (16 bytes)
  static constexpr int kPad = 8;      // LDS row pad, elements
};
template <> struct MfmaTraits<DT_F32> {
  using T = float;
  static constexpr int kElem = 4;
  static constexpr int kFragK = 8;    // four 32x32x2 MFMAs per fragment read
  static constexpr int kLaneK = 4;
  static constexpr int kPad = 4;
};

// acc += P_frag * Q_frag over the K slice of one fragment read. Lane l holds
// row/col (l % 32) and K slots h*kLaneK .. h*kLaneK + kLaneK-1 (h = l / 32) of
// its operand; both operands use the same slot-to-k assignment, so the sum
// over the slice is complete whatever order the unit adds the slots in.
template <int DT>
__device__ __forceinline__ void mfma_frag(f32x16_t& acc, const uint4& a, const uint4& b) {
  if constexpr (DT == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
}

template <int DT, int BM, int BN, int BK>
struct NsSmem {
  using Tr = MfmaTraits<DT>;
  static constexpr int LDK = BK + Tr::kPad;
  static constexpr int STAGE = (BM + BN) * LDK;
  static constexpr int MAIN = 2 * STAGE * Tr::kElem;
  static constexpr int LDT = BM + Tr::kPad;   // staging S_T[BN][LDT]: rows j, contiguous i
  static constexpr int LDN = BN + Tr::kPad;   // staging S_N[BM][LDN]: rows i, contiguous j
  static constexpr int EPI = (BN * LDT > BM * LDN ? BN * LDT : BM * LDN) * Tr::kElem;
  static constexpr int BYTES = MAIN > EPI ? MAIN : EPI;
};

template <int DT, int EPI, int BM, int BN, int BK>
__global__ void __launch_bounds__(256) ns_gemm_kernel(const NsArgs args) {
  using Tr = MfmaTraits<DT>;
  using T = typename Tr::T;
  using SM = NsSmem<DT, BM, BN, BK>;
  constexpr int LDK = SM::LDK;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int VEC = 16 / Tr::kElem;     // elements per 16-byte vector
  constexpr int VPR = BK / VEC;           // vectors per tile row
  constexpr int PV = BM * VPR / 256;
  constexpr int QV = BN * VPR / 256;
  static_assert(BM * VPR % 256 == 0 && BN * VPR % 256 == 0, "tile/thread mismatch");
  static_assert(BK % Tr::kFragK == 0, "BK");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];

  // ---- job -> (group, matrix, tile) ---------------------------------------
  const int per_xcd = args.padded_blocks >> 3;
  const int job = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (job >= args.total_jobs) return;
  int gi = 0;
#pragma unroll
  for (int q = 1; q < kMaxNsGroups; ++q)
    if (q < args.n_groups && job >= args.g[q].block_begin) gi = q;
  const NsGroup& G = args.g[gi];
  const int local = job - G.block_begin;
  const int mat = local / G.tiles;
  int t = local - mat * G.tiles;
  int bi, bj;
  if (G.symmetric) {
    bi = 0;
    int len = G.tm;
    while (t >= len) { t -= len; ++bi; --len; }
    bj = bi + t;
  } else {
    bi = t / G.tn;
    bj = t - bi * G.tn;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  const T* __restrict__ Pg = reinterpret_cast<const T*>(G.P) + (int64_t)mat * G.sP + (int64_t)bi * BM * G.ldP;
  const T* __restrict__ Qg = reinterpret_cast<const T*>(G.Q) + (int64_t)mat * G.sQ + (int64_t)bj * BN * G.ldQ;
  const int ldP = G.ldP, ldQ = G.ldQ;

  T* sbase = reinterpret_cast<T*>(smem);

  uint4 rp[PV], rq[QV];
#define MA_NS_GLOAD(k0)                                                                   \
  do {                                                                                    \
    _Pragma("unroll") for (int v = 0; v < PV; ++v) {                                      \
      const int idx_ = tid + 256 * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                \
      rp[v] = *reinterpret_cast<const uint4*>(Pg + (int64_t)row_ * ldP + (k0) + ch_ * VEC); \
    }                                                                                     \
    _Pragma("unroll") for (int v = 0; v < QV; ++v) {                                      \
      const int idx_ = tid + 256 * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                \
      rq[v] = *reinterpret_cast<const uint4*>(Qg + (int64_t)row_ * ldQ + (k0) + ch_ * VEC); \
    }                                                                                     \
  } while (0)
#define MA_NS_SSTORE(stage)                                                               \
  do {                                                                                    \
    T* sP_ = sbase + (stage) * SM::STAGE;                                                 \
    T* sQ_ = sP_ + BM * LDK;                                                              \
    _Pragma("unroll") for (int v = 0; v < PV; ++v) {                                      \
      const int idx_ = tid + 256 * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                \
      *reinterpret_cast<uint4*>(sP_ + row_ * LDK + ch_ * VEC) = rp[v];                     \
    }                                                                                     \
    _Pragma("unroll") for (int v = 0; v < QV; ++v) {                                      \
      const int idx_ = tid + 256 * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                \
      *reinterpret_cast<uint4*>(sQ_ + row_ * LDK + ch_ * VEC) = rq[v];                     \
    }                                                                                     \
  } while (0)

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#define MA_NS_COMPUTE(stage)                                                                  \
  do {                                                                                        \
    const T* sP_ = sbase + (stage) * SM::STAGE;                                               \
    const T* sQ_ = sP_ + BM * LDK;                                                            \
    _Pragma("unroll") for (int kk = 0; kk < BK / Tr::kFragK; ++kk) {                          \
      uint4 fa[FM], fb[FN];                                                                   \
      const int koff = kk * Tr::kFragK + lh * Tr::kLaneK;                                     \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
        fa[i] = *reinterpret_cast<const uint4*>(sP_ + (wm * WTM + i * 32 + l32) * LDK + koff); \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                          \
        fb[j] = *reinterpret_cast<const uint4*>(sQ_ + (wn * WTN + j * 32 + l32) * LDK + koff); \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) mfma_frag<DT>(acc[i][j], fa[i], fb[j]); \
    }                                                                                         \
  } while (0)

  const int nk = G.K / BK;
  MA_NS_GLOAD(0);
  MA_NS_SSTORE(0);
  __syncthreads();
  int cur = 0;
  for (int kt = 0; kt + 1 < nk; ++kt) {
    MA_NS_GLOAD((kt + 1) * BK);
    MA_NS_COMPUTE(cur);
    MA_NS_SSTORE(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }
  MA_NS_COMPUTE(cur);
  __syncthreads();   // every wave is done with the operand tiles; LDS is reused below
#undef MA_NS_GLOAD
#undef MA_NS_COMPUTE
#undef MA_NS_SSTORE

  // ---- epilogue ------------------------------------------------------------
  // Accumulator layout of a 32x32 MFMA block: lane l holds column (l % 32)
  // and, in registers 4q..4q+3, rows 8q + 4(l/32) + 0..3.
  const bool diag = G.symmetric && bi == bj;
  T* outT = reinterpret_cast<T*>(G.outT);
  T* outN = diag ? nullptr : reinterpret_cast<T*>(G.outN);

  if constexpr (EPI != EPI_GRAM) {
    // E[j][i..i+3]: A (symmetric) for POLY, X^T for AXPY
    const T* Eg = reinterpret_cast<const T*>(G.E) + (int64_t)mat * G.sE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int jl = wn * WTN + j * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int il = wm * WTM + i * 32 + q * 8 + lh * 4;
          const T* ep = Eg + (int64_t)(bj * BN + jl) * G.ldE + bi * BM + il;
          float e[4];
          if constexpr (DT == DT_BF16) {
            const uint2 u = *reinterpret_cast<const uint2*>(ep);
            e[0] = __uint_as_float(u.x << 16); e[1] = __uint_as_float(u.x & 0xFFFF0000u);
            e[2] = __uint_as_float(u.y << 16); e[3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else {
            const float4 u = *reinterpret_cast<const float4*>(ep);
            e[0] = u.x; e[1] = u.y; e[2] = u.z; e[3] = u.w;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (EPI == EPI_POLY)
              acc[i][j][4 * q + r] = __builtin_fmaf(args.b, e[r], args.c * acc[i][j][4 * q + r]);
            else
              acc[i][j][4 * q + r] = __builtin_fmaf(args.a, e[r], acc[i][j][4 * q + r]);
          }
        }
      }
  }

  T* stg = reinterpret_cast<T*>(smem);
  if (outT) {
    // stage S_T[j][i] (rows j, contiguous i), then 16-byte stores of C^T rows
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int jl = wn * WTN + j * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int il = wm * WTM + i * 32 + q * 8 + lh * 4;
          if constexpr (DT == DT_BF16) {
            uint2 u;
            u.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            u.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<uint2*>(stg + jl * SM::LDT + il) = u;
          } else {
            *reinterpret_cast<float4*>(stg + jl * SM::LDT + il) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
        }
      }
    __syncthreads();
    T* dst = outT + (int64_t)mat * G.sT + (int64_t)(bj * BN) * G.ldT + bi * BM;
    constexpr int CPR = BM / VEC;   // 16-byte chunks per staged row
#pragma unroll
    for (int u = 0; u < BN * CPR / 256; ++u) {
      const int idx = tid + 256 * u, r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(dst + (int64_t)r * G.ldT + ch * VEC) =
          *reinterpret_cast<const uint4*>(stg + r * SM::LDT + ch * VEC);
    }
    if (outN) __syncthreads();
  }
  if (outN) {
    // stage S_N[i][j] (rows i, contiguous j), then 16-byte stores of C rows
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int jl = wn * WTN + j * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int il = wm * WTM + i * 32 + q * 8 + lh * 4;
          if constexpr (DT == DT_BF16) {
            const uint32_t p01 = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            const uint32_t p23 = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            stg[(il + 0) * SM::LDN + jl] = (uint16_t)(p01 & 0xFFFFu);
            stg[(il + 1) * SM::LDN + jl] = (uint16_t)(p01 >> 16);
            stg[(il + 2) * SM::LDN + jl] = (uint16_t)(p23 & 0xFFFFu);
            stg[(il + 3) * SM::LDN + jl] = (uint16_t)(p23 >> 16);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) stg[(il + r) * SM::LDN + jl] = acc[i][j][4 * q + r];
          }
        }
      }
    __syncthreads();
    T* dst = outN + (int64_t)mat * G.sN + (int64_t)(bi * BM) * G.ldN + bj * BN;
    constexpr int CPR = BN / VEC;
#pragma unroll
    for (int u = 0; u < BM * CPR / 256; ++u) {
      const int idx = tid + 256 * u, r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(dst + (int64_t)r * G.ldN + ch * VEC) =
          *reinterpret_cast<const uint4*>(stg + r * SM::LDN + ch * VEC);
    }
  }
}

template <int DT, int EPI, int BM, int BN, int BK>
static hipError_t launch_one(const NsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ns_gemm_kernel<DT, EPI, BM, BN, BK>), dim3(a.padded_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int BM, int BN, int BK>
static hipError_t launch_epi(int epi, const NsArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_GRAM: return launch_one<DT, EPI_GRAM, BM, BN, BK>(a, s);
    case EPI_POLY: return launch_one<DT, EPI_POLY, BM, BN, BK>(a, s);
    case EPI_AXPY: return launch_one<DT, EPI_AXPY, BM, BN, BK>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_ns_gemm(int dtype, int epi, NsTile tile, const NsArgs& a, hipStream_t s) {
  if (a.padded_blocks <= 0) return hipSuccess;
  if (dtype == DT_BF16) {
    if (tile.bm == 128 && tile.bn == 128 && tile.bk == 64) return launch_epi<DT_BF16, 128, 128, 64>(epi, a, s);
    if (tile.bm == 256 && tile.bn == 256 && tile.bk == 64) return launch_epi<DT_BF16, 256, 256, 64>(epi, a, s);
  } else {
    if (tile.bm == 128 && tile.bn == 128 && tile.bk == 32) return launch_epi<DT_F32, 128, 128, 32>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ma
