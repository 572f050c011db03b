// Batched Newton-Schulz GEMMs on MFMA (gfx950).
//
// One quintic Newton-Schulz step X <- a X + (b A + c A A) X, A = X X^T, is
// three products ("Chapter 4: The MuonAdamW Optimizer", section "Polar
// Express: Newton-Schulz Orthogonalization"; "3.9 Optimizers ...", section
// "Muon: Orthogonalizing the Update"). All three are of one form,
//     C[i][j] = sum_k P[i][k] * Q[j][k]:
//   GRAM  A  = X X^T        P = Q = X       K = n   A symmetric: tiles bi <= bj
//   POLY  B  = b A + c A A  P = Q = A       K = m   A A = A A^T; B symmetric
//   AXPY  X' = a X + B X    P = B, Q = X^T  K = m
// with the iterate X (m x n, m <= n) row-major. P and Q are read as
// K-contiguous rows, except AXPY's Q in the 8-wave bf16 kernel: its k-tiles
// are rows of X, and the fragments come from transposing LDS reads, so X^T is
// never stored (AXPY writes X' only). The fp32 kernel reads an X^T copy,
// which its AXPY writes beside X'. The epilogues fuse the a/b/c combination
// and the mirrored or dual-layout stores, staged through LDS so that global
// stores are 16-byte coalesced.
//
// Two kernels share the job mapping and the epilogue:
//  * ns_gemm_dma (bf16): 256 x 256 block tile, 8 waves of 128 x 64, two per
//    SIMD (32x32x16 MFMAs, 8 accumulator blocks per wave). Operand tiles of 256 x 64 move from global
//    memory straight into a 2-stage LDS ring with global_load_lds_dwordx4 (no
//    VGPR staging), one tile ahead of the one being multiplied; 16-byte chunks
//    are XOR-swizzled by row so that the fragment reads are conflict-free.
//    Blocks are persistent, one per CU, each walking a fixed share of its
//    XCD's tile list. In a diagonal tile of GRAM or POLY the two waves below
//    the diagonal skip the K loop; the epilogue mirrors their quadrant.
//  * ns_gemm_reg: a register-staged double-buffered kernel, 128 x 128 x 32
//    tiles of 2 x 2 waves (64 x 64 x 32 for launches with few jobs): every
//    fp32 product on 32x32x2 fp32 MFMAs, and bf16 Gram and POLY launches of
//    few jobs on 32x32x16 bf16 MFMAs.
// Blocks are dealt to the 8 XCDs so that each XCD gets an eighth of every
// shape group, whole matrices at a time where possible (see NsArgs).
#include "ns_gemm.hpp"

#include <type_traits>

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
__device__ __forceinline__ void mfma_frag(f32x16_t& acc, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (DT == DT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), acc, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// job -> (group, matrix, tile)
// ---------------------------------------------------------------------------
struct TileJob {
  int gi, mat, bi, bj;
};

// Job `local` of XCD x's list (see NsArgs); false past its end.
__device__ __forceinline__ bool map_job_at(const NsArgs& args, int x, int local, TileJob& J) {
  // walk the groups in order; XCD x owns units u0, u0+8, ... of each, where
  // u0 = (x - rot) mod 8. Not unrolled: a persistent caller would otherwise
  // keep every group's fields live in scalar registers across its job loop.
#pragma unroll 1
  for (int q = 0; q < kMaxNsGroups; ++q) {
    if (q >= args.n_groups) return false;
    const NsGroup& G = args.g[q];
    const int units = G.count * G.tiles / G.unit;
    const int u0 = (x - G.rot + 8) & 7;
    const int mine = units > u0 ? (units - u0 + 7) / 8 : 0;
    const int njobs = mine * G.unit;
    if (local < njobs) {
      const int unit = u0 + 8 * (local / G.unit);
      const int gjob = unit * G.unit + local % G.unit;
      const int mat = gjob / G.tiles;
      int t = gjob - mat * G.tiles;
      int bi, bj;
      if (G.symmetric) {
        bi = 0;
        int len = G.tm;
        while (t >= len) { t -= len; ++bi; --len; }
        bj = bi + t;
      } else {
        // bands of up to 4 tile rows, walked column by column: the blocks of
        // an XCD working at the same time cover a 4 x 8 patch of tiles, whose
        // 12 operand panels are read in step along K and shared in L2 (a row
        // of 32 tiles would stream 32 distinct panels of Q). The symmetric
        // products gained nothing from the same order.
        constexpr int kBand = 4;
        const int band = t / (kBand * G.tn);
        const int rem = G.tm - band * kBand;
        const int bh = rem < kBand ? rem : kBand;
        const int idx = t - band * kBand * G.tn;
        bj = idx / bh;
        bi = band * kBand + (idx - bj * bh);
      }
      J.gi = q;
      J.mat = mat;
      J.bi = bi;
      J.bj = bj;
      return true;
    }
    local -= njobs;
  }
  return false;
}

__device__ __forceinline__ bool map_job(const NsArgs& args, TileJob& J) {
  return map_job_at(args, (int)(blockIdx.x & 7), (int)(blockIdx.x >> 3), J);
}

// ---------------------------------------------------------------------------
// epilogue: a/b/c combination, then staged, coalesced stores
// ---------------------------------------------------------------------------
// registers 4q..4q+3 of an accumulator block to 4 staging rows, one element
// each (stride `ld` elements)
template <int DT>
__device__ __forceinline__ void stage4_strided(typename MfmaTraits<DT>::T* p, int ld, const f32x16_t& a, int q) {
  if constexpr (DT == DT_BF16) {
    const uint32_t p01 = pack_bf16x2(a[4 * q], a[4 * q + 1]);
    const uint32_t p23 = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
    p[0] = (uint16_t)(p01 & 0xFFFFu);
    p[ld] = (uint16_t)(p01 >> 16);
    p[2 * ld] = (uint16_t)(p23 & 0xFFFFu);
    p[3 * ld] = (uint16_t)(p23 >> 16);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r * ld] = a[4 * q + r];
  }
}

// The fused update (see NsGroup::W; bf16 weights): the weight chunks a lane
// updates are loaded before its wave reads the staged U back from LDS
// (wload), so that their latency overlaps the read-back; each 8-value chunk
// at parameter row pr, columns pc .. pc+7 of matrix `mat` is then updated
// with muon_update and written back (wapply). Both accesses non-temporal.
__device__ __forceinline__ bool w_in(const NsGroup& G, int pr, int pc) { return pr < G.R && pc < G.C; }
__device__ __forceinline__ void wload(const NsGroup& G, int mat, int pr, int pc, uint4& w) {
  if (!w_in(G, pr, pc)) return;   // padding of the iteration buffers
  w = ld16<true>(reinterpret_cast<const uint16_t*>(G.W) + (int64_t)mat * G.sW + (int64_t)pr * G.C + pc);
}
__device__ __forceinline__ void wapply(const NsGroup& G, int mat, int pr, int pc, const uint4& wb, const uint4& ub) {
  if (!w_in(G, pr, pc)) return;
  const uint32_t uw[4] = {ub.x, ub.y, ub.z, ub.w}, ww[4] = {wb.x, wb.y, wb.z, wb.w};
  float u[8], w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u[2 * i] = __uint_as_float(uw[i] << 16);
    u[2 * i + 1] = __uint_as_float(uw[i] & 0xFFFF0000u);
    w[2 * i] = __uint_as_float(ww[i] << 16);
    w[2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = muon_update(w[e], u[e], G.c_lr, G.c_wd, G.cautious != 0, G.decay != 0);
  store8<DT_BF16, true>(reinterpret_cast<uint16_t*>(G.W) + (int64_t)mat * G.sW + (int64_t)pr * G.C + pc, w);
}

template <int DT, int BM, int BN>
struct EpiSmem {
  using Tr = MfmaTraits<DT>;
  static constexpr int LDT = BM + Tr::kPad;   // staging S_T[BN][LDT]: rows j, contiguous i
  static constexpr int LDN = BN + Tr::kPad;   // staging S_N[BM][LDN]: rows i, contiguous j
  static constexpr int BYTES = (BN * LDT > BM * LDN ? BN * LDT : BM * LDN) * Tr::kElem;
};

// Epilogue of the register-staged kernel. Accumulator layout of a 32x32 MFMA
// block: lane l holds column (l % 32) and, in registers 4q..4q+3, rows
// 8q + 4(l/32) + 0..3; the transposed staging then writes 8 bytes per lane,
// the row-major one 2. The caller has finished with LDS (a barrier precedes
// the call).
template <int DT, int EPI, int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void ns_epilogue(const NsArgs& args, const NsGroup& G, const TileJob& J,
                                            f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32], unsigned char* smem) {
  using Tr = MfmaTraits<DT>;
  using T = typename Tr::T;
  using ES = EpiSmem<DT, BM, BN>;
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int VEC = 16 / Tr::kElem;
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, lh = lane >> 5;
  const int mat = J.mat, bi = J.bi, bj = J.bj;
  const bool diag = G.symmetric && bi == bj;
  // a symmetric product writes its tile (bi, bj) and the mirror (bj, bi),
  // the diagonal tiles once (transposed: the cheaper staging; the two are the
  // same block of the same buffer); upper_only drops the mirrors
  T* outT = (G.symmetric && G.upper_only && !diag) ? nullptr : reinterpret_cast<T*>(G.outT);
  T* outN = diag ? nullptr : reinterpret_cast<T*>(G.outN);
  // (il, jl): the output row and column of register 4q of block (i, j)
  auto rc = [&](int i, int j, int q, int& il, int& jl) __attribute__((always_inline)) {
    il = wm * WTM + i * 32 + q * 8 + lh * 4;
    jl = wn * WTN + j * 32 + l32;
  };

  if constexpr (EPI != EPI_GRAM) {
    // E[j][i..i+3]: A (symmetric) for POLY, X^T for AXPY; one 32x32 block at
    // a time, so that the loads of all blocks are not held in registers at once.
    const T* Eg = reinterpret_cast<const T*>(G.E) + (int64_t)mat * G.sE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float e[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int il, jl;
          rc(i, j, q, il, jl);
          const T* ep = Eg + (int64_t)(bj * BN + jl) * G.ldE + bi * BM + il;
          if constexpr (DT == DT_BF16) {
            const uint2 u = *reinterpret_cast<const uint2*>(ep);
            e[q][0] = __uint_as_float(u.x << 16); e[q][1] = __uint_as_float(u.x & 0xFFFF0000u);
            e[q][2] = __uint_as_float(u.y << 16); e[q][3] = __uint_as_float(u.y & 0xFFFF0000u);
          } else {
            const float4 u = *reinterpret_cast<const float4*>(ep);
            e[q][0] = u.x; e[q][1] = u.y; e[q][2] = u.z; e[q][3] = u.w;
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (EPI == EPI_POLY)
              acc[i][j][4 * q + r] = __builtin_fmaf(args.b, e[q][r], args.c * acc[i][j][4 * q + r]);
            else
              acc[i][j][4 * q + r] = __builtin_fmaf(args.a, e[q][r], acc[i][j][4 * q + r]);
          }
        asm volatile("" ::: "memory");
      }
  }
  if constexpr (EPI != EPI_POLY) {
    if (G.scale) {
      // X = s Y with Y in the operand buffers: A = s^2 Y Y^T, X' = s (a Y + B Y)
      float sc = G.scale[(int64_t)mat * G.scale_stride];
      if constexpr (EPI == EPI_GRAM) sc = sc * sc;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= sc;
    }
  }

  T* stg = reinterpret_cast<T*>(smem);
  if (outT) {
    // stage S_T[j][i] (rows j, contiguous i), then 16-byte stores of C^T rows
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int il, jl;
          rc(i, j, q, il, jl);
          if constexpr (DT == DT_BF16) {
            uint2 u;
            u.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            u.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<uint2*>(stg + jl * ES::LDT + il) = u;
          } else {
            *reinterpret_cast<float4*>(stg + jl * ES::LDT + il) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
        }
      }
    T* dst = outT + (int64_t)mat * G.sT + (int64_t)(bj * BN) * G.ldT + bi * BM;
    constexpr int CPR = BM / VEC;   // 16-byte chunks per staged row
    __syncthreads();
#pragma unroll
    for (int u = 0; u < BN * CPR / NT; ++u) {
      const int idx = tid + NT * u, r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(dst + (int64_t)r * G.ldT + ch * VEC) =
          *reinterpret_cast<const uint4*>(stg + r * ES::LDT + ch * VEC);
    }
    if (outN) __syncthreads();
  }
  if (outN) {
    // stage S_N[i][j] (rows i, contiguous j), then 16-byte stores of C rows
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int il, jl;
          rc(i, j, q, il, jl);
          stage4_strided<DT>(stg + il * ES::LDN + jl, ES::LDN, acc[i][j], q);
        }
      }
    T* dst = outN + (int64_t)mat * G.sN + (int64_t)(bi * BM) * G.ldN + bj * BN;
    constexpr int CPR = BN / VEC;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < BM * CPR / NT; ++u) {
      const int idx = tid + NT * u, r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(dst + (int64_t)r * G.ldN + ch * VEC) =
          *reinterpret_cast<const uint4*>(stg + r * ES::LDN + ch * VEC);
    }
  }
}

// ---------------------------------------------------------------------------
// register-staged kernel
// ---------------------------------------------------------------------------
template <int DT, int BM, int BN, int BK>
struct RegSmem {
  using Tr = MfmaTraits<DT>;
  static constexpr int LDK = BK + Tr::kPad;
  static constexpr int STAGE = (BM + BN) * LDK;
  static constexpr int MAIN = 2 * STAGE * Tr::kElem;
  static constexpr int EPI = EpiSmem<DT, BM, BN>::BYTES;
  static constexpr int BYTES = MAIN > EPI ? MAIN : EPI;
};

template <int DT, int EPI, int BM, int BN, int BK, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(1, 2)))
ns_gemm_reg(const NsArgs args) {
  using Tr = MfmaTraits<DT>;
  using T = typename Tr::T;
  using SM = RegSmem<DT, BM, BN, BK>;
  constexpr int NT = 64 * WGM * WGN;      // threads: WGM x WGN waves
  constexpr int LDK = SM::LDK;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int VEC = 16 / Tr::kElem;     // elements per 16-byte vector
  constexpr int VPR = BK / VEC;           // vectors per tile row
  constexpr int PV = BM * VPR / NT;
  constexpr int QV = BN * VPR / NT;
  static_assert(BM * VPR % NT == 0 && BN * VPR % NT == 0, "tile/thread mismatch");
  static_assert(BK % Tr::kFragK == 0, "BK");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];
  TileJob J;
  if (!map_job(args, J)) return;
  const NsGroup& G = args.g[J.gi];
  const int mat = J.mat, bi = J.bi, bj = J.bj;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, lh = lane >> 5;

  const T* __restrict__ Pg = reinterpret_cast<const T*>(G.P) + (int64_t)mat * G.sP + (int64_t)bi * BM * G.ldP;
  const T* __restrict__ Qg = reinterpret_cast<const T*>(G.Q) + (int64_t)mat * G.sQ + (int64_t)bj * BN * G.ldQ;
  const int ldP = G.ldP, ldQ = G.ldQ;

  T* sbase = reinterpret_cast<T*>(smem);

  // two register sets: the global loads of tile k+2 are in flight while tile
  // k is multiplied and tile k+1 moves from registers to LDS
  u32x4_t rp0[PV], rq0[QV], rp1[PV], rq1[QV];
#define MA_NS_GLOAD(RP, RQ, k0)                                                           \
  do {                                                                                    \
    _Pragma("unroll") for (int v = 0; v < PV; ++v) {                                      \
      const int idx_ = tid + NT * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                 \
      RP[v] = *reinterpret_cast<const u32x4_t*>(Pg + (int64_t)row_ * ldP + (k0) + ch_ * VEC); \
    }                                                                                     \
    _Pragma("unroll") for (int v = 0; v < QV; ++v) {                                      \
      const int idx_ = tid + NT * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                 \
      RQ[v] = *reinterpret_cast<const u32x4_t*>(Qg + (int64_t)row_ * ldQ + (k0) + ch_ * VEC); \
    }                                                                                     \
  } while (0)
#define MA_NS_SSTORE(RP, RQ, stage)                                                       \
  do {                                                                                    \
    T* sP_ = sbase + (stage) * SM::STAGE;                                                 \
    T* sQ_ = sP_ + BM * LDK;                                                              \
    _Pragma("unroll") for (int v = 0; v < PV; ++v) {                                      \
      const int idx_ = tid + NT * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                 \
      *reinterpret_cast<u32x4_t*>(sP_ + row_ * LDK + ch_ * VEC) = RP[v];                   \
    }                                                                                     \
    _Pragma("unroll") for (int v = 0; v < QV; ++v) {                                      \
      const int idx_ = tid + NT * v, row_ = idx_ / VPR, ch_ = idx_ % VPR;                 \
      *reinterpret_cast<u32x4_t*>(sQ_ + row_ * LDK + ch_ * VEC) = RQ[v];                   \
    }                                                                                     \
  } while (0)
#define MA_NS_COMPUTE(stage)                                                                  \
  do {                                                                                        \
    const T* sP_ = sbase + (stage) * SM::STAGE;                                               \
    const T* sQ_ = sP_ + BM * LDK;                                                            \
    _Pragma("unroll") for (int kk = 0; kk < BK / Tr::kFragK; ++kk) {                          \
      u32x4_t fa[FM], fb[FN];                                                                 \
      const int koff = kk * Tr::kFragK + lh * Tr::kLaneK;                                     \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
        fa[i] = *reinterpret_cast<const u32x4_t*>(sP_ + (wm * WTM + i * 32 + l32) * LDK + koff); \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                          \
        fb[j] = *reinterpret_cast<const u32x4_t*>(sQ_ + (wn * WTN + j * 32 + l32) * LDK + koff); \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) mfma_frag<DT>(acc[i][j], fa[i], fb[j]); \
    }                                                                                         \
  } while (0)
// keeps the global loads issued above it from being sunk below it
#define MA_NS_PIN() asm volatile("" ::: "memory")

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // K is a multiple of 256, so nk >= 2 for every tile configuration used
  const int nk = G.K / BK;
  MA_NS_GLOAD(rp0, rq0, 0);
  MA_NS_GLOAD(rp1, rq1, BK);
  MA_NS_SSTORE(rp0, rq0, 0);
  __syncthreads();
  // steady state, two k-tiles per trip: tile kt uses stage 0 and register set
  // 0 for its successor's successor, tile kt+1 stage 1 and set 1
  int kt = 0;
  for (; kt + 3 < nk; kt += 2) {
    MA_NS_GLOAD(rp0, rq0, (kt + 2) * BK);
    MA_NS_PIN();
    MA_NS_COMPUTE(0);
    MA_NS_PIN();
    MA_NS_SSTORE(rp1, rq1, 1);
    __syncthreads();
    MA_NS_GLOAD(rp1, rq1, (kt + 3) * BK);
    MA_NS_PIN();
    MA_NS_COMPUTE(1);
    MA_NS_PIN();
    MA_NS_SSTORE(rp0, rq0, 0);
    __syncthreads();
  }
  // tail: tiles kt .. nk-1 (two or three of them); set 1 holds tile kt+1
  if (kt + 2 < nk) {        // three left: kt (stage 0), kt+1 (set 1), kt+2 (to load)
    MA_NS_GLOAD(rp0, rq0, (kt + 2) * BK);
    MA_NS_PIN();
    MA_NS_COMPUTE(0);
    MA_NS_PIN();
    MA_NS_SSTORE(rp1, rq1, 1);
    __syncthreads();
    MA_NS_COMPUTE(1);
    MA_NS_SSTORE(rp0, rq0, 0);
    __syncthreads();
    MA_NS_COMPUTE(0);
  } else {                  // two left: kt (stage 0), kt+1 (set 1)
    MA_NS_COMPUTE(0);
    MA_NS_SSTORE(rp1, rq1, 1);
    __syncthreads();
    MA_NS_COMPUTE(1);
  }
  __syncthreads();   // every wave is done with the operand tiles; LDS is reused below
#undef MA_NS_GLOAD
#undef MA_NS_COMPUTE
#undef MA_NS_PIN
#undef MA_NS_SSTORE

  ns_epilogue<DT, EPI, BM, BN, WGM, WGN>(args, G, J, acc, smem);
}

// ---------------------------------------------------------------------------
// LDS-DMA kernel (bf16): 256 x 256 x BK tiles, 2 x 4 waves of 128 x 64, two
// per SIMD so that one wave's fragment reads and waits overlap the other's
// MFMAs, a ring of STAGES k-tiles in LDS
// ---------------------------------------------------------------------------
namespace dma {
constexpr int BM = 256, BN = 256, BK = 64, STAGES = 2;
constexpr int ROWB = BK * 2;                      // bytes per tile row
constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
constexpr int RPI = 1024 / ROWB;                  // rows per 1 KiB DMA instruction
constexpr int KK = BK / 16;                       // MFMA k-steps per k-tile
constexpr int STAGE_BYTES = (BM + BN) * ROWB;     // P rows 0..255, Q rows 256..511
constexpr int MAIN = STAGES * STAGE_BYTES;
// The epilogue stages each wave's output block through a private area of 64
// rows of LDW values above stage 0 (which may already hold the block's next
// job's first k-tile); rows stay 16-byte aligned
constexpr int LDW = 64 + MfmaTraits<DT_BF16>::kPad;
constexpr int EPI_WAVE = 64 * LDW * 2;
constexpr int EPI_END = STAGE_BYTES + 8 * EPI_WAVE;
constexpr int BYTES = MAIN > EPI_END ? MAIN : EPI_END;
static_assert(BK == 64 && KK == 4, "k-tiles of 64: four MFMA k-steps");
static_assert(STAGES >= 2 && BYTES <= 160 * 1024, "LDS ring must fit in 160 KiB");
// per wave-grid sizes: wave sub-tile WTM x WTN of FM x FN 32x32 blocks; each
// wave fills PANEL consecutive stage rows with DPW 1 KiB DMA instructions
template <int WGM, int WGN>
struct Grid {
  static constexpr int NW = WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int PANEL = (BM + BN) / NW;
  static constexpr int DPW = STAGE_BYTES / NW / 1024;
  static_assert((STAGES - 1) * DPW <= 63, "vmcnt range");
  static_assert(WTM == 128, "the folded term covers 128 output rows per wave");
  static_assert(PANEL % 64 == 0 && BM % PANEL == 0, "panels start at multiples of 64 rows, inside P or Q");
};
// Row r's logical 16-byte chunk c is stored at physical chunk c ^ swz(r).
// An LDS cycle serves 16 lanes of a ds_read_b128: rows r..r+15 (r a
// multiple of 16) at one logical chunk. Rows repeat the 64-bank pattern
// every 256 / ROWB rows, and swz spreads the 16 rows over 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r / (16 / CPR)) & (CPR - 1); }
}  // namespace dma

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
#define MA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// Block barrier for LDS: this wave's LDS accesses are complete, then
// s_barrier. Unlike __syncthreads it does not wait for outstanding global
// loads and stores, so LDS-DMA fills and output stores stay in flight across
// it (a DMA's own landing is waited for with dma_wait_tiles); the memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most `tiles` k-tile DMAs of this wave are outstanding
template <int DPW>
__device__ __forceinline__ void dma_wait_tiles(int tiles) {
  using namespace dma;
  switch (tiles) {
    case 0: MA_WAIT_VMCNT(0); break;
    case 1: MA_WAIT_VMCNT(1 * DPW); break;
    case 2: MA_WAIT_VMCNT((STAGES > 2 ? 2 : 1) * DPW); break;
    case 3: MA_WAIT_VMCNT((STAGES > 3 ? 3 : 1) * DPW); break;
    default: MA_WAIT_VMCNT((STAGES > 4 ? 4 : 1) * DPW); break;
  }
}

// Fragment reads of MFMA k-step kk (16 values of k) of a k-tile: this wave's
// FM 32-row blocks of P (fa) and FN of Q (fb); lane (l32, lh) reads row l32
// of each block at logical chunk 2 kk + lh.
template <int WGM, int WGN, bool QT = false, bool READ_P = true>
__device__ __forceinline__ void dma_read_step(const unsigned char* cur, int kk, int lane, int wm, int wn,
                                              u32x4_t (&fa)[dma::Grid<WGM, WGN>::FM],
                                              u32x4_t (&fb)[dma::Grid<WGM, WGN>::FN]) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  const int l32 = lane & 31, c = kk * 2 + (lane >> 5);
  if constexpr (READ_P) {
#pragma unroll
    for (int i = 0; i < Gd::FM; ++i) {
      const int r = wm * Gd::WTM + i * 32 + l32;
      fa[i] = *reinterpret_cast<const u32x4_t*>(cur + r * ROWB + ((c ^ swz(r)) << 4));
    }
  }
  if constexpr (!QT) {
#pragma unroll
    for (int j = 0; j < Gd::FN; ++j) {
      const int r = BM + wn * Gd::WTN + j * 32 + l32;
      fb[j] = *reinterpret_cast<const u32x4_t*>(cur + r * ROWB + ((c ^ swz(r)) << 4));
    }
  }
}

// Q read transposed (QT): the Q half of a stage holds 64 rows k of Q^T (row
// pitch 512 bytes: 256 values j), 16-byte chunk c of row k stored at chunk
// c ^ (4 (k % 4)). ds_read_b64_tr_b16 works on groups of 16 lanes: lane
// 4a + b of a group addresses 4 values (a row, 4 consecutive columns) and
// receives value b' of the addresses of lanes 4e + a' (e = 0..3), where
// 4a' + b' is its own index in the group. With lane 4a + b addressing row
// r0 + a, columns c0 + 4b .. +3, lane 4a' + b' receives column c0 + 4a' + b'
// of rows r0 .. r0 + 3. Two such reads per 32 columns give lane (l32, lh)
// the values k = 16 kk + 8 lh + 0..7 of column l32, in the slot order of the
// P fragments. qoff[j] (per lane, bytes from the Q half) addresses row
// 8 (g / 2) + a, columns 32 j' + 16 (g % 2) + 4 b of block j, g = lane / 16;
// the row offsets 16 kk and 16 kk + 4 are immediates. The reads wait for
// their results inside the statement.
constexpr int QT_HALF = dma::BM * dma::ROWB;   // byte offset of the Q half in a stage
template <int KK>
__device__ __forceinline__ void qtr_read(const unsigned char* stage, const uint32_t (&qoff)[2], u32x4_t (&fb)[2]) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) const unsigned char lds_cu8_t;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_cu8_t*)stage + QT_HALF;
  u32x2_t r00, r01, r10, r11;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r00), "=&v"(r01), "=&v"(r10), "=&v"(r11)
      : "v"(base + qoff[0]), "v"(base + qoff[1]), "i"(KK * 16 * 512), "i"((KK * 16 + 4) * 512)
      : "memory");
  fb[0] = u32x4_t{r00.x, r00.y, r01.x, r01.y};
  fb[1] = u32x4_t{r10.x, r10.y, r11.x, r11.y};
}

// P and Q both read transposed (PT phase of AXPY): P's k-tile is 64 rows k of
// the stored upper triangle of B (B[k][i] = B[i][k]) in the P half, laid out
// like the Q half; poff[f] addresses fragment f (32 values i). Twelve reads,
// one wait.
template <int KK>
__device__ __forceinline__ void pqtr_read(const unsigned char* stage, const uint32_t (&poff)[4], const uint32_t (&qoff)[2],
                                          u32x4_t (&fa)[4], u32x4_t (&fb)[2]) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) const unsigned char lds_cu8_t;
  const uint32_t base = (uint32_t)(uintptr_t)(lds_cu8_t*)stage;
  u32x2_t p00, p01, p10, p11, p20, p21, p30, p31, q00, q01, q10, q11;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12 offset:%18\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:%19\n\t"
      "ds_read_b64_tr_b16 %2, %13 offset:%18\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:%19\n\t"
      "ds_read_b64_tr_b16 %4, %14 offset:%18\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:%19\n\t"
      "ds_read_b64_tr_b16 %6, %15 offset:%18\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%19\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:%21\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(p00), "=&v"(p01), "=&v"(p10), "=&v"(p11), "=&v"(p20), "=&v"(p21), "=&v"(p30), "=&v"(p31),
        "=&v"(q00), "=&v"(q01), "=&v"(q10), "=&v"(q11)
      : "v"(base + poff[0]), "v"(base + poff[1]), "v"(base + poff[2]), "v"(base + poff[3]),
        "v"(base + QT_HALF + qoff[0]), "v"(base + QT_HALF + qoff[1]),
        "i"(KK * 16 * 512), "i"((KK * 16 + 4) * 512), "i"(KK * 16 * 512), "i"((KK * 16 + 4) * 512)
      : "memory");
  fa[0] = u32x4_t{p00.x, p00.y, p01.x, p01.y};
  fa[1] = u32x4_t{p10.x, p10.y, p11.x, p11.y};
  fa[2] = u32x4_t{p20.x, p20.y, p21.x, p21.y};
  fa[3] = u32x4_t{p30.x, p30.y, p31.x, p31.y};
  fb[0] = u32x4_t{q00.x, q00.y, q01.x, q01.y};
  fb[1] = u32x4_t{q10.x, q10.y, q11.x, q11.y};
}

// This wave's DMA of one k-tile (its panel of the stage: PANEL rows of P or
// Q) into `fill`. Instruction q covers rows
// q*RPI .. q*RPI+RPI-1 of the wave's panel; lane i lands at byte 1024 q + 16 i
// (row q*RPI + i/CPR, physical chunk i%CPR) and so loads logical chunk
// (i%CPR) ^ swz(row) from memory: lane_off[q & 1] holds that offset.
// q_step: elements between the sources of consecutive instructions (RPI
// rows); koff: the k-tile's offset in elements. With Q read transposed, a Q
// wave's instruction covers 2 rows of 512 bytes instead (q_step = 2 rows,
// koff = k0 rows).
template <int DPW>
__device__ __forceinline__ void dma_issue(unsigned char* fill, const uint16_t* src, int64_t q_step,
                                          const int (&lane_off)[2], int64_t koff) {
#pragma unroll
  for (int q = 0; q < DPW; ++q)
    __builtin_amdgcn_global_load_lds(src + q * q_step + lane_off[q & 1] + koff, (lds_void_t*)(fill + q * 1024), 16, 0, 0);
}

// One DMA instruction q of this wave's share of a k-tile (see dma_issue)
__device__ __forceinline__ void dma_issue_one(unsigned char* fill, const uint16_t* src, int64_t q_step,
                                              const int (&lane_off)[2], int64_t koff, int q) {
  __builtin_amdgcn_global_load_lds(src + q * q_step + lane_off[q & 1] + koff, (lds_void_t*)(fill + q * 1024), 16, 0, 0);
}

// acc += P-block Q-block^T, accumulated transposed: with Q as the MFMA's
// first operand each lane holds 4 consecutive columns of one output row, so
// the row-major output is staged 8 bytes per lane (the product of each pair
// of values, and the order of the sums, are the same either way)
__device__ __forceinline__ void mfma_pq(f32x16_t& acc, const u32x4_t& p, const u32x4_t& q) {
  mfma_frag<DT_BF16>(acc, q, p);
}

// MFMAs of one k-step for accumulator rows [I0, I1)
template <int I0, int I1, int FM, int FN>
__device__ __forceinline__ void mfma_rows(f32x16_t (&acc)[FM][FN], const u32x4_t (&fa)[FM], const u32x4_t (&fb)[FN]) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) mfma_pq(acc[i][j], fa[i], fb[j]);
}

// acc[II][j] += (a I) X^T-block for k-step h (0 or 1) of row block II, with
// a = a_hi + a_lo (both exact in bf16). Lane (l32, lh) holds k = 16 h + 8 lh + e
// of the block, and row i = l32 of a I is nonzero only at k = i (the same
// registers serve as either MFMA operand: a I is symmetric).
template <int II, int FM, int FN>
__device__ __forceinline__ void ident_step(f32x16_t (&acc)[FM][FN], const u32x4_t (&fb)[FN], int h, int lane,
                                           float a_coef) {
  const int l32 = lane & 31, lh = lane >> 5;
  const float a_hi = __builtin_bit_cast(float, __float_as_uint(a_coef) & 0xFFFF0000u);
  const float a_lo = a_coef - a_hi;
  const uint32_t hi16 = __float_as_uint(a_hi) >> 16;
  const uint32_t lo16 = pack_bf16x2(a_lo, 0.0f) & 0xFFFFu;
  const int e = l32 - 16 * h - 8 * lh;   // the lane's nonzero slot, if in 0..7
  u32x4_t id_hi = {0u, 0u, 0u, 0u}, id_lo = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    id_hi[w] = (e == 2 * w ? hi16 : 0u) | (e == 2 * w + 1 ? hi16 << 16 : 0u);
    id_lo[w] = (e == 2 * w ? lo16 : 0u) | (e == 2 * w + 1 ? lo16 << 16 : 0u);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    mfma_pq(acc[II][j], id_hi, fb[j]);
    mfma_pq(acc[II][j], id_lo, fb[j]);
  }
}

struct DmaCtx {
  unsigned char* smem;
  unsigned char* wave_fill;
  const uint16_t* src;
  int64_t q_step, k_step;   // DMA source step per instruction and per k-tile (elements)
  int ld_src, lane, wm, wn, nk;
  int lane_off[2];
  uint32_t qoff[2];         // transposed Q fragment addresses (QT)
  // P read transposed for k-tiles < pt_end (B stored as its upper triangle:
  // the blocks left of the diagonal come from the blocks above it); the P
  // waves' DMA uses the *_t source for those k-tiles
  int pt_end, dma_t_end;
  const uint16_t* src_t;
  int64_t q_step_t, k_step_t;
  int lane_off_t[2];
  uint32_t poff[4];
  float a;
  // the block's next job, whose k-tile 0 this wave loads into stage 0 after
  // its last k-tile (pre): its source, as src / q_step / lane_off
  bool pre;
  bool n_trans;             // the next job's tile 0 in the transposed (two-row) layout
  const uint16_t* n_src;
  int64_t n_q_step;
  int n_ld;                 // its row pitch: the lane offsets are computed at the issue
};

// k-step KKI of k-tile kt: its MFMAs run on the fragments in (fa, fb) while
// the next k-step's fragments are read into (na, nb). At the last k-step the
// next read is of the next tile, after the barrier that also releases this
// tile's stage to the DMA of tile kt + STAGES.
// IIB >= 0 (folded term): this k-tile's values of k are rows of this wave's
// output blocks IIB + KKI/2, and the Q fragments hold Q[j][i] = X[i][j] (AXPY,
// Q = X^T) or A[i][j] (POLY, A symmetric) for them, so (a I) Q-block adds
// a*X, or (b/c)*A, to the accumulators instead of reading it back in the
// epilogue.
template <int KKI, int IIB, int WGM, int WGN, bool QT, bool PT>
__device__ __forceinline__ void dma_kstep(const DmaCtx& c, int kt,
                                          f32x16_t (&acc)[dma::Grid<WGM, WGN>::FM][dma::Grid<WGM, WGN>::FN],
                                          u32x4_t (&fa)[dma::Grid<WGM, WGN>::FM], u32x4_t (&fb)[dma::Grid<WGM, WGN>::FN],
                                          u32x4_t (&na)[dma::Grid<WGM, WGN>::FM], u32x4_t (&nb)[dma::Grid<WGM, WGN>::FN]) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  constexpr int FM = Gd::FM, FN = Gd::FN, DPW = Gd::DPW;
  const int s_cur = kt % STAGES;
  if constexpr (KKI + 1 < KK) {
    // the first row block goes before the reads, so that the wait for (fa, fb)
    // (read during the previous k-step) is not also a wait for the new reads
    mfma_rows<0, 1>(acc, fa, fb);
    __builtin_amdgcn_sched_barrier(0);
    dma_read_step<WGM, WGN, QT, !PT>(c.smem + s_cur * STAGE_BYTES, KKI + 1, c.lane, c.wm, c.wn, na, nb);
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows<1, FM>(acc, fa, fb);
  } else {
    // this wave's reads of tile kt are complete (on every path, so that the
    // MFMAs below need no wait for them)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if (kt + 1 < c.nk) {
      // tiles up to min(nk-1, kt+STAGES-1) have been issued: tile kt+1 has
      // landed for this wave once only the later ones are outstanding; after
      // the barrier every wave has read all of tile kt, so its stage may be
      // refilled with tile kt+STAGES
      const int later = c.nk - 2 - kt;
      dma_wait_tiles<DPW>(later < STAGES - 2 ? later : STAGES - 2);
      __builtin_amdgcn_s_barrier();
      // the next tile's P fragments, unless they are read transposed below
      if (!PT || kt + 1 >= c.pt_end)
        dma_read_step<WGM, WGN, QT>(c.smem + ((kt + 1) % STAGES) * STAGE_BYTES, 0, c.lane, c.wm, c.wn, na, nb);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the DMA of tile kt+STAGES into the stage just released, one instruction
    // between MFMAs: issued back to back, the four waves' instructions queue
    // at the CU's one texture-address unit and hold up the MFMAs behind them
    const bool fill = kt + STAGES < c.nk;
    unsigned char* fill_at = c.wave_fill + s_cur * STAGE_BYTES;
    // the source layout of the tile being loaded (QT: the P waves' transposed
    // source for the k-tiles left of the diagonal block)
    const bool tsrc = QT && kt + STAGES < c.dma_t_end;
    const uint16_t* src = tsrc ? c.src_t : c.src;
    const int64_t q_step = tsrc ? c.q_step_t : c.q_step;
    const int64_t koff = (int64_t)(kt + STAGES) * (tsrc ? c.k_step_t : c.k_step);
    const int lo[2] = {tsrc ? c.lane_off_t[0] : c.lane_off[0], tsrc ? c.lane_off_t[1] : c.lane_off[1]};
#pragma unroll
    for (int idx = 0; idx < FM * FN; ++idx) {
      mfma_pq(acc[idx / FN][idx % FN], fa[idx / FN], fb[idx % FN]);
#pragma unroll
      for (int q = idx * DPW / (FM * FN); q < (idx + 1) * DPW / (FM * FN); ++q)
        if (fill) dma_issue_one(fill_at, src, q_step, lo, koff, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (IIB >= 0) ident_step<IIB + KKI / 2>(acc, fb, KKI % 2, c.lane, c.a);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (QT) {
    // the next k-step's Q fragments (and, transposed, P's), after this
    // k-step's MFMAs are queued
    if constexpr (KKI + 1 < KK) {
      if constexpr (PT) pqtr_read<KKI + 1>(c.smem + s_cur * STAGE_BYTES, c.poff, c.qoff, na, nb);
      else qtr_read<KKI + 1>(c.smem + s_cur * STAGE_BYTES, c.qoff, nb);
    } else {
      if (kt + 1 < c.nk) {
        if (PT && kt + 1 < c.pt_end) pqtr_read<0>(c.smem + ((kt + 1) % STAGES) * STAGE_BYTES, c.poff, c.qoff, na, nb);
        else qtr_read<0>(c.smem + ((kt + 1) % STAGES) * STAGE_BYTES, c.qoff, nb);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The k-loop of a wave whose output blocks all lie below the diagonal of a
// diagonal tile of a symmetric product: it keeps its part of the pipeline
// (its DMA share of every k-tile, the same waits and block barriers as the
// computing waves) but reads no fragments and issues no MFMAs; the epilogue
// fills its blocks from the transposed blocks above the diagonal.
template <int WGM, int WGN>
__device__ __forceinline__ void dma_skip_ktiles(const DmaCtx& c) {
  using namespace dma;
  constexpr int DPW = Grid<WGM, WGN>::DPW;
  for (int kt = 0; kt < c.nk; ++kt) {
    if (kt + 1 < c.nk) {
      const int later = c.nk - 2 - kt;
      dma_wait_tiles<DPW>(later < STAGES - 2 ? later : STAGES - 2);
      __builtin_amdgcn_s_barrier();
    }
    if (kt + STAGES < c.nk) {
      unsigned char* fill_at = c.wave_fill + (kt % STAGES) * STAGE_BYTES;
      const int lo[2] = {c.lane_off[0], c.lane_off[1]};
#pragma unroll
      for (int q = 0; q < DPW; ++q) dma_issue_one(fill_at, c.src, c.q_step, lo, (int64_t)(kt + STAGES) * c.k_step, q);
    }
  }
}

// One k-tile: KK k-steps, the fragment sets alternating (0, 1) -> (1, 0) -> ...
// so that (f0a, f0b) again hold the next tile's first k-step afterwards.
template <int IIB, int WGM, int WGN, bool QT, bool PT = false>
__device__ __forceinline__ void dma_ktile(const DmaCtx& c, int kt,
                                          f32x16_t (&acc)[dma::Grid<WGM, WGN>::FM][dma::Grid<WGM, WGN>::FN],
                                          u32x4_t (&f0a)[dma::Grid<WGM, WGN>::FM], u32x4_t (&f0b)[dma::Grid<WGM, WGN>::FN],
                                          u32x4_t (&f1a)[dma::Grid<WGM, WGN>::FM], u32x4_t (&f1b)[dma::Grid<WGM, WGN>::FN]) {
  dma_kstep<0, IIB, WGM, WGN, QT, PT>(c, kt, acc, f0a, f0b, f1a, f1b);
  dma_kstep<1, IIB, WGM, WGN, QT, PT>(c, kt, acc, f1a, f1b, f0a, f0b);
  dma_kstep<2, IIB, WGM, WGN, QT, PT>(c, kt, acc, f0a, f0b, f1a, f1b);
  dma_kstep<3, IIB, WGM, WGN, QT, PT>(c, kt, acc, f1a, f1b, f0a, f0b);
}

// Job slot in LDS: the block's next job (gi, mat, bi, bj; gi < 0: none),
// written by wave 0 while its first operand DMA is in flight
__device__ __forceinline__ void put_job(int* slot, bool ok, const TileJob& N) {
  slot[0] = ok ? N.gi : -1;
  slot[1] = N.mat;
  slot[2] = N.bi;
  slot[3] = N.bj;
}

// This wave's DMA context for job J: operand sources, fragment addresses and
// the transposed-read bounds (the pipeline state apart from the accumulators)
template <int EPI, int WGM, int WGN, bool QT>
__device__ __forceinline__ DmaCtx dma_ctx(const NsArgs& args, const TileJob& J, unsigned char* smem, int wave,
                                          int lane) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  constexpr int DPW = Gd::DPW, NW = Gd::NW;
  const NsGroup& G = args.g[J.gi];
  // DMA source of this wave: the first NW/2 waves load P rows
  // [w*PANEL, +PANEL), the others the matching rows of Q; P and Q rows are
  // contiguous in the stage.
  DmaCtx c;
  c.smem = smem;
  c.wave_fill = smem + wave * (DPW * 1024);
  c.lane = lane;
  c.wm = wave / WGN;
  c.wn = wave % WGN;
  c.nk = G.K / BK;   // K is a multiple of 256: nk >= 4, a multiple of 4
  c.a = EPI == EPI_POLY ? args.b / args.c : args.a;
  const bool isP = wave < NW / 2;
  c.ld_src = isP ? G.ldP : G.ldQ;
  if (QT && !isP) {
    // Q read transposed: Q^T row-major ([k][j], pitch ldQ); this wave loads
    // rows k0 + 16 w .. +15 (w = wave - NW/2), columns bj*BN .. +BN, two
    // 512-byte rows per instruction; lane i lands at row i / 32, physical
    // chunk i % 32, so it loads logical chunk (i % 32) ^ (4 (row % 4))
    static_assert(!QT || (NW == 8 && Gd::FN == 2 && BN == 256 && BK == 64 && STAGES == 2), "QT layout");
    c.src = reinterpret_cast<const uint16_t*>(G.Q) + (int64_t)J.mat * G.sQ +
            (int64_t)((wave - NW / 2) * 16) * c.ld_src + (int64_t)J.bj * BN;
    c.q_step = 2 * (int64_t)c.ld_src;
    c.k_step = (int64_t)BK * c.ld_src;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      c.lane_off[par] = (lane >> 5) * c.ld_src + (((lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3))) << 3);
  } else {
    c.src = reinterpret_cast<const uint16_t*>(isP ? G.P : G.Q) + (int64_t)J.mat * (isP ? G.sP : G.sQ) +
            (int64_t)((isP ? J.bi * BM : J.bj * BN) + (wave % (NW / 2)) * Gd::PANEL) * c.ld_src;
    c.q_step = (int64_t)RPI * c.ld_src;
    c.k_step = BK;
    // instruction q adds q*RPI rows; swz of the stage row depends on q only
    // through q & 1 (panels start at multiples of 64 rows)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      c.lane_off[par] = (lane / CPR) * c.ld_src + (((lane % CPR) ^ swz(par * RPI + lane / CPR)) << 3);
  }
  c.pt_end = 0;
  c.dma_t_end = 0;
  if constexpr (QT) {
    // transposed Q fragment addresses (see qtr_read)
    const int g = lane >> 4, a4 = (lane >> 2) & 3, b4 = lane & 3;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = (c.wn * Gd::WTN + j * 32) / 8 + 2 * (g & 1) + (b4 >> 1);
      c.qoff[j] = (uint32_t)((8 * (g >> 1) + a4) * 512 + ((chunk ^ (4 * a4)) << 4) + (b4 & 1) * 8);
    }
    if (G.p_upper) {
      // P = B stored as its upper triangle: for k < bi*BM, B[i][k] = B[k][i]
      // is read transposed from the block above the diagonal, rows k of
      // columns bi*BM .. +BM, exactly as Q is (P half, same swizzle)
      c.pt_end = J.bi * (BM / BK);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int chunk = (c.wm * Gd::WTM + f * 32) / 8 + 2 * (g & 1) + (b4 >> 1);
        c.poff[f] = (uint32_t)((8 * (g >> 1) + a4) * 512 + ((chunk ^ (4 * a4)) << 4) + (b4 & 1) * 8);
      }
      if (isP) {
        c.dma_t_end = c.pt_end;
        c.src_t = reinterpret_cast<const uint16_t*>(G.P) + (int64_t)J.mat * G.sP + (int64_t)(wave * 16) * c.ld_src +
                  (int64_t)J.bi * BM;
        c.q_step_t = 2 * (int64_t)c.ld_src;
        c.k_step_t = (int64_t)BK * c.ld_src;
#pragma unroll
        for (int par = 0; par < 2; ++par)
          c.lane_off_t[par] = (lane >> 5) * c.ld_src + (((lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3))) << 3);
      }
    }
  }
  c.pre = false;
  return c;
}

// The source of this wave's share of job J's tile 0 (dma_ctx's src / q_step /
// lane_off, or its transposed *_t form for a P wave of a QT job with bi > 0),
// as the next job's source of a DmaCtx
template <int WGM, int WGN, bool QT>
__device__ __forceinline__ void dma_next_src(const NsArgs& args, const TileJob& J, int wave, int lane, DmaCtx& c) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  constexpr int NW = Gd::NW;
  const NsGroup& G = args.g[J.gi];
  const bool isP = wave < NW / 2;
  const int ld = isP ? G.ldP : G.ldQ;
  c.pre = true;
  c.n_ld = ld;
  c.n_trans = QT && (!isP || (G.p_upper && J.bi > 0));
  if (QT && (!isP || (G.p_upper && J.bi > 0))) {
    // rows k 0..63 of Q^T (Q waves) or of B's stored upper triangle (P waves
    // left of the diagonal block), two 512-byte rows per instruction
    const uint16_t* base = isP ? reinterpret_cast<const uint16_t*>(G.P) + (int64_t)J.mat * G.sP +
                                     (int64_t)(wave * 16) * ld + (int64_t)J.bi * BM
                               : reinterpret_cast<const uint16_t*>(G.Q) + (int64_t)J.mat * G.sQ +
                                     (int64_t)((wave - NW / 2) * 16) * ld + (int64_t)J.bj * BN;
    c.n_src = base;
    c.n_q_step = 2 * (int64_t)ld;
  } else {
    c.n_src = reinterpret_cast<const uint16_t*>(isP ? G.P : G.Q) + (int64_t)J.mat * (isP ? G.sP : G.sQ) +
              (int64_t)((isP ? J.bi * BM : J.bj * BN) + (wave % (NW / 2)) * Gd::PANEL) * ld;
    c.n_q_step = (int64_t)RPI * ld;
  }
}

// Issue this wave's share of the next job's tile 0 into stage 0 (see
// dma_next_src), the lane offsets computed here from the lane and the pitch,
// so that they are not held in registers through the main loop
template <int DPW>
__device__ __forceinline__ void dma_issue_next(const DmaCtx& c) {
  using namespace dma;
  const int lane = c.lane, ld = c.n_ld;
  int lo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    lo[par] = c.n_trans ? (lane >> 5) * ld + (((lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3))) << 3)
                        : (lane / CPR) * ld + (((lane % CPR) ^ swz(par * RPI + lane / CPR)) << 3);
  dma_issue<DPW>(c.wave_fill, c.n_src, c.n_q_step, lo, 0);
}

// f(std::integral_constant<int, I>()) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// the LDS byte address of a pointer into a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const unsigned char lds_cu8_t;
  return (uint32_t)(uintptr_t)(lds_cu8_t*)p;
}

// LDS accesses of the epilogue staging in asm: before a compiler-visible LDS
// access that it cannot tell apart from the target of an LDS-DMA load in
// flight, the compiler waits for every vector-memory operation, and the
// staging lies above stage 0, where the next job's tile 0 is landing.
// One 8-byte staging write at byte address addr + OFF.
template <int OFF>
__device__ __forceinline__ void lds_write_b64(uint32_t addr, uint32_t lo, uint32_t hi) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = {lo, hi};
  asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(addr), "v"(v), "i"(OFF) : "memory");
}
// Four 16-byte reads at byte addresses addr + u * STEP (u = 0..3), waited
// for inside the statement
template <int STEP>
__device__ __forceinline__ void lds_read4_b128(uint32_t addr, u32x4_t (&v)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:%5\n\t"
      "ds_read_b128 %2, %4 offset:%6\n\t"
      "ds_read_b128 %3, %4 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(addr), "i"(STEP), "i"(2 * STEP), "i"(3 * STEP)
      : "memory");
}

// Epilogue of the LDS-DMA kernel (accumulators transposed, bf16 output): the
// a/b/c combination of ns_epilogue, then each wave writes out its own 128 x 64
// block through its private staging area above stage 0, 64 output rows at a
// time and with no block barrier: it reads back only what it staged, 16
// bytes per lane, so that each store instruction writes eight whole 128-byte
// rows. Stage 0, where the next job's tile 0 may be landing, is not touched.
// S_N (rows i, contiguous j) stages the block itself, S_T (rows j, contiguous
// i) its transpose, for the mirror tile of a symmetric product.
// mirror: a diagonal tile of a symmetric product, whose waves below the
// diagonal (rows 128..255, columns 0..127; skip: this wave is one) ran no
// MFMAs; those rows are the transpose of rows 0..127, columns 128..255, which
// waves (0, 2) and (0, 3) also write out transposed (the tile comes out
// exactly symmetric). sc: the operand scale (GRAM, AXPY; 1 without one),
// loaded before the main loop.
template <int EPI, int WGM, int WGN, bool E_DONE, bool UPD>
__device__ __forceinline__ void dma_epilogue(const NsArgs& args, const NsGroup& G, const TileJob& J,
                                             f32x16_t (&acc)[dma::Grid<WGM, WGN>::FM][dma::Grid<WGM, WGN>::FN],
                                             unsigned char* smem, int tid, bool mirror, bool skip, float sc) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  using T = uint16_t;
  static_assert(!UPD || EPI == EPI_AXPY, "the update is fused into the AXPY only");
  constexpr int WTM = Gd::WTM, WTN = Gd::WTN, FM = Gd::FM, FN = Gd::FN, VEC = 8;
  static_assert(WGM == 2 && WGN == 4 && WTM == 128 && WTN == 64 && FM == 4 && FN == 2, "waves of 128 x 64");
  // an opaque copy of the thread index: the lane-dependent addresses below
  // are then computed here, not kept in registers through the main loop
  int opaque;
  asm volatile("v_mov_b32 %0, %1" : "=v"(opaque) : "v"(tid));
  const int lane = opaque & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, lh = lane >> 5;
  const int mat = J.mat, bi = J.bi, bj = J.bj;
  const bool diag = G.symmetric && bi == bj;
  // a symmetric product writes its tile (bi, bj) and the mirror (bj, bi), the
  // diagonal tiles once; upper_only drops the mirrors
  T* outT = (diag || (G.symmetric && G.upper_only)) ? nullptr : reinterpret_cast<T*>(G.outT);
  T* outN = reinterpret_cast<T*>(G.outN);

  if constexpr (EPI != EPI_GRAM && !E_DONE) {
    // E[i][j..j+3] (= E[j][i..], E = A symmetric): one 32x32 block at a time
    static_assert(EPI == EPI_POLY, "transposed accumulators read E as a symmetric matrix");
    const T* Eg = reinterpret_cast<const T*>(G.E) + (int64_t)mat * G.sE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float e[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int il = wm * WTM + i * 32 + l32, jl = wn * WTN + j * 32 + q * 8 + lh * 4;
          const uint2 u = *reinterpret_cast<const uint2*>(Eg + (int64_t)(bi * BM + il) * G.ldE + bj * BN + jl);
          e[q][0] = __uint_as_float(u.x << 16); e[q][1] = __uint_as_float(u.x & 0xFFFF0000u);
          e[q][2] = __uint_as_float(u.y << 16); e[q][3] = __uint_as_float(u.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][4 * q + r] = __builtin_fmaf(args.b, e[q][r], args.c * acc[i][j][4 * q + r]);
        asm volatile("" ::: "memory");
      }
  }
  if constexpr (EPI != EPI_POLY) {
    // X = s Y with Y in the operand buffers: A = s^2 Y Y^T, X' = s (a Y + B Y)
    if (G.scale) {
      const float s2 = EPI == EPI_GRAM ? sc * sc : sc;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= s2;
    }
  }
  if constexpr (EPI == EPI_POLY && E_DONE) {
    // the main loop accumulated A A + (b/c) A
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] *= args.c;
  }

  // this wave's staging area; lane reads back row rr + 8u (u = 0..7), values
  // rc .. rc+7
  T* const wst = reinterpret_cast<T*>(smem + STAGE_BYTES + wave * EPI_WAVE);
  const int rr = lane >> 3, rc = (lane & 7) * VEC;
  const uint32_t rd = lds_addr(wst + rr * LDW + rc);
  // the block's first output row and column
  const int i0 = bi * BM + wm * WTM, j0 = bj * BN + wn * WTN;
  // The block transposed, half h (block rows h*64 .. +63) at a time: staging
  // row = block column (64), contiguous block rows; stored to rows j0 + 0..63,
  // columns i0 + h*64 .. of the matrix at dst (pitch ld).
  auto store_t = [&](T* dst, int64_t ld, bool upd) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            stage4_strided<DT_BF16>(wst + (j * 32 + q * 8 + lh * 4) * LDW + ii * 32 + l32, LDW, acc[2 * h + ii][j], q);
      uint4 wc[UPD ? 8 : 1];
      if constexpr (UPD) {
        if (upd) {
#pragma unroll
          for (int u = 0; u < 8; ++u) wload(G, mat, j0 + rr + 8 * u, i0 + h * 64 + rc, wc[u]);
        }
      }
      // the weight chunks have landed: one wait here (on every path, so that
      // the compiler knows it), rather than the compiler's wait for
      // everything in flight before each use (the LDS-DMA load in flight
      // makes it count vector-memory operations as unordered)
      if constexpr (UPD) MA_WAIT_VMCNT(0);
      u32x4_t sv[4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u % 4 == 0) lds_read4_b128<8 * LDW * 2>(rd + (u / 4) * (32 * LDW * 2), sv);
        const uint4 v = make_uint4(sv[u % 4][0], sv[u % 4][1], sv[u % 4][2], sv[u % 4][3]);
        *reinterpret_cast<uint4*>(dst + (int64_t)(rr + 8 * u) * ld + h * 64 + rc) = v;
        if constexpr (UPD)
          if (upd) wapply(G, mat, j0 + rr + 8 * u, i0 + h * 64 + rc, wc[u], v);
      }
    }
  };

  if (outT) {
    const bool upd = UPD && G.W && G.w_trans && !(G.nonfinite && G.nonfinite[mat]);
    store_t(outT + (int64_t)mat * G.sT + (int64_t)j0 * G.ldT + i0, G.ldT, upd);
  }
  if (outN && !skip) {
    // the block row-major, half h (block rows h*64 .. +63) at a time: lane
    // (l32, lh) stages block row h*64 + ii*32 + l32 at staging row ii*32 + l32,
    // columns j*32 + q*8 + lh*4 .. +3
    T* const dst = outN + (int64_t)mat * G.sN + (int64_t)i0 * G.ldN + j0;
    const bool upd = UPD && G.W && !G.w_trans && !(G.nonfinite && G.nonfinite[mat]);
    const uint32_t wr = lds_addr(wst + l32 * LDW + lh * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      static_for<0, 2 * FN * 4>([&](auto k) {
        constexpr int ii = decltype(k)::value / (FN * 4), j = decltype(k)::value / 4 % FN, q = decltype(k)::value % 4;
        const f32x16_t& a = acc[2 * h + ii][j];
        lds_write_b64<(ii * 32 * LDW + j * 32 + q * 8) * 2>(wr, pack_bf16x2(a[4 * q], a[4 * q + 1]),
                                                            pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
      });
      uint4 wc[UPD ? 8 : 1];
      if constexpr (UPD) {
        if (upd) {
#pragma unroll
          for (int u = 0; u < 8; ++u) wload(G, mat, i0 + h * 64 + rr + 8 * u, j0 + rc, wc[u]);
        }
      }
      if constexpr (UPD) MA_WAIT_VMCNT(0);   // the weight chunks have landed (as above)
      u32x4_t sv[4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u % 4 == 0) lds_read4_b128<8 * LDW * 2>(rd + (u / 4) * (32 * LDW * 2), sv);
        const int row = h * 64 + rr + 8 * u;
        const uint4 v = make_uint4(sv[u % 4][0], sv[u % 4][1], sv[u % 4][2], sv[u % 4][3]);
        *reinterpret_cast<uint4*>(dst + (int64_t)row * G.ldN + rc) = v;
        if constexpr (UPD)
          if (upd) wapply(G, mat, i0 + row, j0 + rc, wc[u], v);
      }
    }
  }
  // the mirror: output rows j0 + 0..63 (below the diagonal), columns i0 ..
  if (mirror && wm == 0 && wn * WTN >= BN / 2) store_t(outN + (int64_t)mat * G.sN + (int64_t)j0 * G.ldN + i0, G.ldN, false);
}

// One output tile: prologue DMA, main loop, epilogue.
// FOLD: the term that is not a product of the two operands -- a X in AXPY,
// b A in POLY (as (b/c) A, the epilogue then scaling by c; needs c != 0) --
// is added inside the main loop by scaled-identity MFMAs against the Q
// fragments, so the epilogue reads nothing back from global memory. AXPY
// always folds.
// Wave 0 stores job `next_local` of XCD `xcd`'s list in next_slot while the
// first k-tiles land; every wave reads it after the prologue barrier (next,
// have_next).
// Each wave loads its share of the next job's tile 0 into stage 0 (free
// since the barrier after tile nk - 2) once its last k-step's MFMAs are
// issued (DmaCtx::pre), so that the load overlaps their drain and the
// epilogue (which stages above stage 0) instead of queueing behind the
// epilogue's stores; pre_issued: this job's tile 0 was loaded so.
template <int EPI, bool FOLD, int WGM, int WGN, bool QT, bool UPD>
__device__ __forceinline__ void dma_tile(const NsArgs& args, const TileJob& J, unsigned char* smem, int xcd,
                                         int next_local, int* next_slot, bool pre_issued, TileJob& next,
                                         bool& have_next) {
  using namespace dma;
  using Gd = Grid<WGM, WGN>;
  constexpr int FM = Gd::FM, FN = Gd::FN, DPW = Gd::DPW;
  const NsGroup& G = args.g[J.gi];
  // an opaque copy of the thread index: without it the compiler hoists every
  // lane-dependent address of the tile out of a persistent block's job loop
  // and keeps them all live, through the epilogue too
  int opaque;
  asm volatile("v_mov_b32 %0, %1" : "=v"(opaque) : "v"((int)threadIdx.x));
  const int lane = opaque & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int tid = (wave << 6) | lane;
  DmaCtx c = dma_ctx<EPI, WGM, WGN, QT>(args, J, smem, wave, lane);
  // the operand scale (written by an earlier launch), read through the
  // constant address space: a scalar load, which no wait for the DMA in
  // flight holds up
  typedef __attribute__((address_space(4))) const float const_f32_t;
  const float sc = (EPI != EPI_POLY && G.scale) ? *((const_f32_t*)G.scale + (int64_t)J.mat * G.scale_stride) : 1.0f;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Pipeline over k-tiles kt (stage kt % S, S = STAGES): the DMA of tile
  // kt+S is issued during tile kt, once every wave has read all of tile kt,
  // and each k-step's fragments are read while the previous k-step's MFMAs
  // run.
#pragma unroll
  for (int t = 0; t < STAGES; ++t) {
    if (t == 0 && pre_issued) continue;
    if (QT && t < c.dma_t_end)
      dma_issue<DPW>(c.wave_fill + t * STAGE_BYTES, c.src_t, c.q_step_t, c.lane_off_t, (int64_t)t * c.k_step_t);
    else
      dma_issue<DPW>(c.wave_fill + t * STAGE_BYTES, c.src, c.q_step, c.lane_off, (int64_t)t * c.k_step);
  }
  if (wave == 0) {
    // the next job's (scalar) mapping, while the first k-tiles land
    TileJob N;
    const bool ok = map_job_at(args, xcd, next_local, N);
    if (lane == 0) put_job(next_slot, ok, N);
  }
  // this wave's part of tile 0 has landed (tile 0 was issued before tile 1,
  // here or during the previous job: loads land in order), and the slot is
  // written
  dma_wait_tiles<DPW>(STAGES - 1);
  lds_barrier();
  next.gi = __builtin_amdgcn_readfirstlane(next_slot[0]);
  next.mat = __builtin_amdgcn_readfirstlane(next_slot[1]);
  next.bi = __builtin_amdgcn_readfirstlane(next_slot[2]);
  next.bj = __builtin_amdgcn_readfirstlane(next_slot[3]);
  have_next = next.gi >= 0;
  c.n_src = c.src;
  c.n_q_step = c.q_step;
  c.n_ld = 0;
  c.n_trans = false;
  if (have_next) dma_next_src<WGM, WGN, QT>(args, next, wave, lane, c);
  // a diagonal tile of a symmetric product: the waves whose blocks all lie
  // below the diagonal (rows 128..255, columns 0..127) compute nothing
  const bool mirror_lower = !QT && G.symmetric && J.bi == J.bj;
  if (mirror_lower && c.wm * Gd::WTM >= BM / 2 && (c.wn + 1) * Gd::WTN <= BN / 2) {
    static_assert(QT || BM == BN, "square tiles");
    dma_skip_ktiles<WGM, WGN>(c);
    if (c.pre) dma_issue_next<DPW>(c);
    lds_barrier();   // as the other waves' barrier before their epilogue
    return;
  }
  u32x4_t f0a[FM], f0b[FN], f1a[FM], f1b[FN];
  int kt = 0;
  if constexpr (QT) {
    if (c.pt_end > 0) {
      pqtr_read<0>(smem, c.poff, c.qoff, f0a, f0b);
    } else {
      dma_read_step<WGM, WGN, QT>(smem, 0, lane, c.wm, c.wn, f0a, f0b);
      qtr_read<0>(smem, c.qoff, f0b);
    }
    // the k-tiles left of the diagonal block, P read transposed (none of
    // them carries the folded term: those start at bi*BM)
    for (; kt < c.pt_end; ++kt) dma_ktile<-1, WGM, WGN, QT, true>(c, kt, acc, f0a, f0b, f1a, f1b);
  } else {
    dma_read_step<WGM, WGN, QT>(smem, 0, lane, c.wm, c.wn, f0a, f0b);
  }
  if constexpr (FOLD) {
    // the k-tiles whose k range is this wave's 128 output rows (K = m_pad,
    // so they lie inside [0, nk)) carry the a*X (AXPY) or (b/c)*A (POLY)
    // term: Q rows j hold X^T[j][k] = X[k][j], or A[j][k] = A[k][j]
    const int e_first = (J.bi * BM + c.wm * Gd::WTM) / BK;
    for (; kt < e_first; ++kt) dma_ktile<-1, WGM, WGN, QT>(c, kt, acc, f0a, f0b, f1a, f1b);
    dma_ktile<0, WGM, WGN, QT>(c, kt++, acc, f0a, f0b, f1a, f1b);
    dma_ktile<2, WGM, WGN, QT>(c, kt++, acc, f0a, f0b, f1a, f1b);
  }
  for (; kt < c.nk; ++kt) dma_ktile<-1, WGM, WGN, QT>(c, kt, acc, f0a, f0b, f1a, f1b);
  // stage 0 last held tile nk - 2 (nk is a multiple of 4), which every wave
  // had read before the barrier at the end of that tile
  if (c.pre) dma_issue_next<DPW>(c);
  lds_barrier();   // every wave has read the last k-tile (stage 1, reused by the staging)
  dma_epilogue<EPI, WGM, WGN, FOLD, UPD>(args, G, J, acc, smem, tid, mirror_lower, false, sc);
}

// Persistent over its XCD's job list: block b (XCD b % 8, P blocks per XCD)
// runs jobs b/8, b/8 + P, b/8 + 2P, ... of that list. With at most one block
// per CU this saves a block launch and its set-up per tile; the lists hold
// the longest jobs first and, where jobs differ in K, a fixed stride ends
// about as late as taking jobs on demand would (the blocks holding one long
// and two short jobs set the end either way).
// UPD: the AXPY of the last step, which also applies the Muon update to the
// weights of the groups that carry one (NsGroup::W)
template <int EPI, bool FOLD, int WGM, int WGN, bool QT, bool UPD>
__global__ void __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4)))
ns_gemm_dma(const NsArgs args) {
  using namespace dma;
  // one LDS object (see above): the two job slots follow the operand ring /
  // epilogue staging
  __shared__ __attribute__((aligned(1024))) unsigned char smem[BYTES + 32];
  int* const slots = reinterpret_cast<int*>(smem + BYTES);
  // issue priority over waves of other kernels sharing the CU (the AdamW
  // update that may run beside the iteration on another stream, at priority 0)
  __builtin_amdgcn_s_setprio(1);
  const int x = (int)(blockIdx.x & 7);
  const int P = (int)(gridDim.x >> 3);
  TileJob J;
  int local = (int)(blockIdx.x >> 3);
  bool have = map_job_at(args, x, local, J);
  bool pre = false;
  // job j's successor goes to slot (j + 1) & 1: a slot is rewritten two jobs
  // later, after every wave has passed the barriers that follow its reads
  for (int j = 0; have; ++j) {
    int* const slot = slots + 4 * ((j + 1) & 1);
    TileJob N;
    bool more;
    dma_tile<EPI, FOLD, WGM, WGN, QT, UPD>(args, J, smem, x, local + P, slot, pre, N, more);
    // every wave has read the staged output before the next job's DMA lands
    // over it (its tile 0, in stage 0, is already in flight)
    lds_barrier();
    local += P;
    J = N;
    have = more;
    pre = more;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int DT, int EPI, int BM, int BN, int BK, int WGM, int WGN>
static hipError_t launch_reg(const NsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ns_gemm_reg<DT, EPI, BM, BN, BK, WGM, WGN>), dim3(a.padded_blocks), dim3(64 * WGM * WGN),
                     0, s, a);
  return hipGetLastError();
}

template <int DT, int BM, int BN, int BK, int WGM, int WGN>
static hipError_t launch_reg_epi(int epi, const NsArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_GRAM: return launch_reg<DT, EPI_GRAM, BM, BN, BK, WGM, WGN>(a, s);
    case EPI_POLY: return launch_reg<DT, EPI_POLY, BM, BN, BK, WGM, WGN>(a, s);
    case EPI_AXPY:
      // bf16 AXPY always runs the LDS-DMA kernel (it reads X^T out of X)
      if constexpr (DT == DT_F32) return launch_reg<DT, EPI_AXPY, BM, BN, BK, WGM, WGN>(a, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int EPI, bool FOLD, int WGM, int WGN, bool QT = false, bool UPD = false>
static hipError_t launch_dma(const NsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((ns_gemm_dma<EPI, FOLD, WGM, WGN, QT, UPD>), dim3(a.padded_blocks), dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int WGM, int WGN>
static hipError_t launch_dma_epi(int epi, bool qt, const NsArgs& a, hipStream_t s) {
  if (qt) {
    // AXPY with Q read transposed (8-wave form only)
    if constexpr (WGM == 2 && WGN == 4) {
      if (epi == EPI_AXPY) {
        bool upd = false;
        for (int q = 0; q < a.n_groups; ++q) upd = upd || a.g[q].W != nullptr;
        return upd ? launch_dma<EPI_AXPY, true, WGM, WGN, true, true>(a, s)
                   : launch_dma<EPI_AXPY, true, WGM, WGN, true, false>(a, s);
      }
    }
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_GRAM: return launch_dma<EPI_GRAM, false, WGM, WGN>(a, s);
    case EPI_POLY:
      return a.c != 0.0f ? launch_dma<EPI_POLY, true, WGM, WGN>(a, s) : launch_dma<EPI_POLY, false, WGM, WGN>(a, s);
    case EPI_AXPY: return launch_dma<EPI_AXPY, true, WGM, WGN>(a, s);
  }
  return hipErrorInvalidValue;
}

#define MA_REG_TILE(BM_, BN_, BK_, WGM_, WGN_)                                                      \
  if (tile.bm == BM_ && tile.bn == BN_ && tile.bk == BK_ && tile.wgm == WGM_ && tile.wgn == WGN_) \
    return launch_reg_epi<DTv, BM_, BN_, BK_, WGM_, WGN_>(epi, a, s);

int ns_dma_bk() { return dma::BK; }

// ---------------------------------------------------------------------------
// sum of the K slices of a split fp32 Gram product (see SplitSumArgs)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_split_sum(const SplitSumArgs a) {
  const int64_t b = blockIdx.x;
  int q = 0;
#pragma unroll 1
  while (q + 1 < a.n && b >= a.g[q + 1].block_begin) ++q;
  const SplitSumGroup& g = a.g[q];
  const int64_t i = (b - g.block_begin) * kSplitSumBlockElems + (int64_t)threadIdx.x * 4;
  float4 v = *reinterpret_cast<const float4*>(g.part + i);
#pragma unroll 1
  for (int sl = 1; sl < g.slices; ++sl) {
    const float4 w = *reinterpret_cast<const float4*>(g.part + sl * g.split_stride + i);
    v.x = __fadd_rn(v.x, w.x);
    v.y = __fadd_rn(v.y, w.y);
    v.z = __fadd_rn(v.z, w.z);
    v.w = __fadd_rn(v.w, w.w);
  }
  *reinterpret_cast<float4*>(g.out + i) = v;
}

hipError_t launch_split_sum(const SplitSumArgs& a, hipStream_t s) {
  if (a.blocks <= 0) return hipSuccess;
  for (int q = 0; q < a.n; ++q)
    if (a.g[q].mat_elems % kSplitSumBlockElems || a.g[q].slices < 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_split_sum, dim3((unsigned)a.blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ns_gemm(int dtype, int epi, NsTile tile, const NsArgs& a, hipStream_t s) {
  if (a.padded_blocks <= 0) return hipSuccess;
  if (dtype == DT_BF16) {
    if (!tile.dma) {
      // launches of few jobs (GRAM and POLY only): the register-staged kernel
      constexpr int DTv = DT_BF16;
      if (epi == EPI_AXPY || tile.qt) return hipErrorInvalidValue;
      MA_REG_TILE(128, 128, 32, 2, 2)
      MA_REG_TILE(64, 64, 32, 2, 2)
      return hipErrorInvalidValue;
    }
    // the LDS-DMA kernel, 256 x 256 x 64 tiles, 2 x 4 waves
    if (tile.bm != dma::BM || tile.bn != dma::BN || tile.bk != dma::BK || tile.wgm != 2 || tile.wgn != 4)
      return hipErrorInvalidValue;
    return launch_dma_epi<2, 4>(epi, tile.qt != 0, a, s);
  } else {
    constexpr int DTv = DT_F32;
    MA_REG_TILE(128, 128, 32, 2, 2)
    MA_REG_TILE(64, 64, 32, 2, 2)   // launches with few jobs
  }
  return hipErrorInvalidValue;
}
#undef MA_REG_TILE

}  // namespace ma
