// Muon elementwise and reduction kernels (gfx950), HBM-bound.
//
//   k_rowsumsq_rows      per row of the Nesterov look-ahead Mt = G + beta*m1,
//                        m1 = beta*M + G: sum of squares (a wave per row of at
//                        most 4096 columns, all of a lane's 16-byte loads in
//                        flight, butterfly shuffle reduction; no atomics)
//   k_rowsumsq_momentum  the same for longer or unaligned rows (a wave per 4
//                        rows, up to 16 16-byte loads per lane in flight)
//   k_finalize           per matrix: Frobenius scale, MuonEq row factors,
//                        NorMuon row factors
//   k_pre                momentum update M <- m1 (stored), X0 = Mt * f_row,
//                        written in the parameter's layout and transposed
//                        (through an LDS tile) into the Newton-Schulz buffers;
//                        k_pre_t (transposed copy only, wider tiles) and
//                        k_pre_d (parameter's layout only, no tile) are its
//                        one-copy forms
//   k_post               cautious decoupled decay and the update, W <- W'
//
// Sources: momentum and look-ahead -- "Chapter 4: The MuonAdamW Optimizer",
// section "The Muon Update Rule" and "3.9 Optimizers ...", section "From
// Gradient Descent to Momentum"; Frobenius normalisation -- "Chapter 4",
// section "Polar Express: Newton-Schulz Orthogonalization"; cautious mask,
// MuonEq and the lr multiplier -- nanochat discussion "Stuck at the optimizer
// after figuring out backward()", reply by mira687; decay before the update
// -- "Chapter 4", section "The Full Muon Step".
//
// The elementwise arithmetic is binary32 with one rounding per operation and
// no contraction (this file is built with -ffp-contract=off); stores to bf16
// round to nearest even.
#include "muon_elem.hpp"

namespace ma {

template <int DT>
__device__ __forceinline__ const void* eptr(const void* base, int64_t i) {
  return reinterpret_cast<const unsigned char*>(base) + i * elem_bytes<DT>();
}
template <int DT>
__device__ __forceinline__ void* eptr(void* base, int64_t i) {
  return reinterpret_cast<unsigned char*>(base) + i * elem_bytes<DT>();
}

// m1 = beta*m + g;  mt = nesterov ? g + beta*m1 : m1
__device__ __forceinline__ void momentum1(float g, float m, float beta, int nesterov, float& m1,
                                          float& mt) {
  m1 = __fadd_rn(__fmul_rn(beta, m), g);
  mt = nesterov ? __fadd_rn(g, __fmul_rn(beta, m1)) : m1;
}

constexpr int kRowsPerBlock = 16;

// 8 elements of a 16-byte-aligned run, as loaded (two 16-byte words for
// fp32, one for bf16), unpacked only when used
template <int DT>
struct Raw8 {
  uint4 w[DT == DT_BF16 ? 1 : 2];
};
template <int DT, bool NT = false>
__device__ __forceinline__ void raw_load(const void* p, Raw8<DT>& r) {
#pragma unroll
  for (int i = 0; i < (DT == DT_BF16 ? 1 : 2); ++i) r.w[i] = ld16<NT>(reinterpret_cast<const uint4*>(p) + i);
}
template <int DT>
__device__ __forceinline__ float raw_at(const Raw8<DT>& r, int e) {
  if constexpr (DT == DT_BF16) {
    const uint32_t w = r.w[0][e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return __uint_as_float(r.w[e >> 2][e & 3]);
  }
}

// A wave owns 4 consecutive rows of its block's 16. Vector path: the row's
// 512-element chunks (8 per lane) are read CPB at a time for RB rows at once,
// 8 chunks of G and 8 of M per lane in flight, kept packed until used; each
// lane adds its elements in column order, so the sums do not depend on CPB.
template <int DTG, int DTM, int CPB>
__global__ void __launch_bounds__(256) k_rowsumsq_momentum(const ElemArgs a) {
  constexpr int RB = 8 / CPB < 4 ? 8 / CPB : 4;   // rows per batch
  constexpr int NS = RB * CPB;                     // chunk slots per operand
  const int bpm = (a.R + kRowsPerBlock - 1) / kRowsPerBlock;
  const int k = blockIdx.x / bpm;
  const int rb = blockIdx.x - k * bpm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const void* gp = a.mat[k].g;
  const void* mp = a.mat[k].m;
  const int row0 = rb * kRowsPerBlock + wave * 4;
  if (a.vec) {
    const int cpr = (a.C + 511) >> 9;
#pragma unroll 1
    for (int rr = 0; rr < 4; rr += RB) {
      float acc[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) acc[q] = 0.0f;
#pragma unroll 1
      for (int c0 = 0; c0 < cpr; c0 += CPB) {
        Raw8<DTG> g[NS];
        Raw8<DTM> m[NS];
        // every slot loads (out-of-range slots re-read the matrix's first
        // chunk and add nothing), so that all loads issue back to back
        bool ok[NS];
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const int r = row0 + rr + u / CPB, c = (c0 + u % CPB) * 512 + lane * 8;
          ok[u] = r < a.R && c < a.C;
          const int64_t off = ok[u] ? (int64_t)r * a.C + c : 0;
          raw_load<DTG, kNT>(eptr<DTG>(gp, off), g[u]);
          raw_load<DTM, kNT>(eptr<DTM>(mp, off), m[u]);
        }
#pragma unroll
        for (int u = 0; u < NS; ++u) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float m1, mt;
            momentum1(raw_at<DTG>(g[u], e), raw_at<DTM>(m[u], e), a.beta, a.nesterov, m1, mt);
            const float t = __builtin_fmaf(mt, mt, acc[u / CPB]);
            acc[u / CPB] = ok[u] ? t : acc[u / CPB];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const float t = wave_sum(acc[q]);
        const int r = row0 + rr + q;
        if (lane == 0 && r < a.R) a.rowsq[(int64_t)k * a.row_stride + r] = t;
      }
    }
  } else {
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      const int r = row0 + q;
      if (r >= a.R) break;
      const int64_t base = (int64_t)r * a.C;
      float acc = 0.0f;
      for (int c = lane; c < a.C; c += 64) {
        float m1, mt;
        momentum1(load1<DTG>(gp, base + c), load1<DTM>(mp, base + c), a.beta, a.nesterov, m1, mt);
        acc = __builtin_fmaf(mt, mt, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) a.rowsq[(int64_t)k * a.row_stride + r] = acc;
    }
  }
}

// One wave per row, four rows per block, rows of at most 512 CH columns
// (vector path): a lane's CH chunks of G and of M are loaded together, then
// summed in the order k_rowsumsq_momentum uses (its chunks in column order,
// then the butterfly), so both give the same bits. Many small blocks keep the
// loads of the whole launch in flight with no tail of half-empty waves. The
// loads are non-temporal. The group's second read of G and M (k_pre_t or
// k_pre) comes after the factors of every group are known, so when other
// groups take their one-pass form in between, their traffic has evicted these
// lines anyway; allocating them would only push out the previous pass's
// dirty lines earlier, in the middle of this read.
template <int DTG, int DTM, int CH>
__global__ void __launch_bounds__(256) k_rowsumsq_rows(const ElemArgs a) {
  const int bpm = (a.R + 3) >> 2;
  const int k = blockIdx.x / bpm;
  const int r = (blockIdx.x - k * bpm) * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= a.R) return;
  const void* gp = a.mat[k].g;
  const void* mp = a.mat[k].m;
  Raw8<DTG> g[CH];
  Raw8<DTM> m[CH];
  bool ok[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int c = u * 512 + lane * 8;
    ok[u] = c < a.C;
    const int64_t off = ok[u] ? (int64_t)r * a.C + c : 0;
    raw_load<DTG, kNT>(eptr<DTG>(gp, off), g[u]);
    raw_load<DTM, kNT>(eptr<DTM>(mp, off), m[u]);
  }
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float m1, mt;
      momentum1(raw_at<DTG>(g[u], e), raw_at<DTM>(m[u], e), a.beta, a.nesterov, m1, mt);
      const float t = __builtin_fmaf(mt, mt, acc);
      acc = ok[u] ? t : acc;
    }
  }
  const float n2 = wave_sum(acc);
  if (lane == 0) a.rowsq[(int64_t)k * a.row_stride + r] = n2;
}

// Row sums of squares of a workspace buffer in the parameter's layout (the
// update U, for MuonEq POST).
template <int DTX>
__global__ void __launch_bounds__(256) k_rowsumsq_buffer(const ElemArgs a) {
  const int bpm = (a.R + kRowsPerBlock - 1) / kRowsPerBlock;
  const int k = blockIdx.x / bpm;
  const int rb = blockIdx.x - k * bpm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const void* xp = eptr<DTX>(static_cast<const void*>(a.xd), (int64_t)k * a.x_stride);
  for (int rr = wave; rr < kRowsPerBlock; rr += 4) {
    const int r = rb * kRowsPerBlock + rr;
    if (r >= a.R) break;
    const int64_t base = (int64_t)r * a.ld_d;
    float acc = 0.0f;
    // the buffer pitch is a multiple of 256; columns C.. are zero
    for (int c = lane * 8; c < a.C; c += 512) {
      float x[8];
      load8<DTX>(eptr<DTX>(xp, base + c), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], x[e], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) a.rowsq[(int64_t)k * a.row_stride + r] = acc;
  }
}

// Row values are read kFinBatch per thread at a time, every load issued before
// the first use, so a matrix of R rows costs R / (256 kFinBatch) memory
// round trips per pass instead of R / 256 dependent ones.
constexpr int kFinBatch = 16;

// One block per matrix, every group of the launch (a group's matrices are
// blocks g.block_begin ..); fixed-order reduction (thread t sums rows t,
// t + 256, ... in that order, then an LDS tree), so results do not depend on
// scheduling or on the batching of the loads.
__global__ void __launch_bounds__(256) k_finalize(const FinalizeArgs fa) {
  __shared__ float red[256];
  int gi = 0;
  while (gi + 1 < fa.n && (int)blockIdx.x >= fa.g[gi + 1].block_begin) ++gi;
  const FinalizeGroup& a = fa.g[gi];
  const int k = (int)blockIdx.x - a.block_begin;
  const float* rs = a.rowsq + (int64_t)k * a.row_stride;
  float* rf = a.rowf + (int64_t)k * a.row_stride;
  const int t = threadIdx.x;
  const int mode = a.mode;
  float part = 0.0f;
#pragma unroll 1
  for (int i0 = t; i0 < a.R; i0 += 256 * kFinBatch) {
    float q[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) q[j] = rs[min(i0 + 256 * j, a.R - 1)];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      if (i0 + 256 * j >= a.R) break;
      if (mode == 1 || mode == 4) {
        const float n = sqrtf(q[j]);
        const float y = n / (n + fa.eq_eps);   // norm of the equilibrated row
        part += y * y;
      } else {
        part += q[j];
      }
    }
  }
  red[t] = part;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  const float total = red[0];
  if (a.nonfinite && t == 0) {
    // a non-finite entry (or an overflowing square) makes the sum non-finite
    const bool bad = !__builtin_isfinite(total);
    if (mode == 0 || mode == 1 || mode == 4) a.nonfinite[k] = bad ? 1 : 0;
    else if (bad) a.nonfinite[k] = 1;
  }
  if (mode == 0) {
    const float s = 1.0f / (sqrtf(total) + fa.norm_eps);
    for (int i = t; i < a.R; i += 256) rf[i] = s;
  } else if (mode == 4) {
    // MuonEq pre with the row factors already applied (k_pre_rows): only the
    // matrix's Frobenius factor, in the row-factor slot of row 0
    if (t == 0) rf[0] = 1.0f / (sqrtf(total) + fa.norm_eps);
  } else {
    // per-row factors from the row sums: mode 1 s / (||row|| + eq_eps), mode 2
    // rho / (||row|| + eq_eps), mode 3 (row RMS) 1 / (||row|| / sqrt(C) + eq_eps)
    const float num = mode == 1 ? 1.0f / (sqrtf(total) + fa.norm_eps)
                    : mode == 2 ? sqrtf(total) / sqrtf((float)a.R) : 1.0f;
    const float sc = sqrtf((float)a.C);
#pragma unroll 1
    for (int i0 = t; i0 < a.R; i0 += 256 * kFinBatch) {
      float q[kFinBatch];
#pragma unroll
      for (int j = 0; j < kFinBatch; ++j) q[j] = rs[min(i0 + 256 * j, a.R - 1)];
#pragma unroll
      for (int j = 0; j < kFinBatch; ++j) {
        const int i = i0 + 256 * j;
        if (i >= a.R) break;
        rf[i] = mode == 3 ? 1.0f / (sqrtf(q[j]) / sc + fa.eq_eps) : num / (sqrtf(q[j]) + fa.eq_eps);
      }
    }
  }
}

// 64 x 64 tiles of the parameter layout; thread t covers rows t/8 and t/8+32,
// columns 8*(t%8) .. +7 of its tile.
template <int DTG, int DTM, int DTX>
__global__ void __launch_bounds__(256) k_pre(const ElemArgs a) {
  __shared__ float tile[64][65];
  const int tiles = a.tiles_r * a.tiles_c;
  const int k = blockIdx.x / tiles;
  const int t = blockIdx.x - k * tiles;
  const int tr = t / a.tiles_c, tc = t - tr * a.tiles_c;
  const int r0 = tr * 64, c0 = tc * 64;
  const void* gp = a.mat[k].g;
  void* mp = a.mat[k].m;
  const int tid = threadIdx.x;
  const int cl = (tid & 7) * 8;
  const bool vec = a.vec != 0;
  // either copy may be skipped (null): the iteration may need only one layout
  void* xd = a.xd ? eptr<DTX>(a.xd, (int64_t)k * a.x_stride) : nullptr;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rl = (tid >> 3) + 32 * h;
    const int r = r0 + rl, c = c0 + cl;
    float x[8];
    if (r < a.R && c < a.C) {
      const float f = a.rowf ? a.rowf[(int64_t)k * a.row_stride + r] : 1.0f;
      const int64_t off = (int64_t)r * a.C + c;
      if (a.pure_copy) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = c + e < a.C ? load1<DTG>(gp, off + e) : 0.0f;
      } else if (vec) {
        float g[8], m[8], m1[8];
        load8<DTG, kNT>(eptr<DTG>(gp, off), g);
        load8<DTM, kNT>(eptr<DTM>(static_cast<const void*>(mp), off), m);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float mt;
          momentum1(g[e], m[e], a.beta, a.nesterov, m1[e], mt);
          x[e] = __fmul_rn(mt, f);
        }
        store8<DTM, kNT>(eptr<DTM>(mp, off), m1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (c + e < a.C) {
            float m1, mt;
            momentum1(load1<DTG>(gp, off + e), load1<DTM>(mp, off + e), a.beta, a.nesterov, m1, mt);
            store1<DTM>(mp, off + e, m1);
            x[e] = __fmul_rn(mt, f);
          } else {
            x[e] = 0.0f;
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    if (xd && r < a.r_ext) {
      const int64_t off = (int64_t)r * a.ld_d + c;
      if (c + 8 <= a.c_ext && (a.ld_d & 7) == 0) {
        store8<DTX>(eptr<DTX>(xd, off), x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < a.c_ext) store1<DTX>(xd, off + e, x[e]);
      }
    }
    if (a.xt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rl][cl + e] = x[e];
    }
  }
  if (a.xt) {
    // transposed copy: row (c0 + cc) of xt holds column cc of the tile
    __syncthreads();
    void* xt = eptr<DTX>(a.xt, (int64_t)k * a.x_stride);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = (tid >> 3) + 32 * h;
      const int rr = (tid & 7) * 8;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = tile[rr + e][cc];
      store8<DTX>(eptr<DTX>(xt, (int64_t)(c0 + cc) * a.ld_t + r0 + rr), y);
    }
  }
}

// The transposed-only form of k_pre (vector path, no copy in the
// parameter's layout): tiles of 64 rows x kPreTileCols columns, so that each
// row of G and M is read and M written in runs of 2 kPreTileCols bytes
// rather than 128. Thread t covers columns 8 (t % (kPreTileCols / 8)) .. +7
// of every (256 / (kPreTileCols / 8))-th row, all of its loads issued before
// the first use; X0^T is written 16 bytes per thread from the LDS tile, rows
// of X0^T beyond the 64-column tiles of the extent left alone. Same
// arithmetic and the same stored values as k_pre.
constexpr int kPreTileCols = 128;

template <int DTG, int DTM, int DTX>
__global__ void __launch_bounds__(256) k_pre_t(const ElemArgs a, const int tiles_cw) {
  constexpr int TC = kPreTileCols;
  constexpr int TPR = TC / 8;      // threads per tile row
  constexpr int RPP = 256 / TPR;   // tile rows per pass
  constexpr int NP = 64 / RPP;     // passes
  __shared__ float tile[64][TC + 1];
  const int tiles = a.tiles_r * tiles_cw;
  const int k = blockIdx.x / tiles;
  const int t = blockIdx.x - k * tiles;
  const int tr = t / tiles_cw, tc = t - tr * tiles_cw;
  const int r0 = tr * 64, c0 = tc * TC;
  const void* gp = a.mat[k].g;
  void* mp = a.mat[k].m;
  const int tid = threadIdx.x;
  const int cl = (tid % TPR) * 8;
  const int c = c0 + cl;
  Raw8<DTG> g[NP];
  Raw8<DTM> m[NP];
  bool ok[NP];
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int r = r0 + tid / TPR + RPP * h;
    ok[h] = r < a.R && c < a.C;
    const int64_t off = ok[h] ? (int64_t)r * a.C + c : 0;
    raw_load<DTG, kNT>(eptr<DTG>(gp, off), g[h]);
    raw_load<DTM, kNT>(eptr<DTM>(static_cast<const void*>(mp), off), m[h]);
  }
#pragma unroll
  for (int h = 0; h < NP; ++h) {
    const int rl = tid / TPR + RPP * h;
    const int r = r0 + rl;
    float x[8];
    if (ok[h]) {
      const float f = a.rowf ? a.rowf[(int64_t)k * a.row_stride + r] : 1.0f;
      float m1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float mt;
        momentum1(raw_at<DTG>(g[h], e), raw_at<DTM>(m[h], e), a.beta, a.nesterov, m1[e], mt);
        x[e] = __fmul_rn(mt, f);
      }
      store8<DTM, kNT>(eptr<DTM>(mp, (int64_t)r * a.C + c), m1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[rl][cl + e] = x[e];
  }
  __syncthreads();
  // row (c0 + cc) of xt holds column cc of the tile
  void* xt = eptr<DTX>(a.xt, (int64_t)k * a.x_stride);
  const int rows_t = a.tiles_c * 64;
#pragma unroll
  for (int h = 0; h < TC / 32; ++h) {
    const int cc = (tid >> 3) + 32 * h;
    const int rr = (tid & 7) * 8;
    if (c0 + cc < rows_t) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = tile[rr + e][cc];
      store8<DTX>(eptr<DTX>(xt, (int64_t)(c0 + cc) * a.ld_t + r0 + rr), y);
    }
  }
}

// The direct-only form of k_pre (vector path, no transposed copy): nothing
// is transposed, so no tile either. Thread i of the launch covers 16-byte
// chunks i, i + stride, ... of the matrix's extent r_ext x c_ext in row-major
// order (whole rows of chunks are read and written in one run), kPreDirectCh
// chunks per thread, every load issued before the first use. Chunks outside
// R x C are stored as zeros (the iteration buffer's padding). Same arithmetic
// and the same stored values as k_pre.
constexpr int kPreDirectCh = 4;

template <int DTG, int DTM, int DTX>
__global__ void __launch_bounds__(256) k_pre_d(const ElemArgs a, const int bpm) {
  const int k = blockIdx.x / bpm;
  const int b = blockIdx.x - k * bpm;
  const int cpr = a.c_ext >> 3;                       // chunks per extent row
  const int64_t nch = (int64_t)a.r_ext * cpr;
  const void* gp = a.mat[k].g;
  void* mp = a.mat[k].m;
  void* xd = eptr<DTX>(a.xd, (int64_t)k * a.x_stride);
  Raw8<DTG> g[kPreDirectCh];
  Raw8<DTM> m[kPreDirectCh];
  bool ok[kPreDirectCh];
  int rr[kPreDirectCh], cc[kPreDirectCh];
#pragma unroll
  for (int u = 0; u < kPreDirectCh; ++u) {
    const int64_t i = ((int64_t)b * kPreDirectCh + u) * 256 + threadIdx.x;
    const bool in = i < nch;
    rr[u] = in ? (int)(i / cpr) : a.r_ext;
    cc[u] = in ? (int)(i - (int64_t)rr[u] * cpr) * 8 : 0;
    ok[u] = rr[u] < a.R && cc[u] < a.C;
    const int64_t off = ok[u] ? (int64_t)rr[u] * a.C + cc[u] : 0;
    raw_load<DTG, kNT>(eptr<DTG>(gp, off), g[u]);
    raw_load<DTM, kNT>(eptr<DTM>(static_cast<const void*>(mp), off), m[u]);
  }
#pragma unroll
  for (int u = 0; u < kPreDirectCh; ++u) {
    if (rr[u] >= a.r_ext) continue;
    float x[8];
    if (ok[u]) {
      const float f = a.rowf ? a.rowf[(int64_t)k * a.row_stride + rr[u]] : 1.0f;
      float m1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float mt;
        momentum1(raw_at<DTG>(g[u], e), raw_at<DTM>(m[u], e), a.beta, a.nesterov, m1[e], mt);
        x[e] = __fmul_rn(mt, f);
      }
      store8<DTM, kNT>(eptr<DTM>(mp, (int64_t)rr[u] * a.C + cc[u]), m1);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    store8<DTX>(eptr<DTX>(xd, (int64_t)rr[u] * a.ld_d + cc[u]), x);
  }
}

// One wave per row of a matrix with no more rows than columns (its
// iteration layout is the parameter's): M <- m1, the row's sum of squares of
// Mt (summed in the order k_rowsumsq_momentum uses) and the X0 row
// Mt / (||Mt_row|| + eq_eps), the MuonEq row scaling, with the padding
// columns and rows of the iteration buffer zeroed. The matrix's Frobenius
// factor (k_finalize mode 4) is applied by the first Newton-Schulz products
// instead, so G and M are read once. Vector path only (C % 8 == 0, aligned),
// C <= 512 CH.
template <int DTG, int DTM, int DTX, int CH>
__global__ void __launch_bounds__(256) k_pre_rows(const ElemArgs a) {
  const int bpm = (a.r_ext + 3) >> 2;
  const int k = blockIdx.x / bpm;
  const int r = (blockIdx.x - k * bpm) * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= a.r_ext) return;
  void* xd = eptr<DTX>(a.xd, (int64_t)k * a.x_stride);
  const int64_t xrow = (int64_t)r * a.ld_d;
  if (r >= a.R) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = u * 512 + lane * 8;
      float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (c < a.c_ext) store8<DTX>(eptr<DTX>(xd, xrow + c), z);
    }
    return;
  }
  const void* gp = a.mat[k].g;
  void* mp = a.mat[k].m;
  Raw8<DTG> g[CH];
  Raw8<DTM> m[CH];
  bool ok[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int c = u * 512 + lane * 8;
    ok[u] = c < a.C;
    const int64_t off = ok[u] ? (int64_t)r * a.C + c : 0;
    raw_load<DTG, kNT>(eptr<DTG>(gp, off), g[u]);
    raw_load<DTM, kNT>(eptr<DTM>(static_cast<const void*>(mp), off), m[u]);
  }
  float mt[CH][8];
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    float m1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      momentum1(raw_at<DTG>(g[u], e), raw_at<DTM>(m[u], e), a.beta, a.nesterov, m1[e], mt[u][e]);
      const float t = __builtin_fmaf(mt[u][e], mt[u][e], acc);
      acc = ok[u] ? t : acc;
    }
    if (ok[u]) store8<DTM, kNT>(eptr<DTM>(mp, (int64_t)r * a.C + u * 512 + lane * 8), m1);
  }
  const float n2 = wave_sum(acc);
  if (lane == 0) a.rowsq[(int64_t)k * a.row_stride + r] = n2;
  const float f = 1.0f / (sqrtf(n2) + a.eq_eps);
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int c = u * 512 + lane * 8;
    if (c < a.c_ext) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ok[u] ? __fmul_rn(mt[u][e], f) : 0.0f;
      store8<DTX>(eptr<DTX>(xd, xrow + c), x);
    }
  }
}

// Accumulate the squared change of one weight as stored (W' rounded to the
// parameter's type) and its squared old value.
template <int DTP>
__device__ __forceinline__ void update_sums(float w_old, float w_new, float& sd, float& sw) {
  const float stored = DTP == DT_BF16 ? bf16_bits_to_f32(f32_to_bf16(w_new)) : w_new;
  const float d = stored - w_old;
  sd = __builtin_fmaf(d, d, sd);
  sw = __builtin_fmaf(w_old, w_old, sw);
}

// Block-wide sums of (sd, sw) written to out[0..1] (256 threads, all reach it).
__device__ __forceinline__ void block_sums_out(float sd, float sw, float* out) {
  __shared__ float red[2][4];
  sd = wave_sum(sd);
  sw = wave_sum(sw);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = sd;
    red[1][wave] = sw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    out[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    out[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

__device__ __forceinline__ float post_elem(float w, float u, float f, bool has_f, const ElemArgs& a) {
  return muon_update(w, has_f ? __fmul_rn(u, f) : u, a.c_lr, a.c_wd, a.cautious != 0, a.decay != 0);
}

constexpr int kPostChunks = 4;   // 8-element chunks per thread (vector path)

// Vector path (C % 8 == 0, 16-byte aligned rows): the matrices' 8-element
// chunks in row-major order; thread t of block b takes chunks
// (b*256 + t) + 256*blocks*u... of its matrix, all loads before any update.
// STATS: also the block's sums of (W' - W)^2 and W^2 into a.part.
template <int DTP, int DTX, bool STATS>
__device__ __forceinline__ void post_vec_body(const ElemArgs& a, int blocks_per_mat) {
  const int k = blockIdx.x / blocks_per_mat;
  const int b = blockIdx.x - k * blocks_per_mat;
  const uint32_t cpr = (uint32_t)a.C >> 3;                 // chunks per row
  const uint32_t nch = (uint32_t)a.R * cpr;                // < 2^28: a matrix holds < 2^31 elements
  void* wp = a.mat[k].w;
  const void* xd = eptr<DTX>(static_cast<const void*>(a.xd), (int64_t)k * a.x_stride);
  const float* rowf = a.rowf ? a.rowf + (int64_t)k * a.row_stride : nullptr;
  const uint32_t step = (uint32_t)blocks_per_mat * 256u;
  // a matrix flagged non-finite keeps its weight (the sums still see W)
  const bool keep = a.nonfinite && a.nonfinite[k];
  if (keep && !STATS) return;
  float sd = 0.0f, sw = 0.0f;   // sums of (W' - W)^2 and W^2 (stored values)
  for (uint32_t q0 = (uint32_t)b * 256u + threadIdx.x; q0 < nch; q0 += step * kPostChunks) {
    float w[kPostChunks][8], u[kPostChunks][8];
    uint32_t rr[kPostChunks], cc[kPostChunks];
#pragma unroll
    for (int v = 0; v < kPostChunks; ++v) {
      const uint32_t q = q0 + step * v;
      rr[v] = q / cpr;
      cc[v] = (q - rr[v] * cpr) * 8u;
      if (q < nch) {
        load8<DTP, kNT>(eptr<DTP>(static_cast<const void*>(wp), (int64_t)rr[v] * a.C + cc[v]), w[v]);
        load8<DTX, kNT>(eptr<DTX>(xd, (int64_t)rr[v] * a.ld_d + cc[v]), u[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < kPostChunks; ++v) {
      if (q0 + step * v < nch) {
        const float f = rowf ? rowf[rr[v]] : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float w0 = w[v][e];
          w[v][e] = keep ? w0 : post_elem(w0, u[v][e], f, rowf != nullptr, a);
          if constexpr (STATS) update_sums<DTP>(w0, w[v][e], sd, sw);
        }
        if (!keep) store8<DTP, kNT>(eptr<DTP>(wp, (int64_t)rr[v] * a.C + cc[v]), w[v]);
      }
    }
  }
  if constexpr (STATS) block_sums_out(sd, sw, a.part + 2 * (int64_t)blockIdx.x);
}

template <int DTP, int DTX>
__global__ void __launch_bounds__(256) k_post_vec(const ElemArgs a, int blocks_per_mat) {
  post_vec_body<DTP, DTX, false>(a, blocks_per_mat);
}
template <int DTP, int DTX>
__global__ void __launch_bounds__(256) k_post_vec_stats(const ElemArgs a, int blocks_per_mat) {
  post_vec_body<DTP, DTX, true>(a, blocks_per_mat);
}

// W <- RNE( (mask ? W - c_wd*W : W) - c_lr*U ), mask = cautious ? (U*W >= 0) : 1.
template <int DTP, int DTX, bool STATS>
__device__ __forceinline__ void post_tile_body(const ElemArgs& a) {
  const int tiles = a.tiles_r * a.tiles_c;
  const int k = blockIdx.x / tiles;
  const int t = blockIdx.x - k * tiles;
  const int tr = t / a.tiles_c, tc = t - tr * a.tiles_c;
  const int r0 = tr * 64, c0 = tc * 64;
  void* wp = a.mat[k].w;
  const void* xd = eptr<DTX>(static_cast<const void*>(a.xd), (int64_t)k * a.x_stride);
  const int tid = threadIdx.x;
  const int cl = (tid & 7) * 8;
  const bool vec = a.vec && (a.ld_d & 7) == 0;
  const bool keep = a.nonfinite && a.nonfinite[k];   // flagged: the weight stays
  if (keep && !STATS) return;
  float sd = 0.0f, sw = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + (tid >> 3) + 32 * h, c = c0 + cl;
    if (r >= a.R || c >= a.C) continue;
    const float f = a.rowf ? a.rowf[(int64_t)k * a.row_stride + r] : 1.0f;
    const int64_t off = (int64_t)r * a.C + c;
    const int64_t uoff = (int64_t)r * a.ld_d + c;
    float w[8], u[8];
    const int n = vec ? 8 : (a.C - c < 8 ? a.C - c : 8);
    if (vec) {
      load8<DTP>(eptr<DTP>(static_cast<const void*>(wp), off), w);
      load8<DTX>(eptr<DTX>(xd, uoff), u);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w[e] = e < n ? load1<DTP>(wp, off + e) : 0.0f;
        u[e] = e < n ? load1<DTX>(xd, uoff + e) : 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w0 = w[e];
      w[e] = keep ? w0 : post_elem(w0, u[e], f, a.rowf != nullptr, a);
      if (STATS && e < n) update_sums<DTP>(w0, w[e], sd, sw);
    }
    if (keep) continue;
    if (vec) {
      store8<DTP>(eptr<DTP>(wp, off), w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < n) store1<DTP>(wp, off + e, w[e]);
    }
  }
  if constexpr (STATS) block_sums_out(sd, sw, a.part + 2 * (int64_t)blockIdx.x);
}

template <int DTP, int DTX>
__global__ void __launch_bounds__(256) k_post(const ElemArgs a) {
  post_tile_body<DTP, DTX, false>(a);
}
template <int DTP, int DTX>
__global__ void __launch_bounds__(256) k_post_stats(const ElemArgs a) {
  post_tile_body<DTP, DTX, true>(a);
}

__global__ void __launch_bounds__(256) k_bf16_round(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = f32_to_bf16(in[i]);
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
#define MA_DISPATCH2(d1, d2, KER, ...)                                                  \
  do {                                                                                  \
    if ((d1) == DT_BF16 && (d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_BF16>), __VA_ARGS__); \
    else if ((d1) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_F32>), __VA_ARGS__);  \
    else if ((d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_F32, DT_BF16>), __VA_ARGS__);  \
    else hipLaunchKernelGGL((KER<DT_F32, DT_F32>), __VA_ARGS__);                         \
  } while (0)

#define MA_DISPATCH2C(d1, d2, KER, C3, ...)                                                       \
  do {                                                                                            \
    if ((d1) == DT_BF16 && (d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_BF16, C3>), __VA_ARGS__); \
    else if ((d1) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_F32, C3>), __VA_ARGS__);        \
    else if ((d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_F32, DT_BF16, C3>), __VA_ARGS__);        \
    else hipLaunchKernelGGL((KER<DT_F32, DT_F32, C3>), __VA_ARGS__);                               \
  } while (0)

hipError_t launch_rowsumsq_momentum(int dt_g, int dt_m, const ElemArgs& a, hipStream_t s) {
  // chunks of 512 columns per row
  const int cpr = (a.C + 511) / 512;
  if (a.vec && a.C <= kPreRowsMaxCols) {
    const int blocks = a.count * ((a.R + 3) / 4);
    if (blocks <= 0) return hipSuccess;
    if (cpr <= 1) MA_DISPATCH2C(dt_g, dt_m, k_rowsumsq_rows, 1, dim3(blocks), dim3(256), 0, s, a);
    else if (cpr <= 2) MA_DISPATCH2C(dt_g, dt_m, k_rowsumsq_rows, 2, dim3(blocks), dim3(256), 0, s, a);
    else if (cpr <= 4) MA_DISPATCH2C(dt_g, dt_m, k_rowsumsq_rows, 4, dim3(blocks), dim3(256), 0, s, a);
    else MA_DISPATCH2C(dt_g, dt_m, k_rowsumsq_rows, 8, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // longer rows (eight-chunk batches) or unaligned ones (scalar loads): four
  // rows per wave
  const int blocks = a.count * ((a.R + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks <= 0) return hipSuccess;
  MA_DISPATCH2C(dt_g, dt_m, k_rowsumsq_momentum, 8, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define MA_DISPATCH3C(d1, d2, d3, KER, C4, ...)                                            \
  do {                                                                                     \
    if ((d3) == DT_BF16) MA_DISPATCH2C3(d1, d2, DT_BF16, KER, C4, __VA_ARGS__);            \
    else MA_DISPATCH2C3(d1, d2, DT_F32, KER, C4, __VA_ARGS__);                             \
  } while (0)
#define MA_DISPATCH2C3(d1, d2, D3, KER, C4, ...)                                                          \
  do {                                                                                                    \
    if ((d1) == DT_BF16 && (d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_BF16, D3, C4>), __VA_ARGS__); \
    else if ((d1) == DT_BF16) hipLaunchKernelGGL((KER<DT_BF16, DT_F32, D3, C4>), __VA_ARGS__);            \
    else if ((d2) == DT_BF16) hipLaunchKernelGGL((KER<DT_F32, DT_BF16, D3, C4>), __VA_ARGS__);            \
    else hipLaunchKernelGGL((KER<DT_F32, DT_F32, D3, C4>), __VA_ARGS__);                                   \
  } while (0)

hipError_t launch_pre_rows(int dt_g, int dt_m, int dt_x, const ElemArgs& a, hipStream_t s) {
  if (!a.vec || !a.xd || a.R > a.r_ext || a.C > a.c_ext || a.c_ext > kPreRowsMaxCols || (a.ld_d % 8) != 0)
    return hipErrorInvalidValue;
  const int blocks = a.count * ((a.r_ext + 3) / 4);
  if (blocks <= 0) return hipSuccess;
  const int ch = (a.c_ext + 511) / 512;
  if (ch <= 1) MA_DISPATCH3C(dt_g, dt_m, dt_x, k_pre_rows, 1, dim3(blocks), dim3(256), 0, s, a);
  else if (ch <= 2) MA_DISPATCH3C(dt_g, dt_m, dt_x, k_pre_rows, 2, dim3(blocks), dim3(256), 0, s, a);
  else if (ch <= 4) MA_DISPATCH3C(dt_g, dt_m, dt_x, k_pre_rows, 4, dim3(blocks), dim3(256), 0, s, a);
  else MA_DISPATCH3C(dt_g, dt_m, dt_x, k_pre_rows, 8, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowsumsq_buffer(int dt_x, const ElemArgs& a, hipStream_t s) {
  const int blocks = a.count * ((a.R + kRowsPerBlock - 1) / kRowsPerBlock);
  if (blocks <= 0) return hipSuccess;
  if (dt_x == DT_BF16) hipLaunchKernelGGL((k_rowsumsq_buffer<DT_BF16>), dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_rowsumsq_buffer<DT_F32>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DTX>
static void launch_pre_x(int dt_g, int dt_m, const ElemArgs& a, int blocks, hipStream_t s) {
  if (dt_g == DT_BF16 && dt_m == DT_BF16) hipLaunchKernelGGL((k_pre<DT_BF16, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a);
  else if (dt_g == DT_BF16) hipLaunchKernelGGL((k_pre<DT_BF16, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a);
  else if (dt_m == DT_BF16) hipLaunchKernelGGL((k_pre<DT_F32, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_pre<DT_F32, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a);
}

template <int DTX>
static void launch_pre_t_x(int dt_g, int dt_m, const ElemArgs& a, int blocks, int tiles_cw, hipStream_t s) {
  if (dt_g == DT_BF16 && dt_m == DT_BF16)
    hipLaunchKernelGGL((k_pre_t<DT_BF16, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a, tiles_cw);
  else if (dt_g == DT_BF16) hipLaunchKernelGGL((k_pre_t<DT_BF16, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a, tiles_cw);
  else if (dt_m == DT_BF16) hipLaunchKernelGGL((k_pre_t<DT_F32, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a, tiles_cw);
  else hipLaunchKernelGGL((k_pre_t<DT_F32, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a, tiles_cw);
}

template <int DTX>
static void launch_pre_d_x(int dt_g, int dt_m, const ElemArgs& a, int blocks, int bpm, hipStream_t s) {
  if (dt_g == DT_BF16 && dt_m == DT_BF16)
    hipLaunchKernelGGL((k_pre_d<DT_BF16, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a, bpm);
  else if (dt_g == DT_BF16) hipLaunchKernelGGL((k_pre_d<DT_BF16, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a, bpm);
  else if (dt_m == DT_BF16) hipLaunchKernelGGL((k_pre_d<DT_F32, DT_BF16, DTX>), dim3(blocks), dim3(256), 0, s, a, bpm);
  else hipLaunchKernelGGL((k_pre_d<DT_F32, DT_F32, DTX>), dim3(blocks), dim3(256), 0, s, a, bpm);
}

hipError_t launch_pre(int dt_g, int dt_m, int dt_x, const ElemArgs& a, hipStream_t s) {
  if (a.xt && !a.xd && a.vec && !a.pure_copy) {
    // the transposed copy alone: wide tiles (the 64-column tiles of the
    // extent, kPreTileCols / 64 to a tile, the last one part empty)
    const int per = kPreTileCols / 64;
    const int tiles_cw = (a.tiles_c + per - 1) / per;
    const int blocks = a.count * a.tiles_r * tiles_cw;
    if (blocks <= 0) return hipSuccess;
    if (dt_x == DT_BF16) launch_pre_t_x<DT_BF16>(dt_g, dt_m, a, blocks, tiles_cw, s);
    else launch_pre_t_x<DT_F32>(dt_g, dt_m, a, blocks, tiles_cw, s);
    return hipGetLastError();
  }
  if (a.xd && !a.xt && a.vec && !a.pure_copy && (a.ld_d & 7) == 0 && (a.c_ext & 7) == 0 && a.c_ext <= a.ld_d) {
    // the direct copy alone: row-major runs, no tile
    const int64_t nch = (int64_t)a.r_ext * (a.c_ext >> 3);
    const int bpm = (int)((nch + 256 * kPreDirectCh - 1) / (256 * kPreDirectCh));
    const int blocks = a.count * bpm;
    if (blocks <= 0) return hipSuccess;
    if (dt_x == DT_BF16) launch_pre_d_x<DT_BF16>(dt_g, dt_m, a, blocks, bpm, s);
    else launch_pre_d_x<DT_F32>(dt_g, dt_m, a, blocks, bpm, s);
    return hipGetLastError();
  }
  const int blocks = a.count * a.tiles_r * a.tiles_c;
  if (blocks <= 0) return hipSuccess;
  if (dt_x == DT_BF16) launch_pre_x<DT_BF16>(dt_g, dt_m, a, blocks, s);
  else launch_pre_x<DT_F32>(dt_g, dt_m, a, blocks, s);
  return hipGetLastError();
}

// about 4 chunks per thread on the vector path: enough blocks to fill the
// chip without tiny blocks
static int post_vec_blocks(int64_t R, int64_t C) {
  const int64_t nch = R * (C >> 3);
  const int64_t bpm = (nch + 256 * kPostChunks - 1) / (256 * kPostChunks);
  return bpm < 1 ? 1 : (int)bpm;
}

static bool post_uses_vec(const ElemArgs& a) { return a.vec && (a.C & 7) == 0 && (a.ld_d & 7) == 0; }

int post_blocks_per_mat(const ElemArgs& a) {
  return post_uses_vec(a) ? post_vec_blocks(a.R, a.C) : a.tiles_r * a.tiles_c;
}

int post_blocks_per_mat_max(int64_t R, int64_t C) {
  const int tiles = (int)(((R + 63) / 64) * ((C + 63) / 64));
  const int vecb = (C & 7) == 0 ? post_vec_blocks(R, C) : 0;
  return tiles > vecb ? tiles : vecb;
}

hipError_t launch_post(int dt_p, int dt_x, const ElemArgs& a, hipStream_t s) {
  if (a.count <= 0 || a.R <= 0 || a.C <= 0) return hipSuccess;
  const int bpm = post_blocks_per_mat(a);
  if (post_uses_vec(a)) {
    if (a.part) MA_DISPATCH2(dt_p, dt_x, k_post_vec_stats, dim3(a.count * bpm), dim3(256), 0, s, a, bpm);
    else MA_DISPATCH2(dt_p, dt_x, k_post_vec, dim3(a.count * bpm), dim3(256), 0, s, a, bpm);
    return hipGetLastError();
  }
  if (a.count * bpm <= 0) return hipSuccess;
  if (a.part) MA_DISPATCH2(dt_p, dt_x, k_post_stats, dim3(a.count * bpm), dim3(256), 0, s, a);
  else MA_DISPATCH2(dt_p, dt_x, k_post, dim3(a.count * bpm), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One block per matrix: the two sums over its ppm partials in fp64, each
// thread taking a fixed stride and the block reducing in a fixed tree, so the
// result does not depend on timing.
__global__ void __launch_bounds__(256) k_update_stats(const float* part, int ppm, float* out) {
  __shared__ double red[2][256];
  const int k = blockIdx.x;
  const float* p = part + 2 * (int64_t)k * ppm;
  double sd = 0.0, sw = 0.0;
  for (int b = threadIdx.x; b < ppm; b += 256) {
    sd += (double)p[2 * b];
    sw += (double)p[2 * b + 1];
  }
  red[0][threadIdx.x] = sd;
  red[1][threadIdx.x] = sw;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      red[0][threadIdx.x] += red[0][threadIdx.x + h];
      red[1][threadIdx.x] += red[1][threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[2 * k] = (float)sqrt(red[0][0]);
    out[2 * k + 1] = (float)sqrt(red[1][0]);
  }
}

hipError_t launch_update_stats(const float* part, int ppm, int count, float* out, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_update_stats, dim3(count), dim3(256), 0, s, part, ppm, out);
  return hipGetLastError();
}

hipError_t launch_bf16_round(const float* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_bf16_round, dim3((unsigned)blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace ma
