// Launch descriptors of the Newton-Schulz GEMM kernels.
#pragma once
#include "common.hpp"

namespace ma {

// Epilogues of C = P Q^T (fp32 accumulation), one per sub-step of a quintic
// Newton-Schulz step X <- a X + (b A + c A A) X with A = X X^T:
enum NsEpilogue : int {
  EPI_GRAM = 0,  // A = X X^T                (symmetric: upper tiles, mirrored)
  EPI_POLY = 1,  // B = b*A + c*(A A^T)      (A symmetric, so A A^T = A A; mirrored)
  EPI_AXPY = 2,  // X' = a*X + B X           (Q = X^T; writes X' and/or X'^T)
};

constexpr int kMaxNsGroups = 8;

// One shape group of a batched launch: `count` independent products.
// Element strides between consecutive matrices are s*, row pitches ld*.
struct NsGroup {
  const void* P;    // rows i, K contiguous
  const void* Q;    // rows j, K contiguous
  const void* E;    // epilogue input read as E[j][i] (A for POLY, X^T for AXPY)
  void* outN;       // C[i][j] (row-major output), may be null
  void* outT;       // C[j][i] (transposed output), may be null
  int64_t sP, sQ, sE, sN, sT;
  int32_t ldP, ldQ, ldE, ldN, ldT;
  int32_t K;        // reduction length (multiple of the K tile)
  int32_t tm, tn;   // output tile grid
  int32_t tiles;    // tiles per matrix
  int32_t count;
  int32_t unit;       // jobs per scheduling unit: tiles (whole matrix) or 1 (one tile)
  int32_t rot;        // unit u of this group goes to XCD (u + rot) % 8
  int32_t symmetric;  // 1: only tiles bi <= bj, mirrored through outN/outT
  int32_t upper_only; // symmetric: write each tile once (no mirror); the
                      // lower triangle of the output is left unwritten
  int32_t p_upper;    // AXPY with qt: P holds only its upper triangle (B
                      // symmetric); blocks left of the diagonal are read
                      // transposed from those above it
  // per-matrix factor s of the operand X (matrix k's at scale[k*scale_stride]),
  // or null: the output is multiplied by s^2 (GRAM, A of s X) or s (AXPY,
  // X' of s X given B of s X)
  const float* scale;
  int64_t scale_stride;
  // Fused update (AXPY of the last step, bf16 iteration; W null: none). Matrix
  // k's weight, bf16, row-major R x C with C % 8 == 0, at W + k * sW elements
  // (16-byte aligned), takes the Muon update with
  // the stored U tile in the parameter's layout: rows i of outN, or rows j of
  // outT for a tall matrix (w_trans); matrices with nonfinite[k] != 0 are
  // left unchanged.
  void* W;
  int64_t sW;
  int32_t R, C, w_trans, cautious, decay;
  float c_lr, c_wd;
  const int32_t* nonfinite;
};

// Scheduling: the hardware deals consecutive workgroups round-robin to the 8
// XCDs, so block b runs on XCD b % 8 as its (b / 8)-th block there. Each
// group's jobs are cut into units (a whole matrix when the group has at least
// 8 matrices, else single tiles); unit u goes to XCD (u + rot) % 8. Every XCD then
// gets one eighth of every group (balanced when groups differ in K) and, for
// whole-matrix units, all tiles of a matrix share one L2. Each group's first
// unit goes to the XCD after the previous group's last one.
//
// The LDS-DMA kernel is persistent: padded_blocks = 8 x P with P <= 32 (one
// block per CU); block b runs jobs b/8, b/8 + P, ... of XCD b % 8.
struct NsArgs {
  int32_t n_groups;
  int32_t per_xcd;         // jobs of the busiest XCD
  int32_t padded_blocks;   // blocks launched
  float a, b, c;
  NsGroup g[kMaxNsGroups];
};

constexpr int kNsPersBlocksPerXcd = 32;   // CUs per XCD

// tile configuration chosen per launch: block tile bm x bn, K tile bk,
// wgm x wgn waves; dma selects the LDS-DMA kernel (bf16, 256 x 256 x BK, 2 x 4 waves);
// qt (AXPY, 2 x 4 waves): Q = X^T is read from X (row-major) through
// transposing LDS reads, so the iteration needs no X^T copy
struct NsTile { int bm, bn, bk, wgm, wgn, dma, qt = 0; };


hipError_t launch_ns_gemm(int dtype, int epi, NsTile tile, const NsArgs& args, hipStream_t s);

// Sum of the K slices of a split fp32 Gram product (k_split_sum): per group,
// out[i] = (part_0[i] + part_1[i] + ...) in slice order, over count matrices
// of mat_elems floats (a multiple of kSplitSumBlockElems). Blocks
// block_begin .. of the launch belong to the group.
constexpr int kSplitSumBlockElems = 1024;   // 256 threads x 4 floats
struct SplitSumGroup {
  const float* part;
  float* out;
  int64_t mat_elems;        // floats per matrix
  int64_t split_stride;     // floats between slices (count x mat_elems)
  int64_t block_begin;
  int32_t slices;
};
struct SplitSumArgs {
  int32_t n;
  int64_t blocks;
  SplitSumGroup g[kMaxNsGroups];
};
hipError_t launch_split_sum(const SplitSumArgs& args, hipStream_t s);

// k-tile of the LDS-DMA kernel (its block tile is 256 x 256, 2 x 4 waves)
int ns_dma_bk();

}  // namespace ma
