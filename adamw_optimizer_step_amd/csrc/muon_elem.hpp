// Launch descriptors of the Muon elementwise and reduction kernels.
#pragma once
#include "common.hpp"

namespace ma {

struct MatPtr {
  const void* g;   // gradient (param layout)
  void* m;         // momentum buffer (param layout)
  void* w;         // weight (param layout)
};

// One launch covers up to kMaxMatsPerLaunch matrices of one shape group.
struct ElemArgs {
  int32_t R, C;              // parameter shape (rows x cols)
  int32_t count;             // matrices in this launch
  int32_t r_ext, c_ext;      // param-layout extent the tile grid covers (>= R, C)
  int32_t tiles_r, tiles_c;  // 64 x 64 tiles per matrix
  // workspace views of matrix k start k*x_stride elements after the bases
  void* xd;                  // copy in the parameter's layout, row pitch ld_d
  void* xt;                  // transposed copy (may be null), row pitch ld_t
  int64_t ld_d, ld_t, x_stride;
  float* rowsq;              // per-row sums of squares, matrix k at k*row_stride
  float* rowf;               // per-row factors (null: 1)
  int64_t row_stride;
  float beta;
  int32_t nesterov;
  float c_lr, c_wd;
  int32_t cautious, decay;
  float norm_eps, eq_eps;
  int32_t vec;               // C % 8 == 0 and every matrix pointer 16-byte aligned
  int32_t pure_copy;         // k_pre: X0 = G (no momentum; M untouched)
  float* part;               // k_post: per-block (sum (W'-W)^2, sum W^2), 2 floats per block, or null
  // per-matrix non-finite flags (matrix k at nonfinite[k]) or null (no check):
  // k_finalize sets a matrix's flag when its sums of squares are not finite
  // (modes 0, 1, 4 write it, modes 2, 3 only raise it); k_post then leaves
  // that matrix's weight as it was
  int32_t* nonfinite;
  MatPtr mat[kMaxMatsPerLaunch];
};

// k_finalize over several groups in one launch: one block per matrix, group
// g's matrices at blocks block_begin .. (increasing over the groups).
constexpr int kMaxFinalizeGroups = 16;
struct FinalizeGroup {
  const float* rowsq;        // matrix k's row sums of squares at k*row_stride
  float* rowf;               // matrix k's factors at k*row_stride
  int32_t* nonfinite;        // matrix k's flag at nonfinite[k], or null
  int64_t row_stride;
  int32_t R, C, block_begin;
  // 0: Frobenius only, 1: MuonEq pre, 2: MuonEq post, 3: row RMS,
  // 4: MuonEq pre, Frobenius factor only (into rowf[0])
  int32_t mode;
};
struct FinalizeArgs {
  int32_t n;
  float norm_eps, eq_eps;
  FinalizeGroup g[kMaxFinalizeGroups];
};

// dtype codes: DT_F32 / DT_BF16
hipError_t launch_rowsumsq_momentum(int dt_g, int dt_m, const ElemArgs& a, hipStream_t s);
hipError_t launch_rowsumsq_buffer(int dt_x, const ElemArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, int blocks, hipStream_t s);
hipError_t launch_pre(int dt_g, int dt_m, int dt_x, const ElemArgs& a, hipStream_t s);
// k_pre_rows (momentum, row sums and the row-scaled X0 in one pass; the
// Frobenius factor left to the iteration) for matrices whose iteration layout
// is the parameter's; launch_pre_rows fails with hipErrorInvalidValue unless
// a.vec, a.xd is set, R <= r_ext, C <= c_ext <= kPreRowsMaxCols and ld_d % 8 == 0
constexpr int kPreRowsMaxCols = 4096;
hipError_t launch_pre_rows(int dt_g, int dt_m, int dt_x, const ElemArgs& a, hipStream_t s);
hipError_t launch_post(int dt_p, int dt_x, const ElemArgs& a, hipStream_t s);
// blocks per matrix of the launch_post call for `a` (the partial sums it writes)
int post_blocks_per_mat(const ElemArgs& a);
// at most this many, whatever the matrices' alignment (workspace sizing)
int post_blocks_per_mat_max(int64_t R, int64_t C);
// out[2k] = sqrt(sum of part[2(k*ppm + b)]), out[2k+1] = sqrt(sum of part[2(k*ppm + b) + 1]),
// b < ppm, summed in a fixed order in fp64, for k < count
hipError_t launch_update_stats(const float* part, int ppm, int count, float* out, hipStream_t s);
hipError_t launch_bf16_round(const float* in, uint16_t* out, int64_t n, hipStream_t s);

}  // namespace ma
