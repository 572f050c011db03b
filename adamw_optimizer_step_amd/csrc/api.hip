// C ABI of the Muon + AdamW library: argument validation, the host plan
// (orientation, padding, fp64 scalars, workspace carving) and the launch
// order. See include/muon_adamw.h for the contract of every entry point.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/muon_adamw.h"
#include "adamw.hpp"
#include "lion.hpp"
#include "calib.hpp"
#include "muon_elem.hpp"
#include "ns_gemm.hpp"

using namespace ma;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ----------------------------------------------------------------------------
// kernel timing (ma_profile_*)
// ----------------------------------------------------------------------------
struct Profiler {
  bool active = false;
  int used = 0;
  std::vector<hipEvent_t> ev;   // 2 per launch
  std::vector<int> kind;        // per launch
} g_prof;

struct ProfScope {
  int slot = -1;
  hipStream_t s;
  ProfScope(int k, hipStream_t st) : s(st) {
    if (g_prof.active && g_prof.used < (int)g_prof.kind.size()) {
      slot = g_prof.used++;
      g_prof.kind[slot] = k;
      (void)hipEventRecord(g_prof.ev[2 * slot], s);
    }
  }
  ~ProfScope() {
    if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
  }
};

// ----------------------------------------------------------------------------
// roctx ranges on the calling thread (rocprofv3 --marker-trace): every entry
// point that enqueues work is one range, and the Muon step's phases nest in
// it. They span the host's enqueueing, not the GPU's execution.
// ----------------------------------------------------------------------------
struct EntryMark {
  explicit EntryMark(const char* what) { roctxRangePushA(what); }
  ~EntryMark() { roctxRangePop(); }
  EntryMark(const EntryMark&) = delete;
  EntryMark& operator=(const EntryMark&) = delete;
};

struct PhaseMark {
  bool open = false;
  void enter(const char* what) {
    leave();
    roctxRangePushA(what);
    open = true;
  }
  void leave() {
    if (open) roctxRangePop();
    open = false;
  }
  ~PhaseMark() { leave(); }
};

inline int64_t dt_bytes(int dt) { return dt == MA_BF16 ? 2 : 4; }
inline bool dt_valid(int dt) { return dt == MA_F32 || dt == MA_BF16; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

NsTile ns_tile(int dtype, bool symmetric);

// Whether the AXPY launches read X^T from the row-major X through transposing
// LDS reads (NsTile::qt): the 8-wave bf16 LDS-DMA tile, unless MA_NS_QT=0.
// Then no X^T copy of the iterate is written.
bool ns_q_transposed(int dtype) {
  if (dtype != MA_BF16) return false;
  static const bool off = [] { const char* e = getenv("MA_NS_QT"); return e && strcmp(e, "0") == 0; }();
  const NsTile t = ns_tile(dtype, false);
  return !off && t.dma && t.wgm == 2 && t.wgn == 4 && t.bk == 64;
}

// Whether POLY writes only the upper triangle of B (no mirrored tiles), AXPY
// reading the blocks left of the diagonal transposed from those above it:
// with the transposed AXPY operands, unless MA_NS_SYMUP=0.
bool ns_b_upper(int dtype) {
  static const bool off = [] { const char* e = getenv("MA_NS_SYMUP"); return e && strcmp(e, "0") == 0; }();
  return !off && ns_q_transposed(dtype);
}


// Newton-Schulz GEMM tiles (the symmetric products need square ones): in bf16
// the LDS-DMA kernel, 256 x 256 x 64 with 8 waves (2 x 4 of 128 x 64, two per
// SIMD); in fp32 the register-staged kernel, 128 x 128 x 32 with 2 x 2 waves.
NsTile ns_tile(int dtype, bool /*symmetric*/) {
  if (dtype != MA_BF16) return {128, 128, 32, 2, 2, 0};
  return {256, 256, ns_dma_bk(), 2, 4, 1};
}

// An fp32 launch with fewer 128 x 128 jobs than this takes 64 x 64 tiles (2 x 2
// waves of 32 x 32): a few long jobs would leave most of the 256 CUs idle, and
// a quarter of the tile runs its K loop in a quarter of the time. Both tiles
// accumulate every output over k in the same order with the same
// instructions, so they give the same bits.
constexpr int kF32SmallLaunchJobs = 128;
constexpr NsTile kF32SmallTile = {64, 64, 32, 2, 2, 0};

// A bf16 Gram or POLY launch with fewer than this many 256 x 256 jobs (the
// 4-layer d=256 set has 24) runs the register-staged kernel on 128 x 128
// tiles, or on 64 x 64 ones under the fp32 rule above: a launch of a few long
// LDS-DMA jobs lasts as long as one job's prologue, K loop and epilogue,
// while the smaller tiles spread the same work over 4-16 times as many CUs.
// POLY then writes B with its mirrored tiles, and the AXPY of the same
// matrices reads B as stored (its transposed reads of the upper triangle
// assume 256 x 256 blocks). AXPY itself keeps the LDS-DMA kernel, which reads
// X^T out of X.
constexpr int kBf16SmallLaunchJobs = 64;
constexpr NsTile kBf16SmallTile = {128, 128, 32, 2, 2, 0};

// Such a launch's Gram product (K = the long side, up to 4x the short one)
// is also split along K into up to 4 slices of whole 256-column blocks, so
// that its jobs x slices stay within this many blocks: each slice's partial
// product goes to a workspace buffer of its own, and k_split_sum adds the
// slices in order (deterministic, but rounded differently from one pass over
// K). An fp32 iterate is never stored before its Frobenius factor (the
// one-pass X0 is bf16 only), so there is no factor to apply to the sum.
constexpr int kF32SplitMaxBlocks = 256;

// Slices for an fp32 group's Gram product when launched alone: 1 (no split)
// unless the group takes the 64 x 64 tiles and K spans at least two
// 256-column blocks; the slice count divides those blocks.
int f32_gram_split(int64_t count, int64_t m_pad, int64_t n_pad) {
  const int64_t t128 = m_pad / 128, t64 = m_pad / 64;
  if (count * t128 * (t128 + 1) / 2 >= kF32SmallLaunchJobs) return 1;
  const int64_t jobs = count * t64 * (t64 + 1) / 2;
  const int64_t kb = n_pad / 256;
  int sl = (int)std::min<int64_t>({4, kb, kF32SplitMaxBlocks / std::max<int64_t>(jobs, 1)});
  while (sl > 1 && kb % sl) --sl;
  return sl;
}

// ----------------------------------------------------------------------------
// plan of one Muon call
// ----------------------------------------------------------------------------
struct GroupPlan {
  int64_t R, C, m, n, m_pad, n_pad, r_ext, c_ext;
  bool tall;                 // R > C: the iteration runs on X0^T
  int count;
  int dt_p, dt_g, dt_m, dt_x;
  float c_lr, c_wd;
  int64_t x_stride, a_stride, row_stride;   // elements / floats
  size_t off_x[2], off_xt[2], off_a, off_b, off_rowsq, off_rowf;   // bytes
  size_t off_part;           // update-norm partial sums: count x ppm_max x 2 floats
  size_t off_flags;          // non-finite flags: count int32
  int gram_split;            // fp32 Gram product split along K into this many slices (1: none)
  size_t off_gpart;          // their partial products: gram_split x count x a_stride floats
  bool check_finite;
  int ppm_max;
  const ma_muon_group* src;
  // views in the parameter's layout ("direct") and transposed
  size_t off_direct(int buf) const { return tall ? off_xt[buf] : off_x[buf]; }
  size_t off_trans(int buf) const { return tall ? off_x[buf] : off_xt[buf]; }
  int64_t ld_direct() const { return tall ? m_pad : n_pad; }
  int64_t ld_trans() const { return tall ? n_pad : m_pad; }
};

struct Plan {
  std::vector<GroupPlan> g;
  size_t bytes = 0;
};

void plan_group(GroupPlan& p, int64_t R, int64_t C, int count, int dt_x, size_t& off) {
  p.R = R;
  p.C = C;
  p.count = count;
  p.tall = R > C;
  p.m = std::min(R, C);
  p.n = std::max(R, C);
  p.m_pad = round_up(p.m, kPad);
  p.n_pad = round_up(p.n, kPad);
  p.r_ext = p.tall ? p.n_pad : p.m_pad;
  p.c_ext = p.tall ? p.m_pad : p.n_pad;
  p.dt_x = dt_x;
  const int64_t e = dt_bytes(dt_x);
  p.x_stride = p.m_pad * p.n_pad;
  p.a_stride = p.m_pad * p.m_pad;
  p.row_stride = round_up(R, 64);
  // X^T buffers: read by the fp32 iteration; in bf16 (AXPY reads X^T out of
  // X) only a tall matrix uses them, as its parameter's layout. Otherwise
  // they alias X and are never accessed.
  const bool need_xt = p.tall || !ns_q_transposed(dt_x);
  for (int b = 0; b < 2; ++b) {
    p.off_x[b] = off;  off = align_up(off + (size_t)(count * p.x_stride * e), MA_WORKSPACE_ALIGN);
    p.off_xt[b] = p.off_x[b];
    if (need_xt) { p.off_xt[b] = off; off = align_up(off + (size_t)(count * p.x_stride * e), MA_WORKSPACE_ALIGN); }
  }
  p.off_a = off;     off = align_up(off + (size_t)(count * p.a_stride * e), MA_WORKSPACE_ALIGN);
  p.off_b = off;     off = align_up(off + (size_t)(count * p.a_stride * e), MA_WORKSPACE_ALIGN);
  p.off_rowsq = off; off = align_up(off + (size_t)(count * p.row_stride * 4), MA_WORKSPACE_ALIGN);
  p.off_rowf = off;  off = align_up(off + (size_t)(count * p.row_stride * 4), MA_WORKSPACE_ALIGN);
  p.ppm_max = post_blocks_per_mat_max(R, C);
  p.off_part = off;  off = align_up(off + (size_t)count * p.ppm_max * 2 * 4, MA_WORKSPACE_ALIGN);
  p.off_flags = off; off = align_up(off + (size_t)count * 4, MA_WORKSPACE_ALIGN);
  p.gram_split = dt_x == MA_F32 ? f32_gram_split(count, p.m_pad, p.n_pad) : 1;
  p.off_gpart = off;
  if (p.gram_split > 1) off = align_up(off + (size_t)p.gram_split * count * p.a_stride * 4, MA_WORKSPACE_ALIGN);
}

// Largest Muon group (count x rows x cols) and flat AdamW / Lion segment, in
// elements: 2^40 is 2 TiB of bf16, far beyond one GPU's memory.
constexpr int64_t kMaxGroupElems = (int64_t)1 << 40;
constexpr int64_t kMaxSegmentElems = (int64_t)1 << 40;

int validate_hparams(const ma_muon_hparams* hp) {
  if (!hp) return fail(MA_ERR_INVALID_ARG, "hparams is null");
  if (hp->ns_steps < 0 || hp->ns_steps > MA_MAX_NS_STEPS)
    return fail(MA_ERR_INVALID_ARG, "ns_steps %d outside 0..%d", hp->ns_steps, MA_MAX_NS_STEPS);
  if (hp->ns_steps > 0 && !hp->abc) return fail(MA_ERR_INVALID_ARG, "abc is null with ns_steps > 0");
  if (hp->equilibrate < MA_EQ_OFF || hp->equilibrate > MA_EQ_ROWS_RMS)
    return fail(MA_ERR_INVALID_ARG, "equilibrate %d is not an ma_eq value", hp->equilibrate);
  if (hp->lr_scale < MA_SCALE_NONE || hp->lr_scale > MA_SCALE_SQRT_MAX)
    return fail(MA_ERR_INVALID_ARG, "lr_scale %d is not an ma_scale value", hp->lr_scale);
  if (!dt_valid(hp->ns_precision)) return fail(MA_ERR_UNSUPPORTED, "ns_precision %d", hp->ns_precision);
  if (hp->check_finite != 0 && hp->check_finite != 1)
    return fail(MA_ERR_INVALID_ARG, "check_finite %d is not 0 or 1", hp->check_finite);
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->momentum) || !std::isfinite(hp->weight_decay) ||
      !std::isfinite(hp->norm_eps) || !std::isfinite(hp->eq_eps))
    return fail(MA_ERR_INVALID_ARG, "non-finite hyperparameter");
  for (int i = 0; i < 3 * hp->ns_steps; ++i)
    if (!std::isfinite(hp->abc[i])) return fail(MA_ERR_INVALID_ARG, "non-finite coefficient abc[%d]", i);
  return MA_OK;
}

// A device buffer's byte range and what it is (for the message).
enum RangeTag { R_PARAM, R_GRAD, R_MOMENTUM, R_WORKSPACE, R_STATS, R_ADAMW, R_LION };
struct Range { uintptr_t lo, hi; int tag; };

const char* range_name(int tag) {
  switch (tag) {
    case R_PARAM: return "a Muon parameter";
    case R_GRAD: return "a Muon gradient";
    case R_MOMENTUM: return "a Muon momentum buffer";
    case R_WORKSPACE: return "the workspace";
    case R_STATS: return "the stats array";
    case R_ADAMW: return "an AdamW buffer";
    case R_LION: return "a Lion buffer";
  }
  return "a buffer";
}

int check_overlaps(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < rs.size(); ++i)
    if (rs[i].lo < rs[i - 1].hi)
      return fail(MA_ERR_INVALID_ARG, "device buffers overlap (%s and %s)", range_name(rs[i - 1].tag),
                  range_name(rs[i].tag));
  return MA_OK;
}

int validate_group(const ma_muon_group& g, int idx, bool need_ptrs) {
  if (g.rows <= 0 || g.cols <= 0 || g.count < 0)
    return fail(MA_ERR_INVALID_ARG, "group %d: rows/cols must be > 0 and count >= 0", idx);
  if (g.rows > (1 << 24) || g.cols > (1 << 24) || g.rows * g.cols > (int64_t)1 << 31)
    return fail(MA_ERR_INVALID_ARG, "group %d: matrix too large", idx);
  // keeps every tile-job count and launch size of the group within int32
  if ((int64_t)g.count * g.rows * g.cols > kMaxGroupElems)
    return fail(MA_ERR_INVALID_ARG, "group %d: more than 2^40 elements in all", idx);
  if (!dt_valid(g.param_dtype) || !dt_valid(g.grad_dtype) || !dt_valid(g.mom_dtype))
    return fail(MA_ERR_UNSUPPORTED, "group %d: dtype must be MA_F32 or MA_BF16", idx);
  if (need_ptrs && g.count > 0) {
    if (!g.params || !g.grads || !g.momentum)
      return fail(MA_ERR_INVALID_ARG, "group %d: pointer array is null", idx);
    for (int i = 0; i < g.count; ++i) {
      if (!g.params[i] || !g.grads[i] || !g.momentum[i])
        return fail(MA_ERR_INVALID_ARG, "group %d matrix %d: null device pointer", idx, i);
      if (((uintptr_t)g.params[i] % dt_bytes(g.param_dtype)) || ((uintptr_t)g.grads[i] % dt_bytes(g.grad_dtype)) ||
          ((uintptr_t)g.momentum[i] % dt_bytes(g.mom_dtype)))
        return fail(MA_ERR_INVALID_ARG, "group %d matrix %d: pointer not aligned to its element size", idx, i);
    }
  }
  return MA_OK;
}

// Per-matrix lr multiplier (see ma_scale), in double on the host.
double lr_multiplier(int scale, int64_t R, int64_t C) {
  switch (scale) {
    case MA_SCALE_SQRT_MAX1_R_OVER_C: return std::sqrt(std::max(1.0, (double)R / (double)C));
    case MA_SCALE_MOONSHOT: return 0.2 * std::sqrt((double)std::max(R, C));
    case MA_SCALE_SQRT_MAX: return std::sqrt((double)std::max(R, C));
    default: return 1.0;
  }
}

int build_plan(const ma_muon_group* groups, int32_t n, const ma_muon_hparams* hp, Plan& plan,
               bool need_ptrs) {
  if (n < 0 || (n > 0 && !groups)) return fail(MA_ERR_INVALID_ARG, "groups is null or n_groups < 0");
  int rc = validate_hparams(hp);
  if (rc) return rc;
  plan.g.clear();
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    rc = validate_group(groups[i], i, need_ptrs);
    if (rc) return rc;
    GroupPlan p{};
    plan_group(p, groups[i].rows, groups[i].cols, groups[i].count, hp->ns_precision, off);
    p.dt_p = groups[i].param_dtype;
    p.dt_g = groups[i].grad_dtype;
    p.dt_m = groups[i].mom_dtype;
    const double mult = lr_multiplier(hp->lr_scale, p.R, p.C);
    const double lr_eff = (double)hp->lr * mult;
    p.c_lr = (float)lr_eff;
    p.c_wd = (float)(lr_eff * (double)hp->weight_decay);
    p.check_finite = hp->check_finite != 0;
    p.src = &groups[i];
    plan.g.push_back(p);
  }
  plan.bytes = off;
  return MA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// C % 8 == 0 and every parameter, gradient and momentum buffer of the group
// 16-byte aligned: the elementwise kernels' vector path
bool group_vec(const GroupPlan& p) {
  bool vec = (p.C % 8) == 0;
  if (p.src)
    for (int k = 0; k < p.count; ++k)
      vec = vec && aligned16(p.src->grads[k]) && aligned16(p.src->momentum[k]) && aligned16(p.src->params[k]);
  return vec;
}

ElemArgs elem_args(const GroupPlan& p, const ma_muon_hparams* hp, unsigned char* ws, int first,
                   int cnt) {
  ElemArgs a{};
  a.R = (int32_t)p.R;
  a.C = (int32_t)p.C;
  a.count = cnt;
  a.r_ext = (int32_t)p.r_ext;
  a.c_ext = (int32_t)p.c_ext;
  a.tiles_r = (int32_t)(p.r_ext / 64);
  a.tiles_c = (int32_t)(p.c_ext / 64);
  const int64_t e = dt_bytes(p.dt_x);
  a.x_stride = p.x_stride;
  a.xd = ws + p.off_direct(0) + (size_t)(first * p.x_stride * e);
  a.xt = ws + p.off_trans(0) + (size_t)(first * p.x_stride * e);
  a.ld_d = p.ld_direct();
  a.ld_t = p.ld_trans();
  a.row_stride = p.row_stride;
  a.rowsq = reinterpret_cast<float*>(ws + p.off_rowsq) + first * p.row_stride;
  a.rowf = reinterpret_cast<float*>(ws + p.off_rowf) + first * p.row_stride;
  a.beta = hp->momentum;
  a.nesterov = hp->nesterov ? 1 : 0;
  a.c_lr = p.c_lr;
  a.c_wd = p.c_wd;
  a.cautious = hp->cautious ? 1 : 0;
  a.decay = hp->weight_decay != 0.0f ? 1 : 0;
  a.norm_eps = hp->norm_eps;
  a.eq_eps = hp->eq_eps;
  for (int i = 0; i < cnt; ++i) {
    const int k = first + i;
    a.mat[i].g = p.src ? p.src->grads[k] : nullptr;
    a.mat[i].m = p.src ? p.src->momentum[k] : nullptr;
    a.mat[i].w = p.src ? p.src->params[k] : nullptr;
  }
  a.vec = group_vec(p) ? 1 : 0;
  a.nonfinite = hp->check_finite ? reinterpret_cast<int32_t*>(ws + p.off_flags) + first : nullptr;
  return a;
}

// Enqueue T quintic steps for every group of the plan; X[0]/X^T[0] hold X0.
// scaled (optional): per group, whether X0 holds Y with X0 = s Y, s in the
// group's row-factor slot of row 0 of each matrix (k_finalize mode 4).
// before_axpy (optional): called once, before the first AXPY launch is enqueued.
// fused (optional): per group, the update to apply in the last AXPY's
// epilogue (NsGroup::W null: none).
// the AdamW fork of ma_muon_adamw_step: before product 3 * step + (GRAM 0,
// POLY 1, AXPY 2) = the first AXPY
constexpr int kForkAt = 2;
int enqueue_ns(const Plan& plan, unsigned char* ws, const float* abc, int T, int dtype,
               hipStream_t s, const std::vector<char>* scaled = nullptr,
               const std::function<int()>* before_axpy = nullptr,
               const std::vector<NsGroup>* fused = nullptr) {
  if (T == 0 || plan.g.empty()) return MA_OK;
  // groups with the most work per tile first (they set the tail of a launch)
  std::vector<int> order;
  for (int i = 0; i < (int)plan.g.size(); ++i)
    if (plan.g[i].count > 0) order.push_back(i);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return plan.g[a].n_pad > plan.g[b].n_pad; });
  const int64_t e = dt_bytes(dtype);

  for (int step = 0; step < T; ++step) {
    const int cur = step & 1, nxt = cur ^ 1;
    const bool last = step == T - 1;
    for (int epi = EPI_GRAM; epi <= EPI_AXPY; ++epi) {
      if (step * 3 + epi == kForkAt && before_axpy) {
        const int rc = (*before_axpy)();
        if (rc) return rc;
      }
      NsTile tile0 = ns_tile(dtype, epi != EPI_AXPY);
      const bool qt = epi == EPI_AXPY && ns_q_transposed(dtype);
      tile0.qt = qt ? 1 : 0;
      // B is stored as its upper triangle when AXPY reads the rest transposed
      const bool b_upper = ns_b_upper(dtype);
      if (epi != EPI_AXPY && tile0.bm != tile0.bn) return fail(MA_ERR_INVALID_ARG, "symmetric GEMM tile must be square");
      for (size_t base = 0; base < order.size(); base += kMaxNsGroups) {
        const size_t nb = std::min(order.size() - base, (size_t)kMaxNsGroups);
        NsTile tile = tile0;
        // bf16: the symmetric products of this batch on the register-staged kernel
        bool sym_reg = false;
        if (tile0.dma) {
          int64_t jobs = 0;
          for (size_t q = 0; q < nb; ++q) {
            const GroupPlan& p = plan.g[order[base + q]];
            const int64_t tm = p.m_pad / tile0.bm;
            jobs += p.count * tm * (tm + 1) / 2;
          }
          sym_reg = jobs < kBf16SmallLaunchJobs;
          if (sym_reg && epi != EPI_AXPY) tile = kBf16SmallTile;
        }
        if (!tile.dma) {
          int64_t jobs = 0;
          for (size_t q = 0; q < nb; ++q) {
            const GroupPlan& p = plan.g[order[base + q]];
            const int64_t tm = p.m_pad / tile.bm, tn = p.n_pad / tile.bn;
            jobs += p.count * (epi == EPI_AXPY ? tm * tn : tm * (tm + 1) / 2);
          }
          if (jobs < kF32SmallLaunchJobs) tile = kF32SmallTile;
        }
        NsArgs A{};
        A.a = abc[3 * step];
        A.b = abc[3 * step + 1];
        A.c = abc[3 * step + 2];
        int rot = 0;
        bool any_fused = false;
        for (size_t q = 0; q < nb; ++q) {
          const GroupPlan& p = plan.g[order[base + q]];
          NsGroup& G = A.g[q];
          const int tm = (int)(p.m_pad / tile.bm);
          const int tn = (int)(p.n_pad / tile.bn);
          G.count = p.count;
          if (epi == EPI_GRAM || epi == EPI_POLY) {
            const unsigned char* src = ws + (epi == EPI_GRAM ? p.off_x[cur] : p.off_a);
            G.P = G.Q = src;
            G.sP = G.sQ = epi == EPI_GRAM ? p.x_stride : p.a_stride;
            G.ldP = G.ldQ = (int32_t)(epi == EPI_GRAM ? p.n_pad : p.m_pad);
            G.K = (int32_t)(epi == EPI_GRAM ? p.n_pad : p.m_pad);
            G.E = ws + p.off_a;
            G.sE = p.a_stride;
            G.ldE = (int32_t)p.m_pad;
            void* out = ws + (epi == EPI_GRAM ? p.off_a : p.off_b);
            G.outN = G.outT = out;
            G.sN = G.sT = p.a_stride;
            G.ldN = G.ldT = (int32_t)p.m_pad;
            G.tm = G.tn = tm;
            G.tiles = tm * (tm + 1) / 2;
            G.symmetric = 1;
            G.upper_only = epi == EPI_POLY && b_upper && !sym_reg ? 1 : 0;
          } else {
            G.P = ws + p.off_b;
            G.sP = p.a_stride;
            G.ldP = (int32_t)p.m_pad;
            // Q = X^T: its own copy, or (qt) X itself read transposed
            G.Q = ws + (qt ? p.off_x[cur] : p.off_xt[cur]);
            G.sQ = p.x_stride;
            G.ldQ = (int32_t)(qt ? p.n_pad : p.m_pad);
            G.K = (int32_t)p.m_pad;
            G.E = ws + p.off_xt[cur];   // not read: AXPY folds a*X into its main loop
            G.sE = p.x_stride;
            G.ldE = (int32_t)p.m_pad;
            // the last step writes only the copy in the parameter's layout;
            // the others X' and, unless qt, X'^T
            G.outN = (!last || !p.tall) ? (void*)(ws + p.off_x[nxt]) : nullptr;
            G.outT = ((!last && !qt) || (last && p.tall)) ? (void*)(ws + p.off_xt[nxt]) : nullptr;
            G.sN = G.sT = p.x_stride;
            G.ldN = (int32_t)p.n_pad;
            G.ldT = (int32_t)p.m_pad;
            G.tm = tm;
            G.tn = tn;
            G.tiles = tm * tn;
            G.symmetric = 0;
            G.p_upper = b_upper && !sym_reg ? 1 : 0;
          }
          // the first GRAM and AXPY apply the deferred Frobenius factor
          const bool sc = step == 0 && epi != EPI_POLY && scaled && (*scaled)[order[base + q]];
          G.scale = sc ? reinterpret_cast<const float*>(ws + p.off_rowf) : nullptr;
          G.scale_stride = p.row_stride;
          if (epi == EPI_AXPY && last && fused && (*fused)[order[base + q]].W) {
            const NsGroup& F = (*fused)[order[base + q]];
            G.W = F.W;
            G.sW = F.sW;
            G.R = F.R;
            G.C = F.C;
            G.w_trans = F.w_trans;
            G.cautious = F.cautious;
            G.decay = F.decay;
            G.c_lr = F.c_lr;
            G.c_wd = F.c_wd;
            G.nonfinite = F.nonfinite;
            any_fused = true;
          }
          G.unit = G.count >= 8 ? G.tiles : 1;
          G.rot = rot;
          rot = (rot + G.count * G.tiles / G.unit) & 7;
        }
        (void)e;
        A.n_groups = (int32_t)nb;
        // an fp32 Gram launch of few long jobs: every group's K in `split`
        // slices, each slice a group of its own writing a partial product
        int split = 1;
        if (epi == EPI_GRAM && !tile.dma && tile.bm == kF32SmallTile.bm) {
          split = 4;
          int64_t jobs = 0;
          for (size_t q = 0; q < nb; ++q) {
            split = std::min(split, plan.g[order[base + q]].gram_split);
            jobs += (int64_t)A.g[q].count * A.g[q].tiles;
          }
          if (split < 2 || (int)nb * split > kMaxNsGroups || jobs * split > kF32SplitMaxBlocks) split = 1;
          for (size_t q = 0; q < nb && split > 1; ++q)
            if ((A.g[q].K / 256) % split || A.g[q].scale) split = 1;
        }
        if (split > 1) {
          NsArgs S = A;
          int k = 0;
          rot = 0;
          for (size_t q = 0; q < nb; ++q) {
            const GroupPlan& p = plan.g[order[base + q]];
            const int32_t kc = A.g[q].K / split;
            for (int sl = 0; sl < split; ++sl, ++k) {
              NsGroup G = A.g[q];
              G.P = G.Q = reinterpret_cast<const unsigned char*>(A.g[q].P) + (size_t)sl * kc * e;
              G.K = kc;
              void* part = ws + p.off_gpart + (size_t)sl * p.count * p.a_stride * e;
              G.outN = G.outT = part;
              G.rot = rot;
              rot = (rot + G.count * G.tiles / G.unit) & 7;
              S.g[k] = G;
            }
          }
          S.n_groups = k;
          A = S;
        }
        int per_xcd = 0;
        for (int x = 0; x < 8; ++x) {
          int jx = 0;
          for (int q = 0; q < A.n_groups; ++q) {
            const NsGroup& G = A.g[q];
            const int units = G.count * G.tiles / G.unit;
            const int u0 = (x - G.rot + 8) & 7;
            jx += (units > u0 ? (units - u0 + 7) / 8 : 0) * G.unit;
          }
          per_xcd = std::max(per_xcd, jx);
        }
        A.per_xcd = per_xcd;
        A.padded_blocks = 8 * per_xcd;
        if (tile.dma) A.padded_blocks = 8 * std::min(per_xcd, kNsPersBlocksPerXcd);
        hipError_t err;
        {
          ProfScope ps(any_fused ? MA_K_AXPY_UPDATE : MA_K_GRAM + epi, s);
          err = launch_ns_gemm(dtype, epi, tile, A, s);
        }
        if (err != hipSuccess) return hip_fail(err, "Newton-Schulz GEMM launch");
        if (split > 1) {
          SplitSumArgs R{};
          R.n = (int32_t)nb;
          int64_t blocks = 0;
          for (size_t q = 0; q < nb; ++q) {
            const GroupPlan& p = plan.g[order[base + q]];
            SplitSumGroup& g = R.g[q];
            g.part = reinterpret_cast<const float*>(ws + p.off_gpart);
            g.out = reinterpret_cast<float*>(ws + p.off_a);
            g.split_stride = (int64_t)p.count * p.a_stride;
            g.mat_elems = p.a_stride;
            g.slices = split;
            g.block_begin = blocks;
            blocks += g.split_stride / kSplitSumBlockElems;
          }
          R.blocks = blocks;
          {
            ProfScope ps(MA_K_GRAM, s);
            err = launch_split_sum(R, s);
          }
          if (err != hipSuccess) return hip_fail(err, "Gram slice sum");
        }
      }
    }
  }
  return MA_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

const char* ma_version(void) { return "muon_adamw 0.1 (gfx950)"; }

const char* ma_status_string(int status) {
  switch (status) {
    case MA_OK: return "ok";
    case MA_ERR_INVALID_ARG: return "invalid argument";
    case MA_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case MA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MA_ERR_HIP: return "HIP runtime error";
    case MA_ERR_NONFINITE: return "non-finite values in a Muon step";
  }
  return "unknown status";
}

const char* ma_last_error(void) { return g_last_error.c_str(); }

int ma_profile_begin(int32_t max_launches) {
  if (max_launches < 0 || max_launches > (1 << 20)) return fail(MA_ERR_INVALID_ARG, "max_launches out of range");
  const size_t need = 2 * (size_t)max_launches;
  while (g_prof.ev.size() < need) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
    g_prof.ev.push_back(e);
  }
  g_prof.kind.assign(max_launches, -1);
  g_prof.used = 0;
  g_prof.active = true;
  return MA_OK;
}

int ma_profile_end(void) {
  g_prof.active = false;
  return MA_OK;
}

int ma_profile_read(int32_t kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= MA_K_COUNT || !total_ms || !launches) return fail(MA_ERR_INVALID_ARG, "bad kind or null output");
  double t = 0.0;
  int64_t n = 0;
  for (int i = 0; i < g_prof.used; ++i) {
    if (g_prof.kind[i] != kind) continue;
    hipError_t err = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return MA_OK;
}

size_t ma_muon_workspace_size(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp) {
  Plan plan;
  if (build_plan(groups, n_groups, hp, plan, false) != MA_OK) return 0;
  return plan.bytes;
}

// Whether a group's momentum update, row sums and X0 run as one row pass
// (k_pre_rows), the Frobenius factor then applied by the first GRAM and AXPY:
// MuonEq pre with at least one Newton-Schulz step, a matrix whose iteration
// layout is the parameter's (no more rows than columns), an iteration that
// needs no X0^T (AXPY reads X^T out of X) and rows the pass holds in
// registers; unless MA_PRE_ROWS=0.
bool pre_rows_for(const GroupPlan& p, const ma_muon_hparams* hp) {
  static const bool off = [] { const char* e = getenv("MA_PRE_ROWS"); return e && strcmp(e, "0") == 0; }();
  return !off && hp->equilibrate == MA_EQ_ROWS_PRE && hp->ns_steps > 0 && !p.tall && ns_q_transposed(p.dt_x) &&
         group_vec(p) && p.C <= kPreRowsMaxCols && p.c_ext <= kPreRowsMaxCols && p.ld_direct() % 8 == 0;
}

namespace {
// Whether the iteration's result is row-scaled before the update (MuonEq
// after the iteration, NorMuon): the update then waits for those factors.
bool rows_after_ns(const ma_muon_hparams* hp) {
  return hp->equilibrate == MA_EQ_ROWS_POST || hp->equilibrate == MA_EQ_ROWS_RMS;
}

// Whether the last AXPY can apply a group's update in its epilogue: a bf16
// iteration with at least one step (the LDS-DMA kernel writes U), bf16
// weights with rows of a multiple of 8 elements, stacked at one
// 16-byte-aligned stride (*stride_elems), as same-shape matrices stored in one
// tensor are.
bool update_fusable(const GroupPlan& p, const ma_muon_hparams* hp, int64_t* stride_elems) {
  if (p.count == 0 || !p.src || hp->ns_steps == 0 || p.dt_x != MA_BF16 || !ns_q_transposed(p.dt_x)) return false;
  if (p.dt_p != MA_BF16) return false;
  if (p.C % 8 != 0) return false;
  const int64_t eb = dt_bytes(p.dt_p);
  const uintptr_t w0 = (uintptr_t)p.src->params[0];
  if (w0 % 16) return false;
  const int64_t stride = p.count > 1 ? (int64_t)((uintptr_t)p.src->params[1] - w0) : p.R * p.C * eb;
  if (stride < p.R * p.C * eb || stride % 16) return false;
  for (int k = 2; k < p.count; ++k)
    if ((uintptr_t)p.src->params[k] != w0 + (uintptr_t)(k * stride)) return false;
  *stride_elems = stride / eb;
  return true;
}

// k_finalize launches batched over groups: add() queues one group's
// matrices, flush() launches what is queued (also when a batch fills).
struct FinalizeBatch {
  FinalizeArgs a{};
  int blocks = 0;
  hipStream_t s;
  FinalizeBatch(const ma_muon_hparams* hp, hipStream_t st) : s(st) {
    a.norm_eps = hp->norm_eps;
    a.eq_eps = hp->eq_eps;
  }
  int add(const GroupPlan& p, unsigned char* ws, int mode) {
    if (p.count == 0) return MA_OK;
    if (a.n == kMaxFinalizeGroups) {
      const int rc = flush();
      if (rc) return rc;
    }
    FinalizeGroup& g = a.g[a.n++];
    g.rowsq = reinterpret_cast<const float*>(ws + p.off_rowsq);
    g.rowf = reinterpret_cast<float*>(ws + p.off_rowf);
    g.nonfinite = p.check_finite ? reinterpret_cast<int32_t*>(ws + p.off_flags) : nullptr;
    g.row_stride = p.row_stride;
    g.R = (int32_t)p.R;
    g.C = (int32_t)p.C;
    g.mode = mode;
    g.block_begin = blocks;
    blocks += p.count;
    return MA_OK;
  }
  int flush() {
    if (a.n == 0) return MA_OK;
    hipError_t err;
    {
      ProfScope ps(MA_K_FINALIZE, s);
      err = launch_finalize(a, blocks, s);
    }
    a.n = 0;
    blocks = 0;
    return err == hipSuccess ? MA_OK : hip_fail(err, "norm finalize");
  }
};

// Everything a Muon call checks before its first launch (no HIP call): the
// plan, the workspace, and the byte range of every device buffer it touches,
// appended to `rs` for the overlap check.
// caller_ws false: the workspace is the library's own scratch array
// (ma_muon_step_noalloc; not checked, not in `rs`).
int muon_prepare(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, void* workspace,
                 size_t workspace_bytes, float* stats, Plan& plan, std::vector<Range>& rs, bool caller_ws = true) {
  int rc = build_plan(groups, n_groups, hp, plan, true);
  if (rc) return rc;
  int64_t total = 0;
  for (const GroupPlan& p : plan.g) total += p.count;
  if (caller_ws && plan.bytes > 0) {
    if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is null");
    if ((uintptr_t)workspace % MA_WORKSPACE_ALIGN)
      return fail(MA_ERR_WORKSPACE, "workspace is not %d-byte aligned", MA_WORKSPACE_ALIGN);
    if (workspace_bytes < plan.bytes)
      return fail(MA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.bytes);
  }
  for (const GroupPlan& p : plan.g) {
    const ma_muon_group& g = *p.src;
    const uintptr_t ne = (uintptr_t)(p.R * p.C);
    for (int i = 0; i < g.count; ++i) {
      rs.push_back({(uintptr_t)g.params[i], (uintptr_t)g.params[i] + ne * dt_bytes(p.dt_p), R_PARAM});
      rs.push_back({(uintptr_t)g.grads[i], (uintptr_t)g.grads[i] + ne * dt_bytes(p.dt_g), R_GRAD});
      rs.push_back({(uintptr_t)g.momentum[i], (uintptr_t)g.momentum[i] + ne * dt_bytes(p.dt_m), R_MOMENTUM});
    }
  }
  if (caller_ws && plan.bytes > 0) rs.push_back({(uintptr_t)workspace, (uintptr_t)workspace + plan.bytes, R_WORKSPACE});
  if (stats && total > 0) rs.push_back({(uintptr_t)stats, (uintptr_t)(stats + 2 * total), R_STATS});
  return MA_OK;
}

// The launches of a Muon call that muon_prepare accepted. fork (optional):
// called once, when the first AXPY is about to be enqueued (or after the last
// launch when there is none).
int muon_enqueue(const Plan& plan, const ma_muon_hparams* hp, void* workspace, float* stats, void* stream,
                 const std::function<int()>* fork = nullptr) {
  bool forked = false;
  std::function<int()> fork_once = [&]() -> int {
    if (forked || !fork) return MA_OK;
    forked = true;
    return (*fork)();
  };
  int rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  hipError_t err;
  PhaseMark phase;
  // 1. per group: the row pass (momentum, row sums and the row-scaled X0), or
  // the row sums alone; 2. one launch of the per-matrix factors for every
  // group; 3. per two-pass group: the momentum update and X0
  phase.enter("muon: momentum, norms, X0");
  std::vector<char> scaled(plan.g.size(), 0);
  FinalizeBatch fin(hp, s);
  for (size_t gi = 0; gi < plan.g.size(); ++gi) {
    const GroupPlan& p = plan.g[gi];
    scaled[gi] = pre_rows_for(p, hp) ? 1 : 0;
    if (p.count == 0) continue;
    for (int first = 0; first < p.count; first += kMaxMatsPerLaunch) {
      const int cnt = std::min(kMaxMatsPerLaunch, p.count - first);
      const ElemArgs a = elem_args(p, hp, ws, first, cnt);
      if (scaled[gi]) {
        // a.xd is X0 in the parameter's layout, which is the iteration's
        { ProfScope ps(MA_K_PRE, s); err = launch_pre_rows(p.dt_g, p.dt_m, p.dt_x, a, s); }
        if (err != hipSuccess) return hip_fail(err, "momentum/row norms/X0");
      } else {
        { ProfScope ps(MA_K_ROWNORM, s); err = launch_rowsumsq_momentum(p.dt_g, p.dt_m, a, s); }
        if (err != hipSuccess) return hip_fail(err, "row norms");
      }
    }
    if ((rc = fin.add(p, ws, scaled[gi] ? 4 : (hp->equilibrate == MA_EQ_ROWS_PRE ? 1 : 0)))) return rc;
  }
  if ((rc = fin.flush())) return rc;
  for (size_t gi = 0; gi < plan.g.size(); ++gi) {
    const GroupPlan& p = plan.g[gi];
    if (scaled[gi]) continue;
    for (int first = 0; first < p.count; first += kMaxMatsPerLaunch) {
      const int cnt = std::min(kMaxMatsPerLaunch, p.count - first);
      ElemArgs ap = elem_args(p, hp, ws, first, cnt);
      if (ns_q_transposed(p.dt_x)) {
        // X0 in the iteration's layout X (for T > 0) and in the parameter's
        // layout (for T = 0); X0^T is not needed
        const bool t0 = hp->ns_steps == 0;
        if (!t0 && p.tall) ap.xd = nullptr;   // parameter's layout is X^T
        if (t0 || !p.tall) ap.xt = nullptr;   // the transposed view is X^T
      }
      { ProfScope ps(MA_K_PRE, s); err = launch_pre(p.dt_g, p.dt_m, p.dt_x, ap, s); }
      if (err != hipSuccess) return hip_fail(err, "momentum/X0");
    }
  }
  // 4. T quintic steps
  phase.enter("muon: Newton-Schulz");
  // the update of groups whose weights the last AXPY can update in its
  // epilogue (the separate update pass then skips them)
  std::vector<NsGroup> fused(plan.g.size());
  for (size_t gi = 0; gi < plan.g.size(); ++gi) {
    const GroupPlan& p = plan.g[gi];
    int64_t sw = 0;
    if (!stats && !rows_after_ns(hp) && update_fusable(p, hp, &sw)) {
      NsGroup& F = fused[gi];
      F.W = p.src->params[0];
      F.sW = sw;
      F.R = (int32_t)p.R;
      F.C = (int32_t)p.C;
      F.w_trans = p.tall ? 1 : 0;
      F.cautious = hp->cautious ? 1 : 0;
      F.decay = hp->weight_decay != 0.0f ? 1 : 0;
      F.c_lr = p.c_lr;
      F.c_wd = p.c_wd;
      F.nonfinite = hp->check_finite ? reinterpret_cast<const int32_t*>(ws + p.off_flags) : nullptr;
    }
  }
  rc = enqueue_ns(plan, ws, hp->abc, hp->ns_steps, hp->ns_precision, s, &scaled, &fork_once, &fused);
  if (rc) return rc;
  // 5. (MuonEq POST, NorMuon: the update's row sums, one launch of the row
  // factors) and the update (and the update norms)
  phase.enter("muon: update");
  const int ub = hp->ns_steps & 1;
  const bool rows_after = rows_after_ns(hp);
  auto update_args = [&](const GroupPlan& p, int first, int cnt) {
    ElemArgs a = elem_args(p, hp, ws, first, cnt);
    a.xd = ws + p.off_direct(ub) + (size_t)(first * p.x_stride * dt_bytes(p.dt_x));
    a.xt = nullptr;
    if (!rows_after) a.rowf = nullptr;
    return a;
  };
  if (rows_after) {
    for (const GroupPlan& p : plan.g) {
      if (p.count == 0) continue;
      for (int first = 0; first < p.count; first += kMaxMatsPerLaunch) {
        const ElemArgs a = update_args(p, first, std::min(kMaxMatsPerLaunch, p.count - first));
        { ProfScope ps(MA_K_ROWNORM, s); err = launch_rowsumsq_buffer(p.dt_x, a, s); }
        if (err != hipSuccess) return hip_fail(err, "update row norms");
      }
      if ((rc = fin.add(p, ws, hp->equilibrate == MA_EQ_ROWS_POST ? 2 : 3))) return rc;
    }
    if ((rc = fin.flush())) return rc;
  }
  int64_t mat0 = 0;   // index of the group's first matrix in `stats`
  for (size_t gi = 0; gi < plan.g.size(); ++gi) {
    const GroupPlan& p = plan.g[gi];
    if (fused[gi].W) continue;   // updated by the last AXPY
    for (int first = 0; first < p.count; first += kMaxMatsPerLaunch) {
      const int cnt = std::min(kMaxMatsPerLaunch, p.count - first);
      ElemArgs a = update_args(p, first, cnt);
      a.tiles_r = (int32_t)((p.R + 63) / 64);
      a.tiles_c = (int32_t)((p.C + 63) / 64);
      const int ppm = post_blocks_per_mat(a);   // <= p.ppm_max
      if (stats) a.part = reinterpret_cast<float*>(ws + p.off_part) + (int64_t)first * ppm * 2;
      { ProfScope ps(MA_K_POST, s); err = launch_post(p.dt_p, p.dt_x, a, s); }
      if (err != hipSuccess) return hip_fail(err, "update");
      if (stats) {
        err = launch_update_stats(a.part, ppm, cnt, stats + 2 * (mat0 + first), s);
        if (err != hipSuccess) return hip_fail(err, "update norms");
      }
    }
    mat0 += p.count;
  }
  return fork_once();
}

int muon_step_impl(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, void* workspace,
                   size_t workspace_bytes, float* stats, void* stream) {
  Plan plan;
  std::vector<Range> rs;
  int rc = muon_prepare(groups, n_groups, hp, workspace, workspace_bytes, stats, plan, rs);
  if (rc) return rc;
  if ((rc = check_overlaps(rs))) return rc;   // no two buffers may overlap, workspace included
  return muon_enqueue(plan, hp, workspace, stats, stream);
}
}  // namespace

int ma_muon_step(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                 void* workspace, size_t workspace_bytes, void* stream) {
  EntryMark mark("ma_muon_step");
  return muon_step_impl(groups, n_groups, hp, workspace, workspace_bytes, nullptr, stream);
}

// ---------------------------------------------------------------------------
// ma_muon_step_noalloc: the step's scratch memory in a fixed device array
// ---------------------------------------------------------------------------
// One copy per GPU the library runs on, held until the process ends. Host
// code never uses `scratch` itself (its host-side name is not a device
// address): the address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The library's own per-device objects (the scratch array, the fork and join
// events) are the current device's: a stream of another device must not be
// given them.
int check_stream_device(void* stream, const char* what) {
  int cur = 0;
  hipError_t err = hipGetDevice(&cur);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (!stream) return MA_OK;
  hipDevice_t sd = 0;
  err = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sd);
  if (err != hipSuccess) return hip_fail(err, "hipStreamGetDevice");
  if ((int)sd != cur)
    return fail(MA_ERR_INVALID_ARG, "%s belongs to device %d while device %d is current", what, (int)sd, cur);
  return MA_OK;
}

// The current device's address of `scratch` (looked up on the device's first
// call, with that device current).
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MA_ERR_INVALID_ARG, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    if ((uintptr_t)ptr % MA_WORKSPACE_ALIGN) return fail(MA_ERR_WORKSPACE, "scratch array is not aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MA_OK;
}
}  // namespace

int ma_muon_step_noalloc(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, void* stream) {
  EntryMark mark("ma_muon_step_noalloc");
  Plan plan;
  std::vector<Range> rs;
  int rc = muon_prepare(groups, n_groups, hp, nullptr, 0, nullptr, plan, rs, false);
  if (rc) return rc;
  if ((rc = check_overlaps(rs))) return rc;
  if (plan.bytes > (size_t)MA_NOALLOC_SCRATCH_BYTES)
    return fail(MA_ERR_WORKSPACE, "the step needs %zu bytes of scratch; ma_muon_step_noalloc has %zu (use ma_muon_step)",
                plan.bytes, (size_t)MA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = check_stream_device(stream, "the stream"))) return rc;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return muon_enqueue(plan, hp, ws, nullptr, stream);
}

int ma_muon_step_stats(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                       void* workspace, size_t workspace_bytes, float* stats, void* stream) {
  EntryMark mark("ma_muon_step_stats");
  if (!stats || ((uintptr_t)stats & 3)) return fail(MA_ERR_INVALID_ARG, "stats is null or not 4-byte aligned");
  return muon_step_impl(groups, n_groups, hp, workspace, workspace_bytes, stats, stream);
}

int ma_muon_nonfinite(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                      const void* workspace, int32_t* flags) {
  Plan plan;
  int rc = build_plan(groups, n_groups, hp, plan, false);
  if (rc) return rc;
  if (!hp->check_finite) return fail(MA_ERR_INVALID_ARG, "the step was not asked to check (check_finite == 0)");
  if (!workspace) return fail(MA_ERR_WORKSPACE, "workspace is null");
  std::vector<int32_t> f;
  bool any = false;
  for (const GroupPlan& p : plan.g) {
    if (p.count == 0) continue;
    const size_t at = f.size();
    f.resize(at + p.count);
    const hipError_t err = hipMemcpy(f.data() + at, reinterpret_cast<const unsigned char*>(workspace) + p.off_flags,
                                     (size_t)p.count * 4, hipMemcpyDeviceToHost);
    if (err != hipSuccess) return hip_fail(err, "reading the non-finite flags");
  }
  for (size_t i = 0; i < f.size(); ++i) {
    any = any || f[i] != 0;
    if (flags) flags[i] = f[i] != 0 ? 1 : 0;
  }
  return any ? fail(MA_ERR_NONFINITE, "a Muon matrix had non-finite norms; its weight was left unchanged") : MA_OK;
}

int ma_muon_row_pass(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp, int32_t group) {
  Plan plan;
  int rc = build_plan(groups, n_groups, hp, plan, false);
  if (rc) return rc;
  if (group < 0 || group >= n_groups) return fail(MA_ERR_INVALID_ARG, "group %d out of range", group);
  return pre_rows_for(plan.g[group], hp) ? 1 : 0;
}

int ma_muon_workspace_update(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                             void* workspace, int32_t group, int32_t index, void** u, int64_t* ld,
                             int32_t* transposed, int32_t* elem_bytes) {
  Plan plan;
  int rc = build_plan(groups, n_groups, hp, plan, false);
  if (rc) return rc;
  if (!workspace || !u || !ld || !elem_bytes) return fail(MA_ERR_INVALID_ARG, "null output pointer");
  if (group < 0 || group >= n_groups) return fail(MA_ERR_INVALID_ARG, "group %d out of range", group);
  const GroupPlan& p = plan.g[group];
  if (index < 0 || index >= p.count) return fail(MA_ERR_INVALID_ARG, "index %d out of range", index);
  const int ub = hp->ns_steps & 1;
  *u = reinterpret_cast<unsigned char*>(workspace) + p.off_direct(ub) +
       (size_t)((int64_t)index * p.x_stride * dt_bytes(p.dt_x));
  *ld = p.ld_direct();
  if (transposed) *transposed = 0;
  *elem_bytes = (int32_t)dt_bytes(p.dt_x);
  return MA_OK;
}

namespace {
// Argument checks of an AdamW call (no HIP call); the buffers' byte ranges
// are appended to `rs` for the overlap check.
int adamw_prepare(const ma_adamw_segment* segs, int32_t n, std::vector<Range>& rs) {
  if (n < 0 || (n > 0 && !segs)) return fail(MA_ERR_INVALID_ARG, "segments is null or n < 0");
  for (int i = 0; i < n; ++i) {
    const ma_adamw_segment& S = segs[i];
    if (S.n < 0 || S.n > kMaxSegmentElems) return fail(MA_ERR_INVALID_ARG, "segment %d: n < 0 or n > 2^40", i);
    if (S.param_dtype != MA_F32 || S.grad_dtype != MA_F32)
      return fail(MA_ERR_UNSUPPORTED, "segment %d: AdamW buffers must be MA_F32", i);
    if (S.n == 0) continue;
    if (!S.param || !S.grad || !S.exp_avg || !S.exp_avg_sq)
      return fail(MA_ERR_INVALID_ARG, "segment %d: null device pointer", i);
    if (((uintptr_t)S.param | (uintptr_t)S.grad | (uintptr_t)S.exp_avg | (uintptr_t)S.exp_avg_sq) & 3)
      return fail(MA_ERR_INVALID_ARG, "segment %d: pointer not 4-byte aligned", i);
    if (S.step < 1) return fail(MA_ERR_INVALID_ARG, "segment %d: step must be >= 1", i);
    if (!std::isfinite(S.lr) || !std::isfinite(S.beta1) || !std::isfinite(S.beta2) || !std::isfinite(S.eps) ||
        !std::isfinite(S.weight_decay) || S.beta1 < 0.f || S.beta1 >= 1.f || S.beta2 < 0.f || S.beta2 >= 1.f)
      return fail(MA_ERR_INVALID_ARG, "segment %d: hyperparameters out of range", i);
    const uintptr_t nb = (uintptr_t)S.n * 4;
    rs.push_back({(uintptr_t)S.param, (uintptr_t)S.param + nb, R_ADAMW});
    rs.push_back({(uintptr_t)S.grad, (uintptr_t)S.grad + nb, R_ADAMW});
    rs.push_back({(uintptr_t)S.exp_avg, (uintptr_t)S.exp_avg + nb, R_ADAMW});
    rs.push_back({(uintptr_t)S.exp_avg_sq, (uintptr_t)S.exp_avg_sq + nb, R_ADAMW});
  }
  return MA_OK;
}

int adamw_validate(const ma_adamw_segment* segs, int32_t n) {
  std::vector<Range> rs;
  const int rc = adamw_prepare(segs, n, rs);
  return rc ? rc : check_overlaps(rs);
}

// Launches for segments that adamw_validate accepted.
int adamw_enqueue(const ma_adamw_segment* segs, int32_t n, int32_t lean_blocks, void* stream) {
  int rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  AdamArgs A{};
  int64_t blocks = 0;
  auto flush = [&]() -> int {
    if (A.nseg == 0) return MA_OK;
    A.total_blocks = (int32_t)blocks;
    hipError_t err;
    {
      ProfScope ps(MA_K_ADAMW, s);
      err = launch_adamw(A, s);
    }
    A = AdamArgs{};
    A.lean_blocks = lean_blocks;
    blocks = 0;
    return err == hipSuccess ? MA_OK : hip_fail(err, "AdamW launch");
  };
  A.lean_blocks = lean_blocks;
  for (int i = 0; i < n; ++i) {
    const ma_adamw_segment& S = segs[i];
    if (S.n == 0) continue;
    const int64_t nb = (S.n + kAdamBlockElems - 1) / kAdamBlockElems;
    if (A.nseg == kMaxAdamSegs || blocks + nb > (int64_t)0x7fffffff) {
      if ((rc = flush())) return rc;
    }
    AdamSeg& D = A.s[A.nseg++];
    D.p = reinterpret_cast<float*>(S.param);
    D.g = reinterpret_cast<const float*>(S.grad);
    D.m = reinterpret_cast<float*>(S.exp_avg);
    D.v = reinterpret_cast<float*>(S.exp_avg_sq);
    D.n = S.n;
    D.block_begin = blocks;
    const double lr = S.lr, b1 = S.beta1, b2 = S.beta2, wd = S.weight_decay;
    const double t = (double)S.step;
    D.cd = (float)(1.0 - lr * wd);
    D.b1 = (float)b1;
    D.b2 = (float)b2;
    D.c1 = (float)(1.0 - b1);
    D.c2 = (float)(1.0 - b2);
    D.ss = (float)(lr / (1.0 - std::pow(b1, t)));
    D.s2 = (float)std::sqrt(1.0 - std::pow(b2, t));
    D.eps = S.eps;
    D.decay = S.weight_decay != 0.0f ? 1 : 0;
    D.vec = aligned16(S.param) && aligned16(S.grad) && aligned16(S.exp_avg) && aligned16(S.exp_avg_sq);
    blocks += nb;
  }
  return flush();
}

int adamw_impl(const ma_adamw_segment* segs, int32_t n, int32_t lean_blocks, void* stream) {
  const int rc = adamw_validate(segs, n);
  return rc ? rc : adamw_enqueue(segs, n, lean_blocks, stream);
}

// Two events per device and host thread for the fork and join of
// ma_muon_adamw_step (created once, never destroyed, so that a step being
// captured into a graph never sees one destroyed).
int fork_events(hipEvent_t& e_fork, hipEvent_t& e_join) {
  thread_local std::map<int, std::pair<hipEvent_t, hipEvent_t>> ev;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  auto it = ev.find(dev);
  if (it == ev.end()) {
    hipEvent_t a = nullptr, b = nullptr;
    if ((err = hipEventCreateWithFlags(&a, hipEventDisableTiming)) != hipSuccess) return hip_fail(err, "event");
    if ((err = hipEventCreateWithFlags(&b, hipEventDisableTiming)) != hipSuccess) return hip_fail(err, "event");
    it = ev.emplace(dev, std::make_pair(a, b)).first;
  }
  e_fork = it->second.first;
  e_join = it->second.second;
  return MA_OK;
}

// Test hook (ma_test_fail_after_fork): the calling thread's next
// ma_muon_adamw_step fails right after its fork, as a launch error there would.
thread_local bool g_fail_after_fork = false;
}  // namespace

int ma_muon_adamw_step(const ma_muon_group* groups, int32_t n_groups, const ma_muon_hparams* hp,
                       void* workspace, size_t workspace_bytes, const ma_adamw_segment* segs, int32_t n_segs,
                       int32_t workgroups, void* stream, void* side_stream) {
  EntryMark mark("ma_muon_adamw_step");
  if (workgroups < 1) return fail(MA_ERR_INVALID_ARG, "workgroups must be >= 1");
  if (side_stream == stream) return fail(MA_ERR_INVALID_ARG, "side_stream must differ from stream");
  // every argument of both steps, and one overlap check over the buffers of
  // both (they run concurrently), before anything is enqueued
  Plan plan;
  std::vector<Range> rs;
  int rc = muon_prepare(groups, n_groups, hp, workspace, workspace_bytes, nullptr, plan, rs);
  if (rc) return rc;
  if ((rc = adamw_prepare(segs, n_segs, rs))) return rc;
  if ((rc = check_overlaps(rs))) return rc;
  if ((rc = check_stream_device(stream, "stream")) || (rc = check_stream_device(side_stream, "side_stream")))
    return rc;
  const bool inject = g_fail_after_fork;
  g_fail_after_fork = false;
  hipEvent_t e_fork = nullptr, e_join = nullptr;
  if ((rc = fork_events(e_fork, e_join))) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream), side = reinterpret_cast<hipStream_t>(side_stream);
  // AdamW joins once the Muon step's elementwise passes and first GRAM and
  // POLY are done: it then runs beside the AXPY and later products
  bool side_waits = false;   // the side stream has work ordered after the fork
  std::function<int()> fork = [&]() -> int {
    hipError_t err;
    if ((err = hipEventRecord(e_fork, s)) != hipSuccess) return hip_fail(err, "fork record");
    if ((err = hipStreamWaitEvent(side, e_fork, 0)) != hipSuccess) return hip_fail(err, "fork wait");
    side_waits = true;
    EntryMark side_mark("adamw on the side stream");
    const int r = adamw_enqueue(segs, n_segs, workgroups, side_stream);
    if (r == MA_OK && inject) return fail(MA_ERR_HIP, "failure injected after the fork (test hook)");
    return r;
  };
  rc = muon_enqueue(plan, hp, workspace, nullptr, stream, &fork);
  if (side_waits) {
    // the join, on every path once the side stream waits on the fork: the
    // caller's stream must not run ahead of AdamW work already queued, and a
    // graph capture must not end with the side stream unjoined
    hipError_t err = hipEventRecord(e_join, side);
    if (err == hipSuccess) err = hipStreamWaitEvent(s, e_join, 0);
    if (err != hipSuccess && rc == MA_OK) rc = hip_fail(err, "join");
  }
  return rc;
}

int ma_test_fail_after_fork(void) {
  g_fail_after_fork = true;
  return MA_OK;
}

int ma_adamw_step(const ma_adamw_segment* segs, int32_t n, void* stream) {
  EntryMark mark("ma_adamw_step");
  return adamw_impl(segs, n, 0, stream);
}

int ma_adamw_step_background(const ma_adamw_segment* segs, int32_t n, int32_t workgroups, void* stream) {
  EntryMark mark("ma_adamw_step_background");
  if (workgroups < 1) return fail(MA_ERR_INVALID_ARG, "workgroups must be >= 1");
  return adamw_impl(segs, n, workgroups, stream);
}

int ma_lion_step(const ma_lion_segment* segs, int32_t n, void* stream) {
  EntryMark mark("ma_lion_step");
  if (n < 0 || (n > 0 && !segs)) return fail(MA_ERR_INVALID_ARG, "segments is null or n < 0");
  std::vector<Range> rs;
  for (int i = 0; i < n; ++i) {
    const ma_lion_segment& S = segs[i];
    if (S.n < 0 || S.n > kMaxSegmentElems) return fail(MA_ERR_INVALID_ARG, "segment %d: n < 0 or n > 2^40", i);
    if (S.param_dtype != MA_F32 || S.grad_dtype != MA_F32)
      return fail(MA_ERR_UNSUPPORTED, "segment %d: Lion buffers must be MA_F32", i);
    if (S.n == 0) continue;
    if (!S.param || !S.grad || !S.exp_avg) return fail(MA_ERR_INVALID_ARG, "segment %d: null device pointer", i);
    if (((uintptr_t)S.param | (uintptr_t)S.grad | (uintptr_t)S.exp_avg) & 3)
      return fail(MA_ERR_INVALID_ARG, "segment %d: pointer not 4-byte aligned", i);
    if (!std::isfinite(S.lr) || !std::isfinite(S.weight_decay) || !(S.beta1 >= 0.f && S.beta1 < 1.f) ||
        !(S.beta2 >= 0.f && S.beta2 < 1.f))
      return fail(MA_ERR_INVALID_ARG, "segment %d: hyperparameters out of range", i);
    const uintptr_t nb = (uintptr_t)S.n * 4;
    rs.push_back({(uintptr_t)S.param, (uintptr_t)S.param + nb, R_LION});
    rs.push_back({(uintptr_t)S.grad, (uintptr_t)S.grad + nb, R_LION});
    rs.push_back({(uintptr_t)S.exp_avg, (uintptr_t)S.exp_avg + nb, R_LION});
  }
  int rc = check_overlaps(rs);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LionArgs A{};
  int64_t blocks = 0;
  auto flush = [&]() -> int {
    if (A.nseg == 0) return MA_OK;
    A.total_blocks = (int32_t)blocks;
    hipError_t err;
    {
      ProfScope ps(MA_K_LION, s);
      err = launch_lion(A, s);
    }
    A = LionArgs{};
    blocks = 0;
    return err == hipSuccess ? MA_OK : hip_fail(err, "Lion launch");
  };
  for (int i = 0; i < n; ++i) {
    const ma_lion_segment& S = segs[i];
    if (S.n == 0) continue;
    const int64_t nb = (S.n + kLionBlockElems - 1) / kLionBlockElems;
    if (A.nseg == kMaxLionSegs || blocks + nb > (int64_t)0x7fffffff) {
      if ((rc = flush())) return rc;
    }
    LionSeg& D = A.s[A.nseg++];
    D.p = reinterpret_cast<float*>(S.param);
    D.g = reinterpret_cast<const float*>(S.grad);
    D.m = reinterpret_cast<float*>(S.exp_avg);
    D.n = S.n;
    D.block_begin = blocks;
    const double lr = S.lr, b1 = S.beta1, b2 = S.beta2, wd = S.weight_decay;
    D.lr = S.lr;
    D.cd = (float)(1.0 - lr * wd);
    D.b1 = S.beta1;
    D.b2 = S.beta2;
    D.c1 = (float)(1.0 - b1);
    D.c2 = (float)(1.0 - b2);
    D.decay = S.weight_decay != 0.0f ? 1 : 0;
    D.vec = aligned16(S.param) && aligned16(S.grad) && aligned16(S.exp_avg);
    blocks += nb;
  }
  return flush();
}

// ---------------------------------------------------------------------------
// calibration
// ---------------------------------------------------------------------------
int ma_calib_mfma(int32_t blocks, int32_t iters, int32_t changing, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !sink || ((uintptr_t)sink & 3) || (changing != 0 && changing != 1))
    return fail(MA_ERR_INVALID_ARG, "blocks and iters must be > 0, changing 0 or 1 and sink a 4-byte aligned pointer");
  hipError_t err = launch_calib_mfma(blocks, iters, changing, sink, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MA_OK : hip_fail(err, "calibration launch");
}

// ---------------------------------------------------------------------------
// stage entry points
// ---------------------------------------------------------------------------
int ma_test_bf16_round(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!in || !out))) return fail(MA_ERR_INVALID_ARG, "null buffer or n < 0");
  hipError_t err = launch_bf16_round(in, out, n, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? MA_OK : hip_fail(err, "bf16 round launch");
}

int ma_test_muon_momentum(const ma_muon_group* group, float beta, int32_t nesterov, float* mt_out,
                          void* stream) {
  if (!group || !mt_out) return fail(MA_ERR_INVALID_ARG, "null argument");
  int rc = validate_group(*group, 0, true);
  if (rc) return rc;
  if (!std::isfinite(beta)) return fail(MA_ERR_INVALID_ARG, "beta is not finite");
  const ma_muon_group& g = *group;
  for (int first = 0; first < g.count; first += kMaxMatsPerLaunch) {
    const int cnt = std::min(kMaxMatsPerLaunch, g.count - first);
    ElemArgs a{};
    a.R = (int32_t)g.rows;
    a.C = (int32_t)g.cols;
    a.count = cnt;
    a.r_ext = a.R;
    a.c_ext = a.C;
    a.tiles_r = (int32_t)((g.rows + 63) / 64);
    a.tiles_c = (int32_t)((g.cols + 63) / 64);
    a.x_stride = g.rows * g.cols;
    a.xd = mt_out + (size_t)first * a.x_stride;
    a.ld_d = g.cols;
    a.beta = beta;
    a.nesterov = nesterov ? 1 : 0;
    bool vec = (g.cols % 8) == 0 && aligned16(a.xd);
    for (int i = 0; i < cnt; ++i) {
      a.mat[i].g = g.grads[first + i];
      a.mat[i].m = g.momentum[first + i];
      vec = vec && aligned16(a.mat[i].g) && aligned16(a.mat[i].m);
    }
    a.vec = vec;
    hipError_t err = launch_pre(g.grad_dtype, g.mom_dtype, DT_F32, a, reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "momentum stage launch");
  }
  return MA_OK;
}

int ma_test_muon_update(const ma_muon_group* group, const void* u, int32_t u_dtype, float c_lr, float c_wd,
                        int32_t cautious, int32_t decay, void* stream) {
  if (!group || !u) return fail(MA_ERR_INVALID_ARG, "null argument");
  int rc = validate_group(*group, 0, true);
  if (rc) return rc;
  if (!dt_valid(u_dtype)) return fail(MA_ERR_UNSUPPORTED, "u_dtype %d", u_dtype);
  const ma_muon_group& g = *group;
  const int64_t ue = dt_bytes(u_dtype);
  for (int first = 0; first < g.count; first += kMaxMatsPerLaunch) {
    const int cnt = std::min(kMaxMatsPerLaunch, g.count - first);
    ElemArgs a{};
    a.R = (int32_t)g.rows;
    a.C = (int32_t)g.cols;
    a.count = cnt;
    a.tiles_r = (int32_t)((g.rows + 63) / 64);
    a.tiles_c = (int32_t)((g.cols + 63) / 64);
    a.x_stride = g.rows * g.cols;
    a.xd = (void*)((const unsigned char*)u + (size_t)(first * a.x_stride * ue));
    a.ld_d = g.cols;
    a.c_lr = c_lr;
    a.c_wd = c_wd;
    a.cautious = cautious ? 1 : 0;
    a.decay = decay ? 1 : 0;
    bool vec = (g.cols % 8) == 0 && aligned16(a.xd);
    for (int i = 0; i < cnt; ++i) {
      a.mat[i].w = g.params[first + i];
      vec = vec && aligned16(a.mat[i].w);
    }
    a.vec = vec;
    hipError_t err = launch_post(g.param_dtype, u_dtype, a, reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "update stage launch");
  }
  return MA_OK;
}

size_t ma_test_ns_workspace_size(int64_t m, int64_t n, int32_t count, int32_t precision) {
  if (m <= 0 || n < m || count < 0 || !dt_valid(precision)) {
    fail(MA_ERR_INVALID_ARG, "need 0 < m <= n, count >= 0, valid precision");
    return 0;
  }
  GroupPlan p{};
  size_t off = 0;
  plan_group(p, m, n, count, precision, off);
  return off;
}

int ma_test_ns(int64_t m, int64_t n, int32_t count, int32_t precision, const void* x0, void* u,
               const float* abc, int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream) {
  if (m <= 0 || n < m || count < 0 || !dt_valid(precision))
    return fail(MA_ERR_INVALID_ARG, "need 0 < m <= n, count >= 0, valid precision");
  if (m * n > (int64_t)1 << 31) return fail(MA_ERR_INVALID_ARG, "matrix too large");
  if (count > 0 && (!x0 || !u)) return fail(MA_ERR_INVALID_ARG, "null buffer");
  if (ns_steps < 0 || ns_steps > MA_MAX_NS_STEPS || (ns_steps > 0 && !abc))
    return fail(MA_ERR_INVALID_ARG, "bad ns_steps or abc");
  Plan plan;
  plan.g.resize(1);
  GroupPlan& p = plan.g[0];
  size_t off = 0;
  plan_group(p, m, n, count, precision, off);
  plan.bytes = off;
  p.dt_p = p.dt_g = p.dt_m = precision;
  p.src = nullptr;
  if (!workspace || workspace_bytes < off || (uintptr_t)workspace % MA_WORKSPACE_ALIGN)
    return fail(MA_ERR_WORKSPACE, "workspace null, misaligned or smaller than %zu bytes", off);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const int64_t e = dt_bytes(precision);
  hipError_t err;
  // pack x0 into the padded X / X^T buffers
  for (int first = 0; first < count; first += kMaxMatsPerLaunch) {
    const int cnt = std::min(kMaxMatsPerLaunch, count - first);
    ElemArgs a{};
    a.R = (int32_t)m;
    a.C = (int32_t)n;
    a.count = cnt;
    a.r_ext = (int32_t)p.r_ext;
    a.c_ext = (int32_t)p.c_ext;
    a.tiles_r = (int32_t)(p.r_ext / 64);
    a.tiles_c = (int32_t)(p.c_ext / 64);
    a.x_stride = p.x_stride;
    a.xd = ws + p.off_x[0] + (size_t)(first * p.x_stride * e);
    // m <= n: X^T is read only by the iteration without transposed AXPY reads
    a.xt = ns_q_transposed(precision) ? nullptr : ws + p.off_xt[0] + (size_t)(first * p.x_stride * e);
    a.ld_d = p.n_pad;
    a.ld_t = p.m_pad;
    a.pure_copy = 1;
    for (int i = 0; i < cnt; ++i) a.mat[i].g = (const unsigned char*)x0 + (size_t)((first + i) * m * n * e);
    if ((err = launch_pre(precision, precision, precision, a, s)) != hipSuccess) return hip_fail(err, "pack");
  }
  int rc = enqueue_ns(plan, ws, abc, ns_steps, precision, s);
  if (rc) return rc;
  const int ub = ns_steps & 1;
  for (int i = 0; i < count; ++i) {
    err = hipMemcpy2DAsync((unsigned char*)u + (size_t)(i * m * n * e), (size_t)(n * e),
                           ws + p.off_x[ub] + (size_t)(i * p.x_stride * e), (size_t)(p.n_pad * e),
                           (size_t)(n * e), (size_t)m, hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return hip_fail(err, "copy-out");
  }
  return MA_OK;
}

}  // extern "C"
