// Host side of the C ABI declared in include/muon.h: plans, validation, workspace layout
// and the order of launches of one Muon step.
//
// The step's three phases (momentum, Newton-Schulz orthogonalisation, parameter update)
// follow page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术", section
// "Muon优化器：动量正交化技术"; the grouping of matrices by size into batches follows the
// same page's section "训练优化技巧" / "分布式训练优化" (processing grouped by parameter
// size). Here a group is every matrix with the same padded wide shape, so each product of
// a Newton-Schulz round is one batched launch per group.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

using namespace muon;

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace muon {

thread_local LaunchTiming g_launch_timing;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int check_overlaps(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  uintptr_t max_any = 0, max_w = 0;
  for (const Range& r : rs) {
    if (r.lo < max_w || (r.writable && r.lo < max_any))
      return fail(MUON_ERR_INVALID_ARG,
                  "buffer [%p, %p) overlaps another buffer of the call, and one of them is "
                  "written", (void*)r.lo, (void*)r.hi);
    max_any = std::max(max_any, r.hi);
    if (r.writable) max_w = std::max(max_w, r.hi);
  }
  return MUON_OK;
}

}  // namespace muon

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int pad_up(int64_t x) { return (int)((x + kPad - 1) / kPad * kPad); }
size_t dt_size(muon_dtype d) { return d == MUON_DT_BF16 ? 2 : 4; }

struct LaunchSet {  // matrices of one shape and dtype pair, contiguous slots of a group
  int group = 0, slot0 = 0;
  int rows = 0, cols = 0;
  muon_dtype pdt = MUON_DT_BF16, gdt = MUON_DT_BF16;
  std::vector<int> mats;  // matrix indices, in slot order
};

struct Group {
  int mp = 0, np = 0, count = 0, tiles64 = 0;
  size_t off_x0 = 0, off_x1 = 0, off_a = 0, off_b = 0, off_part = 0, off_scales = 0;
  size_t off_rowsum = 0, off_rowf = 0;  // row equaliser: count x 8 x np and count x np floats
  std::vector<int> sets;
};

}  // namespace

struct muon_plan {
  int64_t n = 0;
  muon_precision prec = MUON_NS_BF16;
  std::vector<int64_t> rows, cols;
  std::vector<muon_dtype> pdt, gdt;
  std::vector<Group> groups;
  std::vector<LaunchSet> sets;
  size_t ws_bytes = 0;
  size_t off_sync = 0;   // the fused rounds' counters (kFusedSyncRounds rounds)
  bool fused = true;     // muon_plan_set_fused
  int fused_max_polls = 1 << 22;  // MUON_FUSED_MAX_POLLS when the plan was made
  // last argument set that passed the overlap check
  std::vector<muon_matrix> checked_mats;
  std::vector<const void*> checked_ptrs;
  const void* checked_ws = nullptr;
  bool checked_roweq = false;
  // profiling
  bool prof = false;
  std::vector<hipEvent_t> ev;  // pairs (start, stop)
  std::vector<int> ev_kind;    // kind of each recorded pair of the pending call
  int ev_used = 0;             // pairs recorded by the pending call
  double prof_ms[MUON_KERNEL_KINDS] = {};
  int64_t prof_launches[MUON_KERNEL_KINDS] = {};
  // concurrent shape groups (muon_plan_set_concurrency): side streams at the default
  // priority and their fork/join events, made on device `dev`
  int dev = -1;
  std::vector<hipStream_t> side;
  hipEvent_t fork = nullptr;
  std::vector<hipEvent_t> join;
};

namespace {

bool finite(float x) { return std::isfinite(x); }

int check_cfg(const muon_config* cfg, bool momentum) {
  if (!cfg) return fail(MUON_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->ns_steps < 0 || cfg->ns_steps > 64)
    return fail(MUON_ERR_INVALID_ARG, "ns_steps = %d outside [0, 64]", cfg->ns_steps);
  if (!finite(cfg->a) || !finite(cfg->b) || !finite(cfg->c))
    return fail(MUON_ERR_INVALID_ARG, "coefficients (a, b, c) must be finite");
  if (!finite(cfg->eps) || cfg->eps < 0.f)
    return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (momentum && (!finite(cfg->lr) || !finite(cfg->beta)))
    return fail(MUON_ERR_INVALID_ARG, "lr and beta must be finite");
  if (cfg->schedule)
    for (int k = 0; k < 3 * cfg->ns_steps; ++k)
      if (!finite(cfg->schedule[k]))
        return fail(MUON_ERR_INVALID_ARG, "schedule entry %d is not finite", k);
  if (momentum && cfg->row_equalize) {
    if (cfg->row_equalize != 1)
      return fail(MUON_ERR_INVALID_ARG, "row_equalize = %d (0 or 1)", cfg->row_equalize);
    if (!(cfg->row_beta >= 0.f && cfg->row_beta < 1.f))
      return fail(MUON_ERR_INVALID_ARG, "row_beta must lie in [0, 1)");
    if (!finite(cfg->row_eps) || cfg->row_eps < 0.f)
      return fail(MUON_ERR_INVALID_ARG, "row_eps must be finite and >= 0");
  }
  return MUON_OK;
}

int check_workspace(const muon_plan* p, const void* ws, size_t bytes) {
  if (p->ws_bytes == 0) return MUON_OK;
  if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", p->ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(MUON_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
  if (bytes < p->ws_bytes)
    return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, p->ws_bytes);
  return MUON_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ---- profiling -------------------------------------------------------------------------

void prof_collect(muon_plan* p) {
  if (!p->prof || p->ev_used == 0) return;
  (void)hipEventSynchronize(p->ev[2 * p->ev_used - 1]);
  for (int i = 0; i < p->ev_used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p->ev[2 * i], p->ev[2 * i + 1]) == hipSuccess) {
      p->prof_ms[p->ev_kind[i]] += ms;
      p->prof_launches[p->ev_kind[i]] += 1;
    }
  }
  p->ev_used = 0;
}

struct Launcher {
  muon_plan* p;
  hipStream_t s;
  int status = MUON_OK;

  template <class F>
  void run(int kind, const char* what, F&& f) {
    if (status != MUON_OK) return;
    const bool timed = p->prof && p->ev_used < (int)p->ev.size() / 2;
    if (timed) g_launch_timing = {p->ev[2 * p->ev_used], p->ev[2 * p->ev_used + 1]};
    const hipError_t e = f();
    g_launch_timing = {};
    if (e != hipSuccess) {
      status = fail(MUON_ERR_HIP, "launch of %s failed: %s", what, hipGetErrorString(e));
      return;
    }
    if (timed) {
      p->ev_kind[p->ev_used] = kind;
      ++p->ev_used;
    }
  }
};

// ---- the step ----------------------------------------------------------------------------

// Whether a step runs each phase over all shape groups together (one launch per product for
// every group) instead of group by group. Group by group, consecutive launches of one group
// find their operands (X, A, B', at most ~60 MB for a group of GPT-2 matrices) still in the
// MI355X's 256 MB Infinity Cache, and running each phase over all groups was measured 3-6%
// slower per kernel on the GPT-2-124M set (1296 apply tiles). A set too small to fill the
// device group by group (one GPU's share of a data-parallel step: 6 x 768x768 + 3 x
// 768x3072 leaves 54 and 108 apply tiles for 256 compute units) runs its groups side by side
// instead: fewer than kMergeTilesPerCu apply tiles of 256x256 per compute unit in all.
constexpr int kMergeTilesPerCu = 2;

bool merge_groups(const muon_plan* p) {
  if (p->prec == MUON_NS_F32_DEBUG || p->groups.size() < 2) return false;
  long long tiles = 0;
  for (const Group& G : p->groups)
    tiles += (long long)((G.mp + 255) / 256) * ((G.np + 255) / 256) * G.count;
  return tiles < (long long)kMergeTilesPerCu * device_cus();
}

// All rounds as one persistent launch (ns_fused_bf16.hip), unless disabled
// (muon_plan_set_fused): bf16 rounds, at most kFusedSyncRounds of them, at most 4 groups, each
// 256-aligned on both sides with at least 8 matrices (the launch deals a group's matrices to
// the 8 XCDs), on a whole device of 8 XCDs (256 compute units: every XCD's queue then has
// blocks to take its items), and sets of at most kFusedTilesPerCu apply tiles of 256x256 per
// compute unit per round: the GPT-2-124M set (5.1 per unit) measured 1-2% faster per step
// with the single launch, the tall stress set (13.5 per unit), whose launches are long
// enough to fill the device on their own, 4% slower.
constexpr int kFusedSyncRounds = 16;
constexpr int kFusedTilesPerCu = 8;

bool use_fused(const muon_plan* p, int rounds) {
  if (!p->fused || p->prec != MUON_NS_BF16 || rounds < 1 || rounds > kFusedSyncRounds ||
      p->groups.empty() || p->groups.size() > 4 || device_cus() != 256)
    return false;
  long long tiles = 0;
  for (const Group& G : p->groups) {
    if (G.mp % 256 != 0 || G.np % 256 != 0 || G.count < 8) return false;
    tiles += (long long)(G.mp / 256) * (G.np / 256) * G.count;
  }
  return tiles <= (long long)kFusedTilesPerCu * device_cus();
}

// Whether a step that may run its groups concurrently does: when their kernels are short
// enough that each launch's ramp, tail and write-out leave the device partly idle, which the
// other groups' kernels then fill. At most kConcurrentTilesPerCu apply tiles of 256x256 per
// compute unit in all: the GPT-2-124M set (5.1 per unit) measured 2-3% faster per step
// with its two groups side by side, the GPT-2-1.5B set (102 per unit), whose kernels run for
// milliseconds, 0.9% slower.
constexpr int kConcurrentTilesPerCu = 16;

bool concurrent_groups(const muon_plan* p) {
  long long tiles = 0;
  for (const Group& G : p->groups)
    tiles += (long long)((G.mp + 255) / 256) * ((G.np + 255) / 256) * G.count;
  return tiles <= (long long)kConcurrentTilesPerCu * device_cus();
}

// Side streams of a step that runs its shape groups concurrently (muon_plan_set_concurrency):
// none while profiling (each kernel is then timed alone), on another device than the one
// they were made on, or for sets whose groups run faster in sequence (concurrent_groups).
int side_streams(const muon_plan* p) {
  if (p->side.empty() || p->prof || !concurrent_groups(p)) return 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != p->dev) return 0;
  return (int)p->side.size();
}

void release_streams(muon_plan* p) {
  for (hipStream_t st : p->side) (void)hipStreamDestroy(st);
  for (hipEvent_t e : p->join) (void)hipEventDestroy(e);
  if (p->fork) (void)hipEventDestroy(p->fork);
  p->side.clear();
  p->join.clear();
  p->fork = nullptr;
  p->dev = -1;
}

// The step: momentum, norm, the Newton-Schulz rounds and the update of each shape group,
// either one group after the other or, for small sets (merge_groups), phase by phase over all
// groups.
// grads: per matrix input (grad or NS input); moms: momentum (nullable array = no momentum
// phase); params: W (nullable array = no update); outs: O destination (nullable entries);
// out_param_dtype: O is written in the param dtype (else fp32).
int enqueue(muon_plan* p, const void* const* grads, float* const* moms, void* const* params,
            void* const* outs, float* const* row_vars, bool out_param_dtype,
            const muon_config* cfg, void* ws, hipStream_t stream) {
  prof_collect(p);
  Launcher L{p, stream};
  const bool f32 = p->prec == MUON_NS_F32_DEBUG;
  const size_t esz = f32 ? 4 : 2;
  char* base = static_cast<char*>(ws);
  auto xslot = [&](const Group& G) { return (size_t)G.mp * G.np * esz; };
  auto scales_of = [&](const Group& G) { return reinterpret_cast<float*>(base + G.off_scales); };

  // phase 1: momentum, norm partials, X0; then the norms
  auto momentum_and_norm = [&](const Group& G, hipStream_t stream) {
    double* part = reinterpret_cast<double*>(base + G.off_part);
    for (int si : G.sets) {
      const LaunchSet& S = p->sets[si];
      for (size_t q0 = 0; q0 < S.mats.size(); q0 += kMaxPerLaunch) {
        ElemLaunch E{};
        E.count = (int)std::min<size_t>(kMaxPerLaunch, S.mats.size() - q0);
        for (int q = 0; q < E.count; ++q) {
          const int m = S.mats[q0 + q];
          E.in[q] = grads[m];
          E.mom[q] = moms ? moms[m] : nullptr;
        }
        E.rows = S.rows;
        E.cols = S.cols;
        E.tall = S.rows > S.cols;
        E.mp = G.mp;
        E.np = G.np;
        E.vec = (S.cols % 4) == 0;
        const int slot = S.slot0 + (int)q0;
        E.x = base + G.off_x0 + (size_t)slot * xslot(G);
        E.partials = part + (size_t)slot * G.tiles64;
        E.beta = cfg->beta;
        E.nesterov = cfg->nesterov ? 1 : 0;
        L.run(MUON_KERNEL_MOMENTUM, "momentum",
              [&] { return launch_momentum(E, S.gdt == MUON_DT_F32, f32, stream); });
      }
    }
    L.run(MUON_KERNEL_NORM, "norm", [&] {
      return launch_norm(part, G.tiles64, scales_of(G), G.count, cfg->eps, base + G.off_x0,
                         (size_t)G.mp * G.np, f32 ? 1 : 0, stream);
    });
  };

  // phase 2: Newton-Schulz rounds over the listed groups, ping-pong between x0 and x1; the
  // bf16 products take all of them in one launch each. Returns where each group's result is.
  auto rounds = [&](const std::vector<int>& gis, hipStream_t stream) {
    std::vector<NsGroup> N(gis.size());
    for (size_t k = 0; k < gis.size(); ++k) {
      const Group& G = p->groups[gis[k]];
      N[k] = NsGroup{};
      N[k].x_in = base + G.off_x0;
      N[k].x_out = base + G.off_x1;
      N[k].a = base + G.off_a;
      N[k].b = base + G.off_b;
      N[k].scales = scales_of(G);
      N[k].batch = G.count;
      N[k].mp = G.mp;
      N[k].np = G.np;
    }
    const int n = (int)N.size();
    for (int r = 0; r < cfg->ns_steps; ++r) {
      for (NsGroup& g : N) g.first = r == 0;
      const float* abc = cfg->schedule ? cfg->schedule + 3 * r : &cfg->a;
      const float ca = abc[0], cb = abc[1], cc = abc[2];
      if (f32) {
        for (NsGroup& g : N) {
          L.run(MUON_KERNEL_GRAM, "gram", [&] { return launch_gram_f32(g, stream); });
          L.run(MUON_KERNEL_POLY, "poly", [&] { return launch_poly_f32(g, cb, cc, stream); });
          L.run(MUON_KERNEL_APPLY, "apply", [&] { return launch_apply_f32(g, ca, stream); });
        }
      } else {
        L.run(MUON_KERNEL_GRAM, "gram", [&] { return launch_gram_bf16(N.data(), n, stream); });
        L.run(MUON_KERNEL_POLY, "poly",
              [&] { return launch_poly_bf16(N.data(), n, ca, cb, cc, stream); });
        L.run(MUON_KERNEL_APPLY, "apply", [&] { return launch_apply_bf16(N.data(), n, stream); });
      }
      for (NsGroup& g : N) std::swap(g.x_in, g.x_out);
    }
    std::vector<char*> res(gis.size());
    for (size_t k = 0; k < gis.size(); ++k) res[k] = static_cast<char*>(N[k].x_in);
    return res;
  };

  // the single launch's error word (set: its rounds failed, and the update writes NaN)
  const uint32_t* fault = nullptr;
  // phase 3: row equaliser (optional), parameter update (and O output) from X = xres
  auto finish = [&](const Group& G, char* xres, hipStream_t stream) {
    float* scales = scales_of(G);
    float* rowsum = reinterpret_cast<float*>(base + G.off_rowsum);
    float* rowf = reinterpret_cast<float*>(base + G.off_rowf);
    if (row_vars) {
      for (int si : G.sets) {
        const LaunchSet& S = p->sets[si];
        for (size_t q0 = 0; q0 < S.mats.size(); q0 += kMaxPerLaunch) {
          ElemLaunch E{};
          E.count = (int)std::min<size_t>(kMaxPerLaunch, S.mats.size() - q0);
          for (int q = 0; q < E.count; ++q) E.rowvar[q] = row_vars[S.mats[q0 + q]];
          E.rows = S.rows;
          E.cols = S.cols;
          E.tall = S.rows > S.cols;
          E.mp = G.mp;
          E.np = G.np;
          const int slot = S.slot0 + (int)q0;
          E.x = xres + (size_t)slot * xslot(G);
          E.scales = scales + 4 * (size_t)slot;
          E.apply_scale = cfg->ns_steps == 0;
          E.rowsum = rowsum + (size_t)slot * kRowParts * G.np;
          E.rowf = rowf + (size_t)slot * G.np;
          E.row_beta = cfg->row_beta;
          E.row_eps = cfg->row_eps;
          L.run(MUON_KERNEL_ROWEQ, "row sums", [&] { return launch_rowstat(E, f32, stream); });
          L.run(MUON_KERNEL_ROWEQ, "row factors",
                [&] { return launch_roweq_finish(E, stream); });
        }
      }
    }
    for (int si : G.sets) {
      const LaunchSet& S = p->sets[si];
      for (size_t q0 = 0; q0 < S.mats.size(); q0 += kMaxPerLaunch) {
        ElemLaunch E{};
        E.count = (int)std::min<size_t>(kMaxPerLaunch, S.mats.size() - q0);
        for (int q = 0; q < E.count; ++q) {
          const int m = S.mats[q0 + q];
          E.param[q] = params ? params[m] : nullptr;
          E.out[q] = outs ? outs[m] : nullptr;
        }
        E.rows = S.rows;
        E.cols = S.cols;
        E.tall = S.rows > S.cols;
        E.mp = G.mp;
        E.np = G.np;
        E.vec = (S.cols % 4) == 0;
        const int slot = S.slot0 + (int)q0;
        E.x = xres + (size_t)slot * xslot(G);
        E.scales = scales + 4 * (size_t)slot;
        E.apply_scale = cfg->ns_steps == 0;
        E.lr = cfg->lr;
        E.rowf = row_vars ? rowf + (size_t)slot * G.np : nullptr;
        E.fault = fault;
        const int out_dt = out_param_dtype ? (S.pdt == MUON_DT_F32) : 1;
        L.run(MUON_KERNEL_UPDATE, "update",
              [&] { return launch_update(E, S.pdt == MUON_DT_F32, out_dt, f32, stream); });
      }
    }
  };

  const int ng = (int)p->groups.size();
  if (use_fused(p, cfg->ns_steps)) {
    std::vector<NsGroup> N(ng);
    for (int gi = 0; gi < ng; ++gi) {
      const Group& G = p->groups[gi];
      momentum_and_norm(G, stream);
      N[gi] = NsGroup{};
      N[gi].x_in = base + G.off_x0;
      N[gi].x_out = base + G.off_x1;
      N[gi].a = base + G.off_a;
      N[gi].b = base + G.off_b;
      N[gi].scales = scales_of(G);
      N[gi].batch = G.count;
      N[gi].mp = G.mp;
      N[gi].np = G.np;
      N[gi].first = 1;
    }
    std::vector<float> abc(3 * cfg->ns_steps);
    for (int r = 0; r < cfg->ns_steps; ++r)
      for (int c = 0; c < 3; ++c) abc[3 * r + c] = cfg->schedule ? cfg->schedule[3 * r + c]
                                                                 : (&cfg->a)[c];
    uint32_t* sync = reinterpret_cast<uint32_t*>(base + p->off_sync);
    L.run(MUON_KERNEL_ROUNDS, "rounds", [&] {
      return launch_fused_bf16(N.data(), ng, cfg->ns_steps, abc.data(), sync,
                               p->fused_max_polls, stream);
    });
    fault = fused_error_word(sync);
    for (int gi = 0; gi < ng; ++gi) {
      const Group& G = p->groups[gi];
      finish(G, base + ((cfg->ns_steps & 1) ? G.off_x1 : G.off_x0), stream);
    }
  } else if (merge_groups(p)) {
    std::vector<int> all(ng);
    for (int gi = 0; gi < ng; ++gi) {
      all[gi] = gi;
      momentum_and_norm(p->groups[gi], stream);
    }
    const std::vector<char*> res = rounds(all, stream);
    for (int gi = 0; gi < ng; ++gi) finish(p->groups[gi], res[gi], stream);
  } else {
    const int nside = side_streams(p);
    if (nside > 0) {
      if (hipError_t e = hipEventRecord(p->fork, stream))
        return fail(MUON_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
      for (int k = 0; k < nside; ++k)
        if (hipError_t e = hipStreamWaitEvent(p->side[k], p->fork, 0))
          return fail(MUON_ERR_HIP, "hipStreamWaitEvent failed: %s", hipGetErrorString(e));
    }
    for (int gi = 0; gi < ng && L.status == MUON_OK; ++gi) {
      const hipStream_t st = (gi == 0 || nside == 0) ? stream : p->side[(gi - 1) % nside];
      momentum_and_norm(p->groups[gi], st);
      finish(p->groups[gi], rounds({gi}, st)[0], st);
    }
    for (int k = 0; k < nside; ++k) {
      if (hipError_t e = hipEventRecord(p->join[k], p->side[k]))
        return fail(MUON_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
      if (hipError_t e = hipStreamWaitEvent(stream, p->join[k], 0))
        return fail(MUON_ERR_HIP, "hipStreamWaitEvent failed: %s", hipGetErrorString(e));
    }
  }
  return L.status;
}

}  // namespace

extern "C" {

void muon_config_default(muon_config* cfg) {
  if (!cfg) return;
  cfg->lr = 0.02f;
  cfg->beta = 0.95f;
  cfg->nesterov = 1;
  cfg->ns_steps = 5;
  cfg->a = 3.4445f;
  cfg->b = -4.7750f;
  cfg->c = 2.0315f;
  cfg->eps = 1e-7f;
  cfg->schedule = nullptr;
  cfg->row_equalize = 0;
  cfg->row_beta = 0.95f;
  cfg->row_eps = 1e-8f;
}

int muon_plan_create(muon_plan** out, const int64_t* rows, const int64_t* cols,
                     const muon_dtype* param_dtype, const muon_dtype* grad_dtype, int64_t n,
                     muon_precision precision) {
  clear_error();
  if (!out) return fail(MUON_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n > 0 && (!rows || !cols || !param_dtype || !grad_dtype))
    return fail(MUON_ERR_INVALID_ARG, "rows, cols, param_dtype and grad_dtype must be non-NULL");
  if (precision != MUON_NS_BF16 && precision != MUON_NS_F32_DEBUG)
    return fail(MUON_ERR_INVALID_ARG, "unknown precision %d", (int)precision);
  for (int64_t i = 0; i < n; ++i) {
    if (rows[i] < 1 || cols[i] < 1)
      return fail(MUON_ERR_INVALID_ARG, "matrix %lld has shape %lld x %lld", (long long)i,
                  (long long)rows[i], (long long)cols[i]);
    if (rows[i] > 32768 || cols[i] > 32768 || rows[i] * cols[i] > (int64_t(1) << 28))
      return fail(MUON_ERR_UNSUPPORTED, "matrix %lld: %lld x %lld exceeds the limits",
                  (long long)i, (long long)rows[i], (long long)cols[i]);
    for (muon_dtype d : {param_dtype[i], grad_dtype[i]})
      if (d != MUON_DT_BF16 && d != MUON_DT_F32)
        return fail(MUON_ERR_INVALID_ARG, "matrix %lld: unknown dtype %d", (long long)i, (int)d);
  }

  muon_plan* p = new (std::nothrow) muon_plan();
  if (!p) return fail(MUON_ERR_INVALID_ARG, "out of host memory");
  p->n = n;
  p->prec = precision;
  p->rows.assign(rows, rows + n);
  p->cols.assign(cols, cols + n);
  p->pdt.assign(param_dtype, param_dtype + n);
  p->gdt.assign(grad_dtype, grad_dtype + n);

  // groups by padded wide shape, launch sets by (rows, cols, dtypes), in order of appearance
  for (int64_t i = 0; i < n; ++i) {
    const int64_t m = std::min(rows[i], cols[i]), w = std::max(rows[i], cols[i]);
    const int mp = pad_up(m), np = pad_up(w);
    int g = -1;
    for (size_t k = 0; k < p->groups.size(); ++k)
      if (p->groups[k].mp == mp && p->groups[k].np == np) g = (int)k;
    if (g < 0) {
      g = (int)p->groups.size();
      Group G;
      G.mp = mp;
      G.np = np;
      G.tiles64 = (mp / kTile) * (np / kTile);
      p->groups.push_back(G);
    }
    int s = -1;
    for (int k : p->groups[g].sets) {
      const LaunchSet& S = p->sets[k];
      if (S.rows == rows[i] && S.cols == cols[i] && S.pdt == param_dtype[i] &&
          S.gdt == grad_dtype[i])
        s = k;
    }
    if (s < 0) {
      s = (int)p->sets.size();
      LaunchSet S;
      S.group = g;
      S.rows = (int)rows[i];
      S.cols = (int)cols[i];
      S.pdt = param_dtype[i];
      S.gdt = grad_dtype[i];
      p->sets.push_back(S);
      p->groups[g].sets.push_back(s);
    }
    p->sets[s].mats.push_back((int)i);
  }

  const size_t esz = precision == MUON_NS_F32_DEBUG ? 4 : 2;
  size_t off = 0;
  for (Group& G : p->groups) {
    int slot = 0;
    for (int s : G.sets) {
      p->sets[s].slot0 = slot;
      slot += (int)p->sets[s].mats.size();
    }
    G.count = slot;
    const size_t xs = (size_t)G.count * G.mp * G.np * esz;
    const size_t as = (size_t)G.count * G.mp * G.mp * esz;
    G.off_x0 = off; off = align256(off + xs);
    G.off_x1 = off; off = align256(off + xs);
    G.off_a = off; off = align256(off + as);
    G.off_b = off; off = align256(off + as);
    G.off_part = off; off = align256(off + (size_t)G.count * G.tiles64 * 8);
    G.off_scales = off; off = align256(off + (size_t)G.count * 16);
    G.off_rowsum = off; off = align256(off + (size_t)G.count * kRowParts * G.np * 4);
    G.off_rowf = off; off = align256(off + (size_t)G.count * G.np * 4);
  }
  // the fused rounds' queues, flag and completion counters (ns_fused_bf16.hip), sized for
  // the largest round count it takes
  if (!p->groups.empty()) {
    size_t words = 8 * 16 + 16;
    for (const Group& G : p->groups) words += (size_t)3 * kFusedSyncRounds * G.count;
    p->off_sync = off;
    off = align256(off + 4 * words);
  }
  p->ws_bytes = off;
  // the single launch's wait limit (polls); a test sets it to 0 to exercise the failure path
  if (const char* e = std::getenv("MUON_FUSED_MAX_POLLS")) {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v >= 0 && v <= (1L << 30)) p->fused_max_polls = (int)v;
  }

  *out = p;
  return MUON_OK;
}

size_t muon_plan_workspace_size(const muon_plan* plan) { return plan ? plan->ws_bytes : 0; }

int muon_step(muon_plan* plan, const muon_matrix* mats, int64_t n, const muon_config* cfg,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (n != plan->n)
    return fail(MUON_ERR_INVALID_ARG, "n = %lld but the plan has %lld matrices", (long long)n,
                (long long)plan->n);
  if (int st = check_cfg(cfg, true)) return st;
  if (n == 0) return MUON_OK;
  if (!mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
  if (int st = check_workspace(plan, workspace, workspace_bytes)) return st;

  const bool roweq = cfg->row_equalize != 0;
  const bool same = plan->checked_ws == workspace && plan->checked_roweq == roweq &&
                    plan->checked_mats.size() == (size_t)n &&
                    std::memcmp(plan->checked_mats.data(), mats, sizeof(muon_matrix) * n) == 0;
  if (!same) {
    std::vector<Range> rs;
    rs.reserve(4 * n + 1);
    for (int64_t i = 0; i < n; ++i) {
      const muon_matrix& M = mats[i];
      if (M.rows != plan->rows[i] || M.cols != plan->cols[i] ||
          M.param_dtype != plan->pdt[i] || M.grad_dtype != plan->gdt[i])
        return fail(MUON_ERR_INVALID_ARG,
                    "matrix %lld: shape/dtype (%lld x %lld, %d, %d) differ from the plan's",
                    (long long)i, (long long)M.rows, (long long)M.cols, (int)M.param_dtype,
                    (int)M.grad_dtype);
      if (!M.param || !M.grad || !M.momentum)
        return fail(MUON_ERR_INVALID_ARG, "matrix %lld: param, grad and momentum must be non-NULL",
                    (long long)i);
      if (!aligned16(M.param) || !aligned16(M.grad) || !aligned16(M.momentum) ||
          (M.update_out && !aligned16(M.update_out)) || (roweq && !aligned16(M.row_var)))
        return fail(MUON_ERR_INVALID_ARG, "matrix %lld: buffers must be 16-byte aligned",
                    (long long)i);
      if (roweq && !M.row_var)
        return fail(MUON_ERR_INVALID_ARG,
                    "matrix %lld: row_var must be non-NULL when row_equalize is set",
                    (long long)i);
      const size_t elems = (size_t)M.rows * M.cols;
      auto add = [&](const void* ptr, size_t bytes, bool w) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
        rs.push_back({lo, lo + bytes, w});
      };
      add(M.param, elems * dt_size(M.param_dtype), true);
      add(M.grad, elems * dt_size(M.grad_dtype), false);
      add(M.momentum, elems * 4, true);
      if (M.update_out) add(M.update_out, elems * 4, true);
      if (roweq) add(M.row_var, (size_t)M.rows * 4, true);
    }
    if (plan->ws_bytes) rs.push_back({reinterpret_cast<uintptr_t>(workspace),
                                      reinterpret_cast<uintptr_t>(workspace) + plan->ws_bytes,
                                      true});
    if (int st = check_overlaps(rs)) return st;
    plan->checked_mats.assign(mats, mats + n);
    plan->checked_ws = workspace;
    plan->checked_roweq = roweq;
  }

  std::vector<const void*> grads(n);
  std::vector<float*> moms(n), row_vars(n);
  std::vector<void*> params(n), outs(n);
  for (int64_t i = 0; i < n; ++i) {
    grads[i] = mats[i].grad;
    moms[i] = mats[i].momentum;
    params[i] = mats[i].param;
    outs[i] = mats[i].update_out;
    row_vars[i] = mats[i].row_var;
  }
  return enqueue(plan, grads.data(), moms.data(), params.data(), outs.data(),
                 roweq ? row_vars.data() : nullptr, false, cfg, workspace, stream);
}

int muon_newton_schulz(muon_plan* plan, const void* const* in, void* const* out, int64_t n,
                       const muon_config* cfg, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (n != plan->n)
    return fail(MUON_ERR_INVALID_ARG, "n = %lld but the plan has %lld matrices", (long long)n,
                (long long)plan->n);
  if (int st = check_cfg(cfg, false)) return st;
  if (n == 0) return MUON_OK;
  if (!in || !out) return fail(MUON_ERR_INVALID_ARG, "in and out must be non-NULL");
  if (int st = check_workspace(plan, workspace, workspace_bytes)) return st;
  std::vector<Range> rs;
  for (int64_t i = 0; i < n; ++i) {
    if (!in[i] || !out[i])
      return fail(MUON_ERR_INVALID_ARG, "matrix %lld: in and out must be non-NULL", (long long)i);
    if (!aligned16(in[i]) || !aligned16(out[i]))
      return fail(MUON_ERR_INVALID_ARG, "matrix %lld: buffers must be 16-byte aligned",
                  (long long)i);
    const size_t elems = (size_t)plan->rows[i] * plan->cols[i];
    const uintptr_t a = reinterpret_cast<uintptr_t>(in[i]), b = reinterpret_cast<uintptr_t>(out[i]);
    rs.push_back({a, a + elems * dt_size(plan->gdt[i]), false});
    rs.push_back({b, b + elems * dt_size(plan->pdt[i]), true});
  }
  if (plan->ws_bytes)
    rs.push_back({reinterpret_cast<uintptr_t>(workspace),
                  reinterpret_cast<uintptr_t>(workspace) + plan->ws_bytes, true});
  if (int st = check_overlaps(rs)) return st;
  return enqueue(plan, in, nullptr, nullptr, out, nullptr, true, cfg, workspace, stream);
}

void muon_plan_destroy(muon_plan* plan) {
  if (!plan) return;
  if (plan->prof) {
    prof_collect(plan);
    for (hipEvent_t e : plan->ev) (void)hipEventDestroy(e);
  }
  release_streams(plan);
  delete plan;
}

int muon_plan_set_fused(muon_plan* plan, int enable) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (enable != 0 && enable != 1) return fail(MUON_ERR_INVALID_ARG, "enable = %d (0 or 1)", enable);
  plan->fused = enable == 1;
  return MUON_OK;
}

int muon_plan_set_concurrency(muon_plan* plan, int streams) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (streams < 1 || streams > MUON_MAX_STREAMS)
    return fail(MUON_ERR_INVALID_ARG, "streams = %d outside [1, %d]", streams, MUON_MAX_STREAMS);
  release_streams(plan);
  const int want = std::min<int>(streams, (int)plan->groups.size()) - 1;
  if (want <= 0) return MUON_OK;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&plan->fork, hipEventDisableTiming);
  for (int k = 0; k < want && e == hipSuccess; ++k) {
    hipStream_t st = nullptr;
    hipEvent_t ev = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) break;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipStreamDestroy(st);
      break;
    }
    plan->side.push_back(st);
    plan->join.push_back(ev);
  }
  if (e != hipSuccess) {
    release_streams(plan);
    return fail(MUON_ERR_HIP, "creating the plan's streams failed: %s", hipGetErrorString(e));
  }
  plan->dev = dev;
  return MUON_OK;
}

int muon_plan_set_profiling(muon_plan* plan, int enable) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (plan->prof) {
    prof_collect(plan);
    for (hipEvent_t e : plan->ev) (void)hipEventDestroy(e);
    plan->ev.clear();
    plan->ev_kind.clear();
    plan->prof = false;
  }
  std::fill(std::begin(plan->prof_ms), std::end(plan->prof_ms), 0.0);
  std::fill(std::begin(plan->prof_launches), std::end(plan->prof_launches), 0);
  if (!enable) return MUON_OK;
  // launches of one call with the largest ns_steps: per group 2 elementwise passes, the norm
  // and 3 products per round
  size_t pairs = 0;
  for (const Group& G : plan->groups) {
    size_t chunks = 0;
    for (int s : G.sets) chunks += (plan->sets[s].mats.size() + kMaxPerLaunch - 1) / kMaxPerLaunch;
    pairs += 2 * chunks + 1 + 3 * 64;
  }
  plan->ev.resize(2 * pairs);
  plan->ev_kind.assign(pairs, 0);
  for (size_t i = 0; i < plan->ev.size(); ++i) {
    const hipError_t e = hipEventCreate(&plan->ev[i]);
    if (e != hipSuccess) {
      for (size_t k = 0; k < i; ++k) (void)hipEventDestroy(plan->ev[k]);
      plan->ev.clear();
      return fail(MUON_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(e));
    }
  }
  plan->ev_used = 0;
  plan->prof = true;
  return MUON_OK;
}

int muon_plan_read_profile(muon_plan* plan, double* ms, int64_t* launches, int nkinds) {
  clear_error();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "plan is NULL");
  if (nkinds < 0 || (nkinds > 0 && (!ms || !launches)))
    return fail(MUON_ERR_INVALID_ARG, "ms and launches must hold nkinds entries");
  prof_collect(plan);
  for (int k = 0; k < nkinds && k < MUON_KERNEL_KINDS; ++k) {
    ms[k] = plan->prof_ms[k];
    launches[k] = plan->prof_launches[k];
  }
  for (int k = MUON_KERNEL_KINDS; k < nkinds; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  return MUON_OK;
}

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
    default: return "unknown muon status";
  }
}

const char* muon_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
