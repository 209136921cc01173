// libmuon C ABI: argument validation, workspace planning and the launch
// schedule of one Muon step (declared in include/muon.h).
//
// Schedule of one call, on the caller's stream, across all shape groups:
//   1. momentum pass per group (M in place, oriented iterate X0, partials)
//   2. small matrices: one on-chip Newton-Schulz launch per group
//   3. large bf16 matrices: per Newton-Schulz step one Gram launch and one
//      combine launch covering every such group (grouped, XCD-aware)
//   4. large fp32 matrices: Gram / combine launches per group and step
//   5. apply pass per group (W in place, optional copy of O).
// Nothing is allocated and nothing synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/muon.h"
#include "launch.h"

using namespace muon;

namespace {

constexpr int kMaxSteps = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int round_up(int x, int a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t dtype_size(int dt) { return dt == MUON_BF16 ? 2 : 4; }

struct NsCoefs {
  int steps;
  float a[kMaxSteps], b[kMaxSteps];
};

int parse_cfg(const muon_ns_cfg* cfg, NsCoefs* out) {
  if (cfg == nullptr) return MUON_EINVAL;
  if (cfg->steps < 0 || cfg->steps > kMaxSteps) return MUON_EINVAL;
  if (cfg->ncoef != 2 && cfg->ncoef != 3) return MUON_EINVAL;
  if (!(cfg->eps >= 0.0f) || !std::isfinite(cfg->eps)) return MUON_EINVAL;
  if (cfg->precision != MUON_F32 && cfg->precision != MUON_BF16) return MUON_EINVAL;
  if (cfg->steps > 0 && cfg->coeffs == nullptr) return MUON_EINVAL;
  out->steps = cfg->steps;
  for (int k = 0; k < cfg->steps; ++k) {
    const float* row = cfg->coeffs + (cfg->per_step ? k * cfg->ncoef : 0);
    if (!std::isfinite(row[0]) || !std::isfinite(row[1])) return MUON_EINVAL;
    if (cfg->ncoef == 3) {
      if (!std::isfinite(row[2])) return MUON_EINVAL;
      if (row[2] != 0.0f) return MUON_EUNSUPPORTED;
    }
    out->a[k] = row[0];
    out->b[k] = row[1];
  }
  return MUON_OK;
}

enum Engine { kSmall, kTiledBf16, kTiledF32 };

// Workspace plan of one shape group.
struct GroupPlan {
  int m = 0, n = 0, s = 0, l = 0, count = 0;
  bool tall = false, bf16 = false;
  Engine engine = kSmall;
  int s_pad = 0, ld = 0, kdim = 0, P = 0;
  size_t esz = 0;
  size_t off_x0 = 0, off_x1 = 0, off_a = 0, off_part = 0, end = 0;
};

int plan_group(int m, int n, int count, bool bf16, size_t base, GroupPlan* g) {
  if (m <= 0 || n <= 0 || count < 0) return MUON_EINVAL;
  if (static_cast<long long>(m) * n > (1LL << 31)) return MUON_EUNSUPPORTED;
  g->m = m;
  g->n = n;
  g->count = count;
  g->tall = m > n;
  g->s = g->tall ? n : m;
  g->l = g->tall ? m : n;
  g->bf16 = bf16;
  g->esz = bf16 ? 2 : 4;
  if (ns_small_supported(bf16, g->s, g->l)) {
    g->engine = kSmall;
    g->s_pad = g->s;
    g->ld = round_up(g->l, 8);
  } else if (bf16) {
    g->engine = kTiledBf16;
    g->s_pad = round_up(g->s, kTileS);
    g->ld = round_up(g->l, kTileL);
  } else {
    g->engine = kTiledF32;
    g->s_pad = round_up(g->s, kTileF32);
    g->ld = round_up(g->l, kTileF32);
  }
  g->kdim = std::min(g->ld, round_up(g->l, 64));
  g->P = momentum_blocks_per_matrix(g->tall, g->s_pad, g->ld);
  const size_t xbytes = static_cast<size_t>(count) * g->s_pad * g->ld * g->esz;
  size_t off = align_up(base, kAlign);
  g->off_x0 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_x1 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_a = off;
  if (g->engine != kSmall) off = align_up(off + static_cast<size_t>(count) * g->s_pad * g->s_pad * g->esz, kAlign);
  g->off_part = off;
  off = align_up(off + static_cast<size_t>(count) * g->P * sizeof(float), kAlign);
  g->end = off;
  return MUON_OK;
}

int validate_group(const muon_group& gr) {
  if (gr.m <= 0 || gr.n <= 0 || gr.count < 0) return MUON_EINVAL;
  if (gr.grad_dtype != MUON_F32 && gr.grad_dtype != MUON_BF16) return MUON_EINVAL;
  if (!std::isfinite(gr.lr) || !std::isfinite(gr.beta) || !std::isfinite(gr.scale)) return MUON_EINVAL;
  if (gr.count == 0) return MUON_OK;
  if (gr.W == nullptr || gr.M == nullptr || gr.G == nullptr) return MUON_EINVAL;
  for (int i = 0; i < gr.count; ++i) {
    if (gr.W[i] == nullptr || gr.M[i] == nullptr || gr.G[i] == nullptr) return MUON_EINVAL;
    if (!aligned_to(gr.W[i], 4) || !aligned_to(gr.M[i], 4) || !aligned_to(gr.G[i], dtype_size(gr.grad_dtype)))
      return MUON_EINVAL;
    if (gr.O != nullptr && gr.O[i] == nullptr) return MUON_EINVAL;
  }
  return MUON_OK;
}

// Everything the launch schedule needs for one group of matrices.
struct GroupRun {
  GroupPlan plan;
  int grad_dtype = MUON_BF16;
  const void* const* G = nullptr;
  float* const* M = nullptr;   // null: U = G
  float* const* W = nullptr;   // null: no apply
  void* const* O = nullptr;    // null: no copy-out
  std::vector<const void*> g_own;  // storage when pointers are derived from a base
  std::vector<void*> o_own;
  float beta = 0.0f, neg_lr_scale = 0.0f;
  int nesterov = 0;
};

// Optional phase markers: caller-created events recorded on the stream after
// launches of the schedule (profiling only; the arithmetic is unchanged).
struct EventRec {
  void* const* ev = nullptr;
  int n = 0, used = 0;
  bool mark(hipStream_t st) {
    if (ev == nullptr) return true;
    if (used >= n) return false;
    return hipEventRecord(static_cast<hipEvent_t>(ev[used++]), st) == hipSuccess;
  }
};

int events_needed(const std::vector<GroupRun>& runs, int steps) {
  int n = 1, tiled_bf16 = 0;
  for (const GroupRun& r : runs) {
    if (r.plan.count == 0) continue;
    n += 2;  // momentum, apply
    if (steps > 0 && r.plan.engine == kSmall) n += 1;
    if (steps > 0 && r.plan.engine == kTiledF32) n += 2 * steps;
    if (r.plan.engine == kTiledBf16) tiled_bf16 = 1;
  }
  if (steps > 0 && tiled_bf16) n += 2 * steps;
  return n;
}

char* x_of(const GroupPlan& p, char* ws, int which) { return ws + (which ? p.off_x1 : p.off_x0); }

int run_all(std::vector<GroupRun>& runs, const NsCoefs& C, float eps, char* ws, float* norms_out, hipStream_t st,
            EventRec& E) {
  if (!E.mark(st)) return MUON_EHIP;
  // 1. momentum
  int base = 0;
  for (GroupRun& R : runs) {
    const GroupPlan& p = R.plan;
    if (p.count == 0) continue;
    const long long xstride = static_cast<long long>(p.s_pad) * p.ld;
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    for (int c0 = 0; c0 < p.count; c0 += kMaxTable) {
      const int cn = std::min(kMaxTable, p.count - c0);
      MomentumLaunch L{};
      for (int i = 0; i < cn; ++i) {
        L.G.p[i] = R.G[c0 + i];
        L.M.p[i] = R.M ? R.M[c0 + i] : nullptr;
      }
      L.X = ws + p.off_x0 + static_cast<size_t>(c0) * xstride * p.esz;
      L.xstride = xstride;
      L.m = p.m; L.n = p.n; L.s_pad = p.s_pad; L.ld = p.ld; L.count = cn; L.P = p.P;
      L.tall = p.tall; L.grad_bf16 = R.grad_dtype == MUON_BF16; L.x_bf16 = p.bf16;
      L.beta = R.beta; L.nesterov = R.nesterov;
      L.partials = part + static_cast<size_t>(c0) * p.P;
      if (launch_momentum(L, st) != hipSuccess) return MUON_EHIP;
    }
    if (norms_out != nullptr && launch_norms(part, p.P, p.count, norms_out + base, st) != hipSuccess)
      return MUON_EHIP;
    base += p.count;
    if (!E.mark(st)) return MUON_EHIP;
  }

  // 2. small matrices on chip
  std::vector<int> fin(runs.size(), 0);  // which buffer holds the final iterate
  for (size_t gi = 0; gi < runs.size(); ++gi) {
    const GroupPlan& p = runs[gi].plan;
    if (p.count == 0 || p.engine != kSmall || C.steps == 0) continue;
    const long long xstride = static_cast<long long>(p.s_pad) * p.ld;
    NsSmallLaunch S{};
    S.X = ws + p.off_x0; S.Y = ws + p.off_x1;
    S.in_stride = xstride; S.out_stride = xstride;
    S.s = p.s; S.l = p.l; S.ld_in = p.ld; S.ld_out = p.ld;
    S.count = p.count; S.transposed = false; S.steps = C.steps;
    for (int k = 0; k < C.steps; ++k) { S.a[k] = C.a[k]; S.b[k] = C.b[k]; }
    S.partials = reinterpret_cast<const float*>(ws + p.off_part); S.P = p.P; S.eps = eps;
    if (launch_ns_small(S, p.bf16, st) != hipSuccess) return MUON_EHIP;
    fin[gi] = 1;
    if (!E.mark(st)) return MUON_EHIP;
  }

  // 3. large bf16 matrices, grouped launches
  std::vector<int> tb;
  for (size_t gi = 0; gi < runs.size(); ++gi)
    if (runs[gi].plan.count > 0 && runs[gi].plan.engine == kTiledBf16) tb.push_back(static_cast<int>(gi));
  if (!tb.empty() && C.steps > 0) {
    std::vector<int> by_k = tb, by_s = tb;  // heaviest tiles first
    std::stable_sort(by_k.begin(), by_k.end(), [&](int x, int y) { return runs[x].plan.kdim > runs[y].plan.kdim; });
    std::stable_sort(by_s.begin(), by_s.end(), [&](int x, int y) { return runs[x].plan.s_pad > runs[y].plan.s_pad; });
    for (int k = 0; k < C.steps; ++k) {
      for (int pass = 0; pass < 2; ++pass) {
        const std::vector<int>& order = pass == 0 ? by_k : by_s;
        for (size_t c0 = 0; c0 < order.size(); c0 += kMaxSeg) {
          GemmArgs G{};
          G.nseg = static_cast<int>(std::min<size_t>(kMaxSeg, order.size() - c0));
          for (int si = 0; si < G.nseg; ++si) {
            const GroupPlan& p = runs[order[c0 + si]].plan;
            GemmSeg& S = G.seg[si];
            const int cur = k & 1;
            S.X = reinterpret_cast<const bf16_t*>(x_of(p, ws, cur));
            S.Y = reinterpret_cast<bf16_t*>(x_of(p, ws, cur ^ 1));
            S.A = reinterpret_cast<bf16_t*>(ws + p.off_a);
            S.xstride = static_cast<long long>(p.s_pad) * p.ld;
            S.astride = static_cast<long long>(p.s_pad) * p.s_pad;
            S.s_pad = p.s_pad; S.ld = p.ld; S.kdim = p.kdim; S.count = p.count;
            S.tiles_per_mat = pass == 0 ? gram_tiles_per_matrix(p.s_pad) : combine_tiles_per_matrix(p.s_pad, p.ld);
            S.partials = k == 0 ? reinterpret_cast<const float*>(ws + p.off_part) : nullptr;
            S.P = p.P; S.eps = eps;
            S.a = C.a[k]; S.b = C.b[k];
          }
          const hipError_t e = pass == 0 ? launch_gram_bf16(G, st) : launch_combine_bf16(G, st);
          if (e != hipSuccess) return MUON_EHIP;
        }
        if (!E.mark(st)) return MUON_EHIP;
      }
    }
    for (int gi : tb) fin[gi] = C.steps & 1;
  }

  // 4. large fp32 matrices
  for (size_t gi = 0; gi < runs.size(); ++gi) {
    const GroupPlan& p = runs[gi].plan;
    if (p.count == 0 || p.engine != kTiledF32 || C.steps == 0) continue;
    for (int k = 0; k < C.steps; ++k) {
      NsGemmLaunch L{};
      const int cur = k & 1;
      L.X = x_of(p, ws, cur);
      L.Y = x_of(p, ws, cur ^ 1);
      L.A = ws + p.off_a;
      L.xstride = static_cast<long long>(p.s_pad) * p.ld;
      L.astride = static_cast<long long>(p.s_pad) * p.s_pad;
      L.s_pad = p.s_pad; L.ld = p.ld; L.count = p.count;
      L.partials = k == 0 ? reinterpret_cast<const float*>(ws + p.off_part) : nullptr;
      L.P = p.P; L.eps = eps;
      L.alpha = C.a[k]; L.beta = C.b[k];
      if (launch_gram_f32(L, st) != hipSuccess || !E.mark(st)) return MUON_EHIP;
      if (launch_combine_f32(L, st) != hipSuccess || !E.mark(st)) return MUON_EHIP;
    }
    fin[gi] = C.steps & 1;
  }

  // 5. apply
  for (size_t gi = 0; gi < runs.size(); ++gi) {
    const GroupRun& R = runs[gi];
    const GroupPlan& p = R.plan;
    if (p.count == 0) continue;
    if (R.W != nullptr || R.O != nullptr) {
      const long long xstride = static_cast<long long>(p.s_pad) * p.ld;
      for (int c0 = 0; c0 < p.count; c0 += kMaxTable) {
        const int cn = std::min(kMaxTable, p.count - c0);
        ApplyLaunch A{};
        for (int i = 0; i < cn; ++i) {
          A.W.p[i] = R.W ? R.W[c0 + i] : nullptr;
          A.O.p[i] = R.O ? R.O[c0 + i] : nullptr;
        }
        A.X = x_of(p, ws, fin[gi]) + static_cast<size_t>(c0) * xstride * p.esz;
        A.xstride = xstride;
        A.m = p.m; A.n = p.n; A.ld = p.ld; A.count = cn;
        A.tall = p.tall; A.x_bf16 = p.bf16;
        A.partials = C.steps == 0 ? reinterpret_cast<const float*>(ws + p.off_part) + static_cast<size_t>(c0) * p.P
                                  : nullptr;
        A.P = p.P; A.eps = eps;
        A.neg_lr_scale = R.neg_lr_scale;
        if (launch_apply(A, st) != hipSuccess) return MUON_EHIP;
      }
    }
    if (!E.mark(st)) return MUON_EHIP;
  }
  return MUON_OK;
}

int step_impl(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace, size_t workspace_bytes,
              float* norms_out, void* stream, void* const* events, int nevents) {
  if (groups == nullptr || ngroups <= 0) return MUON_EINVAL;
  NsCoefs C;
  int rc = parse_cfg(cfg, &C);
  if (rc != MUON_OK) return rc;
  if (norms_out != nullptr && !aligned_to(norms_out, 4)) return MUON_EINVAL;
  std::vector<GroupRun> runs(ngroups);
  size_t off = 0;
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& gr = groups[i];
    rc = validate_group(gr);
    if (rc != MUON_OK) return rc;
    if (gr.O != nullptr)
      for (int j = 0; j < gr.count; ++j)
        if (!aligned_to(gr.O[j], dtype_size(cfg->precision))) return MUON_EINVAL;
    rc = plan_group(gr.m, gr.n, gr.count, cfg->precision == MUON_BF16, off, &runs[i].plan);
    if (rc != MUON_OK) return rc;
    off = runs[i].plan.end;
    runs[i].grad_dtype = gr.grad_dtype;
    runs[i].G = gr.G;
    runs[i].M = gr.M;
    runs[i].W = gr.W;
    runs[i].O = gr.O;
    runs[i].beta = gr.beta;
    runs[i].neg_lr_scale = -gr.lr * gr.scale;
    runs[i].nesterov = gr.nesterov;
  }
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < off) return MUON_EWORKSPACE;
  EventRec E;
  if (events != nullptr) {
    const int need = events_needed(runs, C.steps);
    if (nevents < need) return MUON_EINVAL;
    for (int i = 0; i < need; ++i)
      if (events[i] == nullptr) return MUON_EINVAL;
    E.ev = events;
    E.n = nevents;
  }
  return run_all(runs, C, cfg->eps, static_cast<char*>(workspace), norms_out, static_cast<hipStream_t>(stream), E);
}

}  // namespace

extern "C" {

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_EINVAL: return "invalid argument";
    case MUON_EUNSUPPORTED: return "unsupported shape or precision";
    case MUON_EWORKSPACE: return "workspace missing or too small";
    case MUON_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int muon_version(void) { return MUON_VERSION; }

size_t muon_step_workspace_size(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg) {
  NsCoefs C;
  if (groups == nullptr || ngroups <= 0 || parse_cfg(cfg, &C) != MUON_OK) return 0;
  size_t off = 0;
  for (int i = 0; i < ngroups; ++i) {
    GroupPlan g;
    if (plan_group(groups[i].m, groups[i].n, groups[i].count, cfg->precision == MUON_BF16, off, &g) != MUON_OK)
      return 0;
    off = g.end;
  }
  return off == 0 ? kAlign : off;
}

int muon_step(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace,
              size_t workspace_bytes, float* norms_out, void* stream) {
  return step_impl(groups, ngroups, cfg, workspace, workspace_bytes, norms_out, stream, nullptr, 0);
}

int muon_step_timed(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace,
                    size_t workspace_bytes, float* norms_out, void* stream, void* const* events, int nevents) {
  if (events == nullptr) return MUON_EINVAL;
  return step_impl(groups, ngroups, cfg, workspace, workspace_bytes, norms_out, stream, events, nevents);
}

size_t muon_ns_workspace_size(int m, int n, int batch, int dtype, const muon_ns_cfg* cfg) {
  NsCoefs C;
  if (parse_cfg(cfg, &C) != MUON_OK || (dtype != MUON_F32 && dtype != MUON_BF16)) return 0;
  GroupPlan g;
  if (plan_group(m, n, batch, dtype == MUON_BF16, 0, &g) != MUON_OK) return 0;
  return g.end == 0 ? kAlign : g.end;
}

int muon_ns_orthogonalize(const void* G, void* O, int dtype, int m, int n, int batch, const muon_ns_cfg* cfg,
                          void* workspace, size_t workspace_bytes, void* stream) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C);
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (cfg->precision != dtype) return MUON_EUNSUPPORTED;
  if (m <= 0 || n <= 0 || batch < 0) return MUON_EINVAL;
  if (batch == 0) return MUON_OK;
  if (G == nullptr || O == nullptr || !aligned_to(G, dtype_size(dtype)) || !aligned_to(O, dtype_size(dtype)))
    return MUON_EINVAL;
  std::vector<GroupRun> runs(1);
  GroupRun& R = runs[0];
  rc = plan_group(m, n, batch, dtype == MUON_BF16, 0, &R.plan);
  if (rc != MUON_OK) return rc;
  const size_t mat = static_cast<size_t>(m) * n * dtype_size(dtype);
  const char* gb = static_cast<const char*>(G);
  char* ob = static_cast<char*>(O);
  if (ob < gb + mat * batch && gb < ob + mat * batch) return MUON_EINVAL;  // overlap
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < R.plan.end) return MUON_EWORKSPACE;
  R.g_own.resize(batch);
  R.o_own.resize(batch);
  for (int b = 0; b < batch; ++b) {
    R.g_own[b] = gb + mat * b;
    R.o_own[b] = ob + mat * b;
  }
  R.grad_dtype = dtype;
  R.G = R.g_own.data();
  R.O = R.o_own.data();
  EventRec E;
  return run_all(runs, C, cfg->eps, static_cast<char*>(workspace), nullptr, static_cast<hipStream_t>(stream), E);
}

int muon_ns_batched_small(const void* X, void* Y, int dtype, int m, int n, long long batch, const muon_ns_cfg* cfg,
                          void* stream) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C);
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (cfg->precision != dtype) return MUON_EUNSUPPORTED;
  if (m <= 0 || n <= 0 || batch < 0) return MUON_EINVAL;
  const bool bf16 = dtype == MUON_BF16;
  const bool tall = m > n;
  const int s = tall ? n : m, l = tall ? m : n;
  if (bf16 && tall) return MUON_EUNSUPPORTED;
  if (!ns_small_supported(bf16, s, l)) return MUON_EUNSUPPORTED;
  if (batch == 0) return MUON_OK;
  // the bf16 kernel moves 16-byte chunks (every matrix is a multiple of 2 KB)
  if (X == nullptr || Y == nullptr || !aligned_to(X, bf16 ? 16 : 4) || !aligned_to(Y, bf16 ? 16 : 4))
    return MUON_EINVAL;
  const size_t bytes = static_cast<size_t>(m) * n * dtype_size(dtype) * static_cast<size_t>(batch);
  const char* xb = static_cast<const char*>(X);
  const char* yb = static_cast<const char*>(Y);
  if (yb < xb + bytes && xb < yb + bytes) return MUON_EINVAL;  // overlap
  NsSmallLaunch S{};
  S.X = X; S.Y = Y;
  S.in_stride = static_cast<long long>(m) * n;
  S.out_stride = S.in_stride;
  S.s = s; S.l = l;
  S.ld_in = n;  // row stride of the stored m x n matrix
  S.ld_out = n;
  S.count = batch;
  S.transposed = tall;
  S.steps = C.steps;
  for (int k = 0; k < C.steps; ++k) { S.a[k] = C.a[k]; S.b[k] = C.b[k]; }
  S.partials = nullptr;
  S.P = 0;
  S.eps = cfg->eps;
  return launch_ns_small(S, bf16, static_cast<hipStream_t>(stream)) == hipSuccess ? MUON_OK : MUON_EHIP;
}

}  // extern "C"
