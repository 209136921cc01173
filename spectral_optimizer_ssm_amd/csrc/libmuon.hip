// libmuon C ABI: argument validation, workspace planning and the launch
// schedule of one Muon step (declared in include/muon.h).
//
// Per shape group, on the caller's stream:
//   momentum pass (M in place, oriented iterate X0, norm partials)
//   -> Newton-Schulz: on-chip kernel for small matrices, or
//      steps x (symmetric Gram, polynomial combine) on the matrix cores
//   -> apply pass (W in place, optional copy of O).
// Nothing is allocated and nothing synchronises.
#include <hip/hip_runtime.h>

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

// Workspace plan of one shape group.
struct GroupPlan {
  int m = 0, n = 0, s = 0, l = 0, count = 0;
  bool tall = false, bf16 = false, small = false;
  int s_pad = 0, ld = 0, P = 0;
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
  g->small = ns_small_supported(bf16, g->s, g->l);
  if (g->small) {
    g->s_pad = g->s;
    g->ld = round_up(g->l, 8);
  } else if (bf16) {
    g->s_pad = round_up(g->s, kTileS);
    g->ld = round_up(g->l, kTileL);
  } else {
    g->s_pad = round_up(g->s, kTileF32);
    g->ld = round_up(g->l, kTileF32);
  }
  g->P = momentum_blocks_per_matrix(g->tall, g->s_pad, g->ld);
  const size_t xbytes = static_cast<size_t>(count) * g->s_pad * g->ld * g->esz;
  size_t off = align_up(base, kAlign);
  g->off_x0 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_x1 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_a = off;
  if (!g->small) off = align_up(off + static_cast<size_t>(count) * g->s_pad * g->s_pad * g->esz, kAlign);
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
    if (!aligned16(gr.W[i]) || !aligned16(gr.M[i]) || !aligned16(gr.G[i])) return MUON_EINVAL;
    if (gr.O != nullptr && (gr.O[i] == nullptr || !aligned16(gr.O[i]))) return MUON_EINVAL;
  }
  return MUON_OK;
}

// Everything the launch schedule needs for one group of matrices.
struct GroupRun {
  GroupPlan plan;
  int grad_dtype;
  const void* const* G;
  float* const* M;   // null: U = G
  float* const* W;   // null: no apply
  void* const* O;    // null: no copy-out
  std::vector<const void*> g_own;  // storage when pointers are derived from a base
  std::vector<void*> o_own;
  float beta, neg_lr_scale;
  int nesterov;
};

// Optional phase markers: caller-created events recorded on the stream after
// each launch of the schedule (profiling only; the arithmetic is unchanged).
struct EventRec {
  void* const* ev = nullptr;
  int n = 0, used = 0;
  hipError_t mark(hipStream_t st) {
    if (ev == nullptr) return hipSuccess;
    if (used >= n) return hipErrorInvalidValue;
    return hipEventRecord(static_cast<hipEvent_t>(ev[used++]), st);
  }
};

int events_per_group(int steps, bool small) { return small ? 4 : 3 + 2 * steps; }

int run_group(const GroupRun& R, const NsCoefs& C, float eps, char* ws, float* norms_out, hipStream_t st,
              EventRec* evr = nullptr) {
  const GroupPlan& p = R.plan;
  EventRec none;
  EventRec& E = evr ? *evr : none;
  if (p.count == 0) return MUON_OK;
  if (E.mark(st) != hipSuccess) return MUON_EHIP;
  char* x0 = ws + p.off_x0;
  char* x1 = ws + p.off_x1;
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  const long long xstride = static_cast<long long>(p.s_pad) * p.ld;

  // momentum pass, up to kMaxTable matrices per launch
  for (int c0 = 0; c0 < p.count; c0 += kMaxTable) {
    const int cn = p.count - c0 < kMaxTable ? p.count - c0 : kMaxTable;
    MomentumLaunch L{};
    for (int i = 0; i < cn; ++i) {
      L.G.p[i] = R.G[c0 + i];
      L.M.p[i] = R.M ? R.M[c0 + i] : nullptr;
    }
    L.X = x0 + static_cast<size_t>(c0) * xstride * p.esz;
    L.xstride = xstride;
    L.m = p.m; L.n = p.n; L.s_pad = p.s_pad; L.ld = p.ld; L.count = cn; L.P = p.P;
    L.tall = p.tall; L.grad_bf16 = R.grad_dtype == MUON_BF16; L.x_bf16 = p.bf16;
    L.beta = R.beta; L.nesterov = R.nesterov;
    L.partials = part + static_cast<size_t>(c0) * p.P;
    if (launch_momentum(L, st) != hipSuccess) return MUON_EHIP;
  }
  if (norms_out != nullptr && launch_norms(part, p.P, p.count, norms_out, st) != hipSuccess) return MUON_EHIP;
  if (E.mark(st) != hipSuccess) return MUON_EHIP;

  // Newton-Schulz
  const char* xfin = x0;
  bool scale_in_apply = false;
  if (C.steps == 0) {
    scale_in_apply = true;
  } else if (p.small) {
    NsSmallLaunch S{};
    S.X = x0; S.Y = x1;
    S.in_stride = xstride; S.out_stride = xstride;
    S.s = p.s; S.l = p.l; S.ld_in = p.ld; S.ld_out = p.ld;
    S.count = p.count; S.transposed = false; S.steps = C.steps;
    for (int k = 0; k < C.steps; ++k) { S.a[k] = C.a[k]; S.b[k] = C.b[k]; }
    S.partials = part; S.P = p.P; S.eps = eps;
    if (launch_ns_small(S, p.bf16, st) != hipSuccess) return MUON_EHIP;
    if (E.mark(st) != hipSuccess) return MUON_EHIP;
    xfin = x1;
  } else {
    char* cur = x0;
    char* nxt = x1;
    for (int k = 0; k < C.steps; ++k) {
      NsGemmLaunch L{};
      L.X = cur; L.Y = nxt; L.A = ws + p.off_a;
      L.xstride = xstride;
      L.astride = static_cast<long long>(p.s_pad) * p.s_pad;
      L.s_pad = p.s_pad; L.ld = p.ld; L.count = p.count;
      L.partials = k == 0 ? part : nullptr;
      L.P = p.P; L.eps = eps;
      L.alpha = C.a[k]; L.beta = C.b[k];
      const hipError_t e1 = p.bf16 ? launch_gram_bf16(L, st) : launch_gram_f32(L, st);
      if (e1 != hipSuccess || E.mark(st) != hipSuccess) return MUON_EHIP;
      const hipError_t e2 = p.bf16 ? launch_combine_bf16(L, st) : launch_combine_f32(L, st);
      if (e2 != hipSuccess || E.mark(st) != hipSuccess) return MUON_EHIP;
      char* t = cur; cur = nxt; nxt = t;
    }
    xfin = cur;
  }

  // apply pass
  if (R.W == nullptr && R.O == nullptr) return E.mark(st) == hipSuccess ? MUON_OK : MUON_EHIP;
  for (int c0 = 0; c0 < p.count; c0 += kMaxTable) {
    const int cn = p.count - c0 < kMaxTable ? p.count - c0 : kMaxTable;
    ApplyLaunch A{};
    for (int i = 0; i < cn; ++i) {
      A.W.p[i] = R.W ? R.W[c0 + i] : nullptr;
      A.O.p[i] = R.O ? R.O[c0 + i] : nullptr;
    }
    A.X = xfin + static_cast<size_t>(c0) * xstride * p.esz;
    A.xstride = xstride;
    A.m = p.m; A.n = p.n; A.ld = p.ld; A.count = cn;
    A.tall = p.tall; A.x_bf16 = p.bf16;
    A.partials = scale_in_apply ? part + static_cast<size_t>(c0) * p.P : nullptr;
    A.P = p.P; A.eps = eps;
    A.neg_lr_scale = R.neg_lr_scale;
    if (launch_apply(A, st) != hipSuccess) return MUON_EHIP;
  }
  return E.mark(st) == hipSuccess ? MUON_OK : MUON_EHIP;
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

static int step_impl(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace,
                     size_t workspace_bytes, float* norms_out, void* stream, void* const* events, int nevents) {
  if (groups == nullptr || ngroups <= 0) return MUON_EINVAL;
  NsCoefs C;
  int rc = parse_cfg(cfg, &C);
  if (rc != MUON_OK) return rc;
  if (norms_out != nullptr && (reinterpret_cast<uintptr_t>(norms_out) & 3u)) return MUON_EINVAL;
  std::vector<GroupRun> runs(ngroups);
  size_t off = 0;
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& gr = groups[i];
    rc = validate_group(gr);
    if (rc != MUON_OK) return rc;
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
  EventRec evr;
  if (events != nullptr) {
    int need = 0;
    for (int i = 0; i < ngroups; ++i)
      if (runs[i].plan.count > 0) need += events_per_group(C.steps, runs[i].plan.small && C.steps > 0);
    if (nevents < need) return MUON_EINVAL;
    for (int i = 0; i < need; ++i)
      if (events[i] == nullptr) return MUON_EINVAL;
    evr.ev = events;
    evr.n = nevents;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  int base = 0;
  for (int i = 0; i < ngroups; ++i) {
    rc = run_group(runs[i], C, cfg->eps, static_cast<char*>(workspace), norms_out ? norms_out + base : nullptr, st,
                   events ? &evr : nullptr);
    if (rc != MUON_OK) return rc;
    base += runs[i].plan.count;
  }
  return MUON_OK;
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
  if (G == nullptr || O == nullptr || !aligned16(G) || !aligned16(O)) return MUON_EINVAL;
  GroupRun R;
  rc = plan_group(m, n, batch, dtype == MUON_BF16, 0, &R.plan);
  if (rc != MUON_OK) return rc;
  const size_t esz = dtype == MUON_BF16 ? 2 : 4;
  const size_t mat = static_cast<size_t>(m) * n * esz;
  if (mat % 16 != 0 && batch > 1) return MUON_EINVAL;  // every matrix must stay 16-B aligned
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
  R.M = nullptr;
  R.W = nullptr;
  R.O = R.o_own.data();
  R.beta = 0.0f;
  R.neg_lr_scale = 0.0f;
  R.nesterov = 0;
  return run_group(R, C, cfg->eps, static_cast<char*>(workspace), nullptr, static_cast<hipStream_t>(stream));
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
  if (X == nullptr || Y == nullptr || !aligned16(X) || !aligned16(Y)) return MUON_EINVAL;
  const size_t esz = bf16 ? 2 : 4;
  const size_t bytes = static_cast<size_t>(m) * n * esz * static_cast<size_t>(batch);
  const char* xb = static_cast<const char*>(X);
  const char* yb = static_cast<const char*>(Y);
  if (yb < xb + bytes && xb < yb + bytes) return MUON_EINVAL;  // overlap
  NsSmallLaunch S{};
  S.X = X; S.Y = Y;
  S.in_stride = static_cast<long long>(m) * n;
  S.out_stride = S.in_stride;
  S.s = s; S.l = l;
  S.ld_in = n;  // row stride of the stored m x n matrix
  S.ld_out = S.ld_in;
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
