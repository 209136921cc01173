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
#include <mutex>
#include <vector>

#include "../../include/muon.h"
#include "launch.h"

using namespace muon;

namespace {

constexpr int kMaxSteps = 64;
constexpr size_t kAlign = 256;
// Every muon_step / muon_ns_orthogonalize workspace opens with this header:
// word 0 is the non-finite flag of the last call (muon_query_flags); the
// per-block partial sums of squares of all groups follow it, contiguous.
constexpr size_t kHeader = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int round_up(int x, int a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t dtype_size(int dt) { return dt == MUON_BF16 ? 2 : 4; }

struct NsCoefs {
  int steps;
  int schedule;
  bool quintic;  // some step has c != 0
  bool separate_apply;
  float a[kMaxSteps], b[kMaxSteps], c[kMaxSteps];
};

// quintic: whether the caller supports c != 0 (else MUON_EUNSUPPORTED)
int parse_cfg(const muon_ns_cfg* cfg, NsCoefs* out, bool quintic = false) {
  if (cfg == nullptr) return MUON_EINVAL;
  if (cfg->steps < 0 || cfg->steps > kMaxSteps) return MUON_EINVAL;
  if (cfg->ncoef != 2 && cfg->ncoef != 3) return MUON_EINVAL;
  if (!(cfg->eps >= 0.0f) || !std::isfinite(cfg->eps)) return MUON_EINVAL;
  if (cfg->precision != MUON_F32 && cfg->precision != MUON_BF16) return MUON_EINVAL;
  if (cfg->schedule != MUON_NS_AUTO && cfg->schedule != MUON_NS_ITERATE && cfg->schedule != MUON_NS_ACCUMULATE)
    return MUON_EINVAL;
  if (cfg->streams != 0 && cfg->streams != 1) return MUON_EINVAL;
  if (cfg->separate_apply != 0 && cfg->separate_apply != 1) return MUON_EINVAL;
  if (cfg->steps > 0 && cfg->coeffs == nullptr) return MUON_EINVAL;
  out->steps = cfg->steps;
  out->schedule = cfg->schedule;
  out->separate_apply = cfg->separate_apply != 0;
  out->quintic = false;
  for (int k = 0; k < cfg->steps; ++k) {
    const float* row = cfg->coeffs + (cfg->per_step ? k * cfg->ncoef : 0);
    if (!std::isfinite(row[0]) || !std::isfinite(row[1])) return MUON_EINVAL;
    out->c[k] = 0.0f;
    if (cfg->ncoef == 3) {
      if (!std::isfinite(row[2])) return MUON_EINVAL;
      if (row[2] != 0.0f && !quintic) return MUON_EUNSUPPORTED;
      out->c[k] = row[2];
      if (row[2] != 0.0f) out->quintic = true;
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
  bool accumulate = false;  // Newton-Schulz as a polynomial in X0 X0^T (bf16 tiled only)
  int s_pad = 0, ld = 0, kdim = 0, P = 0;
  size_t esz = 0;
  size_t off_x0 = 0, off_x1 = 0, off_a = 0, off_part = 0, end = 0;
  bool cap = false;                 // spectral cap: partials of u^T O v and of the power step
  size_t off_cap = 0, off_y = 0, off_z = 0, off_zp = 0, off_yn = 0, off_zn = 0;
};

// s_pad x s_pad buffers after the iterates.  Iterated schedule: A' (cubic) or
// A, H, P (quintic, kSqA0, kSqA1, kSqB0).  Accumulated schedule: all of
// them, H only for quintic coefficients.
enum SqBuf { kSqA0 = 0, kSqA1, kSqB0, kSqB1, kSqE, kSqQ0, kSqQ1, kSqH, kSqMax };
int sq_buffers(bool accumulate, bool quintic) {
  if (accumulate) return quintic ? kSqMax : kSqH;
  return quintic ? 3 : 1;
}

// Matrix-core work of the two schedules (multiply-adds of the tiles actually
// computed): per step a Gram (kdim deep) and a combine (s_pad deep), against
// one Gram, one combine and 3 (steps - 1) symmetric s_pad^3 products.
// (Quintic adds one s x s product per step to either schedule.)
bool choose_accumulate(const GroupPlan& g, const NsCoefs& C) {
  if (g.engine != kTiledBf16 || C.steps < 2 || C.schedule == MUON_NS_ITERATE) return false;
  if (C.schedule == MUON_NS_ACCUMULATE) return true;
  const double t2 = symprod_tile(g.s_pad);
  const double gram = symprod_tiles_per_matrix(g.s_pad) * t2 * t2 * g.kdim;
  const double comb = static_cast<double>(g.s_pad) * g.ld * g.s_pad;  // whatever the combine's tile shape
  const double prod = symprod_tiles_per_matrix(g.s_pad) * t2 * t2 * g.s_pad;
  const double q = C.quintic ? 1.0 : 0.0;
  return gram + comb + (3.0 * (C.steps - 1) + q * C.steps) * prod < 0.85 * C.steps * (gram + comb + q * prod);
}

// Shapes, engine, schedule and the group's own buffers from `base` on; its
// partial sums go to `part_off` (all groups' partials sit together after the
// workspace header, see plan_groups).
int plan_group(int m, int n, int count, bool bf16, const NsCoefs& C, size_t base, GroupPlan* g, bool cap = false,
               size_t part_off = kHeader) {
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
  // quintic steps (c != 0) run on the matrix-core path at every shape
  if (ns_small_supported(bf16, g->s, g->l) && !(bf16 && C.quintic)) {
    g->engine = kSmall;
    // the bf16 kernels take both sides in multiples of 32 (the zero rows and
    // columns the momentum pass appends stay zero through every product)
    g->s_pad = bf16 ? round_up(g->s, 32) : g->s;
    g->ld = round_up(g->l, bf16 ? 32 : 8);
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
  // the matrix-core kernels address one padded iterate with 32-bit buffer
  // offsets: below 2 GiB per matrix
  if (g->engine == kTiledBf16 && static_cast<long long>(g->s_pad) * g->ld * 2 >= (1LL << 31))
    return MUON_EUNSUPPORTED;
  if (C.quintic && g->engine != kTiledBf16) return MUON_EUNSUPPORTED;  // c != 0: bf16 matrix-core path only
  g->accumulate = choose_accumulate(*g, C);
  g->P = momentum_blocks_per_matrix(g->tall, g->s_pad, g->ld);
  g->off_part = part_off;
  const size_t xbytes = static_cast<size_t>(count) * g->s_pad * g->ld * g->esz;
  size_t off = align_up(base, kAlign);
  g->off_x0 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_x1 = off;
  off = align_up(off + xbytes, kAlign);
  g->off_a = off;
  if (g->engine != kSmall)
    off = align_up(off + sq_buffers(g->accumulate, C.quintic) * static_cast<size_t>(count) * g->s_pad * g->s_pad *
                             g->esz,
                   kAlign);
  g->cap = cap;
  if (cap) {
    g->off_cap = off;
    off = align_up(off + static_cast<size_t>(count) * cap_coef_blocks(g->s) * sizeof(float), kAlign);
    const size_t cnt = static_cast<size_t>(count), f = sizeof(float);
    g->off_y = off;
    off = align_up(off + cnt * m * f, kAlign);
    g->off_z = off;
    off = align_up(off + cnt * n * f, kAlign);
    g->off_zp = off;
    off = align_up(off + cnt * power_row_blocks(m) * n * f, kAlign);
    g->off_yn = off;
    off = align_up(off + cnt * power_row_blocks(m) * f, kAlign);
    g->off_zn = off;
    off = align_up(off + cnt * power_col_blocks(n) * f, kAlign);
  }
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
  if (gr.cap_u != nullptr) {
    if (gr.cap_v == nullptr || gr.cap_sigma == nullptr || !aligned_to(gr.cap_sigma, 4) || !std::isfinite(gr.cap))
      return MUON_EINVAL;
    for (int i = 0; i < gr.count; ++i)
      if (gr.cap_u[i] == nullptr || gr.cap_v[i] == nullptr || !aligned_to(gr.cap_u[i], 4) ||
          !aligned_to(gr.cap_v[i], 4))
        return MUON_EINVAL;
  }
  return MUON_OK;
}

// Workspace plan of a list of groups: the header, then the partial sums of
// every group (contiguous, so that one pass can scan them), then each group's
// buffers.  Returns MUON_OK and the total size in *end, the number of partial
// sums in *nparts.
struct GroupShape {
  int m, n, count;
  bool cap;
};
int plan_groups(const std::vector<GroupShape>& shapes, bool bf16, const NsCoefs& C, std::vector<GroupPlan>& plans,
                size_t* end, long long* nparts) {
  plans.assign(shapes.size(), GroupPlan{});
  long long parts = 0;
  for (size_t i = 0; i < shapes.size(); ++i) {
    const int rc = plan_group(shapes[i].m, shapes[i].n, shapes[i].count, bf16, C, 0, &plans[i], shapes[i].cap);
    if (rc != MUON_OK) return rc;
    parts += static_cast<long long>(plans[i].count) * plans[i].P;
  }
  size_t off = align_up(kHeader + static_cast<size_t>(parts) * sizeof(float), kAlign);
  size_t part = kHeader;
  for (size_t i = 0; i < shapes.size(); ++i) {
    plan_group(shapes[i].m, shapes[i].n, shapes[i].count, bf16, C, off, &plans[i], shapes[i].cap, part);
    part += static_cast<size_t>(plans[i].count) * plans[i].P * sizeof(float);
    off = plans[i].end;
  }
  *end = off;
  *nparts = parts;
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
  int ldg = 0, ldo = 0;            // row strides of G and O (elements; 0: n)
  int norm_base = 0;               // first slot of this group in norms_out
  float* const* cap_u = nullptr;   // spectral cap state (null: off)
  float* const* cap_v = nullptr;
  float* cap_sigma = nullptr;
  float cap = 0.0f;
};

// Optional phase markers: caller-created events recorded on the stream after
// each phase of the schedule (profiling only; the arithmetic is unchanged).
// A dry run launches nothing and only lists the phases.
struct EventRec {
  void* const* ev = nullptr;
  int n = 0, used = 0;
  bool dry = false;
  std::vector<int> phases;
  bool mark(hipStream_t st, int phase) {
    if (dry) {
      phases.push_back(phase);
      return true;
    }
    if (ev == nullptr) return true;
    if (used >= n) return false;
    return hipEventRecord(static_cast<hipEvent_t>(ev[used++]), st) == hipSuccess;
  }
  bool live() const { return !dry; }
};

char* x_of(const GroupPlan& p, char* ws, int which) { return ws + (which ? p.off_x1 : p.off_x0); }

bf16_t* sq_of(const GroupPlan& p, char* ws, int which) {
  return reinterpret_cast<bf16_t*>(ws + p.off_a + static_cast<size_t>(which) * p.count * p.s_pad * p.s_pad * p.esz);
}

// Grouped launches of up to kMaxSeg segments each.
template <class Args, class Seg, class Launch>
bool launch_segments(const std::vector<Seg>& segs, Launch launch, hipStream_t st, bool live) {
  for (size_t c0 = 0; c0 < segs.size(); c0 += kMaxSeg) {
    Args G{};
    G.nseg = static_cast<int>(std::min<size_t>(kMaxSeg, segs.size() - c0));
    for (int i = 0; i < G.nseg; ++i) G.seg[i] = segs[c0 + i];
    if (live && launch(G, st) != hipSuccess) return false;
  }
  return true;
}

// The Gram X X^T runs on the symmetric-product kernel (L = R = the iterate):
// same outputs, coefficients and normalisation powers as the Gram segment.
SymSeg gram_as_sym(const GemmSeg& G) {
  SymSeg S{};
  S.L = G.X; S.R = G.X;
  S.O1 = G.A; S.O2 = G.A2;
  S.stride = G.astride; S.in_stride = G.xstride;
  S.ld = G.ld; S.kdim = G.kdim;
  S.s_pad = G.s_pad; S.count = G.count; S.tiles_per_mat = symprod_tiles_per_matrix(G.s_pad);
  S.partials = G.partials; S.P = G.P; S.eps = G.eps;
  S.a1 = G.a; S.b1 = G.b; S.a2 = G.a2; S.b2 = G.b2;
  S.pa = G.pa; S.pb = G.pb;
  return S;
}
// tri_out: the outputs keep only their upper block triangle (they feed
// symmetric products only).
std::vector<SymSeg> grams_as_sym(const std::vector<GemmSeg>& gs, bool tri_out = false) {
  std::vector<SymSeg> out;
  for (const GemmSeg& G : gs) {
    out.push_back(gram_as_sym(G));
    out.back().tri_out = tri_out ? 1 : 0;
  }
  return out;
}

int flags_pass(long long nparts, char* ws, hipStream_t st, EventRec& E);

// fork: when non-null, recorded on st once the Gram of the accumulated
// schedule (if any group of this run takes it), else the momentum passes, of
// these groups have been enqueued (the momentum partial sums are complete by
// then either way).  flags_nparts >= 0: after the momentum
// passes, the call's non-finite flag from the first flags_nparts partial sums (every
// group's partials are complete by then: this run's momentum passes are the
// call's last ones).
int run_all(std::vector<GroupRun>& runs, const NsCoefs& C, float eps, char* ws, float* norms_out, hipStream_t st,
            EventRec& E, hipEvent_t fork = nullptr, long long flags_nparts = -1) {
  if (!E.mark(st, 0)) return MUON_EHIP;
  // 1. momentum
  for (GroupRun& R : runs) {
    const GroupPlan& p = R.plan;
    if (p.count == 0) continue;
    const long long xstride = static_cast<long long>(p.s_pad) * p.ld;
    float* part = reinterpret_cast<float*>(ws + p.off_part);
    for (int c0 = 0; E.live() && c0 < p.count; c0 += kMaxTable) {
      const int cn = std::min(kMaxTable, p.count - c0);
      MomentumLaunch L{};
      for (int i = 0; i < cn; ++i) {
        L.G.p[i] = R.G[c0 + i];
        L.M.p[i] = R.M ? R.M[c0 + i] : nullptr;
      }
      L.X = ws + p.off_x0 + static_cast<size_t>(c0) * xstride * p.esz;
      L.xstride = xstride;
      L.m = p.m; L.n = p.n; L.s_pad = p.s_pad; L.ld = p.ld; L.count = cn; L.P = p.P;
      L.ldg = R.ldg > 0 ? R.ldg : p.n;
      L.tall = p.tall; L.grad_bf16 = R.grad_dtype == MUON_BF16; L.x_bf16 = p.bf16;
      L.beta = R.beta; L.nesterov = R.nesterov;
      L.partials = part + static_cast<size_t>(c0) * p.P;
      if (launch_momentum(L, st) != hipSuccess) return MUON_EHIP;
    }
    if (E.live() && norms_out != nullptr &&
        launch_norms(part, p.P, p.count, norms_out + R.norm_base, st) != hipSuccess)
      return MUON_EHIP;
    if (!E.mark(st, MUON_PHASE_MOMENTUM)) return MUON_EHIP;
  }
  // the fork point: after the accumulated schedule's Gram when this run has
  // one (the Gram then runs alone instead of beside the other chain's
  // bandwidth-bound momentum pass, which overlaps the products instead), else
  // after the momentum passes.  With the spectral cap (its separate apply and
  // power-step passes lengthen the end of each chain) the earlier fork
  // measured faster.
  bool fork_after_gram = false, any_cap = false;
  if (fork != nullptr)
    for (GroupRun& R : runs)
      if (R.plan.count > 0) {
        fork_after_gram = fork_after_gram || R.plan.accumulate;
        any_cap = any_cap || R.plan.cap;
      }
  if (any_cap) fork_after_gram = false;
  if (fork != nullptr && !fork_after_gram && E.live() && hipEventRecord(fork, st) != hipSuccess) return MUON_EHIP;
  if (flags_nparts >= 0) {
    const int rc = flags_pass(flags_nparts, ws, st, E);
    if (rc != MUON_OK) return rc;
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
    S.s = p.bf16 ? p.s_pad : p.s; S.l = p.bf16 ? p.ld : p.l; S.ld_in = p.ld; S.ld_out = p.ld;
    S.count = p.count; S.transposed = false; S.steps = C.steps;
    for (int k = 0; k < C.steps; ++k) { S.a[k] = C.a[k]; S.b[k] = C.b[k]; }
    S.partials = reinterpret_cast<const float*>(ws + p.off_part); S.P = p.P; S.eps = eps;
    if (E.live() && launch_ns_small(S, p.bf16, st) != hipSuccess) return MUON_EHIP;
    fin[gi] = 1;
    if (!E.mark(st, MUON_PHASE_NS_SMALL)) return MUON_EHIP;
  }

  // 3. large bf16 matrices, grouped launches: the iterated schedule first,
  //    then the accumulated one
  std::vector<int> it, ac;
  for (size_t gi = 0; gi < runs.size(); ++gi) {
    const GroupPlan& p = runs[gi].plan;
    if (p.count > 0 && p.engine == kTiledBf16) (p.accumulate ? ac : it).push_back(static_cast<int>(gi));
  }
  auto heavy_first = [&](std::vector<int> v, bool by_kdim) {
    std::stable_sort(v.begin(), v.end(), [&](int x, int y) {
      return by_kdim ? runs[x].plan.kdim > runs[y].plan.kdim : runs[x].plan.s_pad > runs[y].plan.s_pad;
    });
    return v;
  };
  auto gemm_seg = [&](const GroupPlan& p, bool gram) {
    GemmSeg S{};
    S.xstride = static_cast<long long>(p.s_pad) * p.ld;
    S.astride = static_cast<long long>(p.s_pad) * p.s_pad;
    S.s_pad = p.s_pad; S.ld = p.ld; S.kdim = p.kdim; S.count = p.count;
    S.tiles_per_mat = gram ? symprod_tiles_per_matrix(p.s_pad) : combine_tiles_per_matrix(p.s_pad, p.ld);
    S.P = p.P; S.eps = eps;
    return S;
  };
  auto sym_seg = [&](const GroupPlan& p) {
    SymSeg S{};
    S.stride = static_cast<long long>(p.s_pad) * p.s_pad;
    S.in_stride = S.stride;
    S.ld = p.s_pad; S.kdim = p.s_pad;
    S.s_pad = p.s_pad; S.count = p.count; S.tiles_per_mat = symprod_tiles_per_matrix(p.s_pad);
    S.P = p.P; S.eps = eps;
    S.b1 = 1.0f;
    return S;
  };
  // The final combine of a group also applies its update when nothing else
  // needs the final iterate (no spectral cap); the W and O tables of one
  // launch hold at most kMaxTable matrices.
  std::vector<char> fused(runs.size(), 0);
  auto decide_fused = [&](const std::vector<int>& order) {
    for (size_t c0 = 0; c0 < order.size(); c0 += kMaxSeg) {
      int tab = 0;
      for (size_t i = c0; i < std::min(order.size(), c0 + kMaxSeg); ++i) {
        const GroupRun& R = runs[order[i]];
        // (the fused epilogue writes O with rows n apart: a strided O keeps the apply pass)
        const bool ok = !C.separate_apply && !R.plan.cap && (R.W != nullptr || R.O != nullptr) &&
                        (R.ldo == 0 || R.ldo == R.plan.n) && tab + R.plan.count <= kMaxTable;
        fused[order[i]] = ok;
        if (ok) tab += R.plan.count;
      }
    }
  };
  auto final_combine = [&](std::vector<GemmSeg>& cs, const std::vector<int>& order) {
    bool any = false;
    for (size_t c0 = 0; c0 < cs.size(); c0 += kMaxSeg) {
      GemmArgs G{};
      G.nseg = static_cast<int>(std::min<size_t>(kMaxSeg, cs.size() - c0));
      int tab = 0;
      for (int i = 0; i < G.nseg; ++i) {
        GemmSeg S = cs[c0 + i];
        const GroupRun& R = runs[order[c0 + i]];
        const GroupPlan& p = R.plan;
        if (fused[order[c0 + i]]) {
          any = true;
          S.fuse = 1;
          S.Y = nullptr;
          S.tab0 = tab;
          S.m = p.m; S.n = p.n; S.s = p.s; S.l = p.l; S.tall = p.tall;
          S.neg_lr_scale = R.neg_lr_scale;
          for (int z = 0; z < p.count; ++z) {
            G.W.p[tab + z] = R.W ? R.W[z] : nullptr;
            G.O.p[tab + z] = R.O ? R.O[z] : nullptr;
          }
          tab += p.count;
        }
        G.seg[i] = S;
      }
      if (E.live() && launch_combine_bf16(G, st) != hipSuccess) return false;
    }
    return E.mark(st, any ? MUON_PHASE_COMBINE_APPLY : MUON_PHASE_COMBINE);
  };
  if (!it.empty() && C.steps > 0) {
    // per step: A' = a I + b X X^T (step 1 on the unnormalised U, with the
    // normalisation folded into the coefficients), then X = A' X.  Quintic:
    // A = X X^T and H = b I + c A from the Gram, P = a I + A H (= a I + b A +
    // c A^2) from one symmetric product, then X = P X.
    const std::vector<int> by_k = heavy_first(it, true), by_s = heavy_first(it, false);
    for (int k = 0; k < C.steps; ++k) {
      const int cur = k & 1;
      std::vector<GemmSeg> gs, cs;
      std::vector<SymSeg> ps;
      for (int gi : by_k) {
        const GroupPlan& p = runs[gi].plan;
        GemmSeg S = gemm_seg(p, true);
        S.X = reinterpret_cast<const bf16_t*>(x_of(p, ws, cur));
        S.A = sq_of(p, ws, kSqA0);
        S.partials = k == 0 ? reinterpret_cast<const float*>(ws + p.off_part) : nullptr;
        if (!C.quintic) {
          S.a = C.a[k]; S.b = C.b[k];
          S.pa = k == 0 ? 1 : 0; S.pb = k == 0 ? 3 : 0;
        } else {
          S.a = 0.0f; S.b = 1.0f; S.pa = 0; S.pb = k == 0 ? 2 : 0;   // A
          S.A2 = sq_of(p, ws, kSqA1); S.a2 = C.b[k]; S.b2 = C.c[k];  // H = b I + c A
          SymSeg Q = sym_seg(p);                                      // P = a I + A H
          Q.L = sq_of(p, ws, kSqA0); Q.R = sq_of(p, ws, kSqA1); Q.O1 = sq_of(p, ws, kSqB0);
          Q.a1 = C.a[k];
          if (k == 0) {  // X0 = inv U: fold inv into P
            Q.partials = reinterpret_cast<const float*>(ws + p.off_part);
            Q.pa = 1; Q.pb = 1;
          }
          ps.push_back(Q);
        }
        gs.push_back(S);
      }
      for (int gi : by_s) {
        const GroupPlan& p = runs[gi].plan;
        GemmSeg S = gemm_seg(p, false);
        S.X = reinterpret_cast<const bf16_t*>(x_of(p, ws, cur));
        S.Y = reinterpret_cast<bf16_t*>(x_of(p, ws, cur ^ 1));
        S.A = sq_of(p, ws, C.quintic ? kSqB0 : kSqA0);
        cs.push_back(S);
      }
      if (!launch_segments<SymArgs>(grams_as_sym(gs), launch_symprod_bf16, st, E.live()) ||
          !E.mark(st, MUON_PHASE_GRAM))
        return MUON_EHIP;
      if (C.quintic &&
          (!launch_segments<SymArgs>(ps, launch_symprod_bf16, st, E.live()) || !E.mark(st, MUON_PHASE_SYMPROD)))
        return MUON_EHIP;
      if (k + 1 < C.steps) {
        if (!launch_segments<GemmArgs>(cs, launch_combine_bf16, st, E.live()) || !E.mark(st, MUON_PHASE_COMBINE))
          return MUON_EHIP;
      } else {
        decide_fused(by_s);
        if (!final_combine(cs, by_s)) return MUON_EHIP;
      }
    }
    for (int gi : it) fin[gi] = C.steps & 1;
  }
  if (!ac.empty()) {
    // Every step's factor is a polynomial in A_0 = X0 X0^T (X0 normalised), so
    // with B_k = a_k I + b_k A_k the steps are
    //   A_{k+1} = A_k B_k^2,   Q = B_{steps-1} ... B_1 B_0,   X = Q X0,
    // s_pad x s_pad products instead of s_pad x ld ones.  Buffers: A_k in
    // A[k & 1], B_k in B[k & 1], E = B_k^2, Q_1 = B_0, Q_k (k >= 2) in Q[k & 1].
    // Quintic: B_k = a_k I + A_k H_k with H_k = b_k I + c_k A_k (buffer H),
    // one more product per step.
    const int n = C.steps;
    const std::vector<int> by_k = heavy_first(ac, true), by_s = heavy_first(ac, false);
    std::vector<GemmSeg> gs;
    for (int gi : by_k) {
      const GroupPlan& p = runs[gi].plan;
      GemmSeg S = gemm_seg(p, true);
      S.X = reinterpret_cast<const bf16_t*>(x_of(p, ws, 0));
      S.A = sq_of(p, ws, kSqA0);
      S.A2 = sq_of(p, ws, kSqB0);
      S.partials = reinterpret_cast<const float*>(ws + p.off_part);
      S.a = 0.0f; S.b = 1.0f; S.pa = 0; S.pb = 2;  // A_0 = inv^2 U U^T
      if (!C.quintic) {
        S.a2 = C.a[0]; S.b2 = C.b[0];              // B_0
      } else {
        S.A2 = sq_of(p, ws, kSqH);                 // H_0 = b_0 I + c_0 A_0
        S.a2 = C.b[0]; S.b2 = C.c[0];
      }
      gs.push_back(S);
    }
    if (!launch_segments<SymArgs>(grams_as_sym(gs, true), launch_symprod_bf16, st, E.live()) ||
        !E.mark(st, MUON_PHASE_GRAM))
      return MUON_EHIP;
    if (fork_after_gram && E.live() && hipEventRecord(fork, st) != hipSuccess) return MUON_EHIP;
    // every s x s matrix of the chain keeps only its upper block triangle
    // (the products read the rest transposed), except the final Q, which the
    // combine reads whole
    for (int k = 0; k < n; ++k) {
      if (C.quintic) {  // B_k = a_k I + A_k H_k
        std::vector<SymSeg> lb;
        for (int gi : ac) {
          const GroupPlan& p = runs[gi].plan;
          SymSeg S = sym_seg(p);
          S.L = sq_of(p, ws, kSqA0 + (k & 1)); S.R = sq_of(p, ws, kSqH); S.O1 = sq_of(p, ws, kSqB0 + (k & 1));
          S.a1 = C.a[k];
          S.tri_in = 1; S.tri_out = 1;
          lb.push_back(S);
        }
        if (!launch_segments<SymArgs>(lb, launch_symprod_bf16, st, E.live()) || !E.mark(st, MUON_PHASE_SYMPROD))
          return MUON_EHIP;
      }
      std::vector<SymSeg> l1, l2;
      for (int gi : ac) {
        const GroupPlan& p = runs[gi].plan;
        bf16_t* Bk = sq_of(p, ws, kSqB0 + (k & 1));
        if (k + 1 < n) {  // E = B_k B_k (shares B_k with the Q product of the same matrix)
          SymSeg S = sym_seg(p);
          S.L = Bk; S.R = Bk; S.O1 = sq_of(p, ws, kSqE);
          S.zip_next = k >= 1 ? 1 : 0;
          S.tri_in = 1; S.tri_out = 1;
          l1.push_back(S);
        }
        if (k >= 1) {  // Q_{k+1} = B_k Q_k; the last one carries the normalisation
          SymSeg S = sym_seg(p);
          S.L = Bk;
          S.R = k == 1 ? sq_of(p, ws, kSqB0) : sq_of(p, ws, kSqQ0 + (k & 1));
          S.O1 = sq_of(p, ws, kSqQ0 + ((k + 1) & 1));
          S.tri_in = 1;
          S.tri_out = k + 1 < n ? 1 : 0;
          if (k + 1 == n) {
            S.partials = reinterpret_cast<const float*>(ws + p.off_part);
            S.pb = 1;
          }
          l1.push_back(S);
        }
        if (k + 1 < n) {  // A_{k+1} = A_k E, B_{k+1} = a I + b A_{k+1} (quintic: H_{k+1} = b I + c A_{k+1})
          SymSeg S = sym_seg(p);
          S.L = sq_of(p, ws, kSqA0 + (k & 1));
          S.R = sq_of(p, ws, kSqE);
          S.tri_in = 1; S.tri_out = 1;
          if (!C.quintic) {
            S.O1 = k + 2 < n ? sq_of(p, ws, kSqA0 + ((k + 1) & 1)) : nullptr;  // the last A is not needed
            S.O2 = sq_of(p, ws, kSqB0 + ((k + 1) & 1));
            S.a2 = C.a[k + 1]; S.b2 = C.b[k + 1];
          } else {
            S.O1 = sq_of(p, ws, kSqA0 + ((k + 1) & 1));
            S.O2 = sq_of(p, ws, kSqH);
            S.a2 = C.b[k + 1]; S.b2 = C.c[k + 1];
          }
          l2.push_back(S);
        }
      }
      if (!launch_segments<SymArgs>(l1, launch_symprod_bf16, st, E.live()) || !E.mark(st, MUON_PHASE_SYMPROD))
        return MUON_EHIP;
      if (!l2.empty() &&
          (!launch_segments<SymArgs>(l2, launch_symprod_bf16, st, E.live()) || !E.mark(st, MUON_PHASE_SYMPROD)))
        return MUON_EHIP;
    }
    std::vector<GemmSeg> cs;
    for (int gi : by_s) {
      const GroupPlan& p = runs[gi].plan;
      GemmSeg S = gemm_seg(p, false);
      S.X = reinterpret_cast<const bf16_t*>(x_of(p, ws, 0));
      S.Y = reinterpret_cast<bf16_t*>(x_of(p, ws, 1));
      S.A = sq_of(p, ws, kSqQ0 + (n & 1));
      cs.push_back(S);
    }
    decide_fused(by_s);
    if (!final_combine(cs, by_s)) return MUON_EHIP;
    for (int gi : ac) fin[gi] = 1;
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
      if ((E.live() && launch_gram_f32(L, st) != hipSuccess) || !E.mark(st, MUON_PHASE_F32_GRAM)) return MUON_EHIP;
      if ((E.live() && launch_combine_f32(L, st) != hipSuccess) || !E.mark(st, MUON_PHASE_F32_COMBINE))
        return MUON_EHIP;
    }
    fin[gi] = C.steps & 1;
  }

  // 5. apply (spectral cap: coefficient before, power step after)
  for (size_t gi = 0; gi < runs.size(); ++gi) {
    const GroupRun& R = runs[gi];
    const GroupPlan& p = R.plan;
    if (p.count == 0 || fused[gi]) continue;
    const long long xs = static_cast<long long>(p.s_pad) * p.ld;
    if (p.cap) {
      for (int c0 = 0; E.live() && c0 < p.count; c0 += kMaxTable) {
        const int cn = std::min(kMaxTable, p.count - c0);
        CapCoefLaunch K{};
        K.X = x_of(p, ws, fin[gi]) + static_cast<size_t>(c0) * xs * p.esz;
        K.xstride = xs;
        K.s = p.s; K.l = p.l; K.ld = p.ld; K.count = cn; K.tall = p.tall;
        for (int i = 0; i < cn; ++i) { K.u.p[i] = R.cap_u[c0 + i]; K.v.p[i] = R.cap_v[c0 + i]; }
        K.P = cap_coef_blocks(p.s);
        K.part = reinterpret_cast<float*>(ws + p.off_cap) + static_cast<size_t>(c0) * K.P;
        if (launch_cap_coef(K, p.bf16, st) != hipSuccess) return MUON_EHIP;
      }
      if (!E.mark(st, MUON_PHASE_CAP)) return MUON_EHIP;
    }
    if (E.live() && (R.W != nullptr || R.O != nullptr)) {
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
        A.ldo = R.ldo > 0 ? R.ldo : p.n;
        A.tall = p.tall; A.x_bf16 = p.bf16;
        A.partials = C.steps == 0 ? reinterpret_cast<const float*>(ws + p.off_part) + static_cast<size_t>(c0) * p.P
                                  : nullptr;
        A.P = p.P; A.eps = eps;
        A.neg_lr_scale = R.neg_lr_scale;
        if (p.cap) {
          A.cap_P = cap_coef_blocks(p.s);
          A.cap_part = reinterpret_cast<const float*>(ws + p.off_cap) + static_cast<size_t>(c0) * A.cap_P;
          A.cap_sigma = R.cap_sigma + c0;
          A.cap = R.cap;
          for (int i = 0; i < cn; ++i) { A.cu.p[i] = R.cap_u[c0 + i]; A.cv.p[i] = R.cap_v[c0 + i]; }
        }
        if (launch_apply(A, st) != hipSuccess) return MUON_EHIP;
      }
    }
    if (!E.mark(st, MUON_PHASE_APPLY)) return MUON_EHIP;
    if (p.cap) {
      for (int c0 = 0; E.live() && c0 < p.count; c0 += kMaxTable) {
        const int cn = std::min(kMaxTable, p.count - c0);
        PowerLaunch L{};
        for (int i = 0; i < cn; ++i) {
          L.W.p[i] = R.W[c0 + i]; L.u.p[i] = R.cap_u[c0 + i]; L.v.p[i] = R.cap_v[c0 + i];
        }
        L.sigma = R.cap_sigma + c0;
        L.m = p.m; L.n = p.n; L.count = cn;
        L.nrc = power_row_blocks(p.m); L.ncb = power_col_blocks(p.n);
        L.ybuf = reinterpret_cast<float*>(ws + p.off_y) + static_cast<size_t>(c0) * p.m;
        L.zbuf = reinterpret_cast<float*>(ws + p.off_z) + static_cast<size_t>(c0) * p.n;
        L.zpart = reinterpret_cast<float*>(ws + p.off_zp) + static_cast<size_t>(c0) * L.nrc * p.n;
        L.ynorm = reinterpret_cast<float*>(ws + p.off_yn) + static_cast<size_t>(c0) * L.nrc;
        L.znorm = reinterpret_cast<float*>(ws + p.off_zn) + static_cast<size_t>(c0) * L.ncb;
        if (launch_power_step(L, st) != hipSuccess) return MUON_EHIP;
      }
      if (!E.mark(st, MUON_PHASE_POWER)) return MUON_EHIP;
    }
  }
  return MUON_OK;
}

// The non-finite flag of the header from the partial sums of all groups,
// enqueued once every momentum pass of the call is.
int flags_pass(long long nparts, char* ws, hipStream_t st, EventRec& E) {
  if (nparts == 0) return MUON_OK;  // no matrix: nothing ran, the flag is left as it was
  if (E.live() && launch_flags(reinterpret_cast<const float*>(ws + kHeader), nparts, reinterpret_cast<unsigned*>(ws),
                               st) != hipSuccess)
    return MUON_EHIP;
  return E.mark(st, MUON_PHASE_FLAGS) ? MUON_OK : MUON_EHIP;
}

// The marks run_all makes, in order (the first is the start mark, phase 0),
// from a dry run that launches nothing and touches no memory.
std::vector<int> list_phases(std::vector<GroupRun>& runs, const NsCoefs& C, float eps, long long nparts) {
  EventRec D;
  D.dry = true;
  char* fake_ws = reinterpret_cast<char*>(static_cast<uintptr_t>(kAlign));
  run_all(runs, C, eps, fake_ws, nullptr, nullptr, D, nullptr, nparts);
  return D.phases;
}

// Per device, created on first use and kept until the process ends: one
// auxiliary stream (default priority, non-blocking) and the fork / join
// events that order it against the caller's stream.  The table is a fixed
// array of plain pointers, so the library registers no destructor that would
// run at exit (devices past 64 run on the caller's stream alone).
struct Aux {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t partials = nullptr;  // the auxiliary chain's momentum partial sums are complete
  std::mutex mu;  // one fork / join sequence at a time
};

Aux* aux_for_current_device() {
  constexpr int kMaxDev = 64;
  static std::mutex table_mu;
  static Aux* table[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> lock(table_mu);
  if (table[dev] == nullptr) {
    Aux* a = new Aux();
    if (hipStreamCreateWithFlags(&a->s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&a->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&a->join, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&a->partials, hipEventDisableTiming) != hipSuccess) {
      delete a;  // leaves this device on one stream
      return nullptr;
    }
    table[dev] = a;
  }
  return table[dev];
}

// Validates every group, plans the workspace and fills the launch records.
int prepare_step(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, NsCoefs* C,
                 std::vector<GroupRun>& runs, size_t* end, long long* nparts, bool validate_ptrs) {
  if (groups == nullptr || ngroups <= 0) return MUON_EINVAL;
  int rc = parse_cfg(cfg, C, true);
  if (rc != MUON_OK) return rc;
  std::vector<GroupShape> shapes(ngroups);
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& gr = groups[i];
    if (validate_ptrs) {
      rc = validate_group(gr);
      if (rc != MUON_OK) return rc;
      if (gr.O != nullptr)
        for (int j = 0; j < gr.count; ++j)
          if (!aligned_to(gr.O[j], dtype_size(cfg->precision))) return MUON_EINVAL;
      if (gr.cap_u != nullptr && gr.W == nullptr) return MUON_EINVAL;
    } else if (gr.grad_dtype != MUON_F32 && gr.grad_dtype != MUON_BF16) {
      return MUON_EINVAL;
    }
    shapes[i] = GroupShape{gr.m, gr.n, gr.count, gr.cap_u != nullptr};
  }
  std::vector<GroupPlan> plans;
  rc = plan_groups(shapes, cfg->precision == MUON_BF16, *C, plans, end, nparts);
  if (rc != MUON_OK) return rc;
  runs.assign(ngroups, GroupRun{});
  for (int i = 0; i < ngroups; ++i) {
    const muon_group& gr = groups[i];
    runs[i].plan = plans[i];
    runs[i].cap_u = gr.cap_u;
    runs[i].cap_v = gr.cap_v;
    runs[i].cap_sigma = gr.cap_sigma;
    runs[i].cap = gr.cap;
    runs[i].grad_dtype = gr.grad_dtype;
    runs[i].G = gr.G;
    runs[i].M = gr.M;
    runs[i].W = gr.W;
    runs[i].O = gr.O;
    runs[i].beta = gr.beta;
    runs[i].neg_lr_scale = -gr.lr * gr.scale;
    runs[i].nesterov = gr.nesterov;
    runs[i].norm_base = i == 0 ? 0 : runs[i - 1].norm_base + groups[i - 1].count;
  }
  return MUON_OK;
}

int step_impl(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace, size_t workspace_bytes,
              float* norms_out, void* stream, void* const* events, int nevents) {
  NsCoefs C;
  std::vector<GroupRun> runs;
  size_t need = 0;
  long long nparts = 0;
  int rc = prepare_step(groups, ngroups, cfg, &C, runs, &need, &nparts, true);
  if (rc != MUON_OK) return rc;
  if (norms_out != nullptr && !aligned_to(norms_out, 4)) return MUON_EINVAL;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return MUON_EWORKSPACE;
  EventRec E;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (events != nullptr) {
    const int need_ev = static_cast<int>(list_phases(runs, C, cfg->eps, nparts).size());
    if (nevents < need_ev) return MUON_EINVAL;
    for (int i = 0; i < need_ev; ++i)
      if (events[i] == nullptr) return MUON_EINVAL;
    E.ev = events;
    E.n = nevents;
    return run_all(runs, C, cfg->eps, ws, norms_out, st, E, nullptr, nparts);  // timed: one stream, phases in order
  }
  // Independent shape groups run as two chains on two streams (the caller's
  // and an auxiliary one, joined back before returning), so that one chain's
  // launch tails and bandwidth-bound passes overlap the other's matrix-core
  // work.  Groups are dealt to the chains by estimated cost, heaviest first;
  // the lighter chain starts once the heavier one's momentum pass and, with
  // the accumulated schedule, its Gram are done, so that the critical chain's
  // bandwidth-bound first pass and its Gram run alone and the lighter chain's
  // momentum pass overlaps the heavier chain's products (measured faster than
  // starting after the momentum pass, which was faster than starting both
  // together).
  std::vector<int> live;
  for (int i = 0; i < ngroups; ++i)
    if (runs[i].plan.count > 0) live.push_back(i);
  Aux* aux = cfg->streams == 1 || live.size() < 2 ? nullptr : aux_for_current_device();
  if (aux == nullptr) return run_all(runs, C, cfg->eps, ws, norms_out, st, E, nullptr, nparts);
  auto cost = [&](int i) {
    const GroupPlan& p = runs[i].plan;
    return static_cast<double>(p.count) * p.m * p.n * (p.engine == kSmall ? 16.0 : p.s + 64.0);
  };
  std::stable_sort(live.begin(), live.end(), [&](int x, int y) { return cost(x) > cost(y); });
  std::vector<GroupRun> chain[2];
  double load[2] = {0.0, 0.0};
  for (int i : live) {
    const int c = load[0] <= load[1] ? 0 : 1;
    chain[c].push_back(runs[i]);
    load[c] += cost(i);
  }
  std::lock_guard<std::mutex> lock(aux->mu);
  EventRec E1;
  rc = run_all(chain[0], C, cfg->eps, ws, norms_out, st, E, aux->fork);  // fork: after chain 0's Gram
  if (hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess) return MUON_EHIP;
  // the second chain records `partials` once its momentum passes (the call's
  // last) are done, at its own fork point; the call's non-finite flag is then
  // taken on the caller's stream after the first chain's work, which ends
  // earlier than the second chain's, so the flag pass is off the longer chain
  const int rc1 = rc == MUON_OK ? run_all(chain[1], C, cfg->eps, ws, norms_out, aux->s, E1, aux->partials)
                                : MUON_OK;
  int rc2 = MUON_OK;
  if (rc == MUON_OK && rc1 == MUON_OK)
    rc2 = hipStreamWaitEvent(st, aux->partials, 0) != hipSuccess ? MUON_EHIP : flags_pass(nparts, ws, st, E);
  // join even after a failed launch, so that the caller's stream never runs ahead of the auxiliary work
  if (hipEventRecord(aux->join, aux->s) != hipSuccess || hipStreamWaitEvent(st, aux->join, 0) != hipSuccess)
    return MUON_EHIP;
  return rc != MUON_OK ? rc : rc1 != MUON_OK ? rc1 : rc2;
}

// ---- spectral diagnostics ------------------------------------------------------
constexpr int kDiagMaxS = 4096;
constexpr int kDiagMaxIters = 512;
constexpr size_t kDiagChunkBytes = size_t(1) << 31;  // workspace of one chunk of matrices

struct DiagPlan {
  int s, l, s_pad, kdim, ld, k;
  bool tall, f32;
  size_t op_bytes, h_bytes, q_bytes;  // per matrix
  long long chunk;                    // matrices per pass
  size_t off_l, off_h, off_q, end;
};

int plan_diag(int m, int n, long long batch, int dtype, int iters, DiagPlan* p) {
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (m <= 0 || n <= 0 || batch < 0 || iters < 1) return MUON_EINVAL;
  p->tall = m > n;
  p->s = std::min(m, n);
  p->l = std::max(m, n);
  p->f32 = dtype == MUON_F32;
  if (p->s > kDiagMaxS || iters > kDiagMaxIters) return MUON_EUNSUPPORTED;
  p->s_pad = round_up(p->s, 128);
  if (p->l > (1 << 22)) return MUON_EUNSUPPORTED;
  p->kdim = round_up(p->l, 64);
  p->ld = p->kdim * (p->f32 ? 3 : 1);
  if (static_cast<long long>(p->s_pad) * p->ld * 2 >= (1LL << 31)) return MUON_EUNSUPPORTED;  // 32-bit offsets
  p->k = std::min(iters, p->s);
  p->op_bytes = align_up(static_cast<size_t>(p->s_pad) * p->ld * 2, kAlign);
  p->h_bytes = align_up(static_cast<size_t>(p->s_pad) * p->s_pad * 4, kAlign);
  p->q_bytes = align_up(static_cast<size_t>(p->k) * p->s_pad * 4, kAlign);
  const size_t per = p->op_bytes + p->h_bytes + p->q_bytes;
  p->chunk = std::max<long long>(1, std::min<long long>(batch, static_cast<long long>(kDiagChunkBytes / per)));
  const size_t c = static_cast<size_t>(p->chunk);
  p->off_l = 0;
  p->off_h = p->off_l + c * p->op_bytes;
  p->off_q = p->off_h + c * p->h_bytes;
  p->end = p->off_q + c * p->q_bytes;
  return MUON_OK;
}

}  // namespace

namespace {

// Shapes, padding, LDS split and coefficients of a factored Newton-Schulz
// launch (pointers and the vector-load flag are the caller's).
int factored_launch(int m, int n, int r, long long batch, const NsCoefs& C, float eps, bool dense, FactLaunch* F) {
  if (m <= 0 || n <= 0 || r <= 0 || batch < 0) return MUON_EINVAL;
  if (r > 8 || m > 256 || n > 256) return MUON_EUNSUPPORTED;
  if (dense && n % 8 != 0) return MUON_EUNSUPPORTED;
  const int m_pad = round_up(m, 16), n_pad = round_up(n, 16);
  int f_off = 0;
  const int per_wave = factored_lds_per_wave(m_pad, n_pad, dense, &f_off);
  if (per_wave > 65536) return MUON_EUNSUPPORTED;
  F->batch = batch;
  F->m = m; F->n = n; F->r = r; F->m_pad = m_pad; F->n_pad = n_pad;
  F->waves = std::max(1, std::min(4, 65536 / per_wave));
  F->per_wave = per_wave;
  F->f_off = f_off;
  F->steps = C.steps;
  F->eps = eps;
  for (int k = 0; k < C.steps; ++k) { F->a[k] = C.a[k]; F->b[k] = C.b[k]; F->c[k] = C.c[k]; }
  return MUON_OK;
}

bool overlaps(const char* a, size_t na, const char* b, size_t nb) { return a < b + nb && b < a + na; }

// Workspace of the momentum pathway: the per-chunk partial sums (two 64 x 128
// float32 tiles each) and the chunk coefficients.
struct SsmMomPlan {
  int nchunks = 0;
  size_t off_part = 0, off_coef = 0, end = 0;
};
int plan_ssm_momentum(int m, int n, int r, long long nseq, int T, SsmMomPlan* p) {
  if (m <= 0 || n <= 0 || r <= 0 || nseq < 0 || T < 0) return MUON_EINVAL;
  if (r != 8 || m > 64 || n > 128) return MUON_EUNSUPPORTED;
  p->nchunks = (T + kSsmMomQ - 1) / kSsmMomQ;
  const long long wgs = nseq * p->nchunks;
  if (wgs > (1LL << 31) - 1 || nseq * m * n / 256 > (1LL << 31) - 1) return MUON_EUNSUPPORTED;
  size_t off = 0;
  p->off_part = off;
  off = align_up(off + static_cast<size_t>(wgs) * 2 * 64 * 128 * sizeof(float), kAlign);
  p->off_coef = off;
  off = align_up(off + static_cast<size_t>(wgs) * 4 * sizeof(float), kAlign);
  p->end = std::max<size_t>(off, kAlign);
  return MUON_OK;
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
  std::vector<GroupRun> runs;
  size_t need = 0;
  long long nparts = 0;
  if (prepare_step(groups, ngroups, cfg, &C, runs, &need, &nparts, false) != MUON_OK) return 0;
  return need;
}

int muon_step(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace,
              size_t workspace_bytes, float* norms_out, void* stream) {
  return step_impl(groups, ngroups, cfg, workspace, workspace_bytes, norms_out, stream, nullptr, 0);
}

int muon_step_phases(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, int* phases, int max_phases) {
  if (groups == nullptr || ngroups <= 0 || max_phases < 0 || (phases == nullptr && max_phases > 0))
    return MUON_EINVAL;
  NsCoefs C;
  std::vector<GroupRun> runs;
  size_t need = 0;
  long long nparts = 0;
  const int rc = prepare_step(groups, ngroups, cfg, &C, runs, &need, &nparts, false);
  if (rc != MUON_OK) return rc;
  const std::vector<int> marks = list_phases(runs, C, cfg->eps, nparts);
  const int n = static_cast<int>(marks.size()) - 1;
  for (int i = 0; i < n && i < max_phases; ++i) phases[i] = marks[i + 1];
  return n;
}

int muon_step_timed(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, void* workspace,
                    size_t workspace_bytes, float* norms_out, void* stream, void* const* events, int nevents) {
  if (events == nullptr) return MUON_EINVAL;
  return step_impl(groups, ngroups, cfg, workspace, workspace_bytes, norms_out, stream, events, nevents);
}

size_t muon_ns_workspace_size(int m, int n, int batch, int dtype, const muon_ns_cfg* cfg) {
  NsCoefs C;
  if (parse_cfg(cfg, &C, true) != MUON_OK || (dtype != MUON_F32 && dtype != MUON_BF16)) return 0;
  if (batch < 0) return 0;
  std::vector<GroupPlan> plans;
  size_t need = 0;
  long long nparts = 0;
  if (plan_groups({GroupShape{m, n, batch, false}}, dtype == MUON_BF16, C, plans, &need, &nparts) != MUON_OK)
    return 0;
  return need;
}

int muon_ns_orthogonalize(const void* G, void* O, int dtype, int m, int n, int ld, int batch, long long stride,
                          const muon_ns_cfg* cfg, void* workspace, size_t workspace_bytes, void* stream) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C, true);
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (cfg->precision != dtype) return MUON_EUNSUPPORTED;
  if (m <= 0 || n <= 0 || batch < 0 || ld < n) return MUON_EINVAL;
  const long long span = static_cast<long long>(m - 1) * ld + n;  // elements of one matrix's rows
  if (batch > 1 && stride < span) return MUON_EINVAL;
  std::vector<GroupRun> runs(1);
  GroupRun& R = runs[0];
  std::vector<GroupPlan> plans;
  size_t need = 0;
  long long nparts = 0;
  rc = plan_groups({GroupShape{m, n, batch, false}}, dtype == MUON_BF16, C, plans, &need, &nparts);
  if (rc != MUON_OK) return rc;
  if (batch == 0) return MUON_OK;
  const size_t es = dtype_size(dtype);
  if (G == nullptr || O == nullptr || !aligned_to(G, es) || !aligned_to(O, es)) return MUON_EINVAL;
  const size_t bytes = (static_cast<size_t>(batch - 1) * (batch > 1 ? stride : 0) + span) * es;
  const char* gb = static_cast<const char*>(G);
  char* ob = static_cast<char*>(O);
  // in place (O == G) is allowed: every element of G is read by the first pass, before any write of O
  if (ob != gb && ob < gb + bytes && gb < ob + bytes) return MUON_EINVAL;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return MUON_EWORKSPACE;
  R.plan = plans[0];
  R.g_own.resize(batch);
  R.o_own.resize(batch);
  for (int b = 0; b < batch; ++b) {
    R.g_own[b] = gb + static_cast<size_t>(b) * stride * es;
    R.o_own[b] = ob + static_cast<size_t>(b) * stride * es;
  }
  R.grad_dtype = dtype;
  R.G = R.g_own.data();
  R.O = R.o_own.data();
  R.ldg = ld;
  R.ldo = ld;
  EventRec E;
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return run_all(runs, C, cfg->eps, ws, nullptr, st, E, nullptr, nparts);
}

}  // extern "C"

namespace {
// Workspace of muon_ns_orthogonalize_noalloc: one array per GPU, held by the
// loaded code object until the process ends.  Host code never uses its name
// as an address (that is a host-side stand-in): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kNoAllocBytes];

char* scratch_for_current_device(int* status) {
  static std::mutex mu;
  static char* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *status = MUON_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *status = MUON_EHIP;
      return nullptr;
    }
    ptrs[dev] = static_cast<char*>(p);
  }
  *status = MUON_OK;
  return ptrs[dev];
}
}  // namespace

extern "C" {

size_t muon_ns_noalloc_max_bytes(void) { return kNoAllocBytes; }

int muon_ns_orthogonalize_noalloc(const void* G, void* O, int dtype, int m, int n, int ld, int batch,
                                  long long stride, const muon_ns_cfg* cfg, void* stream) {
  // every argument check of muon_ns_orthogonalize first (without a workspace
  // it validates, then stops at MUON_EWORKSPACE before any launch), so that
  // errors do not depend on the scratch array
  const int rc = muon_ns_orthogonalize(G, O, dtype, m, n, ld, batch, stride, cfg, nullptr, 0, stream);
  if (rc != MUON_EWORKSPACE) return rc;  // a validation error, or nothing to do
  if (muon_ns_workspace_size(m, n, batch, dtype, cfg) > kNoAllocBytes) return MUON_EWORKSPACE;
  int st = MUON_OK;
  char* ws = scratch_for_current_device(&st);
  if (ws == nullptr) return st;
  return muon_ns_orthogonalize(G, O, dtype, m, n, ld, batch, stride, cfg, ws, kNoAllocBytes, stream);
}

int muon_query_flags(const void* workspace, int* nonfinite_out) {
  if (workspace == nullptr || nonfinite_out == nullptr || !aligned16(workspace)) return MUON_EINVAL;
  unsigned f = 0;
  if (hipMemcpy(&f, workspace, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess) return MUON_EHIP;
  *nonfinite_out = f != 0u ? 1 : 0;
  return MUON_OK;
}

int muon_adamw(int ntensors, float* const* params, const void* const* grads, float* const* exp_avg,
               float* const* exp_avg_sq, const long long* numel, int grad_dtype, float lr, float beta1, float beta2,
               float eps, float weight_decay, long long step, void* stream) {
  if (ntensors < 0) return MUON_EINVAL;
  if (ntensors == 0) return MUON_OK;
  if (params == nullptr || grads == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr || numel == nullptr)
    return MUON_EINVAL;
  if (grad_dtype != MUON_F32 && grad_dtype != MUON_BF16) return MUON_EINVAL;
  if (!std::isfinite(lr) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps >= 0.0f) ||
      !std::isfinite(eps) || !std::isfinite(weight_decay) || step < 1)
    return MUON_EINVAL;
  for (int i = 0; i < ntensors; ++i) {
    if (numel[i] < 0) return MUON_EINVAL;
    if (numel[i] >= (1LL << 31)) return MUON_EUNSUPPORTED;
    if (numel[i] == 0) continue;
    if (params[i] == nullptr || grads[i] == nullptr || exp_avg[i] == nullptr || exp_avg_sq[i] == nullptr)
      return MUON_EINVAL;
    if (!aligned_to(params[i], 4) || !aligned_to(exp_avg[i], 4) || !aligned_to(exp_avg_sq[i], 4) ||
        !aligned_to(grads[i], dtype_size(grad_dtype)))
      return MUON_EINVAL;
  }
  AdamwLaunch A{};
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step));
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step));
  A.beta1 = beta1; A.beta2 = beta2;
  A.one_m_b1 = 1.0f - beta1; A.one_m_b2 = 1.0f - beta2;
  A.eps = eps;
  A.decay = 1.0f - lr * weight_decay;
  A.lr_bc = static_cast<float>(lr / bc1);
  A.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = grad_dtype == MUON_BF16;
  // launches of up to kAdamwMax tensors (the table travels in the kernel arguments)
  std::vector<AdamwLaunch> chunks;
  std::vector<long long> chunk_blocks;
  long long blocks = 0;
  for (int i = 0; i < ntensors; ++i) {
    if (numel[i] == 0) continue;
    const long long nb = (numel[i] + kAdamwBlock - 1) / kAdamwBlock;
    if (A.nt == kAdamwMax || blocks + nb > (1LL << 30)) {  // block indices stay in int
      chunks.push_back(A);
      chunk_blocks.push_back(blocks);
      A.nt = 0;
      blocks = 0;
    }
    AdamwTensor& T = A.t[A.nt++];
    T.p = params[i]; T.m = exp_avg[i]; T.v = exp_avg_sq[i]; T.g = grads[i];
    T.n = static_cast<int>(numel[i]);
    T.block0 = static_cast<int>(blocks);
    blocks += nb;
  }
  if (A.nt > 0) {
    chunks.push_back(A);
    chunk_blocks.push_back(blocks);
  }
  auto run = [&](size_t c, hipStream_t s) {
    return launch_adamw(chunks[c], bf16, static_cast<int>(chunk_blocks[c]), s) == hipSuccess;
  };
  Aux* aux = chunks.size() > 1 ? aux_for_current_device() : nullptr;
  if (aux == nullptr) {
    for (size_t c = 0; c < chunks.size(); ++c)
      if (!run(c, st)) return MUON_EHIP;
    return MUON_OK;
  }
  // The tensors are independent: the chunk with the most work runs on the
  // caller's stream while the others (typically the many small tensors, which
  // alone would leave most of the chip idle) run beside it on the auxiliary
  // stream, joined back before returning.
  size_t big = 0;
  for (size_t c = 1; c < chunks.size(); ++c)
    if (chunk_blocks[c] > chunk_blocks[big]) big = c;
  std::lock_guard<std::mutex> lock(aux->mu);
  if (hipEventRecord(aux->fork, st) != hipSuccess || hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
    return MUON_EHIP;
  bool ok = run(big, st);
  for (size_t c = 0; ok && c < chunks.size(); ++c)
    if (c != big) ok = run(c, aux->s);
  // join even after a failed launch, so that the caller's stream never runs ahead of the auxiliary work
  if (hipEventRecord(aux->join, aux->s) != hipSuccess || hipStreamWaitEvent(st, aux->join, 0) != hipSuccess)
    return MUON_EHIP;
  return ok ? MUON_OK : MUON_EHIP;
}

int muon_ns_factored(const void* V, const void* K, int dtype, int m, int n, int r, long long batch,
                     const muon_ns_cfg* cfg, float* C_out, void* O_out, void* stream) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C, true);
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (m <= 0 || n <= 0 || r <= 0 || batch < 0) return MUON_EINVAL;
  if (dtype != MUON_BF16 || cfg->precision != MUON_BF16) return MUON_EUNSUPPORTED;
  FactLaunch F{};
  rc = factored_launch(m, n, r, batch, C, cfg->eps, O_out != nullptr, &F);
  if (rc != MUON_OK) return rc;
  if (batch == 0) return MUON_OK;
  if (V == nullptr || K == nullptr || C_out == nullptr || !aligned_to(V, 2) || !aligned_to(K, 2) ||
      !aligned_to(C_out, 4) || (O_out != nullptr && !aligned16(O_out)))
    return MUON_EINVAL;
  const char* vb = static_cast<const char*>(V);
  const char* kb = static_cast<const char*>(K);
  const char* cb = reinterpret_cast<const char*>(C_out);
  const size_t vbytes = static_cast<size_t>(batch) * m * r * 2, kbytes = static_cast<size_t>(batch) * n * r * 2;
  const size_t cbytes = static_cast<size_t>(batch) * r * r * 4;
  if (overlaps(cb, cbytes, vb, vbytes) || overlaps(cb, cbytes, kb, kbytes)) return MUON_EINVAL;
  if (O_out != nullptr) {
    const char* ob = static_cast<const char*>(O_out);
    const size_t obytes = static_cast<size_t>(batch) * m * n * 2;
    if (overlaps(ob, obytes, vb, vbytes) || overlaps(ob, obytes, kb, kbytes) || overlaps(ob, obytes, cb, cbytes))
      return MUON_EINVAL;
  }
  F.V = static_cast<const bf16_t*>(V);
  F.K = static_cast<const bf16_t*>(K);
  F.C = C_out;
  F.O = static_cast<bf16_t*>(O_out);
  F.vec = r == 8 && aligned16(V) && aligned16(K);
  return launch_ns_factored(F, static_cast<hipStream_t>(stream)) == hipSuccess ? MUON_OK : MUON_EHIP;
}

size_t muon_ssm_momentum_workspace_size(int m, int n, int r, long long nseq, int T) {
  SsmMomPlan p;
  return plan_ssm_momentum(m, n, r, nseq, T, &p) == MUON_OK ? p.end : 0;
}

int muon_ssm_momentum_timed(const void* V, const void* K, int dtype, int m, int n, int r, long long nseq, int T,
                            float beta, const float* decay, float* M, float* S, const muon_ns_cfg* cfg,
                            void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C, true);
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (dtype != MUON_BF16 || cfg->precision != MUON_BF16) return MUON_EUNSUPPORTED;
  SsmMomPlan p;
  rc = plan_ssm_momentum(m, n, r, nseq, T, &p);
  if (rc != MUON_OK) return rc;
  if (!std::isfinite(beta)) return MUON_EINVAL;
  if (events != nullptr && nevents < 3) return MUON_EINVAL;
  if (nseq == 0 || T == 0) return MUON_OK;
  if (V == nullptr || K == nullptr || M == nullptr || !aligned16(V) || !aligned16(K) || !aligned_to(M, 4) ||
      (S != nullptr && (decay == nullptr || !aligned_to(S, 4) || !aligned_to(decay, 4))))
    return MUON_EINVAL;
  const size_t tokens = static_cast<size_t>(nseq) * T;
  const size_t sbytes = static_cast<size_t>(nseq) * m * n * 4;
  const char* vb = static_cast<const char*>(V);
  const char* kb = static_cast<const char*>(K);
  const char* mb = reinterpret_cast<const char*>(M);
  const size_t vbytes = tokens * m * r * 2, kbytes = tokens * n * r * 2;
  if (overlaps(mb, sbytes, vb, vbytes) || overlaps(mb, sbytes, kb, kbytes)) return MUON_EINVAL;
  if (S != nullptr) {
    const char* sb = reinterpret_cast<const char*>(S);
    const char* db = reinterpret_cast<const char*>(decay);
    if (overlaps(sb, sbytes, vb, vbytes) || overlaps(sb, sbytes, kb, kbytes) || overlaps(sb, sbytes, mb, sbytes) ||
        overlaps(sb, sbytes, db, tokens * 4) || overlaps(mb, sbytes, db, tokens * 4))
      return MUON_EINVAL;
  }
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < p.end) return MUON_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  for (const auto& b : {std::make_pair(vb, vbytes), std::make_pair(kb, kbytes), std::make_pair(mb, sbytes)})
    if (overlaps(ws, p.end, b.first, b.second)) return MUON_EINVAL;
  if (S != nullptr && (overlaps(ws, p.end, reinterpret_cast<const char*>(S), sbytes) ||
                       overlaps(ws, p.end, reinterpret_cast<const char*>(decay), tokens * 4)))
    return MUON_EINVAL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  EventRec E;
  E.ev = events;
  E.n = nevents;
  if (!E.mark(st, 0)) return MUON_EHIP;
  // 1. every token's Newton-Schulz core and the per-chunk partial sums,
  // 2. the chunk maps applied in token order
  SsmMomLaunch L{};
  L.V = static_cast<const bf16_t*>(V);
  L.K = static_cast<const bf16_t*>(K);
  L.a = S != nullptr ? decay : nullptr;
  L.beta = beta;
  L.m = m; L.n = n; L.T = T; L.Q = kSsmMomQ; L.nchunks = p.nchunks;
  L.nseq = nseq;
  L.part = reinterpret_cast<float*>(ws + p.off_part);
  L.coef = reinterpret_cast<float*>(ws + p.off_coef);
  L.M = M;
  L.S = S;
  L.ns.m_pad = 64; L.ns.n_pad = 128; L.ns.r = r;
  L.ns.steps = C.steps;
  L.ns.eps = cfg->eps;
  for (int k = 0; k < C.steps; ++k) { L.ns.a[k] = C.a[k]; L.ns.b[k] = C.b[k]; L.ns.c[k] = C.c[k]; }
  if (launch_ssm_momentum(L, st, 0) != hipSuccess || !E.mark(st, 0)) return MUON_EHIP;
  if (launch_ssm_momentum(L, st, 1) != hipSuccess || !E.mark(st, 0)) return MUON_EHIP;
  return MUON_OK;
}

int muon_ssm_momentum(const void* V, const void* K, int dtype, int m, int n, int r, long long nseq, int T, float beta,
                      const float* decay, float* M, float* S, const muon_ns_cfg* cfg, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return muon_ssm_momentum_timed(V, K, dtype, m, n, r, nseq, T, beta, decay, M, S, cfg, workspace,
                                 workspace_bytes, stream, nullptr, 0);
}

size_t muon_spectral_diag_workspace_size(int m, int n, long long batch, int dtype, int iters) {
  DiagPlan p;
  if (plan_diag(m, n, batch, dtype, iters, &p) != MUON_OK) return 0;
  return batch == 0 ? kAlign : p.end;
}

int muon_spectral_diag_timed(const void* A, int dtype, int m, int n, long long batch, int iters, float* orth_err,
                             float* sigma_max, float* sigma_min, void* workspace, size_t workspace_bytes,
                             void* stream, void** events, int nevents) {
  DiagPlan p;
  const int rc = plan_diag(m, n, batch, dtype, iters, &p);
  if (rc != MUON_OK) return rc;
  if (batch == 0 || (orth_err == nullptr && sigma_max == nullptr && sigma_min == nullptr)) return MUON_OK;
  const long long chunks = (batch + p.chunk - 1) / p.chunk;
  if (events != nullptr && nevents < 1 + 3 * chunks) return MUON_EINVAL;
  const size_t es = dtype_size(dtype);
  if (A == nullptr || !aligned_to(A, es)) return MUON_EINVAL;
  const char* ab = static_cast<const char*>(A);
  const size_t abytes = static_cast<size_t>(batch) * m * n * es;
  for (float* o : {orth_err, sigma_max, sigma_min}) {
    if (o == nullptr) continue;
    const char* ob = reinterpret_cast<const char*>(o);
    if (!aligned_to(o, 4) || (ob < ab + abytes && ab < ob + static_cast<size_t>(batch) * 4)) return MUON_EINVAL;
  }
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < p.end) return MUON_EWORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  bf16_t* L = reinterpret_cast<bf16_t*>(ws + p.off_l);
  float* H = reinterpret_cast<float*>(ws + p.off_h);
  float* Q = reinterpret_cast<float*>(ws + p.off_q);
  int ev = 0;
  auto mark = [&]() {
    return events == nullptr || hipEventRecord(static_cast<hipEvent_t>(events[ev++]), st) == hipSuccess;
  };
  if (!mark()) return MUON_EHIP;
  for (long long c0 = 0; c0 < batch; c0 += p.chunk) {
    const long long cnt = std::min(p.chunk, batch - c0);
    DiagPackLaunch P{};
    P.A = ab + static_cast<size_t>(c0) * m * n * es;
    P.astride = static_cast<long long>(m) * n;
    P.n = n; P.s = p.s; P.l = p.l;
    P.tall = p.tall; P.f32 = p.f32;
    P.L = L;
    P.ostride = static_cast<long long>(p.op_bytes / 2);
    P.s_pad = p.s_pad; P.kdim = p.kdim; P.ld = p.ld;
    P.count = cnt;
    DiagLaunch D{};
    D.H = H;
    D.hstride = static_cast<long long>(p.h_bytes / 4);
    D.Q = Q;
    D.qstride = static_cast<long long>(p.q_bytes / 4);
    D.s = p.s; D.s_pad = p.s_pad; D.iters = iters; D.kmax = p.k;
    D.orth = orth_err ? orth_err + c0 : nullptr;
    D.smax = sigma_max ? sigma_max + c0 : nullptr;
    D.smin = sigma_min ? sigma_min + c0 : nullptr;
    D.count = cnt;
    P.clr_words = diag_split_clear_words(D);
    P.clr = P.clr_words > 0 ? reinterpret_cast<unsigned*>(Q) : nullptr;
    P.cstride = D.qstride;
    if (launch_diag_pack(P, st) != hipSuccess || !mark()) return MUON_EHIP;
    SymArgs G{};
    SymSeg& S = G.seg[0];
    G.nseg = 1;
    S.L = L;
    S.R = L;
    S.F = H;
    S.stride = static_cast<long long>(p.h_bytes / 4);
    S.in_stride = P.ostride;
    S.ld = p.ld;
    if (p.f32) {  // six segments over the pieces [h | d | e]: hh + hd + dh + dd + he + eh
      S.kdim = 6 * p.kdim;
      S.kseg = p.kdim;
      S.lmap = 0x201100u;  // segments 0..5 of L: h h d d h e
      S.rmap = 0x021010u;  // segments 0..5 of R: h d h d e h
    } else {
      S.kdim = p.kdim;
    }
    S.s_pad = p.s_pad;
    S.count = static_cast<int>(cnt);
    S.tiles_per_mat = symprod_tiles_per_matrix(p.s_pad);
    S.a1 = 0.0f; S.b1 = 1.0f;
    if (launch_symprod_bf16(G, st) != hipSuccess || !mark()) return MUON_EHIP;
    if (launch_diag_lanczos(D, st) != hipSuccess || !mark()) return MUON_EHIP;
  }
  return MUON_OK;
}

int muon_spectral_diag(const void* A, int dtype, int m, int n, long long batch, int iters, float* orth_err,
                       float* sigma_max, float* sigma_min, void* workspace, size_t workspace_bytes, void* stream) {
  return muon_spectral_diag_timed(A, dtype, m, n, batch, iters, orth_err, sigma_max, sigma_min, workspace,
                                  workspace_bytes, stream, nullptr, 0);
}

int muon_ns_batched_small(const void* X, void* Y, int dtype, int m, int n, long long batch, const muon_ns_cfg* cfg,
                          void* stream) {
  NsCoefs C;
  int rc = parse_cfg(cfg, &C);  // quintic not on the on-chip kernels
  if (rc != MUON_OK) return rc;
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_EINVAL;
  if (cfg->precision != dtype) return MUON_EUNSUPPORTED;
  if (m <= 0 || n <= 0 || batch < 0) return MUON_EINVAL;
  const bool bf16 = dtype == MUON_BF16;
  const bool tall = m > n;
  const int s = tall ? n : m, l = tall ? m : n;
  if (bf16 && (tall || s % 32 != 0 || l % 32 != 0)) return MUON_EUNSUPPORTED;
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
