/*
 * libmuon -- the Muon update on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; no C++ or framework types cross it.
 *
 * What the library computes
 * -------------------------
 * "Muon Meets Mamba: Spectral Optimization for State Space Models" (arXiv
 * 2608.03941, abstract): Muon orthogonalises the update of each weight matrix
 * with a Newton-Schulz iteration, i.e. steepest descent under the spectral
 * norm, and the paper applies it per weight group (input projection, output
 * projection or both) of Mamba-2 130M.  "MuonSSM: Orthogonalizing State Space
 * Models for Sequence Modeling" (ICML 2026; method section on light
 * Newton-Schulz orthogonalisation, and the ablation on the number of
 * Newton-Schulz steps) runs a single Newton-Schulz step, without SVD, on the
 * low-rank value-key injections of every token and head.
 *
 * The pages fix neither the polynomial nor the normalisation nor the momentum
 * rule; the readings implemented here (all numbers passed in by the caller):
 *
 *   M' = beta * M + G                                  (momentum, in place)
 *   U  = G + beta * M'   (nesterov)   or   U = M'
 *   X  = U, or U^T when m > n, so X is s x l with s = min(m, n)
 *   X0 = X / (||X||_F + eps)
 *   repeat steps times:  A = X X^T;  X = a X + b A X (+ c A A X)
 *   O  = X, or X^T when m > n
 *   W  = W - lr * scale * O                            (in place)
 *
 * Precision.  MUON_BF16: U is rounded to bfloat16, the Gram and combine
 * products run on the matrix cores with bfloat16 inputs and float32
 * accumulation, the iterate and A are stored as bfloat16, the epilogues are
 * float32.  MUON_F32: everything in float32.  M and W are always float32.
 *
 * Layout.  Every matrix is row-major, contiguous, m rows of n elements
 * (PyTorch's (out, in) layout for a Linear weight).  Device pointers must be
 * aligned to their element size (muon_ns_batched_small with bfloat16: 16
 * bytes); 16-byte aligned matrices with n % 8 == 0 take vectorised paths.
 * bfloat16 data is passed as 16-bit storage (uint16 bits).
 *
 * Ownership and asynchrony.  The caller owns every buffer, including the
 * workspace; the library never allocates device memory and keeps no state
 * between calls.  All work is enqueued on `stream` (a hipStream_t; NULL is
 * the null stream) and the call returns without synchronising; a kernel fault
 * surfaces at the caller's next synchronisation.  Host pointer arrays are read
 * during the call only.  Two calls that share a workspace must be ordered on
 * one stream.
 *
 * Errors.  Every entry point validates all arguments before enqueueing any
 * work and returns MUON_OK (0) or a negative muon_status; nothing has been
 * enqueued when a validation error is returned.  MUON_EHIP reports a failed
 * kernel launch (work enqueued before it is not rolled back).
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_VERSION 1

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

typedef enum {
  MUON_OK = 0,
  MUON_EINVAL = -1,       /* bad argument: null pointer, bad size, misaligned, bad dtype */
  MUON_EUNSUPPORTED = -2, /* valid but not implemented for this shape / precision */
  MUON_EWORKSPACE = -3,   /* workspace pointer null or smaller than the size query */
  MUON_EHIP = -4          /* the HIP runtime refused a launch */
} muon_status;

/* Newton-Schulz settings.
 *   steps     number of iterations, 0..64 (0: O is the normalised U)
 *   ncoef     2 (cubic: a, b) or 3 (quintic: a, b, c)
 *   coeffs    host array: ncoef values, or steps * ncoef values when per_step
 *   per_step  0: one (a, b[, c]) for every step; 1: one row per step
 *   eps       added to ||U||_F before dividing (>= 0)
 *   precision MUON_BF16 or MUON_F32 (see Precision above)
 * A quintic c != 0 returns MUON_EUNSUPPORTED on the GPU path. */
typedef struct {
  int steps;
  int ncoef;
  const float* coeffs;
  int per_step;
  float eps;
  int precision;
} muon_ns_cfg;

/* One parameter group of `count` same-shape m x n matrices (the pages group
 * Muon's parameters by projection; here a group is a shape).
 *   W, M       host arrays of `count` device pointers to float32 m x n
 *   G          host array of `count` device pointers to m x n gradients of
 *              grad_dtype (MUON_BF16 or MUON_F32)
 *   O          NULL, or a host array of `count` device pointers receiving the
 *              orthogonalised update, m x n in the precision of the cfg
 *   lr, beta, scale, nesterov   as in the formulas above */
typedef struct {
  int m, n, count;
  int grad_dtype;
  float* const* W;
  float* const* M;
  const void* const* G;
  void* const* O;
  float lr, beta, scale;
  int nesterov;
} muon_group;

/* Bytes of device workspace muon_step needs for these groups (0 on invalid
 * arguments). */
size_t muon_step_workspace_size(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg);

/* One Muon step over every matrix of every group: momentum (M in place),
 * Newton-Schulz orthogonalisation, and W -= lr * scale * O (W in place).
 * norms_out: NULL, or a device float array with one slot per matrix (groups in
 * order, matrices in order) receiving ||U||_F. */
int muon_step(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg,
              void* workspace, size_t workspace_bytes, float* norms_out, void* stream);

/* muon_step for measurement: identical work, and it records caller-created
 * hipEvent_t handles (`events`, host array) on `stream` at the boundaries of
 * the launch schedule, per group with count > 0, in order:
 *   start, after the momentum pass,
 *   then after every Gram launch and every combine launch (large matrices,
 *   2 * steps events) or after the on-chip Newton-Schulz launch (small
 *   matrices, 1 event; none when steps == 0),
 *   after the apply pass.
 * nevents must cover all groups (MUON_EINVAL otherwise).  Elapsed times
 * between consecutive events give per-kernel GPU durations. */
int muon_step_timed(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg,
                    void* workspace, size_t workspace_bytes, float* norms_out, void* stream,
                    void* const* events, int nevents);

/* Bytes of device workspace muon_ns_orthogonalize needs. */
size_t muon_ns_workspace_size(int m, int n, int batch, int dtype, const muon_ns_cfg* cfg);

/* Newton-Schulz only: O[b] = NS(G[b]) for a contiguous [batch][m][n] stack.
 * G and O have element type `dtype`; the iteration runs in cfg->precision,
 * which must equal dtype.  O must not overlap G. */
int muon_ns_orthogonalize(const void* G, void* O, int dtype, int m, int n, int batch,
                          const muon_ns_cfg* cfg, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Newton-Schulz on a large batch of small matrices (MuonSSM's per-token,
 * per-head injections), each held on chip for the whole iteration:
 * Y[b] = NS(X[b]) for a contiguous [batch][m][n] stack, no workspace.
 * Supported: MUON_BF16 with min(m, n) in {32, 64}, max(m, n) a multiple of 32
 * up to 256, m <= n; MUON_F32 with min(m, n) <= 64 and max(m, n) <= 256.
 * Other shapes return MUON_EUNSUPPORTED.  Y must not overlap X. */
int muon_ns_batched_small(const void* X, void* Y, int dtype, int m, int n, long long batch,
                          const muon_ns_cfg* cfg, void* stream);

/* Human-readable name of a muon_status. */
const char* muon_status_string(int status);

/* MUON_VERSION of the built library. */
int muon_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMUON_MUON_H */
