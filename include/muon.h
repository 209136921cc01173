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
 * workspace; the library never allocates device memory.  Its only state is,
 * per device, one auxiliary stream and two events created on first use by
 * muon_step (see muon_ns_cfg.streams) or muon_adamw.  All work is ordered on `stream` (a
 * hipStream_t; NULL is the null stream): work placed on the auxiliary stream
 * starts after everything enqueued on `stream` before the call and finishes
 * before anything enqueued on `stream` after it.  Calls return without
 * synchronising; a kernel fault surfaces at the caller's next
 * synchronisation.  Host pointer arrays are read during the call only.  Two
 * calls that share a workspace must be ordered on one stream.
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

#define MUON_VERSION 9

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

typedef enum {
  MUON_OK = 0,
  MUON_EINVAL = -1,       /* bad argument: null pointer, bad size, misaligned, bad dtype */
  MUON_EUNSUPPORTED = -2, /* valid but not implemented for this shape / precision */
  MUON_EWORKSPACE = -3,   /* workspace pointer null or smaller than the size query */
  MUON_EHIP = -4          /* the HIP runtime refused a launch */
} muon_status;

/* Newton-Schulz schedule of large bfloat16 matrices (the result is the same
 * polynomial of X0 either way; rounding differs).
 *   MUON_NS_ITERATE     per step A = X X^T, then X = (a I + b A) X: two
 *                       products of s x l work each
 *   MUON_NS_ACCUMULATE  every iterate is Q X0 with Q a polynomial in
 *                       A_0 = X0 X0^T, so with B_k = a_k I + b_k A_k:
 *                       A_{k+1} = A_k B_k^2 (= X_{k+1} X_{k+1}^T),
 *                       Q = B_{steps-1} ... B_1 B_0, O = Q X0; one Gram, one
 *                       final product, and 3 (steps - 1) symmetric s x s
 *                       products; less work when l > s
 *   MUON_NS_AUTO        per shape group, whichever needs fewer matrix-core
 *                       operations (ACCUMULATE needs steps >= 2)
 * float32 and small (on-chip) matrices always iterate. */
typedef enum { MUON_NS_AUTO = 0, MUON_NS_ITERATE = 1, MUON_NS_ACCUMULATE = 2 } muon_ns_schedule;

/* Newton-Schulz settings.
 *   steps     number of iterations, 0..64 (0: O is the normalised U)
 *   ncoef     2 (cubic: a, b) or 3 (quintic: a, b, c)
 *   coeffs    host array: ncoef values, or steps * ncoef values when per_step
 *   per_step  0: one (a, b[, c]) for every step; 1: one row per step
 *   eps       added to ||U||_F before dividing (>= 0)
 *   precision MUON_BF16 or MUON_F32 (see Precision above)
 *   schedule  a muon_ns_schedule
 *   streams   muon_step only: 0 runs independent shape groups as two chains,
 *             on `stream` and on an auxiliary stream the library creates per
 *             device on first use (joined back into `stream` before the call
 *             returns); 1 uses `stream` alone.  muon_step_timed always uses
 *             `stream` alone.
 *   separate_apply  0: the final matrix product of a large bfloat16 group
 *             also applies the update (W -= lr scale O from the bf16-rounded
 *             product, and the copy to O) in its epilogue, so the update is
 *             never stored and re-read; groups with the spectral cap, or
 *             beyond 64 matrices in one launch, keep a separate pass.  1:
 *             always a separate apply pass.  The results are bitwise equal.
 * Quintic c != 0 runs on bfloat16 matrices of every shape (on the
 * matrix-core path, one more s x s product per step; small matrices then take
 * that path instead of the on-chip kernel) and in muon_ns_factored; with
 * float32 precision and in muon_ns_batched_small it returns
 * MUON_EUNSUPPORTED. */
typedef struct {
  int steps;
  int ncoef;
  const float* coeffs;
  int per_step;
  float eps;
  int precision;
  int schedule;
  int streams;
  int separate_apply;
} muon_ns_cfg;

/* One parameter group of `count` same-shape m x n matrices (the pages group
 * Muon's parameters by projection; here a group is a shape).
 *   W, M       host arrays of `count` device pointers to float32 m x n
 *   G          host array of `count` device pointers to m x n gradients of
 *              grad_dtype (MUON_BF16 or MUON_F32)
 *   O          NULL, or a host array of `count` device pointers receiving the
 *              orthogonalised update, m x n in the precision of the cfg
 *              (after the spectral cap when it acts)
 *   lr, beta, scale, nesterov   as in the formulas above
 * Spectral cap ("An Isotropy-Preserving Spectral Cap for Muon": remove the
 * update direction that grows the weight's top singular value, keep the
 * rest).  cap_u NULL: off.  Otherwise, per matrix, with caller-initialised
 * estimates u (unit, float32[m]) and v (unit, float32[n]) of W's top singular
 * vectors and sigma of its top singular value:
 *   c = u^T O v;  if sigma >= cap and c < 0:  O = O - c u v^T
 *   W = W - lr * scale * O
 *   u = W v / ||W v||,  v = W^T u / ||W^T u||,  sigma = ||W v||   (old u, v on
 *   the right; a zero product keeps its vector)
 * so u, v, sigma track W's top pair by one power step per update.
 *   cap_u, cap_v  host arrays of count device pointers to float32[m], [n],
 *                 read and updated in place
 *   cap_sigma     device float32[count], read and updated
 *   cap           threshold (<= 0: the cap may act at every step)
 * Requires W.  Zero-initialised fields (cap_u NULL) leave the cap off. */
typedef struct {
  int m, n, count;
  int grad_dtype;
  float* const* W;
  float* const* M;
  const void* const* G;
  void* const* O;
  float lr, beta, scale;
  int nesterov;
  float* const* cap_u;
  float* const* cap_v;
  float* cap_sigma;
  float cap;
} muon_group;

/* Sizes.  m * n <= 2^31 per matrix; on the matrix-core path (bfloat16, not
 * small) also s_pad * ld * 2 < 2^31 bytes, where s_pad is min(m, n) and ld is
 * max(m, n), each rounded up to a multiple of 256 (one padded iterate below
 * 2 GiB: e.g. 16384 x 65280 is accepted, 16384 x 65536 is not); beyond either
 * bound muon_step, its size queries and muon_step_phases return
 * MUON_EUNSUPPORTED (muon_step_workspace_size: 0). */

/* Bytes of device workspace muon_step needs for these groups (0 on invalid
 * arguments). */
size_t muon_step_workspace_size(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg);

/* One Muon step over every matrix of every group: momentum (M in place),
 * Newton-Schulz orthogonalisation, and W -= lr * scale * O (W in place).
 * norms_out: NULL, or a device float array with one slot per matrix (groups in
 * order, matrices in order) receiving ||U||_F.  The workspace (at least the
 * size query's bytes, 16-byte aligned) holds the iterates and, in its first
 * bytes, the non-finite flag of the step (muon_query_flags). */
int muon_step(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg,
              void* workspace, size_t workspace_bytes, float* norms_out, void* stream);

/* Phases of muon_step's launch schedule, for labelling measurements. */
typedef enum {
  MUON_PHASE_MOMENTUM = 1,    /* momentum pass of one group */
  MUON_PHASE_NS_SMALL = 2,    /* on-chip Newton-Schulz of one group of small matrices */
  MUON_PHASE_GRAM = 3,        /* grouped Gram launch (large bf16 matrices) */
  MUON_PHASE_COMBINE = 4,     /* grouped combine launch (large bf16 matrices) */
  MUON_PHASE_SYMPROD = 5,     /* grouped symmetric s x s products (accumulated schedule) */
  MUON_PHASE_APPLY = 6,       /* apply pass of one group */
  MUON_PHASE_F32_GRAM = 7,    /* Gram of one float32 group */
  MUON_PHASE_F32_COMBINE = 8, /* combine of one float32 group */
  MUON_PHASE_CAP = 9,         /* spectral-cap coefficient u^T O v of one group */
  MUON_PHASE_POWER = 10,      /* power step on one group's updated weights */
  MUON_PHASE_COMBINE_APPLY = 11, /* final grouped combine with the apply fused (large bf16 matrices) */
  MUON_PHASE_FLAGS = 12       /* the call's non-finite flag (see muon_query_flags) */
} muon_phase;

/* The phases muon_step would run for these groups and cfg, in order: returns
 * their number n (or a negative muon_status) and writes the first
 * min(n, max_phases) of them to phases (may be NULL when max_phases is 0).
 * Only shapes, counts, dtypes and cfg are read; no GPU work. */
int muon_step_phases(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg, int* phases,
                     int max_phases);

/* muon_step for measurement: identical work, and it records caller-created
 * hipEvent_t handles (`events`, host array) on `stream`: one at the start and
 * one at the end of every phase listed by muon_step_phases, so nevents must be
 * at least that count + 1 (MUON_EINVAL otherwise).  Elapsed times between
 * consecutive events give each phase's GPU duration. */
int muon_step_timed(const muon_group* groups, int ngroups, const muon_ns_cfg* cfg,
                    void* workspace, size_t workspace_bytes, float* norms_out, void* stream,
                    void* const* events, int nevents);

/* Bytes of device workspace muon_ns_orthogonalize needs (independent of ld
 * and stride). */
size_t muon_ns_workspace_size(int m, int n, int batch, int dtype, const muon_ns_cfg* cfg);

/* Newton-Schulz only ("Muon Meets Mamba", abstract: the orthogonalisation of
 * one weight update), without momentum or apply: O[b] = NS(G[b]) for b <
 * batch.  Matrix b of G starts at element b * stride of G, its rows are ld
 * elements apart (ld >= n; stride >= (m - 1) * ld + n when batch > 1); O uses
 * the same ld and stride.  G and O have element type `dtype`; the iteration
 * runs in cfg->precision, which must equal dtype (MUON_EUNSUPPORTED
 * otherwise).  O may be G itself (in place: every element of G is read before
 * any element of O is written); otherwise the two must not overlap
 * (MUON_EINVAL).  Rows with ld % 8 == 0 and 16-byte aligned matrices take
 * vectorised paths.  Also sets the workspace's non-finite flag (see
 * muon_query_flags). */
int muon_ns_orthogonalize(const void* G, void* O, int dtype, int m, int n, int ld, int batch,
                          long long stride, const muon_ns_cfg* cfg, void* workspace,
                          size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * muon_ns_orthogonalize without a workspace argument.  Its workspace is a
 * library-owned device array of muon_ns_noalloc_max_bytes() bytes (32 MiB),
 * one per GPU, part of the loaded library and held until the process ends;
 * the call allocates nothing (no hipMalloc or hipFree; the array's device
 * address is looked up once per device).  Arguments, results and errors as in
 * muon_ns_orthogonalize, plus MUON_EWORKSPACE when muon_ns_workspace_size for
 * these arguments exceeds the array.  Nothing in the array needs to start at
 * zero; the last call's contents stay in it (its non-finite flag among them,
 * which muon_query_flags cannot reach).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (concurrent streams,
 * other threads) race and must be ordered by the caller. */
size_t muon_ns_noalloc_max_bytes(void);
int muon_ns_orthogonalize_noalloc(const void* G, void* O, int dtype, int m, int n, int ld, int batch,
                                  long long stride, const muon_ns_cfg* cfg, void* stream);

/* The non-finite flag of the last muon_step or muon_ns_orthogonalize call that
 * used this workspace ("Muon Meets Mamba" practitioner article, long-term
 * engineering and the training checkpoints: stop and alert on abnormal
 * gradient norms, check for NaN).  The call computes ||U||_F^2 of every
 * matrix's update direction U from per-block partial sums; the flag is 1 when
 * any of those sums is not finite (a NaN or Inf in G or M, or an overflow),
 * else 0.  The flag lives in the first bytes of the workspace and is written
 * by a kernel that the call enqueues on `stream` (with two concurrent chains,
 * after the first chain's work, once the second chain's momentum passes are
 * done), so read it only after that stream has been synchronised (this
 * function copies 4 bytes device -> host with hipMemcpy).  A call with no
 * matrices leaves it unchanged.
 *   workspace     the workspace passed to that call (16-byte aligned)
 *   nonfinite_out host int receiving 0 or 1
 * Returns MUON_EINVAL on null or misaligned pointers, MUON_EHIP if the copy
 * fails. */
int muon_query_flags(const void* workspace, int* nonfinite_out);

/* Newton-Schulz on a large batch of small matrices (MuonSSM's per-token,
 * per-head injections), each held on chip for the whole iteration:
 * Y[b] = NS(X[b]) for a contiguous [batch][m][n] stack, no workspace.
 * Supported: MUON_BF16 with min(m, n) in {32, 64, 96, 128}, max(m, n) a
 * multiple of 32 up to 512, m <= n; MUON_F32 with min(m, n) <= 64 and
 * max(m, n) <= 256.  Other shapes return MUON_EUNSUPPORTED.  Y must not
 * overlap X.  (muon_step and muon_ns_orthogonalize send bfloat16 groups with
 * these short sides and any long side up to 512 to the same kernels.) */
int muon_ns_batched_small(const void* X, void* Y, int dtype, int m, int n, long long batch,
                          const muon_ns_cfg* cfg, void* stream);

/* Newton-Schulz of matrices given as factors, X[b] = V[b] K[b]^T ("MuonSSM",
 * method section: each per-token, per-head injection is a sum of r
 * value-key outer products, orthogonalised by a light Newton-Schulz step).
 * Every step keeps the form V C K^T, so only an r x r core is computed:
 *   P = V^T V, S = K^T K, C_0 = I / (sqrt(tr(P S)) + eps),
 *   per step N = C S C^T P, C = a C + b N C + c N N C     (c from cfg, may be != 0)
 * giving NS(X[b]) = V[b] C_out[b] K[b]^T exactly up to rounding (the same
 * result as muon_ns_orthogonalize on the dense X; C is unique when V and K
 * have full column rank).
 *   V      [batch][m][r] bfloat16, row-major, contiguous
 *   K      [batch][n][r] bfloat16
 *   C_out  [batch][r][r] float32 (written)
 *   O_out  NULL, or [batch][m][n] bfloat16 receiving the dense V C K^T
 *          (16-byte aligned, n % 8 == 0)
 * dtype and cfg->precision must be MUON_BF16 (P and S on the matrix cores
 * with float32 accumulation, the core recurrence in float32).  Supported:
 * 1 <= r <= 8, m, n <= 256 (with O_out also (m16 + n16) * 64 + m16 * 128 +
 * 6144 <= 65536 bytes, m16 = m rounded up to 16); otherwise
 * MUON_EUNSUPPORTED.  Outputs must not overlap inputs or each other. */
int muon_ns_factored(const void* V, const void* K, int dtype, int m, int n, int r, long long batch,
                     const muon_ns_cfg* cfg, float* C_out, void* O_out, void* stream);

/* The momentum pathway of MuonSSM over sequences of factored injections
 * ("MuonSSM", method section on the momentum-augmented state update, and the
 * theory section's parallelism paragraph: a momentum state M_t beside the
 * memory state S_t accumulates the conditioned injections; the pair follows
 * a block-affine recurrence).  The pages give no equation; the reading
 * implemented is heavy-ball momentum on the memory.  For every sequence and
 * token t = 1..T, with X_t = V_t K_t^T:
 *   U_t = NS(X_t)                      (cfg: steps, coefficients, eps)
 *   M_t = beta M_{t-1} + U_t
 *   S_t = a_t S_{t-1} + M_t            (only when S is given)
 * and (M, S) are replaced by (M_T, S_T).  U_t is formed in factored form,
 * V_t C_t K_t^T with an r x r core (as muon_ns_factored), and never stored
 * densely; a long sequence may be processed in consecutive calls (the states
 * carry over exactly up to rounding).
 *   V      [nseq][T][m][r] bfloat16, contiguous, 16-byte aligned
 *   K      [nseq][T][n][r] bfloat16, contiguous, 16-byte aligned
 *   beta   momentum coefficient (finite)
 *   decay  [nseq][T] float32 per-token decays a_t; read only when S != NULL
 *   M      [nseq][m][n] float32, in/out
 *   S      NULL, or [nseq][m][n] float32, in/out
 * dtype and cfg->precision must be MUON_BF16 (cores as in muon_ns_factored;
 * the rank-r products accumulate in float32 from bf16 operands scaled by each
 * token's weight).  Supported: r == 8, m <= 64, n <= 128; otherwise
 * MUON_EUNSUPPORTED.  M, S, decay, the factors and the workspace must not
 * overlap.  nseq == 0 or T == 0 leaves the states unchanged.  The workspace
 * (muon_ssm_momentum_workspace_size bytes, 16-byte aligned) holds the
 * per-chunk partial sums (two 64 x 128 float32 tiles per 256 tokens of a
 * sequence); muon_query_flags does not apply to it. */
size_t muon_ssm_momentum_workspace_size(int m, int n, int r, long long nseq, int T);
int muon_ssm_momentum(const void* V, const void* K, int dtype, int m, int n, int r, long long nseq, int T,
                      float beta, const float* decay, float* M, float* S, const muon_ns_cfg* cfg,
                      void* workspace, size_t workspace_bytes, void* stream);
/* muon_ssm_momentum for measurement: records three caller-created hipEvent_t
 * handles on `stream` (nevents >= 3): before the fused pass (every token's
 * core and the per-chunk partial sums), after it and after the in-order
 * combine. */
int muon_ssm_momentum_timed(const void* V, const void* K, int dtype, int m, int n, int r, long long nseq, int T,
                            float beta, const float* decay, float* M, float* S, const muon_ns_cfg* cfg,
                            void* workspace, size_t workspace_bytes, void* stream, void** events, int nevents);

/* AdamW for the parameters outside the Muon groups ("Muon Meets Mamba":
 * AdamW is the baseline optimizer and keeps the non-projection parameters),
 * with decoupled weight decay and bias-corrected moments; for each tensor i
 * and element, with t = step (from 1):
 *   m = beta1 m + (1 - beta1) g,   v = beta2 v + (1 - beta2) g^2
 *   p = p (1 - lr weight_decay) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *   params, exp_avg, exp_avg_sq  host arrays of ntensors device pointers to
 *                                float32 (p, m, v updated in place)
 *   grads                         host array of device pointers (grad_dtype)
 *   numel                         host array of element counts (0: skipped)
 * Tensors are contiguous; 16-byte aligned tensors take vectorised loads.
 * 0 <= beta < 1, eps >= 0, step >= 1 (MUON_EINVAL otherwise); a tensor of
 * 2^31 or more elements returns MUON_EUNSUPPORTED.  One launch per 80 tensors
 * (the tensor table travels in the kernel arguments); with more than one, the
 * launch with the most work runs on `stream` and the others beside it on the
 * auxiliary stream.  No workspace. */
int muon_adamw(int ntensors, float* const* params, const void* const* grads, float* const* exp_avg,
               float* const* exp_avg_sq, const long long* numel, int grad_dtype, float lr, float beta1,
               float beta2, float eps, float weight_decay, long long step, void* stream);

/* Bytes of device workspace muon_spectral_diag needs (0 for invalid or
 * unsupported arguments).  Matrices are processed in chunks whose scratch
 * stays within 2 GiB, so the size stops growing with batch beyond one chunk. */
size_t muon_spectral_diag_workspace_size(int m, int n, long long batch, int dtype, int iters);

/* Spectral diagnostics of a stack of matrices: the "Muon Meets Mamba"
 * practitioner article (training checkpoints; long-term engineering) asks
 * for the largest singular value of each weight or state matrix every few
 * steps, checked against a threshold, and for singular values in the training
 * log; the orthogonality error tells how far an orthogonalised update is from
 * orthogonal.  For A[b] (m x n), X its short-side orientation (s x l, X = A
 * or A^T) and H = X X^T:
 *   orth_err[b]   ||H - I_s||_F / sqrt(s)
 *   sigma_max[b]  sqrt(theta_max), sigma_min[b] = sqrt(max(theta_min, 0)),
 *                 theta the extreme Ritz values of min(iters, s) Lanczos steps
 *                 on H with full reorthogonalisation (two classical
 *                 Gram-Schmidt passes) from the start vector
 *                 q_i = t_i / 2^24 - 1/2, t_i the top 24 bits of
 *                 (i * 2654435769) mod 2^32, normalised; the run ends early
 *                 when the residual beta_{j+1} <= 2^-20 ||H q_j|| (an
 *                 invariant Krylov space) or is not finite.  With
 *                 iters >= s these are the extreme singular values; with
 *                 fewer they lie inside [sigma_min, sigma_max] of A.
 *   A      [batch][m][n] contiguous, dtype MUON_BF16 or MUON_F32 (finite
 *          float32 values below 2^127 are split exactly into three bfloat16
 *          pieces; the six products above 2^-24 relative are kept, so H has
 *          float32 accuracy)
 *   orth_err, sigma_max, sigma_min  device float[batch] each, or NULL (not
 *          computed); none may overlap A.  All NULL: nothing is done.
 * H is formed on the matrix cores (float32 accumulation), the Lanczos run is
 * float32, the tridiagonal extremes float64.  Supported: min(m, n) <= 4096,
 * max(m, n) <= 2^22, 1 <= iters <= 512 (larger: MUON_EUNSUPPORTED; iters < 1:
 * MUON_EINVAL).  A NaN or Inf in A[b] gives NaN outputs for b.
 * When one workgroup per matrix would leave most compute units idle, the
 * Lanczos pass runs as one cooperative launch with several workgroups per
 * matrix that exchange partial products through the workspace (their waits
 * are bounded: a matrix whose workgroups ever gave up waiting gets NaN
 * outputs); if the device refuses that launch, one workgroup per matrix is
 * used.  Debug only, for tests of that give-up path: the environment
 * variable MUON_DEBUG_DIAG_SPIN_LIMIT (read at each launch; it can only lower
 * the bound) cuts the number of polls of those waits.  Deterministic for a given device (the split depends on its compute
 * unit count); no allocation; asynchronous on `stream`; calls that share a
 * workspace must not overlap. */
int muon_spectral_diag(const void* A, int dtype, int m, int n, long long batch, int iters, float* orth_err,
                       float* sigma_max, float* sigma_min, void* workspace, size_t workspace_bytes,
                       void* stream);

/* muon_spectral_diag that also records HIP events on `stream`: events[0]
 * before the first launch, then one after each of the three passes (pack,
 * Gram, Lanczos) of every chunk; nevents must be at least 1 + 3 * chunks
 * (chunks = 1 whenever the workspace size for `batch` is below 2 GiB), else
 * MUON_EINVAL.  Events are created by the caller (hipEvent_t). */
int muon_spectral_diag_timed(const void* A, int dtype, int m, int n, long long batch, int iters, float* orth_err,
                             float* sigma_max, float* sigma_min, void* workspace, size_t workspace_bytes,
                             void* stream, void** events, int nevents);

/* Human-readable name of a muon_status. */
const char* muon_status_string(int status);

/* MUON_VERSION of the built library. */
int muon_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMUON_MUON_H */
