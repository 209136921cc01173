// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.cuh"

namespace muon {

// Fused momentum / Nesterov / Frobenius-partials pass (one launch covers up to
// kMaxTable matrices of one shape group).
struct MomentumLaunch {
  PtrTable G;          // user gradients (m x n)
  MutPtrTable M;       // user momentum (m x n, float), entries may be null: U = G
  void* X;             // oriented iterate of the first matrix, s_pad x ld
  long long xstride;   // elements between consecutive matrices of X
  int m, n, s_pad, ld, count, P;
  int ldg;             // row stride of G (elements, >= n); M is contiguous (n)
  bool tall, grad_bf16, x_bf16;
  float beta;
  int nesterov;
  float* partials;     // [count][P] sums of squares
};

struct ApplyLaunch {
  const void* X;       // final iterate (oriented), s_pad x ld
  long long xstride;
  int m, n, ld, count;
  int ldo;             // row stride of O (elements, >= n); W is contiguous (n)
  bool tall, x_bf16;
  MutPtrTable W;       // entries may be null (no apply)
  MutPtrTable O;       // entries may be null (no copy-out); element type = X's
  const float* partials;  // non-null: scale by 1/(nu+eps) (zero Newton-Schulz steps)
  int P;
  float eps;
  float neg_lr_scale;
  // spectral cap (cap_part null: none): O <- O - gamma u v^T with
  // c = sum of the cap_P partials, gamma = c if sigma >= cap and c < 0, else 0
  const float* cap_part;
  int cap_P;
  const float* cap_sigma;
  float cap;
  PtrTable cu, cv;     // u (m floats), v (n floats) per matrix
};

// Spectral cap: partials of u^T O v over the oriented final iterate.
struct CapCoefLaunch {
  const void* X;       // [count][s_pad][ld], bf16 or float
  long long xstride;
  int s, l, ld, count;
  bool tall;           // X = O^T
  PtrTable u, v;       // float[m], float[n] per matrix
  float* part;         // [count][P]
  int P;
};
int cap_coef_blocks(int s);
hipError_t launch_cap_coef(const CapCoefLaunch& L, bool x_bf16, hipStream_t st);

// One simultaneous power step on the updated weights.
struct PowerLaunch {
  PtrTable W;          // float m x n per matrix
  MutPtrTable u, v;    // in: current estimates; out: the next ones
  float* sigma;        // [count]: ||W v||
  float* ybuf;         // [count][m]   W v
  float* zbuf;         // [count][n]   W^T u
  float* zpart;        // [count][nrc][n] partials of W^T u over row blocks
  float* ynorm;        // [count][nrc] partial sums of (W v)_r^2
  float* znorm;        // [count][ncb] partial sums of (W^T u)_j^2
  int m, n, count, nrc, ncb;
};
int power_row_blocks(int m);
int power_col_blocks(int n);
hipError_t launch_power_step(const PowerLaunch& L, hipStream_t st);

// One batched Newton-Schulz GEMM over `count` matrices of one shape, laid out
// contiguously: X [count][s_pad][ld], A [count][s_pad][s_pad].
struct NsGemmLaunch {
  const void* X;       // iterate in
  void* Y;             // iterate out (combine only)
  void* A;             // Gram matrix (out for gram, in for combine)
  long long xstride, astride;
  int s_pad, ld, count;
  // step-1 normalisation folded into the epilogues: when partials is non-null
  // the Gram scales by inv^2 and the combine multiplies alpha, beta by inv,
  // with inv = 1 / (sqrt(sum of partials) + eps).
  const float* partials;
  int P;
  float eps;
  float alpha, beta;   // combine coefficients (a, b)
};

int momentum_blocks_per_matrix(bool tall, int s_pad, int ld);
hipError_t launch_momentum(const MomentumLaunch& L, hipStream_t st);
hipError_t launch_apply(const ApplyLaunch& L, hipStream_t st);
hipError_t launch_norms(const float* partials, int P, int count, float* out, hipStream_t st);
// flag = 1 if any of the n partial sums of squares is not finite, else 0
// (one workgroup; a plain store)
hipError_t launch_flags(const float* partials, long long n, unsigned* flag, hipStream_t st);

// bf16 matrix-core path.  One launch covers up to kMaxSeg shape groups
// (segments) of one Newton-Schulz step.
constexpr int kTileS = 256;   // s_pad multiple for the bf16 tiled path
constexpr int kTileL = 256;   // ld multiple for the bf16 tiled path
constexpr int kMaxSeg = 4;
struct GemmSeg {
  const bf16_t* X;     // iterate in  [count][s_pad][ld]
  bf16_t* Y;           // iterate out (combine)
  bf16_t* A;           // Gram out 1 / combine's left operand  [count][s_pad][s_pad]
  bf16_t* A2;          // Gram out 2 (null: none)
  long long xstride, astride;
  int s_pad, ld, kdim, count, tiles_per_mat;
  // Gram outputs: A = a inv^pa I + b inv^pb X X^T and A2 = a2 I + b2 A (from
  // A's rounded values), inv = 1 / (sqrt(sum of partials) + eps), or 1 when
  // partials is null.
  const float* partials;
  int P;
  float eps;
  float a, b, a2, b2;
  int pa, pb;
  // Combine with the apply fused (the final product of the iteration): Y is
  // not written; with o the bf16 rounding of the result at (i, k) of the
  // oriented iterate (i < s, k < l), matrix z of the segment updates
  // W = GemmArgs.W[tab0 + z] (m x n float32, entry (i, k) wide, (k, i) tall)
  // to fmaf(neg_lr_scale, o, W) and stores o to GemmArgs.O[tab0 + z]
  // (m x n bf16); null table entries skip that output.
  int fuse;
  int tab0, m, n, s, l, tall;
  float neg_lr_scale;
};
struct GemmArgs {
  GemmSeg seg[kMaxSeg];
  int nseg;
  MutPtrTable W, O;    // fused apply: per-matrix outputs of the segments
};
int combine_tiles_per_matrix(int s_pad, int ld);
hipError_t launch_combine_bf16(const GemmArgs& G, hipStream_t st);

// Products L R^T whose result is symmetric: the Gram X X^T (L = R = X, the
// iterate), and products of two symmetric, commuting s_pad x s_pad bf16
// matrices (polynomials in the same Gram matrix, where R^T = R):
// O1 = a1 inv^pa I + b1 inv^pb L R and (optional) O2 = a2 I + b2 O1 from
// O1's rounded values.  Only tiles on or above the diagonal are computed;
// each is stored in place and mirrored.
struct SymSeg {
  const bf16_t* L;     // left factor   [count][s_pad][ld], contraction over kdim columns
  const bf16_t* R;     // right factor  (may equal L)
  bf16_t* O1;          // [count][s_pad][s_pad]
  bf16_t* O2;          // null: none
  long long stride;    // elements between consecutive outputs
  long long in_stride; // elements between consecutive operands
  int ld, kdim;        // operand row stride; contraction length (multiple of 32)
  int s_pad, count, tiles_per_mat;
  const float* partials;
  int P;
  float eps;
  float a1, b1, a2, b2;
  int pa, pb;
  int zip_next;        // 1: the next segment has the same count and s_pad and
                       // runs matrix by matrix together with this one
  int tile;            // 0: symprod_tile(s_pad); else 128 or 192 (dividing s_pad)
  float* F;            // non-null: O1 = a1 inv^pa I + b1 inv^pb L R as float32 here
                       // [count][s_pad][s_pad] (stride), exactly symmetric; O1, O2 unused
  int tri_in;          // 1: L and R hold only their upper block triangle (tile-sized
                       // blocks on and above the diagonal); the others are read transposed
  int tri_out;         // 1: O1 and O2 get only their upper block triangle
  int kseg;            // float32-output runs: > 0 splits the contraction into kdim / kseg
                       // segments of kseg columns; segment g of L reads columns
                       // [lmap_g kseg, (lmap_g + 1) kseg) of the rows, of R those of
                       // rmap_g (4 bits per segment); 0: the columns in order
  unsigned lmap, rmap;
};
struct SymArgs {
  SymSeg seg[kMaxSeg];
  int nseg;
};
int symprod_tile(int s_pad);  // 192 when it divides s_pad, else 128
int symprod_tiles_per_matrix(int s_pad, int tile = 0);
hipError_t launch_symprod_bf16(const SymArgs& G, hipStream_t st);

// float32 path (tile multiples: s_pad % 64 == 0, ld % 64 == 0).
constexpr int kTileF32 = 64;
hipError_t launch_gram_f32(const NsGemmLaunch& L, hipStream_t st);
hipError_t launch_combine_f32(const NsGemmLaunch& L, hipStream_t st);

// Whole Newton-Schulz on chip for small matrices.
struct NsSmallLaunch {
  const void* X;       // [count] matrices, row stride ld_in
  void* Y;             // [count] matrices, row stride ld_out
  long long in_stride, out_stride;
  int s, l, ld_in, ld_out;
  long long count;
  bool transposed;     // X stored as l x s (tall); the kernel orients it
  int steps;
  float a[64], b[64];  // per-step coefficients (passed by value)
  const float* partials;  // non-null: nu from the momentum pass partials
  int P;
  float eps;
};
bool ns_small_supported(bool bf16, int s, int l);
hipError_t launch_ns_small(const NsSmallLaunch& L, bool bf16, hipStream_t st);

// Newton-Schulz of factored matrices X = V K^T (bf16 factors, r <= 8): the
// r x r core and optionally the dense result.
struct FactLaunch {
  const bf16_t* V;     // [batch][m][r]
  const bf16_t* K;     // [batch][n][r]
  float* C;            // [batch][r][r], or null
  bf16_t* O;           // [batch][m][n] or null
  long long batch;
  int m, n, r, m_pad, n_pad;  // pads: multiples of 16
  int vec;             // r == 8 and 16-byte aligned factors: 16-byte row loads
  int waves;           // wavefronts per workgroup
  int per_wave, f_off; // LDS bytes per wavefront; offset of the r x r work matrices in it
  int steps;
  float eps;
  float a[64], b[64], c[64];
};
int factored_lds_per_wave(int m_pad, int n_pad, bool dense, int* f_off = nullptr);
hipError_t launch_ns_factored(const FactLaunch& F, hipStream_t st);

// Padded sides, rank and Newton-Schulz coefficients of a factored core.
struct FactCoreArgs {
  int m_pad, n_pad, r, steps;
  float eps;
  float a[64], b[64], c[64];
};

// Momentum pathway over sequences of factored injections (ssm_momentum.hip):
// one workgroup per (sequence, chunk of kSsmMomQ tokens) forms the NS cores
// of the chunk's tokens and the chunk's float32 partial sums; then the chunk
// maps are applied in token order to the caller's states.
constexpr int kSsmMomQ = 256;
struct SsmMomLaunch {
  const bf16_t* V;     // [nseq][T][m][8]
  const bf16_t* K;     // [nseq][T][n][8]
  const float* a;      // [nseq][T] decays (with S), else null
  float beta;
  int m, n, T, Q, nchunks;  // m <= 64, n <= 128, Q tokens per chunk
  long long nseq;
  float* part;         // [nseq][nchunks][1 or 2][64][128] partial sums
  float* coef;         // [nseq][nchunks][4]: beta^L, prod a, B, 0
  float* M;            // [nseq][m][n] in/out
  float* S;            // null, or [nseq][m][n] in/out
  FactCoreArgs ns;     // m_pad 64, n_pad 128, r 8
};
// phase 0: cores and partial sums; phase 1: combine into M (and S)
hipError_t launch_ssm_momentum(const SsmMomLaunch& P, hipStream_t st, int phase);

// Spectral diagnostics (a chunk of `count` matrices per launch).
struct DiagPackLaunch {
  const void* A;       // [count][m][n], float32 or bf16 (f32)
  long long astride;   // m * n
  int n, s, l;         // row stride of A; short and long side
  bool tall, f32;
  bf16_t* L;           // [count][s_pad][ld] operand rows: X, or for float32 inputs its
                       // three bf16 pieces side by side [h | d | e]
  long long ostride;   // s_pad * ld
  int s_pad, kdim, ld; // s_pad % 128 == 0, kdim % 64 == 0, ld = kdim (bf16) or 3 kdim
  long long count;
  unsigned* clr;       // split run: the first clr_words words of each matrix's scratch
  long long cstride;   //   (stride cstride) are zeroed; or null
  long long clr_words;
};
hipError_t launch_diag_pack(const DiagPackLaunch& P, hipStream_t st);
struct DiagLaunch {
  const float* H;      // [count][s_pad][s_pad] Gram matrices (exactly symmetric)
  long long hstride;
  float* Q;            // [count][kmax][s_pad] Lanczos basis, or the split run's scratch
  long long qstride;
  int s, s_pad, iters, kmax;
  int split_p, split_r, split_nb;  // split run (set by the planner): blocks per side, row ranges, workgroups
  unsigned spin_limit;             // split run: polls before a wait is given up (set by the launcher)
  float* orth;         // [count] or null
  float* smax;         // [count] or null
  float* smin;         // [count] or null
  long long count;
};
size_t diag_lanczos_lds(int s_pad, int kmax);
// Plans the launch (split run or one workgroup per matrix); returns the
// 32-bit words of each matrix's scratch to zero beforehand (0: none).
long long diag_split_clear_words(DiagLaunch& D);
hipError_t launch_diag_lanczos(const DiagLaunch& D, hipStream_t st);

// AdamW over a list of float32 tensors (one launch: up to kAdamwMax tensors).
constexpr int kAdamwMax = 80;      // 40 bytes each: the table fits the kernel arguments
constexpr int kAdamwBlock = 4096;  // elements per workgroup
struct AdamwTensor {
  float* p;
  float* m;
  float* v;
  const void* g;       // float32 or bf16
  int n;               // elements (< 2^31)
  int block0;          // first workgroup of this tensor
};
struct AdamwLaunch {
  AdamwTensor t[kAdamwMax];
  int nt;
  float beta1, beta2, one_m_b1, one_m_b2, eps;
  float decay;         // 1 - lr * weight_decay
  float lr_bc;         // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
};
hipError_t launch_adamw(const AdamwLaunch& A, bool grad_bf16, int blocks, hipStream_t st);

}  // namespace muon
