"""fp64 CPU oracle for the Muon update and its Newton-Schulz orthogonalisation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never calls it
and shares no code with it; it consumes the same seeded input bits and nothing
else.

What is computed, and where it comes from
-----------------------------------------
"Muon Meets Mamba: Spectral Optimization for State Space Models" (arXiv
2608.03941, abstract): Muon orthogonalises the update of every weight matrix
with a Newton-Schulz iteration, which amounts to steepest descent under the
spectral norm.  "MuonSSM: Orthogonalizing State Space Models" (ICML 2026,
method section "Newton-Schulz 轻量正交化") applies a light, single-step
Newton-Schulz transform, with no explicit SVD, to low-rank value-key
injections; its ablation ("Newton-Schulz 迭代次数") compares one step with
five.  "An Isotropy-Preserving Spectral Cap for Muon" calls the same operation
Muon's matrix-sign step.

The pages leave the following open; the readings taken here are the plain ones
(each is also listed in the design notes):

* polynomial: odd polynomial p(x) = a x + b x^3 (+ c x^5), coefficients passed
  in; the cubic (a, b) = (1.5, -0.5) is the default.  In matrix form one step
  is X <- a X + b (X X^T) X + c (X X^T)(X X^T) X.
* normalisation before the iteration: Frobenius, X0 = U / (||U||_F + eps), so
  that every singular value of X0 is at most 1.
* optimizer momentum (not stated on the pages): heavy-ball without dampening,
  M' = beta M + G, with the Nesterov look-ahead U = G + beta M' (or U = M').
* update: W' = W - lr * scale * O, O the orthogonalised update.
* orientation: a tall matrix (m > n) is iterated as its transpose, so the Gram
  matrix is formed on the short side; mathematically this is the same result.

Everything runs in float64 with numpy; matrix products use numpy's matmul as a
library primitive, with no blocking, fusion or reordering beyond the steps
above.
"""
from __future__ import annotations

import numpy as np

CUBIC = (1.5, -0.5)
DEFAULT_EPS = 1e-7


# ----------------------------------------------------------------------------
# Exact widening of stored inputs
# ----------------------------------------------------------------------------
def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bfloat16 number is the upper half of an IEEE binary32 number, so shifting
    the 16 bits into the top of a 32-bit word gives the binary32 value exactly.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def widen_f32(x: np.ndarray) -> np.ndarray:
    """binary32 values -> exact float64 values."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Step 1-2: momentum buffer and the update direction
# ----------------------------------------------------------------------------
def momentum(M: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """New momentum buffer M' = beta * M + G (heavy-ball, no dampening)."""
    return beta * M + G


def update_direction(G: np.ndarray, M_new: np.ndarray, beta: float, nesterov: bool) -> np.ndarray:
    """Direction fed to the orthogonalisation: G + beta * M' (Nesterov) or M'."""
    return G + beta * M_new if nesterov else M_new


# ----------------------------------------------------------------------------
# Step 3-6: Newton-Schulz orthogonalisation of one matrix
# ----------------------------------------------------------------------------
def frobenius_normalize(X: np.ndarray, eps: float):
    """X0 = X / (||X||_F + eps); returns (X0, nu) with nu = ||X||_F."""
    nu = float(np.sqrt(np.sum(X * X)))
    return X / (nu + eps), nu


def step_coefficients(coeffs, steps: int, per_step: bool):
    """List of (a, b, c) for every step; c = 0 for the cubic polynomial."""
    c = np.asarray(coeffs, dtype=np.float64).ravel()
    if per_step:
        k = c.size // steps if steps else 0
        rows = [c[i * k:(i + 1) * k] for i in range(steps)]
    else:
        rows = [c] * steps
    out = []
    for r in rows:
        if r.size == 2:
            out.append((float(r[0]), float(r[1]), 0.0))
        elif r.size == 3:
            out.append((float(r[0]), float(r[1]), float(r[2])))
        else:
            raise ValueError("each step needs 2 (cubic) or 3 (quintic) coefficients")
    return out


def ns_iterate(X: np.ndarray, steps: int, coeffs=CUBIC, per_step: bool = False) -> np.ndarray:
    """Run `steps` Newton-Schulz steps on an already normalised s x l matrix X.

    One step: A = X X^T (full s x s product), then
    X <- a X + b (A X) + c (A (A X)).
    """
    for a, b, c in step_coefficients(coeffs, steps, per_step):
        A = X @ X.T
        AX = A @ X
        Xn = a * X + b * AX
        if c != 0.0:
            Xn = Xn + c * (A @ AX)
        X = Xn
    return X


def newton_schulz(U: np.ndarray, steps: int, coeffs=CUBIC, eps: float = DEFAULT_EPS,
                  per_step: bool = False):
    """Orthogonalise one m x n matrix; returns (O, nu).

    The short side is made the row side (transpose when m > n), the matrix is
    Frobenius-normalised, iterated, and transposed back.
    """
    U = np.asarray(U, dtype=np.float64)
    tall = U.shape[0] > U.shape[1]
    X = U.T if tall else U
    X, nu = frobenius_normalize(X, eps)
    X = ns_iterate(X, steps, coeffs, per_step)
    return (X.T if tall else X), nu


def ns_batched(X: np.ndarray, steps: int, coeffs=CUBIC, eps: float = DEFAULT_EPS,
               per_step: bool = False) -> np.ndarray:
    """Newton-Schulz on every matrix of a [batch, m, n] stack independently."""
    X = np.asarray(X, dtype=np.float64)
    out = np.empty_like(X)
    for i in range(X.shape[0]):
        out[i], _ = newton_schulz(X[i], steps, coeffs, eps, per_step)
    return out


# ----------------------------------------------------------------------------
# Step 7: the whole optimizer step for one matrix
# ----------------------------------------------------------------------------
def muon_step(W, M, G, *, beta: float, lr: float, nesterov: bool = True, steps: int = 5,
              coeffs=CUBIC, eps: float = DEFAULT_EPS, scale: float = 1.0, per_step: bool = False):
    """One Muon step on one weight matrix.

    Returns a dict with the new weight W', the new momentum M', the update O and
    nu = ||U||_F of the direction before normalisation.
    """
    W = np.asarray(W, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M_new = momentum(M, G, beta)
    U = update_direction(G, M_new, beta, nesterov)
    O, nu = newton_schulz(U, steps, coeffs, eps, per_step)
    W_new = W - lr * scale * O
    return {"W": W_new, "M": M_new, "O": O, "nu": nu, "U": U}


# ----------------------------------------------------------------------------
# Factored injections: X = V K^T (MuonSSM, method section on the low-rank
# value-key injections and their light Newton-Schulz step)
# ----------------------------------------------------------------------------
def factored_ns(V: np.ndarray, K: np.ndarray, steps: int, coeffs=CUBIC, eps: float = DEFAULT_EPS,
                per_step: bool = False):
    """Newton-Schulz of the injection X = V K^T (V m x r, K n x r), returned
    both dense and as the r x r core C with O = V C K^T.

    The dense result is the plain definition, newton_schulz(V K^T).  The core
    is the unique C reproducing it when V and K have full column rank:
    C = V^+ O (K^+)^T with the Moore-Penrose pseudo-inverses (LAPACK SVD
    through numpy).  Returns (O, C, nu)."""
    V = np.asarray(V, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    O, nu = newton_schulz(V @ K.T, steps, coeffs, eps, per_step)
    C = np.linalg.pinv(V) @ O @ np.linalg.pinv(K).T
    return O, C, nu


# ----------------------------------------------------------------------------
# Momentum pathway (MuonSSM, method section on the momentum-augmented state
# update, and the parallelism paragraph of its theory section): a momentum
# state M_t, beside the memory state S_t, accumulates the conditioned
# injections, and the pair follows a block-affine recurrence.  The pages give
# no equation; the reading taken is heavy-ball momentum on the memory:
#   U_t = NS(V_t K_t^T)                 (the light Newton-Schulz step above)
#   M_t = beta M_{t-1} + U_t
#   S_t = a_t S_{t-1} + M_t             (a_t the backbone's per-token decay)
# i.e. [S_t; M_t] = [[a_t, beta], [0, beta]] [S_{t-1}; M_{t-1}] + [U_t; U_t].
# ----------------------------------------------------------------------------
def momentum_recurrence(U, a, beta: float, M0: np.ndarray, S0=None):
    """Run the pair recurrence over the updates U[t] (t = 0..T-1, each m x n)
    from (S0, M0); a[t] is the decay of token t (unused when S0 is None).
    Returns (M_T, S_T) (S_T None when S0 is None)."""
    M = np.array(M0, dtype=np.float64)
    S = None if S0 is None else np.array(S0, dtype=np.float64)
    for t in range(len(U)):
        M = beta * M + np.asarray(U[t], dtype=np.float64)
        if S is not None:
            S = float(a[t]) * S + M
    return M, S


def ssm_momentum(V, K, a, beta: float, M0, S0=None, steps: int = 1, coeffs=CUBIC, eps: float = DEFAULT_EPS,
                 per_step: bool = False):
    """The momentum pathway over one sequence of factored injections:
    V [T, m, r], K [T, n, r] (token t's injection X_t = V[t] K[t]^T), decays
    a [T].  Each U_t is the dense Newton-Schulz result of X_t (newton_schulz
    above, the plain definition); then momentum_recurrence.  Returns
    (M_T, S_T)."""
    V = np.asarray(V, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    U = [newton_schulz(V[t] @ K[t].T, steps, coeffs, eps, per_step)[0] for t in range(V.shape[0])]
    return momentum_recurrence(U, a, beta, M0, S0)


# ----------------------------------------------------------------------------
# Spectral cap ("An Isotropy-Preserving Spectral Cap for Muon"): at each update
# remove the direction that contributes most, to first order, to the growth of
# the weight's top singular value; the other directions keep learning.  The
# page gives no formula; the reading taken: with W's top singular pair (u, v)
# and W' = W - lr * scale * O, sigma_1 moves by -lr * scale * u^T O v to first
# order, and only the u v^T component of O contributes.  When the estimate
# sigma of sigma_1(W) has reached the cap and u^T O v < 0 (sigma_1 would grow),
# that component is removed: O <- O - (u^T O v) u v^T.  The pair is tracked
# across steps by one simultaneous power step per update on the new weight.
# ----------------------------------------------------------------------------
def spectral_cap_update(O: np.ndarray, u: np.ndarray, v: np.ndarray, sigma: float, cap: float):
    """The capped update for one matrix given the current estimates u (m), v
    (n) of W's top singular vectors (unit norm) and sigma of its top singular
    value.  Returns (O', gamma) with O' = O - gamma u v^T."""
    O = np.asarray(O, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    c = float(u @ O @ v)
    gamma = c if (sigma >= cap and c < 0.0) else 0.0
    return O - gamma * np.outer(u, v), gamma


def power_step(W: np.ndarray, u: np.ndarray, v: np.ndarray):
    """One simultaneous power step on W: u' = W v / ||W v||, v' = W^T u /
    ||W^T u||, sigma' = ||W v||.  A zero product leaves that vector as it was."""
    W = np.asarray(W, dtype=np.float64)
    y, z = W @ np.asarray(v, dtype=np.float64), W.T @ np.asarray(u, dtype=np.float64)
    ny, nz = np.linalg.norm(y), np.linalg.norm(z)
    u2 = y / ny if ny > 0 else np.asarray(u, dtype=np.float64)
    v2 = z / nz if nz > 0 else np.asarray(v, dtype=np.float64)
    return u2, v2, float(ny)


def muon_step_capped(W, M, G, u, v, sigma, *, cap: float, beta: float, lr: float, nesterov: bool = True,
                     steps: int = 5, coeffs=CUBIC, eps: float = DEFAULT_EPS, scale: float = 1.0,
                     per_step: bool = False):
    """muon_step with the spectral cap: the NS update is capped with the
    incoming estimates, applied, and the estimates advance by one power step
    on the new weight.  Returns muon_step's dict plus gamma, u, v, sigma."""
    W = np.asarray(W, dtype=np.float64)
    M_new = momentum(np.asarray(M, dtype=np.float64), np.asarray(G, dtype=np.float64), beta)
    U = update_direction(np.asarray(G, dtype=np.float64), M_new, beta, nesterov)
    O, nu = newton_schulz(U, steps, coeffs, eps, per_step)
    O_cap, gamma = spectral_cap_update(O, u, v, sigma, cap)
    W_new = W - lr * scale * O_cap
    u2, v2, s2 = power_step(W_new, u, v)
    return {"W": W_new, "M": M_new, "O": O_cap, "O_uncapped": O, "nu": nu, "U": U, "gamma": gamma,
            "u": u2, "v": v2, "sigma": s2}


# ----------------------------------------------------------------------------
# Companion AdamW for the parameters that Muon does not take ("Muon Meets
# Mamba": AdamW is the baseline optimizer, and the parameters outside the
# Muon groups keep it).  The pages give no formula; the reading is AdamW with
# decoupled weight decay and bias-corrected moments.
# ----------------------------------------------------------------------------
def adamw_step(p, g, m, v, *, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
               step: int):
    """One AdamW step (step counts from 1):
    m' = b1 m + (1 - b1) g,  v' = b2 v + (1 - b2) g^2,
    p' = p (1 - lr wd) - lr (m' / (1 - b1^t)) / (sqrt(v' / (1 - b2^t)) + eps).
    Returns (p', m', v')."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m2 = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v2 = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    mhat = m2 / (1.0 - beta1 ** step)
    vhat = v2 / (1.0 - beta2 ** step)
    p2 = p * (1.0 - lr * weight_decay) - lr * mhat / (np.sqrt(vhat) + eps)
    return p2, m2, v2


# ----------------------------------------------------------------------------
# Diagnostics (reported, never part of the update)
# ----------------------------------------------------------------------------
def orthogonality_error(O: np.ndarray) -> float:
    """||X X^T - I_s||_F / sqrt(s) for the short-side orientation X of O."""
    O = np.asarray(O, dtype=np.float64)
    X = O.T if O.shape[0] > O.shape[1] else O
    s = X.shape[0]
    return float(np.linalg.norm(X @ X.T - np.eye(s)) / np.sqrt(s))


# ----------------------------------------------------------------------------
# Spectral diagnostics.  The first page (the "Muon Meets Mamba" practitioner
# article, its sections on long-term engineering and on the training
# checkpoints) asks that the largest singular value of each weight/state
# matrix be computed every few steps and checked against a safety threshold,
# and that singular values be logged.  It names no algorithm; the reading
# taken here: with X the short-side orientation of A (s x l) and H = X X^T,
# the extreme eigenvalues of H are estimated by `iters` Lanczos steps with
# full reorthogonalisation from a fixed start vector, and sigma = sqrt(theta).
# With iters >= s the Krylov space is the whole space and the estimates are
# the exact extreme singular values (up to rounding).
# ----------------------------------------------------------------------------
WEYL_STEP = 2654435769  # floor(2^32 / golden ratio), odd
LANCZOS_BREAKDOWN = 2.0 ** -20  # relative size of a residual taken as zero


def lanczos_start(s: int) -> np.ndarray:
    """Unnormalised start vector: entry i is t_i / 2^24 - 1/2 with t_i the top
    24 bits of (i * 2654435769) mod 2^32 (a Weyl sequence of the golden
    ratio); every entry is exact in binary32 and binary64."""
    i = np.arange(s, dtype=np.uint64)
    h = (i * np.uint64(WEYL_STEP)) % np.uint64(1 << 32)
    return (h >> np.uint64(8)).astype(np.float64) / float(1 << 24) - 0.5


def lanczos_extremes(H: np.ndarray, iters: int):
    """min(iters, order) Lanczos steps on the symmetric matrix H from the
    normalised lanczos_start vector:
        w = H q_j,  alpha_j = q_j^T w,  w -= alpha_j q_j + beta_j q_{j-1},
        w -= Q (Q^T w) twice (Q = [q_0 .. q_j], classical Gram-Schmidt, two
        passes),  beta_{j+1} = ||w||,  q_{j+1} = w / beta_{j+1};
    the run ends early when beta_{j+1} <= 2^-20 ||H q_j|| (the Krylov space is
    invariant to working accuracy: the residual left is rounding noise, and
    continuing from it would build a basis that is no longer orthogonal) or
    is not finite.
    Returns (theta_min, theta_max): the extreme eigenvalues of the tridiagonal
    T with the alphas on its diagonal and the betas beside it."""
    H = np.asarray(H, dtype=np.float64)
    s = H.shape[0]
    k = min(int(iters), s)
    Q = np.zeros((k, s))
    q = lanczos_start(s)
    q = q / np.linalg.norm(q)
    q_prev = np.zeros(s)
    beta = 0.0
    alphas, betas = [], []
    for j in range(k):
        Q[j] = q
        w = H @ q
        hq = float(np.linalg.norm(w))
        alpha = float(q @ w)
        w = w - alpha * q - beta * q_prev
        for _ in range(2):
            w = w - Q[:j + 1].T @ (Q[:j + 1] @ w)
        alphas.append(alpha)
        beta_next = float(np.linalg.norm(w))
        if j + 1 == k or not (beta_next > LANCZOS_BREAKDOWN * hq and np.isfinite(beta_next)):
            break
        betas.append(beta_next)
        q_prev, q, beta = q, w / beta_next, beta_next
    if not np.all(np.isfinite(alphas)):
        return float("nan"), float("nan")
    T = np.diag(alphas) + np.diag(betas, 1) + np.diag(betas, -1)
    ev = np.linalg.eigvalsh(T)
    return float(ev[0]), float(ev[-1])


def spectral_diagnostics(A: np.ndarray, iters: int) -> dict:
    """Per matrix: the orthogonality error ||X X^T - I_s||_F / sqrt(s) and the
    Lanczos estimates of the extreme eigenvalues of H = X X^T (theta) and of
    the extreme singular values sqrt(max(theta, 0))."""
    A = np.asarray(A, dtype=np.float64)
    X = A.T if A.shape[0] > A.shape[1] else A
    lo, hi = lanczos_extremes(X @ X.T, iters)
    return {"orth_err": orthogonality_error(A), "theta_min": lo, "theta_max": hi,
            "sigma_min": float(np.sqrt(max(lo, 0.0))) if np.isfinite(lo) else lo,
            "sigma_max": float(np.sqrt(max(hi, 0.0))) if np.isfinite(hi) else hi}


def singular_values(O: np.ndarray) -> np.ndarray:
    """Singular values, descending (LAPACK through numpy)."""
    return np.linalg.svd(np.asarray(O, dtype=np.float64), compute_uv=False)


def rel_frobenius(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_F / ||ref||_F (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)
