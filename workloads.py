"""Seeded synthetic inputs for the Muon / Newton-Schulz hot path.

Shared by the tests, the smoke check and the benchmark; used by both the GPU
path and the CPU oracle, and holding none of the method's arithmetic (no
momentum, normalisation or Newton-Schulz here, only input construction).

Shapes are those of Mamba-2 130M ("Muon Meets Mamba", abstract: Muon on the
input and output projections of Mamba-2 130M): 24 layers, d_model 768,
d_inner 1536, d_state 128, 24 heads, so in_proj is (2*1536 + 2*128 + 24) x 768
= 3352 x 768 and out_proj is 768 x 1536.  The MuonSSM injections ("MuonSSM",
method section on momentum-augmented dynamics: low-rank value-key outer
products) are 64 x 128 sums of 8 outer products.  No corpus, trained weights
or real gradients are available, so these synthetic gradients stand in for
them; the recipes are fixed here and restated in the design notes.

Conventions: N(0, x) means standard deviation x; "-> bf16" is round to
nearest even; Haar factors come from the QR of a Gaussian matrix with the
sign of diag(R) folded into Q.  Every matrix draws from its own child stream
of numpy.random.SeedSequence(seed).spawn(count), in the order documented per
recipe, so any one matrix can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

IN_PROJ = (3352, 768)
OUT_PROJ = (768, 1536)
N_LAYERS = 24
SPIKE_RANK = 8
INJ_SHAPE = (64, 128)
INJ_RANK = 8
INJ_BATCH = 8 * 2048 * 24          # batch 8 x seq 2048 x 24 heads = 393,216
INJ_CHUNK = 8192


# ----------------------------------------------------------------------------
# bfloat16 encoding (input construction only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """binary32 -> bfloat16 bits, round to nearest even, NaN kept quiet."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """binary64 -> bfloat16 bits with a single round to nearest even.

    Goes through binary32 (RNE) and repairs the one case where that double
    rounding can differ: a binary32 result lying exactly on a bfloat16
    midpoint although the binary64 value was not on it.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = x.astype(np.float32)
    bits = y.view(np.uint32)
    out = f32_to_bf16_bits(y).astype(np.uint32)
    tie = (bits & np.uint32(0xFFFF)) == np.uint32(0x8000)
    finite = np.isfinite(y)
    resid = x - y.astype(np.float64)
    up = tie & finite & (resid != 0) & (np.sign(resid) == np.sign(y))
    down = tie & finite & (resid != 0) & (np.sign(resid) != np.sign(y))
    out = np.where(up, (bits >> np.uint32(16)) + np.uint32(1), out)
    out = np.where(down, bits >> np.uint32(16), out)
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bits -> binary32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# Random factors
# ----------------------------------------------------------------------------
def haar(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows x cols matrix with orthonormal columns, Haar distributed (rows >= cols)."""
    z = rng.standard_normal((rows, cols))
    q, r = np.linalg.qr(z)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d


def svd_built(rng: np.random.Generator, m: int, n: int, decades: float) -> np.ndarray:
    """G = U diag(s) V^T in float64 with Haar U (m x r), V (n x r), r = min(m, n),
    and s = 10**(-decades * u), u ~ U[0, 1).  Draw order: U, V, u."""
    r = min(m, n)
    U = haar(rng, m, r)
    V = haar(rng, n, r)
    s = 10.0 ** (-decades * rng.random(r))
    return (U * s) @ V.T


def spiked_gaussian(rng: np.random.Generator, m: int, n: int, rank: int) -> np.ndarray:
    """G = Z + c A B^T with Z ~ N(0,1) (m x n), A (m x rank) and B (n x rank) Haar,
    c = 10 (sqrt(m) + sqrt(n)): the spike is 10x the bulk's top singular value.
    Draw order: Z, A, B."""
    Z = rng.standard_normal((m, n))
    A = haar(rng, m, rank)
    B = haar(rng, n, rank)
    c = 10.0 * (math.sqrt(m) + math.sqrt(n))
    return Z + c * (A @ B.T)


# ----------------------------------------------------------------------------
# Parameter groups
# ----------------------------------------------------------------------------
@dataclass
class Group:
    """One shape group: count matrices of m x n (row-major)."""
    m: int
    n: int
    G: np.ndarray            # [count, m, n] uint16 bf16 bits, or float32
    W: np.ndarray            # [count, m, n] float32
    M: np.ndarray            # [count, m, n] float32
    grad_dtype: str          # "bf16" | "f32"
    name: str = ""

    @property
    def count(self) -> int:
        return self.G.shape[0]


@dataclass
class Workload:
    name: str
    groups: list
    beta: float = 0.95
    lr: float = 0.02
    nesterov: bool = True
    steps: int = 5
    coeffs: tuple = (1.5, -0.5)
    per_step: bool = False
    eps: float = 1e-7
    scale: float = 1.0
    meta: dict = field(default_factory=dict)


def _group(seed: int, count: int, m: int, n: int, kind: str, name: str,
           zero_momentum: bool = False, decades: float = 3.0, first: int = 0) -> Group:
    """Build matrices first..first+count-1 of a group from SeedSequence(seed).

    Per matrix stream, draw order: the gradient (kind "svd" or "spike"), then
    W = 0.02 N(0,1), then M = 1e-3 N(0,1) (skipped when zero_momentum)."""
    children = np.random.SeedSequence(seed).spawn(first + count)[first:]
    G = np.empty((count, m, n), np.uint16)
    W = np.empty((count, m, n), np.float32)
    M = np.zeros((count, m, n), np.float32)
    for i, ss in enumerate(children):
        rng = np.random.default_rng(ss)
        if kind == "svd":
            g = svd_built(rng, m, n, decades)
        elif kind == "spike":
            g = spiked_gaussian(rng, m, n, SPIKE_RANK)
        elif kind == "gauss":
            g = rng.standard_normal((m, n))
        else:
            raise ValueError(kind)
        G[i] = f64_to_bf16_bits(g)
        W[i] = (0.02 * rng.standard_normal((m, n))).astype(np.float32)
        mom = (1e-3 * rng.standard_normal((m, n))).astype(np.float32)
        if not zero_momentum:
            M[i] = mom
    return Group(m, n, G, W, M, "bf16", name)


def config1() -> Workload:
    """Single fp32 gradient 128 x 64: default_rng(0) draws G = N(0,1), then
    W = 0.02 N(0,1); M = 0; beta 0.95 Nesterov, lr 0.02, 5 cubic steps."""
    rng = np.random.default_rng(0)
    G = rng.standard_normal((128, 64)).astype(np.float32)
    W = (0.02 * rng.standard_normal((128, 64))).astype(np.float32)
    M = np.zeros((128, 64), np.float32)
    g = Group(128, 64, G[None], W[None], M[None], "f32", "single")
    return Workload("single-fp32-128x64", [g])


def config2(count: int = N_LAYERS, shape=OUT_PROJ, first: int = 0) -> Workload:
    """out_proj group: count x (768 x 1536) bf16 G = U diag(s) V^T, s log-uniform
    in [1e-3, 1]; W = 0.02 N, M = 1e-3 N (fp32).  SeedSequence(1)."""
    g = _group(1, count, shape[0], shape[1], "svd", "out_proj", decades=3.0, first=first)
    return Workload(f"out_proj-{count}x{shape[0]}x{shape[1]}", [g])


def config3(count: int = N_LAYERS, shape=IN_PROJ, first: int = 0) -> Workload:
    """in_proj group: count x (3352 x 768) bf16 Gaussian G with a rank-8 spike of
    10x the bulk's top singular value; W, M as config 2.  SeedSequence(2)."""
    g = _group(2, count, shape[0], shape[1], "spike", "in_proj", first=first)
    return Workload(f"in_proj-{count}x{shape[0]}x{shape[1]}", [g])


def config4(count: int = N_LAYERS, steps: int = 5, zero_momentum: bool = False,
            out_shape=OUT_PROJ, in_shape=IN_PROJ, first: int = 0) -> Workload:
    """Full Mamba-2-130M step: count out_proj + count in_proj, each U diag(s) V^T
    with s log-uniform in [1e-6, 1]; W, M as config 2.  The out_proj matrices
    come from SeedSequence(3), the in_proj ones from SeedSequence(30).
    zero_momentum gives the M = 0 variant, where U = (1 + beta) G exactly."""
    go = _group(3, count, out_shape[0], out_shape[1], "svd", "out_proj",
                zero_momentum, decades=6.0, first=first)
    gi = _group(30, count, in_shape[0], in_shape[1], "svd", "in_proj",
                zero_momentum, decades=6.0, first=first)
    w = Workload(f"mamba2-130m-full-step-{2 * count}-matrices", [go, gi], steps=steps)
    return w


def random_group(seed: int, count: int, m: int, n: int, grad_dtype: str = "bf16",
                 kind: str = "gauss", zero_momentum: bool = False) -> Group:
    """Small generic group for parity cases (ragged tails, odd shapes)."""
    if grad_dtype == "bf16":
        return _group(seed, count, m, n, kind, f"rand{m}x{n}", zero_momentum)
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((count, m, n)).astype(np.float32)
    W = (0.02 * rng.standard_normal((count, m, n))).astype(np.float32)
    M = np.zeros((count, m, n), np.float32) if zero_momentum else \
        (1e-3 * rng.standard_normal((count, m, n))).astype(np.float32)
    return Group(m, n, G, W, M, "f32", f"rand{m}x{n}")


# ----------------------------------------------------------------------------
# MuonSSM low-rank injections (torch: generated where they are consumed)
# ----------------------------------------------------------------------------
def injections(batch: int = INJ_BATCH, device="cpu", seed: int = 4,
               shape=INJ_SHAPE, rank: int = INJ_RANK, chunk: int = INJ_CHUNK,
               return_factors: bool = False):
    """[batch, 64, 128] bf16 stack of low-rank memory injections X = V K^T.

    A torch.Generator(device).manual_seed(seed) draws, chunk by chunk of 8192
    matrices in index order, V = N(0,1) [chunk, 64, 8] then K = N(0,1)
    [chunk, 128, 8] in fp32, each rounded to bf16; X = sum of the 8 outer
    products v_i k_i^T in fp64, rounded to fp32 and then to bf16.  The CPU and
    GPU generators of torch are different streams, so a stack is only
    reproduced on the same kind of device.
    """
    import torch
    m, n = shape
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((batch, m, n), dtype=torch.bfloat16, device=device)
    Vs, Ks = [], []
    for s0 in range(0, batch, chunk):
        b = min(chunk, batch - s0)
        V = torch.randn((b, m, rank), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        K = torch.randn((b, n, rank), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        X = torch.bmm(V.double(), K.double().transpose(1, 2).contiguous())
        out[s0:s0 + b] = X.float().to(torch.bfloat16)
        if return_factors:
            Vs.append(V)
            Ks.append(K)
    if return_factors:
        return out, torch.cat(Vs), torch.cat(Ks)
    return out


# ----------------------------------------------------------------------------
# Sequences for the momentum pathway (MuonSSM, momentum-augmented state update)
# ----------------------------------------------------------------------------
SSM_SEQS = 8 * 24                   # batch 8 x 24 heads
SSM_T = 2048                        # tokens per sequence (8 x 2048 x 24 injections, as above)
SSM_BETA = 0.875                    # momentum coefficient (exact in float32; the pages give none)


def ssm_sequences(nseq: int = SSM_SEQS, T: int = SSM_T, m: int = INJ_SHAPE[0], n: int = INJ_SHAPE[1],
                  r: int = INJ_RANK, seed: int = 8, device="cpu"):
    """Inputs of the momentum pathway: V [nseq, T, m, r] and K [nseq, T, n, r]
    bf16 (N(0,1) in float32 -> bf16), per-token decays a [nseq, T] float32
    uniform in [0.85, 1) (the range of a selective SSM's per-token decay
    exp(-dt A) for small steps), and initial states M0, S0 [nseq, m, n]
    float32 N(0, 0.1).  A torch.Generator(device).manual_seed(seed) draws V,
    K, a, M0, S0 in that order; as for the injections, CPU and GPU streams
    differ."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    V = torch.randn((nseq, T, m, r), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    K = torch.randn((nseq, T, n, r), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    a = 0.85 + 0.15 * torch.rand((nseq, T), generator=g, device=device, dtype=torch.float32)
    M0 = 0.1 * torch.randn((nseq, m, n), generator=g, device=device, dtype=torch.float32)
    S0 = 0.1 * torch.randn((nseq, m, n), generator=g, device=device, dtype=torch.float32)
    return V, K, a, M0, S0


# ----------------------------------------------------------------------------
# The Mamba-2-130M parameters outside the Muon groups (AdamW companion)
# ----------------------------------------------------------------------------
def mamba2_adamw_shapes(layers: int = 24, d_model: int = 768, d_inner: int = 1536, d_state: int = 128,
                        heads: int = 24, d_conv: int = 4, vocab: int = 50280):
    """(name, shape) of the Mamba-2-130M parameters that are not in_proj or
    out_proj: tied embedding, per layer the pre-norm, the depthwise conv1d over
    x, B, C (weight and bias), dt_bias, A_log, D and the gated-norm weight, and
    the final norm."""
    conv_dim = d_inner + 2 * d_state
    out = [("embedding", (vocab, d_model))]
    for i in range(layers):
        out += [(f"layers.{i}.norm", (d_model,)), (f"layers.{i}.conv1d.weight", (conv_dim, 1, d_conv)),
                (f"layers.{i}.conv1d.bias", (conv_dim,)), (f"layers.{i}.dt_bias", (heads,)),
                (f"layers.{i}.A_log", (heads,)), (f"layers.{i}.D", (heads,)),
                (f"layers.{i}.mixer_norm", (d_inner,))]
    out.append(("norm_f", (d_model,)))
    return out


def adamw_state(shapes, seed: int = 6, grad_dtype: str = "bf16", step: int = 3):
    """Seeded float32 parameters (0.02 N(0,1)), gradients (N(0,1), bf16 bits
    or float32) and moments consistent with `step - 1` earlier steps
    (m ~ 0.1 N(0,1), v ~ 0.01 chi^2_1) for every shape."""
    ss = np.random.SeedSequence(seed).spawn(len(shapes))
    P, G, M, V = [], [], [], []
    for (name, shape), child in zip(shapes, ss):
        rng = np.random.default_rng(child)
        n = int(np.prod(shape))
        P.append((0.02 * rng.standard_normal(n)).astype(np.float32))
        g = rng.standard_normal(n).astype(np.float32)
        G.append(f32_to_bf16_bits(g) if grad_dtype == "bf16" else g)
        M.append((0.1 * rng.standard_normal(n)).astype(np.float32))
        V.append((0.01 * rng.standard_normal(n) ** 2).astype(np.float32))
    return P, G, M, V


def projection_stacks(count: int = N_LAYERS, seed: int = 5):
    """The full step's two projection shapes as float32 stacks drawn N(0, 1)
    (numpy default_rng(seed), out_proj first): [("out_proj", [count, 768,
    1536]), ("in_proj", [count, 3352, 768])].  Scaled by 0.02 they are the
    weights W of the full step; as bf16 they serve as gradients."""
    rng = np.random.default_rng(seed)
    return [(name, rng.standard_normal((count, *shape), dtype=np.float32))
            for name, shape in (("out_proj", OUT_PROJ), ("in_proj", IN_PROJ))]
