"""GPU parity of the MuonSSM momentum pathway (muon_ssm_momentum) against the
fp64 oracle: M_T and S_T after T tokens of M_t = beta M_{t-1} + NS(V_t K_t^T),
S_t = a_t S_{t-1} + M_t, through the C ABI."""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spectral_optimizer_ssm_amd as mu
    mu.lib()
    return mu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield


def f64(t):
    return t.detach().double().cpu().numpy()


def oracle_states(V, K, a, M0, S0, seq, beta, steps, coeffs=(1.5, -0.5), with_s=True):
    return orc.ssm_momentum(f64(V[seq]), f64(K[seq]), f64(a[seq]), beta, f64(M0[seq]),
                            f64(S0[seq]) if with_s else None, steps=steps, coeffs=coeffs)


def run(mu, V, K, a, M0, S0, beta, steps, with_s=True, coeffs=(1.5, -0.5)):
    M = M0.clone().cuda()
    S = S0.clone().cuda() if with_s else None
    mu.muon_ssm_momentum(V.cuda(), K.cuda(), M, S, a.cuda() if with_s else None, beta=beta, steps=steps,
                         coeffs=coeffs)
    torch.cuda.synchronize()
    return M.cpu(), (S.cpu() if with_s else None)


def check(mu, nseq, T, m, n, steps=1, with_s=True, beta=wl.SSM_BETA, coeffs=(1.5, -0.5), seqs=None, seed=8):
    V, K, a, M0, S0 = wl.ssm_sequences(nseq, T, m, n, seed=seed)
    M, S = run(mu, V, K, a, M0, S0, beta, steps, with_s, coeffs)
    worst = 0.0
    for q in (range(nseq) if seqs is None else seqs):
        Mr, Sr = oracle_states(V, K, a, M0, S0, q, beta, steps, coeffs, with_s)
        em = orc.rel_frobenius(f64(M[q]), Mr)
        worst = max(worst, em)
        assert em <= BF16_TOL, (q, em)
        if with_s:
            es = orc.rel_frobenius(f64(S[q]), Sr)
            worst = max(worst, es)
            assert es <= BF16_TOL, (q, es)
    print(f"[parity] ssm_momentum nseq {nseq} T {T} {m}x{n} steps {steps} S {with_s}: max rel {worst:.3e}",
          flush=True)
    return V, K, a, M0, S0, M, S


@pytest.mark.parametrize("T", [1, 16, 37, 256, 600])
def test_ssm_momentum_muonssm_shape(mu, T):
    """64 x 128 rank-8 injections: one and several 256-token chunks, a ragged
    last chunk and sub-batches of 16 tokens."""
    check(mu, 3, T, 64, 128)


@pytest.mark.parametrize("m,n", [(40, 100), (64, 32), (1, 128), (17, 5)])
def test_ssm_momentum_padded_shapes(mu, m, n):
    check(mu, 2, 70, m, n)


def test_ssm_momentum_without_memory_state(mu):
    check(mu, 2, 300, 64, 128, with_s=False)


@pytest.mark.parametrize("steps,coeffs", [(0, (1.5, -0.5)), (1, (2.0, -1.5, 0.5)), (5, (1.5, -0.5)),
                                          (2, (2.0, -1.5, 0.5))])
def test_ssm_momentum_more_steps_and_quintic(mu, steps, coeffs):
    check(mu, 2, 40, 64, 128, steps=steps, coeffs=coeffs)


def test_ssm_momentum_zero_beta_and_decay_is_last_token(mu):
    """beta = 0 and a = 0: both states are the last token's NS result."""
    V, K, a, M0, S0 = wl.ssm_sequences(2, 20, 64, 128, seed=9)
    a.zero_()
    M, S = run(mu, V, K, a, M0, S0, 0.0, 1)
    for q in range(2):
        O, _ = orc.newton_schulz(f64(V[q, -1]) @ f64(K[q, -1]).T, 1)
        assert orc.rel_frobenius(f64(M[q]), O) <= BF16_TOL
        assert orc.rel_frobenius(f64(S[q]), O) <= BF16_TOL


def test_ssm_momentum_consecutive_calls_carry_the_states(mu):
    """Two calls over parts of a sequence give the one-call result: the
    states carry over.  Each token's factor enters the sums weighted relative
    to the end of its 256-token chunk and rounded once to bf16 (2^-9
    relative), so tokens whose chunk ends differently in the two runs are
    rounded differently.  The last chunk ends with the sequence in both runs
    and its tokens dominate M (beta = 0.875); S keeps older tokens longer.
    An fp64 emulation of this arithmetic gives 1.7e-6 (M) and 1.2e-4 (S) for
    this split, hence the bound of 1e-3.  A state dropped or misapplied at
    the split changes them by O(1); the two-call result also stays within
    the parity tolerance of the oracle."""
    V, K, a, M0, S0 = wl.ssm_sequences(2, 500, 64, 128, seed=10)
    M1, S1 = run(mu, V, K, a, M0, S0, wl.SSM_BETA, 1)
    h = 190
    Mh, Sh = run(mu, V[:, :h].contiguous(), K[:, :h].contiguous(), a[:, :h].contiguous(), M0, S0, wl.SSM_BETA, 1)
    M2, S2 = run(mu, V[:, h:].contiguous(), K[:, h:].contiguous(), a[:, h:].contiguous(), Mh, Sh, wl.SSM_BETA, 1)
    dm, ds = orc.rel_frobenius(f64(M2), f64(M1)), orc.rel_frobenius(f64(S2), f64(S1))
    print(f"[parity] ssm_momentum split at {h}: M {dm:.3e} S {ds:.3e}", flush=True)
    assert dm <= 1e-3 and ds <= 1e-3
    Mr, Sr = oracle_states(V, K, a, M0, S0, 0, wl.SSM_BETA, 1)
    assert orc.rel_frobenius(f64(M2[0]), Mr) <= BF16_TOL
    assert orc.rel_frobenius(f64(S2[0]), Sr) <= BF16_TOL


def test_ssm_momentum_deterministic(mu):
    V, K, a, M0, S0 = wl.ssm_sequences(4, 300, 64, 128, seed=11)
    r1 = run(mu, V, K, a, M0, S0, wl.SSM_BETA, 1)
    r2 = run(mu, V, K, a, M0, S0, wl.SSM_BETA, 1)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


def test_ssm_momentum_full_size_sampled(mu):
    """The MuonSSM injection workload as sequences: 192 sequences (batch 8 x
    24 heads) of 2048 tokens, 64 x 128 rank 8; the oracle checks the first
    and last sequence whole (every token's NS and the recurrence)."""
    V, K, a, M0, S0 = wl.ssm_sequences(device="cuda")
    M = M0.clone()
    S = S0.clone()
    mu.muon_ssm_momentum(V, K, M, S, a, beta=wl.SSM_BETA, steps=1)
    torch.cuda.synchronize()
    assert torch.isfinite(M).all() and torch.isfinite(S).all()
    for q in (0, V.shape[0] - 1):
        Mr, Sr = orc.ssm_momentum(f64(V[q]), f64(K[q]), f64(a[q]), wl.SSM_BETA, f64(M0[q]), f64(S0[q]), steps=1)
        em, es = orc.rel_frobenius(f64(M[q]), Mr), orc.rel_frobenius(f64(S[q]), Sr)
        print(f"[parity] ssm_momentum full size, sequence {q}: M {em:.3e} S {es:.3e}", flush=True)
        assert em <= BF16_TOL and es <= BF16_TOL


def _random_case(seed):
    """Shape, length, beta, decay range, S on or off and NS steps drawn from a
    seeded generator: m in 1..64, n in 1..128, T in 1..700 (chunk and round
    boundaries anywhere), beta in [0, 0.99], decays in [lo, 1) with lo in
    [0, 0.95]."""
    rng = np.random.default_rng(1000 + seed)
    return dict(nseq=int(rng.integers(1, 4)), T=int(rng.integers(1, 701)), m=int(rng.integers(1, 65)),
                n=int(rng.integers(1, 129)), beta=float(rng.uniform(0.0, 0.99)), lo=float(rng.uniform(0.0, 0.95)),
                with_s=bool(rng.integers(0, 2)), steps=int(rng.integers(1, 3)))


@pytest.mark.parametrize("seed", range(8))
def test_ssm_momentum_random_cases(mu, seed):
    """Seeded random shapes, lengths, momenta, decay ranges, S on or off and
    NS step counts against the oracle, every sequence whole."""
    c = _random_case(seed)
    V, K, a, M0, S0 = wl.ssm_sequences(c["nseq"], c["T"], c["m"], c["n"], seed=seed)
    a = c["lo"] + (1.0 - c["lo"]) * (a - 0.85) / 0.15   # the drawn decays mapped onto [lo, 1)
    M, S = run(mu, V, K, a, M0, S0, c["beta"], c["steps"], c["with_s"])
    worst = 0.0
    for q in range(c["nseq"]):
        Mr, Sr = oracle_states(V, K, a, M0, S0, q, c["beta"], c["steps"], with_s=c["with_s"])
        worst = max(worst, orc.rel_frobenius(f64(M[q]), Mr))
        if c["with_s"]:
            worst = max(worst, orc.rel_frobenius(f64(S[q]), Sr))
    print(f"[parity] ssm_momentum random {c}: max rel {worst:.3e}", flush=True)
    assert worst <= BF16_TOL
