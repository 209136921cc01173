"""GPU parity of the spectral cap in muon_step against the fp64 oracle
(oracle.muon_step_capped, oracle.power_step).

The cap's decision (act when sigma >= cap and u^T O v < 0) is a comparison of a
floating-point value; the cases are built so that u^T O v is far from zero
(each gradient carries a strong +-u v^T component), so both sides decide alike
and the test checks that they do.  The power step is checked on the weights the
GPU produced (float32 arithmetic, tolerance 1e-5); O, W and M to the usual
bounds of their precision.
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL, F32_TOL, MOM_TOL, t64, to_torch_bits

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


def unit(x):
    return x / np.linalg.norm(x)


def make_case(seed, count, m, n, grad, exact_pair=True):
    """W with a clear top singular value, gradients with a strong +-u v^T part
    (sign alternating over the matrices), u, v either W's exact top pair or
    random unit vectors."""
    rng = np.random.default_rng(seed)
    W = np.empty((count, m, n), np.float32)
    G = np.empty((count, m, n), np.float64)
    U1 = np.empty((count, m), np.float32)
    V1 = np.empty((count, n), np.float32)
    for i in range(count):
        Wi = 0.02 * rng.standard_normal((m, n))
        a, b = unit(rng.standard_normal(m)), unit(rng.standard_normal(n))
        Wi += 0.5 * np.outer(a, b)
        W[i] = Wi.astype(np.float32)
        if exact_pair:
            Us, _, Vt = np.linalg.svd(W[i].astype(np.float64), full_matrices=False)
            u, v = Us[:, 0], Vt[0]
        else:
            u, v = unit(rng.standard_normal(m)), unit(rng.standard_normal(n))
        U1[i], V1[i] = u.astype(np.float32), v.astype(np.float32)
        sgn = -1.0 if i % 2 == 0 else 1.0
        G[i] = rng.standard_normal((m, n)) + sgn * 5.0 * (np.sqrt(m) + np.sqrt(n)) * np.outer(u, v)
    if grad == "bf16":
        Gb = wl.f64_to_bf16_bits(G)
    else:
        Gb = G.astype(np.float32)
    M = (1e-3 * rng.standard_normal((count, m, n))).astype(np.float32)
    return W, M, Gb, U1, V1


def run_capped(mu, W, M, Gb, U1, V1, sigma, cap, grad, precision, steps=5, lr=0.02):
    Wd, Md = torch.from_numpy(W.copy()).cuda(), torch.from_numpy(M.copy()).cuda()
    Gd = (to_torch_bits(Gb) if grad == "bf16" else torch.from_numpy(Gb)).cuda()
    Ud, Vd = torch.from_numpy(U1.copy()).cuda(), torch.from_numpy(V1.copy()).cuda()
    Sd = torch.from_numpy(sigma.astype(np.float32)).cuda()
    odt = torch.bfloat16 if precision == mu.MUON_BF16 else torch.float32
    O = torch.full(W.shape, float("nan"), dtype=odt, device="cuda")
    grp = mu.MuonGroup(W=Wd, M=Md, G=Gd, O=O, lr=lr, beta=0.95, cap_u=Ud, cap_v=Vd, cap_sigma=Sd, cap=cap)
    mu.muon_step([grp], steps=steps, precision=precision)
    torch.cuda.synchronize()
    return Wd, Md, O, Ud, Vd, Sd


def compare(W, M, Gb, U1, V1, sigma, cap, grad, out, tol, steps=5, lr=0.02):
    Wd, Md, O, Ud, Vd, Sd = out
    acted = 0
    for i in range(W.shape[0]):
        g = orc.widen_bf16(Gb[i]) if grad == "bf16" else orc.widen_f32(Gb[i])
        ref = orc.muon_step_capped(orc.widen_f32(W[i]), orc.widen_f32(M[i]), g, orc.widen_f32(U1[i]),
                                   orc.widen_f32(V1[i]), float(sigma[i]), cap=cap, beta=0.95, lr=lr, steps=steps)
        o = t64(O[i])
        assert orc.rel_frobenius(o, ref["O"]) <= tol, (i, orc.rel_frobenius(o, ref["O"]))
        # same decision on both sides: the capped O has (almost) no u v^T part
        c_gpu = float(orc.widen_f32(U1[i]) @ o @ orc.widen_f32(V1[i]))
        if ref["gamma"] != 0.0:
            acted += 1
            assert abs(c_gpu) <= 10 * tol * np.linalg.norm(ref["O_uncapped"]), (i, c_gpu, ref["gamma"])
        else:
            assert abs(c_gpu - float(orc.widen_f32(U1[i]) @ ref["O"] @ orc.widen_f32(V1[i]))) \
                <= 10 * tol * np.linalg.norm(ref["O"])
        w_new = t64(Wd[i])
        dw, dref = w_new - orc.widen_f32(W[i]), ref["W"] - orc.widen_f32(W[i])
        assert orc.rel_frobenius(dw, dref) <= tol
        assert orc.rel_frobenius(t64(Md[i]), ref["M"]) <= MOM_TOL
        # the power step on the weights the GPU wrote
        u2, v2, s2 = orc.power_step(w_new, orc.widen_f32(U1[i]), orc.widen_f32(V1[i]))
        assert orc.rel_frobenius(t64(Ud[i]), u2) <= F32_TOL
        assert orc.rel_frobenius(t64(Vd[i]), v2) <= F32_TOL
        assert abs(float(Sd[i]) - s2) <= F32_TOL * s2
    return acted


@pytest.mark.parametrize("m,n,grad,prec,exact", [
    (256, 640, "bf16", "bf16", True),     # large bf16 tiles, wide
    (520, 200, "bf16", "bf16", True),     # tall
    (64, 128, "bf16", "bf16", False),     # on-chip small kernel
    (96, 160, "f32", "f32", True),        # float32 path
    (130, 70, "bf16", "f32", False),      # bf16 gradients, float32 iterate, ragged
    (50, 70, "bf16", "bf16", True),       # on-chip, both sides zero-padded to 64 x 96
    (300, 96, "bf16", "bf16", False),     # on-chip, tall, rows split over the waves
    (128, 512, "bf16", "bf16", True),     # on-chip, columns split over the waves
])
def test_cap_matches_oracle(mu, m, n, grad, prec, exact):
    count = 4
    W, M, Gb, U1, V1 = make_case(m * 7 + n, count, m, n, grad, exact)
    sigma = np.full(count, 10.0)
    precision = mu.MUON_BF16 if prec == "bf16" else mu.MUON_F32
    out = run_capped(mu, W, M, Gb, U1, V1, sigma, 1.0, grad, precision)
    acted = compare(W, M, Gb, U1, V1, sigma, 1.0, grad, out, BF16_TOL if prec == "bf16" else F32_TOL)
    assert acted == count // 2  # the matrices whose gradient grows sigma_1


def test_cap_below_threshold_is_plain_muon(mu):
    count, m, n = 2, 192, 320
    W, M, Gb, U1, V1 = make_case(3, count, m, n, "bf16")
    sigma = np.full(count, 0.5)
    out = run_capped(mu, W, M, Gb, U1, V1, sigma, 100.0, "bf16", mu.MUON_BF16)
    assert compare(W, M, Gb, U1, V1, sigma, 100.0, "bf16", out, BF16_TOL) == 0
    # and the same W as muon_step without the cap
    Wd = torch.from_numpy(W.copy()).cuda()
    Md = torch.from_numpy(M.copy()).cuda()
    grp = mu.MuonGroup(W=Wd, M=Md, G=to_torch_bits(Gb).cuda(), lr=0.02, beta=0.95)
    mu.muon_step([grp], steps=5)
    torch.cuda.synchronize()
    assert torch.equal(Wd, out[0])


def test_cap_full_step_shapes_sampled(mu):
    """The Mamba-2 projection shapes (one call per shape), cap on, random
    initial estimates; sampled matrices against the oracle."""
    groups, cases = [], []
    for gi, (m, n) in enumerate(((768, 1536), (3352, 768))):
        W, M, Gb, U1, V1 = make_case(100 + gi, 4, m, n, "bf16", exact_pair=False)
        cases.append((W, M, Gb, U1, V1))
    outs = []
    for W, M, Gb, U1, V1 in cases:
        outs.append(run_capped(mu, W, M, Gb, U1, V1, np.full(4, 10.0), 0.0, "bf16", mu.MUON_BF16))
    for (W, M, Gb, U1, V1), out in zip(cases, outs):
        idx = [0, 1]
        sub = lambda a: a[idx]  # noqa: E731
        acted = compare(sub(W), sub(M), sub(Gb), sub(U1), sub(V1), np.full(2, 10.0), 0.0, "bf16",
                        tuple(t[idx] for t in out), BF16_TOL)
        assert acted == 1


def test_cap_tracks_top_pair_over_steps(mu):
    """Repeated steps on a weight with a dominant direction: the estimates,
    started at random, converge to the top singular pair of the current W."""
    m, n = 200, 300
    rng = np.random.default_rng(9)
    a, b = unit(rng.standard_normal(m)), unit(rng.standard_normal(n))
    W = (0.01 * rng.standard_normal((1, m, n)) + 2.0 * np.outer(a, b)[None]).astype(np.float32)
    Wd = torch.from_numpy(W).cuda()
    Md = torch.zeros_like(Wd)
    Ud = torch.from_numpy(unit(rng.standard_normal(m)).astype(np.float32)[None]).cuda()
    Vd = torch.from_numpy(unit(rng.standard_normal(n)).astype(np.float32)[None]).cuda()
    Sd = torch.zeros(1, device="cuda")
    for k in range(25):
        G = torch.from_numpy(rng.standard_normal((1, m, n)).astype(np.float32)).to(torch.bfloat16).cuda()
        grp = mu.MuonGroup(W=Wd, M=Md, G=G, lr=1e-3, beta=0.9, cap_u=Ud, cap_v=Vd, cap_sigma=Sd, cap=1.0)
        mu.muon_step([grp], steps=5)
    torch.cuda.synchronize()
    Us, s, Vt = np.linalg.svd(t64(Wd[0]), full_matrices=False)
    assert abs(abs(float(t64(Ud[0]) @ Us[:, 0])) - 1) < 1e-4
    assert abs(abs(float(t64(Vd[0]) @ Vt[0])) - 1) < 1e-4
    assert abs(float(Sd[0]) - s[0]) < 1e-3 * s[0]


def test_cap_deterministic(mu):
    W, M, Gb, U1, V1 = make_case(12, 3, 256, 384, "bf16", exact_pair=False)
    a = run_capped(mu, W, M, Gb, U1, V1, np.full(3, 5.0), 0.0, "bf16", mu.MUON_BF16)
    b = run_capped(mu, W, M, Gb, U1, V1, np.full(3, 5.0), 0.0, "bf16", mu.MUON_BF16)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
