"""GPU parity of muon_ns_factored (Newton-Schulz of X = V K^T from its factors)
against the fp64 oracle (oracle.factored_ns: the dense NS of V K^T and its
unique r x r core).

Tolerances: the core runs in float32 from exactly widened bf16 factors, so the
core C and V C K^T are held to the float32 bound (1e-5 relative Frobenius; a
CPU emulation of the kernel's arithmetic stays below 5e-7); the optional dense
output is rounded to bf16 and held to 2e-2.
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL, F32_TOL, t64

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


def factors(seed, batch, m, n, r):
    g = torch.Generator().manual_seed(seed)
    V = torch.randn((batch, m, r), generator=g).to(torch.bfloat16)
    K = torch.randn((batch, n, r), generator=g).to(torch.bfloat16)
    return V, K


def check(V, K, C, O, steps, coeffs, per_step, idx):
    errs = []
    for b in idx:
        v, k = t64(V[b]), t64(K[b])
        o_ref, c_ref, _ = orc.factored_ns(v, k, steps, coeffs=coeffs, per_step=per_step)
        c = t64(C[b])
        e_c = orc.rel_frobenius(c, c_ref)
        e_o = orc.rel_frobenius(v @ c @ k.T, o_ref)
        assert e_c <= F32_TOL and e_o <= F32_TOL, (b, e_c, e_o)
        if O is not None:
            e_d = orc.rel_frobenius(t64(O[b]), o_ref)
            assert e_d <= BF16_TOL, (b, e_d)
            errs.append(e_d)
        errs.append(max(e_c, e_o))
    return max(errs)


@pytest.mark.parametrize("m,n,r,steps,coeffs,per_step", [
    (64, 128, 8, 0, (1.5, -0.5), False),                          # normalisation only
    (64, 128, 8, 1, (1.5, -0.5), False),
    (64, 128, 8, 1, (2.0, -1.5, 0.5), False),                     # quintic first step alone
    (64, 128, 8, 5, (1.5, -0.5), False),
    (64, 128, 8, 3, (2.0, -1.5, 0.5), False),                     # quintic
    (64, 128, 8, 2, [(1.6, -0.6), (1.4, -0.4)], True),            # per-step rows
    (32, 96, 4, 3, (1.5, -0.5), False),
    (100, 40, 3, 2, (1.5, -0.5), False),                          # tall, odd r, 2-byte staging
    (200, 256, 8, 1, (1.5, -0.5), False),
    (1, 8, 1, 4, (1.5, -0.5), False),
])
def test_factored_matches_oracle(mu, m, n, r, steps, coeffs, per_step):
    batch = 4 * 13 + 3  # a last wavefront with three matrices
    V, K = factors(m * 1000 + n + r, batch, m, n, r)
    Vd, Kd = V.cuda(), K.cuda()
    dense = n % 8 == 0 and (m + 15) // 16 * 16 * 192 + (n + 15) // 16 * 16 * 64 + 6144 <= 65536
    O = torch.full((batch, m, n), float("nan"), dtype=torch.bfloat16, device="cuda") if dense else None
    C = mu.muon_ns_factored(Vd, Kd, O=O, steps=steps, coeffs=coeffs, per_step=per_step)
    torch.cuda.synchronize()
    worst = check(V, K, C.cpu(), O.cpu() if O is not None else None, steps, coeffs, per_step, range(batch))
    print("worst", worst, "dense" if dense else "core only")


def test_factored_injections_full_size_sampled(mu):
    X, V, K = wl.injections(device="cuda", return_factors=True)
    del X
    assert V.shape == (393216, 64, 8) and K.shape == (393216, 128, 8)
    C = mu.muon_ns_factored(V, K, steps=1)
    torch.cuda.synchronize()
    assert torch.isfinite(C).all()
    rng = np.random.default_rng(2025)
    idx = np.unique(np.concatenate([[0, V.shape[0] - 1], rng.integers(0, V.shape[0], 512)]))
    it = torch.from_numpy(idx).cuda()
    worst = check(V[it].cpu(), K[it].cpu(), C[it].cpu(), None, 1, (1.5, -0.5), False, range(len(idx)))
    print("sampled", len(idx), "worst", worst)


def test_factored_agrees_with_dense_entry_point(mu):
    """The dense muon_ns_batched_small on the same X (formed exactly and
    rounded to bf16) and the factored path agree to the bf16 bound."""
    V, K = factors(11, 256, 64, 128, 8)
    X = torch.bmm(V.double(), K.double().transpose(1, 2).contiguous()).to(torch.bfloat16).cuda()
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=1)
    O = torch.empty_like(X)
    mu.muon_ns_factored(V.cuda(), K.cuda(), O=O, steps=1)
    torch.cuda.synchronize()
    errs = [orc.rel_frobenius(t64(O[b]), t64(Y[b])) for b in range(256)]
    assert max(errs) <= BF16_TOL


def test_factored_zero_and_nan(mu):
    V, K = factors(5, 8, 64, 128, 8)
    V[2] = 0
    V[5, 3, 1] = float("nan")
    O = torch.empty((8, 64, 128), dtype=torch.bfloat16, device="cuda")
    C = mu.muon_ns_factored(V.cuda(), K.cuda(), O=O, steps=5)
    torch.cuda.synchronize()
    assert (O[2].float() == 0).all()              # zero injection -> zero update
    assert torch.isnan(C[5]).all() and torch.isnan(O[5].float()).all()
    assert torch.isfinite(C[4]).all() and torch.isfinite(O[6].float()).all()


def test_factored_deterministic(mu):
    V, K = factors(6, 100, 64, 128, 8)
    Vd, Kd = V.cuda(), K.cuda()
    a = mu.muon_ns_factored(Vd, Kd, steps=3)
    b = mu.muon_ns_factored(Vd, Kd, steps=3)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
