"""GPU parity of muon_spectral_diag against the fp64 oracle
(oracle.spectral_diagnostics: the orthogonality error by its definition, the
extreme singular values by the same Lanczos run in float64).

Tolerances, from the arithmetic: H = X X^T is accumulated in float32 on the
matrix cores from exact bf16 inputs (or from the exact three-piece split of
float32 inputs), so each entry carries an error of a few 2^-24 of
sum_k |x_ik x_jk|; the orthogonality error is held to 1e-5 absolute plus 1e-4
relative.  The Lanczos run is float32: the Ritz values are held to 2e-5 of the
largest eigenvalue theta_max = sigma_max^2 (compared as squares, which is how
they are computed; sigma_min near zero is only resolved to about
sqrt(2e-5) sigma_max).  With iters >= s the values are also checked against
LAPACK's singular values directly.
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import t64, to_torch_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ORTH_ABS, ORTH_REL, THETA_REL = 1e-5, 1e-4, 2e-5


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


def haar(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def stack(seed, batch, m, n, kind):
    """fp64 matrices: 'spread' = U diag(sigma) V^T with sigma in [0.05, 1.3]
    (an orthogonalised update that has not converged), 'gauss' = N(0, 1/l)."""
    rng = np.random.default_rng(seed)
    s = min(m, n)
    out = np.empty((batch, m, n))
    for b in range(batch):
        if kind == "spread":
            sig = rng.uniform(0.05, 1.3, s)
            out[b] = haar(rng, m, s) @ np.diag(sig) @ haar(rng, n, s).T
        else:
            out[b] = rng.standard_normal((m, n)) / np.sqrt(max(m, n))
    return out


def to_device(A, dtype):
    """(device tensor, exact fp64 values of what it holds)."""
    if dtype == "bf16":
        bits = wl.f64_to_bf16_bits(A)
        return to_torch_bits(bits).cuda(), orc.widen_bf16(bits)
    a32 = A.astype(np.float32)
    return torch.from_numpy(a32).cuda(), a32.astype(np.float64)


def check(out, exact, iters, idx):
    worst = [0.0, 0.0]
    for i, b in enumerate(idx):
        ref = orc.spectral_diagnostics(exact[b], iters)
        e_gpu = float(out["orth_err"][i])
        assert abs(e_gpu - ref["orth_err"]) <= ORTH_ABS + ORTH_REL * ref["orth_err"], (b, e_gpu, ref["orth_err"])
        top = ref["theta_max"]
        smax, smin = float(out["sigma_max"][i]), float(out["sigma_min"][i])
        d_hi = abs(smax * smax - ref["theta_max"]) / top
        d_lo = abs(smin * smin - max(ref["theta_min"], 0.0)) / top
        assert d_hi <= THETA_REL and d_lo <= THETA_REL, (b, d_hi, d_lo)
        worst = [max(worst[0], abs(e_gpu - ref["orth_err"])), max(worst[1], d_hi, d_lo)]
    return worst


@pytest.mark.parametrize("m,n,dtype,kind,iters", [
    (64, 128, "bf16", "spread", 64),      # injection-sized, iters = s: exact extremes
    (128, 64, "f32", "spread", 64),       # tall float32
    (200, 520, "bf16", "gauss", 40),      # ragged wide
    (520, 200, "f32", "gauss", 40),       # ragged tall, float32 pieces
    (130, 70, "bf16", "spread", 100),     # ragged tall bf16, iters capped at s
    (1, 37, "f32", "gauss", 5),           # a single row
    (300, 300, "bf16", "spread", 24),     # square
])
def test_diag_matches_oracle(mu, m, n, dtype, kind, iters):
    batch = 5
    A, exact = to_device(stack(m * 31 + n, batch, m, n, kind), dtype)
    out = mu.muon_spectral_diag(A, iters=iters)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    worst = check(out, exact, iters, range(batch))
    print("worst orth / theta", worst)
    if iters >= min(m, n):
        for b in range(batch):
            sv = np.linalg.svd(exact[b], compute_uv=False)
            assert abs(out["sigma_max"][b] ** 2 - sv[0] ** 2) <= THETA_REL * sv[0] ** 2
            assert abs(out["sigma_min"][b] ** 2 - sv[-1] ** 2) <= THETA_REL * sv[0] ** 2


def test_diag_full_size_update_shapes_sampled(mu):
    """The Mamba-2 projection shapes as Muon updates (bf16, 24 each) and as
    float32 weights, in one call per shape; sampled matrices against the
    oracle, every output finite and inside [0, sigma bound]."""
    for (m, n, dtype, batch) in ((768, 1536, "bf16", 24), (3352, 768, "bf16", 24), (3352, 768, "f32", 4)):
        A, exact = to_device(stack(m + n + batch, batch, m, n, "spread") if batch <= 4 else
                             np.concatenate([stack(m + n + c, 4, m, n, "spread") for c in range(batch // 4)]),
                             dtype)
        out = mu.muon_spectral_diag(A, iters=32)
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in out.items()}
        for k in out:
            assert np.isfinite(out[k]).all()
        assert (out["sigma_min"] <= out["sigma_max"]).all() and (out["sigma_max"] <= 1.3 * 1.0001).all()
        worst = check({k: v[[0, batch - 1]] for k, v in out.items()}, exact, 32, [0, batch - 1])
        print(m, n, dtype, "worst orth / theta", worst)


def test_diag_special_matrices(mu):
    m, n = 96, 160
    A = np.zeros((4, m, n))
    A[1, :, :m] = np.eye(m)                      # orthonormal rows
    A[2] = stack(3, 1, m, n, "gauss")[0]
    A[2, 5, 7] = np.nan                          # NaN propagates to this matrix only
    A[3] = 2.0 * A[1]                            # scaled: sigma = 2, error |4 - 1| = 3
    T = torch.from_numpy(A.astype(np.float32)).cuda()
    out = mu.muon_spectral_diag(T, iters=20)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in out.items()}
    assert o["orth_err"][0] == 1.0 and o["sigma_max"][0] == 0.0 and o["sigma_min"][0] == 0.0
    assert o["orth_err"][1] == 0.0 and abs(o["sigma_max"][1] - 1) < 1e-6 and abs(o["sigma_min"][1] - 1) < 1e-6
    assert np.isnan(o["orth_err"][2]) and np.isnan(o["sigma_max"][2]) and np.isnan(o["sigma_min"][2])
    assert o["orth_err"][3] == 3.0 and abs(o["sigma_max"][3] - 2) < 1e-6 and abs(o["sigma_min"][3] - 2) < 1e-6


def test_diag_partial_outputs_and_determinism(mu):
    A, exact = to_device(stack(77, 6, 256, 384, "spread"), "bf16")
    full = mu.muon_spectral_diag(A, iters=24)
    again = mu.muon_spectral_diag(A, iters=24)
    only = mu.muon_spectral_diag(A, iters=24, sigma_max=False, sigma_min=False)
    smax = mu.muon_spectral_diag(A, iters=24, orth_err=False, sigma_min=False)
    torch.cuda.synchronize()
    for k in full:
        assert torch.equal(full[k], again[k])
    assert set(only) == {"orth_err"} and torch.equal(only["orth_err"], full["orth_err"])
    assert set(smax) == {"sigma_max"} and torch.equal(smax["sigma_max"], full["sigma_max"])


def test_diag_two_chunks(mu):
    """More small matrices than one 2 GiB chunk holds (16384 of 64 x 128):
    every matrix is computed, sampled ones match the oracle."""
    batch = 16384 + 37
    g = torch.Generator().manual_seed(4)
    A = (torch.randn((batch, 64, 128), generator=g) / 11.3).to(torch.bfloat16)
    out = mu.muon_spectral_diag(A.cuda(), iters=64)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in out.items()}
    for k in o:
        assert np.isfinite(o[k]).all()
    idx = [0, 16383, 16384, batch - 1]
    check({k: v[idx] for k, v in o.items()}, t64(A).reshape(batch, 64, 128), 64, idx)


def test_diag_of_newton_schulz_output(mu):
    """The orthogonality error of muon_ns_orthogonalize's result, from the GPU
    diagnostics, equals the oracle's on the same bits and falls with steps."""
    G, exact = to_device(stack(9, 4, 256, 512, "gauss"), "bf16")
    errs = []
    for steps in (1, 3, 5):
        O = torch.empty_like(G)
        mu.muon_ns_orthogonalize(G, O, steps=steps)
        d = mu.muon_spectral_diag(O, iters=16, sigma_max=False, sigma_min=False)
        torch.cuda.synchronize()
        e = d["orth_err"].cpu().numpy()
        ref = [orc.orthogonality_error(t64(O[b])) for b in range(4)]
        assert np.all(np.abs(e - ref) <= ORTH_ABS + ORTH_REL * np.array(ref))
        errs.append(e.mean())
    assert errs[0] > errs[1] > errs[2]


def test_diag_workspace_reuse_across_calls(mu):
    """Three calls on one workspace, with different matrices and step counts
    (the split run's tagged partials of an earlier call must never be taken
    for this call's): every call matches the oracle."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for seed, (m, n, it) in enumerate(((300, 300, 24), (300, 300, 12), (256, 640, 20))):
        A, exact = to_device(stack(100 + seed, 5, m, n, "spread"), "bf16")
        out = mu.muon_spectral_diag(A, iters=it, workspace=ws)
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in out.items()}
        check(out, exact, it, range(5))


@pytest.mark.parametrize("m,n,dtype", [(600, 1000, "bf16"), (1000, 600, "f32")])
def test_diag_three_blocks_ragged(mu, m, n, dtype):
    """s = 600 pads to 640: blocks of 256, 256 and a 128-wide last block with
    88 live rows, whose off-diagonal blocks form row sums with half the lanes
    idle (a few matrices: the split run)."""
    A, exact = to_device(stack(m + 7 * n, 3, m, n, "spread"), dtype)
    out = mu.muon_spectral_diag(A, iters=40)
    torch.cuda.synchronize()
    check({k: v.cpu().numpy() for k, v in out.items()}, exact, 40, range(3))


def test_diag_split_run_agrees_with_one_workgroup_per_matrix(mu):
    """The same matrices as a batch of 4 (several workgroups per matrix) and
    inside a batch of 300 (one workgroup per matrix): both match the oracle
    and each other."""
    A, exact = to_device(stack(41, 4, 384, 704, "spread"), "bf16")
    filler = torch.zeros((296, 384, 704), dtype=A.dtype, device=A.device)
    few = mu.muon_spectral_diag(A, iters=24)
    many = mu.muon_spectral_diag(torch.cat([A, filler]), iters=24)
    torch.cuda.synchronize()
    few = {k: v.cpu().numpy() for k, v in few.items()}
    many = {k: v[:4].cpu().numpy() for k, v in many.items()}
    check(few, exact, 24, range(4))
    check(many, exact, 24, range(4))
    for k in few:
        top = float(np.max(few["sigma_max"])) ** 2
        if k == "orth_err":
            assert np.all(np.abs(few[k] - many[k]) <= ORTH_ABS + ORTH_REL * np.abs(many[k]))
        else:
            assert np.all(np.abs(few[k] ** 2 - many[k] ** 2) <= 2 * THETA_REL * top)


def test_diag_split_run_bounded_waits_give_up_cleanly(mu, monkeypatch):
    """The split run's waits on other workgroups are bounded.  With the bound
    cut to nothing (MUON_DEBUG_DIAG_SPIN_LIMIT, a debug hook read at each
    launch) workgroups give up on words that are not there yet: the call
    still ends, a matrix whose run gave up reports NaN and any other matches
    the oracle, and the next call on the same workspace is exact again.  Only
    the split run waits on other workgroups, so at least one NaN shows that
    the split plan was taken and its give-up path ran."""
    A, exact = to_device(stack(5, 6, 384, 704, "spread"), "bf16")
    ws = torch.zeros(mu.lib().muon_spectral_diag_workspace_size(384, 704, 6, mu.MUON_BF16, 24),
                     dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("MUON_DEBUG_DIAG_SPIN_LIMIT", "0")
    out = mu.muon_spectral_diag(A, iters=24, workspace=ws)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in out.items()}
    gave_up = [b for b in range(6) if not (np.isfinite(o["sigma_max"][b]) and np.isfinite(o["sigma_min"][b]))]
    print("matrices whose run gave up:", gave_up)
    assert len(gave_up) >= 1
    done = [b for b in range(6) if b not in gave_up]
    check({k: v[done] for k, v in o.items()}, exact, 24, done)
    monkeypatch.delenv("MUON_DEBUG_DIAG_SPIN_LIMIT")
    again = mu.muon_spectral_diag(A, iters=24, workspace=ws)
    torch.cuda.synchronize()
    check({k: v.cpu().numpy() for k, v in again.items()}, exact, 24, range(6))
