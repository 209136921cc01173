"""GPU parity: libmuon (through its C ABI) against the fp64 oracle.

Every case runs the HIP path on seeded synthetic inputs and compares it with
oracle/muon_oracle.py on the same bits: O (the orthogonalised update) by
relative Frobenius error (<= 1e-5 fp32, <= 2e-2 bf16 matrix cores), the
momentum buffer (<= 1e-6) and the weight increment.  The five benchmark
workloads are compared on every matrix (the injections in streamed chunks),
and each prints the largest singular-value deviation max_i |sigma_i(O_gpu) -
sigma_i(O_oracle)| of its updates (reported, not gated).
"""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL, F32_TOL, Report, compare_step, device_group, grad64, sigma_deviation, t64, \
    to_torch_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spectral_optimizer_ssm_amd as mu
    mu.lib()  # raises if the HIP library is missing
    return mu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield


SCHEDULES = ["iterate", "accumulate"]


def sched(mu, name):
    return {"auto": mu.MUON_NS_AUTO, "iterate": mu.MUON_NS_ITERATE, "accumulate": mu.MUON_NS_ACCUMULATE}[name]


def run_step(mu, w, precision=None, steps=None, want_o=True, coeffs=None, eps=None, schedule="auto"):
    """Run one muon_step over all groups of a workload; returns (devs, outs)."""
    devs, outs, groups = [], [], []
    prec = precision if precision is not None else (mu.MUON_BF16 if w.groups[0].grad_dtype == "bf16" else mu.MUON_F32)
    for g in w.groups:
        d = device_group(g)
        odt = torch.bfloat16 if prec == mu.MUON_BF16 else torch.float32
        o = {"O": torch.full((g.count, g.m, g.n), float("nan"), dtype=odt, device="cuda")} if want_o else {"O": None}
        devs.append(d)
        outs.append(o)
        groups.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], O=o["O"], lr=w.lr, beta=w.beta,
                                   scale=w.scale, nesterov=w.nesterov))
    mu.muon_step(groups, steps=w.steps if steps is None else steps, coeffs=coeffs or w.coeffs,
                 eps=w.eps if eps is None else eps, precision=prec, schedule=sched(mu, schedule),
                 per_step=w.per_step)
    torch.cuda.synchronize()
    return devs, outs


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def test_single_fp32_128x64(mu):
    w = wl.config1()
    devs, outs = run_step(mu, w)
    res, _ = compare_step(w.groups[0], 0, outs[0], devs[0], w, F32_TOL, sigma=True)
    rep = Report("single fp32 128x64")
    rep.add(res)
    print(rep.line())


def _all_matrices(w, devs, outs, name, steps=None, only=None):
    rep = Report(name)
    for gi, g in enumerate(w.groups):
        for i in (range(g.count) if only is None else only):
            res, _ = compare_step(g, i, outs[gi], devs[gi], w, BF16_TOL, steps=steps, sigma=True)
            rep.add(res)
    print(rep.line(), flush=True)
    return rep


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_out_proj_group_full(mu, schedule):
    w = wl.config2()
    devs, outs = run_step(mu, w, schedule=schedule)
    assert _all_matrices(w, devs, outs, f"out_proj 24x768x1536 {schedule}").n == 24


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_in_proj_group_full_tall(mu, schedule):
    w = wl.config3()
    devs, outs = run_step(mu, w, schedule=schedule)
    assert _all_matrices(w, devs, outs, f"in_proj 24x3352x768 {schedule}").n == 24


@pytest.fixture(scope="module")
def full_step_inputs():
    return wl.config4()


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("steps", [1, 2, 3, 5, 8])
def test_full_mamba2_step(mu, full_step_inputs, steps, schedule):
    """Every one of the 48 matrices at the benchmark's 5 steps; matrices 0 and
    17 of each group at the other step counts."""
    w = full_step_inputs
    devs, outs = run_step(mu, w, steps=steps, schedule=schedule)
    rep = _all_matrices(w, devs, outs, f"full step 24+24, {steps} steps {schedule}", steps=steps,
                        only=None if steps == 5 else (0, 17))
    assert rep.n == (48 if steps == 5 else 4)


def test_full_mamba2_step_zero_momentum_closed_form(mu):
    """With M = 0, U = (1 + beta) G and G = U diag(s) V^T by construction, so
    the oracle's update is the singular-value closed form; the GPU must match
    the oracle, and the oracle the closed form (up to the bf16 rounding of G)."""
    w = wl.config4(count=2, zero_momentum=True)
    devs, outs = run_step(mu, w)
    for gi, g in enumerate(w.groups):
        for i in range(2):
            compare_step(g, i, outs[gi], devs[gi], w, BF16_TOL)


def test_orthogonality_error_vs_steps_closed_form(mu):
    """Orthogonality error ||O O^T - I||_F / sqrt(s) of the update after 1, 3,
    5 and 8 steps with M = 0: the GPU's (muon_spectral_diag of the bf16 O),
    the oracle's (its fp64 O), and the closed form from the singular values
    of the rounded gradient (U = (1 + beta) G, X0 = U / (||U||_F + eps),
    every singular value x through p^k).  Oracle and closed form agree to
    rounding; the GPU follows within the bf16 update tolerance; the error
    falls with the step count."""
    w = wl.config4(count=2, zero_momentum=True)
    a, b = w.coeffs
    prev = {}
    for steps in (1, 3, 5, 8):
        devs, outs = run_step(mu, w, steps=steps)
        for gi, g in enumerate(w.groups):
            d = mu.muon_spectral_diag(outs[gi]["O"], iters=16, sigma_max=False, sigma_min=False)
            torch.cuda.synchronize()
            e_gpu = float(d["orth_err"][0].cpu())
            G = grad64(g, 0)
            ref = orc.muon_step(orc.widen_f32(g.W[0]), np.zeros_like(G), G, beta=w.beta, lr=w.lr,
                                nesterov=w.nesterov, steps=steps, coeffs=w.coeffs, eps=w.eps)
            e_orc = orc.orthogonality_error(ref["O"])
            sig = (1 + w.beta) * np.linalg.svd(G, compute_uv=False)
            x = sig / (np.sqrt(np.sum(sig * sig)) + w.eps)
            for _ in range(steps):
                x = a * x + b * x ** 3
            e_cf = float(np.sqrt(np.sum((x * x - 1.0) ** 2) / x.size))
            print(g.name, steps, "orth gpu %.5f oracle %.5f closed form %.5f" % (e_gpu, e_orc, e_cf))
            assert abs(e_orc - e_cf) <= 1e-9 * max(1.0, e_cf)
            assert abs(e_gpu - e_orc) <= 2e-2 * e_orc
            assert e_gpu < prev.get(g.name, np.inf)
            prev[g.name] = e_gpu


@pytest.mark.parametrize("tall", [False, True])
def test_max_size_block_diagonal(mu, tall):
    """The largest accepted matrix-core shape, 16384 x 65280 (the padded bf16
    iterate just under 2 GiB), one matrix, M = W = 0, a gradient of 256 blocks
    of 64 x 255 on the diagonal.  The Frobenius normalisation is global and
    every Gram X X^T is block diagonal, so the update is block diagonal, each
    block the Newton-Schulz iterate of its own block scaled by the norm of
    the whole matrix: the oracle iterates each block; entries outside the
    blocks must be exactly zero, and the weight increment is exactly
    -lr * O (float32 product of the bf16 update)."""
    s, l, nb = 16384, 65280, 256
    bs, bl = s // nb, l // nb
    rng = np.random.default_rng(11)
    bits = wl.f64_to_bf16_bits(rng.standard_normal((nb, bs, bl)) / np.sqrt(bl))
    exact = orc.widen_bf16(bits)
    beta, lr = 0.95, 0.02
    nu = (1 + beta) * np.sqrt(np.sum(exact * exact))
    ref = np.stack([orc.ns_iterate((1 + beta) * exact[b] / (nu + 1e-7), 5) for b in range(nb)])
    idx = torch.arange(nb, device="cuda")
    Gw = torch.zeros((s, l), dtype=torch.bfloat16, device="cuda")
    Gw.view(nb, bs, nb, bl)[idx, :, idx, :] = to_torch_bits(bits).cuda()
    G = (Gw.t().contiguous() if tall else Gw).unsqueeze(0)
    del Gw
    m, n = G.shape[1:]
    W = torch.zeros((1, m, n), dtype=torch.float32, device="cuda")
    M = torch.zeros_like(W)
    O = torch.full((1, m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    mu.muon_step([mu.MuonGroup(W=W, M=M, G=G, O=O, lr=lr, beta=beta, nesterov=True)], steps=5)
    torch.cuda.synchronize()
    Ow = O[0].t() if tall else O[0]
    blocks = Ow.reshape(nb, bs, nb, bl)[idx, :, idx, :] if not tall else \
        torch.stack([Ow[b * bs:(b + 1) * bs, b * bl:(b + 1) * bl] for b in range(nb)])
    err = orc.rel_frobenius(t64(blocks), ref)
    print("max size", "tall" if tall else "wide", "rel_F", err, flush=True)
    assert err <= BF16_TOL
    O2 = O.clone()
    O2v = (O2[0].t() if tall else O2[0])
    if tall:
        for b in range(nb):
            O2v[b * bs:(b + 1) * bs, b * bl:(b + 1) * bl] = 0
    else:
        O2v.view(nb, bs, nb, bl)[idx, :, idx, :] = 0
    assert int(torch.count_nonzero(O2)) == 0
    del O2
    assert torch.equal(W, O.float() * torch.tensor(-lr, dtype=torch.float32, device="cuda"))
    assert torch.equal(M, G.float())


def _injection_oracle(X, steps=1):
    return orc.ns_batched(X.float().cpu().numpy().astype(np.float64), steps)


def _rel_rows(Y, ref):
    """Relative Frobenius error of every matrix of two [b, m, n] stacks."""
    num = np.sqrt(np.sum((Y - ref) ** 2, axis=(1, 2)))
    den = np.sqrt(np.sum(ref ** 2, axis=(1, 2)))
    return num / np.where(den == 0, 1.0, den)


def test_injections_reduced_all_matrices(mu):
    X = wl.injections(batch=4096, device="cuda")
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=1)
    torch.cuda.synchronize()
    ref = _injection_oracle(X, 1)
    errs = _rel_rows(t64(Y), ref)
    print("max rel", errs.max(), "mean", errs.mean())
    assert errs.max() <= BF16_TOL


@pytest.fixture(scope="module")
def injections_full(mu):
    X = wl.injections(device="cuda")
    assert X.shape[0] == 393216
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=1)
    torch.cuda.synchronize()
    return X, Y


@pytest.mark.parametrize("quarter", range(4))
def test_injections_full_size_every_matrix(mu, injections_full, quarter):
    """All 393,216 injections, a quarter per test, against the oracle in
    chunks of 8,192 matrices; the singular-value deviation on a seeded sample
    of 1,024 matrices of the quarter (and the first and last matrix)."""
    X, Y = injections_full
    q = X.shape[0] // 4
    lo, hi = quarter * q, (quarter + 1) * q
    worst = 0.0
    for c0 in range(lo, hi, 8192):
        c1 = min(hi, c0 + 8192)
        ref = _injection_oracle(X[c0:c1], 1)
        errs = _rel_rows(t64(Y[c0:c1]), ref)
        worst = max(worst, float(errs.max()))
        assert errs.max() <= BF16_TOL, (c0, int(errs.argmax()))
    rng = np.random.default_rng(2024 + quarter)
    idx = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 1024)]))
    it = torch.from_numpy(idx).cuda()
    ref = _injection_oracle(X[it], 1)
    Yd = t64(Y[it])
    sdev = max(sigma_deviation(Yd[k], ref[k]) for k in range(len(idx)))
    assert torch.isfinite(Y[lo:hi].float()).all()
    print(f"[parity] injections {lo}..{hi - 1}: {hi - lo} matrices compared, max_O {worst:.3e}, "
          f"max_sigma_dev {sdev:.3e} ({len(idx)} sampled)", flush=True)


@pytest.mark.parametrize("steps", [0, 1, 3, 5])
@pytest.mark.parametrize("shape", [(64, 128), (32, 96), (64, 64), (32, 256)])
def test_batched_small_bf16_shapes(mu, shape, steps):
    m, n = shape
    g = wl.random_group(7 + m + n, 37, m, n, "bf16")
    X = to_torch_bits(g.G).cuda()
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=steps)
    torch.cuda.synchronize()
    Yd = t64(Y)
    for b in (0, 18, 36):
        ref, _ = orc.newton_schulz(grad64(g, b), steps)
        assert orc.rel_frobenius(Yd[b], ref) <= BF16_TOL


@pytest.mark.parametrize("steps", [1, 5])
@pytest.mark.parametrize("shape", [(96, 192), (128, 256), (128, 512), (96, 96), (32, 512), (64, 320), (64, 192)])
def test_batched_small_bf16_wide_shapes(mu, shape, steps):
    """Short sides 96 and 128, and long sides beyond 256, on the on-chip
    kernel with a runtime long side: every matrix against the oracle."""
    m, n = shape
    g = wl.random_group(17 + m + n, 9, m, n, "bf16")
    X = to_torch_bits(g.G).cuda()
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=steps)
    torch.cuda.synchronize()
    Yd = t64(Y)
    worst = sdev = 0.0
    for b in range(9):
        ref, _ = orc.newton_schulz(grad64(g, b), steps)
        worst = max(worst, orc.rel_frobenius(Yd[b], ref))
        sdev = max(sdev, sigma_deviation(Yd[b], ref))
    print(f"[parity] batched_small {m}x{n} steps {steps}: max_O {worst:.3e} max_sigma_dev {sdev:.3e}", flush=True)
    assert worst <= BF16_TOL


# rows split over the waves (three sizes of X in LDS); columns split
@pytest.mark.parametrize("shape", [(96, 96), (128, 256), (96, 320), (128, 512)])
@pytest.mark.parametrize("steps", [1, 3])
def test_batched_small_bf16_past_the_grid(mu, shape, steps):
    """More matrices than the 65,536 workgroups of one launch: each workgroup
    takes a second matrix; samples on both sides of index 65,536 against the
    oracle and every matrix finite."""
    m, n = shape
    count = 70000
    gen = torch.Generator(device="cuda").manual_seed(m + n + steps)
    X = torch.randn((count, m, n), generator=gen, device="cuda").to(torch.bfloat16)
    Y = torch.empty_like(X)
    print(f"[parity] past the grid {m}x{n} steps {steps}", flush=True)
    mu.muon_ns_batched_small(X, Y, steps=steps)
    torch.cuda.synchronize()
    assert torch.isfinite(Y.float()).all()
    for b in (0, 1, 65535, 65536, 65537, count - 1):
        ref, _ = orc.newton_schulz(t64(X[b]), steps)
        assert orc.rel_frobenius(t64(Y[b]), ref) <= BF16_TOL, b


@pytest.mark.parametrize("steps", [0, 1, 5])
@pytest.mark.parametrize("shape", [(128, 512), (96, 300), (300, 96), (128, 128), (100, 100), (1, 70), (33, 500),
                                   (512, 128), (64, 320), (70, 20)])
def test_small_bf16_groups_on_chip(mu, shape, steps):
    """bf16 groups with short side up to 128 and long side up to 512 run on
    chip, both sides padded with zeros to multiples of 32: W, M and O of
    every matrix against the oracle."""
    m, n = shape
    g = wl.random_group(400 + m + n, 5, m, n, "bf16")
    w = wl.Workload(f"small{m}x{n}", [g], steps=steps)
    devs, outs = run_step(mu, w)
    for i in range(5):
        compare_step(g, i, outs[0], devs[0], w, BF16_TOL)


@pytest.mark.parametrize("shape", [(128, 64), (64, 128), (40, 200), (200, 40), (7, 33)])
def test_batched_small_fp32(mu, shape):
    m, n = shape
    g = wl.random_group(11 + m, 5, m, n, "f32")
    X = torch.from_numpy(g.G).cuda()
    Y = torch.empty_like(X)
    mu.muon_ns_batched_small(X, Y, steps=5)
    torch.cuda.synchronize()
    Yd = t64(Y)
    for b in range(5):
        ref, _ = orc.newton_schulz(grad64(g, b), 5)
        assert orc.rel_frobenius(Yd[b], ref) <= F32_TOL


# ---------------------------------------------------------------------------
# ragged shapes, both engines, both precisions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("shape", [(200, 130), (96, 300), (130, 130), (1, 70), (300, 1), (256, 512),
                                   (64, 128), (128, 64), (513, 129), (520, 1100)])
def test_ragged_bf16(mu, shape, schedule):
    m, n = shape
    g = wl.random_group(100 + m + n, 3, m, n, "bf16")
    w = wl.Workload(f"ragged{m}x{n}", [g])
    devs, outs = run_step(mu, w, schedule=schedule)
    for i in range(3):
        compare_step(g, i, outs[0], devs[0], w, BF16_TOL)


@pytest.mark.parametrize("shape", [(100, 150), (150, 100), (64, 64), (65, 300), (128, 64)])
def test_ragged_fp32(mu, shape):
    m, n = shape
    g = wl.random_group(200 + m + n, 2, m, n, "f32")
    w = wl.Workload(f"ragged{m}x{n}", [g])
    devs, outs = run_step(mu, w)
    for i in range(2):
        compare_step(g, i, outs[0], devs[0], w, F32_TOL)


def test_bf16_gradients_fp32_iterate(mu):
    g = wl.random_group(5, 2, 96, 160, "bf16")
    w = wl.Workload("mixed", [g])
    devs, outs = run_step(mu, w, precision=mu.MUON_F32)
    for i in range(2):
        compare_step(g, i, outs[0], devs[0], w, F32_TOL)


def test_many_matrices_multiple_tables(mu):
    g = wl.random_group(9, 70, 64, 96, "bf16")  # more than one pointer table
    w = wl.Workload("many", [g])
    devs, outs = run_step(mu, w)
    for i in (0, 63, 64, 69):
        compare_step(g, i, outs[0], devs[0], w, BF16_TOL)


# ---------------------------------------------------------------------------
# degenerate inputs and invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(256, 384), (50, 70), (100, 100)])  # matrix cores; on chip, one wave / rows split
def test_zero_gradient_leaves_weights(mu, shape):
    g = wl.random_group(1, 2, *shape, "bf16", zero_momentum=True)
    g.G[:] = 0
    w = wl.Workload("zero", [g])
    devs, outs = run_step(mu, w)
    assert torch.equal(devs[0]["W"].cpu(), torch.from_numpy(g.W))
    assert (outs[0]["O"].float() == 0).all()


@pytest.mark.parametrize("shape", [(128, 256), (50, 70), (100, 100), (128, 512)])
def test_nan_propagates(mu, shape):
    g = wl.random_group(2, 1, *shape, "bf16")
    g.G[0, 3, 5] = 0x7FC0
    w = wl.Workload("nan", [g])
    devs, outs = run_step(mu, w)
    assert torch.isnan(devs[0]["W"]).all()


def test_transpose_equivariance(mu):
    g = wl.random_group(3, 2, 256, 640, "bf16", zero_momentum=True)
    G = to_torch_bits(g.G).cuda()
    O1 = torch.empty_like(G)
    mu.muon_ns_orthogonalize(G, O1, steps=5)
    Gt = G.transpose(1, 2).contiguous()
    O2 = torch.empty_like(Gt)
    mu.muon_ns_orthogonalize(Gt, O2, steps=5)
    torch.cuda.synchronize()
    for i in range(2):
        a, b = t64(O1[i]), t64(O2[i]).T
        assert orc.rel_frobenius(a, b) <= BF16_TOL
        ref, _ = orc.newton_schulz(grad64(g, i), 5)
        assert orc.rel_frobenius(a, ref) <= BF16_TOL


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_ns_orthogonalize_matches_oracle(mu, schedule):
    for m, n, dt in ((768, 1536, "bf16"), (3352, 768, "bf16"), (96, 200, "f32")):
        g = wl.random_group(m + n, 2, m, n, dt)
        G = (to_torch_bits(g.G) if dt == "bf16" else torch.from_numpy(g.G)).cuda()
        O = torch.empty_like(G)
        mu.muon_ns_orthogonalize(G, O, steps=5, schedule=sched(mu, schedule))
        torch.cuda.synchronize()
        for i in range(2):
            ref, _ = orc.newton_schulz(grad64(g, i), 5)
            assert orc.rel_frobenius(t64(O[i]), ref) <= (BF16_TOL if dt == "bf16" else F32_TOL)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_deterministic(mu, schedule):
    w = wl.config2(count=3)
    d1, o1 = run_step(mu, w, schedule=schedule)
    d2, o2 = run_step(mu, w, schedule=schedule)
    assert torch.equal(o1[0]["O"], o2[0]["O"])
    assert torch.equal(d1[0]["W"], d2[0]["W"])
    assert torch.equal(d1[0]["M"], d2[0]["M"])


def test_norms_out_and_resume(mu):
    g = wl.random_group(4, 3, 200, 300, "bf16")
    d = device_group(g)
    norms = torch.zeros(3, device="cuda")
    grp = mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], lr=0.02, beta=0.95)
    mu.muon_step([grp], steps=5, norms_out=norms)
    torch.cuda.synchronize()
    for i in range(3):
        U = orc.update_direction(grad64(g, i), orc.momentum(orc.widen_f32(g.M[i]), grad64(g, i), 0.95), 0.95, True)
        assert abs(norms[i].item() - np.linalg.norm(U)) <= 1e-5 * np.linalg.norm(U)
    # resume: saving and restoring W, M between two steps equals running on
    W1, M1 = d["W"].clone(), d["M"].clone()
    mu.muon_step([grp], steps=5)
    torch.cuda.synchronize()
    W2a = d["W"].clone()
    d["W"].copy_(W1)
    d["M"].copy_(M1)
    mu.muon_step([grp], steps=5)
    torch.cuda.synchronize()
    assert torch.equal(d["W"], W2a)


def test_two_groups_one_call(mu):
    w = wl.config4(count=3, out_shape=(128, 256), in_shape=(400, 128))
    devs, outs = run_step(mu, w)
    for gi, g in enumerate(w.groups):
        for i in range(3):
            compare_step(g, i, outs[gi], devs[gi], w, BF16_TOL)


def test_mixed_schedules_one_call(mu):
    """One call whose groups take the accumulated schedule (768 x 1536), the
    iterated one (512 x 512) and the on-chip kernel (64 x 128)."""
    groups = [wl.random_group(31, 2, 768, 1536, "bf16"), wl.random_group(32, 2, 512, 512, "bf16"),
              wl.random_group(33, 3, 64, 128, "bf16")]
    w = wl.Workload("mixed-schedules", groups)
    fake = [mu.MuonGroup(W=torch.empty(g.count, g.m, g.n), M=torch.empty(g.count, g.m, g.n),
                         G=torch.empty(g.count, g.m, g.n, dtype=torch.bfloat16), lr=w.lr, beta=w.beta)
            for g in groups]
    phases = mu.muon_step_phases(fake, steps=5)
    assert phases.count("symprod") == 9 and phases.count("gram") == 6 and phases.count("ns_small") == 1
    devs, outs = run_step(mu, w)
    for gi, g in enumerate(groups):
        for i in range(g.count):
            compare_step(g, i, outs[gi], devs[gi], w, BF16_TOL)


def test_timed_events_cover_phases(mu):
    """muon_step_timed needs one event per phase plus one, and rejects fewer."""
    w = wl.config4(count=2)
    groups = []
    for g in w.groups:
        d = device_group(g)
        groups.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], lr=w.lr, beta=w.beta))
    phases = mu.muon_step_phases(groups, steps=5)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    with pytest.raises(mu.MuonError):
        mu.muon_step(groups, steps=5, events=[e.cuda_event for e in evs[:-1]])
    mu.muon_step(groups, steps=5, events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    times = [evs[k].elapsed_time(evs[k + 1]) for k in range(len(phases))]
    assert all(t >= 0 for t in times)


# ---------------------------------------------------------------------------
# quintic and per-step coefficients (large bf16 matrices, both schedules)
# ---------------------------------------------------------------------------
QUINTIC = (2.0, -1.5, 0.5)
ROWS = [(2.0, -1.5, 0.5), (1.875, -1.25, 0.375), (1.5, -0.5, 0.0)]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("coeffs,per_step,steps", [(QUINTIC, False, 3), (QUINTIC, False, 5), (ROWS, True, 3)])
def test_quintic_mamba2_shapes(mu, schedule, coeffs, per_step, steps):
    w = wl.config4(count=3)
    w.coeffs, w.per_step, w.steps = coeffs, per_step, steps
    devs, outs = run_step(mu, w, schedule=schedule)
    for gi, g in enumerate(w.groups):
        for i in (0, 2):
            res, _ = compare_step(g, i, outs[gi], devs[gi], w, BF16_TOL)
            print(g.name, i, schedule, steps, res)


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("shape", [(256, 512), (520, 1100), (300, 257), (64, 128), (96, 300)])
def test_quintic_ragged(mu, schedule, shape):
    m, n = shape
    g = wl.random_group(300 + m + n, 2, m, n, "bf16")
    w = wl.Workload(f"quintic{m}x{n}", [g], coeffs=QUINTIC, steps=4)
    devs, outs = run_step(mu, w, schedule=schedule)
    for i in range(2):
        compare_step(g, i, outs[0], devs[0], w, BF16_TOL)


def test_quintic_unsupported_paths(mu):
    """c != 0 with float32 precision is refused before any work."""
    for m, n, dt, prec in ((96, 160, "f32", None), (300, 400, "bf16", "f32")):
        g = wl.random_group(7, 1, m, n, dt)
        w = wl.Workload("q", [g], coeffs=QUINTIC, steps=2)
        with pytest.raises(mu.MuonError) as e:
            run_step(mu, w, precision=mu.MUON_F32 if prec == "f32" else None)
        assert e.value.status == mu.binding.MUON_EUNSUPPORTED


def test_two_stream_chains_match_one_stream(mu):
    """muon_step runs independent shape groups as two chains on two streams by
    default; the results are bitwise those of the one-stream run, and
    norms_out keeps its order."""
    w = wl.config4(count=3)
    outs = []
    for streams in (1, 0):
        groups, devs = [], []
        for g in w.groups:
            d = device_group(g)
            devs.append(d)
            groups.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], lr=w.lr, beta=w.beta))
        norms = torch.zeros(6, device="cuda")
        mu.muon_step(groups, steps=5, norms_out=norms, streams=streams)
        torch.cuda.synchronize()
        outs.append((devs, norms))
    (d1, n1), (d2, n2) = outs
    assert torch.equal(n1, n2)
    for a, b in zip(d1, d2):
        assert torch.equal(a["W"], b["W"]) and torch.equal(a["M"], b["M"])
    for gi, g in enumerate(w.groups):
        U = orc.update_direction(grad64(g, 1), orc.momentum(orc.widen_f32(g.M[1]), grad64(g, 1), 0.95), 0.95, True)
        assert abs(n2[3 * gi + 1].item() - np.linalg.norm(U)) <= 1e-5 * np.linalg.norm(U)


@pytest.mark.parametrize("shapes,schedule", [
    ([(768, 1536, 3), (3352, 768, 3)], "accumulate"),   # the Mamba-2 projections
    ([(768, 1536, 2), (3352, 768, 2)], "iterate"),
    ([(200, 516, 3)], "iterate"),                        # ragged wide, n % 8 != 0: unvectorised edge
    ([(516, 200, 3)], "accumulate"),                     # ragged tall
    ([(260, 1000, 2), (1000, 260, 2)], "accumulate"),    # padded tiles on both sides
])
def test_fused_apply_matches_separate_pass(mu, shapes, schedule):
    """The final combine applies the update in its epilogue (W, and the copy to
    O); the separate apply pass gives bitwise the same W, M and O."""
    sch = mu.MUON_NS_ACCUMULATE if schedule == "accumulate" else mu.MUON_NS_ITERATE
    groups = [wl._group(70 + i, c, m, n, "gauss", f"g{i}") for i, (m, n, c) in enumerate(shapes)]
    outs = []
    for sep in (1, 0):
        devs, gs = [], []
        for g in groups:
            d = device_group(g)
            d["O"] = torch.full((g.count, g.m, g.n), float("nan"), dtype=torch.bfloat16, device="cuda")
            devs.append(d)
            gs.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], O=d["O"], lr=0.02, beta=0.95))
        assert mu.muon_step_phases(gs, steps=5, schedule=sch, separate_apply=sep)[-1] == \
            ("apply" if sep else "combine_apply")
        mu.muon_step(gs, steps=5, schedule=sch, separate_apply=sep)
        torch.cuda.synchronize()
        outs.append(devs)
    for a, b in zip(*outs):
        for key in ("W", "M", "O"):
            assert torch.equal(a[key], b[key]), key
    # and against the oracle on one matrix per group
    for g, d in zip(groups, outs[1]):
        ref = orc.muon_step(orc.widen_f32(g.W[0]), orc.widen_f32(g.M[0]), grad64(g, 0), beta=0.95, lr=0.02, steps=5)
        assert orc.rel_frobenius(t64(d["O"][0]), ref["O"]) <= BF16_TOL
        assert orc.rel_frobenius(t64(d["W"][0]) - orc.widen_f32(g.W[0]), ref["W"] - orc.widen_f32(g.W[0])) <= BF16_TOL
