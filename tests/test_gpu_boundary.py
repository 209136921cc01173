"""GPU tests of the boundary's error reporting and layouts: the non-finite flag
that every muon_step / muon_ns_orthogonalize call leaves in its workspace
(muon_query_flags), and muon_ns_orthogonalize on strided and in-place stacks."""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL, F32_TOL, device_group, grad64, t64, to_torch_bits

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


def _groups(mu, gs):
    devs, groups = [], []
    for g in gs:
        d = device_group(g)
        devs.append(d)
        groups.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], lr=0.02, beta=0.95))
    return devs, groups


def _flag(mu, ws):
    torch.cuda.synchronize()
    return mu.muon_query_flags(ws)


@pytest.mark.parametrize("streams", [0, 1])
def test_nonfinite_flag_set_and_cleared(mu, streams):
    """A NaN in one gradient, then an Inf in one momentum buffer, set the flag
    (in either group, so on either chain of the two-stream run); the next clean
    step on the same workspace clears it."""
    gs = [wl.random_group(41, 2, 768, 1536, "bf16"), wl.random_group(42, 3, 200, 64, "bf16")]
    devs, groups = _groups(mu, gs)
    ws = mu.muon_step(groups, steps=3, streams=streams)
    assert _flag(mu, ws) == 0
    devs[1]["G"][2, 17, 5] = float("nan")
    mu.muon_step(groups, steps=3, streams=streams, workspace=ws)
    assert _flag(mu, ws) == 1
    devs[1]["G"].copy_(to_torch_bits(gs[1].G).cuda())
    devs[1]["M"].copy_(torch.from_numpy(gs[1].M).cuda())
    for d, g in zip(devs, gs):
        d["W"].copy_(torch.from_numpy(g.W).cuda())
    mu.muon_step(groups, steps=3, streams=streams, workspace=ws)
    assert _flag(mu, ws) == 0
    devs[0]["M"][1, 700, 3] = float("inf")
    mu.muon_step(groups, steps=3, streams=streams, workspace=ws)
    assert _flag(mu, ws) == 1


def test_nonfinite_flag_of_ns_orthogonalize(mu):
    g = wl.random_group(43, 2, 64, 96, "f32")
    G = torch.from_numpy(g.G).cuda()
    O = torch.empty_like(G)
    ws = mu.muon_ns_orthogonalize(G, O, steps=2)
    assert _flag(mu, ws) == 0
    G[1, 3, 3] = float("-inf")
    mu.muon_ns_orthogonalize(G, O, steps=2, workspace=ws)
    assert _flag(mu, ws) == 1
    assert torch.isfinite(O[0]).all()


@pytest.mark.parametrize("m,n,dt,pad_n", [(768, 1536, "bf16", 24), (3352, 768, "bf16", 24), (130, 200, "bf16", 3),
                                          (96, 200, "f32", 5), (64, 128, "bf16", 24), (48, 40, "f32", 8)])
def test_ns_orthogonalize_strided_and_in_place(mu, m, n, dt, pad_n):
    """A stack whose rows are ld > n elements apart and whose matrices are
    stride > m ld apart (views into a wider buffer): the result equals the
    contiguous call bitwise, only the view's elements are written, and the
    in-place call (O = G) gives the same bits."""
    g = wl.random_group(50 + m, 3, m, n, dt)
    Gc = (to_torch_bits(g.G) if dt == "bf16" else torch.from_numpy(g.G)).cuda()
    Oc = torch.empty_like(Gc)
    mu.muon_ns_orthogonalize(Gc, Oc, steps=5)
    pad_m = 5
    big = torch.zeros((3, m + pad_m, n + pad_n), dtype=Gc.dtype, device="cuda")
    big[:, :m, :n] = Gc
    Gv = big[:, :m, :n]
    outbig = torch.full_like(big, 7.0)
    Ov = outbig[:, :m, :n]
    assert Gv.stride() == ((m + pad_m) * (n + pad_n), n + pad_n, 1)
    mu.muon_ns_orthogonalize(Gv, Ov, steps=5)
    mu.muon_ns_orthogonalize(Gv, Gv, steps=5)  # in place
    torch.cuda.synchronize()
    assert torch.equal(Ov, Oc)
    assert torch.equal(Gv, Oc)
    mask = torch.ones_like(outbig, dtype=torch.bool)
    mask[:, :m, :n] = False
    assert bool((outbig[mask] == 7.0).all())
    assert bool((big[mask] == 0).all())
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    for i in range(3):
        ref, _ = orc.newton_schulz(grad64(g, i), 5)
        assert orc.rel_frobenius(t64(Ov[i]), ref) <= tol
