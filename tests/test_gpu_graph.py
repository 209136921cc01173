"""muon_step captured in a HIP graph (torch.cuda.CUDAGraph): the call makes no
allocation, memset or host synchronisation, and its two-chain fork/join runs
on events, so a training loop can capture the optimizer step and replay it.
Every replay is checked bitwise against the same step run eagerly, with eager
work and synchronisations between the replays."""
import pytest

import workloads as wl
from helpers import device_group

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


def _groups(mu, gs, cap=False):
    devs, groups = [], []
    for g in gs:
        d = device_group(g)
        devs.append(d)
        extra = {}
        if cap:
            u = torch.randn(g.count, g.m, device="cuda")
            v = torch.randn(g.count, g.n, device="cuda")
            d["u"], d["v"] = u / u.norm(dim=1, keepdim=True), v / v.norm(dim=1, keepdim=True)
            d["s"] = torch.full((g.count,), 10.0, device="cuda")
            extra = dict(cap_u=d["u"], cap_v=d["v"], cap_sigma=d["s"], cap=1.0)
        groups.append(mu.MuonGroup(W=d["W"], M=d["M"], G=d["G"], lr=0.02, beta=0.95, **extra))
    return devs, groups


@pytest.mark.parametrize("cap", [False, True])
def test_graph_replay_equals_eager(mu, cap):
    """Three shape groups (a wide and a tall matrix-core group and an on-chip
    group: two chains on two streams), 5 NS steps, the accumulated schedule;
    with the spectral cap, also its power-step state."""
    gs = [wl.random_group(61, 4, 256, 512, "bf16"), wl.random_group(62, 4, 600, 256, "bf16"),
          wl.random_group(63, 8, 64, 128, "bf16")]
    gdev, ggroups = _groups(mu, gs, cap)
    edev, egroups = _groups(mu, gs, cap)
    if cap:  # same random cap state on both sides
        for a, b in zip(gdev, edev):
            for k in ("u", "v", "s"):
                b[k].copy_(a[k])
    ws_g = mu.muon_step(ggroups, steps=5)  # first call: workspace, auxiliary stream and events exist
    ws_e = mu.muon_step(egroups, steps=5)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mu.muon_step(ggroups, steps=5, workspace=ws_g)
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        mu.muon_step(egroups, steps=5, workspace=ws_e)
        torch.cuda.synchronize()
        for a, b in zip(gdev, edev):
            assert torch.equal(a["W"], b["W"]), rep
            assert torch.equal(a["M"], b["M"]), rep
            if cap:
                for k in ("u", "v", "s"):
                    assert torch.equal(a[k], b[k]), (rep, k)
        assert mu.muon_query_flags(ws_g) == 0
