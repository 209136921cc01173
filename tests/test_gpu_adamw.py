"""GPU parity of muon_adamw against the fp64 oracle (oracle.adamw_step).

The kernel runs in float32 on exactly widened inputs, so the moments are held
to 1e-6 and the parameter increment to 1e-5 (relative Frobenius), over several
consecutive steps."""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import F32_TOL, MOM_TOL, t64, to_torch_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KW = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


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


def run_and_check(mu, shapes, grad_dtype, steps, idx=None):
    P, G, M, V = wl.adamw_state(shapes, seed=len(shapes), grad_dtype=grad_dtype)
    dev = lambda a: torch.from_numpy(a.copy()).cuda()  # noqa: E731
    Pd, Md, Vd = [dev(p) for p in P], [dev(m) for m in M], [dev(v) for v in V]
    Gd = [(to_torch_bits(g) if grad_dtype == "bf16" else torch.from_numpy(g)).cuda() for g in G]
    ref = [(orc.widen_f32(p), orc.widen_f32(m), orc.widen_f32(v)) for p, m, v in zip(P, M, V)]
    for t in range(1, steps + 1):
        mu.muon_adamw(Pd, Gd, Md, Vd, step=t, **KW)
        gw = [orc.widen_bf16(g) if grad_dtype == "bf16" else orc.widen_f32(g) for g in G]
        ref = [orc.adamw_step(p, g, m, v, step=t, **KW) for (p, m, v), g in zip(ref, gw)]
    torch.cuda.synchronize()
    for i in (range(len(shapes)) if idx is None else idx):
        p0 = orc.widen_f32(P[i])
        assert orc.rel_frobenius(t64(Pd[i]) - p0, ref[i][0] - p0) <= F32_TOL, i
        assert orc.rel_frobenius(t64(Md[i]), ref[i][1]) <= MOM_TOL, i
        assert orc.rel_frobenius(t64(Vd[i]), ref[i][2]) <= MOM_TOL, i


@pytest.mark.parametrize("grad_dtype", ["bf16", "f32"])
def test_adamw_assorted_sizes(mu, grad_dtype):
    shapes = [(f"t{k}", (n,)) for k, n in enumerate([1, 3, 4, 5, 4095, 4096, 4097, 12288, 100003, 7, 65536])]
    run_and_check(mu, shapes, grad_dtype, steps=3)


def test_adamw_many_tensors_several_launches(mu):
    shapes = [(f"t{k}", (1000 + 37 * k,)) for k in range(175)]  # three launches of up to 80 tensors
    run_and_check(mu, shapes, "bf16", steps=2)


def test_adamw_mamba2_non_muon_parameters(mu):
    shapes = wl.mamba2_adamw_shapes()
    assert sum(int(np.prod(s)) for _, s in shapes) == 38887872
    run_and_check(mu, shapes, "bf16", steps=2, idx=[0, 1, 2, 3, 4, len(shapes) - 1, 77])


def test_adamw_unaligned_views(mu):
    """Tensors that start at odd element offsets take the scalar path."""
    base = torch.zeros(5003, device="cuda")
    p = base[1:4002]
    g = torch.ones(4001, device="cuda").to(torch.bfloat16)
    m, v = torch.zeros(4001, device="cuda"), torch.zeros(4001, device="cuda")
    p.fill_(1.0)
    mu.muon_adamw([p], [g], [m], [v], step=1, **KW)
    torch.cuda.synchronize()
    expect = 1.0 * (1 - 3e-3 * 0.1) - 3e-3 * 1.0 / (1.0 + 1e-8)
    assert torch.allclose(p, torch.full_like(p, expect), rtol=1e-6, atol=0)
    assert base[0].item() == 0.0 and (base[4002:] == 0).all()
