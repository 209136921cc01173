"""muon_ns_orthogonalize_noalloc: the workspace-free variant of
muon_ns_orthogonalize (its workspace is the library's own per-GPU device
array).  Called through the C ABI, it must give bitwise the results of the
workspace entry point on the same inputs, on consecutive calls whose second
input is smaller than the first, and refuse inputs whose workspace would not
fit the array, before any work."""
import numpy as np
import pytest

import oracle as orc
import workloads as wl
from helpers import BF16_TOL, F32_TOL, grad64, t64, to_torch_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spectral_optimizer_ssm_amd as mu
    mu.lib()
    return mu


def _stack(g, dt):
    return (to_torch_bits(g.G) if dt == "bf16" else torch.from_numpy(g.G)).cuda()


def test_noalloc_matches_workspace_entry_point(mu):
    cases = [(768, 1536, 2, "bf16", 61), (200, 300, 3, "bf16", 62), (96, 200, 4, "f32", 63), (64, 128, 5, "bf16", 64)]
    for m, n, b, dt, seed in cases:  # each call after the first is smaller than the one before it
        print(f"[case] noalloc {m}x{n} x{b} {dt}", flush=True)
        g = wl.random_group(seed, b, m, n, dt)
        G = _stack(g, dt)
        ref = torch.full_like(G, float("nan"))
        mu.muon_ns_orthogonalize(G, ref, steps=5)
        O = torch.full_like(G, float("nan"))
        mu.muon_ns_orthogonalize_noalloc(G, O, steps=5)
        torch.cuda.synchronize()
        assert torch.equal(O, ref)
        tol = BF16_TOL if dt == "bf16" else F32_TOL
        for i in range(b):
            want, _ = orc.newton_schulz(grad64(g, i), 5)
            assert orc.rel_frobenius(t64(O[i]), want) <= tol


def test_noalloc_rejects_what_does_not_fit(mu):
    g = wl.random_group(65, 3, 768, 1536, "bf16")
    G = _stack(g, "bf16")
    O = torch.zeros_like(G)
    assert mu.muon_ns_workspace_size(768, 1536, 3, mu.MUON_BF16) > mu.lib().muon_ns_noalloc_max_bytes()
    with pytest.raises(mu.MuonError) as e:
        mu.muon_ns_orthogonalize_noalloc(G, O, steps=5)
    assert e.value.status == mu.binding.MUON_EWORKSPACE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(O)) == 0
    # a batch that fits right after the refused one
    O2 = torch.empty_like(G[:2])
    mu.muon_ns_orthogonalize_noalloc(G[:2], O2, steps=5)
    ref = torch.empty_like(O2)
    mu.muon_ns_orthogonalize(G[:2], ref, steps=5)
    torch.cuda.synchronize()
    assert torch.equal(O2, ref)
