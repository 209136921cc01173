"""Seeded input generators: bf16 rounding, determinism and recipe checks."""
import hashlib

import numpy as np
import pytest

import oracle as orc
import workloads as wl


def _bf16_nearest_bruteforce(x):
    """Nearest bf16 (ties to even) by comparing the two neighbours exactly."""
    out = []
    for v in np.asarray(x, dtype=np.float64).ravel():
        f = np.float32(v)
        hi16 = int(f.view(np.uint32)) >> 16
        cands = [hi16 - 1, hi16, hi16 + 1, hi16 + 2]
        best = None
        for c in cands:
            c &= 0xFFFF
            cv = float(np.array([c << 16], np.uint32).view(np.float32)[0])
            if not np.isfinite(cv):
                continue
            d = abs(cv - v)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        out.append(best[1])
    return np.array(out, np.uint16)


def test_bf16_rounding_special_values():
    f = np.array([1.0, -1.0, 0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)
    b = wl.f32_to_bf16_bits(f)
    assert list(b[:6]) == [0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0xFF80]
    assert (b[6] & 0x7F80) == 0x7F80 and (b[6] & 0x7F) != 0
    ties = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x3F804000], np.uint32).view(np.float32)
    assert list(wl.f32_to_bf16_bits(ties)) == [0x3F80, 0x3F82, 0x3F81, 0x3F80]
    # overflow rounds to infinity
    assert wl.f32_to_bf16_bits(np.array([3.4e38], np.float32))[0] == 0x7F80


def test_bf16_from_f64_single_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4000) * 10.0 ** rng.uniform(-3, 3, 4000)
    # values that double-round wrongly through binary32: just above a bf16 midpoint
    mids = np.array([1.0 + 2 ** -8 + 2 ** -40, -(1.0 + 3 * 2 ** -8 - 2 ** -40), 1.0 + 2 ** -8 - 2 ** -45])
    x = np.concatenate([x, mids])
    assert np.array_equal(wl.f64_to_bf16_bits(x), _bf16_nearest_bruteforce(x))
    back = orc.widen_bf16(wl.f64_to_bf16_bits(x))
    assert np.max(np.abs(back - x) / np.abs(x)) <= 2.0 ** -8


def test_generators_deterministic_and_regenerable():
    a = wl.config2(count=3, shape=(48, 96))
    b = wl.config2(count=3, shape=(48, 96))
    for k in ("G", "W", "M"):
        ha = hashlib.sha256(getattr(a.groups[0], k).tobytes()).hexdigest()
        hb = hashlib.sha256(getattr(b.groups[0], k).tobytes()).hexdigest()
        assert ha == hb
    one = wl.config2(count=1, shape=(48, 96), first=2)
    assert np.array_equal(one.groups[0].G[0], a.groups[0].G[2])
    assert np.array_equal(one.groups[0].W[0], a.groups[0].W[2])


def test_svd_recipe_singular_values():
    rng = np.random.default_rng(123)
    G = wl.svd_built(rng, 40, 90, 3.0)
    s = np.linalg.svd(G, compute_uv=False)
    assert s.max() <= 1.0 and s.min() >= 1e-3 * (1 - 1e-9)


def test_spike_recipe():
    rng = np.random.default_rng(5)
    G = wl.spiked_gaussian(rng, 335, 77, 8)
    s = np.linalg.svd(G, compute_uv=False)
    c = 10 * (np.sqrt(335) + np.sqrt(77))
    assert np.all(np.abs(s[:8] - c) < 0.15 * c)
    assert s[8] < 0.2 * c


def test_full_config_shapes():
    w = wl.config1()
    g = w.groups[0]
    assert (g.m, g.n, g.count, g.grad_dtype) == (128, 64, 1, "f32")
    assert not g.M.any()
    assert wl.IN_PROJ == (2 * 1536 + 2 * 128 + 24, 768)
    assert wl.INJ_BATCH == 393216


def test_injections_structure():
    torch = pytest.importorskip("torch")
    X, V, K = wl.injections(batch=20, chunk=8, return_factors=True)
    assert X.shape == (20, 64, 128) and X.dtype == torch.bfloat16
    Xd = V.double() @ K.double().transpose(1, 2)
    assert torch.equal(Xd.float().to(torch.bfloat16), X)
    sv = torch.linalg.svdvals(X[0].double())
    assert sv[8] < 1e-2 * sv[0]  # rank 8 up to the bf16 rounding of X
