"""The C-ABI library: it loads, exports every function include/muon.h declares,
and rejects bad arguments before enqueueing anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def mu():
    import spectral_optimizer_ssm_amd as mu
    if not os.path.exists(mu.binding.LIB_PATH):
        pytest.fail("libmuon.so is not built: run python -m spectral_optimizer_ssm_amd.build")
    mu.lib()
    return mu


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(muon_\w+)\s*\(", text, flags=re.M)))


def test_header_compiles_as_c_and_cpp(tmp_path):
    for lang, comp in (("c", "gcc"), ("c++", "g++")):
        src = tmp_path / f"t.{ 'c' if lang == 'c' else 'cpp'}"
        src.write_text('#include "muon.h"\nint main(void){return muon_version()==MUON_VERSION?0:1;}\n')
        r = subprocess.run([comp, "-fsyntax-only", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                            str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_exports_match_header(mu):
    names = declared_functions()
    assert set(names) == set(mu.binding.EXPORTS)
    L = mu.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mu.binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (muon_\w+)", out))
    assert set(names) <= exported


def test_version_and_status(mu):
    assert mu.muon_version() == 9
    assert mu.status_string(0) == "ok"
    assert "invalid" in mu.status_string(-1)
    assert "unknown" in mu.status_string(7)


def _cfg(mu, steps=5, coeffs=(1.5, -0.5), eps=1e-7, prec=None):
    return mu.make_cfg(steps, coeffs, eps, mu.MUON_BF16 if prec is None else prec)


def _group(mu, m=128, n=64, count=1, addr=0x100000, dtype=None, o=False):
    W = (ctypes.c_void_p * count)(*[addr + 0x10000 * i for i in range(count)])
    M = (ctypes.c_void_p * count)(*[addr + 0x1000000 + 0x10000 * i for i in range(count)])
    G = (ctypes.c_void_p * count)(*[addr + 0x2000000 + 0x10000 * i for i in range(count)])
    P = ctypes.POINTER(ctypes.c_void_p)
    g = mu.binding.GroupC(m, n, count, mu.MUON_BF16 if dtype is None else dtype, ctypes.cast(W, P),
                          ctypes.cast(M, P), ctypes.cast(G, P), None, 0.02, 0.95, 1.0, 1)
    return g, (W, M, G)


def test_workspace_queries(mu):
    L = mu.lib()
    cfg, keep = _cfg(mu)
    g, k2 = _group(mu, 768, 1536, 24)
    arr = (mu.binding.GroupC * 1)(g)
    ws = L.muon_step_workspace_size(arr, 1, ctypes.byref(cfg))
    # two bf16 iterates + Gram (768 x 768) + partials, padded
    assert ws >= 24 * (2 * 768 * 1536 * 2 + 768 * 768 * 2)
    assert L.muon_step_workspace_size(arr, 0, ctypes.byref(cfg)) == 0
    assert L.muon_ns_workspace_size(768, 1536, 24, mu.MUON_BF16, ctypes.byref(cfg)) >= 24 * 2 * 768 * 1536 * 2
    assert L.muon_ns_workspace_size(0, 1536, 24, mu.MUON_BF16, ctypes.byref(cfg)) == 0
    assert L.muon_ns_workspace_size(8, 8, 1, 7, ctypes.byref(cfg)) == 0


@pytest.mark.parametrize("case,expect", [
    ("steps_negative", -1), ("steps_too_many", -1), ("ncoef_4", -1), ("quintic_c", -2),
    ("bad_precision", -1), ("null_groups", -1), ("misaligned", -1), ("null_matrix", -1),
    ("no_workspace", -3), ("small_workspace", -3), ("bad_dtype", -1), ("negative_eps", -1),
    ("bad_schedule", -1), ("bad_streams", -1), ("bad_separate_apply", -1),
])
def test_step_validation(mu, case, expect):
    L = mu.lib()
    cfg, keep = _cfg(mu, steps={"steps_negative": -1, "steps_too_many": 65}.get(case, 5),
                     coeffs=(1.5, -0.5, 0.25) if case == "quintic_c" else (1.5, -0.5),
                     eps=-1.0 if case == "negative_eps" else 1e-7,
                     prec={"bad_precision": 9, "quintic_c": mu.MUON_F32}.get(case))
    if case == "ncoef_4":
        cfg.ncoef = 4
    if case == "bad_schedule":
        cfg.schedule = 3
    if case == "bad_streams":
        cfg.streams = 2
    if case == "bad_separate_apply":
        cfg.separate_apply = 3
    g, k2 = _group(mu, dtype=5 if case == "bad_dtype" else None)
    if case == "misaligned":
        k2[0][0] = 0x100002  # W is float32: 4-byte alignment required
    if case == "null_matrix":
        k2[2][0] = None
    arr = (mu.binding.GroupC * 1)(g)
    ws_size = {"no_workspace": 0, "small_workspace": 64}.get(case, 1 << 40)
    ws = None if case == "no_workspace" else ctypes.c_void_p(0x7000000)
    grp = None if case == "null_groups" else arr
    rc = L.muon_step(grp, 1, ctypes.byref(cfg), ws, ws_size, None, None)
    assert rc == expect


@pytest.mark.parametrize("m,n,ok", [
    (16384, 65280, True),     # padded iterate 16384 x 65280 bf16: just under 2 GiB
    (65280, 16384, True),     # the same, tall
    (16384, 65536, False),    # exactly 2 GiB: beyond the 32-bit buffer offsets
    (32768, 32768, False),
    (46341, 46341, False),    # m * n > 2^31
])
def test_size_limits(mu, m, n, ok):
    """Shapes at the documented size bounds: accepted by the planner (phases
    listed, workspace sized) or rejected with MUON_EUNSUPPORTED, no GPU work."""
    L = mu.lib()
    cfg, keep = _cfg(mu)
    g, k2 = _group(mu, m, n, 1)
    arr = (mu.binding.GroupC * 1)(g)
    n_ph = L.muon_step_phases(arr, 1, ctypes.byref(cfg), None, 0)
    ws = L.muon_step_workspace_size(arr, 1, ctypes.byref(cfg))
    if ok:
        assert n_ph > 0 and ws >= 2 * min(m, n) * max(m, n) * 2
    else:
        assert n_ph == -2 and ws == 0
        assert L.muon_step(arr, 1, ctypes.byref(cfg), ctypes.c_void_p(0x7000000), 1 << 40, None, None) == -2


def test_small_and_ns_validation(mu):
    L = mu.lib()
    cfg, keep = _cfg(mu, steps=1)
    x, y = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000)
    assert L.muon_ns_batched_small(x, y, mu.MUON_BF16, 48, 128, 10, ctypes.byref(cfg), None) == -2
    assert L.muon_ns_batched_small(x, y, mu.MUON_BF16, 128, 64, 10, ctypes.byref(cfg), None) == -2  # tall bf16
    assert L.muon_ns_batched_small(x, x, mu.MUON_BF16, 64, 128, 10, ctypes.byref(cfg), None) == -1  # overlap
    assert L.muon_ns_batched_small(x, y, mu.MUON_BF16, 64, 128, 0, ctypes.byref(cfg), None) == 0    # empty
    cf32, k2 = _cfg(mu, steps=1, prec=mu.MUON_F32)
    assert L.muon_ns_batched_small(x, y, mu.MUON_BF16, 64, 128, 1, ctypes.byref(cf32), None) == -2  # precision
    ws = ctypes.c_void_p(0x7000000)
    x64 = ctypes.c_void_p(0x100000 + 64)
    ns = L.muon_ns_orthogonalize
    # partial overlap of G and O (in place, O == G, is allowed)
    assert ns(x, x64, mu.MUON_BF16, 64, 128, 128, 2, 64 * 128, ctypes.byref(cfg), ws, 1 << 30, None) == -1
    assert ns(x, y, mu.MUON_BF16, 64, 128, 127, 2, 64 * 128, ctypes.byref(cfg), ws, 1 << 30, None) == -1  # ld < n
    assert ns(x, y, mu.MUON_BF16, 64, 128, 160, 2, 63 * 160 + 127, ctypes.byref(cfg), ws, 1 << 30,
              None) == -1                                                                           # stride < span
    assert ns(x, y, mu.MUON_BF16, 64, 128, 128, 2, 64 * 128, ctypes.byref(cfg), None, 0, None) == -3
    assert ns(x, y, mu.MUON_BF16, 64, 128, 128, 0, 0, ctypes.byref(cfg), None, 0, None) == 0
    assert ns(x, y, mu.MUON_BF16, 64, 128, 128, 2, 64 * 128, ctypes.byref(cf32), ws, 1 << 30, None) == -2
    assert ns(None, y, mu.MUON_BF16, 64, 128, 128, 2, 64 * 128, ctypes.byref(cfg), ws, 1 << 30, None) == -1
    # the workspace-free variant: the same validation, and workspaces beyond its array refused
    na = L.muon_ns_orthogonalize_noalloc
    assert L.muon_ns_noalloc_max_bytes() == 32 << 20
    assert na(x, x64, mu.MUON_BF16, 64, 128, 128, 2, 64 * 128, ctypes.byref(cfg), None) == -1
    assert na(x, y, mu.MUON_BF16, 64, 128, 127, 2, 64 * 128, ctypes.byref(cfg), None) == -1
    assert na(x, y, mu.MUON_BF16, 64, 128, 128, 0, 0, ctypes.byref(cfg), None) == 0
    big = ctypes.c_void_p(0x10000000)
    assert na(x, big, mu.MUON_BF16, 768, 1536, 1536, 24, 768 * 1536, ctypes.byref(cfg), None) == -3
    # the flag query validates its pointers before any copy
    out = ctypes.c_int(-1)
    assert L.muon_query_flags(None, ctypes.byref(out)) == -1
    assert L.muon_query_flags(ctypes.c_void_p(0x7000008), ctypes.byref(out)) == -1
    assert L.muon_query_flags(ws, None) == -1 and out.value == -1


def _phases(mu, shapes, steps, schedule, prec=None, separate_apply=0, coeffs=(1.5, -0.5)):
    L = mu.lib()
    cfg, keep = mu.make_cfg(steps, coeffs, 1e-7, mu.MUON_BF16 if prec is None else prec, False, schedule,
                            separate_apply=separate_apply)
    gs = [_group(mu, m, n, c) for m, n, c in shapes]
    arr = (mu.binding.GroupC * len(gs))(*[g for g, _ in gs])
    n = L.muon_step_phases(arr, len(gs), ctypes.byref(cfg), None, 0)
    out = (ctypes.c_int * max(n, 1))()
    assert L.muon_step_phases(arr, len(gs), ctypes.byref(cfg), out, n) == n
    names = [mu.binding.PHASES[out[i]] for i in range(n)]
    # every call takes its non-finite flag once all momentum passes are done
    assert names.count("flags") == 1
    k = names.index("flags")
    assert names[k - 1] == "momentum" and "momentum" not in names[k:]
    return names[:k] + names[k + 1:]


MAMBA = [(768, 1536, 24), (3352, 768, 24)]


def test_phases_iterate_and_accumulate(mu):
    # the final combine applies the update of the large bf16 groups itself
    it = _phases(mu, MAMBA, 5, mu.MUON_NS_ITERATE)
    assert it == ["momentum"] * 2 + ["gram", "combine"] * 4 + ["gram", "combine_apply"]
    ac = _phases(mu, MAMBA, 5, mu.MUON_NS_ACCUMULATE)
    assert ac == ["momentum"] * 2 + ["gram"] + ["symprod"] * 9 + ["combine_apply"]
    assert _phases(mu, MAMBA, 5, mu.MUON_NS_ACCUMULATE, separate_apply=1) == \
        ["momentum"] * 2 + ["gram"] + ["symprod"] * 9 + ["combine"] + ["apply"] * 2
    # the Mamba-2 projections are wide enough for the accumulated schedule to
    # need fewer matrix-core operations; a square group is not
    assert _phases(mu, MAMBA, 5, mu.MUON_NS_AUTO) == ac
    assert _phases(mu, [(768, 768, 4)], 5, mu.MUON_NS_AUTO) == \
        ["momentum"] + ["gram", "combine"] * 4 + ["gram", "combine_apply"]
    # more than 64 matrices in one final launch: the first group fuses, the next keeps its apply pass
    assert _phases(mu, [(768, 1536, 40), (3352, 768, 40)], 5, mu.MUON_NS_ACCUMULATE)[-2:] == \
        ["combine_apply", "apply"]
    # one step, float32 and small matrices always iterate
    assert _phases(mu, MAMBA, 1, mu.MUON_NS_ACCUMULATE) == ["momentum"] * 2 + ["gram", "combine_apply"]
    assert _phases(mu, [(300, 700, 2)], 2, mu.MUON_NS_ACCUMULATE, mu.MUON_F32) == \
        ["momentum", "f32_gram", "f32_combine", "f32_gram", "f32_combine", "apply"]
    assert _phases(mu, [(64, 128, 9)], 3, mu.MUON_NS_ACCUMULATE) == ["momentum", "ns_small", "apply"]
    # bf16 short sides up to 128 and long sides up to 512 stay on chip (both
    # padded to multiples of 32); beyond either, the matrix-core path
    for shape in ((128, 512), (96, 300), (300, 96), (1, 70), (33, 500), (512, 128)):
        assert _phases(mu, [shape + (3,)], 5, mu.MUON_NS_ITERATE) == ["momentum", "ns_small", "apply"], shape
    for shape in ((129, 512), (128, 513), (600, 100)):
        assert "ns_small" not in _phases(mu, [shape + (3,)], 5, mu.MUON_NS_ITERATE), shape
    # quintic steps take the matrix-core path whatever the shape
    assert "ns_small" not in _phases(mu, [(64, 128, 3)], 3, mu.MUON_NS_ITERATE, coeffs=(2.0, -1.5, 0.5))
    assert _phases(mu, MAMBA, 0, mu.MUON_NS_AUTO) == ["momentum"] * 2 + ["apply"] * 2
    # 2 steps: one E = B_0^2, then A_1 / B_1, then Q_2 = B_1 B_0
    assert _phases(mu, MAMBA, 2, mu.MUON_NS_ACCUMULATE).count("symprod") == 3


def test_accumulate_workspace_is_larger(mu):
    L = mu.lib()
    g, k2 = _group(mu, 768, 1536, 24)
    arr = (mu.binding.GroupC * 1)(g)
    sizes = {}
    for sch in (mu.MUON_NS_ITERATE, mu.MUON_NS_ACCUMULATE):
        cfg, keep = mu.make_cfg(5, (1.5, -0.5), 1e-7, mu.MUON_BF16, False, sch)
        sizes[sch] = L.muon_step_workspace_size(arr, 1, ctypes.byref(cfg))
    # seven 768 x 768 bf16 buffers per matrix instead of one
    assert sizes[mu.MUON_NS_ACCUMULATE] - sizes[mu.MUON_NS_ITERATE] >= 24 * 6 * 768 * 768 * 2


@pytest.mark.parametrize("case,expect", [
    ("ok_empty", 0), ("r9", -2), ("f32", -2), ("m0", -1), ("m300", -2), ("dense_n_odd", -2),
    ("overlap_c", -1), ("overlap_o", -1), ("misaligned_o", -1), ("null_v", -1), ("quintic_ok_empty", 0),
    ("too_big_dense", -2),
])
def test_factored_validation(mu, case, expect):
    L = mu.lib()
    cfg, keep = mu.make_cfg(1, (1.5, -0.5, 0.25) if case == "quintic_ok_empty" else (1.5, -0.5), 1e-7,
                            mu.MUON_F32 if case == "f32" else mu.MUON_BF16)
    m, n, r, batch = 64, 128, 8, 10
    if case == "r9":
        r = 9
    if case == "m0":
        m = 0
    if case == "m300":
        m = 300
    if case == "dense_n_odd":
        n = 127
    if case == "too_big_dense":
        m, n = 256, 256
    if case in ("ok_empty", "quintic_ok_empty"):
        batch = 0
    V, K = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    C = ctypes.cast(ctypes.c_void_p(0x400000 if case != "overlap_c" else 0x100010), ctypes.POINTER(ctypes.c_float))
    O = {"overlap_o": 0x200000, "misaligned_o": 0x800008}.get(case, 0x800000)
    dense = case in ("dense_n_odd", "overlap_o", "misaligned_o", "too_big_dense")
    rc = L.muon_ns_factored(None if case == "null_v" else V, K, mu.MUON_F32 if case == "f32" else mu.MUON_BF16,
                            m, n, r, batch, ctypes.byref(cfg), C, ctypes.c_void_p(O) if dense else None, None)
    assert rc == expect


def test_cap_validation_and_phases(mu):
    L = mu.lib()
    cfg, keep = _cfg(mu)
    P = ctypes.POINTER(ctypes.c_void_p)
    g, k2 = _group(mu, 128, 256, 2)
    cu = (ctypes.c_void_p * 2)(0x3000000, 0x3001000)
    cv = (ctypes.c_void_p * 2)(0x3002000, 0x3003000)
    g.cap_u = ctypes.cast(cu, P)
    arr = (mu.binding.GroupC * 1)(g)
    ws = ctypes.c_void_p(0x7000000)
    assert L.muon_step(arr, 1, ctypes.byref(cfg), ws, 1 << 40, None, None) == -1  # cap_v, cap_sigma missing
    g.cap_v = ctypes.cast(cv, P)
    g.cap_sigma = ctypes.c_void_p(0x3004002)                                       # misaligned
    arr = (mu.binding.GroupC * 1)(g)
    assert L.muon_step(arr, 1, ctypes.byref(cfg), ws, 1 << 40, None, None) == -1
    g.cap_sigma = ctypes.c_void_p(0x3004000)
    g.W = None                                                                      # the cap needs W
    arr = (mu.binding.GroupC * 1)(g)
    assert L.muon_step(arr, 1, ctypes.byref(cfg), ws, 1 << 40, None, None) == -1
    n = L.muon_step_phases(arr, 1, ctypes.byref(cfg), None, 0)
    out = (ctypes.c_int * n)()
    L.muon_step_phases(arr, 1, ctypes.byref(cfg), out, n)
    names = [mu.binding.PHASES[out[i]] for i in range(n)]
    assert names[-3:] == ["cap", "apply", "power"] and names[:2] == ["momentum", "flags"]
    # the cap's partial buffers enlarge the workspace
    base, _ = _group(mu, 128, 256, 2)
    a0 = (mu.binding.GroupC * 1)(base)
    assert L.muon_step_workspace_size(arr, 1, ctypes.byref(cfg)) > L.muon_step_workspace_size(a0, 1, ctypes.byref(cfg))


@pytest.mark.parametrize("case,expect", [
    ("ok_empty", 0), ("beta1_one", -1), ("step0", -1), ("null_p", -1), ("misaligned", -1), ("bad_dtype", -1),
    ("neg_numel", -1), ("zero_numel_null_ok", 0), ("neg_eps", -1),
])
def test_adamw_validation(mu, case, expect):
    L = mu.lib()
    n = 0 if case == "ok_empty" else 2
    ptr = lambda base: (ctypes.c_void_p * 2)(base, base + 0x10000)  # noqa: E731
    P, G, M, V = ptr(0x1000000), ptr(0x2000000), ptr(0x3000000), ptr(0x4000000)
    N = (ctypes.c_longlong * 2)(100, 200)
    if case == "null_p":
        P[1] = None
    if case == "misaligned":
        M[0] = 0x3000002
    if case == "neg_numel":
        N[1] = -1
    if case == "zero_numel_null_ok":
        N[1] = 0
        P[1] = None
        # then the remaining tensor is launched: keep it off the device by making it empty too
        N[0] = 0
    rc = L.muon_adamw(n, P, G, M, V, N, 7 if case == "bad_dtype" else mu.MUON_BF16, 1e-3,
                      1.0 if case == "beta1_one" else 0.9, 0.95, -1.0 if case == "neg_eps" else 1e-8, 0.1,
                      0 if case == "step0" else 1, None)
    assert rc == expect


@pytest.mark.parametrize("case,expect", [
    ("iters0", -1), ("bad_dtype", -1), ("neg_batch", -1), ("zero_m", -1), ("s_too_big", -2), ("iters_too_big", -2),
    ("null_a", -1), ("misaligned_out", -1), ("overlap", -1), ("no_workspace", -3), ("small_workspace", -3),
    ("empty_batch", 0), ("nothing_asked", 0),
])
def test_spectral_diag_validation(mu, case, expect):
    """Every rejection happens on the host before any launch (fake device
    addresses are never touched)."""
    L = mu.lib()
    m, n, b, it, dt = 96, 200, 3, 16, mu.MUON_BF16
    if case == "iters0":
        it = 0
    if case == "bad_dtype":
        dt = 9
    if case == "neg_batch":
        b = -1
    if case == "zero_m":
        m = 0
    if case == "s_too_big":
        m, n = 5000, 6000
    if case == "iters_too_big":
        it = 513
    if case == "empty_batch":
        b = 0
    A = None if case == "null_a" else 0x1000000
    out = 0x2000002 if case == "misaligned_out" else (0x1000000 + 64 if case == "overlap" else 0x2000000)
    ws_size = L.muon_spectral_diag_workspace_size(m, n, b, dt, it)
    if expect == 0 or case in ("no_workspace", "small_workspace", "null_a", "misaligned_out", "overlap"):
        assert ws_size > 0
    ws = None if case == "no_workspace" else 0x40000000
    wsb = ws_size - 256 if case == "small_workspace" else ws_size
    o = None if case == "nothing_asked" else out
    rc = L.muon_spectral_diag(A, dt, m, n, b, it, o, None, None, ws, wsb, None)
    assert rc == expect, (case, rc)


def test_spectral_diag_workspace_sizes(mu):
    L = mu.lib()
    # bf16: one operand, H and the Lanczos basis per matrix
    s_pad, kdim, k = 768, 1536, 32
    per = s_pad * kdim * 2 + s_pad * s_pad * 4 + k * s_pad * 4
    assert L.muon_spectral_diag_workspace_size(768, 1536, 24, mu.MUON_BF16, 32) == 24 * per
    # float32 inputs: one operand array holding the three bf16 pieces side by
    # side; tall is oriented
    per32 = s_pad * 3 * 3392 * 2 + s_pad * s_pad * 4 + k * s_pad * 4
    assert L.muon_spectral_diag_workspace_size(3352, 768, 4, mu.MUON_F32, 32) == 4 * per32
    # chunked: the size stops growing once a chunk is full
    big = L.muon_spectral_diag_workspace_size(64, 128, 393216, mu.MUON_BF16, 64)
    assert big <= 2 ** 31 and big == L.muon_spectral_diag_workspace_size(64, 128, 2 * 393216, mu.MUON_BF16, 64)


def test_spectral_diag_timed_needs_enough_events(mu):
    L = mu.lib()
    ws = L.muon_spectral_diag_workspace_size(96, 200, 3, mu.MUON_BF16, 16)
    ev = (ctypes.c_void_p * 3)()
    rc = L.muon_spectral_diag_timed(0x1000000, mu.MUON_BF16, 96, 200, 3, 16, 0x2000000, None, None, 0x40000000, ws,
                                    None, ev, 3)
    assert rc == -1  # one chunk needs 1 + 3 events


@pytest.mark.parametrize("case,expect", [
    ("ok_empty_seq", 0), ("ok_empty_T", 0), ("r4", -2), ("m65", -2), ("n129", -2), ("m0", -1), ("f32", -2),
    ("s_without_decay", -1), ("misaligned_v", -1), ("null_m", -1), ("overlap_ms", -1), ("overlap_ws_m", -1),
    ("no_workspace", -3), ("small_workspace", -3), ("beta_nan", -1), ("few_events", -1), ("null_k", -1),
])
def test_ssm_momentum_validation(mu, case, expect):
    """muon_ssm_momentum rejects bad arguments before any GPU work."""
    L = mu.lib()
    m, n, r, nseq, T = 64, 128, 8, 2, 300
    if case == "r4":
        r = 4
    if case == "m65":
        m = 65
    if case == "n129":
        n = 129
    if case == "m0":
        m = 0
    if case == "ok_empty_seq":
        nseq = 0
    if case == "ok_empty_T":
        T = 0
    cfg, keep = _cfg(mu, steps=1, prec=mu.MUON_F32 if case == "f32" else None)
    dt = mu.MUON_F32 if case == "f32" else mu.MUON_BF16
    fp = ctypes.POINTER(ctypes.c_float)
    V = ctypes.c_void_p(0x1000000 + (8 if case == "misaligned_v" else 0))
    K = None if case == "null_k" else ctypes.c_void_p(0x3000000)
    M = None if case == "null_m" else ctypes.cast(ctypes.c_void_p(0x5000000), fp)
    S = ctypes.cast(ctypes.c_void_p(0x5000000 + (1024 if case == "overlap_ms" else 0x100000)), fp)
    dec = None if case == "s_without_decay" else ctypes.cast(ctypes.c_void_p(0x5800000), fp)
    need = L.muon_ssm_momentum_workspace_size(max(m, 1), n, r, nseq, T) if case not in ("m0",) else 0
    ws = None if case == "no_workspace" else ctypes.c_void_p(0x5000000 if case == "overlap_ws_m" else 0x10000000)
    wsz = 64 if case == "small_workspace" else (1 << 30)
    beta = float("nan") if case == "beta_nan" else 0.9
    args = (V, K, dt, m, n, r, nseq, T, beta, dec, M, S, ctypes.byref(cfg), ws, wsz, None)
    if case == "few_events":
        ev = (ctypes.c_void_p * 2)()
        rc = L.muon_ssm_momentum_timed(*args, ev, 2)
    else:
        rc = L.muon_ssm_momentum(*args)
    assert rc == expect, (case, rc, need)


def test_ssm_momentum_workspace_size(mu):
    L = mu.lib()
    # two 64 x 128 float32 partials and 4 coefficients per 256-token chunk
    nseq, T = 3, 600
    chunks = 3
    expect = 0
    for b in (nseq * chunks * 2 * 64 * 128 * 4, nseq * chunks * 16):
        expect += -(-b // 256) * 256
    assert L.muon_ssm_momentum_workspace_size(64, 128, 8, nseq, T) == expect
    assert L.muon_ssm_momentum_workspace_size(64, 128, 4, nseq, T) == 0
    assert L.muon_ssm_momentum_workspace_size(64, 129, 8, nseq, T) == 0
    assert L.muon_ssm_momentum_workspace_size(64, 128, 8, 0, 0) > 0
