"""Host-side marshalling of muon_step's groups (no GPU needed: pointer tables
are built from CPU tensors' addresses and never dereferenced here)."""
import ctypes

import pytest

torch = pytest.importorskip("torch")

from spectral_optimizer_ssm_amd import binding as B  # noqa: E402


def table(ptr_array, count):
    return [ptr_array[i] for i in range(count)]


def group(count=3, m=5, n=7, cap=False, **kw):
    W = torch.zeros(count, m, n)
    M = torch.zeros(count, m, n)
    G = torch.zeros(count, m, n, dtype=torch.bfloat16)
    extra = dict(cap_u=torch.zeros(count, m), cap_v=torch.zeros(count, n), cap_sigma=torch.zeros(count), cap=1.0) \
        if cap else {}
    extra.update(kw)
    return B.MuonGroup(W=W, M=M, G=G, lr=0.01, beta=0.9, **extra)


def test_tables_of_stacked_tensors_match_each_matrix():
    g = group(cap=True)
    arr, keep = B._marshal_groups([g])
    c = arr[0]
    assert (c.m, c.n, c.count, c.grad_dtype) == (5, 7, 3, B.MUON_BF16)
    for name, t in (("W", g.W), ("M", g.M), ("G", g.G), ("cap_u", g.cap_u), ("cap_v", g.cap_v)):
        assert table(getattr(c, name), 3) == [t[i].data_ptr() for i in range(3)], name
    assert c.cap_sigma == g.cap_sigma.data_ptr()
    assert not c.O


def test_lists_and_stacks_give_the_same_tables():
    g = group()
    lst = B.MuonGroup(W=list(g.W), M=list(g.M), G=[g.G[i] for i in range(3)], lr=0.01, beta=0.9)
    a, _ = B._marshal_groups([g])
    b, _ = B._marshal_groups([lst])
    for name in ("W", "M", "G"):
        assert table(getattr(a[0], name), 3) == table(getattr(b[0], name), 3)


def test_optional_output_table():
    O = torch.zeros(3, 5, 7, dtype=torch.bfloat16)
    arr, _ = B._marshal_groups([group(O=O)])
    assert table(arr[0].O, 3) == [O[i].data_ptr() for i in range(3)]


@pytest.mark.parametrize("bad", ["noncontiguous", "shape", "count", "cap_len", "cap_count", "sigma"])
def test_invalid_groups_are_rejected(bad):
    g = group(cap=True)
    if bad == "noncontiguous":
        g.W = torch.zeros(3, 7, 5).transpose(1, 2)
    elif bad == "shape":
        g.M = torch.zeros(3, 5, 8)
    elif bad == "count":
        g.G = torch.zeros(2, 5, 7, dtype=torch.bfloat16)
    elif bad == "cap_len":
        g.cap_v = torch.zeros(3, 6)
    elif bad == "cap_count":
        g.cap_u = torch.zeros(2, 5)
    else:
        g.cap_sigma = torch.zeros(4)
    with pytest.raises(ValueError):
        B._marshal_groups([g])


def test_float32_gradients_are_marked():
    g = group()
    g.G = torch.zeros(3, 5, 7)
    arr, _ = B._marshal_groups([g])
    assert arr[0].grad_dtype == B.MUON_F32
    assert isinstance(arr[0].W, ctypes.POINTER(ctypes.c_void_p))


# ---------------------------------------------------------------------------
# dtype and device checks: a wrong element type or a host tensor must never
# reach the kernels as a device pointer of another type
# ---------------------------------------------------------------------------
CPU = torch.device("cpu")
FAKE_GPU = torch.device("cuda", 0)


@pytest.mark.parametrize("bad", ["W_bf16", "M_f64", "G_f16", "O_f32", "cap_u_bf16", "cap_sigma_f64",
                                 "G_mixed_list", "O_bf16_for_f32"])
def test_wrong_dtypes_are_rejected(bad):
    g = group(cap=True, O=torch.zeros(3, 5, 7, dtype=torch.bfloat16))
    prec = B.MUON_BF16
    if bad == "W_bf16":
        g.W = torch.zeros(3, 5, 7, dtype=torch.bfloat16)
    elif bad == "M_f64":
        g.M = torch.zeros(3, 5, 7, dtype=torch.float64)
    elif bad == "G_f16":
        g.G = torch.zeros(3, 5, 7, dtype=torch.float16)
    elif bad == "O_f32":
        g.O = torch.zeros(3, 5, 7)
    elif bad == "cap_u_bf16":
        g.cap_u = torch.zeros(3, 5, dtype=torch.bfloat16)
    elif bad == "cap_sigma_f64":
        g.cap_sigma = torch.zeros(3, dtype=torch.float64)
    elif bad == "G_mixed_list":
        g.G = [torch.zeros(5, 7, dtype=torch.bfloat16), torch.zeros(5, 7), torch.zeros(5, 7, dtype=torch.bfloat16)]
    else:
        prec = B.MUON_F32  # O must then be float32
    with pytest.raises(TypeError):
        B._marshal_groups([g], prec)


@pytest.mark.parametrize("which", ["W", "M", "G", "O", "cap_u", "cap_v", "cap_sigma"])
def test_tensors_off_the_device_are_rejected_for_launches(which):
    """Calls that launch work pass the device the kernels run on: every
    tensor of the group lives on it (the meta device stands in for the GPU
    here) except one host tensor, which must be refused by name."""
    meta = torch.device("meta")
    g = group(cap=True, O=torch.zeros(3, 5, 7, dtype=torch.bfloat16))
    for name in ("W", "M", "G", "O", "cap_u", "cap_v", "cap_sigma"):
        if name != which:
            setattr(g, name, getattr(g, name).to(meta))
    with pytest.raises(ValueError, match=which):
        B._marshal_groups([g], B.MUON_BF16, meta)
    setattr(g, which, getattr(g, which).to(meta))
    arr, _ = B._marshal_groups([g], B.MUON_BF16, meta)
    assert arr[0].count == 3


def test_queries_accept_host_tensors_without_a_device():
    arr, _ = B._marshal_groups([group(cap=True)], B.MUON_BF16, None)
    assert arr[0].count == 3


def test_workspace_checks():
    with pytest.raises(TypeError):
        B._workspace(torch.zeros(16), 8, CPU)
    with pytest.raises(ValueError):
        B._workspace(torch.zeros(16, dtype=torch.uint8), 8, FAKE_GPU)
    ws = torch.zeros(16, dtype=torch.uint8)
    assert B._workspace(ws, 8, CPU) is ws


def test_strided_stack_layout():
    base = torch.zeros(4, 6, 10)
    b, m, n, ld, stride = B._strided_stack(base[:, :, :8])[1:]
    assert (b, m, n, ld, stride) == (4, 6, 8, 10, 60)
    with pytest.raises(ValueError):
        B._strided_stack(base.transpose(1, 2))
    assert B._strided_stack(torch.zeros(6, 8))[1:] == (1, 6, 8, 8, 48)
