"""ctypes binding of libmuon (include/muon.h), argument marshalling only.

torch is used for device memory and streams: tensors are passed by pointer,
the workspace is a torch byte tensor, and every call is enqueued on torch's
current stream.  All arithmetic happens in the HIP kernels of libmuon.so; if
that library is not built this module raises on first use (there is no CPU
fallback).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

MUON_F32, MUON_BF16 = 0, 1
MUON_OK, MUON_EINVAL, MUON_EUNSUPPORTED, MUON_EWORKSPACE, MUON_EHIP = 0, -1, -2, -3, -4
MUON_NS_AUTO, MUON_NS_ITERATE, MUON_NS_ACCUMULATE = 0, 1, 2
PHASES = {1: "momentum", 2: "ns_small", 3: "gram", 4: "combine", 5: "symprod", 6: "apply", 7: "f32_gram",
          8: "f32_combine", 9: "cap", 10: "power", 11: "combine_apply", 12: "flags"}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon.so")
_lib = None


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class NsCfg(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int), ("ncoef", ctypes.c_int),
                ("coeffs", ctypes.POINTER(ctypes.c_float)), ("per_step", ctypes.c_int),
                ("eps", ctypes.c_float), ("precision", ctypes.c_int), ("schedule", ctypes.c_int),
                ("streams", ctypes.c_int), ("separate_apply", ctypes.c_int)]


class GroupC(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int), ("n", ctypes.c_int), ("count", ctypes.c_int),
                ("grad_dtype", ctypes.c_int),
                ("W", ctypes.POINTER(ctypes.c_void_p)), ("M", ctypes.POINTER(ctypes.c_void_p)),
                ("G", ctypes.POINTER(ctypes.c_void_p)), ("O", ctypes.POINTER(ctypes.c_void_p)),
                ("lr", ctypes.c_float), ("beta", ctypes.c_float), ("scale", ctypes.c_float),
                ("nesterov", ctypes.c_int),
                ("cap_u", ctypes.POINTER(ctypes.c_void_p)), ("cap_v", ctypes.POINTER(ctypes.c_void_p)),
                ("cap_sigma", ctypes.c_void_p), ("cap", ctypes.c_float)]


EXPORTS = ("muon_step_workspace_size", "muon_step", "muon_step_phases", "muon_step_timed", "muon_ns_workspace_size",
           "muon_ns_orthogonalize", "muon_ns_noalloc_max_bytes", "muon_ns_orthogonalize_noalloc", "muon_query_flags",
           "muon_ns_batched_small", "muon_ns_factored", "muon_ssm_momentum_workspace_size", "muon_ssm_momentum",
           "muon_ssm_momentum_timed", "muon_adamw",
           "muon_spectral_diag_workspace_size", "muon_spectral_diag", "muon_spectral_diag_timed",
           "muon_status_string", "muon_version")


def lib():
    """Load libmuon.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmuon.so is not built ({LIB_PATH}); run "
                           "`python -m spectral_optimizer_ssm_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.muon_step_workspace_size.argtypes = [ctypes.POINTER(GroupC), i, ctypes.POINTER(NsCfg)]
    L.muon_step_workspace_size.restype = sz
    L.muon_step.argtypes = [ctypes.POINTER(GroupC), i, ctypes.POINTER(NsCfg), vp, sz,
                            ctypes.POINTER(f), vp]
    L.muon_step.restype = i
    L.muon_step_phases.argtypes = [ctypes.POINTER(GroupC), i, ctypes.POINTER(NsCfg), ctypes.POINTER(i), i]
    L.muon_step_phases.restype = i
    L.muon_step_timed.argtypes = [ctypes.POINTER(GroupC), i, ctypes.POINTER(NsCfg), vp, sz,
                                  ctypes.POINTER(f), vp, ctypes.POINTER(ctypes.c_void_p), i]
    L.muon_step_timed.restype = i
    L.muon_ns_workspace_size.argtypes = [i, i, i, i, ctypes.POINTER(NsCfg)]
    L.muon_ns_workspace_size.restype = sz
    L.muon_ns_orthogonalize.argtypes = [vp, vp, i, i, i, i, i, ctypes.c_longlong, ctypes.POINTER(NsCfg), vp, sz, vp]
    L.muon_ns_orthogonalize.restype = i
    L.muon_ns_noalloc_max_bytes.argtypes = []
    L.muon_ns_noalloc_max_bytes.restype = sz
    L.muon_ns_orthogonalize_noalloc.argtypes = [vp, vp, i, i, i, i, i, ctypes.c_longlong, ctypes.POINTER(NsCfg), vp]
    L.muon_ns_orthogonalize_noalloc.restype = i
    L.muon_query_flags.argtypes = [vp, ctypes.POINTER(i)]
    L.muon_query_flags.restype = i
    L.muon_ns_batched_small.argtypes = [vp, vp, i, i, i, ctypes.c_longlong, ctypes.POINTER(NsCfg), vp]
    L.muon_ns_batched_small.restype = i
    L.muon_ns_factored.argtypes = [vp, vp, i, i, i, i, ctypes.c_longlong, ctypes.POINTER(NsCfg),
                                   ctypes.POINTER(f), vp, vp]
    L.muon_ns_factored.restype = i
    L.muon_ssm_momentum_workspace_size.argtypes = [i, i, i, ctypes.c_longlong, i]
    L.muon_ssm_momentum_workspace_size.restype = sz
    L.muon_ssm_momentum.argtypes = [vp, vp, i, i, i, i, ctypes.c_longlong, i, f, ctypes.POINTER(f), ctypes.POINTER(f),
                                    ctypes.POINTER(f), ctypes.POINTER(NsCfg), vp, sz, vp]
    L.muon_ssm_momentum.restype = i
    L.muon_ssm_momentum_timed.argtypes = [vp, vp, i, i, i, i, ctypes.c_longlong, i, f, ctypes.POINTER(f),
                                          ctypes.POINTER(f), ctypes.POINTER(f), ctypes.POINTER(NsCfg), vp, sz, vp,
                                          ctypes.POINTER(ctypes.c_void_p), i]
    L.muon_ssm_momentum_timed.restype = i
    L.muon_adamw.argtypes = [i, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                             ctypes.POINTER(ctypes.c_longlong), i, f, f, f, f, f, ctypes.c_longlong, vp]
    L.muon_adamw.restype = i
    L.muon_spectral_diag_workspace_size.argtypes = [i, i, ctypes.c_longlong, i, i]
    L.muon_spectral_diag_workspace_size.restype = sz
    L.muon_spectral_diag.argtypes = [vp, i, i, i, ctypes.c_longlong, i, vp, vp, vp, vp, sz, vp]
    L.muon_spectral_diag.restype = i
    L.muon_spectral_diag_timed.argtypes = [vp, i, i, i, ctypes.c_longlong, i, vp, vp, vp, vp, sz, vp,
                                           ctypes.POINTER(ctypes.c_void_p), i]
    L.muon_spectral_diag_timed.restype = i
    L.muon_status_string.argtypes = [i]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_version.argtypes = []
    L.muon_version.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().muon_status_string(int(status)).decode()


def muon_version() -> int:
    return int(lib().muon_version())


def _check(rc: int, where: str):
    if rc != MUON_OK:
        raise MuonError(rc, where)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream) or None


def make_cfg(steps: int = 5, coeffs=(1.5, -0.5), eps: float = 1e-7, precision: int = MUON_BF16,
             per_step: bool = False, schedule: int = MUON_NS_AUTO, streams: int = 0, separate_apply: int = 0):
    """NsCfg plus the float array it points to (keep both alive)."""
    flat = [float(c) for row in coeffs for c in (row if isinstance(row, (tuple, list)) else (row,))]
    ncoef = len(coeffs[0]) if per_step else len(coeffs)
    arr = (ctypes.c_float * max(1, len(flat)))(*flat)
    cfg = NsCfg(int(steps), int(ncoef), ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)),
                int(bool(per_step)), float(eps), int(precision), int(schedule), int(streams),
                int(separate_apply))
    return cfg, arr


def _ptrs(ts) -> ctypes.Array:
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _split(x) -> list:
    """A [count, m, n] tensor or a sequence of [m, n] tensors -> list of matrices."""
    if x is None:
        return None
    if hasattr(x, "dim") and x.dim() == 3:
        return [x[i] for i in range(x.shape[0])]
    return list(x)


def _current_device():
    """The CUDA device the library's kernels will run on (torch's current one)."""
    import torch
    return torch.device("cuda", torch.cuda.current_device())


def _check_tensors(ts, what, dtypes, device):
    """Every tensor of ts has one of `dtypes` (all the same one) and, when
    `device` is given, lives on it; raises TypeError / ValueError otherwise."""
    names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
    first = None
    for t in ts:
        if t.dtype not in dtypes:
            raise TypeError(f"{what} must be {names} (got {t.dtype})")
        if first is None:
            first = t.dtype
        elif t.dtype != first:
            raise TypeError(f"every entry of {what} must have one dtype ({first} and {t.dtype} found)")
        if device is not None and t.device != device:
            raise ValueError(f"{what} must be on {device} (got {t.device})")


def _table(x, shape, what, dtypes, device):
    """(device pointer array, count, a tensor of the group) for x: a
    contiguous [count, *shape] tensor, whose pointers are computed from its
    base address (no per-matrix views: this runs on every step), or a
    sequence of contiguous tensors of `shape`.  dtypes / device as in
    _check_tensors."""
    if hasattr(x, "dim") and x.dim() == len(shape) + 1:
        if not x.is_contiguous() or tuple(x.shape[1:]) != tuple(shape):
            raise ValueError(f"{what} must be a contiguous [count, {', '.join(map(str, shape))}] tensor")
        _check_tensors([x], what, dtypes, device)
        count, step = x.shape[0], x.element_size()
        for d in shape:
            step *= d
        base = x.data_ptr()
        return (ctypes.c_void_p * count)(*range(base, base + count * step, step)), count, x
    ts = list(x)
    for t in ts:
        if not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError(f"every entry of {what} must be a contiguous {' x '.join(map(str, shape))} tensor")
    _check_tensors(ts, what, dtypes, device)
    return _ptrs(ts), len(ts), (ts[0] if ts else None)


@dataclass
class MuonGroup:
    """One shape group.  W, M: float32; G: bf16 or float32; O: optional output.
    Each is a [count, m, n] tensor or a list of [m, n] tensors, all contiguous
    CUDA tensors."""
    W: object
    M: object
    G: object
    lr: float
    beta: float
    O: object = None
    scale: float = 1.0
    nesterov: bool = True
    # spectral cap: unit estimates of W's top singular vectors ([count, m] and
    # [count, n] float32, updated in place), of its top singular value
    # ([count] float32, updated), and the threshold; cap_u None: off
    cap_u: object = None
    cap_v: object = None
    cap_sigma: object = None
    cap: float = 0.0


def _marshal_groups(groups: Sequence[MuonGroup], precision: int = MUON_BF16, device=None):
    """C group records for the groups.  W, M, cap_u, cap_v and cap_sigma must
    be float32, G bf16 or float32 (one dtype per group), O the precision's
    dtype; with `device` (calls that launch work) every tensor must be on it."""
    import torch
    f32 = (torch.float32,)
    gdt = (torch.bfloat16, torch.float32)
    odt = (torch.bfloat16,) if precision == MUON_BF16 else f32
    keep, cgroups = [], []
    for g in groups:
        w0 = g.W if hasattr(g.W, "dim") and g.W.dim() == 3 else list(g.W)[0]
        m, n = (g.W.shape[1:] if w0 is g.W else w0.shape)
        m, n = int(m), int(n)
        pw, count, wt = _table(g.W, (m, n), "W", f32, device)
        pm, cm, _ = _table(g.M, (m, n), "M", f32, device)
        pg, cgr, gt = _table(g.G, (m, n), "G", gdt, device)
        po, co = (None, count) if g.O is None else _table(g.O, (m, n), "O", odt, device)[:2]
        if not count == cm == cgr == co:
            raise ValueError("W, M, G (and O) must hold the same number of matrices")
        keep += [pw, pm, pg, po, g.W, g.M, g.G, g.O]
        cu = cv = None
        sig = None
        if g.cap_u is not None:
            cu, cnu, ut = _table(g.cap_u, (m,), "cap_u", f32, device)
            cv, cnv, vt = _table(g.cap_v, (n,), "cap_v", f32, device)
            if cnu != count or cnv != count:
                raise ValueError("cap_u / cap_v must hold one float32 vector of length m / n per matrix")
            if not hasattr(g.cap_sigma, "is_contiguous") or not g.cap_sigma.is_contiguous() or \
                    g.cap_sigma.numel() != count:
                raise ValueError("cap_sigma must be a contiguous float32 tensor with one entry per matrix")
            _check_tensors([g.cap_sigma], "cap_sigma", f32, device)
            sig = ctypes.c_void_p(g.cap_sigma.data_ptr())
            keep += [cu, cv, g.cap_u, g.cap_v, g.cap_sigma]
        cgroups.append(GroupC(m, n, count, _dtype_code(gt) if gt is not None else MUON_BF16,
                              ctypes.cast(pw, ctypes.POINTER(ctypes.c_void_p)),
                              ctypes.cast(pm, ctypes.POINTER(ctypes.c_void_p)),
                              ctypes.cast(pg, ctypes.POINTER(ctypes.c_void_p)),
                              ctypes.cast(po, ctypes.POINTER(ctypes.c_void_p)) if po is not None else None,
                              float(g.lr), float(g.beta), float(g.scale), int(bool(g.nesterov)),
                              ctypes.cast(cu, ctypes.POINTER(ctypes.c_void_p)) if cu is not None else None,
                              ctypes.cast(cv, ctypes.POINTER(ctypes.c_void_p)) if cv is not None else None,
                              sig, float(g.cap)))
    arr = (GroupC * len(cgroups))(*cgroups)
    return arr, keep


def _workspace(workspace, need, device):
    """The caller's workspace when it is a large enough uint8 tensor on the
    device, else a new one."""
    import torch
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise TypeError("workspace must be a contiguous uint8 tensor")
        if workspace.device != device:
            raise ValueError(f"workspace must be on {device} (got {workspace.device})")
        if workspace.numel() >= need:
            return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def muon_step_workspace_size(groups: Sequence[MuonGroup], steps=5, coeffs=(1.5, -0.5), eps=1e-7,
                             precision=MUON_BF16, per_step=False, schedule=MUON_NS_AUTO) -> int:
    cg, keep = _marshal_groups(groups, precision)
    cfg, arr = make_cfg(steps, coeffs, eps, precision, per_step, schedule)
    return int(lib().muon_step_workspace_size(cg, len(groups), ctypes.byref(cfg)))


def muon_step_phases(groups: Sequence[MuonGroup], steps=5, coeffs=(1.5, -0.5), eps=1e-7, precision=MUON_BF16,
                     per_step=False, schedule=MUON_NS_AUTO, separate_apply=0) -> list:
    """Names of the phases muon_step runs for these groups, in order (the
    intervals between the events muon_step_timed records)."""
    L = lib()
    cg, keep = _marshal_groups(groups, precision)
    cfg, arr = make_cfg(steps, coeffs, eps, precision, per_step, schedule, separate_apply=separate_apply)
    n = int(L.muon_step_phases(cg, len(groups), ctypes.byref(cfg), None, 0))
    if n < 0:
        _check(n, "muon_step_phases")
    out = (ctypes.c_int * max(1, n))()
    L.muon_step_phases(cg, len(groups), ctypes.byref(cfg), out, n)
    return [PHASES[out[i]] for i in range(n)]


def muon_step(groups: Sequence[MuonGroup], steps=5, coeffs=(1.5, -0.5), eps=1e-7, precision=MUON_BF16,
              per_step=False, workspace=None, norms_out=None, stream=None, events=None, schedule=MUON_NS_AUTO,
              streams=0, separate_apply=0):
    """One Muon step over every group (W and M updated in place).  Returns the
    workspace tensor so that callers can reuse it.  `events`: optional list of
    raw hipEvent_t handles (ints); when given, muon_step_timed records them at
    the phase boundaries."""
    import torch
    L = lib()
    dev = _current_device()
    cg, keep = _marshal_groups(groups, precision, dev)
    cfg, arr = make_cfg(steps, coeffs, eps, precision, per_step, schedule, streams, separate_apply)
    need = int(L.muon_step_workspace_size(cg, len(groups), ctypes.byref(cfg)))
    if need == 0:  # the size query has no status: ask the step itself, which validates first
        rc = L.muon_step(cg, len(groups), ctypes.byref(cfg), None, 0, None, None)
        _check(MUON_EINVAL if rc in (MUON_OK, MUON_EWORKSPACE) else rc, "muon_step")
    workspace = _workspace(workspace, need, dev)
    if norms_out is not None:
        total = sum(int(c.count) for c in cg)
        if not norms_out.is_contiguous() or norms_out.numel() < total:
            raise ValueError("norms_out must be a contiguous float32 tensor with one entry per matrix")
        _check_tensors([norms_out], "norms_out", (torch.float32,), dev)
    nptr = ctypes.cast(ctypes.c_void_p(norms_out.data_ptr()), ctypes.POINTER(ctypes.c_float)) \
        if norms_out is not None else None
    if events is None:
        rc = L.muon_step(cg, len(groups), ctypes.byref(cfg), ctypes.c_void_p(workspace.data_ptr()),
                         workspace.numel(), nptr, _stream_handle(stream))
        _check(rc, "muon_step")
    else:
        ev = (ctypes.c_void_p * len(events))(*events)
        rc = L.muon_step_timed(cg, len(groups), ctypes.byref(cfg), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel(), nptr, _stream_handle(stream),
                               ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), len(events))
        _check(rc, "muon_step_timed")
    return workspace


def muon_ns_workspace_size(m, n, batch, dtype, steps=5, coeffs=(1.5, -0.5), eps=1e-7, per_step=False,
                           schedule=MUON_NS_AUTO) -> int:
    cfg, arr = make_cfg(steps, coeffs, eps, dtype, per_step, schedule)
    return int(lib().muon_ns_workspace_size(int(m), int(n), int(batch), int(dtype), ctypes.byref(cfg)))


def _strided_stack(t):
    """(batch, m, n, ld, stride) of a [batch, m, n] (or [m, n]) tensor whose
    rows are contiguous (unit column stride)."""
    t3 = t if t.dim() == 3 else t.unsqueeze(0)
    if t3.dim() != 3 or t3.stride(2) != 1:
        raise ValueError("the matrices must have contiguous rows (unit column stride)")
    b, m, n = t3.shape
    ld = t3.stride(1) if m > 1 else n
    stride = t3.stride(0) if b > 1 else m * ld
    return t3, int(b), int(m), int(n), int(ld), int(stride)


def muon_ns_orthogonalize(G, O, steps=5, coeffs=(1.5, -0.5), eps=1e-7, per_step=False, workspace=None,
                          stream=None, schedule=MUON_NS_AUTO):
    """O[b] = NS(G[b]) for [batch, m, n] (or [m, n]) tensors whose rows are
    contiguous: row and matrix strides (ld, stride) are taken from G, and O
    must have the same strides (O may be G itself: in place)."""
    import torch
    L = lib()
    dev = _current_device()
    G3, b, m, n, ld, stride = _strided_stack(G)
    O3, bo, mo, no, ldo, so = _strided_stack(O)
    if (b, m, n) != (bo, mo, no) or (ld, stride) != (ldo, so) or G3.dtype != O3.dtype:
        raise ValueError("G and O must have one shape, dtype and stride layout")
    _check_tensors([G3, O3], "G and O", (torch.bfloat16, torch.float32), dev)
    dt = _dtype_code(G3)
    cfg, arr = make_cfg(steps, coeffs, eps, dt, per_step, schedule)
    need = int(L.muon_ns_workspace_size(m, n, b, dt, ctypes.byref(cfg)))
    if need == 0:
        _check(MUON_EINVAL, "muon_ns_workspace_size")
    workspace = _workspace(workspace, need, dev)
    rc = L.muon_ns_orthogonalize(ctypes.c_void_p(G3.data_ptr()), ctypes.c_void_p(O3.data_ptr()), dt, m, n, ld, b,
                                 stride, ctypes.byref(cfg), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                 _stream_handle(stream))
    _check(rc, "muon_ns_orthogonalize")
    return workspace


def muon_ns_orthogonalize_noalloc(G, O, steps=5, coeffs=(1.5, -0.5), eps=1e-7, per_step=False, stream=None,
                                  schedule=MUON_NS_AUTO):
    """muon_ns_orthogonalize on the library's own device array instead of a
    workspace (nothing is allocated; at most muon_ns_noalloc_max_bytes() of
    workspace need; calls that overlap on one GPU race)."""
    import torch
    L = lib()
    dev = _current_device()
    G3, b, m, n, ld, stride = _strided_stack(G)
    O3, bo, mo, no, ldo, so = _strided_stack(O)
    if (b, m, n) != (bo, mo, no) or (ld, stride) != (ldo, so) or G3.dtype != O3.dtype:
        raise ValueError("G and O must have one shape, dtype and stride layout")
    _check_tensors([G3, O3], "G and O", (torch.bfloat16, torch.float32), dev)
    dt = _dtype_code(G3)
    cfg, arr = make_cfg(steps, coeffs, eps, dt, per_step, schedule)
    rc = L.muon_ns_orthogonalize_noalloc(ctypes.c_void_p(G3.data_ptr()), ctypes.c_void_p(O3.data_ptr()), dt, m, n,
                                         ld, b, stride, ctypes.byref(cfg), _stream_handle(stream))
    _check(rc, "muon_ns_orthogonalize_noalloc")


def muon_query_flags(workspace) -> int:
    """The non-finite flag (0 or 1) of the last muon_step / muon_ns_orthogonalize
    call that used this workspace; synchronise its stream first."""
    import torch
    if workspace is None or workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise TypeError("workspace must be the uint8 device tensor returned by muon_step")
    out = ctypes.c_int(-1)
    _check(lib().muon_query_flags(ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(out)), "muon_query_flags")
    return int(out.value)


def muon_ns_batched_small(X, Y, steps=1, coeffs=(1.5, -0.5), eps=1e-7, per_step=False, stream=None):
    """Y[b] = NS(X[b]) for a contiguous [batch, m, n] stack of small matrices."""
    import torch
    L = lib()
    if X.dim() != 3 or not (X.is_contiguous() and Y.is_contiguous()) or X.shape != Y.shape or X.dtype != Y.dtype:
        raise ValueError("X and Y must be contiguous [batch, m, n] tensors of one shape and dtype")
    _check_tensors([X, Y], "X and Y", (torch.bfloat16, torch.float32), _current_device())
    b, m, n = X.shape
    dt = _dtype_code(X)
    cfg, arr = make_cfg(steps, coeffs, eps, dt, per_step)
    rc = L.muon_ns_batched_small(ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(Y.data_ptr()), dt, m, n, b,
                                 ctypes.byref(cfg), _stream_handle(stream))
    _check(rc, "muon_ns_batched_small")


def muon_ns_factored(V, K, C=None, O=None, steps=1, coeffs=(1.5, -0.5), eps=1e-7, per_step=False, stream=None):
    """NS of X[b] = V[b] K[b]^T from the factors: returns the [batch, r, r]
    float32 core C (NS(X) = V C K^T), and fills O ([batch, m, n] bf16) with the
    dense result when given."""
    import torch
    L = lib()
    if V.dim() != 3 or K.dim() != 3 or V.shape[0] != K.shape[0] or V.shape[2] != K.shape[2]:
        raise ValueError("V, K must be [batch, m, r] and [batch, n, r]")
    if not (V.is_contiguous() and K.is_contiguous()) or V.dtype != K.dtype:
        raise ValueError("V and K must be contiguous tensors of one dtype")
    b, m, r = V.shape
    n = K.shape[1]
    dev = _current_device()
    _check_tensors([V, K], "V and K", (torch.bfloat16, torch.float32), dev)
    dt = _dtype_code(V)
    if C is None:
        C = torch.empty(b, r, r, dtype=torch.float32, device=dev)
    if not C.is_contiguous() or tuple(C.shape) != (b, r, r):
        raise ValueError(f"C must be a contiguous [{b}, {r}, {r}] float32 tensor")
    _check_tensors([C], "C", (torch.float32,), dev)
    if O is not None and (not O.is_contiguous() or tuple(O.shape) != (b, m, n) or O.dtype != V.dtype):
        raise ValueError("O must be a contiguous [batch, m, n] tensor of V's dtype")
    if O is not None:
        _check_tensors([O], "O", (V.dtype,), dev)
    cfg, arr = make_cfg(steps, coeffs, eps, dt, per_step)
    rc = L.muon_ns_factored(ctypes.c_void_p(V.data_ptr()), ctypes.c_void_p(K.data_ptr()), dt, m, n, r, b,
                            ctypes.byref(cfg), ctypes.cast(ctypes.c_void_p(C.data_ptr()), ctypes.POINTER(ctypes.c_float)),
                            ctypes.c_void_p(O.data_ptr()) if O is not None else None, _stream_handle(stream))
    _check(rc, "muon_ns_factored")
    return C


def _fptr(t):
    return None if t is None else ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))


def muon_ssm_momentum(V, K, M, S=None, decay=None, beta=0.9, steps=1, coeffs=(1.5, -0.5), eps=1e-7, per_step=False,
                      workspace=None, stream=None, events=None):
    """The momentum pathway over nseq sequences of T factored injections:
    V [nseq, T, m, r] and K [nseq, T, n, r] bf16, M (and S) [nseq, m, n]
    float32 updated in place to the states after the T tokens
    (M_t = beta M_{t-1} + NS(V_t K_t^T); S_t = decay_t S_{t-1} + M_t with
    decay [nseq, T] float32).  Returns the workspace tensor for reuse.
    `events`: optional list of 3 raw hipEvent_t handles (ints) recorded by
    muon_ssm_momentum_timed at its phase boundaries."""
    import torch
    L = lib()
    if V.dim() != 4 or K.dim() != 4 or V.shape[:2] != K.shape[:2] or V.shape[3] != K.shape[3]:
        raise ValueError("V, K must be [nseq, T, m, r] and [nseq, T, n, r]")
    nseq, T, m, r = V.shape
    n = K.shape[2]
    dev = _current_device()
    if not (V.is_contiguous() and K.is_contiguous()):
        raise ValueError("V and K must be contiguous")
    _check_tensors([V, K], "V and K", (torch.bfloat16,), dev)
    for name, t in (("M", M), ("S", S)):
        if t is not None and (not t.is_contiguous() or tuple(t.shape) != (nseq, m, n)):
            raise ValueError(f"{name} must be a contiguous [{nseq}, {m}, {n}] float32 tensor")
    _check_tensors([M] + ([S] if S is not None else []), "M and S", (torch.float32,), dev)
    if S is not None:
        if decay is None or not decay.is_contiguous() or tuple(decay.shape) != (nseq, T):
            raise ValueError(f"with S, decay must be a contiguous [{nseq}, {T}] float32 tensor")
        _check_tensors([decay], "decay", (torch.float32,), dev)
    need = int(L.muon_ssm_momentum_workspace_size(m, n, r, nseq, T))
    if need == 0:
        raise MuonError(MUON_EUNSUPPORTED, "muon_ssm_momentum_workspace_size")
    ws = _workspace(workspace, need, dev)
    cfg, arr = make_cfg(steps, coeffs, eps, MUON_BF16, per_step)
    args = (ctypes.c_void_p(V.data_ptr()), ctypes.c_void_p(K.data_ptr()), MUON_BF16, m, n, r, nseq, T, float(beta),
            _fptr(decay if S is not None else None), _fptr(M), _fptr(S), ctypes.byref(cfg),
            ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_handle(stream))
    if events is None:
        rc = L.muon_ssm_momentum(*args)
    else:
        ev = (ctypes.c_void_p * len(events))(*events)
        rc = L.muon_ssm_momentum_timed(*args, ev, len(events))
    _check(rc, "muon_ssm_momentum")
    return ws


class AdamwTensors:
    """Marshalled argument arrays of muon_adamw for fixed lists of tensors
    (build once, call every step; the tensors must stay alive)."""

    def __init__(self, params, grads, exp_avg, exp_avg_sq):
        n = len(params)
        if not (len(grads) == len(exp_avg) == len(exp_avg_sq) == n):
            raise ValueError("params, grads, exp_avg, exp_avg_sq must have the same length")
        import torch
        self.n = n
        self.gd = _dtype_code(grads[0]) if n else MUON_F32
        for p, g, m, v in zip(params, grads, exp_avg, exp_avg_sq):
            if not all(t.is_contiguous() for t in (p, g, m, v)) or \
                    not (p.numel() == g.numel() == m.numel() == v.numel()):
                raise ValueError("every tensor must be contiguous, with matching sizes")
        self.device = params[0].device if n else None
        if n and self.device.type != "cuda":
            raise ValueError(f"params must be CUDA tensors (got {self.device})")
        _check_tensors(list(params), "params", (torch.float32,), self.device)
        _check_tensors(list(exp_avg), "exp_avg", (torch.float32,), self.device)
        _check_tensors(list(exp_avg_sq), "exp_avg_sq", (torch.float32,), self.device)
        _check_tensors(list(grads), "grads", (torch.bfloat16, torch.float32), self.device)
        cast = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))  # noqa: E731
        self._keep = [params, grads, exp_avg, exp_avg_sq]
        self._arrays = [_ptrs(params), _ptrs(grads), _ptrs(exp_avg), _ptrs(exp_avg_sq)]
        self.ptrs = [cast(a) for a in self._arrays]
        self.numel = (ctypes.c_longlong * max(1, n))(*[p.numel() for p in params])

    def step(self, lr, step, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, stream=None):
        if self.n == 0:
            return
        if self.device != _current_device():
            raise ValueError(f"the tensors are on {self.device}, the current device is {_current_device()}")
        rc = lib().muon_adamw(self.n, *self.ptrs, self.numel, self.gd, float(lr), float(beta1), float(beta2),
                              float(eps), float(weight_decay), int(step), _stream_handle(stream))
        _check(rc, "muon_adamw")


def muon_adamw(params, grads, exp_avg, exp_avg_sq, lr, step, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
               stream=None):
    """AdamW over lists of contiguous float32 tensors (params, exp_avg,
    exp_avg_sq updated in place); grads float32 or bf16 (one dtype)."""
    AdamwTensors(params, grads, exp_avg, exp_avg_sq).step(lr, step, beta1, beta2, eps, weight_decay, stream)


def muon_spectral_diag(A, iters=32, orth_err=True, sigma_max=True, sigma_min=True, workspace=None, stream=None,
                       events=None):
    """Orthogonality error and Lanczos estimates of the extreme singular values
    of every matrix of A ([batch, m, n] or [m, n], contiguous, float32 or
    bf16).  Returns a dict of float32 [batch] tensors for the quantities
    asked for.  events: optional list of HIP event handles (int), recorded
    before the first pass and after each pass (muon_spectral_diag_timed)."""
    import torch
    L = lib()
    if A.dim() == 2:
        A = A.unsqueeze(0)
    if A.dim() != 3 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [batch, m, n] tensor")
    dev = _current_device()
    _check_tensors([A], "A", (torch.bfloat16, torch.float32), dev)
    b, m, n = A.shape
    dt = _dtype_code(A)
    outs = {}
    for name, want in (("orth_err", orth_err), ("sigma_max", sigma_max), ("sigma_min", sigma_min)):
        if want:
            outs[name] = torch.empty(b, dtype=torch.float32, device=dev)
    need = L.muon_spectral_diag_workspace_size(m, n, b, dt, int(iters))
    if need == 0:
        rc = L.muon_spectral_diag(None, dt, m, n, b, int(iters), None, None, None, None, 0, None)
        _check(rc if rc != MUON_OK else -1, "muon_spectral_diag")
    workspace = _workspace(workspace, max(int(need), 1), dev)
    ptr = lambda k: ctypes.c_void_p(outs[k].data_ptr()) if k in outs else None  # noqa: E731
    args = (ctypes.c_void_p(A.data_ptr()), dt, m, n, b, int(iters), ptr("orth_err"), ptr("sigma_max"),
            ptr("sigma_min"), ctypes.c_void_p(workspace.data_ptr()), need, _stream_handle(stream))
    if events is None:
        rc = L.muon_spectral_diag(*args)
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        rc = L.muon_spectral_diag_timed(*args, arr, len(events))
    _check(rc, "muon_spectral_diag")
    return outs
