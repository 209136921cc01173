"""Shared test helpers: move seeded inputs to the GPU and compare with the oracle."""
import numpy as np

import oracle as orc

BF16_TOL = 2e-2      # relative Frobenius error, bf16 matrix-core path
F32_TOL = 1e-5       # relative Frobenius error, fp32 path
MOM_TOL = 1e-6       # momentum buffer (float32 elementwise)


def to_torch_bits(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def device_group(g, dev="cuda"):
    """Group of numpy arrays -> dict of device tensors [count, m, n]."""
    import torch
    G = to_torch_bits(g.G) if g.grad_dtype == "bf16" else torch.from_numpy(g.G)
    return {"G": G.to(dev).contiguous(), "W": torch.from_numpy(g.W).to(dev).contiguous(),
            "M": torch.from_numpy(g.M).to(dev).contiguous()}


def grad64(g, i):
    return orc.widen_bf16(g.G[i]) if g.grad_dtype == "bf16" else orc.widen_f32(g.G[i])


def t64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def sigma_deviation(O, ref):
    """max_i |sigma_i(O) - sigma_i(ref)| over the sorted singular values
    (LAPACK through numpy, float64): reported, not gated."""
    a = np.linalg.svd(np.asarray(O, dtype=np.float64), compute_uv=False)
    b = np.linalg.svd(np.asarray(ref, dtype=np.float64), compute_uv=False)
    return float(np.max(np.abs(np.sort(a) - np.sort(b))))


def compare_step(g, i, out, dev_tensors, w, tol, steps=None, zero_eps=False, sigma=False):
    """Compare matrix i of a group after a GPU muon_step with the oracle.
    Returns a dict of errors (with sigma: also the max singular-value
    deviation of the update); asserts the tolerances."""
    steps = w.steps if steps is None else steps
    ref = orc.muon_step(orc.widen_f32(g.W[i]), orc.widen_f32(g.M[i]), grad64(g, i), beta=w.beta, lr=w.lr,
                        nesterov=w.nesterov, steps=steps, coeffs=w.coeffs, eps=0.0 if zero_eps else w.eps,
                        scale=w.scale, per_step=w.per_step)
    O = t64(out["O"][i])
    Wn = t64(dev_tensors["W"][i])
    Mn = t64(dev_tensors["M"][i])
    W0 = orc.widen_f32(g.W[i])
    e_o = orc.rel_frobenius(O, ref["O"])
    e_m = orc.rel_frobenius(Mn, ref["M"])
    e_w = orc.rel_frobenius(Wn - W0, ref["W"] - W0)
    ulp = np.spacing(np.maximum(np.abs(W0), np.abs(ref["W"])).astype(np.float32)).astype(np.float64)
    w_abs_ok = np.all(np.abs(Wn - ref["W"]) <= w.lr * w.scale * np.abs(O - ref["O"]).max() + ulp + 1e-12)
    res = {"O": e_o, "M": e_m, "W_inc": e_w, "W_abs_ok": bool(w_abs_ok)}
    if sigma:
        res["sigma_dev"] = sigma_deviation(O, ref["O"])
    assert e_o <= tol, res
    assert e_m <= MOM_TOL, res
    assert e_w <= tol, res
    assert w_abs_ok, res
    return res, ref


class Report:
    """Worst errors over the matrices of one config, printed as one line."""

    def __init__(self, name):
        self.name, self.n, self.worst = name, 0, {}

    def add(self, res):
        self.n += 1
        for k, v in res.items():
            if isinstance(v, float):
                self.worst[k] = max(self.worst.get(k, 0.0), v)

    def line(self):
        body = " ".join(f"max_{k} {v:.3e}" for k, v in sorted(self.worst.items()))
        return f"[parity] {self.name}: {self.n} matrices compared, {body}"
