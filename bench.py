"""Benchmark of the Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_step]

Default workload: one full Muon step over the Mamba-2-130M projection weights,
24 out_proj (768 x 1536) + 24 in_proj (3352 x 768) matrices, bf16 gradients
with singular values log-uniform in [1e-6, 1], fp32 weights and momentum,
beta 0.95 Nesterov, lr 0.02, 5 cubic Newton-Schulz steps.  Inputs are seeded
and synthetic (workloads.py) and resident in HBM before timing starts.

Prints one JSON line: steps/s over exactly K timed steps (wall clock between
two device synchronisations), per-kernel durations from HIP events recorded by
muon_step_timed in K further steps (those run the phases one after another on
one stream), the roofline of the dominant kernel, and the fp64 oracle timed on
a bounded sample on the host cores.
Other workloads: injections, injections_factored, ssm_momentum, adamw, diag, sweep (1/3/5/8
NS steps with the orthogonality error of each update); out_proj, in_proj,
single are for exploration.  --schedule, --separate-apply, --one-stream and
--per-matrix switch single design choices of the full step for A/B runs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon NS steps/s + TFLOP/s, MFMA util (Mamba-2-130M-shaped grads), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak (published)
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector peak (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "spectral_optimizer_ssm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COPY_CAL_BYTES = 1 << 30      # bytes read (and written) by the calibration copy


def copy_calibration(torch):
    """A plain streaming copy of known size (torch's elementwise negation, one
    read and one write of every byte) so that the HBM counters of a profiled
    run can be scaled to bytes."""
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def ingest_counters(fetch_csv: str, write_csv: str, workload: str, kernels: dict):
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; both with
    --copy-calibration) into HBM bytes per launch, scaled so that the copy
    kernel reads and writes COPY_CAL_BYTES, and stores them with the hash of
    the kernel sources they were taken on."""
    import csv
    def load(path, counter):
        rows = sorted((r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter),
                      key=lambda r: (r["Queue_Id"], int(r["Dispatch_Id"])))
        per = {}
        after_momentum = {}  # per queue: a momentum pass ran since the last symmetric product
        for r in rows:
            name, q = r["Kernel_Name"], r["Queue_Id"]
            if "momentum_" in name:
                after_momentum[q] = True
            elif "symprod_bf16_kernel" in name and after_momentum.get(q):
                name = "gram:" + name  # the first symmetric product of a chain is its Gram
                after_momentum[q] = False
            per.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return per
    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    def copy_factor(per):
        vals = [v for k, vs in per.items() if "neg_kernel" in k for v in vs]
        if not vals:
            raise SystemExit("no calibration copy kernel in " + ", ".join(per))
        return COPY_CAL_BYTES / float(np.median(vals))
    fr, fw = copy_factor(fetch), copy_factor(write)
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    for name, (pattern, files) in kernels.items():
        base = pattern[len("gram:"):] if pattern.startswith("gram:") else pattern
        keep = lambda k: base in k and (k.startswith("gram:") == pattern.startswith("gram:"))  # noqa: E731
        rd = [v for k, vs in fetch.items() if keep(k) for v in vs]
        wr = [v for k, vs in write.items() if keep(k) for v in vs]
        if not rd or not wr:
            log(f"[ingest] no dispatches of {pattern}")
            continue
        data[f"{name}@{workload}"] = {
            "source_hash": kernel_source_hash(files), "dispatches": [len(rd), len(wr)],
            "fetch_bytes": float(np.mean(rd)) * fr, "write_bytes": float(np.mean(wr)) * fw,
            "bytes_per_launch": float(np.mean(rd)) * fr + float(np.mean(wr)) * fw,
            "fetch_factor": round(fr, 4), "write_factor": round(fw, 4)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    log(f"[ingest] read factor {fr:.4f}, write factor {fw:.4f} -> {TRAFFIC_FILE}")


def measured_traffic(kernel: str, workload: str, files):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when none were taken or the kernel sources changed since."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = data.get(f"{kernel}@{workload}")
    if not e or e.get("source_hash") != kernel_source_hash(files):
        return None
    return e.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# full Muon step (default)
# ----------------------------------------------------------------------------
def ns_flops(s, l):
    """Algorithmic flops of one cubic step on an s x l iterate: symmetric Gram
    s(s+1)l plus combine 2 s^2 l."""
    return s * (s + 1) * l, 2 * s * s * l


def graph_steps(torch, step, k):
    """The step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed k times: no host work or launch gaps between the kernels."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(k):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / k
    return {"ms_per_step": round(ms, 4), "steps_per_s": round(1e3 / ms, 3), "steps": k}


def workload_for(args, wl):
    """The seeded inputs of a step workload: the full step (both projection
    groups, the headline), one projection group, or the single fp32 matrix."""
    if args.workload == "out_proj":
        return wl.config2(), "mamba2-130m out_proj group: 24x 768x1536, bf16 grads (singular values log-uniform in " \
                             "[1e-3, 1]), fp32 W/M"
    if args.workload == "in_proj":
        return wl.config3(), "mamba2-130m in_proj group: 24x 3352x768 (tall), bf16 Gaussian grads with a rank-8 " \
                             "spike 10x the bulk, fp32 W/M"
    if args.workload == "single":
        return wl.config1(), "single fp32 gradient 128x64 (fp32 path), W N(0,0.02), M = 0"
    return wl.config4(count=args.count, steps=args.ns_steps), \
        f"mamba2-130m-full-step: {args.count}x out_proj 768x1536 + {args.count}x in_proj 3352x768, bf16 grads, fp32 W/M"


def bench_full_step(args, torch, mu, wl):
    steps_ns = args.ns_steps
    log(f"[bench] generating {args.workload} inputs")
    t0 = time.time()
    w, desc = workload_for(args, wl)
    log(f"[bench] generated in {time.time() - t0:.1f}s")
    fp32 = w.groups[0].grad_dtype != "bf16"
    prec = mu.MUON_F32 if fp32 else mu.MUON_BF16
    groups, devs = [], []
    gen = torch.Generator(device="cuda").manual_seed(5)
    for g in w.groups:
        G = (torch.from_numpy(g.G) if fp32 else torch.from_numpy(g.G.view(np.int16)).view(torch.bfloat16)).cuda()
        W = torch.from_numpy(g.W).cuda()
        M = torch.from_numpy(g.M).cuda()
        devs.append((G, W, M))
        cap = {}
        if args.cap:  # spectral cap on, estimates from random unit vectors
            u = torch.randn((g.count, g.m), generator=gen, device="cuda")
            v = torch.randn((g.count, g.n), generator=gen, device="cuda")
            cap = dict(cap_u=u / u.norm(dim=1, keepdim=True), cap_v=v / v.norm(dim=1, keepdim=True),
                       cap_sigma=torch.zeros(g.count, device="cuda"), cap=0.0)
        groups.append(mu.MuonGroup(W=W, M=M, G=G, lr=w.lr, beta=w.beta, nesterov=w.nesterov, **cap))
    streams = 1 if args.one_stream else 0
    sched = {"auto": mu.MUON_NS_AUTO, "iterate": mu.MUON_NS_ITERATE, "accumulate": mu.MUON_NS_ACCUMULATE}[args.schedule]
    opts = dict(steps=steps_ns, streams=streams, schedule=sched, separate_apply=int(args.separate_apply),
                precision=prec)
    if args.per_matrix:  # one muon_step call per matrix (the ungrouped launch pattern)
        return bench_per_matrix(args, torch, mu, w, groups, opts)
    ws = mu.muon_step(groups, **opts)  # allocates the workspace once
    torch.cuda.synchronize()
    # the library lists the phases muon_step_timed brackets with events
    phases = mu.muon_step_phases(groups, steps=steps_ns, schedule=sched, separate_apply=int(args.separate_apply),
                                 precision=prec)
    n_ev = len(phases) + 1
    log(f"[bench] schedule: {' '.join(phases)}")

    def make_events(k):
        evs = []
        for _ in range(k):
            row = []
            for _ in range(n_ev):
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                row.append(e)
            evs.append(row)
        torch.cuda.synchronize()
        return evs

    for _ in range(args.warmup):
        mu.muon_step(groups, workspace=ws, **opts)
    # the timed steps: plain muon_step (shape groups as two concurrent chains)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        mu.muon_step(groups, workspace=ws, **opts)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    cold = cold_cache_steps(torch, lambda: mu.muon_step(groups, workspace=ws, **opts), args.steps)
    graph = graph_steps(torch, lambda: mu.muon_step(groups, workspace=ws, **opts), args.steps) if args.graph else None
    # per-kernel durations: the same steps again through muon_step_timed,
    # which runs the phases one after another on one stream
    evs = make_events(args.steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        mu.muon_step(groups, steps=steps_ns, workspace=ws, events=[e.cuda_event for e in evs[k]], schedule=sched,
                     separate_apply=int(args.separate_apply), precision=prec)
    torch.cuda.synchronize()
    ms_serial = (time.perf_counter() - t2) * 1e3 / args.steps

    # algorithmic work of each launch of the executed schedule (every large
    # group takes the same schedule here; per-group passes follow group order)
    per_group = [(g, min(g.m, g.n), max(g.m, g.n)) for g in w.groups]
    gsz, xsz = (4, 4) if fp32 else (2, 2)  # bytes of a gradient / iterate element
    gram_f = sum(g.count * ns_flops(s, l)[0] for g, s, l in per_group)
    comb_f = sum(g.count * ns_flops(s, l)[1] for g, s, l in per_group)
    sym_f = sum(g.count * s * s * (s + 1) for g, s, l in per_group)  # one symmetric s x s product
    sym_products = []
    if "symprod" in phases:  # the accumulated schedule's products per launch
        for k in range(steps_ns):
            sym_products.append(int(k + 1 < steps_ns) + int(k >= 1))
            if k + 1 < steps_ns:
                sym_products.append(1)
    assert len(sym_products) == phases.count("symprod")
    work = []
    gi_m = gi_a = si = gi_n = 0
    for ph in phases:
        if ph == "momentum":  # G in, M in and out, the iterate out
            g, s, l = per_group[gi_m]
            work.append(g.count * g.m * g.n * (gsz + 8 + xsz))
            gi_m += 1
        elif ph == "apply":  # the iterate in, W in and out
            g, s, l = per_group[gi_a]
            work.append(g.count * g.m * g.n * (xsz + 8))
            gi_a += 1
        elif ph == "gram":
            work.append(gram_f)
        elif ph in ("combine", "combine_apply"):
            work.append(comb_f)
        elif ph == "symprod":
            work.append(sym_products[si] * sym_f)
            si += 1
        elif ph == "flags":  # the non-finite flag: one small read of the partial sums
            work.append(0)
        elif ph == "ns_small":  # the whole iteration on chip: per step a Gram and a combine
            g, s, l = per_group[gi_n]
            work.append(g.count * sum(ns_flops(s, l)) * steps_ns)
            gi_n += 1
        elif ph in ("cap", "power"):  # bytes: read X (2 B/elt) / read W (4 B/elt); power follows apply
            g, s, l = per_group[gi_a if ph == "cap" else gi_a - 1]
            work.append(g.count * g.m * g.n * (2 if ph == "cap" else 4))
        else:
            raise RuntimeError(f"unexpected phase {ph}")
    dur = {}
    for k in range(args.steps):
        e = evs[k]
        for j, ph in enumerate(phases):
            dur.setdefault(ph, []).append((e[j].elapsed_time(e[j + 1]), work[j]))

    kernels = {}
    for kind, rows in dur.items():
        tot_ms = sum(d for d, _ in rows)
        tot_w = sum(wk for _, wk in rows)
        n = len(rows)
        rate = tot_w / (tot_ms * 1e-3)
        if kind == "flags":
            kernels[kind] = {"avg_us": tot_ms / n * 1e3, "launches": n}
        elif kind in ("momentum", "apply", "cap", "power"):
            kernels[kind] = {"avg_us": tot_ms / n * 1e3, "launches": n, "bytes_per_launch": tot_w / n,
                             "gbs": rate / 1e9, "frac": rate / 1e9 / PEAK_HBM_GBS}
        else:
            peak = PEAK_F32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
            kernels[kind] = {"avg_us": tot_ms / n * 1e3, "launches": n, "flops_per_launch": tot_w / n,
                             "tflops": rate / 1e12, "frac": rate / 1e12 / peak}
        kernels[kind]["ms_per_step"] = tot_ms / args.steps
    if "combine_apply" in kernels:  # the fused apply's bytes: X read, W read and written
        nel = sum(g.count * g.m * g.n for g, s, l in per_group)
        ca = kernels["combine_apply"]
        ca["apply_bytes_per_launch"] = nel * 10
        ca["apply_gbs"] = nel * 10 / (ca["avg_us"] * 1e-6) / 1e9
    ns_kinds = [k for k in ("gram", "symprod", "combine", "combine_apply", "ns_small") if k in dur]
    ns_ms = sum(sum(d for d, _ in dur[k]) for k in ns_kinds) / args.steps
    ns_flops_step = sum(sum(wk for _, wk in dur[k]) for k in ns_kinds) / args.steps
    ns_tflops = ns_flops_step / (ns_ms * 1e-3) / 1e12
    # work the plain iteration (a Gram and a combine per step) would need
    iter_flops_step = sum(sum(ns_flops(s, l)) * g.count for g, s, l in per_group) * steps_ns

    # dominant kernel: the one with the most GPU time per step
    dom = max(ns_kinds + [k for k in ("momentum", "apply") if k in kernels], key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    names = {"gram": "symprod_bf16_kernel", "combine": "combine_bf16_kernel", "symprod": "symprod_bf16_kernel",
             "combine_apply": "combine_bf16_kernel<fused apply>", "momentum": "momentum_*_kernel",
             "apply": "apply_*_kernel", "ns_small": "ns_small_f32_kernel" if fp32 else "ns_small_bf16_kernel"}
    if dom in ("momentum", "apply"):
        roofline = {"bound": "hbm", "kernel": names[dom], "achieved": round(kd["gbs"], 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(kd["frac"], 4),
                    "traffic": measured_traffic(names[dom].replace("*", "wide" if dom == "momentum" else "tall"),
                                                args.workload, ELEMENTWISE)}
    elif fp32:
        # float32 iteration on the vector ALUs (no matrix cores): fp32 vector peak
        tf = kd["tflops"]
        roofline = {"bound": "alu", "kernel": names[dom], "achieved": round(tf, 4), "peak": PEAK_F32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / PEAK_F32_TFLOPS, 6), "traffic": None}
    else:
        roofline = {"bound": "mfma", "kernel": names[dom], "achieved": round(kd["tflops"], 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(kd["frac"], 4),
                    "traffic": measured_traffic(names[dom], args.workload, GEMM)}
    result = {
        "metric": METRIC, "value": round(1e3 / ms_per_step, 3), "unit": "steps/s",
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_one_stream": round(ms_serial, 4),
        "cold_cache": cold,
        **({"graph": graph} if graph is not None else {}),
        "ns_iters_per_s": round(steps_ns * 1e3 / ms_per_step, 2),
        "ns_tflops": round(ns_tflops, 2), "mfma_util": round(ns_tflops / PEAK_BF16_TFLOPS, 4),
        "ns_iteration_equivalent_tflops": round(iter_flops_step / (ns_ms * 1e-3) / 1e12, 2),
        "dtype": "f32" if fp32 else "bf16",
        "config": {"workload": f"{desc}, {steps_ns} cubic NS steps",
                   "matrices": sum(g.count for g in w.groups), "ns_steps": steps_ns, "parallelism": "none (1 GPU)",
                   "spectral_cap": bool(args.cap), "ns_schedule": args.schedule,
                   "separate_apply": bool(args.separate_apply), "chains": 1 if args.one_stream else "auto",
                   "schedule": " ".join(phases)},
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_step(w, steps_ns, one_core=args.workload in ("single", "out_proj"))
    return result


def cold_cache_steps(torch, step, k):
    """Per-step durations with L2 and the 256 MB last-level cache flushed
    before each step (a 512 MB fill, outside the events): median, p10, p90."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    for a, b in ev:
        flush.zero_()
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    del flush
    return {"ms_median": round(float(np.median(ms)), 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
            "ms_p90": round(float(np.percentile(ms, 90)), 4), "steps": k}


def bench_per_matrix(args, torch, mu, w, groups, opts):
    """The full step as one muon_step call per matrix (48 calls of one
    matrix each, every kernel launched per matrix): the ungrouped pattern the
    grouped launches replace."""
    single = [mu.MuonGroup(W=g.W[i:i + 1], M=g.M[i:i + 1], G=g.G[i:i + 1], lr=g.lr, beta=g.beta,
                           nesterov=g.nesterov) for g in groups for i in range(g.W.shape[0])]
    ws = None
    for g in single:  # grows the workspace to the largest matrix's need
        ws = mu.muon_step([g], workspace=ws, **opts)
    for _ in range(args.warmup):
        for g in single:
            mu.muon_step([g], workspace=ws, **opts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for g in single:
            mu.muon_step([g], workspace=ws, **opts)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"metric": METRIC, "value": round(1e3 / ms, 3), "unit": "steps/s", "ms_per_step": round(ms, 4),
            "dtype": "bf16",
            "config": {"workload": f"mamba2-130m-full-step, one call per matrix: {args.count}x out_proj 768x1536 + "
                                   f"{args.count}x in_proj 3352x768, {opts['steps']} cubic NS steps",
                       "matrices": 2 * args.count, "calls_per_step": len(single), "ns_schedule": args.schedule,
                       "separate_apply": bool(args.separate_apply)}}


def bench_sweep(args, torch, mu, wl):
    """Steps sweep of the full step (1, 3, 5, 8 NS steps) on the zero-momentum
    variant of the inputs (U = (1 + beta) G): optimizer steps/s at each step
    count, and the orthogonality error ||O O^T - I||_F / sqrt(s) and extreme
    singular value of every update O, measured on the GPU by
    muon_spectral_diag (32 Lanczos steps)."""
    log(f"[bench] generating zero-momentum full-step inputs ({args.count}+{args.count} matrices)")
    w = wl.config4(count=args.count, zero_momentum=True)
    host = [(g.G.view(np.int16), g.W, g.M) for g in w.groups]
    dev = [(torch.from_numpy(G).view(torch.bfloat16).cuda(), torch.from_numpy(W).cuda(), torch.from_numpy(M).cuda())
           for G, W, M in host]
    outs = [torch.empty(G.shape, dtype=torch.bfloat16, device="cuda") for G, _, _ in dev]
    rows = []
    for steps in (1, 3, 5, 8):
        for (G, W, M), (_, W0, M0) in zip(dev, host):
            W.copy_(torch.from_numpy(W0))
            M.copy_(torch.from_numpy(M0))
        groups = [mu.MuonGroup(W=W, M=M, G=G, O=O, lr=w.lr, beta=w.beta, nesterov=w.nesterov)
                  for (G, W, M), O in zip(dev, outs)]
        ws = mu.muon_step(groups, steps=steps)  # the first step from M = 0: its O is the one measured
        diag = [mu.muon_spectral_diag(O, iters=32, sigma_min=False) for O in outs]
        timed = [mu.MuonGroup(W=W, M=M, G=G, lr=w.lr, beta=w.beta, nesterov=w.nesterov) for G, W, M in dev]
        for _ in range(args.warmup):
            mu.muon_step(timed, steps=steps, workspace=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            mu.muon_step(timed, steps=steps, workspace=ws)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        row = {"ns_steps": steps, "steps_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
               "ns_iters_per_s": round(steps * 1e3 / ms, 1)}
        for g, d in zip(w.groups, diag):
            e = d["orth_err"].cpu().numpy()
            row[g.name] = {"orth_err_mean": round(float(e.mean()), 5), "orth_err_max": round(float(e.max()), 5),
                           "sigma_max": round(float(d["sigma_max"].max()), 5)}
        log(f"[bench] sweep {row}")
        rows.append(row)
    five = next(r for r in rows if r["ns_steps"] == 5)
    return {"metric": METRIC, "value": five["steps_per_s"], "unit": "steps/s", "ms_per_step": five["ms_per_step"],
            "dtype": "bf16",
            "config": {"workload": f"mamba2-130m-full-step steps sweep (M = 0): {args.count}x out_proj 768x1536 + "
                                   f"{args.count}x in_proj 3352x768, bf16 grads, 1/3/5/8 cubic NS steps; value at 5"},
            "sweep": rows}


def host_cores():
    """CPU cores this process may run on (the box's share, not the machine's)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return host_cores()


def _oracle_step_time(w, steps_ns, budget_s):
    """Mean oracle time per matrix of each group over a bounded sample
    (matrices taken alternately from each group until budget_s of CPU work,
    at least one per group)."""
    import oracle as orc
    times = {gi: [] for gi in range(len(w.groups))}
    t_start = time.perf_counter()
    i = 0
    while True:
        gi = i % len(w.groups)
        g = w.groups[gi]
        j = (i // len(w.groups)) % g.count
        G = orc.widen_bf16(g.G[j]) if g.grad_dtype == "bf16" else orc.widen_f32(g.G[j])
        t0 = time.perf_counter()
        orc.muon_step(orc.widen_f32(g.W[j]), orc.widen_f32(g.M[j]), G, beta=w.beta, lr=w.lr, nesterov=w.nesterov,
                      steps=steps_ns, eps=w.eps)
        times[gi].append(time.perf_counter() - t0)
        i += 1
        done = all(times.values()) and time.perf_counter() - t_start >= budget_s
        if done or i >= max(4 * sum(g.count for g in w.groups), 256):
            break
    t_step = sum(np.mean(times[gi]) * w.groups[gi].count for gi in times)
    return t_step, {gi: len(v) for gi, v in times.items()}


def cpu_baseline_step(w, steps_ns, budget_s=15.0, one_core=False):
    """The fp64 oracle as it stands on a bounded sample of the workload's
    matrices, scaled to one whole step, on every host core this process may
    use (BLAS threads); with one_core, also on one thread."""
    t_step, n = _oracle_step_time(w, steps_ns, budget_s)
    sample = " + ".join(f"{n[gi]} oracle runs over the {g.count} {g.name} matrices" for gi, g in enumerate(w.groups))
    out = {"value": round(1.0 / t_step, 5), "unit": "steps/s", "cores": int(blas_threads()), "kind": "oracle",
           "sample": f"{sample} (fp64 numpy, {steps_ns} NS steps), mean per-matrix time scaled to the whole step",
           "host_cores": host_cores()}
    if one_core:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(1):
                t1, n1 = _oracle_step_time(w, steps_ns, budget_s / 3)
            out["one_core"] = {"value": round(1.0 / t1, 5), "unit": "steps/s", "cores": 1,
                               "sample": " + ".join(f"{n1[gi]} oracle runs" for gi in n1)}
        except ImportError:
            pass
    return out


def cpu_baseline_injections(X, steps_ns, budget_s=15.0):
    """The oracle's batched NS on a contiguous slice of the injections (chunks
    of 512 matrices from the start until budget_s), extrapolated linearly to
    the whole batch: the matrices are independent."""
    import oracle as orc
    done, t = 0, 0.0
    while t < budget_s and done < X.shape[0]:
        chunk = X[done:done + 512].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        orc.ns_batched(chunk, steps_ns)
        t += time.perf_counter() - t0
        done += chunk.shape[0]
    how = "all" if done >= X.shape[0] else f"the first {done} of {X.shape[0]}, rate extrapolated to all"
    return {"value": round(done / t, 1), "unit": "matrices/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{how} matrices (fp64 numpy, {steps_ns} NS step, chunks of 512)", "host_cores": host_cores()}


def cpu_baseline_factored(V, K, steps_ns, budget_s=10.0):
    """The oracle's factored NS (dense fp64 NS of V K^T, then the core through
    pseudo-inverses) on the first injections until budget_s, as a rate per
    matrix; the matrices are independent."""
    import oracle as orc
    done, t = 0, 0.0
    while t < budget_s and done < V.shape[0]:
        n = min(256, V.shape[0] - done)
        Vc = V[done:done + n].float().cpu().numpy().astype(np.float64)
        Kc = K[done:done + n].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        for i in range(n):
            orc.factored_ns(Vc[i], Kc[i], steps_ns)
        t += time.perf_counter() - t0
        done += n
    how = f"all {done}" if done >= V.shape[0] else f"the first {done} of {V.shape[0]}"
    return {"value": round(done / t, 1), "unit": "matrices/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{how} injections (fp64 numpy: dense NS of V K^T, {steps_ns} step, core by pseudo-inverses), "
                      f"rate per matrix", "host_cores": host_cores()}


def cpu_baseline_adamw(P, G, M, V, kw, budget_s=15.0):
    """The oracle's AdamW step (fp64 numpy) over the tensors in turn until
    budget_s, its time scaled to the whole parameter set by element count."""
    import oracle as orc
    total = sum(p.size for p in P)
    done, t, k = 0, 0.0, 0
    while t < budget_s and k < len(P):
        g = orc.widen_bf16(G[k])
        t0 = time.perf_counter()
        orc.adamw_step(P[k], g, M[k], V[k], step=1, **kw)
        t += time.perf_counter() - t0
        done += P[k].size
        k += 1
    how = "all" if k == len(P) else f"the first {k} of {len(P)}"
    return {"value": round(done / (t * total), 4), "unit": "steps/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{how} tensors ({done} of {total} elements, fp64 numpy), time scaled by element count",
            "host_cores": host_cores()}


def cpu_baseline_diag(stacks, iters, budget_s=15.0):
    """The oracle's diagnostics (fp64: orthogonality error, Lanczos on the
    Gram) over the matrices, alternating the stacks, until budget_s, as a rate
    per matrix."""
    import oracle as orc
    done, t, i = 0, 0.0, 0
    nmax = max(A.shape[0] for _, A in stacks)
    while t < budget_s and i < nmax:
        for _, A in stacks:
            if i < A.shape[0] and t < budget_s:
                a = A[i].float().cpu().numpy().astype(np.float64)
                t0 = time.perf_counter()
                orc.spectral_diagnostics(a, iters)
                t += time.perf_counter() - t0
                done += 1
        i += 1
    total = sum(A.shape[0] for _, A in stacks)
    return {"value": round(done / t, 3), "unit": "matrices/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{done} of the {total} matrices, alternating the shapes (fp64 numpy, {iters} Lanczos steps)",
            "host_cores": host_cores()}


# ----------------------------------------------------------------------------
# exploration workloads
# ----------------------------------------------------------------------------
def traffic_key(args):
    """The workload name under which counter runs are stored: the injections
    carry their shape when it is not the default 64 x 128."""
    if args.workload == "injections" and tuple(args.inj_shape) != (64, 128):
        return f"injections_{args.inj_shape[0]}x{args.inj_shape[1]}"
    return args.workload


def small_bf16_kernel(m, n):
    """The on-chip kernel muon_ns_batched_small launches for a bf16 m x n
    stack (m <= n): one wave per matrix for s = 32 with l <= 256 and s = 64
    with l <= 128, else one workgroup per matrix, its rows split over the
    waves where X fits the 160 KB of LDS twice, its columns otherwise."""
    if (m == 32 and n <= 256) or (m == 64 and n <= 128):
        return f"ns_small_bf16_kernel<{m},{n}>"
    if 160 * 1024 // (m * n * 2) >= 2:
        return f"ns_small_bf16_wgr_kernel<{m}>"
    return f"ns_small_bf16_wg_kernel<{m}>"


def bench_injections(args, torch, mu, wl):
    m, n = args.inj_shape
    batch = args.batch if args.batch is not None else 393216 * 64 * 128 // (m * n)
    X = wl.injections(batch=batch, device="cuda", shape=(m, n))
    Y = torch.empty_like(X)
    for _ in range(args.warmup):
        mu.muon_ns_batched_small(X, Y, steps=args.ns_steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        mu.muon_ns_batched_small(X, Y, steps=args.ns_steps)
        b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    kms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = X.numel() * 2 * 2
    gram, comb = ns_flops(m, n)
    flops = batch * args.ns_steps * (gram + comb)
    gbs = nbytes / (kms * 1e-3) / 1e9
    tflops = flops / (kms * 1e-3) / 1e12
    kernel = small_bf16_kernel(m, n)
    default = (m, n) == (64, 128)
    wname = traffic_key(args)
    traffic = measured_traffic(kernel.split("<")[0], wname, ["ns_small.hip", "common.cuh"])
    # the bound whose peak the kernel's algorithmic work would take longer to reach
    if nbytes / PEAK_HBM_GBS >= flops / 1e3 / PEAK_BF16_TFLOPS:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    extra = {} if args.no_cpu else {"cpu_baseline": cpu_baseline_injections(X, args.ns_steps)}
    return {**extra, "metric": "MuonSSM batched single-step NS matrices/s" if default and args.ns_steps == 1
            else "batched on-chip NS matrices/s", "value": round(batch / (ms * 1e-3), 1),
            "unit": "matrices/s", "ms_per_step": round(ms, 4), "dtype": "bf16",
            "config": {"workload": f"injections {batch}x{m}x{n} bf16 (rank-8 V K^T), {args.ns_steps} NS step"
                       + ("" if args.ns_steps == 1 else "s")},
            "roofline": {**roof, "kernel": kernel, "traffic": traffic,
                         "algorithmic": {"bytes": nbytes, "flops": flops, "achieved_hbm_gbs": round(gbs, 1),
                                         "achieved_tflops": round(tflops, 1)}}}


def bench_injections_factored(args, torch, mu, wl):
    """The same injections given by their factors V [b, 64, 8], K [b, 128, 8]:
    muon_ns_factored writes the 8 x 8 float32 core of each (NS(V K^T) =
    V C K^T), or also the dense result with --dense."""
    batch = args.batch if args.batch is not None else 393216
    X, V, K = wl.injections(batch=batch, device="cuda", return_factors=True)
    del X
    C = torch.empty((batch, 8, 8), dtype=torch.float32, device="cuda")
    O = torch.empty((batch, 64, 128), dtype=torch.bfloat16, device="cuda") if args.dense else None
    for _ in range(args.warmup):
        mu.muon_ns_factored(V, K, C=C, O=O, steps=args.ns_steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        mu.muon_ns_factored(V, K, C=C, O=O, steps=args.ns_steps)
        b.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    per = (64 + 128) * 8 * 2 + 8 * 8 * 4 + (64 * 128 * 2 if args.dense else 0)
    gbs = batch * per / (kms * 1e-3) / 1e9
    extra = {} if args.no_cpu else {"cpu_baseline": cpu_baseline_factored(V, K, args.ns_steps)}
    return {**extra, "metric": "MuonSSM factored single-step NS matrices/s", "value": round(batch / (ms * 1e-3), 1),
            "unit": "matrices/s", "ms_per_step": round(ms, 4), "dtype": "bf16",
            "config": {"workload": f"injections {batch} x (V 64x8, K 128x8) bf16 factors, "
                                   f"{args.ns_steps} NS step, {'core + dense' if args.dense else '8x8 core'} out"},
            "roofline": {"bound": "hbm", "kernel": "ns_factored_kernel", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "bytes_per_matrix": per,
                         "traffic": measured_traffic(
                             "ns_factored_kernel", "injections_factored",
                             COUNTED_KERNELS["injections_factored"]["ns_factored_kernel"][1])}}


def cpu_baseline_ssm_momentum(V, K, a, M0, S0, beta, steps_ns, budget_s=15.0):
    """The oracle's momentum pathway (dense fp64 NS of every token, then the
    recurrence) over the sequences in order, 64 tokens at a time, until
    budget_s, as a token rate; every token costs the same, so the rate scales
    to the workload."""
    import oracle as orc
    done, t, seqs = 0, 0.0, 0
    for q in range(V.shape[0]):
        if t >= budget_s:
            break
        Vs = V[q].float().cpu().numpy().astype(np.float64)
        Ks = K[q].float().cpu().numpy().astype(np.float64)
        As = a[q].cpu().numpy().astype(np.float64)
        M = M0[q].cpu().numpy().astype(np.float64)
        S = S0[q].cpu().numpy().astype(np.float64)
        seqs += 1
        for t0_tok in range(0, Vs.shape[0], 64):
            if t >= budget_s:
                break
            c = slice(t0_tok, t0_tok + 64)
            t0 = time.perf_counter()
            M, S = orc.ssm_momentum(Vs[c], Ks[c], As[c], beta, M, S, steps=steps_ns)
            t += time.perf_counter() - t0
            done += Vs[c].shape[0]
    return {"value": round(done / t, 1), "unit": "injections/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{done} tokens from the first {seqs} of {V.shape[0]} sequences, in order (fp64 numpy: dense "
                      f"NS of each 64x128 injection, {steps_ns} step, then the state recurrence), rate per token",
            "host_cores": host_cores()}


def bench_ssm_momentum(args, torch, mu, wl):
    """MuonSSM's momentum pathway over the injection workload as sequences:
    192 sequences (batch 8 x 24 heads) x 2048 tokens of 64 x 128 rank-8
    injections; per token NS(V K^T) in factored form, M_t = beta M_{t-1} + U_t,
    S_t = a_t S_{t-1} + M_t."""
    V, K, a, M0, S0 = wl.ssm_sequences(device="cuda")
    nseq, T, m, r = V.shape
    n = K.shape[2]
    M, S = M0.clone(), S0.clone()
    beta = wl.SSM_BETA
    ws = mu.muon_ssm_momentum(V, K, M, S, a, beta=beta, steps=args.ns_steps)
    for _ in range(args.warmup):
        mu.muon_ssm_momentum(V, K, M, S, a, beta=beta, steps=args.ns_steps, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mu.muon_ssm_momentum(V, K, M, S, a, beta=beta, steps=args.ns_steps, workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-kernel durations from the events muon_ssm_momentum_timed records
    evs = []
    for _ in range(args.steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for e in row:
            e.record()
        evs.append(row)
    torch.cuda.synchronize()
    for k in range(args.steps):
        mu.muon_ssm_momentum(V, K, M, S, a, beta=beta, steps=args.ns_steps, workspace=ws,
                             events=[e.cuda_event for e in evs[k]])
    torch.cuda.synchronize()
    names = ["ssm_momentum_fused_kernel", "ssm_momentum_combine_kernel"]
    dur = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
           for i, nm in enumerate(names)}
    tokens = nseq * T
    chunks = -(-T // 256)
    fb = (m + n) * r * 2                      # the factors of one token
    part = nseq * chunks * (2 * 64 * 128 * 4 + 16)   # partial sums and map of every chunk
    alg = {"ssm_momentum_fused_kernel": tokens * (fb + 4) + part,
           "ssm_momentum_combine_kernel": nseq * 4 * m * n * 4 + part}
    dom = max(names, key=lambda nm: dur[nm])
    gbs = alg[dom] / (dur[dom] * 1e-3) / 1e9
    kernels = {nm: {"ms": round(dur[nm], 4), "alg_bytes": alg[nm],
                    "gbs": round(alg[nm] / (dur[nm] * 1e-3) / 1e9, 1)} for nm in names}
    extra = {} if args.no_cpu else {"cpu_baseline": cpu_baseline_ssm_momentum(V, K, a, M0, S0, beta, args.ns_steps)}
    return {**extra, "metric": "MuonSSM momentum pathway injections/s", "value": round(tokens / (ms * 1e-3), 1),
            "unit": "injections/s", "ms_per_step": round(ms, 4), "dtype": "bf16",
            "config": {"workload": f"ssm_momentum {nseq} sequences x {T} tokens of {m}x{n} rank-{r} bf16 injections,"
                                   f" {args.ns_steps} NS step, beta {beta}, fp32 M and S"},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(dom, "ssm_momentum", COUNTED_KERNELS["ssm_momentum"][dom][1])},
            "kernels": kernels}


def bench_adamw(args, torch, mu, wl):
    """AdamW over the Mamba-2-130M parameters outside the Muon groups (170
    tensors, 38.9 M elements, bf16 gradients)."""
    shapes = wl.mamba2_adamw_shapes()
    P, G, M, V = wl.adamw_state(shapes)
    Pd = [torch.from_numpy(p).cuda() for p in P]
    Gd = [torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).cuda() for g in G]
    Md = [torch.from_numpy(m).cuda() for m in M]
    Vd = [torch.from_numpy(v).cuda() for v in V]
    kw = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    opt = mu.AdamwTensors(Pd, Gd, Md, Vd)  # argument arrays marshalled once
    for t in range(args.warmup):
        opt.step(step=t + 1, **kw)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k, (a, b) in enumerate(ev):
        a.record()
        opt.step(step=args.warmup + k + 1, **kw)
        b.record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nel = sum(p.numel() for p in Pd)
    gbs = nel * 26 / (kms * 1e-3) / 1e9
    extra = {} if args.no_cpu else {"cpu_baseline": cpu_baseline_adamw(P, G, M, V, kw)}
    return {**extra, "metric": "AdamW companion steps/s (Mamba-2-130M non-Muon parameters)", "value": round(1e3 / ms, 2),
            "unit": "steps/s", "ms_per_step": round(ms, 4), "dtype": "f32",
            "config": {"workload": f"adamw: {len(Pd)} tensors, {nel} elements, bf16 grads"},
            "roofline": {"bound": "hbm", "kernel": "adamw_kernel", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_element": 26,
                         "traffic": None}}


def bench_diag(args, torch, mu, wl):
    """Spectral diagnostics of the Mamba-2-130M projection matrices, one
    muon_spectral_diag call per shape (24 out_proj 768 x 1536 and 24 in_proj
    3352 x 768): by default the float32 weights (W = 0.02 N(0, 1), as in the
    full step: the largest singular value checked every few steps), with
    --diag-input updates their bf16 Muon updates (5 NS steps of bf16 N(0, 1)
    gradients: the orthogonality error of the update).  Per-pass durations
    from HIP events recorded by muon_spectral_diag_timed.  With 24 matrices
    per call the Lanczos pass runs as the split kernel (six co-resident
    workgroups per matrix); its algorithmic bytes count the whole of H per
    step, although the kernel reads only the upper block triangle."""
    stacks = []
    for name, a in wl.projection_stacks(args.count):
        if args.diag_input == "weights":
            A = torch.from_numpy(0.02 * a).cuda()
        else:
            G = torch.from_numpy(a).cuda().to(torch.bfloat16)
            A = torch.empty_like(G)
            mu.muon_ns_orthogonalize(G, A, steps=5)
            del G
        stacks.append((name, A))
    it = args.iters
    wss = [torch.empty(mu.lib().muon_spectral_diag_workspace_size(A.shape[1], A.shape[2], A.shape[0],
                                                                   mu.binding._dtype_code(A), it),
                       dtype=torch.uint8, device="cuda") for _, A in stacks]
    for _ in range(args.warmup):
        for (_, A), ws in zip(stacks, wss):
            mu.muon_spectral_diag(A, iters=it, workspace=ws)

    def events(k):
        out = []
        for _ in range(k):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            out.append(e)
        return out
    evs = [[events(4) for _ in stacks] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for (_, A), ws, ev in zip(stacks, wss, evs[k]):
            mu.muon_spectral_diag(A, iters=it, workspace=ws, events=[e.cuda_event for e in ev])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # algorithmic work per launch: pack reads A and writes the operand rows
    # (three bf16 pieces per float32 element);
    # the Gram's six (float32 input) or one (bf16) bf16 products of
    # s (s + 1) l flops (upper triangle); Lanczos reads H once per step
    kern = {"diag_pack_kernel": [0.0, 0.0], "symprod_bf16_kernel<F32>": [0.0, 0.0], "diag_lanczos_split_kernel": [0.0, 0.0]}
    for si, (name, A) in enumerate(stacks):
        cnt, m, n = A.shape
        s_, l_ = min(m, n), max(m, n)
        f32 = A.dtype == torch.float32
        pieces = 6 if f32 else 1  # products summed by the Gram
        stored = 3 if f32 else 1  # bf16 pieces the pack writes per element
        s_pad, kdim = -(-s_ // 128) * 128, -(-l_ // 64) * 64
        work = [cnt * (m * n * A.element_size() + s_pad * stored * kdim * 2),
                cnt * pieces * s_ * (s_ + 1) * l_,
                cnt * (min(it, s_) + 1) * s_ * s_ * 4]
        for p, key in enumerate(kern):
            t = float(np.mean([evs[k][si][p].elapsed_time(evs[k][si][p + 1]) for k in range(args.steps)]))
            kern[key][0] += t
            kern[key][1] += work[p]
    kernels = {}
    for key, (t, work) in kern.items():
        if key.startswith("symprod"):
            kernels[key] = {"ms": round(t, 4), "tflops": round(work / (t * 1e-3) / 1e12, 1),
                            "frac": round(work / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma"}
        else:
            kernels[key] = {"ms": round(t, 4), "gbs": round(work / (t * 1e-3) / 1e9, 1),
                            "frac": round(work / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bound": "hbm"}
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    if kd["bound"] == "mfma":
        roofline = {"bound": "mfma", "kernel": dom, "achieved": kd["tflops"], "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": kd["frac"], "traffic": None}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": kd["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": kd["frac"], "traffic": None}
    nmat = sum(A.shape[0] for _, A in stacks)
    extra = {} if args.no_cpu else {"cpu_baseline": cpu_baseline_diag(stacks, it)}
    return {**extra, "metric": "Spectral diagnostics matrices/s (orthogonality error + Lanczos sigma_max/sigma_min)",
            "value": round(nmat / (ms * 1e-3), 1), "unit": "matrices/s", "ms_per_step": round(ms, 4),
            "dtype": "f32" if args.diag_input == "weights" else "bf16",
            "config": {"workload": f"diag: {args.diag_input} of {args.count} out_proj 768x1536 + {args.count} "
                                   f"in_proj 3352x768, {it} Lanczos steps"},
            "roofline": roofline, "kernels": kernels}


ELEMENTWISE = ["elementwise.hip", "common.cuh"]
GEMM = ["gemm_bf16.hip", "common.cuh"]
FACTORED_MOM = ["ssm_momentum.hip", "factored_core.cuh", "common.cuh"]
COUNTED_KERNELS = {
    "full_step": {"combine_bf16_kernel": ("combine_bf16_kernel", GEMM),
                  "symprod_bf16_kernel": ("symprod_bf16_kernel", GEMM),
                  "gram": ("gram:symprod_bf16_kernel", GEMM),
                  "momentum_wide_kernel": ("momentum_wide_kernel", ELEMENTWISE),
                  "momentum_tall_kernel": ("momentum_tall_kernel", ELEMENTWISE),
                  "apply_wide_kernel": ("apply_wide_kernel", ELEMENTWISE),
                  "apply_tall_kernel": ("apply_tall_kernel", ELEMENTWISE)},
    "injections": {"ns_small_bf16_kernel": ("ns_small_bf16_kernel", ["ns_small.hip", "common.cuh"]),
                   "ns_small_bf16_wg_kernel": ("ns_small_bf16_wg_kernel", ["ns_small.hip", "common.cuh"]),
                   "ns_small_bf16_wgr_kernel": ("ns_small_bf16_wgr_kernel", ["ns_small.hip", "common.cuh"])},
    "ssm_momentum": {"ssm_momentum_fused_kernel": ("ssm_momentum_fused_kernel", FACTORED_MOM),
                     "ssm_momentum_combine_kernel": ("ssm_momentum_combine_kernel", FACTORED_MOM)},
    "injections_factored": {"ns_factored_kernel": ("ns_factored_kernel",
                                                   ["ns_factored.hip", "factored_core.cuh", "common.cuh"])},
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_step",
                    choices=["full_step", "out_proj", "in_proj", "injections", "injections_factored", "ssm_momentum",
                             "adamw",
                             "diag", "single", "sweep"])
    ap.add_argument("--ns-steps", type=int, default=None)
    ap.add_argument("--count", type=int, default=24, help="matrices per group (full_step)")
    ap.add_argument("--batch", type=int, default=None,
                    help="injections batch (default 393216 64 x 128 matrices, or the same bytes at --inj-shape)")
    ap.add_argument("--inj-shape", type=lambda v: tuple(int(x) for x in v.split("x")), default=(64, 128),
                    help="injections: m x n of the stacked matrices (m <= n), e.g. 128x256")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--dense", action="store_true", help="injections_factored: also write the dense result")
    ap.add_argument("--cap", action="store_true", help="full_step: spectral cap on (power step per update)")
    ap.add_argument("--diag-input", default="weights", choices=["weights", "updates"],
                    help="diag: float32 weights or bf16 Muon updates")
    ap.add_argument("--iters", type=int, default=32, help="diag: Lanczos steps")
    ap.add_argument("--one-stream", action="store_true",
                    help="full_step: every step on one stream (the launch configuration of the per-kernel "
                         "timing; used for the counter runs)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "iterate", "accumulate"],
                    help="full_step: Newton-Schulz schedule of the large groups")
    ap.add_argument("--separate-apply", action="store_true",
                    help="full_step: apply the update in its own pass instead of the final product's epilogue")
    ap.add_argument("--graph", action="store_true",
                    help="full_step: also time the step captured in a HIP graph and replayed (reported beside value)")
    ap.add_argument("--per-matrix", action="store_true",
                    help="full_step: one muon_step call per matrix instead of one grouped call")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB plain copy first (reference for profiler byte counters)")
    ap.add_argument("--ingest", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store HBM bytes per launch from two rocprofv3 counter runs of --workload")
    args = ap.parse_args()
    if args.ingest:
        ingest_counters(*args.ingest, traffic_key(args), COUNTED_KERNELS[args.workload])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the Muon step here has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.ns_steps is None:
        args.ns_steps = 1 if args.workload.startswith("injections") or args.workload == "ssm_momentum" else 5
    import torch
    import spectral_optimizer_ssm_amd as mu
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mu.lib()
    if args.copy_calibration:
        copy_calibration(torch)
    if args.workload in ("full_step", "out_proj", "in_proj", "single"):
        res = bench_full_step(args, torch, mu, wl)
    elif args.workload == "injections":
        res = bench_injections(args, torch, mu, wl)
    elif args.workload == "injections_factored":
        res = bench_injections_factored(args, torch, mu, wl)
    elif args.workload == "ssm_momentum":
        res = bench_ssm_momentum(args, torch, mu, wl)
    elif args.workload == "adamw":
        res = bench_adamw(args, torch, mu, wl)
    elif args.workload == "diag":
        res = bench_diag(args, torch, mu, wl)
    elif args.workload == "sweep":
        res = bench_sweep(args, torch, mu, wl)
    out = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": res.pop("dtype"),
           "data": "synthetic", "config": res.pop("config")}
    out.update(res)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
