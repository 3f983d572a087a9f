"""Benchmark of one Muon step (momentum -> batched Newton-Schulz -> decoupled
weight decay) on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2]

Prints ONE JSON line.  A step is one muon_step call over the whole parameter
set of the workload, with inputs (weights, gradients, momenta) resident in
HBM before timing starts; gradient sets are drawn beforehand and cycled.
`value` is the algorithmic NS throughput in TFLOP/s (3*m^2*n + m^3 flops per
matrix per NS iteration, m <= n).  `roofline` reports the dominant kernel
against its bound, and `cpu_baseline` the fp64 CPU oracle on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector


# HBM traffic per launch of a workload's dominant kernel (the one its
# roofline object names), from two rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE; KiB per dispatch, mean over the profiled dispatches of that
# kernel), each scaled by the ratio of known bytes to the same counter on a
# plain device copy (`bench.py --copy-probe`: 262144 KiB copied, FETCH_SIZE
# 131085 KiB, WRITE_SIZE 262144 KiB).  Valid only for the kernel source it
# was taken on (SHA-256); otherwise `traffic` is reported as null.
TRAFFIC = {
    "c2": {"source": "k_skinny.hip",
           "kernel_source_sha256": "cefd602ce9e54d7d2fd93a486544604e79077dc96bbe74c5fb159af64c6d75cd",
           "fetch_kib_per_dispatch": 83655.9, "write_kib_per_dispatch": 108731.0,
           "fetch_scale": 2.0, "write_scale": 1.0},
    "c5": {"source": "k_large.hip",
           "kernel_source_sha256": "e2aa5de95b016795d9304740bd8376cddffdd0471b56e19b9f34bfb3023351bc",
           "fetch_kib_per_dispatch": 13371509.1, "write_kib_per_dispatch": 1644963.9,
           "fetch_scale": 2.0, "write_scale": 1.0},
}


def _kernel_sha(name: str) -> str:
    import hashlib
    path = os.path.join(ROOT, "newton_schulz_05_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes(key: str):
    t = TRAFFIC.get(key)
    if t is None or t["kernel_source_sha256"] is None or t["kernel_source_sha256"] != _kernel_sha(t["source"]):
        return None
    return 1024.0 * (t["fetch_kib_per_dispatch"] * t["fetch_scale"] + t["write_kib_per_dispatch"] * t["write_scale"])


def copy_probe(nbytes: int, steps: int) -> int:
    """A plain device copy of known size, the calibration run for the HBM
    byte counters: each launch reads and writes `nbytes`."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": steps}), flush=True)
    return 0


def _events_time(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def bench_shard_update(steps, warmup):
    """One rank's update of its 1/8 flat shard of each of two [8192, 28672]
    bf16 matrices from their full fp32 O (the step after NS in the gathered
    design): 8 B per shard element (W read and write 2 + 2, O read 4)."""
    import torch
    from newton_schulz_05_amd import shard_update
    shape, ranks = (8192, 28672), 8
    n = shape[0] * shape[1]
    ws = [torch.randn(n // ranks, device="cuda").to(torch.bfloat16) for _ in range(2)]
    os_ = [torch.randn(shape, device="cuda") * 0.01 for _ in range(2)]
    st = torch.cuda.current_stream()

    def fn():
        for w, o in zip(ws, os_):
            shard_update(w, o, 3 * (n // ranks), lr=0.02, wd=0.1, stream=st)
    ms = _events_time(fn, steps, warmup, st)
    byt = 2 * (n // ranks) * 8.0
    gbs = byt / (ms * 1e-3) / 1e9
    return {"metric": "shard update GB/s (rank 3 of 8, 2 x [8192, 28672] bf16, O fp32)", "value": round(gbs, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "shard_update_rank3_of8_2x8192x28672", "elements": 2 * (n // ranks)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "shard_update_kernel",
                         "launches_per_step": 2}}


def bench_adamw(steps, warmup, elems):
    """AdamW on the 1-D parameters: by default the 65 RMSNorm gains [4096] of
    the 32-layer transformer set (launch-bound); with --adamw-elems N, 64
    tensors of N/64 elements.  22 B per element (p 2 + 2, g 2, m 4 + 4,
    v 4 + 4, bf16 params)."""
    import torch
    from newton_schulz_05_amd import AdamWGroup
    sizes = [4096] * 65 if not elems else [elems // 64] * 64
    ps = [torch.randn(n, device="cuda").to(torch.bfloat16) for n in sizes]
    gs = [(torch.randn(n, device="cuda") * 1e-3).to(torch.bfloat16) for n in sizes]
    ms = [torch.zeros(n, device="cuda") for n in sizes]
    vs = [torch.zeros(n, device="cuda") for n in sizes]
    st = torch.cuda.current_stream()
    t = [0]

    group = AdamWGroup(ps, gs, ms, vs)

    def fn():
        t[0] += 1
        group.step(lr=1e-3, betas=(0.9, 0.95), eps=1e-8, wd=0.1, step=t[0], stream=st)
    ms_ = _events_time(fn, steps, warmup, st)
    tot = sum(sizes)
    gbs = tot * 22.0 / (ms_ * 1e-3) / 1e9
    name = "adamw_1d_gains_32_layers_65x4096" if not elems else f"adamw_1d_64x{elems // 64}"
    return {"metric": "AdamW step on 1-D params (ms, GB/s)", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms_, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": name, "tensors": len(sizes), "elements": tot},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "adamw_kernel",
                         "launches_per_step": (len(sizes) + 31) // 32}}


def time_groups(wl, steps, warmup, dev):
    """Each shape group of a multi-group workload timed alone (its own plan
    over the parameters of that group), with the fraction of its own bound:
    HBM for skinny bf16 groups (m <= 32), bf16 MFMA otherwise."""
    import torch
    from newton_schulz_05_amd import MuonPlan
    from newton_schulz_05_amd import workloads as WL
    keys = []
    for s in wl.shapes:
        k = (min(s[-2:]), max(s[-2:]))
        if k not in keys:
            keys.append(k)
    out = []
    for k in keys:
        idx = [i for i, s in enumerate(wl.shapes) if (min(s[-2:]), max(s[-2:])) == k]
        sub = type(wl)(wl.key, wl.number, wl.name, tuple(wl.shapes[i] for i in idx), wl.dtype, wl.g_std)
        plan = MuonPlan(sub.shapes, sub.dtype)
        ws = plan.new_workspace(dev)
        ps = [WL.make_params(wl, dev, dev)[i] for i in idx]
        ms_ = [torch.zeros(tuple(wl.shapes[i]), dtype=torch.float32, device=dev) for i in idx]
        gs = [[WL.make_grads(wl, t, dev, dev)[i] for i in idx] for t in range(2)]
        bound = [plan.bind(ps, g, ms_, workspace=ws) for g in gs]
        st = torch.cuda.current_stream()
        hyper = wl.hyper()
        step = [0]

        def fn():
            bound[step[0] % 2].step(**hyper, stream=st)
            step[0] += 1
        ms = _events_time(fn, steps, warmup, st)
        skinny = k[0] <= 32 and wl.dtype == torch.bfloat16
        if skinny:
            gbs = alg_bytes(sub) / (ms * 1e-3) / 1e9
            frac = {"bound": "hbm", "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            tf = alg_flops(sub) / (ms * 1e-3) / 1e12
            frac = {"bound": "mfma", "achieved": round(tf, 1), "unit": "TFLOP/s",
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        out.append({"group": f"{sub.n_matrices()} x [{k[0]}, {k[1]}]", "ms_per_step": round(ms, 5), **frac})
        del plan, ws, ps, ms_, gs, bound
        torch.cuda.empty_cache()
    return out


def bench_ns(wl, steps, warmup):
    """muon_ns alone (NS of every matrix, O in fp32) on the workload's
    gradients, for the NS-only comparison with the pages' figures."""
    import torch
    from newton_schulz_05_amd import MuonPlan
    from newton_schulz_05_amd import workloads as WL
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace("cuda")
    ins = WL.make_grads(wl, 0, "cuda", "cuda")
    outs = [torch.empty(tuple(s), dtype=torch.float32, device="cuda") for s in wl.shapes]
    st = torch.cuda.current_stream()

    bound = plan.bind_ns(ins, outs, workspace=ws)

    def fn():
        bound.ns(coeffs=wl.coeffs, ns_steps=wl.ns_steps, stream=st)
    ms = _events_time(fn, steps, warmup, st)
    tf = alg_flops(wl) / (ms * 1e-3) / 1e12
    context = {"c2": "74 x [24, 10240] NS, fused [74, 24, 10240] batch on the pages' Ascend NPU: 2.4 ms"}
    return {"metric": "muon_ns ms per call (NS only)", "value": round(ms, 5), "unit": "ms", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
            "data": "synthetic", "config": {"workload": wl.name, "matrices": wl.n_matrices(),
                                            "alg_tflop_per_call": alg_flops(wl) / 1e12},
            "tflops_alg": round(tf, 3), "context": context.get(wl.key)}


def alg_flops(wl) -> float:
    """3 m^2 n + m^3 per matrix per NS iteration (Gram exploits symmetry)."""
    tot = 0.0
    for s in wl.shapes:
        b = s[0] if len(s) == 3 else 1
        r, c = s[-2], s[-1]
        m, n = min(r, c), max(r, c)
        tot += b * (3.0 * m * m * n + float(m) ** 3)
    return tot * wl.ns_steps


def executed_flops(wl) -> float:
    """MFMA flops the bf16 path executes for one muon_step (symmetric outputs
    on their upper tiles only; true m and n, padding not counted).  Mirrors
    the library's schedule: all NS steps in one group when m < 512, else the
    first min(4, N - 1), then pairs, then a single step; per group one Gram
    m^2 n, per step A^2 (one product m^3 in steps k < min(3, N - 2) when
    m >= 1536, k < min(2, N - 2) when 512 <= m < 1536, else three), after
    the group's first step the products
    T = P A, A' = P T and R = P R (m^3 each), and one apply 2 m^2 n.  The
    lo planes add products: the first Gram takes three (precise recipe,
    m < 4096 or more than 5 steps), the chain products three each (precise;
    R one when m >= 1024 and N <= 5), and an apply one more per lo plane it
    uses (X_0's in the first group, R's in the precise recipe)."""
    N = wl.ns_steps
    tot = 0.0
    for s in wl.shapes:
        b = s[0] if len(s) == 3 else 1
        r, c = s[-2], s[-1]
        m, n = float(min(r, c)), float(max(r, c))
        if m <= 32:
            tot += b * (3.0 * m * m * n + m ** 3) * N
            continue
        whole, precise = m < 512, (m < 4096 or N > 5)
        plain = 3 if m >= 1536 else 2
        a2 = lambda k: (1 if (m >= 512 and k < min(plain, N - 2)) else 3) * m ** 3  # noqa: E731
        chain = 3 if precise else 1
        rprod = 1 if (not precise or (m >= 1024 and N <= 5)) else 3
        f, k = 0.0, 0
        while k < N:
            if whole:
                G = N - k
            elif k == 0:
                G = N if N <= 2 else min(4, N - 1)
            else:
                G = 2 if N - k >= 2 else 1
            gram = (3 if (k == 0 and precise) else 1) * m * m * n
            apply = (1 + (1 if k == 0 else 0) + (1 if precise else 0)) * 2 * m * m * n
            f += gram + sum(a2(k + j) for j in range(G)) + (2 * chain + rprod) * (G - 1) * m ** 3 + apply
            k += G
        tot += b * f
    return tot


def alg_bytes(wl) -> float:
    """Compulsory HBM bytes of a step: read G, M, W; write M, W."""
    import torch
    pes = 2 if wl.dtype == torch.bfloat16 else 4
    return wl.n_elements() * (pes + 4 + 4 + pes + pes)


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle on host cores over a bounded sample of the workload."""
    import numpy as np
    import torch

    from oracle import muon_ref as ref
    from newton_schulz_05_amd import workloads as WL

    a, b, c = wl.coeffs
    hp = ref.MuonHyper(lr=wl.lr, mu=wl.mu, nesterov=wl.nesterov, wd=wl.wd, a=a, b=b, c=c,
                       ns_steps=wl.ns_steps, scale=wl.scale)
    params = WL.make_params(wl, "cpu")
    grads = WL.make_grads(wl, 0, "cpu")
    w = [p.double().numpy() for p in params]
    g = [x.double().numpy() for x in grads]
    mo = [np.zeros(x.shape) for x in w]
    # sample: whole parameters in order until the time budget is spent
    flops_done, t0, n_params = 0.0, time.perf_counter(), 0
    i = 0
    while time.perf_counter() - t0 < budget_s:
        k = i % len(w)
        ref.muon_step([w[k]], [g[k]], [mo[k]], hp)
        sub = type(wl)(wl.key, wl.number, wl.name, (wl.shapes[k],), wl.dtype, wl.g_std)
        flops_done += alg_flops(sub)
        i += 1
        n_params += 1
    el = time.perf_counter() - t0
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([x.get("num_threads", 1) for x in info] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": flops_done / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_params} parameter-steps of {wl.name} (fp64 NumPy, {el:.1f} s)"}


def _skinny_only(plan, wl):
    import torch
    return all(g["m"] <= 32 for g in plan.groups()) and wl.dtype == torch.bfloat16


def bench_step(wl, steps, warmup, dev="cuda", per_group=True, n_sets=None):
    """Time `steps` muon_step calls over the whole parameter set of `wl`
    (inputs resident in HBM, gradient sets drawn beforehand and cycled),
    then the same number again with the apply launches timed by HIP events
    on the launch stream.  Returns the measurements as a dict."""
    import torch

    from newton_schulz_05_amd import MuonPlan
    from newton_schulz_05_amd import binding as B
    from newton_schulz_05_amd import workloads as WL

    big = wl.n_elements() > 500_000_000
    plan = MuonPlan(wl.shapes, wl.dtype)
    ws = plan.new_workspace(dev)
    params = WL.make_params(wl, dev, dev)
    moms = WL.make_moms(wl, dev)
    n_sets = n_sets or (2 if big else 4)
    gsets = [WL.make_grads(wl, s, dev, dev) for s in range(n_sets)]
    torch.cuda.synchronize()
    hyper = wl.hyper()
    stream = torch.cuda.current_stream()
    # tensors are validated once; each timed step is one C call
    bound = [plan.bind(params, g, moms, workspace=ws) for g in gsets]
    for s in range(warmup):
        bound[s % n_sets].step(**hyper, stream=stream)
    torch.cuda.synchronize()
    # HIP events on the stream the kernels are launched on, around the K
    # back-to-back steps (a per-step event would add a marker between kernels)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for s in range(steps):
        bound[s % n_sets].step(**hyper, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    # a skinny-path wait that timed out would have left W partly unwritten
    timed_out = plan.workspace_timed_out(ws, stream) or B.poll_timeout()
    out = {"ms": ms, "wall_s": wall, "timed_out": timed_out, "plan": plan.groups()}
    if not _skinny_only(plan, wl) and wl.dtype == torch.bfloat16:
        # the same steps again with every apply bracketed by events
        B.kernel_timing(True)
        B.kernel_timing_read()
        for s in range(steps):
            bound[s % n_sets].step(**hyper, stream=stream)
        torch.cuda.synchronize()
        kt = B.kernel_timing_read()
        B.kernel_timing(False)
        out["apply"] = kt
        timed_out = timed_out or plan.workspace_timed_out(ws, stream) or B.poll_timeout()
        out["timed_out"] = timed_out
    del bound, gsets, params, moms, ws
    torch.cuda.empty_cache()
    if per_group and len(out["plan"]) > 1:
        out["groups"] = time_groups(wl, steps, warmup, dev)
    return out


def _roofline(wl, res):
    """The dominant kernel against its bound.  Skinny sets: the single
    persistent kernel per chunk (the whole step), HBM-bound, on the 14 B per
    element compulsory bytes.  MFMA sets: the apply launches, bf16 MFMA on
    their algorithmic flops (2 m^2 n per matrix per apply) over their
    event-timed duration; executed flops (lo-plane products) beside them."""
    import torch
    ms = res["ms"]
    if all(g["m"] <= 32 for g in res["plan"]) and wl.dtype == torch.bfloat16:
        gbs = alg_bytes(wl) / (ms * 1e-3) / 1e9
        tr = traffic_bytes(wl.key)
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None if tr is None else round(tr),
                "kernel": "skinny_kernel", "launches_per_step": sum(g["n_chunks"] for g in res["plan"])}
    if wl.dtype != torch.bfloat16:
        tf = alg_flops(wl) / (ms * 1e-3) / 1e12
        return {"bound": "alu", "achieved": round(tf, 3), "peak": F32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / F32_VALU_PEAK_TFLOPS, 6), "traffic": None, "kernel": "whole step"}
    # the apply's MFMA work: one m x m by m x n product per pair of operand
    # planes it multiplies (X_0's lo plane in the first group, R's in the
    # precise recipe), true m and n (padding not counted), over the
    # event-timed duration of the applies
    kt = res["apply"]
    ex = kt["exec_flops"] / (kt["ms"] * 1e-3) / 1e12
    plain = kt["alg_flops"] / (kt["ms"] * 1e-3) / 1e12
    steps = max(1, res.get("steps", 1))
    n = max(1, kt["launches"])
    tr = traffic_bytes(wl.key)
    return {"bound": "mfma", "achieved": round(ex, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ex / BF16_PEAK_TFLOPS, 4), "traffic": None if tr is None else round(tr),
            "kernel": "gemm_bf16_kernel<*, *, EpiApplyBf16> (apply X' = R X)",
            "launches_per_step": round(kt["launches"] / steps, 2),
            "avg_launch_ms": round(kt["ms"] / n, 4),
            "tflop_per_launch": round(kt["exec_flops"] / n / 1e12, 4),
            "single_product_tflop_per_launch": round(kt["alg_flops"] / n / 1e12, 4),
            "single_product_tflops": round(plain, 1),
            "share_of_step": round(kt["ms"] / steps / res["ms"], 3)}


def _summary(wl, res):
    """ms, throughput and fraction of the bound of a whole step."""
    import torch
    ms = res["ms"]
    tf = alg_flops(wl) / (ms * 1e-3) / 1e12
    d = {"workload": wl.name, "ms_per_step": round(ms, 5), "alg_tflops": round(tf, 3)}
    if all(g["m"] <= 32 for g in res["plan"]) and wl.dtype == torch.bfloat16:
        gbs = alg_bytes(wl) / (ms * 1e-3) / 1e9
        d.update(bound="hbm", gbs_compulsory=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        ex = executed_flops(wl) / (ms * 1e-3) / 1e12
        d.update(bound="mfma", frac=round(tf / BF16_PEAK_TFLOPS, 4), executed_tflops=round(ex, 1),
                 executed_frac=round(ex / BF16_PEAK_TFLOPS, 4))
    return d


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads' whole-step figures reported beside the headline")
    ap.add_argument("--op", default="step", choices=["step", "ns", "shard_update", "adamw"],
                    help="step: the Muon step (default); ns: muon_ns alone on the workload; "
                         "shard_update / adamw: the companion kernels")
    ap.add_argument("--adamw-elems", type=int, default=0,
                    help="adamw: total elements of a 64-tensor stress set instead of the model's gains")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run a plain device copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no "
              "multi-GPU path: every GPU would run its own shard's step independently)", file=sys.stderr)
        return 2

    if args.copy_probe:
        return copy_probe(args.copy_probe, args.steps or 5)
    if args.op == "ns":
        from newton_schulz_05_amd import workloads as WL
        wl = WL.WORKLOADS[args.config]
        big = args.config in ("c4", "c5")
        print(json.dumps(bench_ns(wl, args.steps or (5 if big else 100), args.warmup or (1 if big else 10))),
              flush=True)
        return 0
    if args.op == "shard_update":
        print(json.dumps(bench_shard_update(args.steps or 50, args.warmup or 5)), flush=True)
        return 0
    if args.op == "adamw":
        print(json.dumps(bench_adamw(args.steps or 100, args.warmup or 10, args.adamw_elems)), flush=True)
        return 0

    import torch

    from newton_schulz_05_amd import workloads as WL

    wl = WL.WORKLOADS[args.config]
    big = args.config in ("c4", "c5")
    steps = args.steps if args.steps is not None else (10 if big else 100)
    warmup = args.warmup if args.warmup is not None else (2 if big else 10)
    res = bench_step(wl, steps, warmup)
    res["steps"] = steps
    if res["timed_out"]:
        print("a skinny-path wait timed out during the timed steps: the results are invalid", file=sys.stderr)
        return 3
    ms = res["ms"]
    flops = alg_flops(wl)
    byt = alg_bytes(wl)
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "Muon step ms & TFLOP/s (% bf16 MFMA peak / % HBM BW) for batched NS on [B,M,N]",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_wall": round(res["wall_s"] * 1e3 / steps, 5),
        "wall_s": round(res["wall_s"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": wl.n_matrices(), "elements": wl.n_elements(),
                   "ns_steps": wl.ns_steps, "alg_tflop_per_step": flops / 1e12,
                   "executed_tflop_per_step": round(executed_flops(wl) / 1e12, 3),
                   "compulsory_gb_per_step": byt / 1e9, "parallelism": "single_gpu"},
        "roofline": _roofline(wl, res),
        "step": _summary(wl, res),
    }
    if res.get("groups"):
        out["groups"] = res["groups"]
    if not args.no_extra:
        # the other large and the skinny workload, whole-step figures only
        extra = {}
        for key in ("c5", "c2"):
            if key == args.config:
                continue
            w2 = WL.WORKLOADS[key]
            b2 = key in ("c4", "c5")
            r2 = bench_step(w2, 10 if b2 else 100, 2 if b2 else 10, per_group=False)
            if r2["timed_out"]:
                print(f"a skinny-path wait timed out in {key}: the results are invalid", file=sys.stderr)
                return 3
            r2["steps"] = 10 if b2 else 100
            extra[key] = {**_summary(w2, r2), "roofline": _roofline(w2, r2)}
        out["others"] = extra
    if not args.no_cpu_baseline:
        if big:
            # one matrix of each shape group, one step each, extrapolated
            keys = []
            for sh in wl.shapes:
                k = (min(sh[-2:]), max(sh[-2:]))
                if k not in [x[0] for x in keys]:
                    keys.append((k, sh))
            sample = WL.custom([sh for _, sh in keys], dtype=wl.dtype, g_std=wl.g_std, number=wl.number)
            out["cpu_baseline"] = cpu_baseline(sample, args.cpu_seconds)
            out["cpu_baseline"]["sample"] += " (one matrix per shape group; the rate extrapolates to the set)"
        else:
            out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
