#!/usr/bin/env python3
"""Benchmark of the FlashAttention backward on one MI355X.

One step = one fa_bwd_run over one batch of the workload, with every input
already resident in HBM.  The plan takes the stored-dS path: the sfmg
preprocess (rowsum(dY * Y)), the dK/dV kernel (S/P recompute, dP, dS, dV, dK
over key tiles; it also stores dS), the dQ GEMM over the stored dS, whose
launch also adds the fp32 dK/dV partial sums when the plan splits a key tile
(its last workgroups).  (Past 4 GiB of dS
the dK/dV and dQ launches repeat per chunk of KV heads; only where one KV
head's dS alone would not fit does it take the recompute path: the dQ kernel
recomputes S/P/dP/dS over query tiles and forms sfmg, then the dK/dV kernel
and the reduce.)  attn_out and softmax_lse come from the library's own GPU
forward (fa_fwd_run), made once before timing.  The default workload is the
GQA causal one (B=1, N1=32, N2=8, S=4096, D=Dv=128, BSND).

Prints one JSON line: whole-step throughput in TFLOP/s under the standard
FLOP count (2*(3D+2Dv) per visible (query, key) pair per query head; causal
with S1 = S2 counted as exactly half of S1*S2); the roofline entry of the
dominant kernel, the dK/dV kernel (the four products S, dP, dV, dK it forms:
2*(2D+2Dv) FLOP per visible pair per query head), timed by HIP events the
library records around it inside the timed region, with the dK/dV + dQ pair
beside it; the standalone sfmg preprocess kernel's HBM bandwidth
(its own timed launches); the fp64 CPU oracle timed on a bounded sample of the same
workload; and `accuracy`: the library's gradients on that sample (made from
the oracle forward's stored Y and lse) against the oracle's, every element,
so that the speed figure comes with its parity error.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--settle 0.5] [--workload gqa_causal]
                    [--dtype bf16|fp16] [--no-cpu-baseline] [--no-configs] [--copy-calibration]

Before the warmup steps, untimed steps run for --settle seconds: the shader
clock ramps up over the first tens of milliseconds of load and drops again
while the host builds inputs, so a short warmup alone times a cold clock.

The line also carries `configs`: the same step, pair and preprocess figures
for every benchmark configuration (10 timed steps each).
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FA-bwd TFLOP/s and % of MI355X bf16 MFMA peak (S=4096, D=128, GQA, causal)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
# The main part of a step is the dK/dV kernel and the dQ kernel; the library
# records HIP events around that pair on the launch stream.  Which dQ kernel
# runs is the plan's choice (fa_bwd_plan_dq_path).
MAIN_KERNELS = {"stored_ds": "dkdv_kernel+dq_ds_kernel", "recompute": "dkdv_kernel+dq_kernel",
                "fused": "fused_kernel"}
DQ_KERNEL = {"stored_ds": "dq_ds_kernel", "recompute": "dq_kernel"}
DQ_MODES = {
    "stored_ds": "dK/dV kernel stores dS (bf16 tiles in the workspace), dQ = scale*dS*K by a GEMM kernel "
                 "(no atomics, deterministic)",
    "recompute": "separate dQ pass recomputing S and dP (no atomics, deterministic)",
    "fused": "one launch per (sequence, KV head): sfmg, dK/dV and dQ in one kernel (no workspace, deterministic)",
}
SFMG_NOTE = {
    "stored_ds": "standalone fa_bwd_sfmg entry point; the default step launches the same kernel first",
    "recompute": "standalone fa_bwd_sfmg entry point; the step forms sfmg inside dq_kernel",
}
PROFILE_DIR = os.path.join(ROOT, "profiles")


def visible_pairs(cfg):
    """Visible (query, key) pairs per query head, summed over sequences.
    Causal with equal lengths and no left bound counts S*S/2 (the usual
    'halved' convention); every other mask counts exactly."""
    if cfg["layout"] == "TND":
        lens_q = list(cfg["lengths"])
        lens_k = list(cfg.get("lengths_kv", cfg["lengths"]))
    else:
        lens_q, lens_k = [cfg["S1"]] * cfg["B"], [cfg["S2"]] * cfg["B"]
    mode, wl, wr = cfg["mask_mode"], cfg["win_left"], cfg["win_right"]
    if mode == 0:
        wl, wr = -1, -1
    elif mode == 1:
        wr = 0
    total = 0
    for s1, s2 in zip(lens_q, lens_k):
        if mode == 1 and wl < 0 and s1 == s2:
            total += s1 * s2 / 2
            continue
        off = s2 - s1
        for i in range(s1):
            lo = 0 if wl < 0 else max(0, i + off - wl)
            hi = s2 - 1 if wr < 0 else min(s2 - 1, i + off + wr)
            if hi >= lo:
                total += hi - lo + 1
    return total


def algorithmic_flops(cfg):
    return 2.0 * (3 * cfg["D"] + 2 * cfg["Dv"]) * cfg["N1"] * visible_pairs(cfg)


def dkdv_flops(cfg):
    """The dK/dV kernel's share: S = QK^T, dP = dY V^T, dV += P^T dY and
    dK += dS^T Q, 2*(2D + 2Dv) FLOP per visible pair per query head."""
    return 2.0 * (2 * cfg["D"] + 2 * cfg["Dv"]) * cfg["N1"] * visible_pairs(cfg)


def committed_traffic(workload, path=None, sources="det", key="hbm_bytes_per_launch"):
    """HBM bytes per launch (key: the pair's total, or
    hbm_bytes_per_launch.<kernel> for one kernel) from the committed rocprofv3
    --pmc summary, if it was taken from the current kernel source; else None."""
    from flashattention_backward_fa_amd.profile_summary import SOURCES, kernel_code_hash

    path = path or os.path.join(PROFILE_DIR, f"bwd_dkdv_dq_kernels_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_code_sha256_16") != kernel_code_hash(SOURCES[sources]):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, max_heads, name="", dtype="bf16"):
    """The fp64 oracle's backward, untuned, on the first KV-head groups of
    the workload (its forward is run first, untimed, to make Y and lse).
    Returns the baseline entry and the sample (inputs, oracle Y/lse and the
    oracle's gradients) for the accuracy leg."""
    import numpy as np
    import oracle
    from flashattention_backward_fa_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    G = cfg["N1"] // cfg["N2"]
    groups = max(1, min(cfg["N2"], max_heads // G))
    sub = dict(cfg, N1=groups * G, N2=groups)
    import torch

    x = W.make_inputs(cfg, dtype=torch.float16 if dtype == "fp16" else torch.bfloat16)
    lay = cfg["layout"]
    # head slice of the full workload's tensors (the head axis is 2 in BSND,
    # 1 in BNSD and TND)
    if lay == "BSND":
        sl = lambda t, n: t[:, :, :n].contiguous()  # noqa: E731
    else:
        sl = lambda t, n: t[:, :n].contiguous()  # noqa: E731
    tq, tk, tv, tdy = sl(x["q"], sub["N1"]), sl(x["k"], sub["N2"]), sl(x["v"], sub["N2"]), sl(x["dout"], sub["N1"])
    q, k, v, dy = (t.double().numpy() for t in (tq, tk, tv, tdy))
    args = (lay, x["cu_q"], x["cu_kv"], cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    Y, lse = oracle.forward(q, k, v, *args)
    Yst, lst = oracle.store(Y, lse, dtype)
    t0 = time.perf_counter()
    ref = oracle.backward(q, k, v, dy, Yst, lst, *args)
    dt = time.perf_counter() - t0
    flops = algorithmic_flops(sub)
    entry = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"{sub['N1']} of {cfg['N1']} query heads ({groups} KV-head group(s)) of the {name} workload, "
                   f"full sequence; oracle backward (dense fp64 NumPy, masked work not skipped) took {dt:.2f} s; "
                   f"value = algorithmic FLOP of the sample / time"),
    }
    sample = dict(cfg=sub, x=x, t=(tq, tk, tv, tdy), Yst=Yst, lst=lst, ref=ref)
    return entry, sample


def _errors(got, ref):
    """Relative Frobenius error and max |err| / max |ref| of one tensor."""
    import numpy as np

    err = got - ref
    nref = float(np.linalg.norm(ref))
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    rel = float(np.linalg.norm(err)) / nref if nref > 0 else (0.0 if not np.any(err) else math.inf)
    mx = float(np.abs(err).max()) / mref if mref > 0 else (0.0 if not np.any(err) else math.inf)
    return rel, mx


def accuracy(sample, name):
    """Parity error beside the speed figure: the library's backward (same
    entry point and plan as the timed step) on the CPU-baseline sample's
    inputs, with the oracle forward's stored Y and lse as attn_out and
    softmax_lse, compared element by element with the oracle's dq, dk, dv."""
    import numpy as np
    import torch
    from flashattention_backward_fa_amd import fa_bwd as fb

    cfg, x = sample["cfg"], sample["x"]
    dev = torch.device("cuda", 0)
    q, k, v, dout = (t.to(dev) for t in sample["t"])
    attn_out = torch.from_numpy(np.ascontiguousarray(sample["Yst"])).to(q.dtype).to(dev)
    lse = torch.from_numpy(np.ascontiguousarray(sample["lst"], dtype=np.float32)).to(dev)
    cu_q = cu_kv = None
    mq = mk = -1
    if cfg["layout"] == "TND":
        cu_q = torch.from_numpy(x["cu_q"]).to(dev)
        cu_kv = torch.from_numpy(x["cu_kv"]).to(dev)
        mq, mk = int(np.diff(x["cu_q"]).max()), int(np.diff(x["cu_kv"]).max())
    dq, dk, dv = fb.flash_attn_grad(q, k, v, dout, attn_out, lse, cu_q, cu_kv, softmax_scale=cfg["softmax_scale"],
                                    mask_mode=cfg["mask_mode"], win_left=cfg["win_left"],
                                    win_right=cfg["win_right"], max_seqlen_q=mq, max_seqlen_kv=mk,
                                    layout=cfg["layout"])
    torch.cuda.synchronize()
    # the parity tests' bounds: bf16, and 2^3 tighter for fp16 (3 more significant bits)
    tol_rel, tol_max = (1.25e-3, 2.5e-3) if q.dtype == torch.float16 else (1e-2, 2e-2)
    out = {"reference": "fp64 oracle (oracle.backward) on the CPU-baseline sample, every element",
           "tolerance": {"rel_fro": tol_rel, "max_abs_ratio": tol_max}}
    ok = True
    for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), sample["ref"]):
        rel, mx = _errors(got.cpu().double().numpy(), ref)
        out[nm] = {"rel_fro": float(f"{rel:.4g}"), "max_abs_ratio": float(f"{mx:.4g}")}
        ok = ok and rel <= tol_rel and mx <= tol_max
    out["within_tolerance"] = bool(ok)
    out["sample"] = f"{cfg['N1']} query heads of the {name} workload"
    return out


def roofline_entry(name, cfg, m):
    """Roofline of the dominant kernel (the dK/dV kernel; the fused kernel when
    the plan takes that mode): its algorithmic FLOP per launch over its own
    average duration from the library's HIP events in the timed region, with
    the dK/dV + dQ pair (all five products) and the dQ kernel beside it."""
    flops = algorithmic_flops(cfg)
    pair_ms = m["pair_ms"]
    pair = {
        "kernels": MAIN_KERNELS.get(m["dq_path"], m["dq_path"]),
        "achieved": round(flops / (pair_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "frac": round(flops / (pair_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flop_per_launch": flops, "flop_rule": "2*(3D+2Dv) per visible pair per query head",
        "avg_launch_ms": round(pair_ms, 5), "traffic": committed_traffic(name),
    }
    if m["dkdv_ms"] is None:  # one main kernel (fused) or a chunked run: the pair is all there is
        traffic = pair["traffic"]
        if m["dq_path"] == "fused":
            traffic = committed_traffic(name, os.path.join(PROFILE_DIR, f"bwd_fused_kernel_{name}_traffic.txt"),
                                        "fused")
        return {"bound": "mfma", "kernel": pair["kernels"], "achieved": pair["achieved"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": pair["frac"], "traffic": traffic,
                "avg_launch_ms": round(pair_ms, 5), "launches_timed": m["pair_launches"],
                "algorithmic_flop_per_launch": flops, "flop_rule": pair["flop_rule"]}
    kf = dkdv_flops(cfg)
    ach = kf / (m["dkdv_ms"] * 1e-3) / 1e12
    dq = DQ_KERNEL[m["dq_path"]]
    return {
        "bound": "mfma", "kernel": "dkdv_kernel", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
        "traffic": committed_traffic(name, key="hbm_bytes_per_launch.dkdv_kernel"),
        "avg_launch_ms": round(m["dkdv_ms"], 5), "launches_timed": m["pair_launches"],
        "algorithmic_flop_per_launch": kf,
        "flop_rule": "2*(2D+2Dv) per visible pair per query head (S, dP, dV, dK)",
        "pair": pair,
        "dq_kernel": {"kernel": dq, "avg_launch_ms": round(m["dq_ms"], 5),
                      "traffic": committed_traffic(name, key=f"hbm_bytes_per_launch.{dq}")},
    }


def copy_calibration():
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings to bytes."""
    import torch

    n = 256 << 20  # 256 MiB
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def graph_step_ms(step, outs, stream, n, replays=5):
    """Whole steps replayed from a HIP graph of n steps: the device time per
    step once the host's per-launch cost is out of the way (what a caller that
    captures its backward sees; short workloads are bound by that cost in an
    eager loop).  Every replay's outputs must equal the eager step's bit for
    bit (all the default paths are deterministic), else the figure is None."""
    import torch

    try:
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                step()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            for t in outs:
                t.fill_(float("nan"))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outs, ref)):
                return None
            times.append(e0.elapsed_time(e1) / n)
        del g
        return min(times)
    except RuntimeError as e:  # capture refused: report no figure
        print(f"graph timing skipped: {e}", file=sys.stderr, flush=True)
        return None


def measure(name, steps, warmup, settle_s=0.0, dtype="bf16"):
    """Time `steps` backward steps of a workload on the current stream, after
    untimed steps for at least `settle_s` seconds (the shader clock ramps up
    over the first tens of milliseconds of load, and drops again while the host
    builds the next workload's inputs) and then `warmup` untimed ones:
    whole-step time from events around the loop; then `steps` more steps with
    the library's events around and between the dK/dV and dQ kernels (kept
    out of the first loop so that they add nothing to the step time); then
    the preprocess kernel over its own launches.
    Returns times in ms, the preprocess bytes and the settle step count."""
    import torch
    from flashattention_backward_fa_amd import fa_bwd as fb
    from flashattention_backward_fa_amd import workloads as W

    cfg = W.CONFIGS[name]
    dev = torch.device("cuda", 0)
    x = W.make_inputs(cfg, dtype=torch.float16 if dtype == "fp16" else torch.bfloat16)
    q, k, v, dout = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    cu_q = cu_kv = None
    mq = mk = -1
    if cfg["layout"] == "TND":
        cu_q = torch.from_numpy(x["cu_q"]).to(dev)
        cu_kv = torch.from_numpy(x["cu_kv"]).to(dev)
        mq = mk = int(max(cfg["lengths"]))
    kw = dict(softmax_scale=cfg["softmax_scale"], mask_mode=cfg["mask_mode"], win_left=cfg["win_left"],
              win_right=cfg["win_right"], max_seqlen_q=mq, max_seqlen_kv=mk, layout=cfg["layout"])
    attn_out, lse = fb.flash_attn(q, k, v, cu_q, cu_kv, **kw)
    plan = fb.get_plan(q, k, v, cfg["layout"], cu_q, cu_kv, kw["softmax_scale"], kw["mask_mode"], kw["win_left"],
                       kw["win_right"], mq, mk)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # the backward bound once (validation and marshalling out of the loop);
    # each step enqueues the library's run
    step = fb.prepare_grad(q, k, v, dout, attn_out, lse, cu_q, cu_kv, workspace=ws, out=(dq, dk, dv), **kw)

    settle_steps = 0
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
        settle_steps += 8
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole steps, with no event inside them
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / max(steps, 1)
    graph_ms = graph_step_ms(step, (dq, dk, dv), stream, max(steps, 10))
    # the same steps again with the library's events around the two main
    # kernels and between them
    plan.profile_enable(max(steps, 1))
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    split = plan.profile_read_split(steps)
    plan.profile_enable(0)
    n = max(len(split), 1)
    main_avg = sum(a + b for a, b in split) / n
    first, second = sum(a for a, _ in split) / n, sum(b for _, b in split) / n
    path = plan.dq_path()
    dkdv_ms = dq_ms = None
    if path == "stored_ds" and all(b > 0 for _, b in split):
        dkdv_ms, dq_ms = first, second
    elif path == "recompute":
        dq_ms, dkdv_ms = first, second

    # preprocess alone (sfmg = rowsum(dY * Y)): HBM-bound, timed over its own
    # launches on the same stream; algorithmic bytes = dY and Y read once
    # (2 B each per element) plus 4 B of sfmg written per query row
    rows = cfg["N1"] * (int(sum(cfg["lengths"])) if cfg["layout"] == "TND" else cfg["B"] * cfg["S1"])
    pre_bytes = rows * (2 * 2 * cfg["Dv"] + 4)
    sf = torch.empty(rows, dtype=torch.float32, device=dev)
    sargs = (fb._ptr(dout), fb._ptr(attn_out), fb._ptr(cu_q), fb._ptr(sf), ctypes.c_void_p(stream.cuda_stream))
    pre_iters = max(steps, 1)
    for _ in range(2):
        plan.sfmg(*sargs)
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record(stream)
    for _ in range(pre_iters):
        plan.sfmg(*sargs)
    p1.record(stream)
    torch.cuda.synchronize()
    pre_ms = p0.elapsed_time(p1) / pre_iters
    return dict(ms_per_step=ms_per_step, graph_ms=graph_ms, pair_ms=main_avg, pair_launches=len(split), dkdv_ms=dkdv_ms, dq_ms=dq_ms,
                pre_ms=pre_ms, pre_bytes=pre_bytes, settle_steps=settle_steps, dq_path=path)


FLOYD_WORKLOAD = "floyd"


def floyd_stage_units(cfg):
    """FLOP and HBM bytes of each backward stage of the Floyd attention path on
    a workload with no mask: T = heads*N*M*K (n, m, k) triples, R = heads*N*M
    rows.  Each product costs 2*D FLOP per triple.  The bytes are the path's
    own, not algorithmic: every operand of the stage read once and every result
    written once in this library's decomposition, which keeps fp32 scores and
    dP, 16-bit P and dS, and one fp32 dQ partial in HBM between stages."""
    hd = cfg["B"] * cfg["H"]
    N, M, K, D = cfg["N"], cfg["M"], cfg["K"], cfg["D"]
    T, R = hd * N * M * K, hd * N * M
    qsz, k1sz, k2sz = 2 * R * D, 2 * hd * N * K * D, 2 * hd * K * M * D   # bytes of one 16-bit tensor
    return {
        "rowstats": (0, 2 * qsz + R * 16),
        "scores_by_n": (4 * D * T, 2 * qsz + 2 * k1sz + 8 * T),
        "scores_by_m_softmax_grad": (4 * D * T, 2 * qsz + 2 * k2sz + 8 * T + 4 * T + 8 * R),
        "dv1": (2 * D * T, 2 * T + qsz + k1sz),
        "dk1": (2 * D * T, 2 * T + qsz + k1sz),
        "dv2": (2 * D * T, 2 * T + qsz + k2sz),
        "dk2": (2 * D * T, 2 * T + qsz + k2sz),
        "dq_k1": (2 * D * T, 2 * T + k1sz + 2 * qsz),
        "dq_k2": (2 * D * T, 2 * T + k2sz + 2 * qsz + qsz),
    }


def floyd_algorithmic_units(cfg):
    """Algorithmic FLOP and HBM bytes of the whole Floyd backward: ten products
    of 2*D FLOP per (n, m, k) triple; every input read once (query, key1,
    value1, key2, value2, dy, attention_in, and the two fp32 row statistics
    of 8 entries per row) and every gradient written once (dq, dk1, dv1, dk2,
    dv2).  Nothing the path keeps between its stages counts."""
    hd = cfg["B"] * cfg["H"]
    N, M, K, D = cfg["N"], cfg["M"], cfg["K"], cfg["D"]
    R = hd * N * M
    qsz, k1sz, k2sz = 2 * R * D, 2 * hd * N * K * D, 2 * hd * K * M * D
    inputs = 3 * qsz + 2 * k1sz + 2 * k2sz + 2 * R * 8 * 4
    outputs = qsz + 2 * k1sz + 2 * k2sz
    return 20.0 * D * hd * N * M * K, inputs + outputs


def floyd_leg(steps, warmup, settle_s, with_accuracy):
    """Floyd attention backward on its benchmark workload: whole-step time from
    events on the launch stream, per-stage times from the library's timing
    hook, each stage against its bound, and (optionally) the gradients of one
    head against the fp64 oracle."""
    import torch
    from flashattention_backward_fa_amd import floyd as fl
    from flashattention_backward_fa_amd import workloads as W

    cfg = W.FLOYD_CONFIGS[FLOYD_WORKLOAD]
    dev = torch.device("cuda", 0)
    x = W.floyd_inputs(cfg)
    names = ("query", "key1", "value1", "key2", "value2")
    t = [x[n].to(dev) for n in names]
    dy = x["dy"].to(dev)
    y, smax, ssum = fl.floyd_attn(*t)   # the step's inputs come from the library's forward
    desc, *_ = fl._prepare(*t, None)
    ws = torch.empty(fl.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = tuple(torch.empty_like(a) for a in (t[0], t[1], t[2], t[3], t[4]))
    stream = torch.cuda.current_stream(dev)

    def step(stage_ms=None):
        fl.floyd_attn_grad(*t, dy, None, smax, ssum, y, workspace=ws, out=out, stage_ms=stage_ms)

    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 1)
    stage_sum = [0.0] * len(fl.STAGES)
    reps = 5
    for _ in range(reps):
        st = []
        step(st)
        stage_sum = [a + b for a, b in zip(stage_sum, st)]
    stage_ms = [v / reps for v in stage_sum]

    N, M, K, D = cfg["N"], cfg["M"], cfg["K"], cfg["D"]
    flops = 20.0 * D * cfg["B"] * cfg["H"] * N * M * K
    units = floyd_stage_units(cfg)
    stages = {}
    for name, sms in zip(fl.STAGES, stage_ms):
        f, b = units[name]
        t_hbm, t_mfma = b / (PEAK_HBM_GBS * 1e9), f / (PEAK_BF16_TFLOPS * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        gbs, tfs = b / (sms * 1e-3) / 1e9, f / (sms * 1e-3) / 1e12
        stages[name] = {
            "ms": round(sms, 4), "bound": bound, "path_bytes": b, "flop": f,
            "gb_s": round(gbs, 1), "tflop_s": round(tfs, 1),
            "path_frac": round(gbs / PEAK_HBM_GBS if bound == "hbm" else tfs / PEAK_BF16_TFLOPS, 4),
        }
    dom = max(stages, key=lambda k: stages[k]["ms"])
    # the backward as a whole against its algorithmic bound
    a_flop, a_bytes = floyd_algorithmic_units(cfg)
    t_hbm, t_mfma = a_bytes / (PEAK_HBM_GBS * 1e9), a_flop / (PEAK_BF16_TFLOPS * 1e12)
    a_bound = "hbm" if t_hbm >= t_mfma else "mfma"
    leg = {
        "workload": FLOYD_WORKLOAD,
        "config": {k: cfg[k] for k in ("B", "H", "N", "M", "K", "D")} | {"mask": None, "dtype": "bf16"},
        "ms_per_step": round(ms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
        "pct_of_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "flop_rule": "20*D per (n, m, k) triple: ten products of 2*D each",
        "stages": stages,
        "stage_bytes_note": "path_bytes count the path's own fp32 scores / dP and 16-bit P / dS kept in HBM "
                            "between stages; they are not algorithmic bytes",
        "dominant_stage": dom,
        "roofline": {
            "kernel": "whole backward (all stages)", "bound": a_bound,
            "achieved": round(a_bytes / (ms * 1e-3) / 1e9, 1) if a_bound == "hbm" else round(a_flop / (ms * 1e-3) / 1e12, 1),
            "peak": PEAK_HBM_GBS if a_bound == "hbm" else PEAK_BF16_TFLOPS,
            "unit": "GB/s" if a_bound == "hbm" else "TFLOP/s",
            "frac": round(max(t_hbm, t_mfma) / (ms * 1e-3), 4),
            "algorithmic_bytes": a_bytes, "algorithmic_flop": a_flop,
            "units_rule": "inputs (7 tensors and the 2 row statistics) read once, 5 gradients written once; "
                          "20*D FLOP per (n, m, k) triple",
            "traffic": committed_traffic(FLOYD_WORKLOAD, os.path.join(PROFILE_DIR, f"floyd_bwd_kernels_{FLOYD_WORKLOAD}_traffic.txt"),
                                         "floyd"),
        },
        "accuracy": None,
    }
    if with_accuracy:
        leg["accuracy"] = floyd_accuracy(cfg, x)
    return leg


def floyd_accuracy(cfg, x):
    """One head of the Floyd workload through the library with the oracle
    forward's Y (rounded to bf16) and statistics (rounded to fp32), against the
    oracle backward, every element."""
    import numpy as np
    import torch
    import oracle
    import oracle.floyd as OF
    from flashattention_backward_fa_amd import floyd as fl

    names = ("query", "key1", "value1", "key2", "value2", "dy")
    one = {n: x[n][:1, :1].contiguous() for n in names}
    f = {n: one[n].double().numpy() for n in names}
    scale = OF.default_scale(cfg["D"])
    Y, mx, sm = OF.forward(f["query"], f["key1"], f["value1"], f["key2"], f["value2"], scale, None)
    Yst = oracle.bf16_round(Y)
    mx32, sm32 = mx.astype(np.float32), sm.astype(np.float32)
    ref = OF.backward(f["query"], f["key1"], f["value1"], f["key2"], f["value2"], f["dy"], Yst,
                      mx32.astype(np.float64), sm32.astype(np.float64), scale, None)
    dev = torch.device("cuda", 0)
    g = fl.floyd_attn_grad(*(one[n].to(dev) for n in names), None, torch.from_numpy(mx32).to(dev),
                           torch.from_numpy(sm32).to(dev), torch.from_numpy(Yst).to(torch.bfloat16).to(dev))
    torch.cuda.synchronize()
    res = {"reference": "fp64 oracle (oracle.floyd.backward), head 0 of the workload, every element",
           "tolerance": {"rel_fro": 0.01, "max_abs_ratio": 0.02}}
    ok = True
    for name, got, r in zip(("dq", "dk1", "dv1", "dk2", "dv2"), g, ref):
        rel, mxr = _errors(got.double().cpu().numpy(), r)
        res[name] = {"rel_fro": round(rel, 6), "max_abs_ratio": round(mxr, 6)}
        ok = ok and rel <= 0.01 and mxr <= 0.02
    res["within_tolerance"] = ok
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps (clock ramp-up)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default="bf16",
                    help="element type of q, k, v, dout, attn_out and the gradients")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (cpu_baseline and accuracy)")
    ap.add_argument("--cpu-heads", type=int, default=32, help="query heads in the CPU-baseline sample")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration summary")
    ap.add_argument("--no-floyd", action="store_true", help="skip the Floyd attention backward leg")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the kernel shards over "
              "KV-head groups with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    from flashattention_backward_fa_amd import workloads as W

    name = args.workload or W.BENCH_WORKLOAD
    cfg = W.CONFIGS[name]
    m = measure(name, args.steps, args.warmup, args.settle, args.dtype)
    ms_per_step, pre_ms, pre_bytes = m["ms_per_step"], m["pre_ms"], m["pre_bytes"]
    pre_gbs = pre_bytes / (pre_ms * 1e-3) / 1e9

    flops = algorithmic_flops(cfg)
    value = flops / (ms_per_step * 1e-3) / 1e12
    roofline = roofline_entry(name, cfg, m)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "graph_ms_per_step": None if m["graph_ms"] is None else round(m["graph_ms"], 4),
        "settle": {"seconds": args.settle, "untimed_steps": m["settle_steps"],
                   "why": "untimed steps before the warmup so that the timed steps run at the steady-state clock"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": name, "layout": cfg["layout"], "B": cfg.get("B", len(cfg.get("lengths", [])) or None),
            "N1": cfg["N1"], "N2": cfg["N2"], "S1": cfg.get("S1"), "S2": cfg.get("S2"), "D": cfg["D"],
            "Dv": cfg["Dv"], "mask_mode": cfg["mask_mode"], "win_left": cfg["win_left"],
            "win_right": cfg["win_right"], "global_batch": cfg.get("B", len(cfg.get("lengths", []))),
            "seq_len": cfg.get("S1", int(sum(cfg.get("lengths", [0])))), "parallelism": "single-gpu",
            "algorithmic_gflop": round(flops / 1e9, 3), "dq_mode": DQ_MODES.get(m["dq_path"], m["dq_path"]),
        },
        "roofline": roofline,
        "preprocess": {
            "bound": "hbm", "kernel": "preprocess_kernel (sfmg)", "achieved": round(pre_gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(pre_gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": pre_bytes, "avg_launch_ms": round(pre_ms, 5),
            "note": SFMG_NOTE.get(m["dq_path"], "standalone fa_bwd_sfmg entry point"),
        },
        "configs": None,
        "floyd": None,
        "cpu_baseline": None,
        "accuracy": None,
    }
    if not args.no_configs:
        # every benchmark configuration at the same settings (10 timed steps
        # each): whole step, the dK/dV + dQ pair and the preprocess bandwidth
        import torch

        rows = {}
        for other in W.CONFIGS:
            if other == name:
                r = m
            else:
                torch.cuda.empty_cache()
                r = measure(other, 10, 2, args.settle, args.dtype)
            f = algorithmic_flops(W.CONFIGS[other])
            rows[other] = {
                "ms_per_step": round(r["ms_per_step"], 4),
                "graph_ms_per_step": None if r["graph_ms"] is None else round(r["graph_ms"], 4),
                "tflops": round(f / (r["ms_per_step"] * 1e-3) / 1e12, 1),
                "pct_of_peak": round(100 * f / (r["ms_per_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "pair_ms": round(r["pair_ms"], 4),
                "pair_tflops": round(f / (r["pair_ms"] * 1e-3) / 1e12, 1),
                "dkdv_ms": None if r["dkdv_ms"] is None else round(r["dkdv_ms"], 4),
                "dkdv_frac": None if r["dkdv_ms"] is None else
                round(dkdv_flops(W.CONFIGS[other]) / (r["dkdv_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "preprocess_gbs": round(r["pre_bytes"] / (r["pre_ms"] * 1e-3) / 1e9, 1),
                "algorithmic_gflop": round(f / 1e9, 3),
                "dq_path": r["dq_path"],
            }
        line["configs"] = rows
    if not args.no_floyd:
        import torch

        torch.cuda.empty_cache()
        line["floyd"] = floyd_leg(10, 2, args.settle, not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        line["cpu_baseline"], sample = cpu_baseline(cfg, args.cpu_heads, name, args.dtype)
        line["accuracy"] = accuracy(sample, name)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
