#!/usr/bin/env python3
"""Throughput of the jagged flash attention hot path on one MI355X.

One step = one forward (plan + attention kernel) and one backward (delta pre-pass,
plan, backward kernel, dQ finalize) over the whole synthetic batch, with inputs,
outputs and workspaces resident in HBM before the timed region starts.  The
value is useful TFLOP/s over forward + backward: per head and sequence
4 Lq n D (forward) and 10 Lq n D (backward); n^2 instead of Lq n in self mode,
halved under causal masking.

The printed JSON line also carries the roofline of the dominant kernel (its
algorithmic bytes or FLOPs per launch over its HIP-event-measured average launch
duration) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

METRIC = "useful TFLOP/s fwd & bwd, jagged broadcast-Q attn bf16; % of MFMA peak"
KERNEL_SOURCES = ["fwd.hip", "bwd.hip", "plan.hip", "sparse.hip", "mxfp8.hip", "jfa_device.h", "jfa_internal.h"]
PROFILES = os.path.join(ROOT, "profiles")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def useful_flops(w, lengths):
    n = np.asarray(lengths, dtype=np.float64)
    if w.broadcast_q:
        fwd = 4.0 * w.q_len * n.sum() * w.head_dim * w.heads
    else:
        fwd = 4.0 * (n * n).sum() * w.head_dim * w.heads
        if w.causal:
            fwd *= 0.5
    return fwd, 2.5 * fwd


def algorithmic_bytes(w, lengths):
    """Bytes each kernel must move at least once (bf16 tensors, fp32 LSE / delta)."""
    t = float(np.sum(lengths))
    hd = w.heads * w.head_dim
    rows = len(lengths) * w.q_len if w.broadcast_q else t
    q_rows = w.q_len if w.broadcast_q else t
    q = q_rows * hd * 2
    kv = t * hd * 2
    o = rows * hd * 2
    lse = rows * w.heads * 4
    return {
        "fwd": q + 2 * kv + o + lse,                          # Q, K, V in; O, LSE out
        "bwd": q + 2 * kv + o + 2 * lse + 2 * kv + q,         # Q, K, V, dO, LSE, delta in; dK, dV, dQ out
        "bwd_pre": 2 * o + lse,                               # O, dO in; delta out
        "dq_finalize": q,                                     # dQ out (bf16)
    }


def kernel_source_hash() -> str:
    """sha256 over the kernel sources; ties stored counter readings to the sources they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "variable_length_flash_jfa_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources.

    profiles/traffic_<kernel>_<workload>.json holds FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch) and the factors that map them to bytes, measured with a plain
    copy of known size (bench.py --copy-probe)."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return (rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"])


def host_info():
    """The host the oracle runs on: logical CPUs, CPU model, BLAS library and threads."""
    info = {"os_cpu_count": os.cpu_count(), "cpu_model": None, "blas": None, "blas_threads": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            info["blas"] = f"{pools[0].get('internal_api')} {pools[0].get('version')}"
            info["blas_threads"] = max(int(p.get("num_threads", 1)) for p in pools)
    except Exception:  # pragma: no cover
        pass
    return info


def cpu_baseline(case, w, budget_s: float):
    """The fp64 oracle on a bounded sample of sequences of the same workload, forward
    and backward timed apart (the useful-FLOP formula of the GPU figures; the oracle
    does the full n x n work even when causal)."""
    import oracle
    host = host_info()
    off = case["offsets"].cpu().numpy().astype(np.int64)
    lengths = np.diff(off)
    rng = np.random.default_rng(1)
    order = rng.permutation(len(lengths))
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    q_host = f64(case["q"].cpu()) if w.broadcast_q else None
    fwd_flops = bwd_flops = 0.0
    t_fwd = t_bwd = 0.0
    used = 0
    for b in order:
        a, e = int(off[b]), int(off[b + 1])
        r0, r1 = (b * w.q_len, (b + 1) * w.q_len) if w.broadcast_q else (a, e)
        for h in range(w.heads):
            qb = q_host[:, h] if w.broadcast_q else f64(case["q"][a:e, h].cpu())
            kb, vb = f64(case["k"][a:e, h].cpu()), f64(case["v"][a:e, h].cpu())
            gb = f64(case["g"][r0:r1, h].cpu())
            t0 = time.perf_counter()
            oracle.sequence_forward(qb, kb, vb, case["scale"], w.causal)
            t1 = time.perf_counter()
            oracle.sequence_backward(qb, kb, vb, gb, case["scale"], w.causal)
            t2 = time.perf_counter()
            t_fwd += t1 - t0
            t_bwd += t2 - t1
        f, bwd = useful_flops(w, [e - a])
        fwd_flops += f
        bwd_flops += bwd
        used += 1
        if t_fwd + t_bwd >= budget_s:
            break
    dt = t_fwd + t_bwd
    cores = host["blas_threads"] or host["os_cpu_count"] or 1
    return {
        "value": float((fwd_flops + bwd_flops) / dt / 1e12),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{used} of {len(lengths)} sequences (random, seed 1) x {w.heads} heads of "
                  f"{w.name}, fp64 numpy forward+backward, {dt:.1f} s",
        "fwd_tflops": float(fwd_flops / max(t_fwd, 1e-12) / 1e12),
        "bwd_tflops": float(bwd_flops / max(t_bwd, 1e-12) / 1e12),
        "fwd_s": round(t_fwd, 3),
        "bwd_s": round(t_bwd, 3),
        "host": host,
    }


def sparse_comparison(args, jfa, w, case, o, lse, ws_f):
    """Dense forward vs the block-sparse forward (scoring, selection and attention)
    for several top-k values; also the fraction of 64-key blocks the selection keeps."""
    if w.causal:
        print("the block-sparse forward is defined for non-causal workloads", file=sys.stderr)
        sys.exit(2)
    q, k, v, off = case["q"], case["k"], case["v"], case["offsets"]
    bq, scale = w.broadcast_q, case["scale"]
    lengths = case["lengths"]
    nkv = (lengths + 63) // 64
    qblocks = ((w.q_len + 255) // 256) * np.ones_like(lengths) if bq else (lengths + 127) // 128
    stream = torch.cuda.current_stream()

    kernels = {}

    def timed(fn, name):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        jfa.profile_enable(True)
        jfa.profile_read()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        kernels[name] = {k_: round(v_[0] / v_[1], 4) for k_, v_ in jfa.profile_read().items()}
        jfa.profile_enable(False)
        return round(start.elapsed_time(stop) / args.steps, 4)

    res = {"dense": timed(lambda: jfa.fwd(q, k, v, off, broadcast_q=bq, scale=scale, out=o, lse=lse,
                                          workspace=ws_f), "dense")}
    kept = {}
    for kk in [int(x) for x in args.sparse.split(",")]:
        sizes = (len(lengths), w.heads, w.head_dim, w.q_len if bq else 0, int(lengths.sum()), bq, kk)
        ws = torch.empty(jfa._binding.library().jfa_fwd_sparse_workspace_size(*sizes), dtype=torch.uint8,
                         device=q.device)
        res[f"sparse_k{kk}"] = timed(lambda: jfa.fwd_sparse(q, k, v, off, broadcast_q=bq, topk=kk,
                                                            scale=scale, out=o, lse=lse, workspace=ws),
                                     f"sparse_k{kk}")
        kept[f"k{kk}"] = round(float((np.minimum(nkv, kk) * qblocks).sum() / (nkv * qblocks).sum()), 4)
        log(f"k={kk}: {res[f'sparse_k{kk}']:.4f} ms, blocks kept {kept[f'k{kk}']:.3f}")
    print(json.dumps({"mode": "sparse", "workload": w.name, "steps": args.steps, "ms": res,
                      "kernel_ms": kernels, "blocks_kept": kept,
                      "speedup_over_dense": {k_: round(res["dense"] / v_, 4) for k_, v_ in res.items()
                                             if k_ != "dense"}}), flush=True)


def rope_comparison(args, jfa, w, case, o, lse, dq, dk, dv, ws_f, ws_b):
    """Fused rotary backward vs plain backward vs plain backward + separate rotary
    backward, as in the rotary-fusion table of "Meta's TLX Block Attention Beats
    Flash Attention v2 by 2.3x on Blackwell GPUs" (section "The Rotary Fusion Bonus").  The separate
    rotary backward reads the bf16 gradients, rotates them in fp32 and writes bf16."""
    q, k, v, g, off = case["q"], case["k"], case["v"], case["g"], case["offsets"]
    bq, causal, scale = w.broadcast_q, w.causal, case["scale"]
    r = {x: t.cuda() for x, t in workloads.rope_inputs(case).items()}
    rope = (r["cos"], r["sin"], r["pos_q"], r["pos_k"])
    half = w.head_dim // 2
    jfa.fwd(q, k, v, off, broadcast_q=bq, causal=causal, scale=scale, out=o, lse=lse, workspace=ws_f)
    kw = dict(broadcast_q=bq, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws_b)

    def conj(x, pos):
        c, s_ = r["cos"][pos].unsqueeze(1), r["sin"][pos].unsqueeze(1)
        xf = x.float()
        a, b = xf[..., :half], xf[..., half:]
        return torch.cat([a * c + b * s_, b * c - a * s_], dim=-1).to(torch.bfloat16)

    variants = {
        "bwd": lambda: jfa.bwd(q, k, v, off, o, lse, g, **kw),
        "bwd_rope_fused": lambda: jfa.bwd(q, k, v, off, o, lse, g, rope=rope, **kw),
        "bwd_then_rotary": lambda: (jfa.bwd(q, k, v, off, o, lse, g, **kw),
                                    conj(dq, r["pos_q"]), conj(dk, r["pos_k"])),
        "rotary_only": lambda: (conj(dq, r["pos_q"]), conj(dk, r["pos_k"])),
    }
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in variants.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        res[name] = round(start.elapsed_time(stop) / args.steps, 4)
        log(f"{name}: {res[name]:.4f} ms")
    print(json.dumps({"mode": "rope", "workload": w.name, "steps": args.steps, "ms": res,
                      "fused_over_plain": round(res["bwd_rope_fused"] / res["bwd"], 4),
                      "unfused_over_fused": round(res["bwd_then_rotary"] / res["bwd_rope_fused"], 4)}),
          flush=True)


def mxfp8_comparison(args, jfa, w, case, o, lse, ws_f):
    """bf16 forward vs the MXFP8 forward (jfa_fwd_mxfp8 on operands quantized once),
    and the MXFP8 forward with the quantization of Q, K and V included; the kernel
    times come from HIP events around each launch, and the forward's useful FLOP
    rate is set against the dense fp8 and bf16 matrix-core peaks."""
    q, k, v, off = case["q"], case["k"], case["v"], case["offsets"]
    bq, causal, scale = w.broadcast_q, w.causal, case["scale"]
    q8, qs = jfa.mxfp8_quantize_rows(q)
    k8, ks = jfa.mxfp8_quantize_rows(k)
    v8, vs = jfa.mxfp8_quantize_v(v, off)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        jfa.profile_enable(True)
        jfa.profile_read()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        kern = {k_: round(v_[0] / v_[1], 4) for k_, v_ in jfa.profile_read().items()}
        jfa.profile_enable(False)
        return round(start.elapsed_time(stop) / args.steps, 4), kern

    def mx_fwd():
        jfa.fwd_mxfp8(q8, qs, k8, ks, v8, vs, off, broadcast_q=bq, causal=causal, scale=scale, out=o, lse=lse,
                      workspace=ws_f)

    def mx_all():
        jfa.mxfp8_quantize_rows(q, q8, qs)
        jfa.mxfp8_quantize_rows(k, k8, ks)
        jfa.mxfp8_quantize_v(v, off, v8, vs)
        mx_fwd()

    res, kernels = {}, {}
    res["bf16_fwd"], kernels["bf16_fwd"] = timed(
        lambda: jfa.fwd(q, k, v, off, broadcast_q=bq, causal=causal, scale=scale, out=o, lse=lse, workspace=ws_f))
    res["mxfp8_fwd"], kernels["mxfp8_fwd"] = timed(mx_fwd)
    res["mxfp8_quantize_and_fwd"], kernels["mxfp8_quantize_and_fwd"] = timed(mx_all)
    fwd_flops, _ = useful_flops(w, case["lengths"])
    t_mx = kernels["mxfp8_fwd"]["fwd_mxfp8"]
    t_bf = kernels["bf16_fwd"]["fwd"]
    tflops = {"mxfp8_kernel": round(fwd_flops / t_mx / 1e9, 1), "bf16_kernel": round(fwd_flops / t_bf / 1e9, 1)}
    for name in res:
        log(f"{name}: {res[name]:.4f} ms  kernels {kernels[name]}")
    print(json.dumps({"mode": "mxfp8", "workload": w.name, "steps": args.steps, "ms": res, "kernel_ms": kernels,
                      "kernel_tflops": tflops,
                      "frac_of_peak": {"mxfp8_kernel_vs_fp8_5000": round(tflops["mxfp8_kernel"] / 5000.0, 4),
                                       "bf16_kernel_vs_bf16_2500": round(tflops["bf16_kernel"] / 2500.0, 4)},
                      "mxfp8_over_bf16_kernel": round(t_bf / t_mx, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gem_broadcast", choices=workloads.ORDER)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=2, help="0 sorted+zigzag, 1 identity, 2 dynamic (default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rope", action="store_true",
                    help="instead of the step: time the backward with the fused rotary conjugate "
                         "(jfa_bwd_rope) against the plain backward, and against the plain backward "
                         "followed by a separate rotary backward (torch elementwise ops)")
    ap.add_argument("--sparse", type=str, default="", metavar="K[,K...]",
                    help="instead of the step: time the block-sparse forward (jfa_fwd_sparse) with "
                         "these top-k values against the dense forward (non-causal workloads)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="instead of the step: time the MXFP8 forward (jfa_fwd_mxfp8) against the bf16 "
                         "forward, with and without the quantization of Q, K and V")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times); used to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs on "
              "one GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4, "launches": 3}), flush=True)
        return

    import variable_length_flash_jfa_amd as jfa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    case = workloads.make_workload(args.workload, seed=args.seed, device=dev)
    lengths = case["lengths"]
    q, k, v, g, off = case["q"], case["k"], case["v"], case["g"], case["offsets"]
    rows = len(lengths) * w.q_len if w.broadcast_q else int(lengths.sum())
    o = torch.empty((rows, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.heads, rows), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bq, causal, scale = w.broadcast_q, w.causal, case["scale"]
    sizes = (len(lengths), w.heads, w.head_dim, w.q_len if bq else 0, int(lengths.sum()), bq, causal)
    ws_f = torch.empty(jfa.fwd_workspace_size(*sizes), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(jfa.bwd_workspace_size(*sizes), dtype=torch.uint8, device=dev)
    jfa.set_schedule(args.schedule)

    def step():
        jfa.fwd(q, k, v, off, broadcast_q=bq, causal=causal, scale=scale, out=o, lse=lse, workspace=ws_f)
        jfa.bwd(q, k, v, off, o, lse, g, broadcast_q=bq, causal=causal, scale=scale,
                dq=dq, dk=dk, dv=dv, workspace=ws_b)

    if args.rope:
        rope_comparison(args, jfa, w, case, o, lse, dq, dk, dv, ws_f, ws_b)
        return
    if args.sparse:
        sparse_comparison(args, jfa, w, case, o, lse, ws_f)
        return
    if args.mxfp8:
        mxfp8_comparison(args, jfa, w, case, o, lse, ws_f)
        return

    log(f"workload {w.name}: B={len(lengths)} H={w.heads} D={w.head_dim} Lq={w.q_len} "
        f"T={int(lengths.sum())} lengths min/median/mean/max = {lengths.min()}/{np.median(lengths):.0f}/"
        f"{lengths.mean():.1f}/{lengths.max()}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    jfa.profile_enable(True)
    jfa.profile_read()            # clear
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    kernels = jfa.profile_read()
    jfa.profile_enable(False)
    ms_per_step = start.elapsed_time(stop) / args.steps

    fwd_flops, bwd_flops = useful_flops(w, lengths)
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    per_launch = {name: ms / max(cnt, 1) for name, (ms, cnt) in kernels.items()}
    fwd_ms = per_launch.get("plan_fwd", 0.0) + per_launch.get("fwd", 0.0)
    bwd_ms = sum(per_launch.get(x, 0.0) for x in ("bwd_pre", "plan_bwd", "bwd", "dq_finalize"))
    log("per-launch ms (HIP events): " + ", ".join(f"{k_}={v_:.4f}" for k_, v_ in per_launch.items()))

    # roofline of the dominant kernel
    abytes = algorithmic_bytes(w, lengths)
    aflops = {"fwd": fwd_flops, "bwd": bwd_flops}
    dom = max(("fwd", "bwd"), key=lambda x: per_launch.get(x, 0.0))
    dom_s = per_launch[dom] * 1e-3
    t_hbm = abytes[dom] / (PEAK_HBM_GBS * 1e9)
    t_mfma = aflops[dom] / (PEAK_BF16_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        achieved, peak, unit, bound = aflops[dom] / dom_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = abytes[dom] / dom_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    traffic = measured_traffic(dom, w.name)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "algorithmic_bytes": abytes[dom], "algorithmic_flops": aflops[dom],
                "avg_launch_ms": round(per_launch[dom], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on a sample (~{args.cpu_seconds:.0f} s) ...")
        cpu = cpu_baseline(case, w, args.cpu_seconds)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "batch": len(lengths), "heads": w.heads, "head_dim": w.head_dim, "q_len": w.q_len,
            "total_kv": int(lengths.sum()), "causal": causal, "broadcast_q": bq, "seed": args.seed,
            "schedule": ["sorted_zigzag", "identity", "dynamic"][args.schedule],
        },
        "kernel_source_hash": kernel_source_hash(),
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 3) if fwd_ms else None,
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 3) if bwd_ms else None,
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in per_launch.items()},
        "wall_s_timed": round(t_wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if result["fwd_tflops"]:
        result["fwd_pct_mfma_peak"] = round(100.0 * result["fwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    if result["bwd_tflops"]:
        result["bwd_pct_mfma_peak"] = round(100.0 * result["bwd_tflops"] / PEAK_BF16_TFLOPS, 2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
