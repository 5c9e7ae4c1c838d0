"""Benchmark of the one-GPU MoE layer step (forward + backward) on MI355X.

One step is the whole hot path on one batch of synthetic tokens, every part in
the library's kernels: dispatch (route + permute), grouped SwiGLU FFN (gate/up
and down GEMMs), combine, combine backward, FFN backward (two data-gradient and
two weight-gradient GEMMs) and dispatch backward.  The workload is the
Triton-distributed ep_moe_fused benchmark shape: T=8192 tokens, hidden 1536,
ffn 480, 64 experts, top-8, bf16 with fp32 accumulation; all 64 experts live on
the one GPU.

Prints one JSON line.  `value` is the step's algorithmic GEMM throughput
(18*A*H*F FLOP per step, A = routed rows) in TFLOP/s; `roofline` is the dominant
GEMM kernel's FLOP rate against the bf16 MFMA peak, timed with HIP events on the
stream the kernels run on; `combine` is the combine kernel's algorithmic
bandwidth against HBM; `cpu_baseline` is the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOADS = {
    "page1": dict(T=8192, H=1536, F=480, E=64, K=8),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemm_flops(A, H, F):
    return {
        "moe_ffn_gate_up_fwd": 4 * A * H * F,
        "moe_ffn_down_fwd": 2 * A * H * F,
        "moe_ffn_down_bwd_data": 2 * A * H * F,
        "moe_ffn_down_bwd_weight": 2 * A * H * F,
        "moe_ffn_gate_up_bwd_data": 4 * A * H * F,
        "moe_ffn_gate_up_bwd_weight": 4 * A * H * F,
    }


def bytes_moved(name, T, H, F, K, A, E):
    """Algorithmic HBM bytes of the bandwidth-bound entries (bf16 rows, int32/fp32 per slot)."""
    s = 2
    if name == "moe_dispatch":
        return T * H * s + A * H * s + T * K * 4 + (T * K + A) * 4
    if name == "moe_combine":
        return A * H * s + T * K * 12 + T * H * s
    if name == "moe_combine_bwd":
        return T * H * s + 2 * A * H * s + T * K * 16
    if name == "moe_dispatch_bwd":
        return A * H * s + T * H * s + T * K * 8
    return None


def measured_traffic(kernel):
    """HBM bytes per launch of a kernel from the committed counter summary
    (profiles/traffic_page1.json), or None when missing or when the kernel
    source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_page1.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "dispatch_expert_gemm_amd", "csrc", "gemm.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if rec.get("gemm_source_sha256") != digest:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(cfg, seconds=10.0, T_sample=1024):
    """The CPU oracle (parity mode) on a T_sample-token slice of the same workload."""
    import moe_workloads as wl
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    inp = wl.layer_inputs(T_sample, cfg["H"], cfg["F"], cfg["E"], cfg["K"], seed=0)
    runs, t0 = 0, time.perf_counter()
    while True:
        f = orc.layer_fwd(inp, prec="parity")
        orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 50:
            break
    A = f["route"].A
    flops = 18.0 * A * cfg["H"] * cfg["F"] * runs
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle fwd+bwd runs (parity mode, numpy) of a {T_sample}-token slice of the "
                      f"same workload (H={cfg['H']} F={cfg['F']} E={cfg['E']} K={cfg['K']}), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="page1", choices=list(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="override T")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB three times "
                         "(the reference kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer here holds every expert on one device and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import dispatch_expert_gemm_amd as dm
    import moe_workloads as wl

    cfg = dict(WORKLOADS[args.workload])
    if args.tokens:
        cfg["T"] = args.tokens
    T, H, F, E, K = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["K"]
    dev = torch.device("cuda:0")
    log(f"[bench] generating inputs T={T} H={H} F={F} E={E} K={K}")
    inp = wl.layer_inputs(T, H, F, E, K, seed=0)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, gout = bf(inp["x"]), bf(inp["grad_out"])
    wg, wu, wd = bf(inp["w_gate"]), bf(inp["w_up"]), bf(inp["w_down"])
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_weights"]).to(dev)
    shape = dm.make_shape(T, H, K, E, F=F)
    cap = shape.capacity
    bf16, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    ex = torch.empty((cap, H), dtype=bf16, device=dev)
    assist = torch.empty(dm.moe_assist_info_size(shape), dtype=i32, device=dev)
    cnt = torch.empty(E, dtype=i32, device=dev)
    recv = torch.empty(E, dtype=i32, device=dev)
    err = torch.empty(1, dtype=i32, device=dev)
    ws = torch.empty(dm.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    gus = torch.empty((cap, 2 * F), dtype=bf16, device=dev)
    h = torch.empty((cap, F), dtype=bf16, device=dev)
    y = torch.empty((cap, H), dtype=bf16, device=dev)
    out = torch.empty((T, H), dtype=bf16, device=dev)
    gy = torch.empty((cap, H), dtype=bf16, device=dev)
    gw = torch.empty((T, K), dtype=f32, device=dev)
    ggu = torch.empty((cap, 2 * F), dtype=bf16, device=dev)
    gxe = torch.empty((cap, H), dtype=bf16, device=dev)
    gwg = torch.empty((E, F, H), dtype=f32, device=dev)
    gwu = torch.empty((E, F, H), dtype=f32, device=dev)
    gwd = torch.empty((E, H, F), dtype=f32, device=dev)
    gx = torch.empty((T, H), dtype=bf16, device=dev)

    calls = [
        ("moe_dispatch", lambda: dm.moe_dispatch(shape, x, idx, None, ex, assist, cnt, recv, err, ws)),
        ("moe_ffn_gate_up_fwd", lambda: dm.moe_ffn_gate_up_fwd(shape, ex, wg, wu, recv, gus, h)),
        ("moe_ffn_down_fwd", lambda: dm.moe_ffn_down_fwd(shape, h, wd, recv, y)),
        ("moe_combine", lambda: dm.moe_combine(shape, y, idx, w, assist, recv, None, None, x, None, None,
                                               None, out)),
        ("moe_combine_bwd", lambda: dm.moe_combine_bwd(shape, gout, y, idx, w, assist, recv, None, x, None,
                                                       None, None, gy, gw)),
        ("moe_ffn_down_bwd_data", lambda: dm.moe_ffn_down_bwd_data(shape, gy, wd, gus, recv, ggu)),
        ("moe_ffn_down_bwd_weight", lambda: dm.moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)),
        ("moe_ffn_gate_up_bwd_data", lambda: dm.moe_ffn_gate_up_bwd_data(shape, ggu, wg, wu, recv, gxe)),
        ("moe_ffn_gate_up_bwd_weight", lambda: dm.moe_ffn_gate_up_bwd_weight(shape, ggu, ex, recv, gwg, gwu)),
        ("moe_dispatch_bwd", lambda: dm.moe_dispatch_bwd(shape, gxe, assist, idx, w, None, gout, None, None,
                                                         gx)),
    ]

    def step():
        for _, fn in calls:
            fn()

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    A = int(recv[-1].item())
    assert int(err.item()) == 0

    # timed region: K whole steps, synchronised on both sides
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-entry durations: HIP events on torch's current stream (the stream every call launches on)
    log("[bench] per-kernel event timing")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record()
        for i, (_, fn) in enumerate(calls):
            fn()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    per = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
           for i, (name, _) in enumerate(calls)}

    fl = gemm_flops(A, H, F)
    total_flops = sum(fl.values())
    dom = max(fl, key=lambda k: per[k])
    achieved = fl[dom] / (per[dom] * 1e-3) / 1e12
    kernels = {}
    for name, ms in per.items():
        rec = {"ms": round(ms, 4)}
        if name in fl:
            rec["TFLOP/s"] = round(fl[name] / (ms * 1e-3) / 1e12, 1)
            rec["frac_mfma"] = round(rec["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
        b = bytes_moved(name, T, H, F, K, A, E)
        if b is not None:
            rec["GB/s"] = round(b / (ms * 1e-3) / 1e9, 1)
            rec["frac_hbm"] = round(rec["GB/s"] / PEAK_HBM_GBS, 4)
        kernels[name] = rec
    gemm_ms = sum(per[k] for k in fl)

    res = {
        "metric": "MoE layer fwd+bwd ms & TFLOP/s (% MFMA peak); combine GB/s (% HBM) at 1 GPU",
        "value": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
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
        "config": {"workload": f"MoE layer fwd+bwd, Triton-distributed benchmark shape: T={T} tokens, "
                               f"H={H}, F={F} SwiGLU, E={E} experts on one GPU, top-{K}",
                   "T": T, "H": H, "F": F, "E": E, "K": K, "routed_rows": A,
                   "flop_per_step": total_flops},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(dom)},
        "combine": {"GB/s": kernels["moe_combine"]["GB/s"], "peak": PEAK_HBM_GBS,
                    "frac": kernels["moe_combine"]["frac_hbm"]},
        "gemm_ms_per_step": round(gemm_ms, 4),
        "gemm_frac_mfma": round(total_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "context": {"page1_fwd_bwd_ms_4_nvidia_gpus_T8192": 5.488},
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
