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
GEMM kernel's FLOP rate against the MFMA peak of its dtype, timed with HIP events
on the stream the kernels run on; `combine` is the combine kernel's algorithmic
bandwidth against HBM; `cpu_baseline` is the CPU oracle on a bounded sample.

`--workload` picks extra measurements (not the default line): `dsv3_proxy`
(T=4096, hidden 7168, ffn 2048, 32 experts, top-8, Zipf-skewed routing, one
shared expert run as a one-group GEMM over all tokens), `mixtral` (T=8192,
hidden 4096, ffn 14336, 8 experts, top-2, fp8 e4m3 block-scaled forward and
data-gradient GEMMs, bf16 weight gradients, int8 combine payload; x's codes
come out of the dispatch copy and dY's out of the combine backward),
`mixtral_grouped` (the same through the grouped fp8 FFN entries),
`combine_stress` (combine, its backward and dispatch backward alone at T=4096,
hidden 7168, 256 routed + zero + copy + 2 constant experts, 2-D mask, shared
term; `value` is the combine's GB/s) and `page1_rank_share` (what one of the
benchmark page's four ranks computes: 16 local experts receiving 65,536 rows,
modelled as top-8 of 16 over 8192 tokens).

The page-1 workloads' timed steps run the weight-gradient GEMMs on a second
stream (each after the call whose output it reads; the main stream waits for
them at the end of the step); the larger layers run on one stream.  Besides
the per-kernel rates, taken in a one-stream pass with each call bracketed by
events, the line carries the step time statistics of that event pass (mean,
std, mean without the three slowest steps, and whether the spread stays within
5% of the mean), the bandwidth-bound kernels re-timed in isolation after a 512 MB write
that evicts the Infinity Cache (`kernels_hbm_isolated`), and the layer roofline
fraction (every GEMM at its MFMA peak plus every other kernel at HBM peak,
over the measured step time).
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# page1 is the default (the benchmark line); the others are extra measurements
WORKLOADS = {
    # the dispatch permute folded into the two GEMMs that read the expanded rows
    # (moe_route, then x read through the row -> slot map by the gate/up forward
    # and the gate/up weight gradient): no expand_x is written
    # two_stream: the weight-gradient GEMMs on a second stream (measured on the
    # page-1 layer: 1.46-1.50 ms against 1.49-1.53 ms on one stream; on the
    # DeepSeek-V3-proxy and Mixtral-style layers two concurrent GEMMs of that
    # size lost 3-4 %, so those run on one stream)
    "page1": dict(T=8192, H=1536, F=480, E=64, K=8, gather=True, two_stream=True),
    # the same layer with the permute as a kernel of its own (moe_dispatch)
    "page1_permute": dict(T=8192, H=1536, F=480, E=64, K=8, two_stream=True),
    # one of page 1's four ranks: 16 local experts receiving 65,536 rows (top-8
    # of 16 over 8192 tokens gives the same rows per expert, 4096), the a2a
    # replaced by the on-device permute
    "page1_rank_share": dict(T=8192, H=1536, F=480, E=16, K=8, gather=True, two_stream=True),
    "dsv3_proxy": dict(T=4096, H=7168, F=2048, E=32, K=8, zipf=1.2, shared=True),
    "mixtral": dict(T=8192, H=4096, F=14336, E=8, K=2, fp8=True),
    # the same step through the grouped fp8 entries of the C ABI (moe_grouped_ffn_fp8,
    # moe_grouped_ffn_bwd_fp8: each chains its GEMMs and quantisers)
    "mixtral_grouped": dict(T=8192, H=4096, F=14336, E=8, K=2, fp8=True, grouped=True),
    # the same layer with the weight gradients in fp8 too (per-128-token operands)
    "mixtral_fp8w": dict(T=8192, H=4096, F=14336, E=8, K=2, fp8=True, fp8_wgrad=True),
    # the same layer with microscaled e4m3 (E8M0 scale per 32 values, applied by the
    # block-scaled MFMA) for the forward and data-gradient GEMMs
    "mixtral_mx": dict(T=8192, H=4096, F=14336, E=8, K=2, fp8=True, mx=True),
    # combine only: 256 routed + 1 zero + 1 copy + 2 constant experts, 2-D mask
    # with 10% false, shared_expert_x; the step is combine, combine backward and
    # dispatch backward (on the expert-output buffer)
    "combine_stress": dict(T=4096, H=7168, E=256, K=8, Z=1, C=1, Q=2, combine_only=True),
    # the low_latency_combine page's decode regime (BS <= 512 tokens, H = 7168,
    # top-8, 32 experts in its example), every expert on one GPU, forward only
    "decode": dict(T=512, H=7168, F=2048, E=32, K=8, forward_only=True),
    "decode_gather": dict(T=512, H=7168, F=2048, E=32, K=8, forward_only=True, gather=True),
    # the same batch on the page's quant_mode 2 path: int8 dispatch with per-expert
    # smooth scales, w8a8 grouped GEMMs (int8 weights: half the bytes to stream)
    "decode_int8": dict(T=512, H=7168, F=2048, E=32, K=8, forward_only=True, int8=True),
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


def gemm_bytes(name, A, H, F, E, T=0):
    """Algorithmic HBM bytes of a bf16 grouped GEMM: every expert's weights once, its
    input rows (A routed rows, each counted once, also when gathered from x), its
    saved operands and its outputs; weight gradients are written in fp32.  int8
    GEMMs read 1-byte weights and rows plus one fp32 scale per row and channel.
    The shared expert's GEMMs are the same with A = T rows and one expert.  Other
    8-bit GEMMs: 0 (they are set against the MFMA peak only)."""
    if name.startswith("shared "):
        base = name[len("shared "):]
        if base.startswith("moe_grouped_ffn_bwd"):
            return sum(gemm_bytes(n, T, H, F, 1) for n in (
                "moe_ffn_down_bwd_data", "moe_ffn_down_bwd_weight", "moe_ffn_gate_up_bwd_data",
                "moe_ffn_gate_up_bwd_weight"))
        return gemm_bytes(base, T, H, F, 1)
    if name == "moe_ffn_gate_up_fwd_int8":
        return E * 2 * F * (H + 4) + A * (H + 4) + A * 3 * F * 2
    if name == "moe_ffn_down_fwd_int8":
        return E * H * (F + 4) + A * (F + 4) + A * H * 2
    if name.endswith(("_fp8", "_mx", "_int8")) or "fp8" in name:
        return 0
    if name.startswith("moe_ffn_gate_up_fwd"):
        return E * 2 * F * H * 2 + A * H * 2 + A * 3 * F * 2
    if name.startswith("moe_ffn_down_fwd"):
        return E * H * F * 2 + A * F * 2 + A * H * 2
    if name.startswith("moe_ffn_down_bwd_data"):  # dY (or grad_out rows + row weights), W_down, G|U in; dG|dU out
        return A * H * 2 + E * H * F * 2 + A * 2 * F * 2 * 2 + (A * 4 if name.endswith("_gather") else 0)
    if name.startswith("moe_ffn_down_bwd_weight"):  # dY (or grad_out rows + row weights), h in; dW_down out
        return A * H * 2 + A * F * 2 + E * H * F * 4 + (A * 4 if name.endswith("_gather") else 0)
    if name == "moe_ffn_gate_up_bwd_data":   # dG|dU, W_gate, W_up in; dX out
        return A * 2 * F * 2 + E * 2 * F * H * 2 + A * H * 2
    if name.startswith("moe_ffn_gate_up_bwd_weight"):  # dG|dU, x rows in; dW_gate, dW_up (fp32) out
        return A * 2 * F * 2 + A * H * 2 + E * 2 * F * H * 4
    return 0


def bytes_moved(name, T, H, F, K, A, E):
    """Algorithmic HBM bytes of the bandwidth-bound entries (bf16 rows, int32/fp32 per slot)."""
    s = 2
    if name == "moe_dispatch":
        return T * H * s + A * H * s + T * K * 4 + (T * K + A) * 4
    if name == "moe_combine":
        return A * H * s + T * K * 12 + T * H * s
    if name == "moe_combine_bwd":
        return T * H * s + 2 * A * H * s + T * K * 16
    if name == "moe_combine_bwd_weights":  # grad_out, y rows, weights, maps in; dw, row weights out
        return T * H * s + A * H * s + T * K * 16 + A * 4
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
    fp8 = cfg.get("fp8", False)
    fwd_only = cfg.get("forward_only", False)
    T_sample = min(T_sample, cfg["T"])
    inp = wl.layer_inputs(T_sample, cfg["H"], cfg["F"], cfg["E"], cfg["K"], seed=0,
                          zipf=cfg.get("zipf"), shared=cfg.get("shared", False))
    smooth = np.exp(np.random.default_rng(7).standard_normal((cfg["E"], cfg["H"])) * 0.5).astype(np.float32)
    runs, t0 = 0, time.perf_counter()
    while True:
        if cfg.get("int8"):
            f = orc.layer_fwd_int8(inp, smooth)
        elif cfg.get("mx"):
            f = orc.layer_fwd_mx(inp)
            orc.layer_bwd_mx(inp, f, inp["grad_out"])
        elif fp8:
            f = orc.layer_fwd_fp8(inp)
            orc.layer_bwd_fp8(inp, f, inp["grad_out"], wgrad="fp8" if cfg.get("fp8_wgrad") else "bf16")
        else:
            f = orc.layer_fwd(inp, prec="parity")
            if not fwd_only:
                orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 50:
            break
    A = f["route"].A
    flops = (6.0 if fwd_only else 18.0) * (A + (T_sample if cfg.get("shared") else 0)) * cfg["H"] * cfg["F"] * runs
    what = "forward" if fwd_only else "fwd+bwd"
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle {what} runs (parity mode, numpy) of a {T_sample}-token slice of the "
                      f"same workload (H={cfg['H']} F={cfg['F']} E={cfg['E']} K={cfg['K']}), {el:.1f} s"}


def cpu_baseline_8bit(cfg, seconds=10.0, T_sample=512, F_sample=1024):
    """The CPU oracle of the fp8 / MX layer (parity mode) on a bounded sample of the
    same workload: T_sample tokens over all E experts at the full H, with the first
    F_sample intermediate columns of every expert (a smaller SwiGLU FFN of the same
    kind).  The weights are quantised once before the timing, as the step takes
    them quantised (their quantisation is timed apart on the GPU too)."""
    import moe_workloads as wl
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    mx, fp8w = cfg.get("mx", False), cfg.get("fp8_wgrad", False)
    H, E, K = cfg["H"], cfg["E"], cfg["K"]
    F = min(F_sample, cfg["F"])
    inp = wl.layer_inputs(T_sample, H, F, E, K, seed=0)
    quant = orc.quant_weights_mx if mx else orc.quant_weights_fp8
    wq = tuple(quant(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    runs, t0 = 0, time.perf_counter()
    while True:
        r = orc.route(inp["topk_idx"], E)
        X = orc.dispatch(inp["x"], r)
        fwd = orc.ffn_fwd_mx if mx else orc.ffn_fwd_fp8
        G, U, Hh, Y = fwd(X, r.ep_recv_counts, *wq)
        Yc = orc.qdq_rows_int8(Y)
        orc.combine(Yc, r, inp["topk_weights"], None, inp["x"])
        dY, _ = orc.combine_bwd(inp["grad_out"], Yc, r, inp["topk_weights"], inp["x"])
        if mx:
            _, dX, _, _, _ = orc.ffn_bwd_mx(dY, X, G, U, Hh, r.ep_recv_counts, *wq)
        else:
            _, dX, _, _, _ = orc.ffn_bwd_fp8(dY, X, G, U, Hh, r.ep_recv_counts, *wq,
                                             wgrad="fp8" if fp8w else "bf16")
        orc.dispatch_bwd(dX, r, inp["topk_weights"], inp["grad_out"])
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 50:
            break
    flops = 18.0 * r.A * H * F * runs
    kind = "microscaled fp8" if mx else ("fp8 incl. weight gradients" if fp8w else "fp8")
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle {kind} fwd+bwd runs (parity mode, numpy, weights quantised once) of "
                      f"{T_sample} tokens over all {E} experts with the first {F} of F={cfg['F']} intermediate "
                      f"columns (H={H}, K={K}), {el:.1f} s"}


def cpu_baseline_combine(cfg, seconds=10.0, T_sample=512):
    """The CPU oracle's combine (parity mode) on a T_sample-token slice of the combine stress workload."""
    import moe_workloads as wl
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T, H, E, K, Z, C, Q = (cfg[k] for k in ("T", "H", "E", "K", "Z", "C", "Q"))
    inp = wl.combine_inputs(T_sample, H, E, K, Z, C, Q, seed=0)
    r = orc.route(inp["topk_idx"], E, Z, C, Q, inp["mask"])
    Y = orc.bf16_to_f32(inp["y"])[:r.A]
    runs, t0 = 0, time.perf_counter()
    while True:
        orc.combine(Y, r, inp["topk_weights"], inp["shared_expert_x"], inp["x"], inp["const_alpha_1"],
                    inp["const_alpha_2"], inp["const_v"])
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 200:
            break
    nbytes = r.A * H * 2 + T_sample * K * 12 + 2 * T_sample * H * 2
    return {"value": nbytes * runs / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} oracle combine runs (parity mode, numpy) of a {T_sample}-token slice of the same "
                      f"workload (H={H}, E={E}+{Z}+{C}+{Q}, K={K}), {el:.1f} s"}


# The step's weight-gradient GEMMs run on a second stream, each after the call
# whose output it reads (the rest of the backward stays on the main stream, and
# the main stream waits for both at the end of the step): they read nothing the
# main stream writes later in the step, and they fill the time the data-gradient
# chain leaves the matrix cores idle (page 1: 3% shorter steps).
SIDE_DEPS = {
    "moe_ffn_down_bwd_weight": ("moe_combine_bwd", "moe_combine_bwd_fp8"),
    "moe_ffn_down_bwd_weight_fp8": ("moe_quant_cols_fp8 (dY)",),
    "moe_ffn_gate_up_bwd_weight": ("moe_ffn_down_bwd_data", "moe_ffn_down_bwd_data_fp8", "moe_ffn_down_bwd_data_mx"),
    "moe_ffn_down_bwd_weight_gather": ("moe_combine_bwd_weights",),
    "moe_ffn_gate_up_bwd_weight_gather": ("moe_ffn_down_bwd_data", "moe_ffn_down_bwd_data_gather"),
    "moe_ffn_gate_up_bwd_weight_fp8": ("moe_ffn_down_bwd_data_fp8",),
}


def run_calls(calls, side=None):
    """Launch `calls` in order on torch's current stream; with `side`, the
    weight-gradient GEMMs go to that stream after the call they depend on, and
    the current stream waits for them at the end."""
    import torch
    if side is None:
        for _, fn in calls:
            fn()
        return
    main = torch.cuda.current_stream()
    # an event only after the calls a side call waits for: a marker after every
    # call costs the step a few microseconds each
    needed = {d for name, _ in calls for d in SIDE_DEPS.get(name, ())}
    done, last = {}, None
    for name, fn in calls:
        deps = SIDE_DEPS.get(name)
        dep = next((d for d in deps if d in done), None) if deps else None
        if dep is None:
            fn()
            if name in needed:
                ev = torch.cuda.Event()
                ev.record(main)
                done[name] = ev
        else:
            side.wait_event(done[dep])
            with torch.cuda.stream(side):
                fn()
            last = torch.cuda.Event()
            last.record(side)
    if last is not None:
        main.wait_event(last)


class Step:
    """The C-entry calls of one fwd+bwd step of a workload (name, thunk), in order,
    plus calls timed outside the step (fp8 weight quantisation)."""

    def __init__(self):
        self.calls, self.config, self.cfg = [], {}, {}
        self.recv = self.err = self.counts = None
        self.dtype = "bf16"
        self.two_stream = False
        self.extra_calls = []


def _bf(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def build_combine_step(cfg):
    """Combine-only step of the combine stress workload: moe_dispatch runs once
    outside the step to build the routing maps."""
    import torch
    import dispatch_expert_gemm_amd as dm
    import moe_workloads as wl

    T, H, E, K, Z, C, Q = (cfg[k] for k in ("T", "H", "E", "K", "Z", "C", "Q"))
    dev = torch.device("cuda:0")
    log(f"[bench] combine_stress: generating inputs T={T} H={H} E={E}+{Z}+{C}+{Q} K={K}")
    inp = wl.combine_inputs(T, H, E, K, Z, C, Q, seed=0)
    x, y, sh, gout = (_bf(inp[k], dev) for k in ("x", "y", "shared_expert_x", "grad_out"))
    a1, a2, cv = (_bf(inp[k], dev) for k in ("const_alpha_1", "const_alpha_2", "const_v"))
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_weights"]).to(dev)
    mask = torch.from_numpy(inp["mask"]).to(dev)
    shape = dm.make_shape(T, H, K, E, zero_expert_num=Z, copy_expert_num=C, const_expert_num=Q, mask_ndim=2)
    d = dm.dispatch(shape, x, idx, mask)
    torch.cuda.synchronize()
    assert int(d.err_flag.item()) == 0
    cap = shape.capacity
    out, gy, gx = (torch.empty(sz, dtype=torch.bfloat16, device=dev) for sz in ((T, H), (cap, H), (T, H)))
    gw = torch.empty((T, K), dtype=torch.float32, device=dev)
    st = Step()
    st.recv, st.err = d.ep_recv_counts, d.err_flag
    st.calls = [
        ("moe_combine", lambda: dm.moe_combine(shape, y, idx, w, d.assist_info_for_combine, d.ep_recv_counts,
                                               mask, sh, x, a1, a2, cv, out)),
        ("moe_combine_bwd", lambda: dm.moe_combine_bwd(shape, gout, y, idx, w, d.assist_info_for_combine,
                                                       d.ep_recv_counts, mask, x, a1, a2, cv, gy, gw)),
        ("moe_dispatch_bwd", lambda: dm.moe_dispatch_bwd(shape, y, d.assist_info_for_combine, idx, w, mask, gout,
                                                         a1, None, gx)),
    ]
    # tokens with at least one active copy or constant slot read their ori_x /
    # grad_out row once more
    ids, m = inp["topk_idx"], inp["mask"].astype(bool)
    special = ((ids >= E + Z) & m).any(axis=1)
    st.n_ori = int(special.sum())
    st.mask_bytes = T * K
    st.config = {"T": T, "H": H, "F": 0, "E": E, "K": K}
    st.cfg = cfg
    st.shape_info = (T, H, 0, K, E)
    # the router over the 260 ids of this layer (weights not renormalised, as in
    # the combine inputs), timed apart from the step
    _add_router(st, cfg, T, K, E, dev, False)
    return st


def build_step(name, T_override=None):
    import torch
    import dispatch_expert_gemm_amd as dm
    import moe_workloads as wl

    cfg = dict(WORKLOADS[name])
    if T_override:
        cfg["T"] = T_override
    if cfg.get("combine_only"):
        return build_combine_step(cfg)
    T, H, F, E, K = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["K"]
    dev = torch.device("cuda:0")
    shared = cfg.get("shared", False)
    fp8 = cfg.get("fp8", False)
    fp8w = fp8 and cfg.get("fp8_wgrad", False)
    mx = fp8 and cfg.get("mx", False)
    int8 = cfg.get("int8", False)
    log(f"[bench] {name}: generating inputs T={T} H={H} F={F} E={E} K={K}")
    inp = wl.layer_inputs(T, H, F, E, K, seed=0, zipf=cfg.get("zipf"), shared=shared)
    x, gout = _bf(inp["x"], dev), _bf(inp["grad_out"], dev)
    wg, wu, wd = (_bf(inp[k], dev) for k in ("w_gate", "w_up", "w_down"))
    del inp["w_gate"], inp["w_up"], inp["w_down"]
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    w = torch.from_numpy(inp["topk_weights"]).to(dev)
    shape = dm.make_shape(T, H, K, E, F=F, comm_quant_mode=2 if fp8 else 0)
    cap = shape.capacity
    bf16, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    z = lambda *sh, dt=bf16: torch.empty(sh, dtype=dt, device=dev)
    ex, assist = z(cap, H), z(dm.moe_assist_info_size(shape), dt=i32)
    cnt, recv, err = z(E, dt=i32), z(E, dt=i32), z(1, dt=i32)
    ws = z(dm.moe_workspace_size(shape), dt=torch.uint8)
    gus, h, y, out = z(cap, 2 * F), z(cap, F), z(cap, H), z(T, H)
    gy, gw, ggu, gxe, gx = z(cap, H), z(T, K, dt=f32), z(cap, 2 * F), z(cap, H), z(T, H)
    gwg, gwu, gwd = z(E, F, H, dt=f32), z(E, F, H, dt=f32), z(E, H, F, dt=f32)
    st = Step()
    st.recv, st.err, st.counts = recv, err, cnt
    st.two_stream = bool(cfg.get("two_stream", False))
    C = st.calls
    sy = sdx = None
    if int8:
        st.dtype = "int8 (dispatch rows, w8a8 GEMMs), bf16 outputs"
        gen = torch.Generator(device=dev).manual_seed(7)
        smooth = torch.exp(torch.randn((E, H), generator=gen, device=dev) * 0.5)
        exq, dyn = z(cap, H, dt=torch.int8), z(cap, dt=f32)
        wq8 = [dm.quant_rows_int8(t) for t in (wg, wu, wd)]
        hq8, hs8 = z(cap, F, dt=torch.int8), z(cap, dt=f32)
        C.append(("moe_dispatch_int8", lambda: dm.moe_dispatch_int8(shape, x, idx, None, smooth, exq, dyn, assist,
                                                                    cnt, recv, err, ws)))
        # weight quantisation (once per weight update) is timed outside the step
        st.extra_calls.append(("moe_quant_rows_int8 (3 weight tensors)",
                               lambda: [dm.quant_rows_int8(t) for t in (wg, wu, wd)]))
    elif cfg.get("gather"):
        # routing only: the gate/up GEMMs read the rows from x themselves; the
        # permute as a kernel of its own (moe_dispatch) is timed apart
        C.append(("moe_route", lambda: dm.moe_route(shape, idx, None, assist, cnt, recv, err, ws)))
        st.extra_calls.append(("moe_dispatch (route + permute, not in the step)",
                               lambda: dm.moe_dispatch(shape, x, idx, None, ex, assist, cnt, recv, err, ws)))
    elif fp8 and not mx:
        # x's e4m3 codes and scales come out of the dispatch copy (the bf16 rows
        # too: the bf16 gate/up weight gradient reads them)
        xq, xs = z(cap, H, dt=torch.uint8), z(H // 128, cap, dt=f32)
        C.append(("moe_dispatch_fp8", lambda: dm.moe_dispatch_fp8(shape, x, idx, None, ex, xq, xs, assist, cnt,
                                                                  recv, err, ws)))
    else:
        C.append(("moe_dispatch", lambda: dm.moe_dispatch(shape, x, idx, None, ex, assist, cnt, recv, err, ws)))
    if int8:
        C += [
            ("moe_ffn_gate_up_fwd_int8", lambda: dm.moe_ffn_gate_up_fwd_int8(
                shape, exq, dyn, wq8[0][0], wq8[0][1], wq8[1][0], wq8[1][1], recv, gus, h)),
            ("moe_quant_rows_int8 (h)", lambda: dm.moe_quant_rows_int8(h, hq8, hs8, recv[-1:])),
            ("moe_ffn_down_fwd_int8", lambda: dm.moe_ffn_down_fwd_int8(shape, hq8, hs8, wq8[2][0], wq8[2][1],
                                                                       recv, y)),
        ]
    elif mx:
        st.dtype = "fp8 e4m3 with E8M0 scales per 32 values (fwd + data grads), bf16 (weight grads)"
        nrows = recv[-1:]
        wqm = [dm.MxWeights.quantize(t) for t in (wg, wu, wd)]
        u8 = torch.uint8
        xq, xs, hq, hs = z(cap, H, dt=u8), z(cap, H // 32, dt=u8), z(cap, F, dt=u8), z(cap, F // 32, dt=u8)
        dyq, dys, dgq, dgs = z(cap, H, dt=u8), z(cap, H // 32, dt=u8), z(cap, 2 * F, dt=u8), z(cap, 2 * F // 32, dt=u8)
        C += [
            ("moe_quant_rows_mx (x)", lambda: dm.moe_quant_rows_mx(ex, xq, xs, nrows)),
            # h's MX codes come out of the gate/up GEMM
            ("moe_ffn_gate_up_fwd_mx", lambda: dm.moe_ffn_gate_up_fwd_mx(
                shape, xq, xs, wqm[0].codes, wqm[0].scales, wqm[1].codes, wqm[1].scales, recv, gus, h, (hq, hs))),
            ("moe_ffn_down_fwd_mx", lambda: dm.moe_ffn_down_fwd_mx(shape, hq, hs, wqm[2].codes, wqm[2].scales,
                                                                   recv, y)),
        ]
    elif fp8:
        st.dtype = ("fp8 e4m3 (all six GEMMs; weight grads on per-128-token operands)" if fp8w
                    else "fp8 e4m3 (fwd + data grads), bf16 (weight grads)")
        nrows = recv[-1:]
        wq = [dm.Fp8Weights.quantize(t) for t in (wg, wu, wd)]
        # row scales are column-block major: (C/128, capacity)
        hq, hs = z(cap, F, dt=torch.uint8), z(F // 128, cap, dt=f32)
        dyq, dys = z(cap, H, dt=torch.uint8), z(H // 128, cap, dt=f32)
        dgq, dgs = z(cap, 2 * F, dt=torch.uint8), z(2 * F // 128, cap, dt=f32)
        if cfg.get("grouped"):
            fws = z(dm.moe_ffn_fp8_workspace_size(shape), dt=torch.uint8)
            C.append(("moe_grouped_ffn_fp8 (gate/up, h codes, down)", lambda: dm.moe_grouped_ffn_fp8(
                shape, xq, xs, wq, recv, gus, h, y, fws)))
        C += [] if cfg.get("grouped") else [
            ("moe_ffn_gate_up_fwd_fp8", lambda: dm.moe_ffn_gate_up_fwd_fp8(
                shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales, recv, gus, h)),
            ("moe_quant_rows_fp8 (h)", lambda: dm.moe_quant_rows_fp8(h, hq, hs, nrows)),
            ("moe_ffn_down_fwd_fp8", lambda: dm.moe_ffn_down_fwd_fp8(shape, hq, hs, wq[2].codes, wq[2].scales,
                                                                     recv, y)),
        ]
        if fp8w:
            # per-128-token codes of the weight-gradient operands, each taken right
            # after the kernel that wrote its source
            ns = dm.cols_fp8_slots(cap, E)
            cq = {k: (z(d, 128 * ns, dt=torch.uint8), z(ns, d, dt=f32))
                  for k, d in (("x", H), ("h", F), ("dY", H), ("dGU", 2 * F))}
            i = [n for n, _ in C].index("moe_dispatch_fp8")
            C.insert(i + 1, ("moe_quant_cols_fp8 (x)", lambda: dm.moe_quant_cols_fp8(ex, recv, *cq["x"])))
            # h's codes come out of the gate/up GEMM itself
            i = [n for n, _ in C].index("moe_ffn_gate_up_fwd_fp8")
            C[i] = ("moe_ffn_gate_up_fwd_fp8", lambda: dm.moe_ffn_gate_up_fwd_fp8_quant(
                shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales, recv, gus, h, *cq["h"]))
    elif cfg.get("gather"):
        C += [
            ("moe_ffn_gate_up_fwd_gather", lambda: dm.moe_ffn_gate_up_fwd_gather(shape, x, assist, wg, wu, recv,
                                                                                 gus, h)),
            ("moe_ffn_down_fwd", lambda: dm.moe_ffn_down_fwd(shape, h, wd, recv, y)),
        ]
    else:
        C += [
            ("moe_ffn_gate_up_fwd", lambda: dm.moe_ffn_gate_up_fwd(shape, ex, wg, wu, recv, gus, h)),
            ("moe_ffn_down_fwd", lambda: dm.moe_ffn_down_fwd(shape, h, wd, recv, y)),
        ]
    if shared:
        swg, swu, swd = (_bf(inp[k], dev) for k in ("shared_w_gate", "shared_w_up", "shared_w_down"))
        ss = dm.shared_expert_shape(T, H, F)
        scnt = torch.full((1,), T, dtype=i32, device=dev)
        s_gus, s_h, sy = z(T, 2 * F), z(T, F), z(T, H)
        s_ggu, sdx = z(T, 2 * F), z(T, H)
        s_gw = [z(1, F, H, dt=f32), z(1, F, H, dt=f32), z(1, H, F, dt=f32)]
        C += [
            ("shared moe_ffn_gate_up_fwd", lambda: dm.moe_ffn_gate_up_fwd(ss, x, swg, swu, scnt, s_gus, s_h)),
            ("shared moe_ffn_down_fwd", lambda: dm.moe_ffn_down_fwd(ss, s_h, swd, scnt, sy)),
        ]
    C += [
        ("moe_combine", lambda: dm.moe_combine(shape, y, idx, w, assist, recv, None, sy, x, None, None, None,
                                               out)),
    ]
    st.config = {"T": T, "H": H, "F": F, "E": E, "K": K}
    st.cfg = cfg
    st.shape_info = (T, H, F, K, E)
    _add_router(st, cfg, T, K, E, dev, cfg.get("renorm", True))
    if cfg.get("forward_only"):
        return st
    # bf16 layers with a narrow expert FFN (F < 1024) take the combine backward
    # folded into the down GEMMs (the rule moe_layer follows): measured 3% faster
    # at F = 480, 1.3% slower at F = 2048, where the down weight gradient's
    # per-element scaling of its operand costs more than grad_y's bytes
    fold = not fp8 and dm.fold_combine_bwd(F)
    if fp8 and not mx:
        # dY's e4m3 codes and scales come out of the combine backward (with the
        # bf16 dY, which the bf16 down weight gradient reads)
        C.append(("moe_combine_bwd_fp8", lambda: dm.moe_combine_bwd_fp8(
            shape, gout, y, idx, w, assist, recv, None, x, None, None, None, gy, dyq, dys, gw)))
    elif fold:
        # the combine backward folded into the down GEMMs' operand loads: no
        # grad_y rows, only the routing weights' gradient and each row's weight
        roww = z(cap, dt=f32)
        C.append(("moe_combine_bwd_weights", lambda: dm.moe_combine_bwd_weights(
            shape, gout, y, idx, w, assist, recv, None, x, None, None, None, gw, roww)))
    else:
        C.append(("moe_combine_bwd", lambda: dm.moe_combine_bwd(shape, gout, y, idx, w, assist, recv, None, x,
                                                               None, None, None, gy, gw)))
    # backward order: each gather/scatter right after the kernel that produced
    # its input (grad_expand_x goes to dispatch backward before the last
    # weight gradient evicts it from the caches)
    if mx:
        C += [
            ("moe_quant_rows_mx (dY)", lambda: dm.moe_quant_rows_mx(gy, dyq, dys, nrows)),
            # bf16 dG|dU for the bf16 weight gradient and its MX codes, one kernel
            ("moe_ffn_down_bwd_data_mx", lambda: dm.moe_ffn_down_bwd_data_mx(
                shape, dyq, dys, wqm[2].codes_t, wqm[2].scales_t, gus, recv, ggu, (dgq, dgs))),
            ("moe_ffn_down_bwd_weight", lambda: dm.moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)),
            ("moe_ffn_gate_up_bwd_data_mx", lambda: dm.moe_ffn_gate_up_bwd_data_mx(
                shape, dgq, dgs, wqm[0].codes_t, wqm[0].scales_t, wqm[1].codes_t, wqm[1].scales_t, recv, gxe)),
        ]
    elif fp8w:
        C += [
            ("moe_quant_cols_fp8 (dY)", lambda: dm.moe_quant_cols_fp8(gy, recv, *cq["dY"])),
            # dG/dU leave the data gradient as row codes and per-128-token codes
            # only (nothing else reads them)
            ("moe_ffn_down_bwd_data_fp8", lambda: dm.moe_ffn_down_bwd_data_fp8_quant(
                shape, dyq, dys, wq[2].codes_t, wq[2].scales, gus, recv, None, (dgq, dgs), cq["dGU"])),
            ("moe_ffn_down_bwd_weight_fp8", lambda: dm.moe_ffn_down_bwd_weight_fp8(
                shape, *cq["dY"], *cq["h"], recv, gwd)),
            ("moe_ffn_gate_up_bwd_data_fp8", lambda: dm.moe_ffn_gate_up_bwd_data_fp8(
                shape, dgq, dgs, wq[0].codes_t, wq[0].scales, wq[1].codes_t, wq[1].scales, recv, gxe)),
        ]
    elif fp8 and cfg.get("grouped"):
        C += [("moe_grouped_ffn_bwd_fp8 (4 GEMMs, dG|dU codes)", lambda: dm.moe_grouped_ffn_bwd_fp8(
            shape, gy, dyq, dys, ex, gus, h, wq, recv, ggu, gxe, gwg, gwu, gwd, fws))]
    elif fp8:
        C += [
            # bf16 dG/dU (for the bf16 weight gradient) and their row codes
            ("moe_ffn_down_bwd_data_fp8", lambda: dm.moe_ffn_down_bwd_data_fp8_quant(
                shape, dyq, dys, wq[2].codes_t, wq[2].scales, gus, recv, ggu, (dgq, dgs))),
            ("moe_ffn_down_bwd_weight", lambda: dm.moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)),
            ("moe_ffn_gate_up_bwd_data_fp8", lambda: dm.moe_ffn_gate_up_bwd_data_fp8(
                shape, dgq, dgs, wq[0].codes_t, wq[0].scales, wq[1].codes_t, wq[1].scales, recv, gxe)),
        ]
    elif fold:
        C += [
            ("moe_ffn_down_bwd_data_gather", lambda: dm.moe_ffn_down_bwd_data_gather(
                shape, gout, assist, roww, wd, gus, recv, ggu)),
            ("moe_ffn_down_bwd_weight_gather", lambda: dm.moe_ffn_down_bwd_weight_gather(
                shape, gout, assist, roww, h, recv, gwd)),
            ("moe_ffn_gate_up_bwd_data", lambda: dm.moe_ffn_gate_up_bwd_data(shape, ggu, wg, wu, recv, gxe)),
        ]
    else:
        C += [
            ("moe_ffn_down_bwd_data", lambda: dm.moe_ffn_down_bwd_data(shape, gy, wd, gus, recv, ggu)),
            ("moe_ffn_down_bwd_weight", lambda: dm.moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)),
            ("moe_ffn_gate_up_bwd_data", lambda: dm.moe_ffn_gate_up_bwd_data(shape, ggu, wg, wu, recv, gxe)),
        ]
    if shared:
        C.append(("shared moe_grouped_ffn_bwd (4 GEMMs)", lambda: dm.moe_grouped_ffn_bwd(
            ss, gout, x, s_gus, s_h, swg, swu, swd, scnt, s_ggu, sdx, *s_gw)))
    C.append(("moe_dispatch_bwd", lambda: dm.moe_dispatch_bwd(shape, gxe, assist, idx, w, None, gout, None, sdx,
                                                              gx)))
    if fp8w:
        C.append(("moe_ffn_gate_up_bwd_weight_fp8", lambda: dm.moe_ffn_gate_up_bwd_weight_fp8(
            shape, *cq["dGU"], *cq["x"], recv, gwg, gwu)))
    elif cfg.get("gather"):
        C.append(("moe_ffn_gate_up_bwd_weight_gather", lambda: dm.moe_ffn_gate_up_bwd_weight_gather(
            shape, ggu, x, assist, recv, gwg, gwu)))
    elif cfg.get("grouped"):
        pass  # the grouped backward entry ends with the gate/up weight gradient
    else:
        C.append(("moe_ffn_gate_up_bwd_weight", lambda: dm.moe_ffn_gate_up_bwd_weight(shape, ggu, ex, recv, gwg,
                                                                                      gwu)))
    if mx:
        # weight quantisation (once per weight update, both layouts) is timed outside the step
        st.extra_calls.insert(0, ("moe_quantize_weights_mx (3 tensors)",
                                  lambda: [dm.MxWeights.quantize(t) for t in (wg, wu, wd)]))
    elif fp8:
        # weight quantisation (once per weight update) is timed outside the step
        st.extra_calls.insert(0, ("moe_quantize_weights_fp8 (3 tensors)",
                                  lambda: [dm.Fp8Weights.quantize(t) for t in (wg, wu, wd)]))
    return st


def _add_router(st, cfg, T, K, E, dev, renorm):
    """Time the router that produces topk_idx / topk_weights from gating logits, and
    its backward, apart from the step (the step takes the routing as input)."""
    import torch
    import dispatch_expert_gemm_amd as dm
    n_ids = E + cfg.get("Z", 0) + cfg.get("C", 0) + cfg.get("Q", 0)
    gen = torch.Generator(device=dev).manual_seed(5)
    f32 = torch.float32
    logits = torch.randn((T, n_ids), dtype=f32, device=dev, generator=gen)
    r_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    r_w = torch.empty((T, K), dtype=f32, device=dev)
    r_dw = torch.randn((T, K), dtype=f32, device=dev, generator=gen)
    r_dl = torch.empty((T, n_ids), dtype=f32, device=dev)
    st.extra_calls += [
        (f"moe_router ({n_ids} ids, top-{K})", lambda: dm.moe_router(logits, K, renorm, r_idx, r_w)),
        (f"moe_router_bwd ({n_ids} ids, top-{K})",
         lambda: dm.moe_router_bwd(logits, K, renorm, r_idx, r_w, r_dw, r_dl)),
    ]


def account(st, A):
    """FLOP and byte counts of every call of the step, given the routed rows A."""
    T, H, F, K, E = st.shape_info
    if st.cfg.get("combine_only"):
        Q = st.cfg["Q"]
        nb = {"moe_combine": bytes_moved("moe_combine", T, H, F, K, A, E) + T * H * 2 + st.n_ori * H * 2
              + 3 * Q * H * 2 + st.mask_bytes,
              "moe_combine_bwd": bytes_moved("moe_combine_bwd", T, H, F, K, A, E) + st.n_ori * H * 2
              + 3 * Q * H * 2 + st.mask_bytes,
              "moe_dispatch_bwd": bytes_moved("moe_dispatch_bwd", T, H, F, K, A, E) + st.n_ori * H * 2
              + Q * H * 2 + st.mask_bytes}
        return {}, nb
    fp8 = st.cfg.get("fp8", False)
    fp8w = fp8 and st.cfg.get("fp8_wgrad", False)
    int8 = st.cfg.get("int8", False)
    pk = PEAK_INT8_TOPS if int8 else (PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS)
    pkw = PEAK_FP8_TFLOPS if fp8w else PEAK_BF16_TFLOPS
    fl = {}
    fwd_only = st.cfg.get("forward_only", False)
    for n, (mult, peak) in {"moe_ffn_gate_up_fwd": (4, pk), "moe_ffn_down_fwd": (2, pk),
                            "moe_ffn_down_bwd_data": (2, pk), "moe_ffn_down_bwd_weight": (2, pkw),
                            "moe_ffn_gate_up_bwd_data": (4, pk),
                            "moe_ffn_gate_up_bwd_weight": (4, pkw)}.items():
        key = n + "_fp8" if fp8 and ("fwd" in n or "data" in n or fp8w) else n
        if int8:
            key = n + "_int8"
        if st.cfg.get("mx") and ("fwd" in n or "data" in n):
            key = n + "_mx"
        if fwd_only and "fwd" not in n:
            continue
        fl[key] = (mult * A * H * F, peak)
    if st.cfg.get("shared"):
        fl["shared moe_ffn_gate_up_fwd"] = (4 * T * H * F, PEAK_BF16_TFLOPS)
        fl["shared moe_ffn_down_fwd"] = (2 * T * H * F, PEAK_BF16_TFLOPS)
        fl["shared moe_grouped_ffn_bwd (4 GEMMs)"] = (12 * T * H * F, PEAK_BF16_TFLOPS)
    nb = {}
    for n in ("moe_dispatch", "moe_combine") if fwd_only else ("moe_dispatch", "moe_combine", "moe_combine_bwd",
                                                                "moe_dispatch_bwd"):
        nb[n] = bytes_moved(n, T, H, F, K, A, E)
    if st.cfg.get("gather"):
        fl["moe_ffn_gate_up_fwd_gather"] = fl.pop("moe_ffn_gate_up_fwd")
        if "moe_ffn_gate_up_bwd_weight" in fl:
            fl["moe_ffn_gate_up_bwd_weight_gather"] = fl.pop("moe_ffn_gate_up_bwd_weight")
        nb["moe_route"] = nb.pop("moe_dispatch") - T * H * 2 - A * H * 2   # no rows moved
    if "moe_combine_bwd_weights" in [n for n, _ in st.calls]:
        # the combine backward folded into the down GEMMs
        fl["moe_ffn_down_bwd_data_gather"] = fl.pop("moe_ffn_down_bwd_data")
        fl["moe_ffn_down_bwd_weight_gather"] = fl.pop("moe_ffn_down_bwd_weight")
        nb["moe_combine_bwd_weights"] = bytes_moved("moe_combine_bwd_weights", T, H, F, K, A, E)
        del nb["moe_combine_bwd"]
    if int8:
        # int8 rows and one fp32 scale per row written, the smooth scales read once
        nb["moe_dispatch_int8"] = nb.pop("moe_dispatch") - A * H * 2 + A * H + A * 4 + E * H * 4
        nb["moe_quant_rows_int8 (h)"] = A * F * 3 + A * 4
    if st.cfg.get("shared"):
        nb["moe_combine"] += T * H * 2
        nb["moe_dispatch_bwd"] += T * H * 2
    if st.cfg.get("mx"):
        for k, d in (("x", H), ("dY", H)):
            nb[f"moe_quant_rows_mx ({k})"] = A * d * 3 + A * d // 32
    elif fp8:
        # x's and dY's codes (one byte per element) and scales (fp32 per 128)
        # leave the dispatch copy and the combine backward
        q8 = A * H + A * H // 128 * 4
        nb["moe_dispatch_fp8"] = nb.pop("moe_dispatch") + q8
        if "moe_combine_bwd" in nb:
            nb["moe_combine_bwd_fp8"] = nb.pop("moe_combine_bwd") + q8
        if st.cfg.get("grouped"):
            # the grouped entries: their GEMMs at the peak of each GEMM's type
            # (h's row codes are a launch inside the forward entry)
            fwd = [k for k in fl if "fwd" in k]
            f_fwd = sum(fl.pop(k)[0] for k in fwd)
            fl["moe_grouped_ffn_fp8 (gate/up, h codes, down)"] = (f_fwd, PEAK_FP8_TFLOPS)
            if not fwd_only:
                bwd = [k for k in list(fl) if "bwd" in k and not k.startswith("moe_grouped") and
                       not k.startswith("shared")]
                parts = [fl.pop(k) for k in bwd]
                f_bwd = sum(f for f, _ in parts)
                t_bwd = sum(f / pk for f, pk in parts)
                fl["moe_grouped_ffn_bwd_fp8 (4 GEMMs, dG|dU codes)"] = (f_bwd, f_bwd / t_bwd)
        else:
            nb["moe_quant_rows_fp8 (h)"] = A * F * 3 + A * F // 128 * 4
    if fp8w:
        # bf16 in, codes out, one fp32 scale per (128 tokens, column)
        for k, d in (("x", H), ("dY", H)):
            nb[f"moe_quant_cols_fp8 ({k})"] = A * d * 3 + -(-A // 128) * d * 4
    return fl, nb


def time_calls(calls, steps, side=None):
    """Mean wall time (ms) of running `calls` (with `side`: the step's two-stream
    schedule, see run_calls), from HIP events on torch's current stream, after one
    untimed pass."""
    import torch
    run_calls(calls, side)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run_calls(calls, side)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def hbm_ceiling(nbytes=1 << 30, reps=5):
    """GB/s of the library's reference streaming kernel (moe_hbm_stream): a copy of
    nbytes (2 * nbytes moved), a read and a write of nbytes, median of reps launches
    each, timed with HIP events on torch's current stream."""
    import torch
    import dispatch_expert_gemm_amd as dm
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(dm.STREAM_SINK_BYTES, dtype=torch.uint8, device=dev)
    out = {}
    for mode, name, moved in ((0, "copy", 2 * nbytes), (1, "read", nbytes), (2, "write", nbytes)):
        times = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dm.moe_hbm_stream(mode, src, dst, nbytes, sink)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[f"{name}_GB/s"] = round(moved / (float(np.median(times[1:])) * 1e-3) / 1e9, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    out["kernel"] = f"moe_hbm_stream, {nbytes >> 20} MiB, per-workgroup ranges of 16-byte accesses"
    return out


def token_sweep(workload, tokens, steps):
    """fwd and fwd+bwd ms and TFLOP/s of the workload at other token counts (the
    columns of the Triton-distributed benchmark page's summary table), with the
    step's schedule."""
    import torch
    rows = []
    for T in tokens:
        st = build_step(workload, T)
        side = torch.cuda.Stream() if st.two_stream else None
        for _ in range(2):
            for _, fn in st.calls:
                fn()
        torch.cuda.synchronize()
        A = int(st.recv[-1].item())
        nf = [n for n, _ in st.calls].index("moe_combine") + 1
        fb = time_calls(st.calls, steps, side)
        fw = time_calls(st.calls[:nf], steps)
        H, F = st.config["H"], st.config["F"]
        rows.append({"T": T, "routed_rows": A, "fwd_ms": round(fw, 4), "fwd_bwd_ms": round(fb, 4),
                     "fwd_TFLOP/s": round(6 * A * H * F / (fw * 1e-3) / 1e12, 1),
                     "fwd_bwd_TFLOP/s": round(18 * A * H * F / (fb * 1e-3) / 1e12, 1)})
        del st
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: about 30 ms of warm-up steps at the page-1 size, so the timed
    # steps start at the GPU's working clocks (after the idle input generation,
    # the first few steps of a run measured 2-4% slower than the following ones)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="page1", choices=list(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="override T")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the cache-flushed re-timing of the bandwidth-bound kernels")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the page-1 rows at 1024, 2048 and 4096 tokens")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-kernel HBM ceiling")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB three times "
                         "(the reference kernel for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer here holds every expert on one device and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    st = build_step(args.workload, args.tokens)
    calls = st.calls

    side = torch.cuda.Stream() if st.two_stream else None  # default priority

    def step():
        run_calls(calls, side)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    A = int(st.recv[-1].item())
    assert int(st.err.item()) == 0

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
    extra = {}
    for name, fn in st.extra_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        extra[name] = {"ms": round(e0.elapsed_time(e1) / 10, 4)}

    # the forward alone: the step's calls up to and including combine, timed the same way
    fwd_ms = None
    if not st.cfg.get("combine_only") and not st.cfg.get("forward_only"):
        nf = [n for n, _ in calls].index("moe_combine") + 1
        fwd_ms = time_calls(calls[:nf], args.steps)

    fl, nb = account(st, A)
    combine_only = st.cfg.get("combine_only", False)
    kernels = {}
    # the GEMMs' algorithmic bytes: each GEMM is set against the roof it meets
    # first, its FLOPs at the MFMA peak or its bytes at the HBM peak
    Tq, Hq, Fq, Kq, Eq = st.shape_info
    gb = {k: gemm_bytes(k, A, Hq, Fq, Eq, Tq) for k in fl}
    for name, ms in per.items():
        rec = {"ms": round(ms, 4)}
        if name in fl:
            f, pk = fl[name]
            rec["TFLOP/s"] = round(f / (ms * 1e-3) / 1e12, 1)
            rec["frac_mfma"] = round(rec["TFLOP/s"] / pk, 4)
            if gb.get(name):
                rec["GB/s"] = round(gb[name] / (ms * 1e-3) / 1e9, 1)
                rec["frac_hbm"] = round(rec["GB/s"] / PEAK_HBM_GBS, 4)
                t_mfma, t_hbm = f / (pk * 1e12), gb[name] / (PEAK_HBM_GBS * 1e9)
                rec["bound"] = "hbm" if t_hbm > t_mfma else "mfma"
                rec["frac_roofline"] = round(max(t_mfma, t_hbm) / (ms * 1e-3), 4)
        if nb.get(name) is not None:
            rec["GB/s"] = round(nb[name] / (ms * 1e-3) / 1e9, 1)
            rec["frac_hbm"] = round(rec["GB/s"] / PEAK_HBM_GBS, 4)
        kernels[name] = rec
    # per-step durations from the event pass: mean, std and the mean without the
    # three slowest steps (the Megatron page's timing protocol)
    step_ms = sorted(ev[s][0].elapsed_time(ev[s][len(calls)]) for s in range(args.steps))
    kept = step_ms[:-3] if len(step_ms) > 3 else step_ms
    step_stats = {"mean": round(float(np.mean(step_ms)), 4), "std": round(float(np.std(step_ms)), 4),
                  "mean_without_3_slowest": round(float(np.mean(kept)), 4),
                  # a run whose step times spread more than 5% of their mean is flagged
                  "stable": bool(np.std(step_ms) <= 0.05 * np.mean(step_ms))}
    # the bandwidth-bound kernels once more in isolation, after writing a buffer
    # larger than the 256 MB Infinity Cache, so their inputs come from HBM
    isolated = {}
    if not args.no_isolated:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        # plus the dispatch permute of a step that folds it into the GEMMs
        aside = [(n, fn) for n, fn in st.extra_calls if n.startswith("moe_dispatch (")]
        nbi = dict(nb)
        for n, _ in aside:
            Ti, Hi, Fi, Ki, Ei = st.shape_info
            nbi[n] = bytes_moved("moe_dispatch", Ti, Hi, Fi, Ki, A, Ei)
        for name, fn in list(calls) + aside:
            if nbi.get(name) is None:
                continue
            times = []
            for _ in range(5):
                flush.zero_()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            isolated[name] = {"ms": round(ms, 4), "GB/s": round(nbi[name] / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(nbi[name] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del flush
    # layer roofline: every GEMM at its MFMA peak or at the HBM rate its
    # algorithmic bytes allow, whichever is slower, and every other kernel at HBM peak
    fwd_only = st.cfg.get("forward_only", False)
    t_ideal_ms = (sum(max(f / (pk * 1e12), gb.get(k, 0) / (PEAK_HBM_GBS * 1e9)) for k, (f, pk) in fl.items())
                  + sum(b / (PEAK_HBM_GBS * 1e9) for b in nb.values() if b is not None)) * 1e3
    T, H, F, E, K = (st.config[k] for k in ("T", "H", "F", "E", "K"))
    descr = {
        "page1": "Triton-distributed benchmark shape, dispatch permute folded into the gate/up GEMMs' row loads, "
                 "combine backward into the down GEMMs' row loads",
        "page1_permute": "Triton-distributed benchmark shape, dispatch permute as a kernel of its own, combine "
                         "backward folded into the down GEMMs' row loads",
        "page1_rank_share": "one of the Triton-distributed benchmark's four ranks: 16 local experts, 65,536 "
                            "received rows, dispatch permute folded into the gate/up GEMMs' row loads, "
                            "combine backward into the down GEMMs' row loads",
        "dsv3_proxy": "DeepSeek-V3-style proxy, Zipf(1.2) routing, one shared expert",
        "mixtral": "Mixtral-8x7B-style layer, fp8 e4m3 block-scaled GEMMs, int8 combine payload",
        "mixtral_grouped": "Mixtral-8x7B-style layer, fp8 e4m3 block-scaled GEMMs through the grouped fp8 "
                           "entries, int8 combine payload",
        "mixtral_mx": "Mixtral-8x7B-style layer, microscaled fp8 e4m3 GEMMs (E8M0 per 32, block-scaled MFMA), "
                      "int8 combine payload",
        "mixtral_fp8w": "Mixtral-8x7B-style layer, fp8 e4m3 block-scaled GEMMs including the weight "
                        "gradients (per-128-token operands), int8 combine payload",
        "combine_stress": "combine only, 256 routed + 1 zero + 1 copy + 2 constant experts, "
                          "2-D mask 10% false, shared_expert_x",
        "decode": "decode batch (the low_latency_combine page's largest BS), forward only",
        "decode_gather": "decode batch, forward only, dispatch folded into the gate/up GEMM's row loads",
        "decode_int8": "decode batch, forward only, int8 dispatch with smooth scales (quant_mode 2) and "
                       "w8a8 GEMMs",
    }[args.workload]
    fwd_only = st.cfg.get("forward_only", False)
    res = {
        "metric": "MoE layer fwd+bwd ms & TFLOP/s (% MFMA peak); combine GB/s (% HBM) at 1 GPU",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": st.dtype,
        "data": "synthetic",
    }
    if combine_only:
        comb = nb["moe_combine"] / (per["moe_combine"] * 1e-3) / 1e9
        res.update({
            "value": round(comb, 1), "unit": "GB/s",
            "config": {"workload": f"{descr}: T={T} tokens, H={H}, E={E}, top-{K}", "T": T, "H": H, "E": E,
                       "K": K, "routed_rows": A, "combine_bytes": nb["moe_combine"]},
            "roofline": {"bound": "hbm", "kernel": "moe_combine", "achieved": round(comb, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(comb / PEAK_HBM_GBS, 4),
                         "traffic": None},
        })
    else:
        total_flops = sum(f for f, _ in fl.values())
        dom = max(fl, key=lambda k: per[k])
        dflop, dpeak = fl[dom]
        achieved = dflop / (per[dom] * 1e-3) / 1e12
        gemm_ms = sum(per[k] for k in fl)
        ideal_ms = sum(f / (pk * 1e12) for f, pk in fl.values()) * 1e3
        roof_ms = sum(max(f / (pk * 1e12), gb.get(k, 0) / (PEAK_HBM_GBS * 1e9)) for k, (f, pk) in fl.items()) * 1e3
        config = {"workload": f"MoE layer {'forward' if fwd_only else 'fwd+bwd'}, {descr}: T={T} tokens, "
                              f"H={H}, F={F} SwiGLU, "
                              f"E={E} experts on one GPU, top-{K}",
                  "T": T, "H": H, "F": F, "E": E, "K": K, "routed_rows": A, "flop_per_step": total_flops}
        if st.two_stream:
            config["schedule"] = ("weight-gradient GEMMs on a second stream (per-kernel times and "
                                  "step_ms_events: one stream, each call bracketed by events)")
        if st.counts is not None:
            c = st.counts.cpu().numpy()
            config["expert_rows_max_over_mean"] = round(float(c.max() / max(c.mean(), 1e-9)), 3)
        res.update({
            "value": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "config": config,
            # the dominant kernel against the roof it meets first (its FLOPs at the
            # MFMA peak of its type, or its algorithmic bytes at the HBM peak)
            "roofline": ({"bound": "hbm", "kernel": dom,
                          "achieved": round(gb[dom] / (per[dom] * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(gb[dom] / (per[dom] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                         if kernels[dom].get("bound") == "hbm" else
                         {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                          "peak": dpeak, "unit": "TFLOP/s", "frac": round(achieved / dpeak, 4)}),
            "combine": ({"GB/s": kernels["moe_combine"]["GB/s"], "peak": PEAK_HBM_GBS,
                         "frac": kernels["moe_combine"]["frac_hbm"]} if "moe_combine" in kernels else None),
            "gemm_ms_per_step": round(gemm_ms, 4),
            "gemm_frac_of_mfma_roofline": round(ideal_ms / gemm_ms, 4),
            "gemm_frac_of_roofline": round(roof_ms / gemm_ms, 4),
        })
        res["roofline"]["traffic"] = (measured_traffic(dom) if args.workload == "page1" and not args.tokens
                                      else None)
    res["layer_roofline_frac"] = round(t_ideal_ms / ms_per_step, 4)
    res["step_ms_events"] = step_stats
    if fwd_ms is not None:
        res["fwd_ms"] = round(fwd_ms, 4)
    if not args.no_ceiling:
        log("[bench] HBM ceiling of the streaming kernel")
        ceil = hbm_ceiling()
        res["hbm_ceiling"] = ceil
        for rec in list(kernels.values()) + list(isolated.values()):
            if "GB/s" in rec:
                rec["frac_copy_ceiling"] = round(rec["GB/s"] / ceil["copy_GB/s"], 4)
    res["kernels"] = kernels
    if isolated:
        res["kernels_hbm_isolated"] = isolated
    if extra:
        res["outside_step"] = extra
    if args.workload in ("page1", "page1_rank_share"):
        res["context"] = {"page1_fwd_bwd_ms_4_nvidia_gpus_T8192": 5.488}
    if args.workload == "page1":
        if not args.no_sweep and not args.tokens:
            log("[bench] page-1 rows at 1024, 2048, 4096 tokens")
            res["token_rows"] = token_sweep("page1", (1024, 2048, 4096), max(args.steps // 2, 5))
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.no_cpu_baseline:
        pass
    elif combine_only:
        log("[bench] CPU oracle baseline (combine)")
        res["cpu_baseline"] = cpu_baseline_combine(st.cfg, args.cpu_seconds)
    elif st.cfg.get("fp8"):
        log("[bench] CPU oracle baseline (8-bit layer, F sample)")
        res["cpu_baseline"] = cpu_baseline_8bit(st.cfg, args.cpu_seconds)
    else:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(st.cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
