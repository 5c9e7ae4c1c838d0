"""Whole-layer parity (dispatch, grouped FFN, combine and their backward through the
C entries) on seeded random layer shapes, against the oracle in parity mode.

The shapes are drawn once from a fixed seed so the suite is reproducible; they mix
ragged H (a multiple of 8) and F (a multiple of 32), expert counts from 1 to 96,
top-k from 1 to 8, zero/copy/constant experts and masks, and token counts large
enough that some draws select the 256 x 256 forward tiles, the grouped tile order
and the staggered K starts of the GEMMs (which of them is taken depends on the
shape, as in production).  A second set draws fp8 layers (H and F multiples of
128, int8 combine payload) against the oracle's fp8 layer."""
import numpy as np
import pytest

import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import DEV, Fp8Run, Run, bf, check_close, f32

pytestmark = pytest.mark.gpu


def _draw(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        big = i % 3 == 0
        if big:   # many tiles: the tile choices that only pay on large layers
            E = int(rng.choice([3, 8, 16]))
            K = int(rng.integers(1, 4))
            T = int(rng.integers(4000, 8000))
            H = int(8 * rng.integers(32, 73))
            F = int(32 * rng.integers(8, 19))
        else:
            E = int(rng.choice([1, 3, 8, 16, 33, 96]))
            K = int(min(rng.integers(1, 9), E + 4))
            T = int(rng.integers(1, 700))
            H = int(8 * rng.integers(2, 160))
            F = int(32 * rng.integers(1, 24))
        kw = dict(T=T, H=H, F=F, E=E, K=K)
        if rng.random() < 0.4:
            kw.update(Z=int(rng.integers(0, 2)), C=int(rng.integers(0, 2)), Q=int(rng.integers(0, 3)), mask="2d")
        # top-k takes distinct ids: at most the routed plus special experts
        kw["K"] = min(kw["K"], E + kw.get("Z", 0) + kw.get("C", 0) + kw.get("Q", 0))
        cases.append(kw)
    return cases


CASES = _draw(9)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_random_layer_shapes(idx):
    kw = CASES[idx]
    print(f"[random] case={idx} {kw}", flush=True)
    inp = wl.layer_inputs(seed=100 + idx, **kw)
    run = Run(inp)
    run.dispatch()
    run.ffn()
    out = run.combine()
    g = bf(inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe, gwg, gwu, gwd = run.ffn_bwd(gy)
    gx = run.dispatch_bwd(gxe, g)
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    A = f["route"].A
    assert run.A == A
    check_close("out", f32(out), f["out"])
    check_close("grad_topk_weights", f32(gw), b["dw"])
    check_close("grad_gate_up", f32(ggu[:A]), b["dGU"])
    check_close("grad_x", f32(gx), b["dx"])
    check_close("grad_w_gate", f32(gwg), b["dWg"])
    check_close("grad_w_up", f32(gwu), b["dWu"])
    check_close("grad_w_down", f32(gwd), b["dWd"])


def _draw_fp8(n, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 4, 8, 24]))
        K = int(min(rng.integers(1, 5), E + 2))
        T = int(rng.integers(1, 3000))
        H = int(128 * rng.integers(1, 9))
        F = int(128 * rng.integers(1, 7))
        kw = dict(T=T, H=H, F=F, E=E, K=K)
        if rng.random() < 0.4:
            kw.update(Z=int(rng.integers(0, 2)), C=int(rng.integers(0, 2)), mask="2d")
        kw["K"] = min(kw["K"], E + kw.get("Z", 0) + kw.get("C", 0))
        cases.append(kw)
    return cases


FP8_CASES = _draw_fp8(5)
REL_FP8 = 2e-2


@pytest.mark.parametrize("idx", range(len(FP8_CASES)))
def test_random_fp8_layer_shapes(idx):
    kw = FP8_CASES[idx]
    print(f"[random fp8] case={idx} {kw}", flush=True)
    inp = wl.layer_inputs(seed=200 + idx, **kw)
    run = Fp8Run(inp)
    run.shape.comm_quant_mode = 2
    run.dispatch()
    run.quant_weights()
    run.ffn8()
    out = run.combine()
    g = bf(inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe = run.ffn8_bwd_data(gy)
    E, F, H = inp["E"], inp["F"], inp["H"]
    gwg = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
    gwu = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
    gwd = torch.empty((E, H, F), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_weight(run.shape, gy, run.h, run.d.ep_recv_counts, gwd)
    dm.moe_ffn_gate_up_bwd_weight(run.shape, ggu, run.d.expand_x, run.d.ep_recv_counts, gwg, gwu)
    gx = run.dispatch_bwd(gxe, g)
    f = orc.layer_fwd_fp8(inp)
    b = orc.layer_bwd_fp8(inp, f, inp["grad_out"])
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8)
    check_close("grad_topk_weights", f32(gw), b["dw"], rel_l2=REL_FP8)
    check_close("grad_x", f32(gx), b["dx"], rel_l2=REL_FP8)
    check_close("grad_w_gate", f32(gwg), b["dWg"], rel_l2=REL_FP8)
    check_close("grad_w_up", f32(gwu), b["dWu"], rel_l2=REL_FP8)
    check_close("grad_w_down", f32(gwd), b["dWd"], rel_l2=REL_FP8)
