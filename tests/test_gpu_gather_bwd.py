"""GPU parity of the combine backward folded into the down GEMMs' operand loads:
moe_combine_bwd_weights (the routing weights' gradient and each routed row's
routing weight, no grad_y) then moe_ffn_down_bwd_data_gather and
moe_ffn_down_bwd_weight_gather, which read grad_out rows through the row -> slot
map.  The weights' gradient and the down weight gradient (grad_y rows formed in
registers as bf16(w * grad_out)) equal the path through moe_combine_bwd's grad_y
bit for bit; the down data gradient applies each row's weight to its fp32
product with W_down (one rounding fewer than the grad_y path) and is held to the
element-wise parity bar against that path and against the oracle's
w * (grad_out W_down) followed by the SwiGLU backward."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import DEV, ULPS_CHAIN, ULPS_KERNEL, Run, bf, check_close, check_equal, f32

pytestmark = pytest.mark.gpu

CASES = {
    "small_masked_zero": dict(T=300, H=256, F=128, E=6, K=2, mask="2d", Z=1),
    "copy_const_k3": dict(T=77, H=384, F=160, E=5, K=3, C=1, Q=1),
    "k5_many_experts": dict(T=900, H=264, F=96, E=33, K=5),
    "empty_experts": dict(T=20, H=64, F=32, E=16, K=1),
    "one_token": dict(T=1, H=128, F=64, E=4, K=2),
    "mask1d_k16": dict(T=600, H=512, F=256, E=20, K=16, mask="1d"),
    # F >= 1024: the down data gradient on 128 x 256 tiles
    "wide_f": dict(T=301, H=512, F=1024, E=3, K=2),
    "page1_shape": dict(T=8192, H=1536, F=480, E=64, K=8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gathered_down_backward_matches_grad_y_path(name):
    cfg = CASES[name]
    print(f"[gather bwd] case={name}", flush=True)
    inp = wl.layer_inputs(seed=97, mask_active=cfg["T"] // 2 if cfg.get("mask") == "1d" else None, **cfg)
    run = Run(inp)
    d = run.dispatch()
    run.ffn()
    shape, cap, F, H, E, T, K = run.shape, run.cap, inp["F"], inp["H"], inp["E"], run.T, run.K
    A = run.A
    g = bf(inp["grad_out"])
    # the path through grad_y
    gy, gw = run.combine_bwd(g)
    ggu1 = torch.full((cap, 2 * F), float("nan"), dtype=torch.bfloat16, device=DEV)
    gwd1 = torch.full((E, H, F), float("nan"), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_data(shape, gy, run.wd, run.gus, d.ep_recv_counts, ggu1)
    dm.moe_ffn_down_bwd_weight(shape, gy, run.h, d.ep_recv_counts, gwd1)
    # the gathered path
    gw2 = torch.full_like(gw, float("nan"))
    roww = torch.full((cap,), float("nan"), dtype=torch.float32, device=DEV)
    ggu2 = torch.full_like(ggu1, float("nan"))
    gwd2 = torch.full_like(gwd1, float("nan"))
    assist = d.assist_info_for_combine
    dm.moe_combine_bwd_weights(shape, g, run.y, run.idx, run.w, assist, d.ep_recv_counts, run.mask, run.x,
                               run.a1, run.a2, run.cv, gw2, roww)
    dm.moe_ffn_down_bwd_data_gather(shape, g, assist, roww, run.wd, run.gus, d.ep_recv_counts, ggu2)
    dm.moe_ffn_down_bwd_weight_gather(shape, g, assist, roww, run.h, d.ep_recv_counts, gwd2)
    torch.cuda.synchronize()
    assert torch.equal(gw2, gw), "grad_topk_weights differs from moe_combine_bwd"
    # row weights: the routing weight of each routed row's slot
    row2slot = assist[T * K:T * K + A].cpu().numpy()
    check_equal("row_weights", roww[:A].cpu().numpy(), inp["topk_weights"].reshape(-1)[row2slot])
    # the row weights alone (no weights' gradient, y not passed)
    roww3 = torch.full_like(roww, float("nan"))
    dm.moe_combine_bwd_weights(shape, g, None, run.idx, run.w, assist, d.ep_recv_counts, run.mask, run.x,
                               run.a1, run.a2, run.cv, None, roww3)
    torch.cuda.synchronize()
    assert torch.equal(roww3[:A], roww[:A])
    assert torch.equal(gwd2, gwd1), "grad_w_down differs from the grad_y path"
    check_close("grad_gate_up against the grad_y path", f32(ggu2[:A]), f32(ggu1[:A]), ulps=ULPS_CHAIN)
    if T * H <= 900 * 384:
        # the oracle's down backward on its own grad_y (the combine backward's rows)
        r = orc.route(inp["topk_idx"], E, Z=cfg.get("Z", 0), C=cfg.get("C", 0), Q=cfg.get("Q", 0),
                      mask=inp.get("mask"))
        dY = f32(gy[:A])
        Hh = f32(run.h[:A])
        ref = np.zeros((E, H, F))
        lo = 0
        for e in range(E):
            hi = int(r.ep_recv_counts[e])
            ref[e] = dY[lo:hi].astype(np.float64).T @ Hh[lo:hi].astype(np.float64)
            lo = hi
        check_close("grad_w_down", f32(gwd2), ref, ulps=0)
        lo = 0
        gus = f32(run.gus[:A]).astype(np.float64)
        dgu = np.zeros((A, 2 * F))
        Wd = orc.bf16_to_f32(inp["w_down"]).astype(np.float64)
        G = orc.bf16_to_f32(inp["grad_out"]).astype(np.float64)
        tok = row2slot // K
        wr = inp["topk_weights"].reshape(-1)[row2slot].astype(np.float64)
        for e in range(E):
            hi = int(r.ep_recv_counts[e])
            dh = wr[lo:hi, None] * (G[tok[lo:hi]] @ Wd[e])
            gg, uu = gus[lo:hi, :F], gus[lo:hi, F:]
            sg = 1.0 / (1.0 + np.exp(-gg))
            dgu[lo:hi, :F] = dh * uu * sg * (1 + gg * (1 - sg))
            dgu[lo:hi, F:] = dh * gg * sg
            lo = hi
        check_close("grad_gate_up", f32(ggu2[:A]), dgu, ulps=ULPS_KERNEL)


def test_gathered_down_backward_rejects_bad_arguments():
    inp = wl.layer_inputs(seed=98, T=16, H=64, F=32, E=4, K=2)
    run = Run(inp)
    d = run.dispatch()
    run.ffn()
    g = bf(inp["grad_out"])
    roww = torch.empty(run.cap, dtype=torch.float32, device=DEV)
    with pytest.raises(dm.MoeError):   # row_weights missing
        dm.moe_combine_bwd_weights(run.shape, g, run.y, run.idx, run.w, d.assist_info_for_combine,
                                   d.ep_recv_counts, None, run.x, None, None, None,
                                   torch.empty((16, 2), dtype=torch.float32, device=DEV), None)
    with pytest.raises(dm.MoeError):   # too short
        dm.moe_ffn_down_bwd_data_gather(run.shape, g, d.assist_info_for_combine, roww[:3], run.wd, run.gus,
                                        d.ep_recv_counts, torch.empty_like(run.gus))
