"""GPU parity of the dispatch-fused gate/up forward: moe_route (the routing alone)
then moe_ffn_gate_up_fwd_gather, which reads each expanded row straight from x
through the row -> slot map.  The routing outputs equal moe_dispatch's and the
GEMM outputs equal moe_ffn_gate_up_fwd's on the permuted rows bit for bit (same
operand values, same tiles and accumulation order); the small cases are also
checked against the oracle's expert FFN."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import DEV, ULPS_KERNEL, Run, bf, check_close, check_equal, f32

pytestmark = pytest.mark.gpu

CASES = {
    "small_masked_zero": dict(T=300, H=256, F=128, E=6, K=2, mask="2d", Z=1),
    "ragged_tiles": dict(T=77, H=384, F=160, E=5, K=3),
    "one_token": dict(T=1, H=128, F=64, E=4, K=2),
    "page1_shape": dict(T=8192, H=1536, F=480, E=64, K=8),
    "decode_shape": dict(T=512, H=7168, F=2048, E=32, K=8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gather_gate_up_matches_permuted(name):
    cfg = CASES[name]
    print(f"[gather] case={name}", flush=True)
    inp = wl.layer_inputs(seed=91, **cfg)
    run = Run(inp)
    d = run.dispatch()
    shape, cap, F, H = run.shape, run.cap, inp["F"], inp["H"]
    assist = torch.full_like(d.assist_info_for_combine, -7)
    etn, recv = torch.empty_like(d.expert_token_nums), torch.empty_like(d.ep_recv_counts)
    err = torch.empty_like(d.err_flag)
    ws = torch.empty(dm.moe_workspace_size(shape), dtype=torch.uint8, device=DEV)
    dm.moe_route(shape, run.idx, run.mask, assist, etn, recv, err, ws)
    wg, wu = bf(inp["w_gate"]), bf(inp["w_up"])
    gus1, h1 = (torch.empty((cap, n), dtype=torch.bfloat16, device=DEV) for n in (2 * F, F))
    gus2, h2 = (torch.empty((cap, n), dtype=torch.bfloat16, device=DEV) for n in (2 * F, F))
    dm.moe_ffn_gate_up_fwd(shape, d.expand_x, wg, wu, d.ep_recv_counts, gus1, h1)
    dm.moe_ffn_gate_up_fwd_gather(shape, run.x, assist, wg, wu, recv, gus2, h2)
    torch.cuda.synchronize()
    A = run.A
    TK = run.T * run.K
    check_equal("assist", assist[:TK + A].cpu().numpy(), d.assist_info_for_combine[:TK + A].cpu().numpy())
    check_equal("ep_recv_counts", recv.cpu().numpy(), d.ep_recv_counts.cpu().numpy())
    check_equal("expert_token_nums", etn.cpu().numpy(), d.expert_token_nums.cpu().numpy())
    check_equal("err_flag", err.cpu().numpy(), d.err_flag.cpu().numpy())
    assert torch.equal(gus1[:A], gus2[:A]), "gate_up_save differs from the permuted path"
    assert torch.equal(h1[:A], h2[:A]), "h_act differs from the permuted path"
    if inp["T"] * inp["H"] <= 300 * 384:
        r = orc.route(inp["topk_idx"], inp["E"], Z=cfg.get("Z", 0), mask=inp.get("mask"))
        G, U, Hh, _ = orc.ffn_fwd(orc.dispatch(inp["x"], r), r.ep_recv_counts, inp["w_gate"], inp["w_up"],
                                  inp["w_down"])
        check_close("G", f32(gus2[:A, :F]), G, ulps=ULPS_KERNEL)
        check_close("U", f32(gus2[:A, F:]), U, ulps=ULPS_KERNEL)
        check_close("h", f32(h2[:A]), Hh, ulps=ULPS_KERNEL)


WGRAD_CASES = {
    "small_masked_zero": dict(T=300, H=256, F=128, E=6, K=2, mask="2d", Z=1),
    "ragged_tiles_k3": dict(T=77, H=384, F=160, E=5, K=3),
    "k5_many_experts": dict(T=900, H=264, F=96, E=33, K=5),
    "empty_experts": dict(T=20, H=64, F=32, E=16, K=1),
    "one_token": dict(T=1, H=128, F=64, E=4, K=2),
    "page1_shape": dict(T=8192, H=1536, F=480, E=64, K=8),
    "k16_long_experts": dict(T=1500, H=512, F=256, E=20, K=16),
    # 2F x H = 2048 x 2048: the eight-wave 256 x 256 weight-gradient tiles
    "wide_256_tiles": dict(T=301, H=2048, F=1024, E=2, K=2),
    # the same tiles with a partial last row tile (2F = 1984) and an 8-column
    # last column tile (H = 2056)
    "wide_256_ragged": dict(T=257, H=2056, F=992, E=3, K=2),
}


@pytest.mark.parametrize("name", list(WGRAD_CASES))
def test_gather_gate_up_weight_gradient_matches_permuted(name):
    """moe_ffn_gate_up_bwd_weight_gather (x rows through the row -> slot map) equals
    moe_ffn_gate_up_bwd_weight on moe_dispatch's expand_x bit for bit; the small
    cases are also checked against the oracle's weight gradient."""
    cfg = WGRAD_CASES[name]
    print(f"[gather wgrad] case={name}", flush=True)
    inp = wl.layer_inputs(seed=93, **cfg)
    run = Run(inp)
    d = run.dispatch()
    shape, cap, F, H, E = run.shape, run.cap, inp["F"], inp["H"], inp["E"]
    rng = np.random.default_rng(94)
    dgu_bits = wl.to_bf16_bits(rng.standard_normal((cap, 2 * F), dtype=np.float32) * 0.1)
    dgu = bf(dgu_bits)
    w1 = [torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    w2 = [torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    dm.moe_ffn_gate_up_bwd_weight(shape, dgu, d.expand_x, d.ep_recv_counts, *w1)
    dm.moe_ffn_gate_up_bwd_weight_gather(shape, dgu, run.x, d.assist_info_for_combine, d.ep_recv_counts, *w2)
    torch.cuda.synchronize()
    assert torch.equal(w1[0], w2[0]) and torch.equal(w1[1], w2[1]), "differs from the permuted path"
    if inp["T"] * inp["H"] <= 1500 * 512:
        r = orc.route(inp["topk_idx"], E, Z=cfg.get("Z", 0), mask=inp.get("mask"))
        X = orc.dispatch(inp["x"], r)
        dG = orc.bf16_to_f32(dgu_bits)[:r.A]
        ref = np.zeros((E, 2 * F, H))
        lo = 0
        for e in range(E):
            hi = int(r.ep_recv_counts[e])
            ref[e] = dG[lo:hi].astype(np.float64).T @ X[lo:hi].astype(np.float64)
            lo = hi
        check_close("grad_w_gate", f32(w2[0]), ref[:, :F], ulps=0)
        check_close("grad_w_up", f32(w2[1]), ref[:, F:], ulps=0)
