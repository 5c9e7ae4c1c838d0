"""The fp8 layer through its boundary entries: moe_dispatch_fp8 (the permute writes
the e4m3 rows and their scales), moe_grouped_ffn_fp8, moe_combine_bwd_fp8 (dY's
codes from the combine backward) and moe_grouped_ffn_bwd_fp8.  The fused codes
equal the row quantiser's on the same bf16 values bit for bit (and the
quantiser is bit-exact against the oracle in test_gpu_fp8.py); the grouped
entries equal the single-GEMM chain they are made of bit for bit, and the whole
step matches the oracle's fp8 layer at the chained 8-bit bar."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import (DEV, OUTLIERS_8BIT, REL_L2_8BIT, RHO_CHAIN, Run, bf, check_close, check_equal, f32,
                      layer_mags)

pytestmark = pytest.mark.gpu

CASES = {
    "small_masked_special": dict(T=300, H=256, F=384, E=5, K=2, Z=1, C=1, mask="2d"),
    "ragged_rows_k3": dict(T=517, H=512, F=256, E=7, K=3),
    "empty_experts": dict(T=40, H=128, F=128, E=12, K=1),
    "k8_wide": dict(T=640, H=1024, F=512, E=16, K=8),
}


def _u8(t):
    return t.detach().cpu().numpy()


def _step(inp):
    """The fp8 step through the boundary entries (int8 combine payload)."""
    run = Run(inp)
    shape = run.shape
    shape.comm_quant_mode = 2
    cap, T, H, F, E, K = run.cap, run.T, run.H, inp["F"], inp["E"], run.K
    z = lambda *sh, dt=torch.bfloat16: torch.empty(sh, dtype=dt, device=DEV)
    ex, exq, exs = z(cap, H), z(cap, H, dt=torch.uint8), z(H // 128, cap, dt=torch.float32)
    assist, cnt, recv, err = z(dm.moe_assist_info_size(shape), dt=torch.int32), z(E, dt=torch.int32), \
        z(E, dt=torch.int32), z(1, dt=torch.int32)
    ws = z(dm.moe_workspace_size(shape), dt=torch.uint8)
    dm.moe_dispatch_fp8(shape, run.x, run.idx, run.mask, ex, exq, exs, assist, cnt, recv, err, ws)
    wq = [dm.Fp8Weights.quantize(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    wsf = z(dm.moe_ffn_fp8_workspace_size(shape), dt=torch.uint8)
    gus, h, y, out = z(cap, 2 * F), z(cap, F), z(cap, H), z(T, H)
    dm.moe_grouped_ffn_fp8(shape, exq, exs, wq, recv, gus, h, y, wsf)
    dm.moe_combine(shape, y, run.idx, run.w, assist, recv, run.mask, None, run.x, run.a1, run.a2, run.cv, out)
    g = bf(inp["grad_out"])
    gy, gyq, gys, gw = z(cap, H), z(cap, H, dt=torch.uint8), z(H // 128, cap, dt=torch.float32), \
        z(T, K, dt=torch.float32)
    dm.moe_combine_bwd_fp8(shape, g, y, run.idx, run.w, assist, recv, run.mask, run.x, run.a1, run.a2, run.cv,
                           gy, gyq, gys, gw)
    ggu, gxe, gx = z(cap, 2 * F), z(cap, H), z(T, H)
    gwg, gwu, gwd = z(E, F, H, dt=torch.float32), z(E, F, H, dt=torch.float32), z(E, H, F, dt=torch.float32)
    dm.moe_grouped_ffn_bwd_fp8(shape, gy, gyq, gys, ex, gus, h, wq, recv, ggu, gxe, gwg, gwu, gwd, wsf)
    dm.moe_dispatch_bwd(shape, gxe, assist, run.idx, run.w, run.mask, g, run.a1, None, gx)
    torch.cuda.synchronize()
    return dict(run=run, shape=shape, ex=ex, exq=exq, exs=exs, assist=assist, recv=recv, err=err, wq=wq, gus=gus,
                h=h, y=y, out=out, gy=gy, gyq=gyq, gys=gys, gw=gw, ggu=ggu, gxe=gxe, gx=gx, gwg=gwg, gwu=gwu,
                gwd=gwd)


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_boundary_step(name):
    inp = wl.layer_inputs(seed=71, **CASES[name])
    print(f"[fp8 boundary] case={name}", flush=True)
    s = _step(inp)
    run, shape, recv = s["run"], s["shape"], s["recv"]
    r = orc.route(inp["topk_idx"], inp["E"], inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0), inp.get("mask"))
    A, F, H = r.A, inp["F"], inp["H"]
    assert int(s["err"].item()) == 0 and int(recv[-1].item()) == A
    # the dispatch's bf16 rows and maps equal moe_dispatch's
    d = dm.dispatch(run.shape, run.x, run.idx, run.mask)
    torch.cuda.synchronize()
    assert torch.equal(s["ex"][:A].view(torch.int16), d.expand_x[:A].view(torch.int16))
    TK = run.T * run.K
    assert torch.equal(s["assist"][:TK + A], d.assist_info_for_combine[:TK + A])
    # fused codes = the row quantiser on the same bf16 values
    nrows = recv[-1:]
    for name_, src, q, sc in (("x", s["ex"], s["exq"], s["exs"]), ("dY", s["gy"], s["gyq"], s["gys"])):
        q2, s2 = dm.quant_rows_fp8(src, nrows)
        torch.cuda.synchronize()
        check_equal(f"{name_} codes", _u8(q)[:A], _u8(q2)[:A])
        check_equal(f"{name_} scales", s2.cpu().numpy()[:, :A], sc.cpu().numpy()[:, :A])
    # ... and the oracle's quantiser on the oracle's rows
    X = orc.dispatch(inp["x"], r)
    qo, so = orc.quant_e4m3_rows(X)
    check_equal("x codes vs oracle", _u8(s["exq"])[:A], qo)
    check_equal("x scales vs oracle", s["exs"].cpu().numpy()[:, :A].T, so)
    # the grouped entries equal their single-GEMM chain bit for bit
    cap = run.cap
    wg, wu, wd = s["wq"]
    gus2, h2, y2 = (torch.empty_like(t) for t in (s["gus"], s["h"], s["y"]))
    dm.moe_ffn_gate_up_fwd_fp8(shape, s["exq"], s["exs"], wg.codes, wg.scales, wu.codes, wu.scales, recv, gus2, h2)
    hq, hs = dm.quant_rows_fp8(h2, nrows)
    dm.moe_ffn_down_fwd_fp8(shape, hq, hs, wd.codes, wd.scales, recv, y2)
    ggu2 = torch.empty_like(s["ggu"])
    dgq = torch.empty((cap, 2 * F), dtype=torch.uint8, device=DEV)
    dgs = torch.empty((2 * F // 128, cap), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_data_fp8_quant(shape, s["gyq"], s["gys"], wd.codes_t, wd.scales, s["gus"], recv, ggu2,
                                       (dgq, dgs))
    gxe2 = torch.empty_like(s["gxe"])
    dm.moe_ffn_gate_up_bwd_data_fp8(shape, dgq, dgs, wg.codes_t, wg.scales, wu.codes_t, wu.scales, recv, gxe2)
    torch.cuda.synchronize()
    for nm, a_, b_ in (("gate_up_save", s["gus"], gus2), ("h", s["h"], h2), ("y", s["y"], y2),
                       ("grad_gate_up", s["ggu"], ggu2), ("grad_expand_x", s["gxe"], gxe2)):
        assert torch.equal(a_[:A].view(torch.int16), b_[:A].view(torch.int16)), f"{nm} differs from the chain"
    # the whole step against the oracle's fp8 layer (chained 8-bit bar)
    f = orc.layer_fwd_fp8(inp)
    b = orc.layer_bwd_fp8(inp, f, inp["grad_out"])
    m = layer_mags(inp, f, b)
    check_close("out", f32(s["out"]), f["out"], rel_l2=REL_L2_8BIT, outliers=OUTLIERS_8BIT)
    check_close("grad_topk_weights", f32(s["gw"]), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN, rel_l2=REL_L2_8BIT)
    check_close("grad_x", f32(s["gx"]), b["dx"], rel_l2=REL_L2_8BIT, outliers=OUTLIERS_8BIT)
    for k, t in (("dWg", s["gwg"]), ("dWu", s["gwu"]), ("dWd", s["gwd"])):
        check_close(k, f32(t), b[k], ulps=0, mag=m[k], rho=RHO_CHAIN, rel_l2=REL_L2_8BIT)
