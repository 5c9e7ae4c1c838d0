"""GPU parity of the microscaled fp8 (MX) path: the MX quantisers bit-exact against the
oracle (codes and E8M0 scale bytes), the four MX GEMMs (block-scaled MFMA applying the
scales), each MX GEMM fed the oracle's operands at 2e-2 plus one bf16 ulp per
element (relative L2 <= 2e-3 for G and U, 2e-2 otherwise), and the whole chained
MX layer at the chained bar written out in gpu_util."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import (DEV, OUTLIERS_8BIT, REL_L2_8BIT, RHO_CHAIN, ULPS_KERNEL, Run, bf, check_close, check_equal, dev_rows,
                      f32, layer_mags)

pytestmark = pytest.mark.gpu

REL_FP8 = REL_L2_8BIT


def _u8(t):
    return t.detach().cpu().numpy()


def _rows_view(scale_bytes, R, C):
    """Device scale words (C/128 planes of R rows x 4 bytes) -> (R, C/32) scale bytes."""
    return np.asarray(scale_bytes).reshape(C // 128, R, 4).transpose(1, 0, 2).reshape(R, C // 32)


def test_quant_rows_mx_bit_exact():
    rng = np.random.default_rng(81)
    R, C = 75, 512
    a = (rng.standard_normal((R, C)) * np.exp2(rng.integers(-40, 40, size=(R, 1)))).astype(np.float32)
    a[3] = 0.0                                   # all-zero row
    a[5, 32:64] = 0.0                            # all-zero block
    a[7, :32] = 448.0                            # maximum exactly 448 * 2^0
    a[8, :32] = 449.0                            # just above: the next scale
    a[9] = rng.standard_normal(C) * 1e-39        # subnormal block maxima (scale clamps at 2^-127)
    a[10] = rng.standard_normal(C) * 3e36        # near the top of the bf16 range
    a[11, ::5] = -a[11, ::5]
    bits = orc.f32_to_bf16(a)
    codes, scales = dm.quant_rows_mx(bf(bits))
    torch.cuda.synchronize()
    q, s = orc.quant_mx_e4m3_rows(orc.bf16_to_f32(bits))
    check_equal("codes", _u8(codes), q)
    check_equal("scales", _rows_view(_u8(scales), R, C), s)
    # the device row count
    codes2 = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    scales2 = torch.full((R, C // 32), 0xCD, dtype=torch.uint8, device=DEV)
    dm.moe_quant_rows_mx(bf(bits), codes2, scales2, nrows=torch.tensor([30], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    check_equal("codes rows<30", _u8(codes2)[:30], q[:30])
    check_equal("scales rows<30", _rows_view(_u8(scales2), R, C)[:30], s[:30])
    assert (_u8(codes2)[30:] == 0xAB).all() and (_rows_view(_u8(scales2), R, C)[30:] == 0xCD).all()


def test_quantize_weights_mx_bit_exact():
    rng = np.random.default_rng(82)
    E, N, K = 3, 256, 384
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[1, :64, 128:160] = 0.0
    bits = wl.to_bf16_bits(w)
    m = dm.MxWeights.quantize(bf(bits))
    torch.cuda.synchronize()
    c, s, ct, st = orc.quant_weights_mx(bits)
    check_equal("codes", _u8(m.codes), c)
    check_equal("scales", _rows_view(_u8(m.scales), E * N, K).reshape(E, N, K // 32), s)
    check_equal("codes_t", _u8(m.codes_t), ct)
    check_equal("scales_t", _rows_view(_u8(m.scales_t), E * K, N).reshape(E, K, N // 32), st)


MX_CASES = {
    "small": dict(T=300, H=256, F=384, E=5, K=2),
    "ragged_rows": dict(T=517, H=512, F=256, E=7, K=3),
    "empty_experts": dict(T=40, H=128, F=128, E=12, K=1),
    "wide": dict(T=700, H=1024, F=640, E=3, K=2),
    "top1_768": dict(T=2496, H=768, F=768, E=4, K=1),
    # enough tiles for the eight-wave 256 x 256 MX tiles in the gate/up forward,
    # down forward and gate/up data gradient (a half last column tile at
    # H = 2176)
    "w256_ragged": dict(T=4096, H=2176, F=1024, E=4, K=2),
}


@pytest.mark.parametrize("name", list(MX_CASES))
def test_mx_grouped_ffn_forward_and_data_gradients(name):
    inp = wl.layer_inputs(seed=83, **MX_CASES[name])
    print(f"[mx] case={name}", flush=True)
    run = Run(inp)
    run.dispatch()
    F, H, cap = inp["F"], inp["H"], run.cap
    recv = run.d.ep_recv_counts
    nrows = recv[-1:]
    wq = [dm.MxWeights.quantize(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    xq, xs = dm.quant_rows_mx(run.d.expand_x, nrows)
    gus = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    h = torch.empty((cap, F), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    hq2 = torch.empty((cap, F), dtype=torch.uint8, device=DEV)
    hs2 = torch.empty((cap, F // 32), dtype=torch.uint8, device=DEV)
    dm.moe_ffn_gate_up_fwd_mx(run.shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales, recv, gus, h,
                              (hq2, hs2))
    hq, hs = dm.quant_rows_mx(h, nrows)
    dm.moe_ffn_down_fwd_mx(run.shape, hq, hs, wq[2].codes, wq[2].scales, recv, y)
    dY_bits = wl.to_bf16_bits(np.random.default_rng(84).standard_normal((cap, H), dtype=np.float32) * 0.125)
    dyq, dys = dm.quant_rows_mx(bf(dY_bits), nrows)
    ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    dgq2 = torch.empty((cap, 2 * F), dtype=torch.uint8, device=DEV)
    dgs2 = torch.empty((cap, 2 * F // 32), dtype=torch.uint8, device=DEV)
    dm.moe_ffn_down_bwd_data_mx(run.shape, dyq, dys, wq[2].codes_t, wq[2].scales_t, gus, recv, ggu, (dgq2, dgs2))
    dgq, dgs = dm.quant_rows_mx(ggu, nrows)
    gxe = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_gate_up_bwd_data_mx(run.shape, dgq, dgs, wq[0].codes_t, wq[0].scales_t, wq[1].codes_t,
                                   wq[1].scales_t, recv, gxe)
    torch.cuda.synchronize()
    r = orc.route(inp["topk_idx"], inp["E"])
    A = r.A
    # the codes fused into the GEMM epilogues equal the quantiser's on the same bf16 output
    check_equal("h codes (fused)", _u8(hq2)[:A], _u8(hq)[:A])
    check_equal("h scales (fused)", _rows_view(_u8(hs2), cap, F)[:A], _rows_view(_u8(hs), cap, F)[:A])
    check_equal("dGU codes (fused)", _u8(dgq2)[:A], _u8(dgq)[:A])
    check_equal("dGU scales (fused)", _rows_view(_u8(dgs2), cap, 2 * F)[:A], _rows_view(_u8(dgs), cap, 2 * F)[:A])
    X = orc.dispatch(inp["x"], r)
    owq = tuple(orc.quant_weights_mx(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    G, U, Hh, Y = orc.ffn_fwd_mx(X, r.ep_recv_counts, *owq)
    # G and U come from bit-identical codes and scales on both sides: only the fp32
    # accumulation order and the odd bf16 rounding differ, so a tight bar catches a
    # scale applied to the wrong 32-code block
    check_close("G", f32(gus[:A, :F]), G, ulps=ULPS_KERNEL, rel_l2=2e-3)
    check_close("U", f32(gus[:A, F:]), U, ulps=ULPS_KERNEL, rel_l2=2e-3)
    check_close("h", f32(h[:A]), Hh, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    dGU, dX, _, _, _ = orc.ffn_bwd_mx(orc.bf16_to_f32(dY_bits)[:A], X, G, U, Hh, r.ep_recv_counts, *owq)
    # the other three GEMMs fed the oracle's operands: the down GEMM the codes of the
    # oracle's h, the down data gradient the oracle's G|U, the gate/up data gradient
    # the codes of the oracle's dG|dU (the row quantiser is bit-exact, tested above)
    hq3, hs3 = dm.quant_rows_mx(dev_rows(Hh, cap), nrows)
    y3 = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_fwd_mx(run.shape, hq3, hs3, wq[2].codes, wq[2].scales, recv, y3)
    ggu3 = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_bwd_data_mx(run.shape, dyq, dys, wq[2].codes_t, wq[2].scales_t,
                                dev_rows(np.concatenate([G, U], 1), cap), recv, ggu3)
    dgq3, dgs3 = dm.quant_rows_mx(dev_rows(dGU, cap), nrows)
    gxe3 = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_gate_up_bwd_data_mx(run.shape, dgq3, dgs3, wq[0].codes_t, wq[0].scales_t, wq[1].codes_t,
                                   wq[1].scales_t, recv, gxe3)
    torch.cuda.synchronize()
    check_close("y", f32(y3[:A]), Y, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("grad_gate_up", f32(ggu3[:A]), dGU, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("grad_expand_x", f32(gxe3[:A]), dX, ulps=ULPS_KERNEL, rel_l2=REL_FP8)


def test_autograd_layer_mx():
    """moe_layer(fp8=True, mx=True, comm_quant_mode=2) against the oracle's MX layer."""
    inp = wl.layer_inputs(384, 256, 256, 6, 2, seed=85, mask="2d", Z=1)
    x = bf(inp["x"]).requires_grad_(True)
    w = torch.from_numpy(inp["topk_weights"]).to(DEV).requires_grad_(True)
    ws = [bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer(x, torch.from_numpy(inp["topk_idx"]).to(DEV), w, *ws,
                       x_active_mask=torch.from_numpy(inp["mask"]).to(DEV), zero_expert_num=1,
                       fp8=True, mx=True, comm_quant_mode=2)
    out.backward(bf(inp["grad_out"]))
    torch.cuda.synchronize()
    f = orc.layer_fwd_mx(inp)
    b = orc.layer_bwd_mx(inp, f, inp["grad_out"])
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_x", f32(x.grad), b["dx"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_topk_weights", f32(w.grad), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    for t, k in zip(ws, ("dWg", "dWu", "dWd")):
        check_close(k, f32(t.grad), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN, rel_l2=REL_FP8)


def test_mx_layer_with_empty_and_single_row_experts():
    """Most experts without rows, one with a single row (a 1-row tile with clamped
    loads), through the MX autograd layer."""
    inp = wl.layer_inputs(seed=86, T=3, H=256, F=128, E=16, K=1)
    inp["topk_idx"] = np.array([[5], [5], [11]], np.int32)
    x = bf(inp["x"]).requires_grad_(True)
    w = torch.from_numpy(inp["topk_weights"]).to(DEV).requires_grad_(True)
    ws = [bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer(x, torch.from_numpy(inp["topk_idx"]).to(DEV), w, *ws, fp8=True, mx=True)
    out.backward(bf(inp["grad_out"]))
    torch.cuda.synchronize()
    f = orc.layer_fwd_mx(inp, comm_quant=False)
    b = orc.layer_bwd_mx(inp, f, inp["grad_out"])
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_x", f32(x.grad), b["dx"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    for t, k in zip(ws, ("dWg", "dWu", "dWd")):
        check_close(k, f32(t.grad), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN, rel_l2=REL_FP8)
