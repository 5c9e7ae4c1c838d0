"""GPU parity of the int8 path (the decode regime's quant_mode 2): int8 dispatch with
optional per-expert smooth scales and the int8 row quantiser bit-exact against the
oracle; the w8a8 grouped GEMMs fed the oracle's operands within 2e-2 plus one bf16
ulp per element, and the whole decode forward at the chained bar written out in
gpu_util (relative L2 <= 2e-2 throughout)."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import DEV, OUTLIERS_8BIT, REL_L2_8BIT, ULPS_KERNEL, Run, bf, check_close, check_equal, dev, dev_rows, f32

pytestmark = pytest.mark.gpu

REL_8BIT = REL_L2_8BIT


def _smooth(E, H, seed):
    # positive per-channel factors around 1 (a smooth-quant pre-scale)
    return np.exp(np.random.default_rng(seed).standard_normal((E, H)) * 0.5).astype(np.float32)


DISPATCH_CASES = {
    "plain": dict(T=300, H=256, E=8, K=2),
    "special_masked": dict(T=257, H=512, E=6, K=4, Z=1, C=1, Q=1, mask="2d"),
    "ragged_H": dict(T=99, H=200, E=5, K=3),
    "max_H": dict(T=33, H=8192, E=4, K=2),
    "decode": dict(T=512, H=7168, E=32, K=8),
}


@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("name", list(DISPATCH_CASES))
def test_dispatch_int8_bit_exact(name, smooth):
    kw = DISPATCH_CASES[name]
    print(f"[int8 dispatch] case={name} smooth={smooth}", flush=True)
    inp = wl.layer_inputs(seed=61, weights=False, F=0, **kw)
    E, H = kw["E"], kw["H"]
    S = _smooth(E, H, 62) if smooth else None
    run = Run(inp)
    run.dispatch()   # the bf16 dispatch: its maps and counts must be the same
    d, dyn = dm.dispatch_int8(run.shape, run.x, run.idx, run.mask,
                              None if S is None else torch.from_numpy(S).to(DEV))
    torch.cuda.synchronize()
    r = orc.route(inp["topk_idx"], E, kw.get("Z", 0), kw.get("C", 0), kw.get("Q", 0), inp.get("mask"))
    q, s = orc.dispatch_int8(inp["x"], r, S)
    A, TK = r.A, kw["T"] * kw["K"]
    # slot2row and the used part of row2slot (the rest of the buffer is never written)
    got, ref = d.assist_info_for_combine.cpu().numpy(), run.d.assist_info_for_combine.cpu().numpy()
    check_equal("assist", got[:TK + A], ref[:TK + A])
    check_equal("ep_recv_counts", d.ep_recv_counts.cpu().numpy(), run.d.ep_recv_counts.cpu().numpy())
    check_equal("expand_x codes", d.expand_x.cpu().numpy()[:A], q)
    check_equal("dynamic_scales", dyn.cpu().numpy()[:A], s)


def test_quant_rows_int8_bit_exact():
    rng = np.random.default_rng(63)
    R, C = 77, 1000
    a = rng.standard_normal((R, C)).astype(np.float32)
    a[3] = 0.0
    a[5] *= 1e-30
    a[9] *= 1e4
    a[11, ::3] = 0.0
    bits = wl.to_bf16_bits(a)
    codes, scales = dm.quant_rows_int8(bf(bits))
    codes2 = torch.full((R, C), 77, dtype=torch.int8, device=DEV)
    scales2 = torch.zeros(R, dtype=torch.float32, device=DEV)
    dm.moe_quant_rows_int8(bf(bits), codes2, scales2, nrows=torch.tensor([40], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    q, s = orc.quant_int8_rows(orc.bf16_to_f32(bits))
    check_equal("codes", codes.cpu().numpy(), q)
    check_equal("scales", scales.cpu().numpy(), s)
    check_equal("codes rows<40", codes2.cpu().numpy()[:40], q[:40])
    assert (codes2.cpu().numpy()[40:] == 77).all()


FFN_CASES = {
    "small": dict(T=300, H=256, F=384, E=5, K=2),
    "ragged_rows": dict(T=517, H=512, F=256, E=7, K=3),
    "empty_experts": dict(T=40, H=128, F=128, E=12, K=1),
}


def _int8_forward(inp, S=None):
    """dispatch_int8 -> w8a8 gate/up -> int8 h -> w8a8 down -> bf16 combine, through the C entries."""
    H, F = inp["H"], inp["F"]
    run = Run(inp)
    shape, cap = run.shape, run.cap
    run.d, dyn = dm.dispatch_int8(shape, run.x, run.idx, run.mask,
                                  None if S is None else torch.from_numpy(S).to(DEV))
    wq = [dm.quant_rows_int8(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    gus = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    h = torch.empty((cap, F), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    recv = run.d.ep_recv_counts
    dm.moe_ffn_gate_up_fwd_int8(shape, run.d.expand_x, dyn, wq[0][0], wq[0][1], wq[1][0], wq[1][1], recv, gus, h)
    hq, hs = dm.quant_rows_int8(h, recv[-1:])
    dm.moe_ffn_down_fwd_int8(shape, hq, hs, wq[2][0], wq[2][1], recv, y)
    out = run.combine(y=y)
    return dict(gus=gus, h=h, y=y, out=out, wq=wq)


@pytest.mark.parametrize("name", list(FFN_CASES))
def test_int8_grouped_ffn_forward(name):
    inp = wl.layer_inputs(seed=64, **FFN_CASES[name])
    print(f"[int8 ffn] case={name}", flush=True)
    S = _smooth(inp["E"], inp["H"], 65)
    g = _int8_forward(inp, S)
    f = orc.layer_fwd_int8(inp, S)
    A, F = f["route"].A, inp["F"]
    for k, (wc, ws) in zip(("w_gate", "w_up", "w_down"), g["wq"]):
        q, s = orc.quant_weights_int8(inp[k])
        check_equal(f"{k} codes", wc.cpu().numpy(), q)
        check_equal(f"{k} scales", ws.cpu().numpy(), s)
    # G, U, h from bit-exact int8 rows (dispatch) and weights: one kernel on the
    # oracle's operands; y and out are chained (the device's own h)
    check_close("G", f32(g["gus"][:A, :F]), f["G"], ulps=ULPS_KERNEL, rel_l2=REL_8BIT)
    check_close("U", f32(g["gus"][:A, F:]), f["U"], ulps=ULPS_KERNEL, rel_l2=REL_8BIT)
    check_close("h", f32(g["h"][:A]), f["Hh"], ulps=ULPS_KERNEL, rel_l2=REL_8BIT)
    check_close("y", f32(g["y"][:A]), f["Y"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)
    check_close("out", f32(g["out"]), f["out"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)
    # the down GEMM fed the int8 codes of the oracle's h (the quantiser is bit-exact)
    shape = Run(inp).shape
    cap, H = shape.capacity, inp["H"]
    recv = dev(f["route"].ep_recv_counts.astype(np.int32))
    hq, hs = dm.quant_rows_int8(dev_rows(f["Hh"], cap), recv[-1:])
    y2 = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_fwd_int8(shape, hq, hs, g["wq"][2][0], g["wq"][2][1], recv, y2)
    torch.cuda.synchronize()
    check_close("y (oracle h)", f32(y2[:A]), f["Y"], ulps=ULPS_KERNEL, rel_l2=REL_8BIT)


def test_int8_decode_forward_full_size():
    """The decode batch at its full size (T=512, H=7168, F=2048, E=32, K=8) with smooth
    scales and a zero and a copy expert, against the oracle's int8 forward."""
    inp = wl.layer_inputs(512, 7168, 2048, 32, 8, seed=66, Z=1, C=1)
    print("[int8 decode] full size", flush=True)
    S = _smooth(32, 7168, 67)
    g = _int8_forward(inp, S)
    f = orc.layer_fwd_int8(inp, S)
    A = f["route"].A
    check_close("h", f32(g["h"][:A]), f["Hh"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)
    check_close("out", f32(g["out"]), f["out"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)


def test_moe_layer_int8_api():
    """moe_layer_int8 (the Python inference entry of the int8 path) with smooth scales,
    constant and copy experts, a 1-D mask and a given shared_expert_x, against the
    oracle's int8 forward."""
    inp = wl.layer_inputs(seed=68, T=333, H=512, F=256, E=6, K=3, C=1, Q=1, mask="1d")
    inp["shared_expert_x"] = wl.to_bf16_bits(np.random.default_rng(69).standard_normal((333, 512), dtype=np.float32))
    S = _smooth(6, 512, 70)
    wq = [dm.Int8Weights.quantize(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer_int8(bf(inp["x"]), dev(inp["topk_idx"]), dev(inp["topk_weights"]), *wq,
                            smooth_scales=torch.from_numpy(S).to(DEV), x_active_mask=dev(inp["mask"]),
                            shared_expert_x=bf(inp["shared_expert_x"]), const_alpha_1=bf(inp["const_alpha_1"]),
                            const_alpha_2=bf(inp["const_alpha_2"]), const_v=bf(inp["const_v"]),
                            copy_expert_num=1, const_expert_num=1)
    torch.cuda.synchronize()
    f = orc.layer_fwd_int8(inp, S)
    check_close("out", f32(out), f["out"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)


def test_int8_path_with_no_routed_rows():
    """Every slot to a zero or copy expert (no expert rows): the int8 dispatch writes no
    rows, the GEMMs run on zero rows and combine gives the closed forms (0 and ori_x)."""
    inp = wl.layer_inputs(seed=71, T=64, H=256, F=128, E=4, K=2, Z=1, C=1)
    inp["topk_idx"] = np.tile(np.array([[4, 5]], np.int32), (64, 1))   # zero expert 4, copy expert 5
    run = Run(inp)
    d, dyn = dm.dispatch_int8(run.shape, run.x, run.idx, None)
    torch.cuda.synchronize()
    assert int(d.ep_recv_counts[-1].item()) == 0
    wq = [dm.Int8Weights.quantize(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer_int8(run.x, run.idx, run.w, *wq, copy_expert_num=1, zero_expert_num=1)
    torch.cuda.synchronize()
    f = orc.layer_fwd_int8(inp)
    check_close("out", f32(out), f["out"], rel_l2=REL_8BIT, outliers=OUTLIERS_8BIT)
