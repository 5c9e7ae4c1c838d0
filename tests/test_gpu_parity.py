"""GPU parity of every C entry point against the CPU oracle, on seeded inputs.

Indices, counts, prefix sums, both slot/row maps and the permuted rows are
compared bit for bit; so are the gather-reduce outputs (combine, the dY rows of
combine_bwd, dispatch_bwd), whose summation order is the oracle's.  Outputs of
the grouped GEMMs are compared against the oracle's parity mode element by
element within 2e-2 plus one bf16 ulp of the reference (a kernel fed the
oracle's own operands) or two ulps (a chained step), fp32 weight gradients
within 2e-2 (identical operands) or 2e-2 + 2^-5 |P|^T|Q| (chained), and
relative L2 <= 5e-3 (the bar is written out in gpu_util).
"""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import (DEV, RHO_CHAIN, ULPS_KERNEL, Run, bf, check_close, check_equal, contraction_mag, dev,
                      dw_mag, f32, layer_mags)

pytestmark = pytest.mark.gpu

# (name, layer_inputs kwargs): several tiles, ragged tails, masks, special experts
ROUTE_CASES = {
    "tiny": dict(T=256, H=128, F=64, E=8, K=2),
    "page1_1k": dict(T=1024, H=1536, F=480, E=64, K=8),
    "special_2d_mask": dict(T=300, H=64, F=32, E=10, K=6, Z=2, C=1, Q=3, mask="2d"),
    "prefix_1d_mask": dict(T=77, H=32, F=32, E=5, K=3, C=1, mask="1d", mask_active=40),
    "one_expert_k1": dict(T=33, H=16, F=32, E=1, K=1),
    "many_experts_k16": dict(T=200, H=16, F=32, E=1024, K=16),
    "single_token": dict(T=1, H=8, F=32, E=4, K=2),
    "no_tokens": dict(T=0, H=8, F=32, E=4, K=2),
}


def _inputs(name, seed=0, weights=False, grad=False):
    kw = dict(ROUTE_CASES[name])
    return wl.layer_inputs(seed=seed, weights=weights, grad=grad, **kw)


def _check_route(run, inp):
    r = orc.route(inp["topk_idx"], inp["E"], inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0),
                  inp.get("mask"))
    d = run.d
    T, K = inp["T"], inp["K"]
    check_equal("expert_token_nums", d.expert_token_nums.cpu().numpy(), r.counts)
    check_equal("ep_recv_counts", d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_equal("slot2row", d.slot2row(T, K).cpu().numpy(), r.slot2row)
    check_equal("row2slot", d.row2slot(T, K)[:r.A].cpu().numpy(), r.row2slot)
    assert int(d.err_flag.item()) == r.err
    return r


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_dispatch_bit_exact(name):
    inp = _inputs(name)
    run = Run(inp)
    print(f"[dispatch] case={name} T={inp['T']} E={inp['E']} K={inp['K']}", flush=True)
    run.dispatch()
    r = _check_route(run, inp)
    X = orc.dispatch(inp["x"], r)
    check_equal("expand_x", f32(run.d.expand_x[:r.A]), X)


def test_dispatch_error_flags():
    T, K, E = 64, 4, 6
    inp = wl.layer_inputs(T, 16, 32, E, K, seed=1, weights=False, grad=False)
    idx = inp["topk_idx"].copy()
    idx[3, 2] = E + 5          # out of range
    idx[7, 3] = idx[7, 0]      # duplicate: the later one is dropped
    idx[9, 0] = -1             # negative
    inp["topk_idx"] = idx
    m = np.ones(T, np.uint8)
    m[10] = 0                  # a false before trues: not a prefix
    inp["mask"] = m
    run = Run(inp)
    run.dispatch()
    r = _check_route(run, inp)
    assert r.err == orc.ERR_ID_RANGE | orc.ERR_ID_DUPLICATE | orc.ERR_MASK_NOT_PREFIX


FFN_CASES = {
    "tiny": dict(T=256, H=128, F=64, E=8, K=2),
    "ragged": dict(T=300, H=256, F=96, E=7, K=3),
    "page1_512": dict(T=512, H=1536, F=480, E=64, K=8),
    "empty_experts": dict(T=20, H=64, F=32, E=16, K=1),
    "special_mask": dict(T=150, H=128, F=64, E=6, K=4, Z=1, C=1, Q=2, mask="2d"),
    # many rows per expert and many weight-gradient tiles, ragged row tiles
    # (8200 rows) and ragged F = 480 (K tail of the down GEMM, gate/up seam
    # inside a K step of the gate/up data gradient)
    "big_tiles_ragged": dict(T=4100, H=4096, F=480, E=16, K=2),
    # H not a multiple of the 64-wide K step: K tail of the gate/up forward
    # and of the down data gradient (K = H), one 8-column last tile in the
    # H-wide outputs and weight-gradient rows
    "ragged_h": dict(T=300, H=200, F=96, E=5, K=2),
    "ragged_h_1k": dict(T=1000, H=1096, F=224, E=9, K=3),
    # wide outputs: the gate/up forward spans 16 column tiles (grouped tile
    # order, 13 row-tile slots = one full group of 8 and a partial one); the
    # down data gradient takes the 128 x 256 tiles (N = F = 1024)
    "wide_ffn": dict(T=700, H=256, F=1024, E=3, K=2),
    # wide weight gradients: the gate/up weight gradient on eight-wave
    # 256 x 256 tiles (a 12 x 16 tile grid per expert), down weight-gradient
    # blocks of 8 x 3 tiles; grouped order for the gate/up forward, down
    # forward and gate/up data gradient (24, 32 and 16 column tiles)
    "wide_wgrad": dict(T=600, H=4096, F=1536, E=2, K=1),
    # enough tiles for the 256 x 256 eight-wave forward tiles: the gate/up
    # forward with a K tail (H = 1096) and a partial last column tile (F = 224)
    "w8_gate_up_ragged": dict(T=8000, H=1096, F=224, E=16, K=2),
    # the down forward on 256 x 256 tiles: partial last column tile (N = H =
    # 1096 = 4 x 256 + 72) and a K tail (F = 224)
    "w8_down_ragged": dict(T=4000, H=1096, F=224, E=8, K=2),
}


def _forward(inp):
    run = Run(inp)
    run.dispatch()
    run.ffn()
    return run


@pytest.mark.parametrize("name", list(FFN_CASES))
def test_grouped_ffn_forward(name):
    inp = wl.layer_inputs(seed=2, **FFN_CASES[name])
    print(f"[ffn fwd] case={name}", flush=True)
    run = _forward(inp)
    f = orc.layer_fwd(inp, prec="parity")
    A, F = run.A, inp["F"]
    assert A == f["route"].A
    # G, U, h come from the bit-exact expand_x and the weights: one kernel on the
    # oracle's operands; y contracts the device's h (chained)
    check_close("G", f32(run.gus[:A, :F]), f["G"], ulps=ULPS_KERNEL)
    check_close("U", f32(run.gus[:A, F:]), f["U"], ulps=ULPS_KERNEL)
    check_close("h", f32(run.h[:A]), f["Hh"], ulps=ULPS_KERNEL)
    check_close("y", f32(run.y[:A]), f["Y"])


COMBINE_CASES = {
    "routed_only": dict(T=257, H=136, E=9, K=4),
    "special_2d_mask_shared": dict(T=300, H=256, E=16, K=8, Z=1, C=1, Q=2, mask="2d", shared=True),
    "copy_const_1d_mask": dict(T=129, H=64, E=4, K=5, C=2, Q=1, mask="1d", shared=False),
}


def _combine_inputs(name, seed=3):
    kw = dict(COMBINE_CASES[name])
    shared = kw.pop("shared", False)
    mask = kw.pop("mask", None)
    inp = wl.layer_inputs(seed=seed, weights=False, grad=True, F=0, mask=mask,
                          mask_active=kw["T"] // 2, **kw)
    rng = np.random.default_rng(seed + 100)
    cap = kw["T"] * min(kw["E"], kw["K"])
    inp["y"] = wl.to_bf16_bits(rng.standard_normal((cap, kw["H"]), dtype=np.float32))
    inp["dX"] = wl.to_bf16_bits(rng.standard_normal((cap, kw["H"]), dtype=np.float32) * 0.1)
    inp["shared_expert_x"] = wl.to_bf16_bits(rng.standard_normal((kw["T"], kw["H"]), dtype=np.float32)) \
        if shared else None
    return inp


@pytest.mark.parametrize("name", list(COMBINE_CASES))
def test_combine_forward_bit_exact(name):
    inp = _combine_inputs(name)
    print(f"[combine] case={name}", flush=True)
    run = Run(inp)
    run.dispatch()
    r = _check_route(run, inp)
    sh = bf(inp["shared_expert_x"]) if inp["shared_expert_x"] is not None else None
    out = run.combine(y=bf(inp["y"]), shared=sh)
    Y = orc.bf16_to_f32(inp["y"])[:r.A]
    ref = orc.combine(Y, r, inp["topk_weights"], inp["shared_expert_x"], inp["x"],
                      inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"))
    check_equal("out", f32(out), ref)


@pytest.mark.parametrize("name", list(COMBINE_CASES))
def test_combine_backward(name):
    inp = _combine_inputs(name)
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"], inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0),
                  inp.get("mask"))
    gy, gw = run.combine_bwd(bf(inp["grad_out"]), y=bf(inp["y"]))
    Y = orc.bf16_to_f32(inp["y"])[:r.A]
    dY, dw = orc.combine_bwd(inp["grad_out"], Y, r, inp["topk_weights"], inp["x"],
                             inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"))
    check_equal("grad_y", f32(gy[:r.A]), dY)
    # dw is a length-H dot product: fp32 summation order differs from numpy's
    check_close("grad_topk_weights", f32(gw), dw, ulps=0, max_abs=1e-3, rel_l2=1e-5)
    assert np.all(f32(gw)[r.slot2row.reshape(r.T, r.K) == -1] == 0)


@pytest.mark.parametrize("qpay", [False, True])
@pytest.mark.parametrize("name", list(COMBINE_CASES))
def test_combine_backward_halves_equal_the_whole(name, qpay):
    """moe_combine_bwd with one output left out (NULL) computes the other alone,
    bit for bit as the call with both (grad_y alone without reading y), also with
    the int8 payload, whose round trip of y only the weights' gradient sees."""
    inp = _combine_inputs(name)
    print(f"[combine bwd halves] case={name} qpay={qpay}", flush=True)
    run = Run(inp)
    if qpay:
        run.shape.comm_quant_mode = 2
    run.dispatch()
    g, yb = bf(inp["grad_out"]), bf(inp["y"])
    gy, gw = run.combine_bwd(g, y=yb)
    args = (run.shape, g, None, run.idx, run.w, run.d.assist_info_for_combine, run.d.ep_recv_counts, run.mask,
            run.x, run.a1, run.a2, run.cv)
    gy1 = torch.zeros_like(gy)
    dm.moe_combine_bwd(*args, gy1, None)                 # grad_y alone, y not passed
    gw2 = torch.full_like(gw, float("nan"))
    a2 = list(args)
    a2[2] = yb
    dm.moe_combine_bwd(*a2, None, gw2)                   # grad_topk_weights alone
    torch.cuda.synchronize()
    assert torch.equal(gy1, gy), "grad_y alone differs from the whole call"
    assert torch.equal(gw2, gw), "grad_topk_weights alone differs from the whole call"
    with pytest.raises(dm.MoeError):
        dm.moe_combine_bwd(*a2, None, None)


@pytest.mark.parametrize("name", list(COMBINE_CASES))
def test_dispatch_backward_bit_exact(name):
    inp = _combine_inputs(name)
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"], inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0),
                  inp.get("mask"))
    rng = np.random.default_rng(7)
    accum = wl.to_bf16_bits(rng.standard_normal((inp["T"], inp["H"]), dtype=np.float32))
    for acc in (None, accum):
        gx = run.dispatch_bwd(bf(inp["dX"]), bf(inp["grad_out"]), None if acc is None else bf(acc))
        dX = orc.bf16_to_f32(inp["dX"])[:r.A]
        ref = orc.dispatch_bwd(dX, r, inp["topk_weights"], inp["grad_out"], inp.get("const_alpha_1"),
                               None if acc is None else orc.bf16_to_f32(acc))
        check_equal("grad_x", f32(gx), ref)


def test_round_trip_is_k_times_x():
    """dispatch then combine of expand_x itself with unit weights gives K*x exactly."""
    for T, H, E, K in ((300, 128, 16, 8), (64, 1536, 64, 8), (50, 40, 5, 3)):
        inp = wl.layer_inputs(T, H, 32, E, K, seed=5, weights=False, grad=False)
        run = Run(inp)
        run.dispatch()
        out = run.combine(y=run.d.expand_x, w=torch.ones((T, K), dtype=torch.float32, device=DEV))
        ref = (run.x.float().cpu() * K).to(torch.bfloat16)
        assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", list(FFN_CASES))
def test_grouped_ffn_backward(name):
    inp = wl.layer_inputs(seed=4, **FFN_CASES[name])
    print(f"[ffn bwd] case={name}", flush=True)
    run = _forward(inp)
    f = orc.layer_fwd(inp, prec="parity")
    r = f["route"]
    A = r.A
    dY_bits = wl.to_bf16_bits(np.random.default_rng(9).standard_normal((run.cap, inp["H"]), dtype=np.float32) * 0.2)
    ggu, gxe, gwg, gwu, gwd = run.ffn_bwd(bf(dY_bits))
    dY = orc.bf16_to_f32(dY_bits)[:A]
    dGU, dX, dWg, dWu, dWd = orc.ffn_bwd(dY, f["X"], f["G"], f["U"], f["Hh"], r.ep_recv_counts,
                                         inp["w_gate"], inp["w_up"], inp["w_down"])
    # chained: the device's own G|U and h feed the backward
    rc, F = r.ep_recv_counts, inp["F"]
    check_close("grad_gate_up", f32(ggu[:A]), dGU)
    check_close("grad_expand_x", f32(gxe[:A]), dX)
    check_close("grad_w_gate", f32(gwg), dWg, ulps=0, mag=contraction_mag(dGU[:, :F], f["X"], rc), rho=RHO_CHAIN)
    check_close("grad_w_up", f32(gwu), dWu, ulps=0, mag=contraction_mag(dGU[:, F:], f["X"], rc), rho=RHO_CHAIN)
    check_close("grad_w_down", f32(gwd), dWd, ulps=0, mag=contraction_mag(dY, f["Hh"], rc), rho=RHO_CHAIN)


@pytest.mark.parametrize("name", list(FFN_CASES))
def test_grouped_ffn_backward_gemms_on_oracle_operands(name):
    """Each of the four backward GEMMs fed the oracle's own operands (G|U, h, dY,
    dG|dU, expand_x): one bf16 ulp for the bf16 outputs, the plain 2e-2 for the
    fp32 weight gradients."""
    import dispatch_expert_gemm_amd as dm
    inp = wl.layer_inputs(seed=4, **FFN_CASES[name])
    print(f"[ffn bwd gemms] case={name}", flush=True)
    f = orc.layer_fwd(inp, prec="parity")
    r = f["route"]
    A, F, H, E = r.A, inp["F"], inp["H"], inp["E"]
    shape = Run(inp).shape
    cap = shape.capacity
    rng = np.random.default_rng(9)
    dY_bits = wl.to_bf16_bits(rng.standard_normal((cap, H), dtype=np.float32) * 0.2)
    dY = orc.bf16_to_f32(dY_bits)[:A]
    dGU, dX, dWg, dWu, dWd = orc.ffn_bwd(dY, f["X"], f["G"], f["U"], f["Hh"], r.ep_recv_counts,
                                         inp["w_gate"], inp["w_up"], inp["w_down"])

    def rows(a, width):   # oracle rows (A, width) -> a capacity-row bf16 device buffer
        full = np.zeros((cap, width), np.float32)
        full[:A] = a
        return bf(orc.f32_to_bf16(full))

    recv = dev(r.ep_recv_counts.astype(np.int32))
    wg, wu, wd = (bf(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    gus = rows(np.concatenate([f["G"], f["U"]], 1), 2 * F)
    ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    gxe = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    gwg = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
    gwu = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
    gwd = torch.empty((E, H, F), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_data(shape, bf(dY_bits), wd, gus, recv, ggu)
    dm.moe_ffn_down_bwd_weight(shape, bf(dY_bits), rows(f["Hh"], F), recv, gwd)
    dgu_dev = rows(dGU, 2 * F)
    dm.moe_ffn_gate_up_bwd_data(shape, dgu_dev, wg, wu, recv, gxe)
    dm.moe_ffn_gate_up_bwd_weight(shape, dgu_dev, rows(f["X"], H), recv, gwg, gwu)
    torch.cuda.synchronize()
    check_close("grad_gate_up", f32(ggu[:A]), dGU, ulps=ULPS_KERNEL)
    check_close("grad_expand_x", f32(gxe[:A]), dX, ulps=ULPS_KERNEL)
    check_close("grad_w_gate", f32(gwg), dWg, ulps=0)
    check_close("grad_w_up", f32(gwu), dWu, ulps=0)
    check_close("grad_w_down", f32(gwd), dWd, ulps=0)


LAYER_CASES = {
    "tiny": dict(T=256, H=128, F=64, E=8, K=2),
    "special_mask": dict(T=200, H=256, F=96, E=12, K=6, Z=1, C=1, Q=2, mask="2d"),
    "page1_1k": dict(T=1024, H=1536, F=480, E=64, K=8),
    "big_tiles_ragged": dict(T=4100, H=4096, F=480, E=16, K=2),
}


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_forward_backward(name):
    """Whole chain through the C entries: dispatch, FFN, combine and their backward."""
    inp = wl.layer_inputs(seed=6, **LAYER_CASES[name])
    print(f"[layer] case={name}", flush=True)
    run = _forward(inp)
    out = run.combine()
    g = bf(inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe, gwg, gwu, gwd = run.ffn_bwd(gy)
    gx = run.dispatch_bwd(gxe, g)
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    A = f["route"].A
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"])
    check_close("grad_y", f32(gy[:A]), b["dY"])
    check_close("grad_topk_weights", f32(gw), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN)
    check_close("grad_gate_up", f32(ggu[:A]), b["dGU"])
    check_close("grad_expand_x", f32(gxe[:A]), b["dX"])
    check_close("grad_x", f32(gx), b["dx"])
    check_close("grad_w_gate", f32(gwg), b["dWg"], ulps=0, mag=m["dWg"], rho=RHO_CHAIN)
    check_close("grad_w_up", f32(gwu), b["dWu"], ulps=0, mag=m["dWu"], rho=RHO_CHAIN)
    check_close("grad_w_down", f32(gwd), b["dWd"], ulps=0, mag=m["dWd"], rho=RHO_CHAIN)


def test_autograd_layer_and_determinism():
    import dispatch_expert_gemm_amd as dm
    inp = wl.layer_inputs(seed=8, **LAYER_CASES["special_mask"])
    res = []
    for _ in range(2):
        x = bf(inp["x"]).requires_grad_(True)
        w = dev(inp["topk_weights"]).requires_grad_(True)
        wg, wu, wd = (bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down"))
        sh = bf(wl.to_bf16_bits(np.random.default_rng(1).standard_normal((inp["T"], inp["H"]),
                                                                          dtype=np.float32))).requires_grad_(True)
        out = dm.moe_layer(x, dev(inp["topk_idx"]), w, wg, wu, wd, x_active_mask=dev(inp["mask"]).bool(),
                           shared_expert_x=sh, const_alpha_1=bf(inp["const_alpha_1"]),
                           const_alpha_2=bf(inp["const_alpha_2"]), const_v=bf(inp["const_v"]),
                           zero_expert_num=1, copy_expert_num=1, const_expert_num=2)
        out.backward(bf(inp["grad_out"]))
        torch.cuda.synchronize()
        res.append([t.detach().cpu().clone() for t in (out, x.grad, w.grad, wg.grad, wu.grad, wd.grad, sh.grad)])
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    inp2 = dict(inp, shared_expert_x=wl.to_bf16_bits(np.random.default_rng(1).standard_normal(
        (inp["T"], inp["H"]), dtype=np.float32)))
    f = orc.layer_fwd(inp2, prec="parity")
    b = orc.layer_bwd(inp2, f, inp["grad_out"], prec="parity")
    out, gx, gw = res[0][0], res[0][1], res[0][2]
    m = layer_mags(inp2, f, b)
    check_close("out", f32(out), f["out"])
    check_close("grad_x", f32(gx), b["dx"])
    check_close("grad_topk_weights", f32(gw), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN)
    for t, k in zip(res[0][3:6], ("dWg", "dWu", "dWd")):
        # returned in bf16 (the weights' dtype): one more rounding of the fp32 result
        check_close(k, f32(t), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN)
    assert torch.equal(res[0][6].view(torch.int16), bf(inp["grad_out"]).cpu().view(torch.int16))


def test_autograd_layer_without_routing_weight_gradient():
    """topk_weights that need no gradient: the layer's backward asks the combine
    backward for grad_y alone, and every other gradient is bit for bit the same."""
    import dispatch_expert_gemm_amd as dm
    inp = wl.layer_inputs(seed=9, **LAYER_CASES["special_mask"])
    print("[autograd] routing weights without gradient", flush=True)
    res = []
    for need_w in (True, False):
        x = bf(inp["x"]).requires_grad_(True)
        w = dev(inp["topk_weights"]).requires_grad_(need_w)
        wg, wu, wd = (bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down"))
        out = dm.moe_layer(x, dev(inp["topk_idx"]), w, wg, wu, wd, x_active_mask=dev(inp["mask"]).bool(),
                           const_alpha_1=bf(inp["const_alpha_1"]), const_alpha_2=bf(inp["const_alpha_2"]),
                           const_v=bf(inp["const_v"]), zero_expert_num=1, copy_expert_num=1, const_expert_num=2)
        out.backward(bf(inp["grad_out"]))
        torch.cuda.synchronize()
        assert (w.grad is not None) == need_w
        res.append([t.detach().cpu().view(torch.int16) for t in (out, x.grad, wg.grad, wu.grad, wd.grad)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_autograd_layer_shared_expert():
    """moe_layer with a SwiGLU shared expert computed inside the layer."""
    import dispatch_expert_gemm_amd as dm
    inp = wl.layer_inputs(200, 256, 96, 6, 2, seed=13, shared=True, Z=1, C=1, mask="2d")
    x = bf(inp["x"]).requires_grad_(True)
    w = dev(inp["topk_weights"]).requires_grad_(True)
    ws = [bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down", "shared_w_gate",
                                                     "shared_w_up", "shared_w_down")]
    out = dm.moe_layer(x, dev(inp["topk_idx"]), w, *ws[:3], x_active_mask=dev(inp["mask"]),
                       shared_w_gate=ws[3], shared_w_up=ws[4], shared_w_down=ws[5],
                       zero_expert_num=1, copy_expert_num=1)
    out.backward(bf(inp["grad_out"]))
    torch.cuda.synchronize()
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"])
    check_close("grad_x", f32(x.grad), b["dx"])
    check_close("grad_topk_weights", f32(w.grad), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN)
    for t, k in zip(ws, ("dWg", "dWu", "dWd", "s_dWg", "s_dWu", "s_dWd")):
        # returned in the weights' dtype (bf16): compare with the rounding of the fp32 result
        check_close(k, f32(t.grad), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN)
