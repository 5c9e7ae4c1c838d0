"""GPU parity of the fp8 path: e4m3 quantisers (bit-exact), block-scaled fp8 grouped
GEMMs (forward and data gradients) and the int8 combine payload, against the
oracle's fp8 functions.  Each fp8 GEMM fed the oracle's operands is held to
2e-2 plus one bf16 ulp per element and relative L2 <= 2e-2 (the fp8 bar); whole
chained layers to the chained bar written out in gpu_util."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import (DEV, OUTLIERS_8BIT, REL_L2_8BIT, RHO_CHAIN, RHO_FP32, contraction_mag, ULPS_KERNEL, Fp8Run, Run, bf, check_close, check_equal, dev,
                      dev_rows, f32, layer_mags)

pytestmark = pytest.mark.gpu

REL_FP8 = REL_L2_8BIT


def _u8(t):
    return t.detach().cpu().numpy()


def test_quant_rows_fp8_bit_exact():
    rng = np.random.default_rng(31)
    R, C = 70, 512
    a = rng.standard_normal((R, C)).astype(np.float32)
    a[3] = 0.0                                   # all-zero row
    a[5, 128:256] = 0.0                          # all-zero block
    a[7] *= 1e-4                                 # subnormal e4m3 range after scaling
    a[9] *= 3e3                                  # large magnitudes
    a[11, ::7] = 0.0
    bits = wl.to_bf16_bits(a)
    codes, scales = dm.quant_rows_fp8(bf(bits))
    torch.cuda.synchronize()
    q, s = orc.quant_e4m3_rows(orc.bf16_to_f32(bits))
    check_equal("codes", _u8(codes), q)
    check_equal("scales", scales.cpu().numpy().T, s)      # stored (C/128, R)
    # only the first n rows when a device row count is given
    codes2 = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    scales2 = torch.zeros((C // 128, R), dtype=torch.float32, device=DEV)
    dm.moe_quant_rows_fp8(bf(bits), codes2, scales2, nrows=torch.tensor([33], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    check_equal("codes rows<33", _u8(codes2)[:33], q[:33])
    check_equal("scales rows<33", scales2.cpu().numpy().T[:33], s[:33])
    assert (_u8(codes2)[33:] == 0xAB).all() and not scales2.cpu().numpy().T[33:].any()


def test_quantize_weights_fp8_bit_exact():
    rng = np.random.default_rng(32)
    E, N, K = 3, 256, 384
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[1, :128, 128:256] = 0.0
    bits = wl.to_bf16_bits(w)
    q = dm.Fp8Weights.quantize(bf(bits))
    torch.cuda.synchronize()
    codes, scales = orc.quant_weights_fp8(bits)
    check_equal("codes", _u8(q.codes), codes)
    check_equal("codes_t", _u8(q.codes_t), codes.transpose(0, 2, 1))
    check_equal("scales", q.scales.cpu().numpy(), scales)


FP8_CASES = {
    "small": dict(T=300, H=256, F=384, E=5, K=2),
    "ragged_rows": dict(T=517, H=512, F=256, E=7, K=3),
    "empty_experts": dict(T=40, H=128, F=128, E=12, K=1),
}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_grouped_ffn_forward_and_data_gradients(name):
    """The four fp8 GEMMs one by one, each fed the oracle's operands: x codes from the
    bit-exact dispatch and quantiser; the down GEMM on the codes of the oracle's h, the
    down data gradient on the oracle's G|U, the gate/up data gradient on the codes of
    the oracle's dG|dU (the quantiser is bit-exact, tested above)."""
    inp = wl.layer_inputs(seed=33, **FP8_CASES[name])
    print(f"[fp8] case={name}", flush=True)
    run = Fp8Run(inp)
    run.dispatch()
    run.quant_weights()
    run.ffn8()
    r = orc.route(inp["topk_idx"], inp["E"])
    A, F, H, cap = r.A, inp["F"], inp["H"], run.cap
    recv, nrows = run.d.ep_recv_counts, run.d.ep_recv_counts[-1:]
    X = orc.dispatch(inp["x"], r)
    wq = tuple(orc.quant_weights_fp8(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    G, U, Hh, Y = orc.ffn_fwd_fp8(X, r.ep_recv_counts, *wq)
    check_close("G", f32(run.gus[:A, :F]), G, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("U", f32(run.gus[:A, F:]), U, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("h", f32(run.h[:A]), Hh, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    wg, wu, wd = run.wq
    hq, hs = dm.quant_rows_fp8(dev_rows(Hh, cap), nrows)
    y = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_fwd_fp8(run.shape, hq, hs, wd.codes, wd.scales, recv, y)
    # data gradients from a bf16 dY of realistic scale (w * dOut ~ 0.125 N(0,1))
    dY_bits = wl.to_bf16_bits(np.random.default_rng(34).standard_normal((cap, H), dtype=np.float32) * 0.125)
    dGU, dX, _, _, _ = orc.ffn_bwd_fp8(orc.bf16_to_f32(dY_bits)[:A], X, G, U, Hh, r.ep_recv_counts, *wq)
    dyq, dys = dm.quant_rows_fp8(bf(dY_bits), nrows)
    ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_bwd_data_fp8(run.shape, dyq, dys, wd.codes_t, wd.scales,
                                 dev_rows(np.concatenate([G, U], 1), cap), recv, ggu)
    dguq, dgus = dm.quant_rows_fp8(dev_rows(dGU, cap), nrows)
    gxe = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_gate_up_bwd_data_fp8(run.shape, dguq, dgus, wg.codes_t, wg.scales, wu.codes_t, wu.scales, recv, gxe)
    torch.cuda.synchronize()
    check_close("y", f32(y[:A]), Y, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("grad_gate_up", f32(ggu[:A]), dGU, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("grad_expand_x", f32(gxe[:A]), dX, ulps=ULPS_KERNEL, rel_l2=REL_FP8)


@pytest.mark.parametrize("special", [False, True])
def test_int8_payload_combine(special):
    kw = dict(T=201, H=256, E=8, K=4)
    if special:
        kw.update(Z=1, C=1, Q=2, mask="2d")
    inp = wl.layer_inputs(seed=35, weights=False, F=0, **kw)
    cap = kw["T"] * min(kw["E"], kw["K"])
    y_bits = wl.to_bf16_bits(np.random.default_rng(36).standard_normal((cap, kw["H"]), dtype=np.float32))
    run = Run(inp)
    run.shape.comm_quant_mode = 2
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"], inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0), inp.get("mask"))
    y = bf(y_bits)
    out = run.combine(y=y)
    Yc = orc.qdq_rows_int8(orc.bf16_to_f32(y_bits)[:r.A])
    ref = orc.combine(Yc, r, inp["topk_weights"], None, inp["x"], inp.get("const_alpha_1"),
                      inp.get("const_alpha_2"), inp.get("const_v"))
    check_equal("out", f32(out), ref)
    gy, gw = run.combine_bwd(bf(inp["grad_out"]), y=y)
    dY, dw = orc.combine_bwd(inp["grad_out"], Yc, r, inp["topk_weights"], inp["x"], inp.get("const_alpha_1"),
                             inp.get("const_alpha_2"), inp.get("const_v"))
    check_equal("grad_y", f32(gy[:r.A]), dY)
    check_close("grad_topk_weights", f32(gw), dw, ulps=0, max_abs=1e-3, rel_l2=1e-5)


def test_fp8_layer_forward_backward():
    """The whole fp8 step (int8 combine payload, bf16 weight gradients) vs the oracle."""
    inp = wl.layer_inputs(400, 256, 256, 6, 2, seed=37)
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
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_topk_weights", f32(gw), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    check_close("grad_x", f32(gx), b["dx"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_w_gate", f32(gwg), b["dWg"], ulps=0, mag=m["dWg"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    check_close("grad_w_up", f32(gwu), b["dWu"], ulps=0, mag=m["dWu"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    check_close("grad_w_down", f32(gwd), b["dWd"], ulps=0, mag=m["dWd"], rho=RHO_CHAIN, rel_l2=REL_FP8)


def test_autograd_layer_fp8_int8_payload():
    """moe_layer(fp8=True, comm_quant_mode=2): the autograd function on the fp8
    path (weights quantised inside the layer) against the oracle's fp8 layer."""
    inp = wl.layer_inputs(384, 256, 256, 6, 2, seed=39, mask="2d", Z=1)
    x = bf(inp["x"]).requires_grad_(True)
    w = dev(inp["topk_weights"]).requires_grad_(True)
    ws = [bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer(x, dev(inp["topk_idx"]), w, *ws, x_active_mask=dev(inp["mask"]), zero_expert_num=1,
                       fp8=True, comm_quant_mode=2)
    out.backward(bf(inp["grad_out"]))
    torch.cuda.synchronize()
    f = orc.layer_fwd_fp8(inp)
    b = orc.layer_bwd_fp8(inp, f, inp["grad_out"])
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_x", f32(x.grad), b["dx"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_topk_weights", f32(w.grad), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    for t, k in zip(ws, ("dWg", "dWu", "dWd")):
        # returned in the weights' dtype (bf16)
        check_close(k, f32(t.grad), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN, rel_l2=REL_FP8)


# ----------------------------------------------------------------------------- fp8 weight gradients


def _slot_of(prefix, e, r0):
    """Token slot of the per-128-token block starting at row r0 of expert e: expert
    e's slots are numbered from prefix[e-1]/128 + e (the C header's layout)."""
    start = int(prefix[e - 1]) if e else 0
    return start // 128 + e + (r0 - start) // 128


def test_quant_cols_fp8_bit_exact():
    rng = np.random.default_rng(41)
    sizes = [0, 1, 127, 128, 129, 300, 0, 5]
    prefix = np.cumsum(sizes)
    A, E, D = int(prefix[-1]), len(sizes), 384
    cap = A + 37                                  # rows past the experts' rows are not read
    a = rng.standard_normal((cap, D)).astype(np.float32)
    a[300:428, 5] = 0.0                           # an all-zero column of one block
    a[:, 7] *= 1e-4                               # e4m3 subnormals after scaling
    a[:, 9] *= 3e3
    a[:, 200:256] *= np.exp(rng.standard_normal((1, 56)) * 3).astype(np.float32)
    bits = wl.to_bf16_bits(a)
    counts = torch.from_numpy(prefix.astype(np.int32)).to(DEV)
    codes_t, scales = dm.quant_cols_fp8(bf(bits), counts)
    torch.cuda.synchronize()
    ns = cap // 128 + E
    assert codes_t.shape == (D, 128 * ns) and scales.shape == (ns, D)
    ct, sc = _u8(codes_t), scales.cpu().numpy()
    blocks = orc.quant_cols_fp8(orc.bf16_to_f32(bits)[:A], prefix)
    assert len(blocks) == 1 + 1 + 1 + 2 + 3 + 1
    for e, r0, r1, q, s in blocks:
        sl = _slot_of(prefix, e, r0)
        n = r1 - r0
        check_equal(f"codes e={e} r0={r0}", ct[:, sl * 128:sl * 128 + n], q.T)
        assert not ct[:, sl * 128 + n:(sl + 1) * 128].any(), "rows past the expert's end must be code 0"
        check_equal(f"scales e={e} r0={r0}", sc[sl], s)


WG_CASES = {
    # expert row counts, H, F
    "ragged": ([0, 1, 127, 128, 129, 300, 0, 5], 256, 384),
    "one_long_expert": ([1500], 384, 128),
    "many_experts": (list(np.random.default_rng(42).integers(0, 260, size=40)), 128, 256),
    "no_rows": ([0, 0, 0], 128, 128),
}


@pytest.mark.parametrize("name", list(WG_CASES))
def test_fp8_weight_gradient_gemms(name):
    """moe_quant_cols_fp8 + the two fp8 weight-gradient GEMMs on seeded bf16
    operands against the oracle's wgrad_fp8 of the same operands: the codes are
    bit-exact, so only the accumulation differs (float64 in the oracle; fp32
    sums inside the fp8 MFMA and across token slots on the GPU, measured at
    1.3e-5 relative L2 on the ragged case, hence the 1e-4 bar)."""
    sizes, H, F = WG_CASES[name]
    print(f"[fp8 wgrad] case={name}", flush=True)
    prefix = np.cumsum(sizes).astype(np.int64)
    A, E = int(prefix[-1]), len(sizes)
    cap = A + 20
    rng = np.random.default_rng(43)
    mats = {k: wl.to_bf16_bits((rng.standard_normal((cap, d)) * s).astype(np.float32))
            for k, d, s in (("dY", H, 0.1), ("h", F, 1.0), ("dGU", 2 * F, 0.05), ("x", H, 1.0))}
    counts = torch.from_numpy(prefix.astype(np.int32)).to(DEV)
    shape = dm.make_shape(max(A, 1), H, 1, E, F=F, capacity=cap)
    q = {k: dm.quant_cols_fp8(bf(v), counts) for k, v in mats.items()}
    gwd = torch.full((E, H, F), float("nan"), dtype=torch.float32, device=DEV)
    gwg = torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV)
    gwu = torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_weight_fp8(shape, *q["dY"], *q["h"], counts, gwd)
    dm.moe_ffn_gate_up_bwd_weight_fp8(shape, *q["dGU"], *q["x"], counts, gwg, gwu)
    torch.cuda.synchronize()
    f = {k: orc.bf16_to_f32(v)[:A] for k, v in mats.items()}
    ref_d = orc.wgrad_fp8(f["dY"], f["h"], prefix)
    ref_gu = orc.wgrad_fp8(f["dGU"], f["x"], prefix)
    dq = {k: orc.qdq_cols_fp8(v, prefix) for k, v in f.items()}
    md = contraction_mag(dq["dY"], dq["h"], prefix)
    mgu = contraction_mag(dq["dGU"], dq["x"], prefix)
    # identical codes: only fp32 accumulation against float64 (RHO_FP32)
    check_close("grad_w_down", f32(gwd), ref_d, ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=md, rho=RHO_FP32)
    check_close("grad_w_gate", f32(gwg), ref_gu[:, :F], ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=mgu[:, :F], rho=RHO_FP32)
    check_close("grad_w_up", f32(gwu), ref_gu[:, F:], ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=mgu[:, F:], rho=RHO_FP32)


def test_fp8_layer_with_fp8_weight_gradients():
    """The whole fp8 step with fp8 weight gradients (moe_layer(fp8_wgrad=True))
    against the oracle's fp8 layer with wgrad='fp8'.

    The weight gradients here quantise the GPU's own dG/dU, h and dY, which differ
    from the oracle's in the last bf16 bit at a fraction of entries (accumulation
    order of the GEMMs that produce them).  e4m3 rounding is discontinuous: moving
    0.1-1% of dG/dU entries by one bf16 ulp moves the fp8 weight gradient of this
    layer by 1-2% of its largest entry (measured on the oracle alone), so its max|err|
    bar is 5e-2 of the largest entry; the L2 bar stays the fp8 one, and the GEMMs
    themselves are held to 1e-4 on identical operands above."""
    inp = wl.layer_inputs(700, 256, 384, 5, 2, seed=44, mask="2d", C=1)
    x = bf(inp["x"]).requires_grad_(True)
    w = dev(inp["topk_weights"]).requires_grad_(True)
    ws = [bf(inp[k]).requires_grad_(True) for k in ("w_gate", "w_up", "w_down")]
    out = dm.moe_layer(x, dev(inp["topk_idx"]), w, *ws, x_active_mask=dev(inp["mask"]), copy_expert_num=1,
                       fp8=True, comm_quant_mode=2, fp8_wgrad=True)
    out.backward(bf(inp["grad_out"]))
    torch.cuda.synchronize()
    f = orc.layer_fwd_fp8(inp)
    b = orc.layer_bwd_fp8(inp, f, inp["grad_out"], wgrad="fp8")
    m = layer_mags(inp, f, b)
    check_close("out", f32(out), f["out"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_x", f32(x.grad), b["dx"], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_topk_weights", f32(w.grad), b["dw"], ulps=0, mag=m["dw"], rho=RHO_CHAIN, rel_l2=REL_FP8)
    for t, k in zip(ws, ("dWg", "dWu", "dWd")):
        check_close(k, f32(t.grad), orc.round_bf16(b[k]), mag=m[k], rho=RHO_CHAIN, rel_l2=REL_FP8)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fused_quantisation_of_the_down_data_gradient(name):
    """moe_ffn_down_bwd_data_fp8_quant: its bf16 dG/dU equal the unfused entry's,
    and its row and per-128-token codes equal the quantiser kernels run on that
    output (both quantisers are bit-exact against the oracle's above)."""
    inp = wl.layer_inputs(seed=45, **FP8_CASES[name])
    print(f"[fp8 fused quant] case={name}", flush=True)
    run = Fp8Run(inp)
    run.dispatch()
    run.quant_weights()
    run.ffn8()
    F, H, E, cap = inp["F"], inp["H"], inp["E"], run.cap
    recv = run.d.ep_recv_counts
    nrows = recv[-1:]
    gy = bf(wl.to_bf16_bits(np.random.default_rng(46).standard_normal((cap, H), dtype=np.float32) * 0.125))
    dyq, dys = dm.quant_rows_fp8(gy, nrows)
    wd = run.wq[2]
    ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
    dm.moe_ffn_down_bwd_data_fp8(run.shape, dyq, dys, wd.codes_t, wd.scales, run.gus, recv, ggu)
    rows_ref = dm.quant_rows_fp8(ggu, nrows)
    cols_ref = dm.quant_cols_fp8(ggu, recv)
    ns = dm.cols_fp8_slots(cap, E)
    ggu2 = torch.empty_like(ggu)
    rows = (torch.empty((cap, 2 * F), dtype=torch.uint8, device=DEV),
            torch.empty((2 * F // 128, cap), dtype=torch.float32, device=DEV))
    cols = (torch.empty((2 * F, 128 * ns), dtype=torch.uint8, device=DEV),
            torch.empty((ns, 2 * F), dtype=torch.float32, device=DEV))
    dm.moe_ffn_down_bwd_data_fp8_quant(run.shape, dyq, dys, wd.codes_t, wd.scales, run.gus, recv, ggu2,
                                       rows, cols)
    # codes only (the fp8 weight-gradient path): no bf16 output
    cols3 = (torch.empty_like(cols[0]), torch.empty_like(cols[1]))
    dm.moe_ffn_down_bwd_data_fp8_quant(run.shape, dyq, dys, wd.codes_t, wd.scales, run.gus, recv, None,
                                       None, cols3)
    torch.cuda.synchronize()
    prefix = recv.cpu().numpy().astype(np.int64)
    A = int(prefix[-1])
    check_equal("grad_gate_up", _u8(ggu2.view(torch.uint8))[:A], _u8(ggu.view(torch.uint8))[:A])
    check_equal("row codes", _u8(rows[0])[:A], _u8(rows_ref[0])[:A])
    check_equal("row scales", rows[1].cpu().numpy()[:, :A], rows_ref[1].cpu().numpy()[:, :A])
    lo = 0
    for e in range(E):
        hi = int(prefix[e])
        for r0 in range(lo, hi, 128):
            sl = _slot_of(prefix, e, r0)
            for got in (cols, cols3):
                check_equal(f"col codes e={e} slot={sl}", _u8(got[0])[:, sl * 128:(sl + 1) * 128],
                            _u8(cols_ref[0])[:, sl * 128:(sl + 1) * 128])
                check_equal(f"col scales e={e} slot={sl}", got[1].cpu().numpy()[sl], cols_ref[1].cpu().numpy()[sl])
        lo = hi


def test_quant_rows_fp8_every_bf16_value():
    """Every finite bf16 value through moe_quant_rows_fp8, bit-exact against the
    oracle's e4m3 rule: values sorted by magnitude, 127 per block plus one anchor
    448 * 2^k >= the block's largest magnitude, so x * (448/amax) = x / 2^k is exact
    and the codes are e4m3(x / 2^k) over the whole bf16 range."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = orc.bf16_to_f32(bits)
    keep = np.isfinite(vals)
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(np.abs(vals), kind="stable")
    bits, vals = bits[order], vals[order]
    nb = -(-len(bits) // 127)
    pad = nb * 127 - len(bits)
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(nb, 127)
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(nb, 127)
    top = np.abs(vals).max(axis=1).astype(np.float64)
    k = np.ceil(np.log2(np.maximum(top, 1e-300) / 448.0)).clip(-120, None)
    anchor = 448.0 * np.exp2(k)
    # the last blocks reach past 448 * 2^119: their anchor is the largest bf16
    anchor = np.where(anchor > 3.3895313892515355e38, 3.3895313892515355e38, anchor).astype(np.float32)
    assert np.all(np.isfinite(anchor)) and np.all(anchor >= top)
    rows = np.concatenate([orc.f32_to_bf16(anchor)[:, None], bits], axis=1)   # (nb, 128) bf16 bits
    codes, scales = dm.quant_rows_fp8(bf(rows))
    torch.cuda.synchronize()
    q, s = orc.quant_e4m3_rows(orc.bf16_to_f32(rows))
    check_equal("codes", _u8(codes), q)
    check_equal("scales", scales.cpu().numpy().T, s)   # stored (C/128, R)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fused_quantisation_of_h_in_the_gate_up_forward(name):
    """moe_ffn_gate_up_fwd_fp8_quant: G, U and h equal the plain entry's, and its
    per-128-token codes of h equal moe_quant_cols_fp8 run on that h."""
    inp = wl.layer_inputs(seed=47, **FP8_CASES[name])
    print(f"[fp8 fused h quant] case={name}", flush=True)
    run = Fp8Run(inp)
    run.dispatch()
    run.quant_weights()
    run.ffn8()
    F, E, cap = inp["F"], inp["E"], run.cap
    recv = run.d.ep_recv_counts
    wg, wu, _ = run.wq
    gus = torch.empty_like(run.gus)
    h = torch.empty_like(run.h)
    ns = dm.cols_fp8_slots(cap, E)
    hq_t = torch.empty((F, 128 * ns), dtype=torch.uint8, device=DEV)
    hs_t = torch.empty((ns, F), dtype=torch.float32, device=DEV)
    dm.moe_ffn_gate_up_fwd_fp8_quant(run.shape, run.xq, run.xs, wg.codes, wg.scales, wu.codes, wu.scales, recv,
                                     gus, h, hq_t, hs_t)
    ref_q, ref_s = dm.quant_cols_fp8(run.h, recv)
    torch.cuda.synchronize()
    prefix = recv.cpu().numpy().astype(np.int64)
    A = int(prefix[-1])
    check_equal("gate_up_save", _u8(gus.view(torch.uint8))[:A], _u8(run.gus.view(torch.uint8))[:A])
    check_equal("h", _u8(h.view(torch.uint8))[:A], _u8(run.h.view(torch.uint8))[:A])
    lo = 0
    for e in range(E):
        hi = int(prefix[e])
        for r0 in range(lo, hi, 128):
            sl = _slot_of(prefix, e, r0)
            check_equal(f"h col codes e={e} slot={sl}", _u8(hq_t)[:, sl * 128:(sl + 1) * 128],
                        _u8(ref_q)[:, sl * 128:(sl + 1) * 128])
            check_equal(f"h col scales e={e} slot={sl}", hs_t.cpu().numpy()[sl], ref_s.cpu().numpy()[sl])
        lo = hi
