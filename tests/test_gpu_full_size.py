"""GPU parity at the workloads' full sizes, through the same C entry points the
benchmark times, checked against the oracle on what it can compute piece by
piece: every index/count/map in full, expert-FFN rows, combine and gradient
tokens on samples, and weight gradients of sampled experts on sampled F columns
(each F column of G, U, h, dG, dU and of the weight gradients depends on no
other column, so the oracle run on a column slice gives those columns exactly).
"""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import (DEV, OUTLIERS_8BIT, REL_L2_8BIT, RHO_CHAIN, RHO_FP32, ULPS_KERNEL, Fp8Run, Run, bf, check_close, check_equal,
                      contraction_mag, dw_mag, f32)

pytestmark = pytest.mark.gpu

REL_FP8 = REL_L2_8BIT


def _expert_of_rows(r, rows):
    return np.searchsorted(r.ep_recv_counts, rows, side="right")


def oracle_rows(inp, r, rows):
    """Oracle G, U, h, y of the given expanded rows, expert by expert."""
    rows = np.asarray(rows)
    K = r.K
    es = _expert_of_rows(r, rows)
    xr = orc.bf16_to_f32(inp["x"])[r.row2slot[rows] // K]
    F, H = inp["F"], inp["H"]
    G = np.zeros((len(rows), F), np.float32)
    U, Hh = np.zeros_like(G), np.zeros_like(G)
    Y = np.zeros((len(rows), H), np.float32)
    for e in np.unique(es):
        sel = np.nonzero(es == e)[0]
        g, u, h, y = orc.ffn_fwd(xr[sel], np.array([len(sel)]), inp["w_gate"][e:e + 1],
                                 inp["w_up"][e:e + 1], inp["w_down"][e:e + 1])
        G[sel], U[sel], Hh[sel], Y[sel] = g, u, h, y
    return G, U, Hh, Y


def sub_route(r, tokens, row_map=None):
    """Route restricted to the given tokens; routed codes renumbered 0.. in slot order."""
    codes = r.slot2row.reshape(r.T, r.K)[tokens].reshape(-1).copy()
    routed = np.nonzero(codes >= 0)[0]
    rows = codes[routed].copy()
    codes[routed] = np.arange(len(routed))
    sr = orc.Route(len(tokens), r.K, r.E, None, None, codes.astype(np.int32), None, 0)
    return sr, rows


def _sample(rng, n, k):
    return np.sort(rng.choice(n, size=min(n, k), replace=False))


def _check_sampled_layer(inp, run, r, out, gy, gw, ggu, gxe, gwg, gwu, gwd, gx, rng,
                         n_rows=96, n_tok=64, experts=None, n_cols=24, shared=None):
    """Sampled checks of a whole layer step; `shared` = (sY16, s_dX16) oracle arrays
    for the sampled tokens' shared expert, or None."""
    K, F = r.K, inp["F"]
    A = r.A
    # expert FFN rows
    rows = _sample(rng, A, n_rows)
    G, U, Hh, Y = oracle_rows(inp, r, rows)
    check_close("G rows", f32(run.gus[rows, :F]), G, ulps=ULPS_KERNEL)
    check_close("U rows", f32(run.gus[rows, F:]), U, ulps=ULPS_KERNEL)
    check_close("h rows", f32(run.h[rows]), Hh, ulps=ULPS_KERNEL)
    check_close("y rows", f32(run.y[rows]), Y)
    # tokens: combine, combine backward, FFN backward of their rows, dispatch backward
    toks = _sample(rng, r.T, n_tok)
    sr, trows = sub_route(r, toks)
    _, _, _, Yt = oracle_rows(inp, r, trows)
    sh = None if shared is None else shared[0](toks)
    ref_out = orc.combine(Yt, sr, inp["topk_weights"][toks], sh, inp["x"][toks],
                          inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"))
    check_close("out tokens", f32(out[toks]), ref_out)
    dY, dw = orc.combine_bwd(inp["grad_out"][toks], Yt, sr, inp["topk_weights"][toks], inp["x"][toks],
                             inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"))
    check_equal("grad_y rows", f32(gy[trows]), dY)
    check_close("grad_topk_weights tokens", f32(gw[toks]), dw, ulps=0, rho=RHO_CHAIN,
                mag=dw_mag(sr, Yt, inp["grad_out"][toks], inp["x"][toks], inp.get("const_alpha_1"),
                           inp.get("const_alpha_2"), inp.get("const_v")))
    Gt, Ut, Ht, _ = oracle_rows(inp, r, trows)
    es = _expert_of_rows(r, trows)
    xr = orc.bf16_to_f32(inp["x"])[r.row2slot[trows] // K]
    dX = np.zeros((len(trows), inp["H"]), np.float32)
    for e in np.unique(es):
        sel = np.nonzero(es == e)[0]
        _, dx_e, _, _, _ = orc.ffn_bwd(dY[sel], xr[sel], Gt[sel], Ut[sel], Ht[sel], np.array([len(sel)]),
                                       inp["w_gate"][e:e + 1], inp["w_up"][e:e + 1], inp["w_down"][e:e + 1])
        dX[sel] = dx_e
    check_close("grad_expand_x rows", f32(gxe[trows]), dX)
    acc = None if shared is None else shared[1](toks)
    ref_dx = orc.dispatch_bwd(dX, sr, inp["topk_weights"][toks], inp["grad_out"][toks],
                              inp.get("const_alpha_1"), acc)
    check_close("grad_x tokens", f32(gx[toks]), ref_dx)
    # weight gradients of sampled experts, sampled F columns
    if experts is None:
        nz = np.nonzero(r.counts)[0]
        experts = [int(nz[0]), int(nz[len(nz) // 2]), int(nz[-1])]
    for e in experts:
        lo, hi = r.row_range(e)
        if hi == lo:
            continue
        erows = np.arange(lo, hi)
        toks_e = r.row2slot[erows] // K
        ks_e = r.row2slot[erows] % K
        w_e = inp["topk_weights"][toks_e, ks_e]
        dY_e = orc.round_bf16((w_e[:, None] * orc.bf16_to_f32(inp["grad_out"][toks_e])).astype(np.float32))
        X_e = orc.bf16_to_f32(inp["x"])[toks_e]
        fs = _sample(rng, F, n_cols)
        wg, wu, wd = inp["w_gate"][e:e + 1, fs], inp["w_up"][e:e + 1, fs], inp["w_down"][e:e + 1][:, :, fs]
        g, u, h, _ = orc.ffn_fwd(X_e, np.array([hi - lo]), wg, wu, wd)
        dgu, _, dwg, dwu, dwd = orc.ffn_bwd(dY_e, X_e, g, u, h, np.array([hi - lo]), wg, wu, wd)
        n_e, nf = np.array([hi - lo]), len(fs)
        check_close(f"grad_gate_up e={e}", f32(ggu[lo:hi][:, np.concatenate([fs, F + fs])]), dgu)
        check_close(f"grad_w_gate e={e}", f32(gwg[e][fs]), dwg[0], ulps=0, rho=RHO_CHAIN,
                    mag=contraction_mag(dgu[:, :nf], X_e, n_e)[0])
        check_close(f"grad_w_up e={e}", f32(gwu[e][fs]), dwu[0], ulps=0, rho=RHO_CHAIN,
                    mag=contraction_mag(dgu[:, nf:], X_e, n_e)[0])
        check_close(f"grad_w_down e={e}", f32(gwd[e][:, fs]), dwd[0], ulps=0, rho=RHO_CHAIN,
                    mag=contraction_mag(dY_e, h, n_e)[0])


def _layer_step(run, shared_x=None, accum=None):
    run.ffn()
    out = run.combine(shared=shared_x)
    g = bf(run.inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe, gwg, gwu, gwd = run.ffn_bwd(gy)
    gx = run.dispatch_bwd(gxe, g, accum)
    return out, gy, gw, ggu, gxe, gwg, gwu, gwd, gx


@pytest.mark.parametrize("T", [2048, 4096, 8192])
def test_page1_benchmark_shape_full_size(T):
    """T tokens at H=1536, F=480, E=64, K=8: the benchmark's workload and launch
    shapes at the token counts of the Triton-distributed page's summary table
    (1024 tokens is a layer parity case of its own)."""
    print(f"[full] page1 T={T}", flush=True)
    cfg = dict(wl.WORKLOADS["page1"], T=T)
    inp = wl.layer_inputs(**cfg, seed=0)
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"])
    check_equal("expert_token_nums", run.d.expert_token_nums.cpu().numpy(), r.counts)
    check_equal("ep_recv_counts", run.d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_equal("slot2row", run.d.slot2row(r.T, r.K).cpu().numpy(), r.slot2row)
    check_equal("row2slot", run.d.row2slot(r.T, r.K)[:r.A].cpu().numpy(), r.row2slot)
    assert r.counts.sum() == T * 8
    rng = np.random.default_rng(11)
    rows = _sample(rng, r.A, 512)
    xf = orc.bf16_to_f32(inp["x"])
    check_equal("expand_x rows", f32(run.d.expand_x[rows]), xf[r.row2slot[rows] // r.K])
    res = _layer_step(run)
    _check_sampled_layer(inp, run, r, *res, rng)


def test_page1_rank_share_full_size():
    """One of the benchmark page's four ranks: 16 experts receiving 65,536 rows
    (top-8 of 16 over 8192 tokens: 4096 rows per expert, bigger GEMM groups than
    the 64-expert layer), H=1536, F=480."""
    print("[full] page1 rank share E=16", flush=True)
    inp = wl.layer_inputs(T=8192, H=1536, F=480, E=16, K=8, seed=0)
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"])
    check_equal("ep_recv_counts", run.d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_equal("row2slot", run.d.row2slot(r.T, r.K)[:r.A].cpu().numpy(), r.row2slot)
    res = _layer_step(run)
    _check_sampled_layer(inp, run, r, *res, np.random.default_rng(12))


def test_combine_stress_full_size():
    """T=4096, H=7168, K=8, 256 routed + 1 zero + 1 copy + 2 constant experts,
    2-D mask with 10% false, shared_expert_x: combine, its backward and dispatch
    backward checked bit for bit (dw within tolerance) on every token."""
    print("[full] combine stress", flush=True)
    inp = wl.combine_inputs(**{k: v for k, v in wl.WORKLOADS["combine_stress"].items()}, seed=0)
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"], inp["Z"], inp["C"], inp["Q"], inp["mask"])
    assert int(run.d.err_flag.item()) == 0 and run.A == r.A
    y = bf(inp["y"])
    out = run.combine(y=y, shared=bf(inp["shared_expert_x"]))
    Y = orc.bf16_to_f32(inp["y"])[:r.A]
    ref = orc.combine(Y, r, inp["topk_weights"], inp["shared_expert_x"], inp["x"], inp["const_alpha_1"],
                      inp["const_alpha_2"], inp["const_v"])
    check_equal("out", f32(out), ref)
    gy, gw = run.combine_bwd(bf(inp["grad_out"]), y=y)
    dY, dw = orc.combine_bwd(inp["grad_out"], Y, r, inp["topk_weights"], inp["x"], inp["const_alpha_1"],
                             inp["const_alpha_2"], inp["const_v"])
    check_equal("grad_y", f32(gy[:r.A]), dY)
    check_close("grad_topk_weights", f32(gw), dw, ulps=0, max_abs=1e-3, rel_l2=1e-5)
    gx = run.dispatch_bwd(y, bf(inp["grad_out"]))
    ref_dx = orc.dispatch_bwd(Y, r, inp["topk_weights"], inp["grad_out"], inp["const_alpha_1"])
    check_equal("grad_x", f32(gx), ref_dx)


def test_decode_forward_full_size():
    """Decode batch, forward only: T=512, H=7168, F=2048, E=32, K=8 (every expert on
    one GPU; about 128 rows per expert, so every GEMM tile is a partial one).  The
    whole forward against the oracle: maps bit-exact, G/U/h/y rows and out in full."""
    print("[full] decode", flush=True)
    inp = wl.layer_inputs(**wl.WORKLOADS["decode"], seed=0, grad=False)
    run = Run(inp)
    run.dispatch()
    run.ffn()
    out = run.combine()
    f = orc.layer_fwd(inp, prec="parity")
    r = f["route"]
    A, F = r.A, inp["F"]
    check_equal("ep_recv_counts", run.d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_close("G", f32(run.gus[:A, :F]), f["G"], ulps=ULPS_KERNEL)
    check_close("U", f32(run.gus[:A, F:]), f["U"], ulps=ULPS_KERNEL)
    check_close("h", f32(run.h[:A]), f["Hh"], ulps=ULPS_KERNEL)
    check_close("y", f32(run.y[:A]), f["Y"])
    check_close("out", f32(out), f["out"])


def test_dsv3_proxy_full_size():
    """T=4096, H=7168, F=2048, E=32, K=8, Zipf(1.2)-skewed routing, one shared
    SwiGLU expert on all tokens, fwd+bwd (the shared expert through the same
    grouped FFN entries with one expert of T rows)."""
    print("[full] dsv3 proxy", flush=True)
    inp = wl.layer_inputs(**wl.WORKLOADS["dsv3_proxy"], seed=0)
    T, H, F = inp["T"], inp["H"], inp["F"]
    run = Run(inp)
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"])
    check_equal("ep_recv_counts", run.d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_equal("row2slot", run.d.row2slot(T, r.K)[:r.A].cpu().numpy(), r.row2slot)
    assert r.counts.max() > 2 * r.counts.mean()   # the routing is skewed
    # shared expert forward on all T tokens
    ss = dm.shared_expert_shape(T, H, F)
    scnt = torch.full((1,), T, dtype=torch.int32, device=DEV)
    swg, swu, swd = bf(inp["shared_w_gate"]), bf(inp["shared_w_up"]), bf(inp["shared_w_down"])
    s_gus = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=DEV)
    s_h = torch.empty((T, F), dtype=torch.bfloat16, device=DEV)
    s_y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    dm.moe_grouped_ffn(ss, run.x, swg, swu, swd, scnt, s_gus, s_h, s_y)
    g = bf(inp["grad_out"])
    s_ggu = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=DEV)
    s_dx = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    s_gw = [torch.empty(t.shape, dtype=torch.float32, device=DEV) for t in (swg, swu, swd)]
    dm.moe_grouped_ffn_bwd(ss, g, run.x, s_gus, s_h, swg, swu, swd, scnt, s_ggu, s_dx, *s_gw)
    torch.cuda.synchronize()
    res = _layer_step(run, shared_x=s_y, accum=s_dx)

    xf = orc.bf16_to_f32(inp["x"])
    sw = (inp["shared_w_gate"], inp["shared_w_up"], inp["shared_w_down"])

    def shared_fwd(toks):
        return orc.ffn_fwd(xf[toks], np.array([len(toks)]), *sw)

    def shared_y(toks):
        return shared_fwd(toks)[3]

    def shared_dx(toks):
        g_, u_, h_, _ = shared_fwd(toks)
        return orc.ffn_bwd(orc.bf16_to_f32(inp["grad_out"][toks]), xf[toks], g_, u_, h_,
                           np.array([len(toks)]), *sw)[1]

    rng = np.random.default_rng(12)
    _check_sampled_layer(inp, run, r, *res, rng, n_rows=64, n_tok=32, n_cols=8,
                         shared=(shared_y, shared_dx))
    # shared expert: its output on sampled tokens, its weight gradients on sampled columns
    toks = _sample(rng, T, 32)
    check_close("shared y tokens", f32(s_y[toks]), shared_y(toks))
    fs = _sample(rng, F, 8)
    wg, wu, wd = sw[0][:, fs], sw[1][:, fs], sw[2][:, :, fs]
    g_, u_, h_, _ = orc.ffn_fwd(xf, np.array([T]), wg, wu, wd)
    dgu, _, dwg, dwu, dwd = orc.ffn_bwd(orc.bf16_to_f32(inp["grad_out"]), xf, g_, u_, h_, np.array([T]),
                                        wg, wu, wd)
    nT, nf, dOut = np.array([T]), len(fs), orc.bf16_to_f32(inp["grad_out"])
    check_close("shared grad_gate_up cols", f32(s_ggu[:, np.concatenate([fs, F + fs])]), dgu)
    check_close("shared grad_w_gate", f32(s_gw[0][0][fs]), dwg[0], ulps=0, rho=RHO_CHAIN,
                mag=contraction_mag(dgu[:, :nf], xf, nT)[0])
    check_close("shared grad_w_up", f32(s_gw[1][0][fs]), dwu[0], ulps=0, rho=RHO_CHAIN,
                mag=contraction_mag(dgu[:, nf:], xf, nT)[0])
    check_close("shared grad_w_down", f32(s_gw[2][0][:, fs]), dwd[0], ulps=0, rho=RHO_CHAIN,
                mag=contraction_mag(dOut, h_, nT)[0])


@pytest.mark.timeout(900)
def test_mixtral_fp8_full_size():
    """T=8192, H=4096, F=14336, E=8, K=2 on the fp8 path (e4m3 block-scaled
    forward and data-gradient GEMMs, bf16 weight gradients, int8 combine
    payload): the chain the benchmark times.  Against the oracle: the route in
    full; the fp8 codes (both layouts) and block scales of the two busiest
    experts bit for bit; sampled rows of those experts through the forward;
    tokens routed to exactly those two experts through combine, its backward,
    the data gradients and dispatch backward; one 128-column F block of the
    busiest expert through G, U, h, dG, dU and the three weight gradients (an F
    block of the weights is one column of quantisation blocks, so the oracle on
    the block slice gives those columns exactly)."""
    print("[full] mixtral fp8", flush=True)
    inp = wl.layer_inputs(**{k: v for k, v in wl.WORKLOADS["mixtral"].items()}, seed=0)
    T, H, F, K = inp["T"], inp["H"], inp["F"], inp["K"]
    run = Fp8Run(inp)
    run.shape.comm_quant_mode = 2
    run.dispatch()
    r = orc.route(inp["topk_idx"], inp["E"])
    check_equal("ep_recv_counts", run.d.ep_recv_counts.cpu().numpy(), r.ep_recv_counts)
    check_equal("row2slot", run.d.row2slot(T, K)[:r.A].cpu().numpy(), r.row2slot)
    run.quant_weights()
    run.ffn8()
    out = run.combine()
    g = bf(inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe = run.ffn8_bwd_data(gy)
    gwg, gwu, gwd = run.weight_grads(gy, ggu)
    gx = run.dispatch_bwd(gxe, g)
    print("[full] mixtral fp8: GPU chain done, oracle quantisation of two experts", flush=True)

    ea, eb = (int(e) for e in np.argsort(-r.counts, kind="stable")[:2])
    names = ("w_gate", "w_up", "w_down")
    wq = {}
    for e in (ea, eb):
        wq[e] = tuple(orc.quant_weights_fp8(inp[k][e:e + 1]) for k in names)
        for (codes, scales), q, name in zip(wq[e], run.wq, names):
            check_equal(f"{name} codes e={e}", q.codes[e].cpu().numpy(), codes[0])
            check_equal(f"{name} codes_t e={e}", q.codes_t[e].cpu().numpy(), codes[0].T)
            check_equal(f"{name} scales e={e}", q.scales[e].cpu().numpy(), scales[0])
    X = orc.bf16_to_f32(inp["x"])
    expert_of = _expert_of_rows(r, np.arange(r.A))

    def fwd_rows(rows):
        """Oracle fp8 forward (G, U, h, y) of expanded rows, expert by expert."""
        G = np.zeros((len(rows), F), np.float32)
        U, Hh = np.zeros_like(G), np.zeros_like(G)
        Y = np.zeros((len(rows), H), np.float32)
        es = expert_of[rows]
        for e in np.unique(es):
            sel = np.nonzero(es == e)[0]
            xr = X[r.row2slot[rows[sel]] // K]
            G[sel], U[sel], Hh[sel], Y[sel] = orc.ffn_fwd_fp8(xr, np.array([len(sel)]), *wq[int(e)])
        return G, U, Hh, Y

    rng = np.random.default_rng(13)
    # sampled rows of both experts, and the rows of tokens routed to exactly
    # those two experts; one oracle forward over all of them
    samp = np.concatenate([lo + _sample(rng, hi - lo, 16) for lo, hi in (r.row_range(ea), r.row_range(eb))])
    idx = inp["topk_idx"]
    pair = np.nonzero(((idx[:, 0] == ea) & (idx[:, 1] == eb)) | ((idx[:, 0] == eb) & (idx[:, 1] == ea)))[0]
    assert len(pair) >= 16
    toks = pair[_sample(rng, len(pair), 16)]
    sr, trows = sub_route(r, toks)
    allrows = np.concatenate([samp, trows])
    Ga, Ua, Ha, Ya = fwd_rows(allrows)
    ns = len(samp)
    check_close("G rows", f32(run.gus[samp, :F]), Ga[:ns], ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("U rows", f32(run.gus[samp, F:]), Ua[:ns], ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("h rows", f32(run.h[samp]), Ha[:ns], ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("y rows", f32(run.y[samp]), Ya[:ns], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    Gt, Ut, Ht, Yt = Ga[ns:], Ua[ns:], Ha[ns:], Ya[ns:]
    Yc = orc.qdq_rows_int8(Yt)
    w_t = inp["topk_weights"][toks]
    ref_out = orc.combine(Yc, sr, w_t, None, inp["x"][toks], None, None, None)
    check_close("out tokens", f32(out[toks]), ref_out, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    dY, dw = orc.combine_bwd(inp["grad_out"][toks], Yc, sr, w_t, inp["x"][toks], None, None, None)
    check_equal("grad_y rows", f32(gy[trows]), dY)
    check_close("grad_topk_weights tokens", f32(gw[toks]), dw, ulps=0, rel_l2=REL_FP8, rho=RHO_CHAIN,
                mag=dw_mag(sr, Yc, inp["grad_out"][toks]))
    dGU = np.zeros((len(trows), 2 * F), np.float32)
    dX = np.zeros((len(trows), H), np.float32)
    es = expert_of[trows]
    for e in np.unique(es):
        sel = np.nonzero(es == e)[0]
        xr = X[r.row2slot[trows[sel]] // K]
        dGU[sel], dX[sel], _, _, _ = orc.ffn_bwd_fp8(dY[sel], xr, Gt[sel], Ut[sel], Ht[sel],
                                                     np.array([len(sel)]), *wq[int(e)])
    check_close("grad_gate_up rows", f32(ggu[trows]), dGU, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_expand_x rows", f32(gxe[trows]), dX, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    ref_dx = orc.dispatch_bwd(dX, sr, w_t, inp["grad_out"][toks], None, None)
    check_close("grad_x tokens", f32(gx[toks]), ref_dx, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)

    # one F block of the busiest expert, all its rows
    lo, hi = r.row_range(ea)
    erows = np.arange(lo, hi)
    toks_e, ks_e = r.row2slot[erows] // K, r.row2slot[erows] % K
    w_e = inp["topk_weights"][toks_e, ks_e]
    dY_e = orc.round_bf16((w_e[:, None] * orc.bf16_to_f32(inp["grad_out"][toks_e])).astype(np.float32))
    X_e = X[toks_e]
    b = F // 256
    cs = slice(128 * b, 128 * b + 128)
    (cg, sg), (cu, su), (cd, sd) = wq[ea]
    wq_b = ((cg[:, cs], sg[:, b:b + 1]), (cu[:, cs], su[:, b:b + 1]), (cd[:, :, cs], sd[:, :, b:b + 1]))
    n_e = np.array([hi - lo])
    G, U, Hh, _ = orc.ffn_fwd_fp8(X_e, n_e, *wq_b)
    check_close("G block", f32(run.gus[lo:hi, cs]), G, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("U block", f32(run.gus[lo:hi, F + 128 * b:F + 128 * b + 128]), U, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    check_close("h block", f32(run.h[lo:hi, cs]), Hh, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
    dgu, _, dwg, dwu, dwd = orc.ffn_bwd_fp8(dY_e, X_e, G, U, Hh, n_e, *wq_b)
    check_close("grad_gate block", f32(ggu[lo:hi, cs]), dgu[:, :128], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_up block", f32(ggu[lo:hi, F + 128 * b:F + 128 * b + 128]), dgu[:, 128:], rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
    check_close("grad_w_gate block", f32(gwg[ea][cs]), dwg[0], ulps=0, rel_l2=REL_FP8, rho=RHO_CHAIN,
                mag=contraction_mag(dgu[:, :128], X_e, n_e)[0])
    check_close("grad_w_up block", f32(gwu[ea][cs]), dwu[0], ulps=0, rel_l2=REL_FP8, rho=RHO_CHAIN,
                mag=contraction_mag(dgu[:, 128:], X_e, n_e)[0])
    check_close("grad_w_down block", f32(gwd[ea][:, cs]), dwd[0], ulps=0, rel_l2=REL_FP8, rho=RHO_CHAIN,
                mag=contraction_mag(dY_e, Hh, n_e)[0])


@pytest.mark.timeout(300)   # the oracle's MX quantisation of one expert's weights takes about a minute
def test_mixtral_mx_full_size():
    """T=8192, H=4096, F=14336, E=8, K=2 through the microscaled GEMM chain the
    benchmark times (the down GEMM and the gate/up data gradient read the MX codes
    that the preceding GEMMs' epilogues wrote).  Against the quantiser: those fused
    codes and scales over every routed row, bit for bit.  Against the oracle: 16
    sampled rows of the busiest expert (its tiles include the ragged last one)
    through G, U, h, y, dG|dU and dX (MX quantisation runs along rows, so a row's results need no
    other row).  y and dX are one requantisation further on (h, dG|dU), where a
    1-ulp bf16 difference can move a code by one step: their max bar is 5e-2, the
    relative L2 bar the same as elsewhere."""
    print("[full] mixtral mx", flush=True)
    inp = wl.layer_inputs(**{k: v for k, v in wl.WORKLOADS["mixtral"].items()}, seed=1)
    T, H, F, K, E = inp["T"], inp["H"], inp["F"], inp["K"], inp["E"]
    run = Run(inp)
    run.dispatch()
    cap = run.cap
    recv = run.d.ep_recv_counts
    nrows = recv[-1:]
    wq = [dm.MxWeights.quantize(bf(inp[k])) for k in ("w_gate", "w_up", "w_down")]
    u8 = lambda *n: torch.empty(n, dtype=torch.uint8, device=DEV)
    b16 = lambda *n: torch.empty(n, dtype=torch.bfloat16, device=DEV)
    xq, xs = dm.quant_rows_mx(run.d.expand_x, nrows)
    gus, h, y = b16(cap, 2 * F), b16(cap, F), b16(cap, H)
    hq, hs = u8(cap, F), u8(cap, F // 32)
    dm.moe_ffn_gate_up_fwd_mx(run.shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales, recv, gus, h,
                              (hq, hs))
    dm.moe_ffn_down_fwd_mx(run.shape, hq, hs, wq[2].codes, wq[2].scales, recv, y)
    dY_bits = wl.to_bf16_bits(np.random.default_rng(31).standard_normal((cap, H), dtype=np.float32) * 0.05)
    dyq, dys = dm.quant_rows_mx(bf(dY_bits), nrows)
    ggu, dgq, dgs = b16(cap, 2 * F), u8(cap, 2 * F), u8(cap, 2 * F // 32)
    dm.moe_ffn_down_bwd_data_mx(run.shape, dyq, dys, wq[2].codes_t, wq[2].scales_t, gus, recv, ggu, (dgq, dgs))
    gxe = b16(cap, H)
    dm.moe_ffn_gate_up_bwd_data_mx(run.shape, dgq, dgs, wq[0].codes_t, wq[0].scales_t, wq[1].codes_t,
                                   wq[1].scales_t, recv, gxe)
    torch.cuda.synchronize()
    r = orc.route(inp["topk_idx"], E)
    A = r.A
    check_equal("ep_recv_counts", recv.cpu().numpy(), r.ep_recv_counts)
    # fused codes against the row quantiser on the same bf16 outputs, on the GPU
    for name, src, q, s, C in (("h", h, hq, hs, F), ("dG|dU", ggu, dgq, dgs, 2 * F)):
        q2, s2 = dm.quant_rows_mx(src, nrows)
        torch.cuda.synchronize()
        assert torch.equal(q[:A], q2[:A]), f"{name} codes (fused) differ"
        sv, sv2 = s.view(C // 128, cap, 4)[:, :A], s2.view(C // 128, cap, 4)[:, :A]
        assert torch.equal(sv, sv2), f"{name} scales (fused) differ"
        del q2, s2
    print("[full] mixtral mx: GPU chain done, oracle of the busiest expert", flush=True)
    rng = np.random.default_rng(32)
    X = orc.bf16_to_f32(inp["x"])
    for e in (int(np.argmax(r.counts)),):
        lo, hi = r.row_range(e)
        rows = lo + np.union1d(_sample(rng, hi - lo, 15), [hi - lo - 1])   # the last row is in the ragged tile
        owq = tuple(orc.quant_weights_mx(inp[k][e:e + 1]) for k in ("w_gate", "w_up", "w_down"))
        n = np.array([len(rows)])
        Xs = X[r.row2slot[rows] // K]
        G, U, Hh, Y = orc.ffn_fwd_mx(Xs, n, *owq)
        check_close(f"G e={e}", f32(gus[rows, :F]), G, ulps=ULPS_KERNEL, rel_l2=2e-3)
        check_close(f"U e={e}", f32(gus[rows, F:]), U, ulps=ULPS_KERNEL, rel_l2=2e-3)
        check_close(f"h e={e}", f32(h[rows]), Hh, ulps=ULPS_KERNEL, rel_l2=REL_FP8)
        check_close(f"y e={e}", f32(y[rows]), Y, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
        dGU, dX, _, _, _ = orc.ffn_bwd_mx(orc.bf16_to_f32(dY_bits[rows]), Xs, G, U, Hh, n, *owq)
        check_close(f"grad_gate_up e={e}", f32(ggu[rows]), dGU, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)
        check_close(f"grad_expand_x e={e}", f32(gxe[rows]), dX, rel_l2=REL_FP8, outliers=OUTLIERS_8BIT)


@pytest.mark.timeout(300)   # host generation of the four full-size operands takes a few seconds
def test_mixtral_fp8_weight_gradients_full_size():
    """The fp8 weight-gradient GEMMs (per-128-token codes) at the Mixtral-style
    size (T=8192, K=2 over E=8 experts, H=4096, F=14336), in the launch the
    benchmark's fp8-weight-gradient variant makes.  Every expert's dW_down on 16
    sampled rows x 16 sampled columns, and dW_gate, dW_up on 16 x 16, against the
    oracle's wgrad_fp8 on the matching operand columns: the quantisation runs
    down each column within a 128-token slot, so a column slice gives those
    entries exactly.  The codes are identical on both sides; the bar is the
    accumulation-order bar of the small cases (1e-4)."""
    print("[full] mixtral fp8 weight gradients", flush=True)
    H, F, E, K, T = 4096, 14336, 8, 2, 8192
    rng = np.random.default_rng(41)
    idx, _ = wl.router(rng.standard_normal((T, E)).astype(np.float32), K, True)
    r = orc.route(idx, E)
    prefix = r.ep_recv_counts.astype(np.int64)
    A = int(prefix[-1])
    cap = A + 128 * E
    mats = {k: wl.to_bf16_bits(rng.standard_normal((cap, d), dtype=np.float32) * s)
            for k, d, s in (("dY", H, 0.1), ("h", F, 1.0), ("dGU", 2 * F, 0.05), ("x", H, 1.0))}
    counts = torch.from_numpy(prefix.astype(np.int32)).to(DEV)
    shape = dm.make_shape(T, H, K, E, F=F, capacity=cap)
    q = {k: dm.quant_cols_fp8(bf(v), counts) for k, v in mats.items()}
    gwd = torch.full((E, H, F), float("nan"), dtype=torch.float32, device=DEV)
    gwg = torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV)
    gwu = torch.full((E, F, H), float("nan"), dtype=torch.float32, device=DEV)
    dm.moe_ffn_down_bwd_weight_fp8(shape, *q["dY"], *q["h"], counts, gwd)
    dm.moe_ffn_gate_up_bwd_weight_fp8(shape, *q["dGU"], *q["x"], counts, gwg, gwu)
    torch.cuda.synchronize()
    print("[full] mixtral fp8 weight gradients: GPU done, oracle on column samples", flush=True)
    hs = np.union1d(_sample(rng, H, 15), [H - 1])
    fs = np.union1d(_sample(rng, F, 15), [F - 1])
    col = lambda k, c: orc.bf16_to_f32(mats[k][:A][:, c])
    ref_d = orc.wgrad_fp8(col("dY", hs), col("h", fs), prefix)
    ref_g = orc.wgrad_fp8(col("dGU", fs), col("x", hs), prefix)
    ref_u = orc.wgrad_fp8(col("dGU", F + fs), col("x", hs), prefix)
    ih, jf = torch.from_numpy(hs).to(DEV), torch.from_numpy(fs).to(DEV)
    dq = lambda k, c: orc.qdq_cols_fp8(col(k, c), prefix)
    md = contraction_mag(dq("dY", hs), dq("h", fs), prefix)
    mg = contraction_mag(dq("dGU", fs), dq("x", hs), prefix)
    mu = contraction_mag(dq("dGU", F + fs), dq("x", hs), prefix)
    # identical codes: only fp32 accumulation against float64 (RHO_FP32)
    check_close("grad_w_down", f32(gwd[:, ih][:, :, jf]), ref_d, ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=md, rho=RHO_FP32)
    check_close("grad_w_gate", f32(gwg[:, jf][:, :, ih]), ref_g, ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=mg, rho=RHO_FP32)
    check_close("grad_w_up", f32(gwu[:, jf][:, :, ih]), ref_u, ulps=0, max_abs=1e-4, rel_l2=1e-4, mag=mu, rho=RHO_FP32)
