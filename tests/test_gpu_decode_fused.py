"""GPU parity of moe_decode_fused, the layer forward of a decode batch in one
persistent launch (routing, gathered gate/up GEMM + SwiGLU, down GEMM, combine).

Its output must equal the separate entries' chain moe_dispatch ->
moe_grouped_ffn -> moe_combine bit for bit (same arithmetic and K order), and
the oracle's layer forward element by element; its err_flag equals
moe_dispatch's.  Cases cover the decode shape of the low_latency_combine page
(T=512, H=7168, top-8, 32 experts), special experts with both mask kinds and a
shared term, the int8 payload, an expert with more than 256 rows (two row passes
over one weight tile), empty experts, K=16 and K not dividing 64, one token, and
two calls in a row on one workspace (the control words are cleared by each call).
"""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl
import oracle as orc
from gpu_util import DEV, Run, bf, check_close, check_equal, f32

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="moe_decode_fused is switched off (returns MOE_ERR_UNSUPPORTED): its first two GPU "
                            "runs did not complete (a run past the time limit, then a memory fault in the "
                            "one-token case) and the cause is not found yet"),
]

CASES = {
    "one_token": dict(T=1, H=128, F=64, E=3, K=1),
    "special_mask2d_shared": dict(T=37, H=256, F=128, E=6, K=3, Z=1, C=1, Q=2, mask="2d", shared=True),
    "mask1d_int8_payload": dict(T=100, H=384, F=192, E=5, K=2, mask="1d", mask_active=71, qpay=True),
    "hot_expert_two_passes": dict(T=400, H=256, F=128, E=4, K=2, hot=True),
    "k16_many_empty_experts": dict(T=24, H=128, F=64, E=300, K=16),
    "decode_shape": dict(T=512, H=7168, F=2048, E=32, K=8),
}


def _inputs(name, seed=61):
    cfg = dict(CASES[name])
    shared, qpay, hot = cfg.pop("shared", False), cfg.pop("qpay", False), cfg.pop("hot", False)
    inp = wl.layer_inputs(seed=seed, grad=False, **cfg)
    if hot:
        # every token routes to expert 0 (first choice): 400 rows, two row passes
        idx = inp["topk_idx"]
        for t in range(idx.shape[0]):
            row = [e for e in idx[t] if e != 0]
            idx[t] = [0] + row[:idx.shape[1] - 1]
    rng = np.random.default_rng(seed + 1)
    inp["shared_expert_x"] = wl.to_bf16_bits(rng.standard_normal((cfg["T"], cfg["H"]), dtype=np.float32)) \
        if shared else None
    return inp, qpay


def _fused(run, inp, shape, ws=None):
    wg, wu, wd = (bf(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    out = torch.full((run.T, run.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    err = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    if ws is None:
        ws = dm.decode_fused_workspace(shape, DEV)
    sh = bf(inp["shared_expert_x"]) if inp.get("shared_expert_x") is not None else None
    dm.moe_decode_fused(shape, run.x, run.idx, run.w, run.mask, wg, wu, wd, sh, run.x, run.a1, run.a2, run.cv,
                        out, err, ws)
    torch.cuda.synchronize()
    return out, err, ws


def _separate(run, inp):
    run.dispatch()
    run.ffn()
    sh = bf(inp["shared_expert_x"]) if inp.get("shared_expert_x") is not None else None
    return run.combine(shared=sh)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_fused_matches_separate_entries_and_oracle(name):
    print(f"[decode fused] case={name}", flush=True)
    inp, qpay = _inputs(name)
    run = Run(inp)
    shape = run.shape
    if qpay:
        shape.comm_quant_mode = 2
        run.shape = shape
    out, err, _ = _fused(run, inp, shape)
    assert not int(err.item()) & dm.MOE_FLAG_SYNC_TIMEOUT, "a wait of the fused kernel timed out"
    ref_out = _separate(run, inp)
    check_equal("err_flag", err.cpu().numpy(), run.d.err_flag.cpu().numpy())
    assert torch.equal(out, ref_out), "differs from dispatch -> grouped FFN -> combine"
    check_close("out", f32(out), _oracle_forward(inp, qpay)["out"])


def _oracle_forward(inp, qpay):
    """The oracle's forward from its steps: route, dispatch, expert FFN, combine."""
    r = orc.route(inp["topk_idx"], inp["E"], Z=inp.get("Z", 0), C=inp.get("C", 0), Q=inp.get("Q", 0),
                  mask=inp.get("mask"))
    X = orc.dispatch(inp["x"], r)
    _, _, _, Y = orc.ffn_fwd(X, r.ep_recv_counts, inp["w_gate"], inp["w_up"], inp["w_down"])
    if qpay:
        Y = orc.qdq_rows_int8(Y)
    out = orc.combine(Y, r, inp["topk_weights"], inp.get("shared_expert_x"), inp["x"], inp.get("const_alpha_1"),
                      inp.get("const_alpha_2"), inp.get("const_v"))
    return {"out": out}


def test_decode_fused_two_calls_share_a_workspace():
    """The second call on the same workspace (smaller batch, other routing) is as
    correct as the first: each call leaves the control words zero."""
    print("[decode fused] two calls", flush=True)
    inp1 = wl.layer_inputs(T=200, H=256, F=128, E=8, K=4, seed=71, grad=False)
    run1 = Run(inp1)
    ws = torch.zeros(dm.moe_decode_fused_workspace_size(run1.shape), dtype=torch.uint8, device=DEV)
    out1, err1, _ = _fused(run1, inp1, run1.shape, ws)
    assert torch.equal(out1, _separate(run1, inp1))
    assert int(err1.item()) == 0
    ctrl = ws[:5 * 128].view(torch.int32)
    assert int(ctrl.abs().sum().item()) == 0, "control words not cleared"
    inp2 = dict(inp1)
    rng = np.random.default_rng(72)
    idx = np.stack([rng.permutation(8)[:4] for _ in range(120)]).astype(np.int32)
    inp2.update(T=120, x=inp1["x"][:120], topk_idx=idx, topk_weights=inp1["topk_weights"][:120])
    run2 = Run(inp2)
    out2, err2, _ = _fused(run2, inp2, run2.shape, ws)
    assert torch.equal(out2, _separate(run2, inp2))
    assert int(err2.item()) == 0
    check_close("out (second call)", f32(out2), _oracle_forward(inp2, False)["out"])
