"""moe_dispatch_noalloc (the dispatch whose routing scratch is the library's own
fixed device array) against moe_dispatch on the same inputs: every output bit
for bit, on two calls in a row, the second with a smaller input.  (That every
valid shape's scratch fits the array is a host-side check in test_abi.py.)"""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import moe_workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _both(kw, seed):
    inp = wl.layer_inputs(seed=seed, weights=False, grad=False, **kw)
    m = inp.get("mask")
    shape = dm.make_shape(inp["T"], inp["H"], inp["K"], inp["E"], zero_expert_num=inp.get("Z", 0),
                          copy_expert_num=inp.get("C", 0), const_expert_num=inp.get("Q", 0),
                          mask_ndim=0 if m is None else m.ndim)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(DEV)
    idx = torch.from_numpy(inp["topk_idx"]).to(DEV)
    mask = None if m is None else torch.from_numpy(m).to(DEV)
    ref = dm.dispatch(shape, x, idx, mask)
    # outputs pre-filled with a pattern, so an unwritten element shows
    out = dict(expand_x=torch.full_like(ref.expand_x, 7.0),
               assist=torch.full_like(ref.assist_info_for_combine, -77),
               etn=torch.full_like(ref.expert_token_nums, -5), recv=torch.full_like(ref.ep_recv_counts, -5),
               err=torch.full_like(ref.err_flag, 12345))
    dm.moe_dispatch_noalloc(shape, x, idx, mask, out["expand_x"], out["assist"], out["etn"], out["recv"],
                            out["err"])
    torch.cuda.synchronize()
    A = int(ref.ep_recv_counts[-1].item()) if kw["E"] else 0
    TK = kw["T"] * kw["K"]
    assert torch.equal(out["etn"], ref.expert_token_nums)
    assert torch.equal(out["recv"], ref.ep_recv_counts)
    assert torch.equal(out["err"], ref.err_flag)
    assert torch.equal(out["assist"][:TK + A], ref.assist_info_for_combine[:TK + A])
    assert torch.equal(out["expand_x"][:A].view(torch.int16), ref.expand_x[:A].view(torch.int16))
    return A


def test_noalloc_dispatch_matches_dispatch_twice_second_smaller():
    big = dict(T=8192, H=1536, F=0, E=64, K=8)                      # the page-1 layer
    small = dict(T=300, H=256, F=0, E=16, K=4, Z=1, C=1, Q=1, mask="2d")
    print("[noalloc] page-1 shape", flush=True)
    assert _both(big, seed=1) == 8192 * 8
    print("[noalloc] smaller second call", flush=True)
    assert _both(small, seed=2) > 0
