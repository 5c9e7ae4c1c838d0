"""GPU parity of the router (moe_router / moe_router_bwd) against the oracle's
softmax top-K gating: the selected ids bit-exact (both sides select on the same
fp32 logits), the weights and the logit gradients within fp32 rounding of the
float64 oracle."""
import numpy as np
import pytest
import torch

import dispatch_expert_gemm_amd as dm
import oracle as orc
from gpu_util import DEV, check_close

pytestmark = pytest.mark.gpu


def _logits(T, n, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        z = rng.standard_normal((T, n)).astype(np.float32) * 2
    elif kind == "ties":       # few distinct values: many equal logits
        z = rng.integers(-2, 3, size=(T, n)).astype(np.float32)
    elif kind == "neg_inf":    # some ids impossible
        z = rng.standard_normal((T, n)).astype(np.float32)
        z[rng.random((T, n)) < 0.3] = -np.inf
        z[:, 0] = 0.5          # every row keeps a finite logit
    else:
        raise ValueError(kind)
    return z


CASES = {
    "page1_64": (1000, 64, 8, "normal"),
    "stress_260": (333, 260, 8, "normal"),
    "one_id": (200, 1, 1, "normal"),
    "all_ids": (77, 7, 7, "normal"),
    "ties": (257, 100, 16, "ties"),
    "neg_inf": (129, 40, 4, "neg_inf"),
    "max_ids": (50, 4096, 16, "normal"),
    "ragged_65": (31, 65, 3, "normal"),
}


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_router_forward_backward(name, renorm):
    T, n, K, kind = CASES[name]
    print(f"[router] case={name} renorm={renorm}", flush=True)
    z = _logits(T, n, kind, seed=list(CASES).index(name))
    lg = torch.from_numpy(z).to(DEV)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    dm.moe_router(lg, K, renorm, idx, w)
    torch.cuda.synchronize()
    ref_idx, ref_w = orc.router_fwd(z, K, renorm)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    rtol = 1e-4 if n > 1000 else 1e-5
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=rtol, atol=1e-7)
    dw = np.random.default_rng(7).standard_normal((T, K)).astype(np.float32)
    gl = torch.full((T, n), float("nan"), dtype=torch.float32, device=DEV)   # every element is written
    dm.moe_router_bwd(lg, K, renorm, idx, w, torch.from_numpy(dw).to(DEV), gl)
    torch.cuda.synchronize()
    ref_gl = orc.router_bwd(z, ref_idx, dw, renorm)
    out = gl.cpu().numpy()
    assert np.isfinite(out).all()
    check_close("grad_logits", out, ref_gl, ulps=0, max_abs=1e-5, rel_l2=1e-5)


def test_router_no_tokens_and_determinism():
    lg = torch.from_numpy(_logits(500, 96, "ties", 3)).to(DEV)
    a = [dm.router(lg, 8) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])
    empty = torch.empty((0, 96), dtype=torch.float32, device=DEV)
    i0, w0 = dm.router(empty, 8)
    assert i0.shape == (0, 8) and w0.shape == (0, 8)


@pytest.mark.parametrize("renorm", [True, False])
def test_router_autograd(renorm):
    z = _logits(300, 72, "normal", 11)
    lg = torch.from_numpy(z).to(DEV).requires_grad_(True)
    idx, w = dm.router(lg, 6, renorm)
    dw = np.random.default_rng(12).standard_normal((300, 6)).astype(np.float32)
    (w * torch.from_numpy(dw).to(DEV)).sum().backward()
    torch.cuda.synchronize()
    ref_idx, _ = orc.router_fwd(z, 6, renorm)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    check_close("grad_logits", lg.grad.cpu().numpy(), orc.router_bwd(z, ref_idx, dw, renorm),
                ulps=0, max_abs=1e-5, rel_l2=1e-5)
