"""Whole-layer parity (dispatch, grouped FFN, combine and their backward through the
C entries) on seeded random layer shapes, against the oracle in parity mode.

The shapes are drawn once from a fixed seed so the suite is reproducible; they mix
ragged H (a multiple of 8) and F (a multiple of 32), expert counts from 1 to 96,
top-k from 1 to 8, zero/copy/constant experts and masks, and token counts large
enough that some draws select the 256 x 256 forward tiles, the grouped tile order
and the staggered K starts of the GEMMs (which of them is taken depends on the
shape, as in production)."""
import numpy as np
import pytest

import moe_workloads as wl
import oracle as orc
from gpu_util import Run, bf, check_close, f32

pytestmark = pytest.mark.gpu


def _draw(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        big = i % 3 == 0
        if big:   # many tiles: the tile choices that only pay on large layers
            E = int(rng.choice([3, 8, 16]))
            K = int(rng.integers(1, 4))
            T = int(rng.integers(4000, 8000))
            H = int(8 * rng.integers(32, 73))
            F = int(32 * rng.integers(8, 19))
        else:
            E = int(rng.choice([1, 3, 8, 16, 33, 96]))
            K = int(min(rng.integers(1, 9), E + 4))
            T = int(rng.integers(1, 700))
            H = int(8 * rng.integers(2, 160))
            F = int(32 * rng.integers(1, 24))
        kw = dict(T=T, H=H, F=F, E=E, K=K)
        if rng.random() < 0.4:
            kw.update(Z=int(rng.integers(0, 2)), C=int(rng.integers(0, 2)), Q=int(rng.integers(0, 3)), mask="2d")
        cases.append(kw)
    return cases


CASES = _draw(9)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_random_layer_shapes(idx):
    kw = CASES[idx]
    print(f"[random] case={idx} {kw}", flush=True)
    inp = wl.layer_inputs(seed=100 + idx, **kw)
    run = Run(inp)
    run.dispatch()
    run.ffn()
    out = run.combine()
    g = bf(inp["grad_out"])
    gy, gw = run.combine_bwd(g)
    ggu, gxe, gwg, gwu, gwd = run.ffn_bwd(gy)
    gx = run.dispatch_bwd(gxe, g)
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    A = f["route"].A
    assert run.A == A
    check_close("out", f32(out), f["out"])
    check_close("grad_topk_weights", f32(gw), b["dw"])
    check_close("grad_gate_up", f32(ggu[:A]), b["dGU"])
    check_close("grad_x", f32(gx), b["dx"])
    check_close("grad_w_gate", f32(gwg), b["dWg"])
    check_close("grad_w_up", f32(gwu), b["dWu"])
    check_close("grad_w_down", f32(gwd), b["dWd"])
