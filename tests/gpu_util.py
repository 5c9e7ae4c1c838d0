"""Helpers of the GPU parity tests: host <-> device conversion, the accuracy bar,
and a runner that pushes one set of generated inputs through the library's C
entry points."""
from __future__ import annotations

import numpy as np
import torch

import dispatch_expert_gemm_amd as dm
import oracle as orc

DEV = torch.device("cuda:0")

# Accuracy bar for floating-point outputs (bf16 path), against the oracle's
# parity mode:  max |err| <= 2e-2 * max(1, max |ref|)  and
# ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3.
# The absolute bound applies to the tensor scaled to unit max-magnitude when that
# magnitude exceeds 1: one bf16 rounding of an intermediate may land on the other
# neighbour when two fp32 accumulation orders differ in the last bit, and at
# |v| >= 4 one bf16 ulp is already >= 0.03 (and fp32 reductions over such
# operands inherit that ulp times the other operand).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def bf(a):
    """uint16 bf16 bits (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f32(t):
    """bf16 / fp32 GPU tensor -> float32 numpy (exact)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return orc.bf16_to_f32(t.cpu().view(torch.int16).numpy().view(np.uint16))
    return t.float().cpu().numpy()


def check_close(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref).max()
    scale = max(1.0, float(np.abs(ref).max()))
    rl2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= max_abs * scale and rl2 <= rel_l2, \
        f"{name}: max|err|={err:.3e} (bound {max_abs * scale:.3e}) rel_l2={rl2:.3e}"


def check_equal(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}: "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")


def shape_of(inp, F=None, capacity=None):
    m = inp.get("mask")
    return dm.make_shape(inp["T"], inp["H"], inp["K"], inp["E"], F=F if F is not None else inp.get("F", 0),
                         capacity=capacity, zero_expert_num=inp.get("Z", 0),
                         copy_expert_num=inp.get("C", 0), const_expert_num=inp.get("Q", 0),
                         mask_ndim=0 if m is None else m.ndim)


class Run:
    """Device copies of one input set and the results of the library calls."""

    def __init__(self, inp):
        self.inp = inp
        self.shape = shape_of(inp)
        self.x = bf(inp["x"])
        self.idx = dev(inp["topk_idx"])
        self.w = dev(inp["topk_weights"])
        self.mask = dev(inp.get("mask"))
        self.a1 = bf(inp["const_alpha_1"]) if inp.get("const_alpha_1") is not None else None
        self.a2 = bf(inp["const_alpha_2"]) if inp.get("const_alpha_2") is not None else None
        self.cv = bf(inp["const_v"]) if inp.get("const_v") is not None else None
        self.T, self.K, self.H = inp["T"], inp["K"], inp["H"]
        self.cap = self.shape.capacity

    def dispatch(self):
        self.d = dm.dispatch(self.shape, self.x, self.idx, self.mask)
        torch.cuda.synchronize()
        self.A = int(self.d.ep_recv_counts[-1].item())
        return self.d

    def ffn(self):
        F, cap, H = self.shape.F, self.cap, self.H
        self.wg, self.wu, self.wd = (bf(self.inp[k]) for k in ("w_gate", "w_up", "w_down"))
        self.gus = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
        self.h = torch.empty((cap, F), dtype=torch.bfloat16, device=DEV)
        self.y = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
        dm.moe_grouped_ffn(self.shape, self.d.expand_x, self.wg, self.wu, self.wd,
                           self.d.ep_recv_counts, self.gus, self.h, self.y)
        torch.cuda.synchronize()

    def combine(self, y=None, shared=None, w=None):
        out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=DEV)
        dm.moe_combine(self.shape, self.y if y is None else y, self.idx, self.w if w is None else w,
                       self.d.assist_info_for_combine, self.d.ep_recv_counts, self.mask, shared, self.x,
                       self.a1, self.a2, self.cv, out)
        torch.cuda.synchronize()
        return out

    def combine_bwd(self, grad_out, y=None):
        gy = torch.zeros((self.cap, self.H), dtype=torch.bfloat16, device=DEV)
        gw = torch.empty((self.T, self.K), dtype=torch.float32, device=DEV)
        dm.moe_combine_bwd(self.shape, grad_out, self.y if y is None else y, self.idx, self.w,
                           self.d.assist_info_for_combine, self.d.ep_recv_counts, self.mask, self.x,
                           self.a1, self.a2, self.cv, gy, gw)
        torch.cuda.synchronize()
        return gy, gw

    def ffn_bwd(self, gy):
        F, cap, H = self.shape.F, self.cap, self.H
        E = self.shape.num_experts
        ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
        gxe = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
        gwg = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
        gwu = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
        gwd = torch.empty((E, H, F), dtype=torch.float32, device=DEV)
        dm.moe_grouped_ffn_bwd(self.shape, gy, self.d.expand_x, self.gus, self.h, self.wg, self.wu,
                               self.wd, self.d.ep_recv_counts, ggu, gxe, gwg, gwu, gwd)
        torch.cuda.synchronize()
        return ggu, gxe, gwg, gwu, gwd

    def dispatch_bwd(self, gxe, grad_out, accum=None):
        gx = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=DEV)
        dm.moe_dispatch_bwd(self.shape, gxe, self.d.assist_info_for_combine, self.idx, self.w, self.mask,
                            grad_out, self.a1, accum, gx)
        torch.cuda.synchronize()
        return gx


class Fp8Run(Run):
    """The fp8 chain through the C entries, on top of the bf16 dispatch."""

    def quant_weights(self):
        self.wq = [dm.Fp8Weights.quantize(bf(self.inp[k])) for k in ("w_gate", "w_up", "w_down")]

    def ffn8(self):
        """fp8 forward: quantise x rows, fp8 gate/up GEMM, quantise h, fp8 down GEMM."""
        F, H, cap = self.shape.F, self.H, self.cap
        nrows = self.d.ep_recv_counts[-1:]
        self.xq, self.xs = dm.quant_rows_fp8(self.d.expand_x, nrows)
        self.gus = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
        self.h = torch.empty((cap, F), dtype=torch.bfloat16, device=DEV)
        self.y = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
        wg, wu, wd = self.wq
        dm.moe_ffn_gate_up_fwd_fp8(self.shape, self.xq, self.xs, wg.codes, wg.scales, wu.codes, wu.scales,
                                   self.d.ep_recv_counts, self.gus, self.h)
        self.hq, self.hs = dm.quant_rows_fp8(self.h, nrows)
        dm.moe_ffn_down_fwd_fp8(self.shape, self.hq, self.hs, wd.codes, wd.scales, self.d.ep_recv_counts,
                                self.y)
        torch.cuda.synchronize()

    def ffn8_bwd_data(self, gy):
        """fp8 data gradients: quantise dY, fp8 down dgrad, quantise dGU, fp8 gate/up dgrad."""
        F, H, cap = self.shape.F, self.H, self.cap
        nrows = self.d.ep_recv_counts[-1:]
        wg, wu, wd = self.wq
        dyq, dys = dm.quant_rows_fp8(gy, nrows)
        ggu = torch.empty((cap, 2 * F), dtype=torch.bfloat16, device=DEV)
        dm.moe_ffn_down_bwd_data_fp8(self.shape, dyq, dys, wd.codes_t, wd.scales, self.gus,
                                     self.d.ep_recv_counts, ggu)
        dguq, dgus = dm.quant_rows_fp8(ggu, nrows)
        gxe = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
        dm.moe_ffn_gate_up_bwd_data_fp8(self.shape, dguq, dgus, wg.codes_t, wg.scales, wu.codes_t, wu.scales,
                                        self.d.ep_recv_counts, gxe)
        torch.cuda.synchronize()
        return ggu, gxe

    def weight_grads(self, gy, ggu):
        """bf16 weight gradients (fp32 out) of the fp8 path."""
        E, F, H = self.shape.num_experts, self.shape.F, self.H
        gwg = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
        gwu = torch.empty((E, F, H), dtype=torch.float32, device=DEV)
        gwd = torch.empty((E, H, F), dtype=torch.float32, device=DEV)
        dm.moe_ffn_down_bwd_weight(self.shape, gy, self.h, self.d.ep_recv_counts, gwd)
        dm.moe_ffn_gate_up_bwd_weight(self.shape, ggu, self.d.expand_x, self.d.ep_recv_counts, gwg, gwu)
        torch.cuda.synchronize()
        return gwg, gwu, gwd
