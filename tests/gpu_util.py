"""Helpers of the GPU parity tests: host <-> device conversion, the accuracy bar,
and a runner that pushes one set of generated inputs through the library's C
entry points."""
from __future__ import annotations

import os

import numpy as np
import torch

import dispatch_expert_gemm_amd as dm
import oracle as orc

DEV = torch.device("cuda:0")

# Accuracy bar for floating-point outputs, against the oracle's parity mode,
# applied element by element:
#
#   |got_i - ref_i| <= MAX_ABS + ulps * ulp_bf16(ref_i) + rho * mag_i
#
# and ||got - ref||_2 / ||ref||_2 <= REL_L2 (bf16 path) or REL_L2_8BIT (fp8,
# MX and int8 paths).
#
# * ulps: a bf16-stored output is the round-to-nearest-even of an fp32 value
#   whose last bits depend on the accumulation order, so the two sides may land
#   on neighbouring bf16 values: one ulp for a kernel fed the oracle's own
#   operands (ULPS_KERNEL), two where the kernel's inputs are themselves device
#   outputs that may sit one ulp off (ULPS_CHAIN).  At |v| >= 4 one bf16 ulp
#   is >= 0.03, above MAX_ABS, which is why the term is needed at all.
# * rho * mag: fp32 outputs that contract bf16 device intermediates (the
#   weight gradients and dw of a chained step).  If every operand entry of
#   P^T Q is within a relative 2^-6 (two bf16 ulps) of the oracle's, then
#   |dP^T Q + P^T dQ + dP^T dQ| <= (2^-6 + 2^-6 + 2^-12) (|P|^T |Q|); RHO_CHAIN
#   rounds that up to 2^-5 and mag = |P|^T |Q| is computed from the oracle's
#   operands (contraction_mag).  On identical operands rho is 0, or RHO_FP32
#   against the oracle's float64 sums: fp32 accumulation over n <= 4096 terms
#   is within n 2^-24 |P|^T |Q| <= 2^-12 |P|^T |Q|.
# * outliers: a chained 8-bit layer requantises the device's own bf16
#   intermediates (h, y, dG|dU), which sit one bf16 ulp off the oracle's at a
#   fraction of entries; where such an entry lies next to a rounding boundary
#   of the 8-bit grid its code moves by one step (an e4m3 step is up to 1/8 of
#   the value), and the outputs that contract it move by that step times a
#   weight.  Those outputs (and nothing else) are held to the element bound on
#   all but OUTLIER_FRAC of their elements (measured: at most 0.02%), and every
#   element to OUTLIER_CAP; each GEMM fed the oracle's own codes meets the
#   plain element bound (the stage-wise tests).
MAX_ABS = 2e-2
REL_L2 = 5e-3
REL_L2_8BIT = 2e-2
ULPS_KERNEL = 1
ULPS_CHAIN = 2
RHO_CHAIN = 2.0 ** -5
RHO_FP32 = 2.0 ** -12
OUTLIER_FRAC = 1e-3
OUTLIER_CAP = 0.15
OUTLIERS_8BIT = (OUTLIER_FRAC, OUTLIER_CAP)

# PARITY_LOG=<path>: append one line per comparison (the figures printed);
# PARITY_REPORT=1: record failures without raising (a measurement run).
_LOG = os.environ.get("PARITY_LOG")
_REPORT = os.environ.get("PARITY_REPORT") == "1"


def ulp_bf16(v):
    """Spacing of bf16 values next to |v|: 2^(e-7) for |v| in [2^e, 2^(e+1)), the
    subnormal spacing 2^-133 below 2^-126."""
    a = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))   # a = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 8)


def contraction_mag(P, Q, ep_recv_counts):
    """|P_e|^T |Q_e| for every expert's row range (float64, (E, P cols, Q cols)):
    the magnitude a weight gradient's error bound scales with."""
    P = np.abs(np.asarray(P, np.float64))
    Q = np.abs(np.asarray(Q, np.float64))
    counts = np.asarray(ep_recv_counts, np.int64)
    out = np.zeros((len(counts), P.shape[1], Q.shape[1]))
    lo = 0
    for e, hi in enumerate(counts.tolist()):
        if hi > lo:
            out[e] = P[lo:hi].T @ Q[lo:hi]
        lo = hi
    return out


def dw_mag(r, Y, grad_out, ori_x=None, const_alpha_1=None, const_alpha_2=None, const_v=None):
    """Sum_h |v(t,k)_h| |dOut_t,h| for every slot (float64 (T, K)): the magnitude
    the bound of dw = <v, dOut> scales with.  Y: the oracle's expert rows (float);
    the bf16 inputs as bits; v as in combine (0 for inactive and zero slots)."""
    T, K = r.T, r.K
    d = np.abs(orc.bf16_to_f32(grad_out).astype(np.float64)) if T else np.zeros((0, 0))
    Y = np.abs(np.asarray(Y, np.float64))
    ox = None if ori_x is None else np.abs(orc.bf16_to_f32(ori_x).astype(np.float64))
    a1, a2, cv = (None if a is None else np.abs(orc.bf16_to_f32(a).astype(np.float64))
                  for a in (const_alpha_1, const_alpha_2, const_v))
    codes = r.slot2row.reshape(T, K)
    mag = np.zeros((T, K))
    for t in range(T):
        for k in range(K):
            c = int(codes[t, k])
            if c >= 0:
                v = Y[c]
            elif c == -2:
                v = ox[t]
            elif c <= -3:
                v = a1[-c - 3] * ox[t] + a2[-c - 3] * cv[-c - 3]
            else:
                continue
            mag[t, k] = float(v @ d[t])
    return mag


def layer_mags(inp, f, b):
    """Magnitudes for the fp32 outputs of a whole layer step (oracle intermediates):
    dw, and |P|^T |Q| of each weight gradient (routed, and the shared expert's when
    the layer has one)."""
    r = f["route"]
    F = inp["F"]
    Yv = f["Yc"] if "Yc" in f else f["Y"]
    m = dict(dw=dw_mag(r, Yv, inp["grad_out"], inp["x"], inp.get("const_alpha_1"),
                       inp.get("const_alpha_2"), inp.get("const_v")),
             dWg=contraction_mag(b["dGU"][:, :F], f["X"], r.ep_recv_counts),
             dWu=contraction_mag(b["dGU"][:, F:], f["X"], r.ep_recv_counts),
             dWd=contraction_mag(b["dY"], f["Hh"], r.ep_recv_counts))
    if "s_dGU" in b:
        T = np.array([f["sX"].shape[0]])
        dOut = orc.bf16_to_f32(inp["grad_out"])
        m.update(s_dWg=contraction_mag(b["s_dGU"][:, :F], f["sX"], T),
                 s_dWu=contraction_mag(b["s_dGU"][:, F:], f["sX"], T),
                 s_dWd=contraction_mag(dOut, f["sH"], T))
    return m


def _log(line):
    print(line, flush=True)
    if _LOG:
        with open(_LOG, "a") as f:
            f.write(line + "\n")


def bf(a):
    """uint16 bf16 bits (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_rows(a, capacity):
    """Oracle rows (A, width) of bf16 values -> a zero-padded (capacity, width) bf16
    device buffer (an expanded-row operand fed to one kernel)."""
    a = np.asarray(a, np.float32)
    full = np.zeros((capacity, a.shape[1]), np.float32)
    full[:a.shape[0]] = a
    return bf(orc.f32_to_bf16(full))


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def f32(t):
    """bf16 / fp32 GPU tensor -> float32 numpy (exact)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return orc.bf16_to_f32(t.cpu().view(torch.int16).numpy().view(np.uint16))
    return t.float().cpu().numpy()


def check_close(name, got, ref, *, ulps=ULPS_CHAIN, max_abs=MAX_ABS, rel_l2=REL_L2, mag=None, rho=0.0,
                outliers=None):
    """Element-wise bar (see the top of this file); prints max|err| next to the
    plain MAX_ABS so any element that needs the ulp or magnitude term shows."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    bound = max_abs + ulps * ulp_bf16(ref)
    if mag is not None and rho:
        bound = bound + rho * np.broadcast_to(np.asarray(mag, np.float64), ref.shape)
    ratio = err / bound
    worst = int(np.argmax(ratio))
    emax = float(err.max())
    rl2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    nbad = int((err > bound).sum())
    if outliers is None:
        ok = nbad == 0 and rl2 <= rel_l2
    else:
        frac, cap = outliers
        ok = nbad <= frac * got.size and emax <= cap and rl2 <= rel_l2
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    _log(f"[parity] {test} {name}: max|err|={emax:.3e} ({'within' if emax <= MAX_ABS else 'above'} plain "
         f"{MAX_ABS:g}) worst err/bound={ratio.flat[worst]:.3f} at ref={ref.flat[worst]:.4g} "
         f"(bound {bound.flat[worst]:.3e}) over={nbad}/{got.size}"
         f"{'' if outliers is None else f' (allowed {outliers[0] * got.size:.0f}, cap {outliers[1]:g})'}"
         f" rel_l2={rl2:.2e} (bar {rel_l2:g}){'' if ok else ' FAIL'}")
    if not ok and not _REPORT:
        raise AssertionError(f"{name}: {nbad} elements above the bound, max|err|={emax:.3e}, "
                             f"worst err/bound={ratio.flat[worst]:.3f}, rel_l2={rl2:.3e} (bar {rel_l2:g})")


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
