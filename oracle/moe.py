"""Plain CPU oracle of the one-device expert-parallel MoE layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the product path never does.  It shares no code
with the HIP library and reads nothing the HIP library wrote.

What it computes, and where that is defined
-------------------------------------------
The layer is the low_latency_dispatch / expert FFN / low_latency_combine chain of
the Ascend CANN API page "low_latency_combine" (section "Function": Description and
Formula; section "Parameters"), run with the expert-parallel world of one device, so
the all-to-all is an identity permutation:

* dispatch: every active routed slot (token t, choice k) of ``topk_idx`` gets one row
  of the expanded buffer ``expand_x``; rows are grouped by expert, the per-expert
  token counts come out as a prefix sum (``ep_recv_counts``, Parameters:
  ``ep_send_counts``).
* expert FFN: each expert runs a SwiGLU feed-forward block with intermediate size
  ``ffn_dim`` (the ``--ffn_dim`` flag of the Triton-distributed benchmark page);
  ``h = silu(x Wg^T) * (x Wu^T)``, ``y = h Wd^T``.  The weights use the (out, in)
  layout of a linear layer.
* combine (Formula): ``out[t] = Sum_k topk_weights[t,k] * v(t,k) + shared_expert_x[t]``
  where v is the expert output of that slot; zero experts give 0, copy experts give
  ``ori_x[t]``, constant expert j gives ``alpha_1[j]*ori_x[t] + alpha_2[j]*v[j]``
  (Formula, special expert use cases; Parameters: zero/copy/const_expert_num give
  the id ranges).  The shared-expert term is added once, unweighted (Parameters:
  ``topk_weights`` and ``shared_expert_x``).
* backward: the derivative of the above, written out step by step.

Readings taken where the page is silent (each is listed in the design notes):
masked slots contribute nothing and get no row; a duplicate id in a row is an
error and its later occurrence is dropped; the prefix sum is inclusive; rows of
one expert are in increasing slot order; sums over k run in k order in fp32 with
the shared term last and one rounding to bf16 at the end.

Precision modes
---------------
``"parity"``  fp32 arithmetic on the exact decode of the bf16 inputs, plus the
              bf16 roundings of the intermediate tensors the device path stores
              (expert output y, SwiGLU output h, saved gate/up, dY, dGU, dX, the
              layer outputs).  Device outputs are judged against this mode.
``"def"``     fp32, no intermediate roundings (the plain definition).
``"f64"``     float64 throughout, no roundings; used for finite differences.

Slot-to-row map (our contents of the opaque ``assist_info_for_combine``):
``slot2row[t*K+k]`` is the row (>= 0) of a routed active slot, -1 for an inactive,
zero-expert or invalid slot, -2 for a copy-expert slot and -(3+j) for constant
expert j.  ``row2slot[r]`` is the slot of row r.

Error bits: 1 = expert id out of range, 2 = duplicate id within a row,
4 = one-dimensional activity mask that is not a prefix of trues.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import (bf16_to_f32, dequant_e4m3_blocks, dequant_e4m3_rows, dequant_int8_rows,
                       dequant_mx_e4m3_rows, e4m3_decode, quant_e4m3_blocks, quant_e4m3_rows,
                       quant_int8_rows, quant_mx_e4m3_rows, round_bf16)

ERR_ID_RANGE = 1
ERR_ID_DUPLICATE = 2
ERR_MASK_NOT_PREFIX = 4

PRECISIONS = ("parity", "def", "f64")


def _ftype(prec):
    if prec not in PRECISIONS:
        raise ValueError(prec)
    return np.float64 if prec == "f64" else np.float32


def _store(prec):
    """The rounding applied when the device path writes a bf16 tensor."""
    if prec == "parity":
        return lambda a: round_bf16(np.asarray(a, dtype=np.float32))
    return lambda a: a


def decode(a, prec="parity"):
    """bf16 bit patterns (uint16) -> float array of the mode's dtype; floats pass through."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = bf16_to_f32(a)
    return a.astype(_ftype(prec))


# ============================================================================ routing


@dataclass
class Route:
    T: int
    K: int
    E: int
    counts: np.ndarray          # (E,) int32 tokens per routed expert (expert_token_nums)
    ep_recv_counts: np.ndarray  # (E,) int32 inclusive prefix sum of counts
    slot2row: np.ndarray        # (T*K,) int32, codes as in the module docstring
    row2slot: np.ndarray        # (A,) int32
    err: int

    @property
    def A(self) -> int:
        return int(self.ep_recv_counts[-1]) if self.E > 0 else 0

    def row_range(self, e):
        lo = 0 if e == 0 else int(self.ep_recv_counts[e - 1])
        return lo, int(self.ep_recv_counts[e])


def route(topk_idx, E, Z=0, C=0, Q=0, mask=None) -> Route:
    """Classify every slot, count tokens per expert and lay the rows out by expert.

    low_latency_combine page, Parameters: ``topk_idx`` (ids in range, no duplicate
    in a row), ``x_active_mask`` (1-D: token participates, trues first; 2-D: per
    slot), ``ep_send_counts`` (prefix-summed counts), zero/copy/const id ranges.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    err = 0
    if mask is None:
        act = np.ones((T, K), dtype=bool)
    else:
        m = np.asarray(mask).astype(bool)
        if m.ndim == 1:
            # trues must precede falses: no false followed by a true
            if T > 1 and np.any(~m[:-1] & m[1:]):
                err |= ERR_MASK_NOT_PREFIX
            act = np.repeat(m[:, None], K, axis=1)
        else:
            act = m.copy()
    e_tot = E + Z + C + Q
    valid = (idx >= 0) & (idx < e_tot)
    if not valid.all():
        err |= ERR_ID_RANGE
    dup = np.zeros((T, K), dtype=bool)
    for k in range(1, K):
        dup[:, k] = np.any(idx[:, :k] == idx[:, k:k + 1], axis=1)
    if (dup & valid).any():
        err |= ERR_ID_DUPLICATE
    ok = act & valid & ~dup
    flat_id = idx.reshape(-1)
    flat_ok = ok.reshape(-1)

    routed = flat_ok & (flat_id < E)
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = np.count_nonzero(routed & (flat_id == e))
    ep_recv_counts = np.cumsum(counts)

    slot2row = np.full(T * K, -1, dtype=np.int64)
    copy = flat_ok & (flat_id >= E + Z) & (flat_id < E + Z + C)
    slot2row[copy] = -2
    const = flat_ok & (flat_id >= E + Z + C) & (flat_id < e_tot)
    slot2row[const] = -(3 + (flat_id[const] - (E + Z + C)))
    A = int(ep_recv_counts[-1]) if E else 0
    row2slot = np.empty(A, dtype=np.int64)
    start = 0
    for e in range(E):
        slots = np.nonzero(routed & (flat_id == e))[0]  # increasing slot order
        rows = start + np.arange(slots.size)
        slot2row[slots] = rows
        row2slot[rows] = slots
        start += slots.size
    return Route(T, K, E, counts.astype(np.int32), ep_recv_counts.astype(np.int32),
                 slot2row.astype(np.int32), row2slot.astype(np.int32), err)


def dispatch(x, r: Route, prec="parity"):
    """expand_x[row] = x[token of row]: the one-device alltoallv of low_latency_dispatch."""
    xf = decode(x, prec)
    return xf[r.row2slot // r.K].copy()


# ============================================================================ expert FFN


def silu(g):
    """g * sigmoid(g).  For g below about -709, exp(-g) overflows to inf and the
    quotient is the limit, -0; the overflow is expected there and not reported."""
    with np.errstate(over="ignore"):
        return g / (1 + np.exp(-g))


def ffn_fwd(X, ep_recv_counts, w_gate, w_up, w_down, prec="parity"):
    """Grouped SwiGLU FFN over the expert-sorted rows of X.

    For expert e, rows [prefix[e-1], prefix[e]):  G = X Wg^T, U = X Wu^T,
    H = silu(G) * U, Y = H Wd^T.  Returns the float arrays G, U, H, Y (with the
    parity mode's bf16 roundings of what the device stores).
    """
    st = _store(prec)
    ft = _ftype(prec)
    X = np.asarray(X, dtype=ft)
    Wg, Wu, Wd = decode(w_gate, prec), decode(w_up, prec), decode(w_down, prec)
    E, F, H = Wg.shape
    A = X.shape[0]
    G = np.zeros((A, F), ft)
    U = np.zeros((A, F), ft)
    Hh = np.zeros((A, F), ft)
    Y = np.zeros((A, H), ft)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            g = X[lo:hi] @ Wg[e].T
            u = X[lo:hi] @ Wu[e].T
            h = st(silu(g) * u)
            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h
            Y[lo:hi] = st(h @ Wd[e].T)
        lo = hi
    return G, U, Hh, Y


def ffn_bwd(dY, X, G, U, Hh, ep_recv_counts, w_gate, w_up, w_down, prec="parity"):
    """Backward of ffn_fwd.

    dH = dY Wd, dWd = dY^T H; with s = sigmoid(G):
    dG = dH * U * s * (1 + G (1 - s)), dU = dH * G * s;
    dX = [dG dU] [Wg; Wu], dWg = dG^T X, dWu = dU^T X.
    Returns dGU (A, 2F), dX (A, H), dWg, dWu, dWd (weight grads unrounded).
    """
    st = _store(prec)
    ft = _ftype(prec)
    Wg, Wu, Wd = decode(w_gate, prec), decode(w_up, prec), decode(w_down, prec)
    E, F, H = Wg.shape
    dY, X, G, U, Hh = (np.asarray(a, dtype=ft) for a in (dY, X, G, U, Hh))
    A = X.shape[0]
    dGU = np.zeros((A, 2 * F), ft)
    dX = np.zeros((A, H), ft)
    dWg = np.zeros((E, F, H), ft)
    dWu = np.zeros((E, F, H), ft)
    dWd = np.zeros((E, H, F), ft)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            dh = dY[lo:hi] @ Wd[e]
            g, u = G[lo:hi], U[lo:hi]
            s = 1 / (1 + np.exp(-g))
            dg = st(dh * u * s * (1 + g * (1 - s)))
            du = st(dh * (g * s))
            dGU[lo:hi, :F], dGU[lo:hi, F:] = dg, du
            dX[lo:hi] = st(np.concatenate([dg, du], 1) @ np.concatenate([Wg[e], Wu[e]], 0))
            dWd[e] = dY[lo:hi].T @ Hh[lo:hi]
            dWg[e] = dg.T @ X[lo:hi]
            dWu[e] = du.T @ X[lo:hi]
        lo = hi
    return dGU, dX, dWg, dWu, dWd


# ============================================================================ combine


def _slot_value(code, t, Y, ori_x, a1, a2, v):
    """Expert output of one slot (Formula of low_latency_combine)."""
    if code >= 0:
        return Y[code]
    if code == -2:
        return ori_x[t]
    j = -code - 3
    return a1[j] * ori_x[t] + a2[j] * v[j]


def combine(Y, r: Route, topk_weights, shared_expert_x=None, ori_x=None,
            const_alpha_1=None, const_alpha_2=None, const_v=None, prec="parity"):
    """out[t] = Sum_k w[t,k] * v(t,k) (+ shared_expert_x[t]); sum in k order, shared last.

    Slots coded -1 (inactive, zero expert) add nothing.
    """
    st = _store(prec)
    ft = _ftype(prec)
    T, K = r.T, r.K
    Y = np.asarray(Y, dtype=ft)
    w = np.asarray(topk_weights, dtype=ft)
    ox = decode(ori_x, prec) if ori_x is not None else None
    a1 = decode(const_alpha_1, prec) if const_alpha_1 is not None else None
    a2 = decode(const_alpha_2, prec) if const_alpha_2 is not None else None
    cv = decode(const_v, prec) if const_v is not None else None
    H = Y.shape[1]
    out = np.zeros((T, H), ft)
    codes = r.slot2row.reshape(T, K)
    for k in range(K):
        c = codes[:, k]
        for t in np.nonzero(c != -1)[0]:
            out[t] = out[t] + w[t, k] * _slot_value(int(c[t]), t, Y, ox, a1, a2, cv)
    if shared_expert_x is not None:
        out = out + decode(shared_expert_x, prec)
    return st(out)


def combine_bwd(dOut, Y, r: Route, topk_weights, ori_x=None, const_alpha_1=None,
                const_alpha_2=None, const_v=None, prec="parity"):
    """Gradient of combine.

    dY[row] = w[t,k] * dOut[t] for routed rows; dw[t,k] = <v(t,k), dOut[t]>
    (0 for inactive and zero-expert slots).  The shared term's gradient is dOut
    itself and the copy/const terms' gradient to ori_x is formed in dispatch_bwd.
    """
    st = _store(prec)
    ft = _ftype(prec)
    T, K = r.T, r.K
    d = decode(dOut, prec)
    Y = np.asarray(Y, dtype=ft)
    w = np.asarray(topk_weights, dtype=ft)
    ox = decode(ori_x, prec) if ori_x is not None else None
    a1 = decode(const_alpha_1, prec) if const_alpha_1 is not None else None
    a2 = decode(const_alpha_2, prec) if const_alpha_2 is not None else None
    cv = decode(const_v, prec) if const_v is not None else None
    dY = np.zeros_like(Y)
    dw = np.zeros((T, K), ft)
    codes = r.slot2row.reshape(T, K)
    for t in range(T):
        for k in range(K):
            c = int(codes[t, k])
            if c == -1:
                continue
            if c >= 0:
                dY[c] = w[t, k] * d[t]
            dw[t, k] = np.sum(_slot_value(c, t, Y, ox, a1, a2, cv) * d[t], dtype=ft)
    return st(dY), dw


def dispatch_bwd(dX, r: Route, topk_weights, dOut=None, const_alpha_1=None,
                 grad_x_accum=None, prec="parity"):
    """dx[t] = Sum_k (k order) of: dX[row] (routed), w*dOut[t] (copy),
    w*(alpha_1[j]*dOut[t]) (constant j); then + grad_x_accum[t]; one rounding."""
    st = _store(prec)
    ft = _ftype(prec)
    T, K = r.T, r.K
    dX = np.asarray(dX, dtype=ft)
    w = np.asarray(topk_weights, dtype=ft)
    d = decode(dOut, prec) if dOut is not None else None
    a1 = decode(const_alpha_1, prec) if const_alpha_1 is not None else None
    H = dX.shape[1]
    dx = np.zeros((T, H), ft)
    codes = r.slot2row.reshape(T, K)
    for k in range(K):
        c = codes[:, k]
        for t in np.nonzero(c != -1)[0]:
            ct = int(c[t])
            if ct >= 0:
                dx[t] = dx[t] + dX[ct]
            elif ct == -2:
                dx[t] = dx[t] + w[t, k] * d[t]
            else:
                dx[t] = dx[t] + w[t, k] * (a1[-ct - 3] * d[t])
    if grad_x_accum is not None:
        dx = dx + np.asarray(grad_x_accum, dtype=ft)
    return st(dx)


# ============================================================================ whole layer


def layer_fwd(inp: dict, prec="parity"):
    """Whole forward: route, dispatch, grouped FFN, (shared FFN), combine.

    ``inp`` keys: x, topk_idx, topk_weights, w_gate, w_up, w_down, E (and optional
    Z, C, Q, mask, const_alpha_1/2, const_v, shared_w_gate/up/down,
    shared_expert_x).  ``ori_x`` is the layer input x.
    Returns a dict of every intermediate.
    """
    E = inp["E"]
    Z, C, Q = inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0)
    r = route(inp["topk_idx"], E, Z, C, Q, inp.get("mask"))
    X = dispatch(inp["x"], r, prec)
    G, U, Hh, Y = ffn_fwd(X, r.ep_recv_counts, inp["w_gate"], inp["w_up"], inp["w_down"], prec)
    res = dict(route=r, X=X, G=G, U=U, Hh=Hh, Y=Y)
    shared = inp.get("shared_expert_x")
    if inp.get("shared_w_gate") is not None:
        xs = decode(inp["x"], prec)
        sG, sU, sH, sY = ffn_fwd(xs, np.array([xs.shape[0]]), inp["shared_w_gate"],
                                 inp["shared_w_up"], inp["shared_w_down"], prec)
        res.update(sX=xs, sG=sG, sU=sU, sH=sH, sY=sY)
        shared = sY
    res["out"] = combine(Y, r, inp["topk_weights"], shared, inp["x"], inp.get("const_alpha_1"),
                         inp.get("const_alpha_2"), inp.get("const_v"), prec)
    return res


def layer_bwd(inp: dict, fwd: dict, grad_out, prec="parity"):
    """Whole backward from grad_out; returns dx, dw, dWg, dWu, dWd (+ shared-expert grads).

    When a precomputed shared_expert_x is passed its gradient is grad_out itself.
    """
    r = fwd["route"]
    ft = _ftype(prec)
    dY, dw = combine_bwd(grad_out, fwd["Y"], r, inp["topk_weights"], inp["x"],
                         inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), prec)
    dGU, dX, dWg, dWu, dWd = ffn_bwd(dY, fwd["X"], fwd["G"], fwd["U"], fwd["Hh"], r.ep_recv_counts,
                                     inp["w_gate"], inp["w_up"], inp["w_down"], prec)
    res = dict(dY=dY, dw=dw, dGU=dGU, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd)
    accum = None
    if "sY" in fwd:
        d = decode(grad_out, prec)
        T = d.shape[0]
        sdGU, sdX, sdWg, sdWu, sdWd = ffn_bwd(d, fwd["sX"], fwd["sG"], fwd["sU"], fwd["sH"],
                                              np.array([T]), inp["shared_w_gate"], inp["shared_w_up"],
                                              inp["shared_w_down"], prec)
        res.update(s_dGU=sdGU, s_dX=sdX, s_dWg=sdWg, s_dWu=sdWu, s_dWd=sdWd)
        accum = sdX
    elif inp.get("shared_expert_x") is not None:
        res["d_shared"] = decode(grad_out, prec).astype(ft)
    res["dx"] = dispatch_bwd(dX, r, inp["topk_weights"], grad_out, inp.get("const_alpha_1"), accum, prec)
    return res


# ============================================================================ fp8 / int8 path
#
# Readings (the pages name FP8 as a precision of the MoE performance tests on the
# Megatron-LM page, section "Added Test Cases", and int8 communication quantisation
# as comm_quant_mode 2 on the low_latency_combine page, Parameters; neither gives a
# recipe, so these are ours):
#  * weights: e4m3 codes with one fp32 scale per 128 x 128 block of each expert's
#    (out, in) matrix; activations entering a fp8 GEMM: e4m3 codes with one scale
#    per (row, 128 consecutive columns of the contraction dimension);
#  * the forward GEMMs and the two data-gradient GEMMs run on the quantised
#    operands (fp32 accumulation of dequantised products); G, U, h, y, dY, dG, dU,
#    dX, dx keep their bf16 storage; the weight-gradient GEMMs run in bf16 on the
#    unquantised bf16 activations (per-token scales do not factor out of a
#    contraction over tokens);
#  * or, with wgrad="fp8", the weight gradients run on operands requantised along
#    the token axis: each expert's rows are cut into blocks of 128 consecutive rows
#    from its first row (the last block may be shorter), and every column of a block
#    gets one e4m3 scale (the row rule above, applied to that column's entries);
#  * the quantisers are applied to the bf16 tensors the device stores;
#  * int8 payload: every expert-output row y is quantised per row (symmetric,
#    127/amax) and dequantised before the weighted sum; dw uses that dequantised y.


def quant_weights_fp8(w_bits):
    """(E, N, K) bf16 weights -> (codes (E,N,K) uint8, scales (E,N/128,K/128) fp32)."""
    W = decode(w_bits, "parity")
    qs = [quant_e4m3_blocks(W[e]) for e in range(W.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def dequant_weights_fp8(codes, scales):
    return np.stack([dequant_e4m3_blocks(codes[e], scales[e]) for e in range(codes.shape[0])])


def qdq_rows_fp8(a):
    """Quantise rows per 128 columns to e4m3 and dequantise (float32)."""
    q, s = quant_e4m3_rows(np.asarray(a, np.float32))
    return dequant_e4m3_rows(q, s)


def quant_cols_fp8(a, ep_recv_counts, block=128):
    """Per-128-token e4m3 quantisation of expert-sorted rows (the weight-gradient
    operands): each expert's rows are cut into blocks of `block` consecutive rows
    starting at its first row, and each column of a block is quantised as one block of
    quant_e4m3_rows.  Returns a list of (expert, first row, end row, codes (rows, D)
    uint8, scales (D,) float32), in row order."""
    a = np.asarray(a, np.float32)
    out = []
    lo = 0
    for e, hi in enumerate(np.asarray(ep_recv_counts, np.int64).tolist()):
        for r0 in range(lo, hi, block):
            r1 = min(r0 + block, hi)
            q, s = quant_e4m3_rows(a[r0:r1].T, block=r1 - r0)  # a column is one block
            out.append((e, r0, r1, q.T.copy(), s[:, 0].copy()))
        lo = hi
    return out


def qdq_cols_fp8(a, ep_recv_counts, block=128):
    """quant_cols_fp8 then dequantisation: code value times scale, exact in float64."""
    a = np.asarray(a, np.float32)
    d = np.zeros(a.shape, np.float64)
    for _, r0, r1, q, s in quant_cols_fp8(a, ep_recv_counts, block):
        d[r0:r1] = e4m3_decode(q).astype(np.float64) * s.astype(np.float64)[None, :]
    return d


def wgrad_fp8(P16, Q16, ep_recv_counts):
    """Weight gradient on per-128-token fp8 operands: for every expert e,
    qdq_cols_fp8(P)[rows of e]^T @ qdq_cols_fp8(Q)[rows of e], float64 (E, Dp, Dq)."""
    Pd, Qd = qdq_cols_fp8(P16, ep_recv_counts), qdq_cols_fp8(Q16, ep_recv_counts)
    E = len(ep_recv_counts)
    out = np.zeros((E, Pd.shape[1], Qd.shape[1]))
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        out[e] = Pd[lo:hi].T @ Qd[lo:hi]
        lo = hi
    return out


def ffn_fwd_fp8(X16, ep_recv_counts, wq_gate, wq_up, wq_down):
    """fp8 forward of the grouped SwiGLU FFN (parity mode).

    wq_*: (codes, scales) from quant_weights_fp8.  X16: the bf16 expanded rows (float32
    values).  Returns G16, U16, H16 (bf16 values) and Y16.
    """
    st = _store("parity")
    Wg, Wu, Wd = (dequant_weights_fp8(*w) for w in (wq_gate, wq_up, wq_down))
    X16 = np.asarray(X16, np.float32)
    Xd = qdq_rows_fp8(X16) if X16.shape[0] else X16
    E, F, H = Wg.shape
    A = X16.shape[0]
    G, U, Hh = (np.zeros((A, F), np.float32) for _ in range(3))
    Y = np.zeros((A, H), np.float32)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            g = Xd[lo:hi] @ Wg[e].T
            u = Xd[lo:hi] @ Wu[e].T
            h = st(silu(g) * u)
            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h
            Y[lo:hi] = st(qdq_rows_fp8(h) @ Wd[e].T)
        lo = hi
    return G, U, Hh, Y


def ffn_bwd_fp8(dY16, X16, G16, U16, H16, ep_recv_counts, wq_gate, wq_up, wq_down, wgrad="bf16"):
    """fp8 backward: data gradients on quantised dY / dGU and fp8 weights, weight
    gradients in bf16, or on per-128-token fp8 operands with wgrad="fp8" (parity
    mode).  Returns dGU, dX, dWg, dWu, dWd."""
    assert wgrad in ("bf16", "fp8")
    st = _store("parity")
    Wg, Wu, Wd = (dequant_weights_fp8(*w) for w in (wq_gate, wq_up, wq_down))
    E, F, H = Wg.shape
    dY16, X16, G16, U16, H16 = (np.asarray(a, np.float32) for a in (dY16, X16, G16, U16, H16))
    A = X16.shape[0]
    dGU = np.zeros((A, 2 * F), np.float32)
    dX = np.zeros((A, H), np.float32)
    dWg, dWu = np.zeros((E, F, H), np.float32), np.zeros((E, F, H), np.float32)
    dWd = np.zeros((E, H, F), np.float32)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            dh = qdq_rows_fp8(dY16[lo:hi]) @ Wd[e]
            g, u = G16[lo:hi], U16[lo:hi]
            s = 1 / (1 + np.exp(-g))
            dg = st(dh * u * s * (1 + g * (1 - s)))
            du = st(dh * (g * s))
            dgu = np.concatenate([dg, du], 1)
            dGU[lo:hi] = dgu
            dX[lo:hi] = st(qdq_rows_fp8(dgu) @ np.concatenate([Wg[e], Wu[e]], 0))
            if wgrad == "bf16":
                dWd[e] = dY16[lo:hi].T @ H16[lo:hi]
                dWg[e] = dg.T @ X16[lo:hi]
                dWu[e] = du.T @ X16[lo:hi]
        lo = hi
    if wgrad == "fp8":
        dWd[:] = wgrad_fp8(dY16, H16, ep_recv_counts)
        dWgu = wgrad_fp8(dGU, X16, ep_recv_counts)
        dWg[:], dWu[:] = dWgu[:, :F], dWgu[:, F:]
    return dGU, dX, dWg, dWu, dWd


def qdq_rows_int8(Y16):
    """The int8 combine payload: per-row symmetric int8 round trip of y."""
    Y16 = np.asarray(Y16, np.float32)
    if Y16.shape[0] == 0:
        return Y16
    return dequant_int8_rows(*quant_int8_rows(Y16))


def layer_fwd_fp8(inp: dict, comm_quant=True):
    """Whole forward on the fp8 path (parity mode): weights and activations
    quantised as described above, int8 combine payload when comm_quant."""
    E = inp["E"]
    Z, C, Q = inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0)
    r = route(inp["topk_idx"], E, Z, C, Q, inp.get("mask"))
    X = dispatch(inp["x"], r, "parity")
    wq = tuple(quant_weights_fp8(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    G, U, Hh, Y = ffn_fwd_fp8(X, r.ep_recv_counts, *wq)
    Yc = qdq_rows_int8(Y) if comm_quant else Y
    out = combine(Yc, r, inp["topk_weights"], inp.get("shared_expert_x"), inp["x"],
                  inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), "parity")
    return dict(route=r, X=X, wq=wq, G=G, U=U, Hh=Hh, Y=Y, Yc=Yc, out=out)


def layer_bwd_fp8(inp: dict, fwd: dict, grad_out, wgrad="bf16"):
    r = fwd["route"]
    dY, dw = combine_bwd(grad_out, fwd["Yc"], r, inp["topk_weights"], inp["x"],
                         inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), "parity")
    dGU, dX, dWg, dWu, dWd = ffn_bwd_fp8(dY, fwd["X"], fwd["G"], fwd["U"], fwd["Hh"], r.ep_recv_counts,
                                         *fwd["wq"], wgrad=wgrad)
    dx = dispatch_bwd(dX, r, inp["topk_weights"], grad_out, inp.get("const_alpha_1"), None, "parity")
    return dict(dY=dY, dw=dw, dGU=dGU, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd, dx=dx)


# ============================================================================ int8 dispatch + w8a8 FFN
#
# Readings (low_latency_dispatch as used on the low_latency_combine page, example
# programs: quant_mode 2 is "dynamic quantization", dispatch then returns an int8
# expand_x with dynamic_scales, and an optional fp32 scales tensor of shape
# (num_experts, H) may be passed; the page gives no formula, so these are ours):
#  * every expanded row (token t sent to routed expert e) is x_t times scales[e]
#    (elementwise, float32; no product without scales), quantised per row with the
#    int8 rule of the combine payload: codes clamp(rint(v * (127/amax)), -127, 127),
#    dynamic scale amax/127 (an all-zero row: codes 0, scale 1);
#  * the grouped FFN on those rows (not on the pages; the decode-regime consumer of
#    an int8 expand_x): int8 weights with one scale per output channel (row of the
#    (out, in) matrix, same rule), integer products summed exactly, times (row scale
#    x channel scale); G, U, h, y stored as bf16; h requantised per row (same rule)
#    for the down projection.


def dispatch_int8(x, r: Route, smooth_scales=None):
    """int8 expand_x (A, H) and dynamic_scales (A,) of the routed rows, in row order."""
    X = dispatch(x, r, "parity").astype(np.float32)
    if smooth_scales is not None:
        S = np.asarray(smooth_scales, np.float32)
        experts = np.repeat(np.arange(len(r.ep_recv_counts)), np.diff(np.concatenate([[0], r.ep_recv_counts])))
        X = (X * S[experts]).astype(np.float32)
    if X.shape[0] == 0:
        return np.zeros(X.shape, np.int8), np.zeros(0, np.float32)
    return quant_int8_rows(X)


def quant_weights_int8(w_bits):
    """(E, N, K) bf16 weights -> (codes (E, N, K) int8, scales (E, N) fp32), one scale per
    output channel."""
    W = decode(w_bits, "parity")
    qs = [quant_int8_rows(W[e]) for e in range(W.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def _i8_gemm(q_rows, s_rows, q_w, s_w):
    """(q_rows @ q_w^T) exactly, times (row scale x channel scale), float64.

    The integer sums are taken as a float64 matrix product: every product is at most
    127^2 and every partial sum an integer of magnitude below 127^2 * K < 2^53 (K < 5e11),
    so each float64 addition is exact and the result equals the integer sum."""
    assert q_rows.shape[1] < (1 << 53) // (127 * 127)
    acc = q_rows.astype(np.float64) @ q_w.astype(np.float64).T
    return acc * s_rows.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]


def ffn_fwd_int8(Xq, xs, ep_recv_counts, wq_gate, wq_up, wq_down):
    """w8a8 forward of the grouped SwiGLU FFN on int8 expanded rows (parity mode).
    Returns G, U, h (bf16 values), the int8 codes/scales of h, and y (bf16 values)."""
    st = _store("parity")
    (gq, gs), (uq, us), (dq, ds) = wq_gate, wq_up, wq_down
    A, E = Xq.shape[0], gq.shape[0]
    F, H = gq.shape[1], dq.shape[1]
    G, U, Hh = (np.zeros((A, F), np.float32) for _ in range(3))
    Y = np.zeros((A, H), np.float32)
    hq, hs = np.zeros((A, F), np.int8), np.ones(A, np.float32)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            g = _i8_gemm(Xq[lo:hi], xs[lo:hi], gq[e], gs[e])
            u = _i8_gemm(Xq[lo:hi], xs[lo:hi], uq[e], us[e])
            h = st(silu(g) * u)
            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h
            hq[lo:hi], hs[lo:hi] = quant_int8_rows(h)
            Y[lo:hi] = st(_i8_gemm(hq[lo:hi], hs[lo:hi], dq[e], ds[e]))
        lo = hi
    return G, U, Hh, hq, hs, Y


def layer_fwd_int8(inp: dict, smooth_scales=None):
    """Decode-regime forward: int8 dispatch (optionally smooth-scaled), w8a8 FFN,
    bf16 combine (parity mode)."""
    E = inp["E"]
    Z, C, Q = inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0)
    r = route(inp["topk_idx"], E, Z, C, Q, inp.get("mask"))
    Xq, xs = dispatch_int8(inp["x"], r, smooth_scales)
    wq = tuple(quant_weights_int8(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    G, U, Hh, hq, hs, Y = ffn_fwd_int8(Xq, xs, r.ep_recv_counts, *wq)
    out = combine(Y, r, inp["topk_weights"], inp.get("shared_expert_x"), inp["x"],
                  inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), "parity")
    return dict(route=r, Xq=Xq, xs=xs, wq=wq, G=G, U=U, Hh=Hh, hq=hq, hs=hs, Y=Y, out=out)


# ============================================================================ MX (microscaled) fp8 path
#
# Reading (the survey's NEXT-2 names gfx950's block-scaled MFMA; the pages give no
# recipe): the same fp8 layer with microscaling instead of fp32 block scales: every
# fp8 operand carries one E8M0 (power of two) scale per 32 consecutive values of its
# contraction dimension (quant_mx_e4m3_rows; the scale is the smallest power of two
# that keeps the block maximum within +-448, so nothing saturates): activations x, h, dY, dG|dU along their
# rows; the weights along H for the forward GEMMs and, for the data gradients, their
# transposes along F (gate/up) or H (down), i.e. the weights are quantised twice.
# Weight gradients stay bf16, G, U, h, y, dG|dU, dX keep bf16 storage.


def qdq_rows_mx(a):
    """MX e4m3 round trip along rows (float64)."""
    a = np.asarray(a, np.float32)
    if a.shape[0] == 0:
        return a.astype(np.float64)
    return dequant_mx_e4m3_rows(*quant_mx_e4m3_rows(a))


def quant_weights_mx(w_bits):
    """(E, N, K) bf16 weights -> MX codes/scales along K, (E, N, K) and (E, N, K/32), and
    of the transposes along N, (E, K, N) and (E, K, N/32)."""
    W = decode(w_bits, "parity")
    fw = [quant_mx_e4m3_rows(W[e]) for e in range(W.shape[0])]
    tw = [quant_mx_e4m3_rows(np.ascontiguousarray(W[e].T)) for e in range(W.shape[0])]
    return (np.stack([q for q, _ in fw]), np.stack([s for _, s in fw]),
            np.stack([q for q, _ in tw]), np.stack([s for _, s in tw]))


def _dq_w_mx(wq, transposed=False):
    """Dequantised weights (float64): (E, N, K) from the K-blocked codes, or the
    (E, K, N) transposes from the N-blocked codes."""
    c, s = (wq[2], wq[3]) if transposed else (wq[0], wq[1])
    return np.stack([dequant_mx_e4m3_rows(c[e], s[e]) for e in range(c.shape[0])])


def ffn_fwd_mx(X16, ep_recv_counts, wq_gate, wq_up, wq_down):
    """MX fp8 forward of the grouped SwiGLU FFN (parity mode); wq_* from quant_weights_mx.
    Returns G16, U16, H16 and Y16 (bf16 values)."""
    st = _store("parity")
    Wg, Wu, Wd = (_dq_w_mx(w) for w in (wq_gate, wq_up, wq_down))
    X16 = np.asarray(X16, np.float32)
    Xd = qdq_rows_mx(X16)
    E, F, H = Wg.shape
    A = X16.shape[0]
    G, U, Hh = (np.zeros((A, F), np.float32) for _ in range(3))
    Y = np.zeros((A, H), np.float32)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            g = Xd[lo:hi] @ Wg[e].T
            u = Xd[lo:hi] @ Wu[e].T
            h = st(silu(g) * u)
            G[lo:hi], U[lo:hi], Hh[lo:hi] = st(g), st(u), h
            Y[lo:hi] = st(qdq_rows_mx(h) @ Wd[e].T)
        lo = hi
    return G, U, Hh, Y


def ffn_bwd_mx(dY16, X16, G16, U16, H16, ep_recv_counts, wq_gate, wq_up, wq_down):
    """MX fp8 data gradients (dY and dG|dU quantised along their rows, the transposed
    weights along F or H), bf16 weight gradients (parity mode).  Returns dGU, dX, dWg,
    dWu, dWd."""
    st = _store("parity")
    WgT, WuT, WdT = (_dq_w_mx(w, transposed=True) for w in (wq_gate, wq_up, wq_down))
    E, H, F = WgT.shape
    dY16, X16, G16, U16, H16 = (np.asarray(a, np.float32) for a in (dY16, X16, G16, U16, H16))
    A = X16.shape[0]
    dGU = np.zeros((A, 2 * F), np.float32)
    dX = np.zeros((A, H), np.float32)
    dWg, dWu = np.zeros((E, F, H), np.float32), np.zeros((E, F, H), np.float32)
    dWd = np.zeros((E, H, F), np.float32)
    lo = 0
    for e in range(E):
        hi = int(ep_recv_counts[e])
        if hi > lo:
            dh = qdq_rows_mx(dY16[lo:hi]) @ WdT[e].T          # WdT[e] is (F, H): dh = dY Wd
            g, u = G16[lo:hi], U16[lo:hi]
            s = 1 / (1 + np.exp(-g))
            dg = st(dh * u * s * (1 + g * (1 - s)))
            du = st(dh * (g * s))
            dgu = np.concatenate([dg, du], 1)
            dGU[lo:hi] = dgu
            dX[lo:hi] = st(qdq_rows_mx(dgu) @ np.concatenate([WgT[e], WuT[e]], 1).T)
            dWd[e] = dY16[lo:hi].T @ H16[lo:hi]
            dWg[e] = dg.T @ X16[lo:hi]
            dWu[e] = du.T @ X16[lo:hi]
        lo = hi
    return dGU, dX, dWg, dWu, dWd


def layer_fwd_mx(inp: dict, comm_quant=True):
    """Whole forward on the MX fp8 path (parity mode), int8 combine payload when comm_quant."""
    E = inp["E"]
    Z, C, Q = inp.get("Z", 0), inp.get("C", 0), inp.get("Q", 0)
    r = route(inp["topk_idx"], E, Z, C, Q, inp.get("mask"))
    X = dispatch(inp["x"], r, "parity")
    wq = tuple(quant_weights_mx(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    G, U, Hh, Y = ffn_fwd_mx(X, r.ep_recv_counts, *wq)
    Yc = qdq_rows_int8(Y) if comm_quant else Y
    out = combine(Yc, r, inp["topk_weights"], inp.get("shared_expert_x"), inp["x"],
                  inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), "parity")
    return dict(route=r, X=X, wq=wq, G=G, U=U, Hh=Hh, Y=Y, Yc=Yc, out=out)


def layer_bwd_mx(inp: dict, fwd: dict, grad_out):
    r = fwd["route"]
    dY, dw = combine_bwd(grad_out, fwd["Yc"], r, inp["topk_weights"], inp["x"],
                         inp.get("const_alpha_1"), inp.get("const_alpha_2"), inp.get("const_v"), "parity")
    dGU, dX, dWg, dWu, dWd = ffn_bwd_mx(dY, fwd["X"], fwd["G"], fwd["U"], fwd["Hh"], r.ep_recv_counts,
                                        *fwd["wq"])
    dx = dispatch_bwd(dX, r, inp["topk_weights"], grad_out, inp.get("const_alpha_1"), None, "parity")
    return dict(dY=dY, dw=dw, dGU=dGU, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd, dx=dx)
