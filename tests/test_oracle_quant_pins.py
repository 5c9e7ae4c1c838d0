"""Hand-computed pins of every quantisation point of the oracle's 8-bit layers.

The fp8 (fp32 block scales, 128 wide) and MX (power-of-two scale per 32 values)
recipes are the build's own readings: the Megatron-LM MoE performance-test page
("Add performance test for MoE layer", section *Added Test Cases*) lists FP8 as
a precision of its tests without a recipe.  Each activation that enters an
8-bit GEMM -- x and h in the forward, dY and dG|dU in the data gradients -- is
pinned here by one row whose block scale is not one and whose value of interest
is not an e4m3 code after scaling, pushed through one-hot weights whose blocks
quantise without loss (block maximum 1.75, 6 or 14: a power of two times 448,
192 or 448 codes).  The expected output is worked out by hand in the comments,
with the value the same step would give if that quantisation were left out, so
dropping any one of the eight quantisation steps changes a pinned value.

bf16 spacing used below: 2^-6 on [2, 4), 2^-5 on [4, 8), 2^-4 on [8, 16),
2 on [256, 512), 4 on [512, 1024).  e4m3 spacing: 2^-4 on [0.5, 1), 2^-3 on
[1, 2), 16 on [128, 256), 32 on [256, 448].
"""
import numpy as np
import pytest

import moe_workloads as wl
import oracle as orc

H = F = 128


def _w(shape, entries):
    """bf16 bits of a weight tensor that is zero except at the given entries."""
    a = np.zeros(shape, np.float32)
    for idx, v in entries.items():
        a[idx] = v
    return wl.to_bf16_bits(a)


def _row(n, entries):
    a = np.zeros((1, n), np.float32)
    for j, v in entries.items():
        a[0, j] = v
    return a


ONE = np.array([1])   # one expert holding the single row


# --------------------------------------------------------------------------- fp32-block-scaled fp8

def _fp8_weights(wg, wu, wd):
    return tuple(orc.quant_weights_fp8(w) for w in (wg, wu, wd))


def test_fp8_forward_quantises_x():
    # x = [450, 1.296875, 0...]: amax 450, x1 * 448/450 = 1.29111 -> e4m3 1.25,
    # dequantised 1.25 * 450/448 = 1.2555803.  Wg[5, 1] = 1.75 (block max 1.75:
    # scale 2^-8, code 448, exact), so G[0, 5] = 1.75 * 1.2555803 = 2.1972656
    # -> bf16 2.203125.  Without the quantisation: 1.75 * 1.296875 = 2.2695 -> 2.265625.
    X = _row(H, {0: 450.0, 1: 1.296875})
    wq = _fp8_weights(_w((1, F, H), {(0, 5, 1): 1.75}), _w((1, F, H), {}), _w((1, H, F), {}))
    G, U, Hh, Y = orc.ffn_fwd_fp8(X, ONE, *wq)
    assert G[0, 5] == 2.203125


def test_fp8_forward_quantises_h():
    # x = [1.75, 0...] quantises without loss.  Wg[0,0] = Wg[1,0] = 14, Wu[0,0] = 14,
    # Wu[1,0] = 6 (block max 14: scale 2^-5, codes 448 and 192): G = [24.5, 24.5],
    # U = [24.5, 10.5]; silu(24.5) = 24.5 to within 1e-9, so h = bf16([600.25,
    # 257.25]) = [600, 258].  h's block: amax 600, 258 * 448/600 = 192.64 -> e4m3 192,
    # dequantised 192 * 600/448 = 257.142857.  Wd[7, 1] = 1.75 (exact): y[0, 7] =
    # 1.75 * 257.142857 = 450 -> bf16 450.  Without the quantisation: 1.75 * 258 =
    # 451.5 -> bf16 452.
    X = _row(H, {0: 1.75})
    wq = _fp8_weights(_w((1, F, H), {(0, 0, 0): 14.0, (0, 1, 0): 14.0}),
                      _w((1, F, H), {(0, 0, 0): 14.0, (0, 1, 0): 6.0}),
                      _w((1, H, F), {(0, 7, 1): 1.75}))
    G, U, Hh, Y = orc.ffn_fwd_fp8(X, ONE, *wq)
    assert Hh[0, 0] == 600.0 and Hh[0, 1] == 258.0
    assert Y[0, 7] == 450.0


def test_fp8_data_gradient_quantises_dy():
    # dY = [450, 1.296875, 0...] -> dY1 dequantised 1.2555803 (as x above).  Wd[1, 5] =
    # 1.75: dh[5] = 2.1972656.  G[5] = 32 (sigmoid 1 to within 1e-13), U[5] = 1:
    # dG[5] = dh * U * s * (1 + G (1 - s)) = dh -> bf16 2.203125.  Without the
    # quantisation: 1.75 * 1.296875 -> bf16 2.265625.
    dY = _row(H, {0: 450.0, 1: 1.296875})
    G16 = _row(F, {5: 32.0})
    U16 = _row(F, {5: 1.0})
    wq = _fp8_weights(_w((1, F, H), {}), _w((1, F, H), {}), _w((1, H, F), {(0, 1, 5): 1.75}))
    dGU, dX, _, _, _ = orc.ffn_bwd_fp8(dY, np.zeros((1, H), np.float32), G16, U16, np.zeros((1, F), np.float32),
                                       ONE, *wq)
    assert dGU[0, 5] == 2.203125


def _dgu_case():
    # dY = [1.75, 0...] (lossless).  Wd[0, 0] = 14, Wd[0, 1] = 6: dh = [24.5, 10.5].
    # G = 0 (s = 1/2, silu 0, so dU = 0), U = [1, 1.0078125]: dG = dh * U / 2 =
    # [12.25, 5.291015625] -> bf16 [12.25, 5.28125].
    dY = _row(H, {0: 1.75})
    U16 = _row(F, {0: 1.0, 1: 1.0078125})
    return dY, np.zeros((1, F), np.float32), U16


def test_fp8_data_gradient_quantises_dgu():
    # dG block: amax 12.25, 5.28125 * 448/12.25 = 193.14 -> e4m3 192, dequantised
    # 192 * 12.25/448 = 5.25.  Wg[1, 9] = 1.75 (exact): dX[0, 9] = 1.75 * 5.25 = 9.1875
    # (a bf16 value).  Without the quantisation: 1.75 * 5.28125 = 9.2421875 -> bf16 9.25.
    dY, G16, U16 = _dgu_case()
    wq = _fp8_weights(_w((1, F, H), {(0, 1, 9): 1.75}), _w((1, F, H), {}),
                      _w((1, H, F), {(0, 0, 0): 14.0, (0, 0, 1): 6.0}))
    dGU, dX, _, _, _ = orc.ffn_bwd_fp8(dY, np.zeros((1, H), np.float32), G16, U16, np.zeros((1, F), np.float32),
                                       ONE, *wq)
    assert dGU[0, 0] == 12.25 and dGU[0, 1] == 5.28125
    assert dX[0, 9] == 9.1875


# --------------------------------------------------------------------------- microscaled (MX) fp8

def _mx_weights(wg, wu, wd):
    return tuple(orc.quant_weights_mx(w) for w in (wg, wu, wd))


def test_mx_forward_quantises_x():
    # x = [450, 1.296875, 0...] in one 32-value block: amax 450 > 448, scale 2^1;
    # 1.296875 / 2 = 0.6484375 -> e4m3 0.625, dequantised 1.25.  Wg[5, 1] = 1.75
    # (block max 1.75: scale 2^-8, code 448, exact): G[0, 5] = 2.1875 (a bf16 value).
    # Without the quantisation: bf16 2.265625.
    X = _row(H, {0: 450.0, 1: 1.296875})
    wq = _mx_weights(_w((1, F, H), {(0, 5, 1): 1.75}), _w((1, F, H), {}), _w((1, H, F), {}))
    G, U, Hh, Y = orc.ffn_fwd_mx(X, ONE, *wq)
    assert G[0, 5] == 2.1875


def test_mx_forward_quantises_h():
    # As the fp8 case: h = [600, 258] (the weights' 32-blocks have maxima 14 -> scale
    # 2^-5 and 6 -> 2^-6, codes 448 and 384, exact).  h's block: amax 600, scale 2^1;
    # 258 / 2 = 129 -> e4m3 128, dequantised 256.  Wd[7, 1] = 1.75: y[0, 7] = 448.
    # Without the quantisation: 1.75 * 258 -> bf16 452.
    X = _row(H, {0: 1.75})
    wq = _mx_weights(_w((1, F, H), {(0, 0, 0): 14.0, (0, 1, 0): 14.0}),
                     _w((1, F, H), {(0, 0, 0): 14.0, (0, 1, 0): 6.0}),
                     _w((1, H, F), {(0, 7, 1): 1.75}))
    G, U, Hh, Y = orc.ffn_fwd_mx(X, ONE, *wq)
    assert Hh[0, 0] == 600.0 and Hh[0, 1] == 258.0
    assert Y[0, 7] == 448.0


def test_mx_data_gradient_quantises_dy():
    # dY = [450, 1.296875, 0...] -> dY1 dequantised 1.25 (as x above).  Wd[1, 5] = 1.75
    # (the transposed weight's block max 1.75, exact): dh[5] = 2.1875; G[5] = 32, U[5]
    # = 1: dG[5] = 2.1875.  Without the quantisation: bf16 2.265625.
    dY = _row(H, {0: 450.0, 1: 1.296875})
    G16 = _row(F, {5: 32.0})
    U16 = _row(F, {5: 1.0})
    wq = _mx_weights(_w((1, F, H), {}), _w((1, F, H), {}), _w((1, H, F), {(0, 1, 5): 1.75}))
    dGU, dX, _, _, _ = orc.ffn_bwd_mx(dY, np.zeros((1, H), np.float32), G16, U16, np.zeros((1, F), np.float32),
                                      ONE, *wq)
    assert dGU[0, 5] == 2.1875


def test_mx_data_gradient_quantises_dgu():
    # dG = [12.25, 5.28125] (the fp8 case's), one 32-value block: amax 12.25 -> scale
    # 2^-5 (12.25 * 32 = 392 <= 448); 5.28125 * 32 = 169 -> e4m3 176, dequantised 5.5.
    # Wg[1, 9] = 1.75: dX[0, 9] = 1.75 * 5.5 = 9.625 (a bf16 value).  Without the
    # quantisation: bf16 9.25.
    dY, G16, U16 = _dgu_case()
    wq = _mx_weights(_w((1, F, H), {(0, 1, 9): 1.75}), _w((1, F, H), {}),
                     _w((1, H, F), {(0, 0, 0): 14.0, (0, 0, 1): 6.0}))
    dGU, dX, _, _, _ = orc.ffn_bwd_mx(dY, np.zeros((1, H), np.float32), G16, U16, np.zeros((1, F), np.float32),
                                      ONE, *wq)
    assert dGU[0, 0] == 12.25 and dGU[0, 1] == 5.28125
    assert dX[0, 9] == 9.625


# --------------------------------------------------------------------------- per-128-token fp8 weight gradients

def test_fp8_weight_gradient_quantises_both_operands():
    # One expert of two rows; P (a dY column) = [450, 1.296875], Q (an h column) =
    # [1.75, 1.75].  Per-128-token blocks run down the columns: P's column block has
    # amax 450 and P[1] dequantises to 1.2555803 (as x above); Q is lossless.
    # dW[0, 0] = 450 * 1.75 + 1.2555803 * 1.75 = 789.697266, to within the float32
    # rounding of the scale 450/448 (1.3e-5 here).  Without P's quantisation:
    # 450 * 1.75 + 1.296875 * 1.75 = 789.769531.
    P = np.zeros((2, H), np.float32)
    P[:, 0] = [450.0, 1.296875]
    Q = np.zeros((2, F), np.float32)
    Q[:, 0] = [1.75, 1.75]
    dW = orc.wgrad_fp8(P, Q, np.array([2]))
    assert abs(dW[0, 0, 0] - 789.697266) < 1e-4
    # ... and the other operand: swapped roles, same value
    dW2 = orc.wgrad_fp8(Q, P, np.array([2]))
    assert abs(dW2[0, 0, 0] - 789.697266) < 1e-4


# --------------------------------------------------------------------------- int8 payload and int8 path

def test_int8_payload_enters_the_weighted_sum():
    # One routed slot with weight 1: out = the int8 round trip of y.  y = [127 * 3,
    # 100, 0...]: amax 381, 100 * 127/381 = 33.33 -> 33, dequantised 33 * 3 = 99.
    # Without the payload quantisation the output would be 100.
    inp = dict(T=1, H=H, F=F, E=1, K=1, x=wl.to_bf16_bits(np.zeros((1, H), np.float32)),
               topk_idx=np.zeros((1, 1), np.int32), topk_weights=np.ones((1, 1), np.float32))
    r = orc.route(inp["topk_idx"], 1)
    Y = _row(H, {0: 381.0, 1: 100.0})
    Yc = orc.qdq_rows_int8(Y)
    out = orc.combine(Yc, r, inp["topk_weights"], None, inp["x"])
    assert Yc[0, 1] == 99.0 and out[0, 1] == 99.0


def test_int8_forward_quantises_h():
    # x = [1, 0...]: int8 code 127, row scale 1/127.  Each weight row is one-hot, so its
    # code is 127 and its channel scale the weight / 127: Wg[0,0] = Wg[1,0] = 24,
    # Wu[0,0] = 25, Wu[1,0] = 10.5 give G = [24, 24], U = [25, 10.5] (to float32
    # rounding of the scales); silu(24) = 24 to within 1e-9, so h = bf16([600, 252]) =
    # [600, 252].  h's int8 row: amax 600, 252 * 127/600 = 53.34 -> code 53.  Wd[7, 1] =
    # 2 (code 127, scale 2/127): y[0, 7] = 53 * 127 * (600/127) * (2/127) = 500.79 ->
    # bf16 500.  Without h's quantisation: 252 * 2 = 504.
    X = wl.to_bf16_bits(_row(H, {0: 1.0}))
    inp = dict(T=1, H=H, F=F, E=1, K=1, x=X, topk_idx=np.zeros((1, 1), np.int32),
               topk_weights=np.ones((1, 1), np.float32),
               w_gate=_w((1, F, H), {(0, 0, 0): 24.0, (0, 1, 0): 24.0}),
               w_up=_w((1, F, H), {(0, 0, 0): 25.0, (0, 1, 0): 10.5}),
               w_down=_w((1, H, F), {(0, 7, 1): 2.0}))
    f = orc.layer_fwd_int8(inp)
    assert f["Hh"][0, 0] == 600.0 and f["Hh"][0, 1] == 252.0
    assert f["Y"][0, 7] == 500.0


def _payload_layer(T=1):
    # x = [1.75, 0...] (lossless); Wg[0,0] = Wu[0,0] = 14: G0 = U0 = 24.5, h0 = bf16(600.25)
    # = 600, the only nonzero entry of h.  Wd[0,0] = 1.75, Wd[1,0] = 0.25 (e4m3 codes at
    # the block's scale): y = [1.75, 0.25] * hd0.
    return dict(T=T, H=H, F=F, E=1, K=1, x=wl.to_bf16_bits(_row(H, {0: 1.75})),
                topk_idx=np.zeros((1, 1), np.int32), topk_weights=np.ones((1, 1), np.float32),
                w_gate=_w((1, F, H), {(0, 0, 0): 14.0}), w_up=_w((1, F, H), {(0, 0, 0): 14.0}),
                w_down=_w((1, H, F), {(0, 0, 0): 1.75, (0, 1, 0): 0.25}))


def test_fp8_layer_applies_the_int8_payload():
    # fp8: h0 = 600 quantises to code 448 at scale 600/448, so y = bf16([1050, 150]) =
    # [1048, 150].  int8 payload of that row: amax 1048, 150 * 127/1048 = 18.18 -> 18,
    # dequantised 18 * 1048/127 = 148.54; out[0, 1] = bf16(148.54) = 149.  Without the
    # payload: 150.
    f = orc.layer_fwd_fp8(_payload_layer())
    assert f["Y"][0, 0] == 1048.0 and f["Y"][0, 1] == 150.0
    assert f["out"][0, 1] == 149.0
    assert orc.layer_fwd_fp8(_payload_layer(), comm_quant=False)["out"][0, 1] == 150.0


def test_mx_layer_applies_the_int8_payload():
    # MX: h0 = 600 has scale 2^1, 300 -> e4m3 288, dequantised 576, so y = [1008, 144]
    # (bf16 values).  int8 payload: amax 1008, 144 * 127/1008 = 18.14 -> 18, dequantised
    # 18 * 1008/127 = 142.87; out[0, 1] = bf16(142.87) = 143.  Without the payload: 144.
    f = orc.layer_fwd_mx(_payload_layer())
    assert f["Y"][0, 0] == 1008.0 and f["Y"][0, 1] == 144.0
    assert f["out"][0, 1] == 143.0
    assert orc.layer_fwd_mx(_payload_layer(), comm_quant=False)["out"][0, 1] == 144.0
