"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library routines, closed forms, hand counts from the low_latency_combine page's
example tables, published format tables, brute force and finite differences.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, an unstable row order, a missing
rounding) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import moe_workloads as wl
import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page2_topk_examples.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


# ============================================================================ formats


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # add exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (rng.integers(0, 2 ** 16, size=4096, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties, np.array([0x7F7FFFFF, 0x7F7F8000, 0x00008000, 0x80018000],
                                                dtype=np.uint32)])
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    ours = orc.f32_to_bf16(x[finite])
    ref = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nanx = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.isnan(orc.bf16_to_f32(orc.f32_to_bf16(nanx))).all()


def test_bf16_decode_is_exact():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = orc.bf16_to_f32(allbits)
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (f == ref) | (np.isnan(f) & np.isnan(ref))
    assert same.all()


def test_e4m3_published_points():
    g = _gold()["ocp_e4m3_points"]
    for code, val in g["code_value"]:
        assert orc.e4m3_decode(np.array([code], np.uint8))[0] == np.float32(val)
    for code in g["nan_codes"]:
        assert np.isnan(orc.e4m3_decode(np.array([code], np.uint8))[0])


def test_e4m3_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = orc.e4m3_decode(codes)
    assert np.array_equal(orc.e4m3_encode(vals), codes)
    # midpoints between neighbouring magnitudes go to the even code
    pos = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all((mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2))  # exact in fp32
    enc = orc.e4m3_encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, expect.astype(np.uint8))
    # saturation and NaN
    assert orc.e4m3_encode(np.array([448.0, 500.0, 1e30, -1e30], np.float32)).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert orc.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 30,
                        rng.standard_normal(20000).astype(np.float32) * 0.01,
                        (rng.random(20000).astype(np.float32) - 0.5) * 2 * 447.0])
    ours = orc.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_quant_rows_amax_maps_to_max_code():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 256)).astype(np.float32)
    q, s = orc.quant_e4m3_rows(x)
    v = orc.e4m3_decode(q)
    for r in range(5):
        for b in range(2):
            blk = x[r, b * 128:(b + 1) * 128]
            j = np.argmax(np.abs(blk))
            assert abs(v[r, b * 128 + j]) == 448.0
            assert s[r, b] == np.float32(np.abs(blk).max() / np.float32(448.0))
    # all-zero block
    q0, s0 = orc.quant_e4m3_rows(np.zeros((1, 128), np.float32))
    assert (q0 == 0).all() and s0[0, 0] == 1.0
    # dequantised error within half an e4m3 step (relative 2^-4) of each value's scale
    deq = orc.dequant_e4m3_rows(q, s)
    assert np.all(np.abs(deq - x) <= np.repeat(s, 128, axis=1) * 448 * 2 ** -4 + 1e-30)
    qi, si = orc.quant_int8_rows(x)
    assert np.all(np.abs(qi).max(axis=1) == 127)
    ri = orc.quant_int8_rows(np.array([[127.0, 0.5, 1.5, 2.5, -2.5]], np.float32))[0]
    assert ri.tolist() == [[127, 0, 2, 2, -2]]  # ties to even with scale 1


def test_quant_blocks_tile_amax():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    q, s = orc.quant_e4m3_blocks(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            t = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(np.abs(t).max() / np.float32(448.0))
    d = orc.dequant_e4m3_blocks(q, s)
    assert np.abs(d - w).max() <= s.max() * 448 * 2 ** -4


# ============================================================================ routing


@pytest.mark.parametrize("case", ["single_operator", "graph_mode"])
def test_route_page2_examples(case):
    g = _gold()[case]
    idx = np.array(g["topk_idx"], np.int32)
    r = orc.route(idx, g["num_experts"], g["zero_expert_num"], g["copy_expert_num"], g["const_expert_num"])
    assert r.err == 0
    assert r.counts.tolist() == g["hand_counts"]
    assert r.A == g["hand_routed_slots"]
    assert r.ep_recv_counts.tolist() == np.cumsum(g["hand_counts"]).tolist()
    codes = r.slot2row.reshape(idx.shape)
    assert int((codes == -2).sum()) == g["hand_copy_slots"]
    for t, k in g.get("hand_copy_slot_positions", []):
        assert codes[t, k] == -2
    for t, k in g.get("hand_zero_slot_positions", []):
        assert codes[t, k] == -1
    assert int((codes >= 0).sum()) == g["hand_routed_slots"]


def _rand_route(T, K, E, Z=0, C=0, Q=0, seed=0):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E + Z + C + Q)[:K] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,K,E", [(1, 1, 1), (7, 3, 5), (64, 8, 64), (300, 2, 8), (33, 16, 16)])
def test_route_counts_and_stable_permutation(T, K, E):
    idx = _rand_route(T, K, E, seed=T * 7 + K)
    r = orc.route(idx, E)
    assert r.err == 0
    assert r.counts.sum() == T * K                     # no mask, no special experts
    assert r.counts.tolist() == np.bincount(idx.reshape(-1), minlength=E).tolist()
    assert r.ep_recv_counts[-1] == r.A
    ref_rows = np.argsort(idx.reshape(-1), kind="stable")  # library stable sort
    assert np.array_equal(r.row2slot, ref_rows)
    assert np.array_equal(r.slot2row[r.row2slot], np.arange(r.A))
    assert sorted(r.slot2row.tolist()) == list(range(T * K))  # bijection


def test_route_masks_and_specials():
    T, K, E, Z, C, Q = 50, 6, 10, 2, 1, 3
    idx = _rand_route(T, K, E, Z, C, Q, seed=5)
    rng = np.random.default_rng(6)
    m2 = (rng.random((T, K)) > 0.3).astype(np.uint8)
    r = orc.route(idx, E, Z, C, Q, m2)
    codes = r.slot2row.reshape(T, K)
    act = m2.astype(bool)
    routed = act & (idx < E)
    assert np.array_equal(codes >= 0, routed)
    assert np.all(codes[~act] == -1)
    assert np.all(codes[act & (idx >= E) & (idx < E + Z)] == -1)
    assert np.all(codes[act & (idx >= E + Z) & (idx < E + Z + C)] == -2)
    cj = act & (idx >= E + Z + C)
    assert np.array_equal(-codes[cj] - 3, idx[cj] - (E + Z + C))
    inactive, special = int((~act).sum()), int((act & (idx >= E)).sum())
    assert r.counts.sum() + inactive + special == T * K
    # 1-D prefix mask: the first 20 tokens participate
    m1 = np.zeros(T, np.uint8)
    m1[:20] = 1
    r1 = orc.route(idx, E, Z, C, Q, m1)
    assert r1.err == 0
    assert np.all(r1.slot2row.reshape(T, K)[20:] == -1)


def test_route_errors():
    idx = np.array([[0, 1], [2, 2], [5, 0]], np.int32)
    r = orc.route(idx, 3)
    assert r.err & orc.ERR_ID_RANGE and r.err & orc.ERR_ID_DUPLICATE
    codes = r.slot2row.reshape(3, 2)
    assert codes[1, 0] >= 0 and codes[1, 1] == -1    # later duplicate dropped
    assert codes[2, 0] == -1                         # out-of-range dropped
    assert r.A == 4
    r2 = orc.route(np.array([[0], [1], [2]], np.int32), 3, mask=np.array([1, 0, 1], np.uint8))
    assert r2.err == orc.ERR_MASK_NOT_PREFIX
    assert orc.route(np.array([[0], [1], [2]], np.int32), 3, mask=np.array([1, 1, 0], np.uint8)).err == 0


def test_dispatch_rows_are_token_copies():
    inp = wl.layer_inputs(40, 16, 8, 6, 3, seed=3, weights=False, grad=False)
    r = orc.route(inp["topk_idx"], 6)
    X = orc.dispatch(inp["x"], r)
    xf = orc.bf16_to_f32(inp["x"])
    for s in range(40 * 3):
        assert np.array_equal(X[r.slot2row[s]], xf[s // 3])


# ============================================================================ combine


@pytest.mark.parametrize("K", [2, 3, 8, 16])
def test_round_trip_unit_weights_is_k_times_x(K):
    """combine(dispatch(x)) with w = 1 and the FFN bypassed is K*x, bit for bit."""
    T, H, E = 37, 24, 16
    inp = wl.layer_inputs(T, H, 8, E, K, seed=K, weights=False, grad=False)
    r = orc.route(inp["topk_idx"], E)
    X = orc.dispatch(inp["x"], r)
    out = orc.combine(X, r, np.ones((T, K), np.float32))
    kx = orc.bf16_to_f32(inp["x"]) * np.float32(K)            # exact in fp32 for K <= 16
    ref = torch.from_numpy(kx).to(torch.bfloat16).float().numpy()
    assert np.array_equal(out, ref)


def _special_setup(T=9, H=12, K=4, seed=0):
    rng = np.random.default_rng(seed)
    d = dict(ori=rng.standard_normal((T, H)), shared=rng.standard_normal((T, H)),
             a1=rng.standard_normal((2, H)), a2=rng.standard_normal((2, H)), v=rng.standard_normal((2, H)),
             w=rng.standard_normal((T, K)))
    return d


def test_combine_closed_forms_special_experts():
    T, H, K, E, Z, C, Q = 9, 12, 4, 5, 4, 4, 2
    d = _special_setup(T, H, K)
    Y = np.zeros((0, H))
    # all zero experts -> shared
    idx = np.tile(np.arange(E, E + 4), (T, 1)).astype(np.int32)
    r = orc.route(idx, E, Z, C, Q)
    out = orc.combine(Y, r, d["w"], d["shared"], d["ori"], d["a1"], d["a2"], d["v"], prec="f64")
    assert np.allclose(out, d["shared"], rtol=0, atol=1e-14)
    out0 = orc.combine(Y, r, d["w"], None, d["ori"], prec="f64")
    assert np.all(out0 == 0)
    # all copy experts -> (sum_k w) * ori_x + shared
    idx = np.tile(np.arange(E + Z, E + Z + 4), (T, 1)).astype(np.int32)
    r = orc.route(idx, E, Z, C, Q)
    out = orc.combine(Y, r, d["w"], d["shared"], d["ori"], d["a1"], d["a2"], d["v"], prec="f64")
    assert np.allclose(out, d["w"].sum(1)[:, None] * d["ori"] + d["shared"], atol=1e-12)
    # constant experts (two of them in slots 0, 1; slots 2, 3 masked off)
    idx = np.tile(np.array([E + Z + C, E + Z + C + 1, 0, 1]), (T, 1)).astype(np.int32)
    m = np.tile(np.array([1, 1, 0, 0], np.uint8), (T, 1))
    r = orc.route(idx, E, Z, C, Q, m)
    out = orc.combine(np.zeros((r.A, H)), r, d["w"], None, d["ori"], d["a1"], d["a2"], d["v"], prec="f64")
    ref = sum(d["w"][:, j:j + 1] * (d["a1"][j] * d["ori"] + d["a2"][j] * d["v"][j]) for j in range(2))
    assert np.allclose(out, ref, atol=1e-12)


def test_combine_is_linear_in_weights_and_masked_tokens_get_shared_only():
    T, H, K, E = 10, 8, 3, 6
    rng = np.random.default_rng(4)
    idx = _rand_route(T, K, E, seed=9)
    m = np.ones((T, K), np.uint8)
    m[3] = 0
    r = orc.route(idx, E, mask=m)
    Y = rng.standard_normal((r.A, H))
    sh = rng.standard_normal((T, H))
    w1, w2 = rng.standard_normal((T, K)), rng.standard_normal((T, K))
    f = lambda w: orc.combine(Y, r, w, None, prec="f64")
    assert np.allclose(f(2 * w1 - 3 * w2), 2 * f(w1) - 3 * f(w2), atol=1e-12)
    out = orc.combine(Y, r, w1, sh, prec="f64")
    assert np.array_equal(out[3], sh[3])


# ============================================================================ expert FFN


def _torch_swiglu(x, wg, wu, wd):
    """Dense SwiGLU FFN of one expert, from torch's own silu and matmul (float64)."""
    x, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T) @ wd.T).numpy()


def test_one_hot_weights_reproduce_single_expert():
    T, H, F, E, K = 24, 32, 16, 5, 3
    inp = wl.layer_inputs(T, H, F, E, K, seed=11, grad=False)
    xf = orc.bf16_to_f32(inp["x"]).astype(np.float64)
    wg, wu, wd = (orc.bf16_to_f32(inp[n]).astype(np.float64) for n in ("w_gate", "w_up", "w_down"))
    for k0 in range(K):
        w = np.zeros((T, K), np.float32)
        w[:, k0] = 1.0
        inp2 = dict(inp, topk_weights=w)
        out = orc.layer_fwd(inp2, prec="f64")["out"]
        ref = np.stack([_torch_swiglu(xf[t:t + 1], wg[e], wu[e], wd[e])[0]
                        for t, e in enumerate(inp["topk_idx"][:, k0])])
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        out32 = orc.layer_fwd(inp2, prec="def")["out"]
        assert np.allclose(out32, ref, rtol=1e-4, atol=1e-5)
    assert orc.silu(np.float64(0.0)) == 0.0


def test_parity_mode_outputs_are_bf16_values():
    inp = wl.layer_inputs(32, 16, 8, 4, 2, seed=12)
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    for a in (f["out"], f["Y"], f["Hh"], f["G"], f["U"], b["dY"], b["dGU"], b["dX"], b["dx"]):
        assert np.array_equal(a, orc.round_bf16(a))
    # and they agree with the unrounded definition to bf16 accuracy
    fd = orc.layer_fwd(inp, prec="def")
    assert np.abs(f["out"] - fd["out"]).max() < 2e-2


# ============================================================================ gradients


def _fd_problem(seed=0, shared_ffn=False):
    T, H, F, E, K, Z, C, Q = 4, 8, 4, 3, 2, 1, 1, 1
    rng = np.random.default_rng(seed)
    idx = np.array([[0, 1], [2, 3], [4, 5], [1, 0]], np.int32)   # routed, zero, copy, const
    m = np.array([[1, 1], [1, 1], [1, 1], [1, 0]], np.uint8)
    inp = dict(T=T, H=H, F=F, E=E, K=K, Z=Z, C=C, Q=Q, topk_idx=idx, mask=m,
               x=rng.standard_normal((T, H)), topk_weights=rng.standard_normal((T, K)),
               w_gate=rng.standard_normal((E, F, H)) * 0.5, w_up=rng.standard_normal((E, F, H)) * 0.5,
               w_down=rng.standard_normal((E, H, F)) * 0.5,
               const_alpha_1=rng.standard_normal((Q, H)), const_alpha_2=rng.standard_normal((Q, H)),
               const_v=rng.standard_normal((Q, H)))
    if shared_ffn:
        inp.update(shared_w_gate=rng.standard_normal((1, F, H)) * 0.5,
                   shared_w_up=rng.standard_normal((1, F, H)) * 0.5,
                   shared_w_down=rng.standard_normal((1, H, F)) * 0.5)
    else:
        inp["shared_expert_x"] = rng.standard_normal((T, H))
    g = rng.standard_normal((T, H))
    return inp, g


def _loss(inp, g):
    return float(np.sum(orc.layer_fwd(inp, prec="f64")["out"] * g))


@pytest.mark.parametrize("shared_ffn", [False, True])
def test_backward_matches_finite_differences(shared_ffn):
    inp, g = _fd_problem(shared_ffn=shared_ffn)
    f = orc.layer_fwd(inp, prec="f64")
    b = orc.layer_bwd(inp, f, g, prec="f64")
    grads = dict(x=b["dx"], topk_weights=b["dw"], w_gate=b["dWg"], w_up=b["dWu"], w_down=b["dWd"])
    if shared_ffn:
        grads.update(shared_w_gate=b["s_dWg"], shared_w_up=b["s_dWu"], shared_w_down=b["s_dWd"])
    else:
        grads["shared_expert_x"] = b["d_shared"]
    h = 1e-6
    for name, an in grads.items():
        base = np.asarray(inp[name], np.float64)
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            p, mnus = base.copy(), base.copy()
            p[i] += h
            mnus[i] -= h
            num[i] = (_loss(dict(inp, **{name: p}), g) - _loss(dict(inp, **{name: mnus}), g)) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(num - an).max() <= 1e-6 * scale, name
    # masked slot (token 3, k=1) has no weight gradient, the zero-expert slot neither
    assert b["dw"][3, 1] == 0 and b["dw"][1, 1] == 0


def test_fp32_backward_close_to_f64():
    inp, g = _fd_problem(seed=3)
    inp32 = {k: (np.asarray(v, np.float32) if isinstance(v, np.ndarray) and v.dtype == np.float64 else v)
             for k, v in inp.items()}
    f64 = orc.layer_bwd(inp, orc.layer_fwd(inp, prec="f64"), g, prec="f64")
    f32 = orc.layer_bwd(inp32, orc.layer_fwd(inp32, prec="def"), g.astype(np.float32), prec="def")
    for k in ("dx", "dw", "dWg", "dWu", "dWd"):
        scale = max(1.0, np.abs(f64[k]).max())
        assert np.abs(f64[k] - f32[k]).max() <= 1e-5 * scale, k


# ============================================================================ fp8 / int8 path


def _lossless_fp8_rows(rng, R, C):
    """Rows whose every 128-column block is e4m3 codes times a power of two, with
    one element at +-448 times that power: per-(row,128) quantisation is exact."""
    codes = rng.integers(0, 0x7F, size=(R, C)).astype(np.uint8) | (rng.integers(0, 2, size=(R, C)) << 7).astype(np.uint8)
    v = orc.e4m3_decode(codes).astype(np.float64)
    v[:, ::128] = 448.0
    pw = 2.0 ** rng.integers(-6, 2, size=(R, C // 128))
    return (v * np.repeat(pw, 128, axis=1)).astype(np.float32)


def _lossless_fp8_blocks(rng, E, N, K):
    out = np.zeros((E, N, K), np.float32)
    for e in range(E):
        codes = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8)
        v = orc.e4m3_decode(codes).astype(np.float64) * np.where(rng.random((N, K)) < 0.5, -1, 1)
        v[::128, ::128] = 448.0
        pw = 2.0 ** rng.integers(-9, -4, size=(N // 128, K // 128))
        out[e] = v * np.kron(pw, np.ones((128, 128)))
    return out


def test_fp8_lossless_inputs_reproduce_bf16_gemm():
    """With inputs that the block quantisers represent exactly, the fp8 forward's
    G and U equal the bf16 path's bit for bit (pins block/scale indexing)."""
    rng = np.random.default_rng(21)
    E, F, H, A = 2, 256, 384, 96
    X = _lossless_fp8_rows(rng, A, H)
    Wg, Wu, Wd = _lossless_fp8_blocks(rng, E, F, H), _lossless_fp8_blocks(rng, E, F, H), \
        _lossless_fp8_blocks(rng, E, H, F)
    bits = [orc.f32_to_bf16(a) for a in (X, Wg, Wu, Wd)]
    assert all(np.array_equal(orc.bf16_to_f32(b), a) for b, a in zip(bits, (X, Wg, Wu, Wd)))
    counts = np.array([40, 96])
    wq = tuple(orc.quant_weights_fp8(b) for b in bits[1:])
    assert np.array_equal(orc.dequant_weights_fp8(*wq[0]), Wg)
    G8, U8, H8, Y8 = orc.ffn_fwd_fp8(X, counts, *wq)
    G, U, Hh, Y = orc.ffn_fwd(X, counts, *bits[1:], prec="parity")
    assert np.array_equal(G8, G) and np.array_equal(U8, U) and np.array_equal(H8, Hh)
    # the down GEMM's input h is quantised: close, not equal
    assert 0 < np.linalg.norm(Y8 - Y) / np.linalg.norm(Y) < 0.1


def test_fp8_layer_close_to_bf16_layer():
    inp = wl.layer_inputs(64, 256, 128, 4, 2, seed=22)
    f8 = orc.layer_fwd_fp8(inp)
    b8 = orc.layer_bwd_fp8(inp, f8, inp["grad_out"])
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    rel = lambda a, c: np.linalg.norm(a - c) / np.linalg.norm(c)
    for k in ("out",):
        assert 0.003 < rel(f8[k], f[k]) < 0.1, k
    for k in ("dx", "dw", "dWg", "dWu", "dWd"):
        assert 0.001 < rel(b8[k], b[k]) < 0.15, k
    # weight gradient of the down projection is a bf16 GEMM of dY and h: with the
    # fp8 path's own dY and h it is exactly the bf16 formula
    A = f8["route"].A
    ref = np.zeros_like(b8["dWd"])
    lo = 0
    for e in range(4):
        hi = int(f8["route"].ep_recv_counts[e])
        ref[e] = b8["dY"][lo:hi].T @ f8["Hh"][lo:hi]
        lo = hi
    assert np.array_equal(ref, b8["dWd"])


# Expert row counts 3, 133, 0 and 128 (inclusive prefix 3, 136, 136, 264): the
# per-128-token blocks, written out by hand, are expert 0 rows [0, 3), expert 1 rows
# [3, 131) and [131, 136), expert 3 rows [136, 264).
_COLS_PREFIX = np.array([3, 136, 136, 264])
_COLS_BLOCKS = [(0, 0, 3), (1, 3, 131), (1, 131, 136), (3, 136, 264)]


def test_cols_fp8_blocks_follow_expert_rows():
    rng = np.random.default_rng(31)
    a = rng.standard_normal((264, 4)).astype(np.float32)
    blocks = orc.quant_cols_fp8(a, _COLS_PREFIX)
    assert [(e, r0, r1) for e, r0, r1, _, _ in blocks] == _COLS_BLOCKS
    # a value changed in one (block, column) changes no other dequantised value,
    # and does change its own block's column (its scale moves)
    base = orc.qdq_cols_fp8(a, _COLS_PREFIX)
    b = a.copy()
    b[132, 1] *= 100.0
    d = orc.qdq_cols_fp8(b, _COLS_PREFIX) - base
    outside = np.ones(d.shape, bool)
    outside[131:136, 1] = False
    assert not d[outside].any()
    assert np.count_nonzero(d[131:136, 1]) >= 4


def _lossless_fp8_cols(rng, D):
    """Rows whose every (block, column) is e4m3 codes times a power of two with one
    entry at +-448 times it: per-128-token quantisation represents them exactly."""
    v = orc.e4m3_decode(rng.integers(0, 0x7F, size=(264, D)).astype(np.uint8)).astype(np.float64)
    v *= np.where(rng.random((264, D)) < 0.5, -1.0, 1.0)
    for _, r0, r1, in _COLS_BLOCKS:
        v[r0 + (r1 - r0) // 2] = 448.0
        v[r0:r1] *= 2.0 ** rng.integers(-12, 3, size=(1, D))
    return v.astype(np.float32)


def test_cols_fp8_lossless_inputs_give_exact_weight_gradient():
    rng = np.random.default_rng(32)
    P, Q = _lossless_fp8_cols(rng, 256), _lossless_fp8_cols(rng, 384)
    assert np.array_equal(orc.qdq_cols_fp8(P, _COLS_PREFIX), P)
    dW = orc.wgrad_fp8(P, Q, _COLS_PREFIX)
    for e, (lo, hi) in enumerate([(0, 3), (3, 136), (136, 136), (136, 264)]):
        ref = P[lo:hi].astype(np.float64).T @ Q[lo:hi].astype(np.float64)
        assert np.allclose(dW[e], ref, rtol=1e-12, atol=0), e
    assert not dW[2].any()  # an expert without rows has a zero gradient


def test_cols_fp8_error_within_half_ulp_of_the_block_scale():
    rng = np.random.default_rng(33)
    a = (rng.standard_normal((264, 8)) * np.exp(rng.standard_normal((1, 8)))).astype(np.float32)
    d = orc.qdq_cols_fp8(a, _COLS_PREFIX)
    worst = 0.0
    for _, r0, r1 in _COLS_BLOCKS:
        blk = a[r0:r1].astype(np.float64)
        step = np.abs(blk).max(axis=0) / 448.0           # the block scale of each column
        # e4m3: 3 mantissa bits (half ulp 2^-4 relative), subnormal spacing 2^-9
        bound = np.maximum(np.abs(blk) * 2.0 ** -4, step * 2.0 ** -10) * (1 + 1e-6)
        err = np.abs(d[r0:r1] - blk)
        assert np.all(err <= bound)
        worst = max(worst, float((err / bound).max()))
    assert worst > 0.5  # the rounding really happens


def test_fp8_weight_gradients_on_requantised_operands():
    inp = wl.layer_inputs(300, 256, 128, 3, 2, seed=34)
    f8 = orc.layer_fwd_fp8(inp)
    b16 = orc.layer_bwd_fp8(inp, f8, inp["grad_out"])
    b8 = orc.layer_bwd_fp8(inp, f8, inp["grad_out"], wgrad="fp8")
    for k in ("dGU", "dX", "dx", "dw"):
        assert np.array_equal(b8[k], b16[k]), k
    rel = lambda x, y: np.linalg.norm(x - y) / np.linalg.norm(y)
    for k in ("dWg", "dWu", "dWd"):
        assert 1e-3 < rel(b8[k], b16[k]) < 0.08, k


def test_int8_payload_lossless_rows_and_rounding():
    rng = np.random.default_rng(23)
    k = rng.integers(-127, 128, size=(10, 64)).astype(np.float64)
    k[:, 0] = 127
    s = 2.0 ** rng.integers(-8, 0, size=(10, 1))
    Y = (k * s).astype(np.float32)
    assert np.array_equal(orc.qdq_rows_int8(Y), Y)
    Y2 = rng.standard_normal((10, 64)).astype(np.float32)
    d = orc.qdq_rows_int8(Y2)
    amax = np.abs(Y2).max(axis=1, keepdims=True)
    assert np.all(np.abs(d - Y2) <= amax / 127 / 2 * 1.0001)


# ============================================================================ router


def test_router_selection_is_the_k_largest_with_ties_to_lower_id():
    """Brute force on small rows with many equal logits: the selection is the first K
    ids in (logit descending, id ascending) order, checked by a plain key sort."""
    rng = np.random.default_rng(41)
    for n, K in ((7, 3), (12, 12), (30, 8), (5, 1)):
        logits = rng.integers(-3, 4, size=(40, n)).astype(np.float32)   # many ties
        idx = orc.select_topk(logits, K)
        for r in range(logits.shape[0]):
            want = sorted(range(n), key=lambda i: (-float(logits[r, i]), i))[:K]
            assert idx[r].tolist() == want


def test_router_closed_forms():
    """logits = log(1..4): softmax = (1,2,3,4)/10; top-2 plain = (.4,.3), renormalised (4/7,3/7)."""
    logits = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    idx, w = orc.router_fwd(logits, 2, renorm=False)
    assert idx.tolist() == [[3, 2]]
    np.testing.assert_allclose(w, [[0.4, 0.3]], rtol=1e-14)
    _, w = orc.router_fwd(logits, 2, renorm=True)
    np.testing.assert_allclose(w, [[4 / 7, 3 / 7]], rtol=1e-14)
    _, w = orc.router_fwd(logits, 4, renorm=False)
    np.testing.assert_allclose(w, [[0.4, 0.3, 0.2, 0.1]], rtol=1e-14)


def test_router_weights_match_torch_softmax():
    """Plain weights = torch.softmax over all ids at the selection; renormalised =
    torch.softmax over the selected logits."""
    rng = np.random.default_rng(42)
    logits = rng.standard_normal((64, 37)) * 3
    t = torch.from_numpy(logits)
    for renorm in (False, True):
        idx, w = orc.router_fwd(logits, 6, renorm)
        ti = torch.from_numpy(idx.astype(np.int64))
        ref = torch.softmax(t.gather(1, ti), dim=1) if renorm else torch.softmax(t, dim=1).gather(1, ti)
        np.testing.assert_allclose(w, ref.numpy(), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("renorm", [False, True])
def test_router_backward_matches_torch_autograd_and_finite_differences(renorm):
    rng = np.random.default_rng(43 + renorm)
    T, n, K = 16, 21, 5
    # distinct, well separated logits: the selection does not move under the FD step
    logits = np.stack([rng.permutation(n) * 0.37 + rng.standard_normal() for _ in range(T)])
    idx, _ = orc.router_fwd(logits, K, renorm)
    dw = rng.standard_normal((T, K))
    dl = orc.router_bwd(logits, idx, dw, renorm)
    # torch autograd through softmax / gather (/ renormalisation), selection fixed
    t = torch.from_numpy(logits).requires_grad_(True)
    ti = torch.from_numpy(idx.astype(np.int64))
    w = torch.softmax(t, dim=1).gather(1, ti)
    if renorm:
        w = w / w.sum(dim=1, keepdim=True)
    (w * torch.from_numpy(dw)).sum().backward()
    np.testing.assert_allclose(dl, t.grad.numpy(), rtol=1e-12, atol=1e-14)
    # central differences of L(l) = sum(dw * w(l))
    def L(z):
        return float((orc.router_fwd(z, K, renorm)[1] * dw).sum())
    eps = 1e-6
    for r, i in ((0, int(idx[0, 0])), (3, int(idx[3, K - 1])), (5, int(np.argmin(logits[5]))), (9, 0)):
        zp, zm = logits.copy(), logits.copy()
        zp[r, i] += eps
        zm[r, i] -= eps
        assert abs((L(zp) - L(zm)) / (2 * eps) - dl[r, i]) < 1e-7
    # softmax-type gradients sum to zero over a row; unselected ids get none when renormalised
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-13)
    if renorm:
        mask = np.ones_like(dl, dtype=bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert (dl[mask] == 0).all()


# ============================================================================ int8 dispatch + w8a8 FFN


def test_int8_dispatch_hand_example():
    """One token routed to expert 1 of 2, H = 8, smooth scales chosen by hand:
    x * scales[1] = [3, -3, 2, 0, 0, 0, 0, 2], amax 3, so the codes are
    rint(v * 127/3) = [127, -127, 85, 0, 0, 0, 0, 85] and the scale 3/127."""
    x = np.array([[3, -6, 1, 0, 0, 0, 0, 0.5]], np.float32)
    S = np.ones((2, 8), np.float32)
    S[1] = [1, 0.5, 2, 1, 1, 1, 1, 4]
    r = orc.route(np.array([[1]], np.int32), 2)
    q, s = orc.dispatch_int8(orc.f32_to_bf16(x), r, S)
    assert q.tolist() == [[127, -127, 85, 0, 0, 0, 0, 85]]
    assert s.tolist() == [np.float32(3.0) / np.float32(127.0)]
    # without smooth scales: amax 6, codes rint(v * 127/6)
    q, s = orc.dispatch_int8(orc.f32_to_bf16(x), r)
    assert q.tolist() == [[64, -127, 21, 0, 0, 0, 0, 11]] and s.tolist() == [np.float32(6.0) / np.float32(127.0)]


def test_int8_dispatch_uses_each_rows_own_expert_scales():
    """Integer rows with a +-127 entry are exact in int8; expert e's smooth scale
    2^e then leaves the codes unchanged and makes the row's dynamic scale exactly
    2^e, which names the scale row each expanded row used."""
    rng = np.random.default_rng(51)
    T, H, E, K = 40, 64, 5, 3
    x = rng.integers(-127, 128, size=(T, H)).astype(np.float32)
    x[:, 7] = 127.0
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    r = orc.route(idx, E)
    q0, s0 = orc.dispatch_int8(orc.f32_to_bf16(x), r)
    X = orc.dispatch(orc.f32_to_bf16(x), r)
    assert np.array_equal(q0.astype(np.float32), X) and np.all(s0 == 1.0)
    S = np.exp2(np.arange(E, dtype=np.float32))[:, None] * np.ones((E, H), np.float32)
    q1, s1 = orc.dispatch_int8(orc.f32_to_bf16(x), r, S)
    assert np.array_equal(q1, q0)
    row_expert = np.repeat(np.arange(E), np.diff(np.concatenate([[0], r.ep_recv_counts])))
    assert np.array_equal(s1, np.exp2(row_expert).astype(np.float32))


def test_int8_ffn_lossless_inputs_reproduce_bf16_gate_up():
    """Integer activations and weights with a +-127 per row and channel quantise
    exactly (scale 1); the integer products are exact in fp32 too, so G, U and h of
    the w8a8 FFN equal the bf16 FFN's bit for bit."""
    rng = np.random.default_rng(52)
    E, F, H, A = 3, 64, 128, 50
    X = rng.integers(-127, 128, size=(A, H)).astype(np.float32)
    X[:, 3] = -127.0
    def w(n, k):
        a = rng.integers(-127, 128, size=(E, n, k)).astype(np.float32)
        a[:, :, 5] = 127.0
        return a
    Wg, Wu, Wd = w(F, H), w(F, H), w(H, F)
    counts = np.array([10, 10, 50])
    wq = tuple(orc.quant_weights_int8(orc.f32_to_bf16(a)) for a in (Wg, Wu, Wd))
    assert np.array_equal(wq[0][0].astype(np.float32), Wg) and np.all(wq[0][1] == 1.0)
    Xq, xs = orc.quant_int8_rows(X)
    assert np.array_equal(Xq.astype(np.float32), X) and np.all(xs == 1.0)
    G8, U8, H8, hq, hs, Y8 = orc.ffn_fwd_int8(Xq, xs, counts, *wq)
    G, U, Hh, Y = orc.ffn_fwd(X, counts, *(orc.f32_to_bf16(a) for a in (Wg, Wu, Wd)), prec="parity")
    assert np.array_equal(G8, G) and np.array_equal(U8, U) and np.array_equal(H8, Hh)
    assert np.array_equal(orc.dequant_int8_rows(hq, hs)[10:], orc.qdq_rows_int8(Hh[10:]))
    assert 0 < np.linalg.norm(Y8 - Y) / np.linalg.norm(Y) < 0.02


def test_int8_layer_close_to_bf16_layer():
    inp = wl.layer_inputs(96, 256, 128, 6, 2, seed=53, Z=1, C=1)
    f8 = orc.layer_fwd_int8(inp)
    f = orc.layer_fwd(inp, prec="parity")
    rel = np.linalg.norm(f8["out"] - f["out"]) / np.linalg.norm(f["out"])
    assert 1e-3 < rel < 0.05


def test_int8_gemm_sums_are_exact_integers():
    """The w8a8 sums equal the integer matrix product (taken in int64 here) at the
    largest magnitudes: all codes +-127 over a long contraction."""
    rng = np.random.default_rng(54)
    K = 20000
    q = np.where(rng.random((6, K)) < 0.5, -127, 127).astype(np.int8)
    w = np.where(rng.random((5, K)) < 0.5, -127, 127).astype(np.int8)
    w[0] = q[0]                                       # a sum of 127^2 * K
    got = orc.moe._i8_gemm(q, np.ones(6, np.float32), w, np.ones(5, np.float32))
    ref = q.astype(np.int64) @ w.astype(np.int64).T
    assert ref[0, 0] == 127 * 127 * K
    assert np.array_equal(got, ref.astype(np.float64))


# ============================================================================ MX (microscaled) fp8


def test_mx_quantiser_hand_examples():
    """448 = 1.75 * 2^8 is the largest block maximum of scale 2^0 (byte 127): codes of
    448, 1, -2, 0.5 are 0x7E, 0x38, 0xC0, 0x30; 449 needs scale 2^1 (byte 128) and
    449 / 2 = 224.5 rounds to 224 = 0x76; an all-zero block gets byte 0."""
    x = np.zeros((3, 32), np.float32)
    x[0, :4] = [448, 1, -2, 0.5]
    x[1, 0] = 449
    q, s = orc.quant_mx_e4m3_rows(x)
    assert q[0, :4].tolist() == [0x7E, 0x38, 0xC0, 0x30] and not q[0, 4:].any()
    assert q[1, 0] == 0x76 and s[:, 0].tolist() == [127, 128, 0]
    assert not q[2].any()


def test_mx_scale_is_the_smallest_power_of_two_without_saturation():
    rng = np.random.default_rng(71)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 1)))).astype(np.float32)
    q, s = orc.quant_mx_e4m3_rows(x)
    X = np.exp2(s.astype(np.float64) - 127.0)
    amax = np.abs(x.astype(np.float64)).reshape(64, 8, 32).max(axis=2)
    assert np.all(amax / X <= 448.0) and np.all(amax / X > 224.0)
    # every code is the rounding of x / X (half an e4m3 step, subnormal spacing 2^-9)
    d = orc.dequant_mx_e4m3_rows(q, s)
    err = np.abs(d - x).reshape(64, 8, 32)
    bound = np.maximum(np.abs(x.astype(np.float64)).reshape(64, 8, 32) * 2.0 ** -4, X[:, :, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))


def test_mx_lossless_inputs_reproduce_bf16_gate_up():
    """Activations and weights whose every 32-block along the contraction is e4m3 codes
    times 2^k with one entry at 448 * 2^k are exact in MX, so the MX forward's G, U, h
    equal the bf16 FFN's bit for bit."""
    rng = np.random.default_rng(72)
    def lossless(shape):
        v = orc.e4m3_decode(rng.integers(0, 0x7F, size=shape).astype(np.uint8)).astype(np.float64)
        v *= np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        v[..., ::32] = 448.0
        k = rng.integers(-14, -6, size=shape[:-1] + (shape[-1] // 32,))
        return (v * np.repeat(np.exp2(k), 32, axis=-1)).astype(np.float32)
    E, F, H, A = 2, 64, 128, 40
    X = lossless((A, H))
    Wg, Wu, Wd = lossless((E, F, H)), lossless((E, F, H)), lossless((E, H, F))
    bits = [orc.f32_to_bf16(a) for a in (X, Wg, Wu, Wd)]
    assert all(np.array_equal(orc.bf16_to_f32(b), a) for b, a in zip(bits, (X, Wg, Wu, Wd)))
    counts = np.array([15, 40])
    wq = tuple(orc.quant_weights_mx(b) for b in bits[1:])
    G8, U8, H8, _ = orc.ffn_fwd_mx(X, counts, *wq)
    G, U, Hh, _ = orc.ffn_fwd(X, counts, *bits[1:], prec="parity")
    assert np.array_equal(G8, G) and np.array_equal(U8, U) and np.array_equal(H8, Hh)


def test_mx_layer_close_to_bf16_layer():
    inp = wl.layer_inputs(96, 256, 128, 4, 2, seed=73)
    fm = orc.layer_fwd_mx(inp)
    bm = orc.layer_bwd_mx(inp, fm, inp["grad_out"])
    f = orc.layer_fwd(inp, prec="parity")
    b = orc.layer_bwd(inp, f, inp["grad_out"], prec="parity")
    rel = lambda a, c: np.linalg.norm(a - c) / np.linalg.norm(c)
    assert 0.003 < rel(fm["out"], f["out"]) < 0.1
    for k in ("dx", "dw", "dWg", "dWu", "dWd"):
        assert 0.001 < rel(bm[k], b[k]) < 0.15, k
