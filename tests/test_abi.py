"""CPU checks of the C ABI: the library loads, exports every function include/moe.h
declares, and its host-side validation returns the documented status codes
before touching the GPU (every call below fails validation, so nothing is
launched)."""
import ctypes
import os
import re

import pytest

import dispatch_expert_gemm_amd as dm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL_ARG, BAD_SHAPE, BAD_RANGE, CAPACITY, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dm.LIB_PATH):
        pytest.skip("libmoe.so not built (run __graft_entry__.build())")
    return dm.lib()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(dm.ENTRY_POINTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in (OK, NULL_ARG, BAD_SHAPE, BAD_RANGE, CAPACITY, UNSUPPORTED, WORKSPACE, -7):
        assert L.moe_status_str(st)
    assert b"unknown" in L.moe_status_str(12345)


def S(**kw):
    base = dict(T=8, H=1536, K=8, num_experts=32, F=480)
    base.update(kw)
    return dm.make_shape(**base)


def ws(shape):
    n = ctypes.c_size_t()
    st = dm.lib().moe_workspace_size(ctypes.byref(shape) if shape is not None else None,
                                     ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,expect", [
    (dict(), OK),
    (dict(K=0), BAD_SHAPE),
    (dict(K=17, zero_expert_num=4), BAD_SHAPE),          # 0 < K <= 16
    (dict(K=8, num_experts=4), BAD_SHAPE),                # K > E+Z+C+Q
    (dict(K=8, num_experts=4, zero_expert_num=2, copy_expert_num=1, const_expert_num=1), OK),
    (dict(num_experts=0), BAD_SHAPE),
    (dict(num_experts=1025), BAD_SHAPE),                  # num_experts in [1, 1024]
    (dict(H=100), BAD_SHAPE),                             # H multiple of 8
    (dict(T=-1), BAD_SHAPE),
    (dict(capacity=8 * 8 - 1), CAPACITY),                 # A >= BS * min(E, K)
    (dict(K=4, num_experts=2, zero_expert_num=2, capacity=8 * 2), OK),
    (dict(zero_expert_num=-1), BAD_SHAPE),
    (dict(mask_ndim=3), BAD_RANGE),
    (dict(T=0), OK),
])
def test_shape_validation(L, kw, expect):
    st, n = ws(S(**kw))
    assert st == expect
    if st == OK:
        assert n > 0 and n % 256 == 0


def test_shape_validation_misc(L):
    assert ws(None)[0] == NULL_ARG
    s = S()
    s.act_dtype = 7
    assert ws(s)[0] == UNSUPPORTED
    s = S()
    s.comm_quant_mode = 1
    assert ws(s)[0] == BAD_RANGE
    s.comm_quant_mode = 2
    assert ws(s)[0] == OK
    n = ctypes.c_int64()
    assert L.moe_assist_info_size(ctypes.byref(S()), ctypes.byref(n)) == OK
    assert n.value == 8 * 8 + 8 * 8


def P(v=0x1000):
    return ctypes.c_void_p(v)   # a non-NULL stand-in: never dereferenced (validation fails first)


def test_entry_points_reject_bad_arguments_before_launch(L):
    s = S()
    sp = ctypes.byref(s)
    Nn = None
    # dispatch: NULL required outputs, missing mask, small workspace
    assert L.moe_dispatch(sp, P(), P(), Nn, P(), P(), P(), P(), Nn, P(), 1 << 20, Nn) == NULL_ARG
    sm = S(mask_ndim=1)
    assert L.moe_dispatch(ctypes.byref(sm), P(), P(), Nn, P(), P(), P(), P(), P(), P(), 1 << 20, Nn) == NULL_ARG
    assert L.moe_dispatch(sp, P(), P(), Nn, P(), P(), P(), P(), P(), P(), 16, Nn) == WORKSPACE
    assert L.moe_dispatch(sp, P(), P(), Nn, P(), P(), P(), P(), P(), Nn, 1 << 20, Nn) == WORKSPACE
    # combine: ori_x required with copy/const experts, const tensors with const experts
    sc = S(copy_expert_num=1)
    assert L.moe_combine(ctypes.byref(sc), P(), P(), P(), P(), P(), Nn, Nn, Nn, Nn, Nn, Nn, P(), Nn) == NULL_ARG
    sq = S(const_expert_num=2)
    assert L.moe_combine(ctypes.byref(sq), P(), P(), P(), P(), P(), Nn, Nn, P(), P(), Nn, P(), P(), Nn) == NULL_ARG
    assert L.moe_combine_bwd(ctypes.byref(sq), P(), P(), P(), P(), P(), P(), Nn, P(), P(), P(), Nn, P(), P(), Nn) == NULL_ARG
    # combine backward: either output may be left out, not both; y only with the weights' gradient
    assert L.moe_combine_bwd(sp, P(), P(), P(), P(), P(), P(), Nn, Nn, Nn, Nn, Nn, Nn, Nn, Nn) == NULL_ARG
    assert L.moe_combine_bwd(sp, P(), Nn, P(), P(), P(), P(), Nn, Nn, Nn, Nn, Nn, Nn, P(), Nn) == NULL_ARG
    assert L.moe_dispatch_bwd(ctypes.byref(sq), P(), P(), P(), P(), Nn, P(), Nn, Nn, P(), Nn) == NULL_ARG
    assert L.moe_dispatch_bwd(ctypes.byref(sc), P(), P(), P(), P(), Nn, Nn, Nn, Nn, P(), Nn) == NULL_ARG
    # FFN: F must be a positive multiple of 32
    for F in (0, 48, -32):
        sf = S(F=F)
        assert L.moe_grouped_ffn(ctypes.byref(sf), P(), P(), P(), P(), P(), P(), P(), P(), Nn) == BAD_SHAPE
        assert L.moe_grouped_ffn_bwd(ctypes.byref(sf), *([P()] * 13), Nn) == BAD_SHAPE
    # one expert's weight matrix must stay below 2 GiB (32-bit offsets)
    big = ctypes.byref(S(H=32768, F=32768))
    assert L.moe_grouped_ffn(big, P(), P(), P(), P(), P(), P(), P(), P(), Nn) == UNSUPPORTED
    assert L.moe_grouped_ffn_bwd(big, *([P()] * 13), Nn) == UNSUPPORTED
    assert L.moe_ffn_gate_up_bwd_weight(big, P(), P(), P(), P(), P(), Nn) == UNSUPPORTED
    # fp8: the activation scales of all rows must stay below 2 GiB
    s8 = S(T=1 << 21, K=8, num_experts=8, H=32768, F=128)   # capacity 2^24 rows x 256 blocks x 4 B
    assert L.moe_ffn_gate_up_fwd_fp8(ctypes.byref(s8), *([P()] * 9), Nn) == UNSUPPORTED
    ok = ctypes.byref(S(H=32768, F=32736))   # 2^31 - 2^21 bytes per matrix: accepted
    assert L.moe_ffn_gate_up_fwd(ok, Nn, P(), P(), P(), P(), P(), Nn) == NULL_ARG
    assert L.moe_grouped_ffn(sp, P(), Nn, P(), P(), P(), P(), P(), P(), Nn) == NULL_ARG
    assert L.moe_ffn_down_bwd_weight(sp, P(), P(), P(), Nn, Nn) == NULL_ARG
    assert L.moe_ffn_gate_up_bwd_weight(sp, P(), P(), P(), P(), Nn, Nn) == NULL_ARG
    assert L.moe_ffn_gate_up_fwd(sp, Nn, P(), P(), P(), P(), P(), Nn) == NULL_ARG
    assert L.moe_ffn_down_fwd(sp, P(), P(), P(), Nn, Nn) == NULL_ARG
    assert L.moe_ffn_down_bwd_data(sp, P(), P(), Nn, P(), P(), Nn) == NULL_ARG
    assert L.moe_ffn_gate_up_bwd_data(sp, P(), P(), Nn, P(), P(), Nn) == NULL_ARG
    # bad shapes are rejected by every entry
    bad = ctypes.byref(S(K=0))
    assert L.moe_combine(bad, *([P()] * 12), Nn) == BAD_SHAPE
    assert L.moe_dispatch(bad, *([P()] * 8), P(), 1 << 20, Nn) == BAD_SHAPE


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and refuses non-GPU tensors."""
    pkg = os.path.join(ROOT, "dispatch_expert_gemm_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle/", ""), fn
    import torch
    with pytest.raises(dm.MoeError):
        dm._ptr(torch.zeros(3), torch.float32, "cpu tensor")


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_gemm_roofs_at_the_page1_shape():
    """The benchmark's algorithmic bytes of the six bf16 GEMMs at the page-1 shape
    (A = 65,536 routed rows, H = 1536, F = 480, E = 64), written out by hand per
    operand, and the roof each meets first (FLOPs at 2.5 PFLOP/s against bytes at
    8 TB/s)."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    A, H, F, E, T = 65536, 1536, 480, 64, 8192
    mb = 1e6
    want = {
        # weights (bf16) + x rows + h, G, U out
        "moe_ffn_gate_up_fwd_gather": (64 * 960 * 1536 * 2 + A * 1536 * 2 + A * 1440 * 2, "mfma"),
        # W_down + h rows + y out
        "moe_ffn_down_fwd": (64 * 1536 * 480 * 2 + A * 480 * 2 + A * 1536 * 2, "hbm"),
        # dY rows + W_down + saved G|U in, dG|dU out
        "moe_ffn_down_bwd_data": (A * 1536 * 2 + 64 * 1536 * 480 * 2 + 2 * A * 960 * 2, "hbm"),
        # dY, h rows in, fp32 dW_down out
        "moe_ffn_down_bwd_weight": (A * 1536 * 2 + A * 480 * 2 + 64 * 1536 * 480 * 4, "hbm"),
        # dG|dU rows + both weights in, dX out
        "moe_ffn_gate_up_bwd_data": (A * 960 * 2 + 64 * 960 * 1536 * 2 + A * 1536 * 2, "mfma"),
        # dG|dU, x rows in, fp32 dW_gate, dW_up out
        "moe_ffn_gate_up_bwd_weight_gather": (A * 960 * 2 + A * 1536 * 2 + 64 * 960 * 1536 * 4, "hbm"),
    }
    flops = {k: (4 if "gate_up" in k else 2) * A * H * F for k in want}
    for k, (nbytes, roof) in want.items():
        got = bench.gemm_bytes(k, A, H, F, E, T)
        assert got == nbytes, (k, got / mb, nbytes / mb)
        t_mfma, t_hbm = flops[k] / 2.5e15, got / 8e12
        assert ("hbm" if t_hbm > t_mfma else "mfma") == roof, k
    # 8-bit GEMMs other than the int8 forward ones are set against the MFMA peak only
    assert bench.gemm_bytes("moe_ffn_down_bwd_data_fp8", A, H, F, E, T) == 0
    # the shared expert: the same counts with T rows and one expert
    assert bench.gemm_bytes("shared moe_ffn_down_fwd", A, H, F, E, T) == bench.gemm_bytes(
        "moe_ffn_down_fwd", T, H, F, 1)


def test_router_rejects_bad_arguments_before_launch(L):
    Nn = None
    # (T, n_ids, K, renorm): K in (0, min(16, n_ids)], n_ids in [1, 4096], renorm 0/1
    for T, n, K, rn, want in ((4, 8, 0, 1, BAD_SHAPE), (4, 8, 9, 1, BAD_SHAPE), (4, 64, 17, 1, BAD_SHAPE),
                              (4, 4097, 8, 1, BAD_SHAPE), (4, 0, 1, 1, BAD_SHAPE), (-1, 8, 2, 1, BAD_SHAPE),
                              (4, 8, 2, 2, BAD_RANGE)):
        assert L.moe_router(T, n, K, rn, P(), P(), P(), Nn) == want
        assert L.moe_router_bwd(T, n, K, rn, P(), P(), P(), P(), P(), Nn) == want
    assert L.moe_router(0, 8, 2, 1, Nn, Nn, Nn, Nn) == OK            # no tokens: nothing to do
    assert L.moe_router(4, 8, 2, 1, P(), Nn, P(), Nn) == NULL_ARG
    assert L.moe_router_bwd(4, 8, 2, 0, Nn, P(), P(), P(), P(), Nn) == NULL_ARG   # plain gating needs logits
    assert L.moe_router_bwd(4, 4096, 16, 1, P(), P(), P(), P(), Nn, Nn) == NULL_ARG


def test_fp8_weight_gradient_entries_reject_bad_arguments_before_launch(L):
    Nn = None
    # column quantiser: D a positive multiple of 128, at least one expert, counts given
    for D in (0, 100, -128):
        assert L.moe_quant_cols_fp8(256, D, 4, P(), P(), P(), P(), Nn) == BAD_SHAPE
    assert L.moe_quant_cols_fp8(256, 128, 0, P(), P(), P(), P(), Nn) == BAD_SHAPE
    assert L.moe_quant_cols_fp8(-1, 128, 4, P(), P(), P(), P(), Nn) == BAD_SHAPE
    assert L.moe_quant_cols_fp8(256, 128, 4, P(), Nn, P(), P(), Nn) == NULL_ARG
    assert L.moe_quant_cols_fp8(256, 128, 4, P(), P(), Nn, P(), Nn) == NULL_ARG
    assert L.moe_quant_cols_fp8(0, 128, 4, Nn, P(), Nn, Nn, Nn) == OK   # nothing to do
    # GEMMs: the fp8 shape rules (H = 1536, F = 480 is not a multiple of 128)
    s = ctypes.byref(S())
    assert L.moe_ffn_down_bwd_weight_fp8(s, *([P()] * 6), Nn) == BAD_SHAPE
    assert L.moe_ffn_gate_up_bwd_weight_fp8(s, *([P()] * 7), Nn) == BAD_SHAPE
    s8 = ctypes.byref(S(F=512))
    assert L.moe_ffn_down_bwd_weight_fp8(s8, P(), P(), P(), P(), Nn, P(), Nn) == NULL_ARG
    assert L.moe_ffn_gate_up_bwd_weight_fp8(s8, P(), P(), P(), P(), P(), P(), Nn, Nn) == NULL_ARG
    assert L.moe_ffn_down_bwd_weight_fp8(s8, Nn, P(), P(), P(), P(), P(), Nn) == NULL_ARG
    # code rows of (capacity/128 + E) * 128 bytes, addressed with 32-bit offsets
    wide = ctypes.byref(S(T=1 << 16, K=8, num_experts=8, H=4096, F=512))   # 2^19 rows: 4096 * 2^19 > 2^31
    assert L.moe_ffn_down_bwd_weight_fp8(wide, *([P()] * 6), Nn) == UNSUPPORTED
    assert L.moe_ffn_gate_up_bwd_weight_fp8(wide, *([P()] * 7), Nn) == UNSUPPORTED


def test_fused_quantising_data_gradient_rejects_bad_arguments(L):
    Nn = None
    s8 = ctypes.byref(S(F=512))
    args = [P()] * 6   # dyq, dys, wdq_t, wds, gate_up_save, ep_recv_counts
    # nothing to produce
    assert L.moe_ffn_down_bwd_data_fp8_quant(s8, *args, Nn, Nn, Nn, Nn, Nn, Nn) == NULL_ARG
    # codes without scales (and the reverse)
    assert L.moe_ffn_down_bwd_data_fp8_quant(s8, *args, Nn, P(), Nn, Nn, Nn, Nn) == NULL_ARG
    assert L.moe_ffn_down_bwd_data_fp8_quant(s8, *args, Nn, Nn, Nn, Nn, P(), Nn) == NULL_ARG
    # fp8 shape rules
    assert L.moe_ffn_down_bwd_data_fp8_quant(ctypes.byref(S()), *args, P(), Nn, Nn, Nn, Nn, Nn) == BAD_SHAPE


def test_int8_entries_reject_bad_arguments_before_launch(L):
    Nn = None
    s = S(F=512)
    sp = ctypes.byref(s)
    # dispatch: the row lives in registers, H <= 8192
    assert L.moe_dispatch_int8(ctypes.byref(S(H=8200)), *([P()] * 11), 1 << 20, Nn) == UNSUPPORTED
    # NULL expanded rows / scales, small workspace
    assert L.moe_dispatch_int8(sp, P(), P(), Nn, Nn, Nn, P(), P(), P(), P(), P(), P(), 1 << 20, Nn) == NULL_ARG
    assert L.moe_dispatch_int8(sp, P(), P(), Nn, Nn, P(), Nn, P(), P(), P(), P(), P(), 1 << 20, Nn) == NULL_ARG
    assert L.moe_dispatch_int8(sp, P(), P(), Nn, Nn, P(), P(), P(), P(), P(), P(), P(), 16, Nn) == WORKSPACE
    # row quantiser: C a positive multiple of 8
    for C in (0, 12, -8):
        assert L.moe_quant_rows_int8(4, C, P(), Nn, P(), P(), Nn) == BAD_SHAPE
    assert L.moe_quant_rows_int8(4, 16, P(), Nn, Nn, P(), Nn) == NULL_ARG
    assert L.moe_quant_rows_int8(0, 16, Nn, Nn, Nn, Nn, Nn) == OK
    # GEMMs: the 8-bit shape rules (F = 480 is not a multiple of 128), NULL weights
    assert L.moe_ffn_gate_up_fwd_int8(ctypes.byref(S()), *([P()] * 9), Nn) == BAD_SHAPE
    assert L.moe_ffn_down_fwd_int8(ctypes.byref(S()), *([P()] * 6), Nn) == BAD_SHAPE
    assert L.moe_ffn_gate_up_fwd_int8(sp, P(), P(), Nn, P(), P(), P(), P(), P(), P(), Nn) == NULL_ARG
    assert L.moe_ffn_down_fwd_int8(sp, P(), P(), P(), Nn, P(), P(), Nn) == NULL_ARG


def test_mx_entries_reject_bad_arguments_before_launch(L):
    Nn = None
    for C in (0, 48, -32):
        assert L.moe_quant_rows_mx(4, C, P(), Nn, P(), P(), Nn) == BAD_SHAPE
    assert L.moe_quant_rows_mx(4, 64, P(), Nn, Nn, P(), Nn) == NULL_ARG
    assert L.moe_quant_rows_mx(0, 64, Nn, Nn, Nn, Nn, Nn) == OK
    assert L.moe_quantize_weights_mx(2, 100, 128, P(), P(), P(), Nn, Nn, Nn) == BAD_SHAPE
    assert L.moe_quantize_weights_mx(2, 128, 128, P(), P(), P(), P(), Nn, Nn) == NULL_ARG   # codes_t without scales_t
    s8 = ctypes.byref(S(F=512))
    assert L.moe_ffn_gate_up_fwd_mx(ctypes.byref(S()), *([P()] * 11), Nn) == BAD_SHAPE    # F = 480
    assert L.moe_ffn_gate_up_fwd_mx(s8, P(), P(), Nn, P(), P(), P(), P(), P(), P(), Nn, Nn, Nn) == NULL_ARG
    assert L.moe_ffn_gate_up_fwd_mx(s8, *([P()] * 9), P(), Nn, Nn) == NULL_ARG       # codes without scales
    assert L.moe_ffn_down_fwd_mx(s8, P(), P(), P(), Nn, P(), P(), Nn) == NULL_ARG
    assert L.moe_ffn_down_bwd_data_mx(s8, P(), P(), P(), P(), P(), P(), Nn, Nn, Nn, Nn) == NULL_ARG  # no output
    assert L.moe_ffn_gate_up_bwd_data_mx(s8, P(), P(), P(), P(), P(), Nn, P(), P(), Nn) == NULL_ARG


def test_wrappers_reject_short_buffers():
    """The Python entries compare each buffer with the size its layout needs before
    any pointer reaches the library (checked ahead of the device check, so CPU
    tensors show it): a short buffer is an error, not an out-of-bounds access."""
    import torch
    import dispatch_expert_gemm_amd as dm
    s = dm.make_shape(T=16, H=128, K=2, num_experts=4, F=128, capacity=64)
    bf = lambda *n: torch.zeros(n, dtype=torch.bfloat16)
    i32 = lambda *n: torch.zeros(n, dtype=torch.int32)
    ok = dict(expand_x=bf(64, 128), w_gate=bf(4, 128, 128), w_up=bf(4, 128, 128),
              ep_recv_counts=i32(4), gate_up_save=bf(64, 256), h_act=bf(64, 128))
    with pytest.raises(dm.MoeError, match="GPU tensor"):      # sizes fine: the device check fires
        dm.moe_ffn_gate_up_fwd(s, **ok)
    for name, short in (("expand_x", bf(63, 128)), ("w_up", bf(4, 127, 128)), ("ep_recv_counts", i32(3)),
                        ("gate_up_save", bf(64, 255)), ("h_act", bf(1))):
        with pytest.raises(dm.MoeError, match=f"{name} holds"):
            dm.moe_ffn_gate_up_fwd(s, **{**ok, name: short})
    with pytest.raises(dm.MoeError, match="codes holds"):
        dm.moe_quant_rows_mx(bf(8, 256), torch.zeros(8 * 256 - 1, dtype=torch.uint8),
                             torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(dm.MoeError, match="scales holds"):
        dm.moe_quant_rows_fp8(bf(8, 256), torch.zeros(8 * 256, dtype=torch.uint8),
                              torch.zeros(15, dtype=torch.float32))


def test_noalloc_dispatch_checks_before_any_device_call(L):
    """moe_dispatch_noalloc validates like moe_dispatch before touching the GPU, and its
    fixed 256 KiB routing scratch holds the workspace of every shape the library accepts
    (at most 256 chunks and 32768 (chunk, expert) counts)."""
    Nn, sp = None, ctypes.byref(S())
    assert L.moe_dispatch_noalloc(ctypes.byref(S(K=0)), P(), P(), Nn, P(), P(), P(), P(), P(), Nn) == BAD_SHAPE
    assert L.moe_dispatch_noalloc(sp, Nn, P(), Nn, P(), P(), P(), P(), P(), Nn) == NULL_ARG
    assert L.moe_dispatch_noalloc(sp, P(), P(), Nn, P(), P(), P(), P(), Nn, Nn) == NULL_ARG
    sm = S(mask_ndim=2)
    assert L.moe_dispatch_noalloc(ctypes.byref(sm), P(), P(), Nn, P(), P(), P(), P(), P(), Nn) == NULL_ARG
    worst = 0
    for E in (1, 3, 7, 64, 255, 256, 1000, 1024):
        for K in (1, 2, 8, 16):
            if K > E:
                continue
            for T in (0, 1, 100, 4096, 65536, 1 << 20, 1 << 24):
                st, n = ws(dm.make_shape(T, 64, K, E))
                assert st == OK
                worst = max(worst, n)
    assert worst <= 256 << 10, worst


def test_decode_fused_checks_before_any_device_call(L):
    """moe_decode_fused (the decode regime: at most 512 tokens) validates the shape,
    its pointers and the workspace before touching the GPU."""
    Nn = None
    n = ctypes.c_size_t()
    dec = dm.make_shape(512, 7168, 8, 32, F=2048)
    assert L.moe_decode_fused_workspace_size(ctypes.byref(dec), ctypes.byref(n)) == OK
    cap = dec.capacity
    # control words, per-expert counters and counts, both maps, h and y rows
    assert n.value >= cap * (2048 + 7168) * 2 + (512 * 8 + cap) * 4
    assert L.moe_decode_fused_workspace_size(ctypes.byref(dec), Nn) == NULL_ARG

    def call(s, ws_bytes=1 << 40, **over):
        args = dict(x=P(), idx=P(), w=P(), mask=Nn, wg=P(), wu=P(), wd=P(), sh=Nn, ori=Nn, a1=Nn, a2=Nn,
                    cv=Nn, out=P(), err=P(), ws=P())
        args.update(over)
        return L.moe_decode_fused(ctypes.byref(s), *args.values(), ws_bytes, Nn)

    for s, want in ((dm.make_shape(513, 7168, 8, 32, F=2048), UNSUPPORTED),   # more than 512 tokens
                    (dm.make_shape(64, 7168 + 64, 8, 32, F=2048), BAD_SHAPE),  # H not a multiple of 128
                    (dm.make_shape(64, 7168, 8, 32, F=2048 + 32), BAD_SHAPE),  # F not a multiple of 64
                    (dm.make_shape(64, 7168, 0, 32, F=2048), BAD_SHAPE)):
        assert call(s) == want
        st = L.moe_decode_fused_workspace_size(ctypes.byref(s), ctypes.byref(n))
        assert st == want
    s = dm.make_shape(64, 7168, 8, 32, F=2048)
    assert call(s, err=Nn) == NULL_ARG
    assert call(s, wd=Nn) == NULL_ARG
    assert call(dm.make_shape(64, 7168, 8, 32, F=2048, mask_ndim=2)) == NULL_ARG
    assert call(dm.make_shape(64, 7168, 8, 32, F=2048, copy_expert_num=1)) == NULL_ARG
    assert L.moe_decode_fused_workspace_size(ctypes.byref(s), ctypes.byref(n)) == OK
    assert call(s, ws_bytes=n.value - 1) == WORKSPACE
    assert call(s, ws=Nn) == WORKSPACE
