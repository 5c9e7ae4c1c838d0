"""Python binding of libmoe.so, the one-device MoE layer library for MI355X (gfx950).

The functions below carry the names of the C entry points in include/moe.h and
only marshal arguments: every step of the layer runs in the library's HIP
kernels, on torch's current stream.  torch provides device memory and streams.
There is no fallback: if libmoe.so is missing, or a tensor is not a contiguous
GPU tensor of the right dtype, the call raises.

``moe_layer`` wraps the whole forward and backward in a torch.autograd.Function.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmoe.so")

MOE_FLAG_ID_RANGE = 1
MOE_FLAG_ID_DUPLICATE = 2
MOE_FLAG_MASK_NOT_PREFIX = 4
MOE_FLAG_SYNC_TIMEOUT = 8
MOE_SLOT_NONE = -1
MOE_SLOT_COPY = -2

# every function include/moe.h declares
ENTRY_POINTS = (
    "moe_status_str", "moe_assist_info_size", "moe_workspace_size", "moe_dispatch", "moe_route",
    "moe_ffn_gate_up_fwd_gather",
    "moe_grouped_ffn", "moe_ffn_gate_up_fwd", "moe_ffn_down_fwd", "moe_combine",
    "moe_combine_bwd", "moe_grouped_ffn_bwd", "moe_ffn_down_bwd_data", "moe_ffn_down_bwd_weight",
    "moe_ffn_gate_up_bwd_data", "moe_ffn_gate_up_bwd_weight", "moe_dispatch_bwd",
    "moe_quant_rows_fp8", "moe_quantize_weights_fp8", "moe_ffn_gate_up_fwd_fp8",
    "moe_ffn_down_fwd_fp8", "moe_ffn_down_bwd_data_fp8", "moe_ffn_gate_up_bwd_data_fp8",
    "moe_router", "moe_router_bwd", "moe_quant_cols_fp8", "moe_ffn_down_bwd_weight_fp8",
    "moe_ffn_gate_up_bwd_weight_fp8", "moe_ffn_down_bwd_data_fp8_quant", "moe_ffn_gate_up_fwd_fp8_quant",
    "moe_dispatch_int8", "moe_quant_rows_int8", "moe_ffn_gate_up_fwd_int8", "moe_ffn_down_fwd_int8",
    "moe_quant_rows_mx", "moe_quantize_weights_mx", "moe_ffn_gate_up_fwd_mx", "moe_ffn_down_fwd_mx",
    "moe_ffn_down_bwd_data_mx", "moe_ffn_gate_up_bwd_data_mx", "moe_dispatch_noalloc",
    "moe_hbm_stream",
    "moe_ffn_gate_up_bwd_weight_gather", "moe_dispatch_fp8", "moe_combine_bwd_fp8",
    "moe_ffn_fp8_workspace_size", "moe_grouped_ffn_fp8", "moe_grouped_ffn_bwd_fp8",
    "moe_decode_fused_workspace_size", "moe_decode_fused",
    "moe_combine_bwd_weights", "moe_ffn_down_bwd_data_gather", "moe_ffn_down_bwd_weight_gather",
)


class MoeShape(ctypes.Structure):
    """Mirror of struct moe_shape."""
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("F", ctypes.c_int64),
                ("capacity", ctypes.c_int64), ("K", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("zero_expert_num", ctypes.c_int32),
                ("copy_expert_num", ctypes.c_int32), ("const_expert_num", ctypes.c_int32),
                ("mask_ndim", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("comm_quant_mode", ctypes.c_int32)]


def make_shape(T, H, K, num_experts, F=0, capacity=None, zero_expert_num=0, copy_expert_num=0,
               const_expert_num=0, mask_ndim=0, comm_quant_mode=0) -> MoeShape:
    if capacity is None:
        capacity = T * min(num_experts, K)
    return MoeShape(T, H, F, capacity, K, num_experts, zero_expert_num, copy_expert_num,
                    const_expert_num, mask_ndim, 0, comm_quant_mode)


class MoeFp8Weight(ctypes.Structure):
    """Mirror of struct moe_fp8_weight (device pointers)."""
    _fields_ = [("codes", ctypes.c_void_p), ("codes_t", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MoeError(RuntimeError):
    pass


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by dispatch_expert_gemm_amd.build) once."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: run `python -m dispatch_expert_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64P, S = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(MoeShape)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int32]
        L.moe_assist_info_size.argtypes = [S, I64P]
        L.moe_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_dispatch.argtypes = [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_dispatch_noalloc.argtypes = [S] + [P] * 9
        L.moe_dispatch_fp8.argtypes = [S] + [P] * 11 + [ctypes.c_size_t, P]
        L.moe_hbm_stream.argtypes = [ctypes.c_int32, P, P, ctypes.c_int64, P, P]
        L.moe_grouped_ffn.argtypes = [S, P, P, P, P, P, P, P, P, P]
        L.moe_ffn_gate_up_fwd.argtypes = [S, P, P, P, P, P, P, P]
        L.moe_route.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_ffn_gate_up_fwd_gather.argtypes = [S] + [P] * 8
        L.moe_ffn_down_fwd.argtypes = [S, P, P, P, P, P]
        L.moe_combine.argtypes = [S] + [P] * 13
        L.moe_combine_bwd.argtypes = [S] + [P] * 14
        L.moe_combine_bwd_fp8.argtypes = [S] + [P] * 16
        W8 = ctypes.POINTER(MoeFp8Weight)
        L.moe_ffn_fp8_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_grouped_ffn_fp8.argtypes = [S, P, P, W8, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_grouped_ffn_bwd_fp8.argtypes = [S, P, P, P, P, P, P, W8, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_decode_fused_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_decode_fused.argtypes = [S] + [P] * 15 + [ctypes.c_size_t, P]
        L.moe_grouped_ffn_bwd.argtypes = [S] + [P] * 14
        L.moe_ffn_down_bwd_data.argtypes = [S, P, P, P, P, P, P]
        L.moe_ffn_down_bwd_weight.argtypes = [S, P, P, P, P, P]
        L.moe_ffn_gate_up_bwd_data.argtypes = [S, P, P, P, P, P, P]
        L.moe_ffn_gate_up_bwd_weight.argtypes = [S, P, P, P, P, P, P]
        L.moe_ffn_gate_up_bwd_weight_gather.argtypes = [S] + [P] * 7
        L.moe_combine_bwd_weights.argtypes = [S] + [P] * 14
        L.moe_ffn_down_bwd_data_gather.argtypes = [S] + [P] * 8
        L.moe_ffn_down_bwd_weight_gather.argtypes = [S] + [P] * 7
        L.moe_dispatch_bwd.argtypes = [S] + [P] * 10
        I64 = ctypes.c_int64
        L.moe_quant_rows_fp8.argtypes = [I64, I64, P, P, P, P, P]
        L.moe_quantize_weights_fp8.argtypes = [I64, I64, I64, P, P, P, P, P]
        L.moe_ffn_gate_up_fwd_fp8.argtypes = [S] + [P] * 10
        L.moe_ffn_down_fwd_fp8.argtypes = [S] + [P] * 7
        L.moe_ffn_down_bwd_data_fp8.argtypes = [S] + [P] * 8
        L.moe_ffn_gate_up_bwd_data_fp8.argtypes = [S] + [P] * 9
        I32C = ctypes.c_int32
        L.moe_router.argtypes = [I64, I64, I32C, I32C, P, P, P, P]
        L.moe_router_bwd.argtypes = [I64, I64, I32C, I32C, P, P, P, P, P, P]
        L.moe_quant_cols_fp8.argtypes = [I64, I64, I32C, P, P, P, P, P]
        L.moe_ffn_down_bwd_weight_fp8.argtypes = [S] + [P] * 7
        L.moe_ffn_gate_up_bwd_weight_fp8.argtypes = [S] + [P] * 8
        L.moe_ffn_down_bwd_data_fp8_quant.argtypes = [S] + [P] * 12
        L.moe_ffn_gate_up_fwd_fp8_quant.argtypes = [S] + [P] * 12
        L.moe_dispatch_int8.argtypes = [S] + [P] * 11 + [ctypes.c_size_t, P]
        L.moe_quant_rows_int8.argtypes = [I64, I64, P, P, P, P, P]
        L.moe_ffn_gate_up_fwd_int8.argtypes = [S] + [P] * 10
        L.moe_ffn_down_fwd_int8.argtypes = [S] + [P] * 7
        L.moe_quant_rows_mx.argtypes = [I64, I64, P, P, P, P, P]
        L.moe_quantize_weights_mx.argtypes = [I64, I64, I64, P, P, P, P, P, P]
        L.moe_ffn_gate_up_fwd_mx.argtypes = [S] + [P] * 12
        L.moe_ffn_down_fwd_mx.argtypes = [S] + [P] * 7
        L.moe_ffn_down_bwd_data_mx.argtypes = [S] + [P] * 10
        L.moe_ffn_gate_up_bwd_data_mx.argtypes = [S] + [P] * 9
        for name in ENTRY_POINTS:
            if name != "moe_status_str":
                getattr(L, name).restype = ctypes.c_int32
        _lib_handle = L
    return _lib_handle


def _check(st: int):
    if st != 0:
        raise MoeError(f"libmoe status {st}: {lib().moe_status_str(st).decode()}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, n, name):
    """Raise unless t (when given) holds at least n elements."""
    if isinstance(t, torch.Tensor) and t.numel() < n:
        raise MoeError(f"{name} holds {t.numel()} elements, needs at least {n}")


def _shape_sizes(shape):
    """Least element count of each buffer the shape-taking entries name, from the
    layouts the C header states (a kernel would read or write that far)."""
    T, H, F, cap, K, E = shape.T, shape.H, shape.F, shape.capacity, shape.K, shape.num_experts
    Q = shape.const_expert_num
    return {
        "x": T * H, "topk_idx": T * K, "topk_weights": T * K, "grad_topk_weights": T * K,
        "x_active_mask": {1: T, 2: T * K}.get(shape.mask_ndim, 0),
        "expand_x": cap * H, "grad_expand_x": cap * H, "y": cap * H, "grad_y": cap * H,
        "gate_up_save": cap * 2 * F, "grad_gate_up": cap * 2 * F, "h_act": cap * F,
        "xq": cap * H, "dyq": cap * H, "hq": cap * F, "dguq": cap * 2 * F,
        "w_gate": E * F * H, "w_up": E * F * H, "w_down": E * H * F,
        "grad_w_gate": E * F * H, "grad_w_up": E * F * H, "grad_w_down": E * H * F,
        "ep_recv_counts": E, "ep_send_counts": E, "expert_token_nums": E, "err_flag": 1,
        "assist_info_for_combine": T * K + cap,
        "out": T * H, "grad_out": T * H, "shared_expert_x": T * H, "ori_x": T * H,
        "grad_x": T * H, "grad_x_accum": T * H,
        "const_alpha_1": Q * H, "const_alpha_2": Q * H, "const_v": Q * H,
        # 8-bit weight codes, one byte each, either layout
        "wgq": E * F * H, "wuq": E * F * H, "wdq": E * H * F,
        "wgq_t": E * F * H, "wuq_t": E * F * H, "wdq_t": E * H * F,
    }


def _check_sizes(shape, args):
    for name, n in _shape_sizes(shape).items():
        _need(args.get(name), n, name)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


BF16, I32, F32, U8 = torch.bfloat16, torch.int32, torch.float32, (torch.uint8, torch.bool)

# ----------------------------------------------------------------------------- C entries


def moe_assist_info_size(shape: MoeShape) -> int:
    n = ctypes.c_int64()
    _check(lib().moe_assist_info_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_dispatch(shape, x, topk_idx, x_active_mask, expand_x, assist_info_for_combine,
                 expert_token_nums, ep_recv_counts, err_flag, workspace, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_dispatch(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(expert_token_nums, I32, "expert_token_nums"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(err_flag, I32, "err_flag"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dispatch_fp8(shape, x, topk_idx, x_active_mask, expand_x, expand_xq, dynamic_scales,
                     assist_info_for_combine, expert_token_nums, ep_recv_counts, err_flag, workspace, stream=None):
    _check_sizes(shape, locals())
    _need(expand_xq, shape.capacity * shape.H, "expand_xq")
    _need(dynamic_scales, shape.capacity * (shape.H // 128), "dynamic_scales")
    _check(lib().moe_dispatch_fp8(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(expand_xq, U8T, "expand_xq"), _ptr(dynamic_scales, F32, "dynamic_scales"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(expert_token_nums, I32, "expert_token_nums"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(err_flag, I32, "err_flag"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dispatch_noalloc(shape, x, topk_idx, x_active_mask, expand_x, assist_info_for_combine,
                         expert_token_nums, ep_recv_counts, err_flag, stream=None):
    """moe_dispatch without a workspace argument: the library's own fixed device
    scratch holds the routing histograms, so the call allocates nothing.  Calls
    that overlap on one GPU share that scratch and race."""
    _check_sizes(shape, locals())
    _check(lib().moe_dispatch_noalloc(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(expert_token_nums, I32, "expert_token_nums"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(err_flag, I32, "err_flag"), _stream(stream)))


STREAM_SINK_BYTES = 4096 * 256 * 16


def moe_hbm_stream(mode, src, dst, nbytes, sink=None, stream=None):
    """The reference streaming kernel: mode 0 copies nbytes from src to dst, 1 reads
    src (sink: STREAM_SINK_BYTES of device memory), 2 writes dst."""
    for t, name in ((src, "src"), (dst, "dst"), (sink, "sink")):
        if t is not None and t.numel() * t.element_size() < (STREAM_SINK_BYTES if name == "sink" else nbytes):
            raise MoeError(f"{name} is smaller than the bytes it must hold")
    _check(lib().moe_hbm_stream(int(mode), _ptr(src, None, "src"), _ptr(dst, None, "dst"), int(nbytes),
                                _ptr(sink, None, "sink"), _stream(stream)))


def moe_route(shape, topk_idx, x_active_mask, assist_info_for_combine, expert_token_nums, ep_recv_counts,
              err_flag, workspace, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_route(
        ctypes.byref(shape), _ptr(topk_idx, I32, "topk_idx"), _ptr(x_active_mask, U8, "x_active_mask"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(expert_token_nums, I32, "expert_token_nums"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(err_flag, I32, "err_flag"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_ffn_gate_up_fwd_gather(shape, x, assist_info_for_combine, w_gate, w_up, ep_recv_counts, gate_up_save,
                               h_act, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_fwd_gather(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(w_gate, BF16, "w_gate"), _ptr(w_up, BF16, "w_up"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(h_act, BF16, "h_act"), _stream(stream)))


def moe_grouped_ffn(shape, expand_x, w_gate, w_up, w_down, ep_recv_counts, gate_up_save, h_act, y,
                    stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_grouped_ffn(
        ctypes.byref(shape), _ptr(expand_x, BF16, "expand_x"), _ptr(w_gate, BF16, "w_gate"),
        _ptr(w_up, BF16, "w_up"), _ptr(w_down, BF16, "w_down"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(h_act, BF16, "h_act"), _ptr(y, BF16, "y"),
        _stream(stream)))


def moe_ffn_gate_up_fwd(shape, expand_x, w_gate, w_up, ep_recv_counts, gate_up_save, h_act, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_fwd(
        ctypes.byref(shape), _ptr(expand_x, BF16, "expand_x"), _ptr(w_gate, BF16, "w_gate"),
        _ptr(w_up, BF16, "w_up"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(h_act, BF16, "h_act"), _stream(stream)))


def moe_ffn_down_fwd(shape, h_act, w_down, ep_recv_counts, y, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_fwd(
        ctypes.byref(shape), _ptr(h_act, BF16, "h_act"), _ptr(w_down, BF16, "w_down"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(y, BF16, "y"), _stream(stream)))


def moe_combine(shape, y, topk_idx, topk_weights, assist_info_for_combine, ep_send_counts,
                x_active_mask, shared_expert_x, ori_x, const_alpha_1, const_alpha_2, const_v, out,
                stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_combine(
        ctypes.byref(shape), _ptr(y, BF16, "y"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(topk_weights, F32, "topk_weights"), _ptr(assist_info_for_combine, I32, "assist"),
        _ptr(ep_send_counts, I32, "ep_send_counts"), _ptr(x_active_mask, U8, "x_active_mask"),
        _ptr(shared_expert_x, BF16, "shared_expert_x"), _ptr(ori_x, BF16, "ori_x"),
        _ptr(const_alpha_1, BF16, "const_alpha_1"), _ptr(const_alpha_2, BF16, "const_alpha_2"),
        _ptr(const_v, BF16, "const_v"), _ptr(out, BF16, "out"), _stream(stream)))


def moe_decode_fused_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_decode_fused_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def decode_fused_workspace(shape: MoeShape, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for moe_decode_fused (zero before its first use;
    each call leaves its control words zero again)."""
    return torch.zeros(moe_decode_fused_workspace_size(shape), dtype=torch.uint8, device=device)


def moe_decode_fused(shape, x, topk_idx, topk_weights, x_active_mask, w_gate, w_up, w_down, shared_expert_x,
                     ori_x, const_alpha_1, const_alpha_2, const_v, out, err_flag, workspace, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_decode_fused(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(topk_weights, F32, "topk_weights"), _ptr(x_active_mask, U8, "x_active_mask"),
        _ptr(w_gate, BF16, "w_gate"), _ptr(w_up, BF16, "w_up"), _ptr(w_down, BF16, "w_down"),
        _ptr(shared_expert_x, BF16, "shared_expert_x"), _ptr(ori_x, BF16, "ori_x"),
        _ptr(const_alpha_1, BF16, "const_alpha_1"), _ptr(const_alpha_2, BF16, "const_alpha_2"),
        _ptr(const_v, BF16, "const_v"), _ptr(out, BF16, "out"), _ptr(err_flag, I32, "err_flag"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_combine_bwd(shape, grad_out, y, topk_idx, topk_weights, assist_info_for_combine,
                    ep_send_counts, x_active_mask, ori_x, const_alpha_1, const_alpha_2, const_v,
                    grad_y, grad_topk_weights, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_combine_bwd(
        ctypes.byref(shape), _ptr(grad_out, BF16, "grad_out"), _ptr(y, BF16, "y"),
        _ptr(topk_idx, I32, "topk_idx"), _ptr(topk_weights, F32, "topk_weights"),
        _ptr(assist_info_for_combine, I32, "assist"), _ptr(ep_send_counts, I32, "ep_send_counts"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(ori_x, BF16, "ori_x"),
        _ptr(const_alpha_1, BF16, "const_alpha_1"), _ptr(const_alpha_2, BF16, "const_alpha_2"),
        _ptr(const_v, BF16, "const_v"), _ptr(grad_y, BF16, "grad_y"),
        _ptr(grad_topk_weights, F32, "grad_topk_weights"), _stream(stream)))


def fold_combine_bwd(F: int) -> bool:
    """Whether the bf16 backward folds the combine backward into the down GEMMs
    (moe_combine_bwd_weights + the *_gather down GEMMs) rather than writing grad_y
    rows: for a narrow expert FFN.  Measured on MI355X: 3% faster steps at F = 480
    (H = 1536), 1.3% slower at F = 2048 (H = 7168), where the down weight
    gradient's scaling of every operand element costs more than grad_y's bytes."""
    return F < 1024


def moe_combine_bwd_weights(shape, grad_out, y, topk_idx, topk_weights, assist_info_for_combine,
                            ep_send_counts, x_active_mask, ori_x, const_alpha_1, const_alpha_2, const_v,
                            grad_topk_weights, row_weights, stream=None):
    _check_sizes(shape, locals())
    _need(row_weights, shape.capacity, "row_weights")
    _check(lib().moe_combine_bwd_weights(
        ctypes.byref(shape), _ptr(grad_out, BF16, "grad_out"), _ptr(y, BF16, "y"),
        _ptr(topk_idx, I32, "topk_idx"), _ptr(topk_weights, F32, "topk_weights"),
        _ptr(assist_info_for_combine, I32, "assist"), _ptr(ep_send_counts, I32, "ep_send_counts"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(ori_x, BF16, "ori_x"),
        _ptr(const_alpha_1, BF16, "const_alpha_1"), _ptr(const_alpha_2, BF16, "const_alpha_2"),
        _ptr(const_v, BF16, "const_v"), _ptr(grad_topk_weights, F32, "grad_topk_weights"),
        _ptr(row_weights, F32, "row_weights"), _stream(stream)))


def moe_ffn_down_bwd_data_gather(shape, grad_out, assist_info_for_combine, row_weights, w_down, gate_up_save,
                                 ep_recv_counts, grad_gate_up, stream=None):
    _check_sizes(shape, locals())
    _need(row_weights, shape.capacity, "row_weights")
    _check(lib().moe_ffn_down_bwd_data_gather(
        ctypes.byref(shape), _ptr(grad_out, BF16, "grad_out"), _ptr(assist_info_for_combine, I32, "assist"),
        _ptr(row_weights, F32, "row_weights"), _ptr(w_down, BF16, "w_down"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_gate_up, BF16, "grad_gate_up"), _stream(stream)))


def moe_ffn_down_bwd_weight_gather(shape, grad_out, assist_info_for_combine, row_weights, h_act, ep_recv_counts,
                                   grad_w_down, stream=None):
    _check_sizes(shape, locals())
    _need(row_weights, shape.capacity, "row_weights")
    _check(lib().moe_ffn_down_bwd_weight_gather(
        ctypes.byref(shape), _ptr(grad_out, BF16, "grad_out"), _ptr(assist_info_for_combine, I32, "assist"),
        _ptr(row_weights, F32, "row_weights"), _ptr(h_act, BF16, "h_act"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_w_down, F32, "grad_w_down"), _stream(stream)))


def moe_combine_bwd_fp8(shape, grad_out, y, topk_idx, topk_weights, assist_info_for_combine, ep_send_counts,
                        x_active_mask, ori_x, const_alpha_1, const_alpha_2, const_v, grad_y, grad_yq, grad_y_scales,
                        grad_topk_weights, stream=None):
    _check_sizes(shape, locals())
    _need(grad_yq, shape.capacity * shape.H, "grad_yq")
    _need(grad_y_scales, shape.capacity * (shape.H // 128), "grad_y_scales")
    _check(lib().moe_combine_bwd_fp8(
        ctypes.byref(shape), _ptr(grad_out, BF16, "grad_out"), _ptr(y, BF16, "y"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(topk_weights, F32, "topk_weights"), _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(ep_send_counts, I32, "ep_send_counts"), _ptr(x_active_mask, U8, "x_active_mask"),
        _ptr(ori_x, BF16, "ori_x"), _ptr(const_alpha_1, BF16, "const_alpha_1"),
        _ptr(const_alpha_2, BF16, "const_alpha_2"), _ptr(const_v, BF16, "const_v"), _ptr(grad_y, BF16, "grad_y"),
        _ptr(grad_yq, U8T, "grad_yq"), _ptr(grad_y_scales, F32, "grad_y_scales"),
        _ptr(grad_topk_weights, F32, "grad_topk_weights"), _stream(stream)))


def moe_ffn_fp8_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_ffn_fp8_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def _fp8_weights(wq):
    """Three Fp8Weights (gate, up, down) -> a moe_fp8_weight[3] array (kept alive by
    the caller's tensors)."""
    for q in wq:
        for t, dt in ((q.codes, U8T), (q.codes_t, U8T), (q.scales, F32T)):
            _ptr(t, dt, "fp8 weights")
    return (MoeFp8Weight * 3)(*[MoeFp8Weight(q.codes.data_ptr(), q.codes_t.data_ptr(), q.scales.data_ptr())
                                for q in wq])


def moe_grouped_ffn_fp8(shape, expand_xq, x_scales, wq, ep_recv_counts, gate_up_save, h_act, y, workspace,
                        stream=None):
    """wq: (gate, up, down) Fp8Weights of moe_quantize_weights_fp8."""
    _check_sizes(shape, locals())
    _need(expand_xq, shape.capacity * shape.H, "expand_xq")
    _need(x_scales, shape.capacity * (shape.H // 128), "x_scales")
    for q, (n, k) in zip(wq, ((shape.F, shape.H), (shape.F, shape.H), (shape.H, shape.F))):
        _need(q.codes, shape.num_experts * n * k, "weight codes")
        _need(q.scales, shape.num_experts * (n // 128) * (k // 128), "weight scales")
    w = _fp8_weights(wq)
    _check(lib().moe_grouped_ffn_fp8(
        ctypes.byref(shape), _ptr(expand_xq, U8T, "expand_xq"), _ptr(x_scales, F32, "x_scales"), w,
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(h_act, BF16, "h_act"), _ptr(y, BF16, "y"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_ffn_bwd_fp8(shape, grad_y, grad_yq, grad_y_scales, expand_x, gate_up_save, h_act, wq,
                            ep_recv_counts, grad_gate_up, grad_expand_x, grad_w_gate, grad_w_up, grad_w_down,
                            workspace, stream=None):
    _check_sizes(shape, locals())
    _need(grad_yq, shape.capacity * shape.H, "grad_yq")
    _need(grad_y_scales, shape.capacity * (shape.H // 128), "grad_y_scales")
    for q, (n, k) in zip(wq, ((shape.F, shape.H), (shape.F, shape.H), (shape.H, shape.F))):
        _need(q.codes_t, shape.num_experts * n * k, "weight codes")
        _need(q.scales, shape.num_experts * (n // 128) * (k // 128), "weight scales")
    w = _fp8_weights(wq)
    _check(lib().moe_grouped_ffn_bwd_fp8(
        ctypes.byref(shape), _ptr(grad_y, BF16, "grad_y"), _ptr(grad_yq, U8T, "grad_yq"),
        _ptr(grad_y_scales, F32, "grad_y_scales"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(h_act, BF16, "h_act"), w,
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_gate_up, BF16, "grad_gate_up"),
        _ptr(grad_expand_x, BF16, "grad_expand_x"), _ptr(grad_w_gate, F32, "grad_w_gate"),
        _ptr(grad_w_up, F32, "grad_w_up"), _ptr(grad_w_down, F32, "grad_w_down"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grouped_ffn_bwd(shape, grad_y, expand_x, gate_up_save, h_act, w_gate, w_up, w_down,
                        ep_recv_counts, grad_gate_up, grad_expand_x, grad_w_gate, grad_w_up,
                        grad_w_down, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_grouped_ffn_bwd(
        ctypes.byref(shape), _ptr(grad_y, BF16, "grad_y"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(h_act, BF16, "h_act"),
        _ptr(w_gate, BF16, "w_gate"), _ptr(w_up, BF16, "w_up"), _ptr(w_down, BF16, "w_down"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_gate_up, BF16, "grad_gate_up"),
        _ptr(grad_expand_x, BF16, "grad_expand_x"), _ptr(grad_w_gate, F32, "grad_w_gate"),
        _ptr(grad_w_up, F32, "grad_w_up"), _ptr(grad_w_down, F32, "grad_w_down"), _stream(stream)))


def moe_ffn_down_bwd_data(shape, grad_y, w_down, gate_up_save, ep_recv_counts, grad_gate_up,
                          stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_bwd_data(
        ctypes.byref(shape), _ptr(grad_y, BF16, "grad_y"), _ptr(w_down, BF16, "w_down"),
        _ptr(gate_up_save, BF16, "gate_up_save"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_gate_up, BF16, "grad_gate_up"), _stream(stream)))


def moe_ffn_down_bwd_weight(shape, grad_y, h_act, ep_recv_counts, grad_w_down, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_bwd_weight(
        ctypes.byref(shape), _ptr(grad_y, BF16, "grad_y"), _ptr(h_act, BF16, "h_act"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_w_down, F32, "grad_w_down"),
        _stream(stream)))


def moe_ffn_gate_up_bwd_data(shape, grad_gate_up, w_gate, w_up, ep_recv_counts, grad_expand_x,
                             stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_data(
        ctypes.byref(shape), _ptr(grad_gate_up, BF16, "grad_gate_up"), _ptr(w_gate, BF16, "w_gate"),
        _ptr(w_up, BF16, "w_up"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_expand_x, BF16, "grad_expand_x"), _stream(stream)))


def moe_ffn_gate_up_bwd_weight(shape, grad_gate_up, expand_x, ep_recv_counts, grad_w_gate,
                               grad_w_up, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_weight(
        ctypes.byref(shape), _ptr(grad_gate_up, BF16, "grad_gate_up"), _ptr(expand_x, BF16, "expand_x"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_w_gate, F32, "grad_w_gate"),
        _ptr(grad_w_up, F32, "grad_w_up"), _stream(stream)))


def moe_ffn_gate_up_bwd_weight_gather(shape, grad_gate_up, x, assist_info_for_combine, ep_recv_counts, grad_w_gate,
                                      grad_w_up, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_weight_gather(
        ctypes.byref(shape), _ptr(grad_gate_up, BF16, "grad_gate_up"), _ptr(x, BF16, "x"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_w_gate, F32, "grad_w_gate"), _ptr(grad_w_up, F32, "grad_w_up"), _stream(stream)))


def moe_dispatch_bwd(shape, grad_expand_x, assist_info_for_combine, topk_idx, topk_weights,
                     x_active_mask, grad_out, const_alpha_1, grad_x_accum, grad_x, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_dispatch_bwd(
        ctypes.byref(shape), _ptr(grad_expand_x, BF16, "grad_expand_x"),
        _ptr(assist_info_for_combine, I32, "assist"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(topk_weights, F32, "topk_weights"), _ptr(x_active_mask, U8, "x_active_mask"),
        _ptr(grad_out, BF16, "grad_out"), _ptr(const_alpha_1, BF16, "const_alpha_1"),
        _ptr(grad_x_accum, BF16, "grad_x_accum"), _ptr(grad_x, BF16, "grad_x"), _stream(stream)))


U8T, F32T = torch.uint8, torch.float32


def moe_quant_rows_fp8(src, codes, scales, nrows=None, stream=None):
    R, C = src.shape
    _need(codes, R * C, "codes")
    _need(scales, R * (C // 128), "scales")
    _check(lib().moe_quant_rows_fp8(R, C, _ptr(src, BF16, "src"), _ptr(nrows, I32, "nrows"),
                                    _ptr(codes, U8T, "codes"), _ptr(scales, F32T, "scales"),
                                    _stream(stream)))


def moe_quantize_weights_fp8(w, codes, codes_t, scales, stream=None):
    E, N, K = w.shape
    for t, nm in ((codes, "codes"), (codes_t, "codes_t")):
        _need(t, E * N * K, nm)
    _check(lib().moe_quantize_weights_fp8(E, N, K, _ptr(w, BF16, "w"), _ptr(codes, U8T, "codes"),
                                          _ptr(codes_t, U8T, "codes_t"), _ptr(scales, F32T, "scales"),
                                          _stream(stream)))


def moe_ffn_gate_up_fwd_fp8(shape, xq, xs, wgq, wgs, wuq, wus, ep_recv_counts, gate_up_save, h_act,
                            stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_fwd_fp8(
        ctypes.byref(shape), _ptr(xq, U8T, "xq"), _ptr(xs, F32T, "xs"), _ptr(wgq, U8T, "wgq"),
        _ptr(wgs, F32T, "wgs"), _ptr(wuq, U8T, "wuq"), _ptr(wus, F32T, "wus"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(h_act, BF16, "h_act"), _stream(stream)))


def moe_ffn_gate_up_fwd_fp8_quant(shape, xq, xs, wgq, wgs, wuq, wus, ep_recv_counts, gate_up_save, h_act,
                                  hq_t, hs_t, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_fwd_fp8_quant(
        ctypes.byref(shape), _ptr(xq, U8T, "xq"), _ptr(xs, F32T, "xs"), _ptr(wgq, U8T, "wgq"),
        _ptr(wgs, F32T, "wgs"), _ptr(wuq, U8T, "wuq"), _ptr(wus, F32T, "wus"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(h_act, BF16, "h_act"), _ptr(hq_t, U8T, "hq_t"), _ptr(hs_t, F32T, "hs_t"), _stream(stream)))


def moe_ffn_down_fwd_fp8(shape, hq, hs, wdq, wds, ep_recv_counts, y, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_fwd_fp8(
        ctypes.byref(shape), _ptr(hq, U8T, "hq"), _ptr(hs, F32T, "hs"), _ptr(wdq, U8T, "wdq"),
        _ptr(wds, F32T, "wds"), _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(y, BF16, "y"),
        _stream(stream)))


def moe_ffn_down_bwd_data_fp8(shape, dyq, dys, wdq_t, wds, gate_up_save, ep_recv_counts, grad_gate_up,
                              stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_bwd_data_fp8(
        ctypes.byref(shape), _ptr(dyq, U8T, "dyq"), _ptr(dys, F32T, "dys"), _ptr(wdq_t, U8T, "wdq_t"),
        _ptr(wds, F32T, "wds"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_gate_up, BF16, "grad_gate_up"),
        _stream(stream)))


def moe_ffn_down_bwd_data_fp8_quant(shape, dyq, dys, wdq_t, wds, gate_up_save, ep_recv_counts,
                                    grad_gate_up=None, rows=None, cols=None, stream=None):
    """moe_ffn_down_bwd_data_fp8 writing any of: bf16 grad_gate_up, rows = (codes,
    scales) of moe_quant_rows_fp8 layout, cols = (codes_t, scales) of
    moe_quant_cols_fp8 layout."""
    _check_sizes(shape, locals())
    dguq, dgus = rows if rows is not None else (None, None)
    dguq_t, dgus_t = cols if cols is not None else (None, None)
    _check(lib().moe_ffn_down_bwd_data_fp8_quant(
        ctypes.byref(shape), _ptr(dyq, U8T, "dyq"), _ptr(dys, F32T, "dys"), _ptr(wdq_t, U8T, "wdq_t"),
        _ptr(wds, F32T, "wds"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_gate_up, BF16, "grad_gate_up"),
        _ptr(dguq, U8T, "dguq"), _ptr(dgus, F32T, "dgus"), _ptr(dguq_t, U8T, "dguq_t"),
        _ptr(dgus_t, F32T, "dgus_t"), _stream(stream)))


def moe_ffn_gate_up_bwd_data_fp8(shape, dguq, dgus, wgq_t, wgs, wuq_t, wus, ep_recv_counts,
                                 grad_expand_x, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_data_fp8(
        ctypes.byref(shape), _ptr(dguq, U8T, "dguq"), _ptr(dgus, F32T, "dgus"),
        _ptr(wgq_t, U8T, "wgq_t"), _ptr(wgs, F32T, "wgs"), _ptr(wuq_t, U8T, "wuq_t"),
        _ptr(wus, F32T, "wus"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_expand_x, BF16, "grad_expand_x"), _stream(stream)))


def cols_fp8_slots(capacity, num_experts):
    """Token slots of the per-128-token fp8 layout: capacity/128 + num_experts."""
    return capacity // 128 + num_experts


def moe_quant_cols_fp8(src, ep_recv_counts, codes_t, scales, stream=None):
    cap, D = src.shape
    _check(lib().moe_quant_cols_fp8(cap, D, ep_recv_counts.numel(), _ptr(src, BF16, "src"),
                                    _ptr(ep_recv_counts, I32, "ep_recv_counts"),
                                    _ptr(codes_t, U8T, "codes_t"), _ptr(scales, F32T, "scales"),
                                    _stream(stream)))


def moe_ffn_down_bwd_weight_fp8(shape, dyq_t, dys, hq_t, hs, ep_recv_counts, grad_w_down, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_bwd_weight_fp8(
        ctypes.byref(shape), _ptr(dyq_t, U8T, "dyq_t"), _ptr(dys, F32T, "dys"), _ptr(hq_t, U8T, "hq_t"),
        _ptr(hs, F32T, "hs"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_w_down, F32T, "grad_w_down"), _stream(stream)))


def moe_ffn_gate_up_bwd_weight_fp8(shape, dguq_t, dgus, xq_t, xs, ep_recv_counts, grad_w_gate, grad_w_up,
                                   stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_weight_fp8(
        ctypes.byref(shape), _ptr(dguq_t, U8T, "dguq_t"), _ptr(dgus, F32T, "dgus"),
        _ptr(xq_t, U8T, "xq_t"), _ptr(xs, F32T, "xs"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(grad_w_gate, F32T, "grad_w_gate"), _ptr(grad_w_up, F32T, "grad_w_up"), _stream(stream)))


I8T = torch.int8


def moe_dispatch_int8(shape, x, topk_idx, x_active_mask, smooth_scales, expand_x, dynamic_scales,
                      assist_info_for_combine, expert_token_nums, ep_recv_counts, err_flag, workspace,
                      stream=None):
    _check_sizes(shape, locals())
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moe_dispatch_int8(
        ctypes.byref(shape), _ptr(x, BF16, "x"), _ptr(topk_idx, I32, "topk_idx"),
        _ptr(x_active_mask, U8, "x_active_mask"), _ptr(smooth_scales, F32, "smooth_scales"),
        _ptr(expand_x, I8T, "expand_x"), _ptr(dynamic_scales, F32, "dynamic_scales"),
        _ptr(assist_info_for_combine, I32, "assist_info_for_combine"),
        _ptr(expert_token_nums, I32, "expert_token_nums"), _ptr(ep_recv_counts, I32, "ep_recv_counts"),
        _ptr(err_flag, I32, "err_flag"), _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream)))


def moe_quant_rows_int8(src, codes, scales, nrows=None, stream=None):
    C = src.shape[-1]
    R = src.numel() // C
    _need(codes, R * C, "codes")
    _need(scales, R, "scales")
    _check(lib().moe_quant_rows_int8(R, C, _ptr(src, BF16, "src"), _ptr(nrows, I32, "nrows"),
                                     _ptr(codes, I8T, "codes"), _ptr(scales, F32, "scales"), _stream(stream)))


def moe_ffn_gate_up_fwd_int8(shape, xq, xs, wgq, wgs, wuq, wus, ep_recv_counts, gate_up_save, h_act,
                             stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_fwd_int8(
        ctypes.byref(shape), _ptr(xq, I8T, "xq"), _ptr(xs, F32, "xs"), _ptr(wgq, I8T, "wgq"),
        _ptr(wgs, F32, "wgs"), _ptr(wuq, I8T, "wuq"), _ptr(wus, F32, "wus"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(h_act, BF16, "h_act"), _stream(stream)))


def moe_ffn_down_fwd_int8(shape, hq, hs, wdq, wds, ep_recv_counts, y, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_fwd_int8(
        ctypes.byref(shape), _ptr(hq, I8T, "hq"), _ptr(hs, F32, "hs"), _ptr(wdq, I8T, "wdq"),
        _ptr(wds, F32, "wds"), _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(y, BF16, "y"),
        _stream(stream)))


def quant_rows_int8(src, nrows=None, stream=None):
    """Per-row int8 codes (same shape as src) and scales (src.shape[:-1]) of a bf16 tensor;
    (E, N, K) weights give one scale per output channel."""
    codes = torch.empty(src.shape, dtype=I8T, device=src.device)
    scales = torch.empty(src.shape[:-1], dtype=F32, device=src.device)
    moe_quant_rows_int8(src, codes, scales, nrows, stream)
    return codes, scales


def moe_quant_rows_mx(src, codes, scales, nrows=None, stream=None):
    R, C = src.shape
    _need(codes, R * C, "codes")
    _need(scales, R * (C // 32), "scales")
    _check(lib().moe_quant_rows_mx(R, C, _ptr(src, BF16, "src"), _ptr(nrows, I32, "nrows"),
                                   _ptr(codes, U8T, "codes"), _ptr(scales, U8T, "scales"), _stream(stream)))


def moe_quantize_weights_mx(w, codes, scales, codes_t=None, scales_t=None, stream=None):
    E, N, K = w.shape
    for t, nm, n in ((codes, "codes", E * N * K), (codes_t, "codes_t", E * N * K),
                     (scales, "scales", E * N * K // 32), (scales_t, "scales_t", E * N * K // 32)):
        _need(t, n, nm)
    _check(lib().moe_quantize_weights_mx(E, N, K, _ptr(w, BF16, "w"), _ptr(codes, U8T, "codes"),
                                         _ptr(scales, U8T, "scales"), _ptr(codes_t, U8T, "codes_t"),
                                         _ptr(scales_t, U8T, "scales_t"), _stream(stream)))


def moe_ffn_gate_up_fwd_mx(shape, xq, xs, wgq, wgs, wuq, wus, ep_recv_counts, gate_up_save, h_act, h_rows=None,
                           stream=None):
    """h_rows: optional (codes, scales) receiving the MX row codes of h_act."""
    _check_sizes(shape, locals())
    hq, hs = h_rows if h_rows is not None else (None, None)
    _check(lib().moe_ffn_gate_up_fwd_mx(
        ctypes.byref(shape), _ptr(xq, U8T, "xq"), _ptr(xs, U8T, "xs"), _ptr(wgq, U8T, "wgq"),
        _ptr(wgs, U8T, "wgs"), _ptr(wuq, U8T, "wuq"), _ptr(wus, U8T, "wus"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(h_act, BF16, "h_act"), _ptr(hq, U8T, "hq"), _ptr(hs, U8T, "hs"), _stream(stream)))


def moe_ffn_down_fwd_mx(shape, hq, hs, wdq, wds, ep_recv_counts, y, stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_down_fwd_mx(
        ctypes.byref(shape), _ptr(hq, U8T, "hq"), _ptr(hs, U8T, "hs"), _ptr(wdq, U8T, "wdq"),
        _ptr(wds, U8T, "wds"), _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(y, BF16, "y"),
        _stream(stream)))


def moe_ffn_down_bwd_data_mx(shape, dyq, dys, wdq_t, wds_t, gate_up_save, ep_recv_counts, grad_gate_up,
                             rows=None, stream=None):
    """rows: optional (codes, scales) receiving the MX row codes of dG|dU."""
    _check_sizes(shape, locals())
    dguq, dgus = rows if rows is not None else (None, None)
    _check(lib().moe_ffn_down_bwd_data_mx(
        ctypes.byref(shape), _ptr(dyq, U8T, "dyq"), _ptr(dys, U8T, "dys"), _ptr(wdq_t, U8T, "wdq_t"),
        _ptr(wds_t, U8T, "wds_t"), _ptr(gate_up_save, BF16, "gate_up_save"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_gate_up, BF16, "grad_gate_up"),
        _ptr(dguq, U8T, "dguq"), _ptr(dgus, U8T, "dgus"), _stream(stream)))


def moe_ffn_gate_up_bwd_data_mx(shape, dguq, dgus, wgq_t, wgs_t, wuq_t, wus_t, ep_recv_counts, grad_expand_x,
                                stream=None):
    _check_sizes(shape, locals())
    _check(lib().moe_ffn_gate_up_bwd_data_mx(
        ctypes.byref(shape), _ptr(dguq, U8T, "dguq"), _ptr(dgus, U8T, "dgus"), _ptr(wgq_t, U8T, "wgq_t"),
        _ptr(wgs_t, U8T, "wgs_t"), _ptr(wuq_t, U8T, "wuq_t"), _ptr(wus_t, U8T, "wus_t"),
        _ptr(ep_recv_counts, I32, "ep_recv_counts"), _ptr(grad_expand_x, BF16, "grad_expand_x"),
        _stream(stream)))


def quant_rows_mx(src, nrows=None, stream=None):
    """MX e4m3 codes (R, C) and E8M0 scale bytes (R, C/32) of a bf16 (R, C) matrix."""
    R, C = src.shape
    codes = torch.empty((R, C), dtype=U8T, device=src.device)
    scales = torch.empty((R, C // 32), dtype=U8T, device=src.device)
    moe_quant_rows_mx(src, codes, scales, nrows, stream)
    return codes, scales


def moe_router(logits, K, renorm, topk_idx, topk_weights, stream=None):
    T, n = logits.shape
    _check(lib().moe_router(T, n, int(K), int(bool(renorm)), _ptr(logits, F32, "logits"),
                            _ptr(topk_idx, I32, "topk_idx"), _ptr(topk_weights, F32, "topk_weights"),
                            _stream(stream)))


def moe_router_bwd(logits, K, renorm, topk_idx, topk_weights, grad_topk_weights, grad_logits,
                   stream=None):
    T, n = grad_logits.shape
    _check(lib().moe_router_bwd(T, n, int(K), int(bool(renorm)), _ptr(logits, F32, "logits"),
                                _ptr(topk_idx, I32, "topk_idx"), _ptr(topk_weights, F32, "topk_weights"),
                                _ptr(grad_topk_weights, F32, "grad_topk_weights"),
                                _ptr(grad_logits, F32, "grad_logits"), _stream(stream)))


class _RouterFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, K, renorm):
        logits = logits.contiguous()
        T = logits.shape[0]
        idx = torch.empty((T, K), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
        moe_router(logits, K, renorm, idx, w)
        ctx.save_for_backward(logits, idx, w)
        ctx.K, ctx.renorm = K, renorm
        ctx.mark_non_differentiable(idx)
        return idx, w

    @staticmethod
    def backward(ctx, g_idx, g_w):
        logits, idx, w = ctx.saved_tensors
        gl = torch.empty_like(logits)
        if g_w is None:
            return torch.zeros_like(logits), None, None
        moe_router_bwd(logits, ctx.K, ctx.renorm, idx, w, g_w.float().contiguous(), gl)
        return gl, None, None


def router(logits, K, renorm=True):
    """Softmax top-K gating of fp32 logits (T, n_ids) -> (topk_idx int32 (T, K),
    topk_weights fp32 (T, K)); differentiable in the logits through topk_weights."""
    if logits.dtype != torch.float32:
        raise MoeError(f"logits must be float32, got {logits.dtype}")
    return _RouterFn.apply(logits, int(K), bool(renorm))


@dataclass
class Fp8Weights:
    """e4m3 codes (and transposed codes) with 128 x 128 block scales of one weight tensor."""
    codes: torch.Tensor
    codes_t: torch.Tensor
    scales: torch.Tensor

    @staticmethod
    def quantize(w, stream=None):
        E, N, K = w.shape
        q = Fp8Weights(torch.empty((E, N, K), dtype=U8T, device=w.device),
                       torch.empty((E, K, N), dtype=U8T, device=w.device),
                       torch.empty((E, N // 128, K // 128), dtype=F32T, device=w.device))
        moe_quantize_weights_fp8(w, q.codes, q.codes_t, q.scales, stream)
        return q


@dataclass
class MxWeights:
    """MX e4m3 codes of one weight tensor (E, N, K): along K (codes, scales) for the
    forward GEMMs and, transposed, along N (codes_t, scales_t) for the data gradients."""
    codes: torch.Tensor
    scales: torch.Tensor
    codes_t: torch.Tensor
    scales_t: torch.Tensor

    @staticmethod
    def quantize(w, stream=None):
        E, N, K = w.shape
        d = w.device
        q = MxWeights(torch.empty((E, N, K), dtype=U8T, device=d), torch.empty((E, N, K // 32), dtype=U8T, device=d),
                      torch.empty((E, K, N), dtype=U8T, device=d), torch.empty((E, K, N // 32), dtype=U8T, device=d))
        moe_quantize_weights_mx(w, q.codes, q.scales, q.codes_t, q.scales_t, stream)
        return q


def quant_cols_fp8(src, ep_recv_counts, stream=None):
    """Per-128-token e4m3 codes of expert-sorted rows (capacity, D): codes_t
    (D, 128 * slots) and scales (slots, D), slots = cols_fp8_slots(capacity, E)."""
    cap, D = src.shape
    ns = cols_fp8_slots(cap, ep_recv_counts.numel())
    codes_t = torch.empty((D, 128 * ns), dtype=U8T, device=src.device)
    scales = torch.empty((ns, D), dtype=F32T, device=src.device)
    moe_quant_cols_fp8(src, ep_recv_counts, codes_t, scales, stream)
    return codes_t, scales


def quant_rows_fp8(src, nrows=None, stream=None):
    R, C = src.shape
    codes = torch.empty((R, C), dtype=U8T, device=src.device)
    scales = torch.empty((C // 128, R), dtype=F32T, device=src.device)   # column-block major
    moe_quant_rows_fp8(src, codes, scales, nrows, stream)
    return codes, scales


# ----------------------------------------------------------------------------- buffers + layer


@dataclass
class DispatchOut:
    expand_x: torch.Tensor
    assist_info_for_combine: torch.Tensor
    expert_token_nums: torch.Tensor
    ep_recv_counts: torch.Tensor
    err_flag: torch.Tensor

    def slot2row(self, T, K):
        return self.assist_info_for_combine[:T * K]

    def row2slot(self, T, K):
        return self.assist_info_for_combine[T * K:]


def dispatch(shape, x, topk_idx, x_active_mask=None, workspace=None, stream=None) -> DispatchOut:
    """Allocate the dispatch outputs with torch and run moe_dispatch."""
    dev = x.device
    d = DispatchOut(
        expand_x=torch.empty((shape.capacity, shape.H), dtype=BF16, device=dev),
        assist_info_for_combine=torch.empty(moe_assist_info_size(shape), dtype=I32, device=dev),
        expert_token_nums=torch.empty(shape.num_experts, dtype=I32, device=dev),
        ep_recv_counts=torch.empty(shape.num_experts, dtype=I32, device=dev),
        err_flag=torch.empty(1, dtype=I32, device=dev))
    if workspace is None:
        workspace = torch.empty(moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    mask = x_active_mask.view(torch.uint8) if x_active_mask is not None and x_active_mask.dtype == torch.bool \
        else x_active_mask
    moe_dispatch(shape, x, topk_idx, mask, d.expand_x, d.assist_info_for_combine,
                 d.expert_token_nums, d.ep_recv_counts, d.err_flag, workspace, stream)
    return d


def dispatch_fp8(shape, x, topk_idx, x_active_mask=None, workspace=None, bf16_rows=True, stream=None):
    """Allocate the outputs with torch and run moe_dispatch_fp8: (DispatchOut with the
    bf16 rows in expand_x (None without bf16_rows), e4m3 rows (capacity, H),
    scales (H/128, capacity))."""
    dev = x.device
    cap, H = shape.capacity, shape.H
    d = DispatchOut(
        expand_x=torch.empty((cap, H), dtype=BF16, device=dev) if bf16_rows else None,
        assist_info_for_combine=torch.empty(moe_assist_info_size(shape), dtype=I32, device=dev),
        expert_token_nums=torch.empty(shape.num_experts, dtype=I32, device=dev),
        ep_recv_counts=torch.empty(shape.num_experts, dtype=I32, device=dev),
        err_flag=torch.empty(1, dtype=I32, device=dev))
    xq = torch.empty((cap, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((H // 128, cap), dtype=F32, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    mask = x_active_mask.view(torch.uint8) if x_active_mask is not None and x_active_mask.dtype == torch.bool \
        else x_active_mask
    moe_dispatch_fp8(shape, x, topk_idx, mask, d.expand_x, xq, xs, d.assist_info_for_combine, d.expert_token_nums,
                     d.ep_recv_counts, d.err_flag, workspace, stream)
    return d, xq, xs


def route(shape, topk_idx, x_active_mask=None, workspace=None, stream=None) -> DispatchOut:
    """Allocate the routing outputs with torch and run moe_route (no expanded rows:
    expand_x is None; the gathered GEMM entries read x through the assist info)."""
    dev = topk_idx.device
    d = DispatchOut(
        expand_x=None,
        assist_info_for_combine=torch.empty(moe_assist_info_size(shape), dtype=I32, device=dev),
        expert_token_nums=torch.empty(shape.num_experts, dtype=I32, device=dev),
        ep_recv_counts=torch.empty(shape.num_experts, dtype=I32, device=dev),
        err_flag=torch.empty(1, dtype=I32, device=dev))
    if workspace is None:
        workspace = torch.empty(moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    mask = x_active_mask.view(torch.uint8) if x_active_mask is not None and x_active_mask.dtype == torch.bool \
        else x_active_mask
    moe_route(shape, topk_idx, mask, d.assist_info_for_combine, d.expert_token_nums, d.ep_recv_counts, d.err_flag,
              workspace, stream)
    return d


def dispatch_int8(shape, x, topk_idx, x_active_mask=None, smooth_scales=None, workspace=None, stream=None):
    """Allocate the outputs with torch and run moe_dispatch_int8: (DispatchOut with an
    int8 expand_x, dynamic_scales (capacity,) fp32)."""
    dev = x.device
    d = DispatchOut(
        expand_x=torch.empty((shape.capacity, shape.H), dtype=I8T, device=dev),
        assist_info_for_combine=torch.empty(moe_assist_info_size(shape), dtype=I32, device=dev),
        expert_token_nums=torch.empty(shape.num_experts, dtype=I32, device=dev),
        ep_recv_counts=torch.empty(shape.num_experts, dtype=I32, device=dev),
        err_flag=torch.empty(1, dtype=I32, device=dev))
    dyn = torch.empty(shape.capacity, dtype=F32, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    mask = x_active_mask.view(torch.uint8) if x_active_mask is not None and x_active_mask.dtype == torch.bool \
        else x_active_mask
    moe_dispatch_int8(shape, x, topk_idx, mask, smooth_scales, d.expand_x, dyn, d.assist_info_for_combine,
                      d.expert_token_nums, d.ep_recv_counts, d.err_flag, workspace, stream)
    return d, dyn


def shared_expert_shape(T, H, F) -> MoeShape:
    """Shape of a shared expert run as a one-expert group over all T tokens."""
    return make_shape(T, H, 1, 1, F=F, capacity=T)


class _MoELayerFn(torch.autograd.Function):
    """Forward: dispatch -> grouped SwiGLU FFN -> combine; backward: the reverse chain.
    In bf16 the dispatch permute is folded into the two GEMMs that read the
    expanded rows (moe_route, then the gathered gate/up forward and gate/up weight
    gradient read x through the row -> slot map), so no expanded rows are kept.

    A shared expert (shared_w_*) runs as the same grouped FFN with one expert
    whose rows are all T tokens in order, so x itself is its expanded input;
    its output is the shared_expert_x of combine and its input gradient is
    added to grad_x by dispatch_bwd (grad_x_accum).

    fp8: the routed experts' forward and data-gradient GEMMs run on e4m3
    operands (weights quantised in 128 x 128 blocks at every forward,
    activations per (row, 128 columns)), the weight gradients in bf16, or with
    fp8_wgrad on e4m3 operands with one scale per (128 tokens of an expert,
    column); the shared expert stays bf16.  comm_quant_mode 2: the int8 combine payload."""

    @staticmethod
    def forward(ctx, x, topk_weights, w_gate, w_up, w_down, shared_expert_x, shared_w_gate,
                shared_w_up, shared_w_down, topk_idx, x_active_mask, const_alpha_1, const_alpha_2,
                const_v, zero_expert_num, copy_expert_num, const_expert_num, fp8, comm_quant_mode,
                fp8_wgrad, mx):
        T, H = x.shape
        K = topk_idx.shape[1]
        E, F, _ = w_gate.shape
        dev = x.device
        mask_ndim = 0 if x_active_mask is None else x_active_mask.dim()
        shape = make_shape(T, H, K, E, F=F, zero_expert_num=zero_expert_num,
                           copy_expert_num=copy_expert_num, const_expert_num=const_expert_num,
                           mask_ndim=mask_ndim, comm_quant_mode=comm_quant_mode)
        mask = None if x_active_mask is None else x_active_mask.view(torch.uint8)
        # bf16: the routing alone; the gate/up GEMMs read x through the row -> slot
        # map (no expanded rows).  The 8-bit paths quantise the expanded rows.
        # fp8 with fp32 block scales and bf16 weight gradients: the whole step through
        # the fused boundary entries (quantising dispatch, fp8 grouped FFN, combine
        # backward writing dY's codes, fp8 grouped FFN backward)
        ctx.fused8 = bool(fp8) and not mx and not fp8_wgrad
        if ctx.fused8:
            d, xq8, xs8 = dispatch_fp8(shape, x, topk_idx, mask)
        else:
            d = dispatch(shape, x, topk_idx, mask) if fp8 else route(shape, topk_idx, mask)
        cap = shape.capacity
        gus = torch.empty((cap, 2 * F), dtype=BF16, device=dev)
        h = torch.empty((cap, F), dtype=BF16, device=dev)
        y = torch.empty((cap, H), dtype=BF16, device=dev)
        ctx.fp8 = bool(fp8)
        ctx.fp8_wgrad = ctx.fp8 and bool(fp8_wgrad)
        ctx.mx = ctx.fp8 and bool(mx)
        if ctx.mx and ctx.fp8_wgrad:
            raise MoeError("mx=True runs the weight gradients in bf16 (fp8_wgrad uses fp32 block scales)")
        wq = ()
        if ctx.mx:
            nrows = d.ep_recv_counts[-1:]
            wq = tuple(MxWeights.quantize(w) for w in (w_gate, w_up, w_down))
            xq, xs = quant_rows_mx(d.expand_x, nrows)
            # h's MX codes come out of the gate/up GEMM
            hq = torch.empty((cap, F), dtype=U8T, device=dev)
            hs = torch.empty((cap, F // 32), dtype=U8T, device=dev)
            moe_ffn_gate_up_fwd_mx(shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales,
                                   d.ep_recv_counts, gus, h, (hq, hs))
            moe_ffn_down_fwd_mx(shape, hq, hs, wq[2].codes, wq[2].scales, d.ep_recv_counts, y)
            del xq, xs, hq, hs
        elif ctx.fused8:
            wq = tuple(Fp8Weights.quantize(w) for w in (w_gate, w_up, w_down))
            ctx.wq8 = wq
            moe_grouped_ffn_fp8(shape, xq8, xs8, wq, d.ep_recv_counts, gus, h, y,
                                torch.empty(moe_ffn_fp8_workspace_size(shape), dtype=torch.uint8, device=dev))
            del xq8, xs8
        elif ctx.fp8:
            nrows = d.ep_recv_counts[-1:]
            wq = tuple(Fp8Weights.quantize(w) for w in (w_gate, w_up, w_down))
            xq, xs = quant_rows_fp8(d.expand_x, nrows)
            if ctx.fp8_wgrad:
                # h's per-128-token codes for the weight gradient come out of the GEMM
                ns = cols_fp8_slots(cap, E)
                h_cols = (torch.empty((F, 128 * ns), dtype=U8T, device=dev),
                          torch.empty((ns, F), dtype=F32T, device=dev))
                moe_ffn_gate_up_fwd_fp8_quant(shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes,
                                              wq[1].scales, d.ep_recv_counts, gus, h, *h_cols)
                ctx.h_cols = h_cols
            else:
                moe_ffn_gate_up_fwd_fp8(shape, xq, xs, wq[0].codes, wq[0].scales, wq[1].codes, wq[1].scales,
                                        d.ep_recv_counts, gus, h)
            hq, hs = quant_rows_fp8(h, nrows)
            moe_ffn_down_fwd_fp8(shape, hq, hs, wq[2].codes, wq[2].scales, d.ep_recv_counts, y)
            del xq, xs, hq, hs
        else:
            moe_ffn_gate_up_fwd_gather(shape, x, d.assist_info_for_combine, w_gate, w_up, d.ep_recv_counts, gus, h)
            moe_ffn_down_fwd(shape, h, w_down, d.ep_recv_counts, y)
        ctx.shared_ffn = shared_w_gate is not None
        s_saved = ()
        if ctx.shared_ffn:
            if shared_expert_x is not None:
                raise MoeError("pass either shared_expert_x or the shared expert weights, not both")
            Fs = shared_w_gate.shape[1]
            ss = shared_expert_shape(T, H, Fs)
            s_counts = torch.full((1,), T, dtype=I32, device=dev)
            s_gus = torch.empty((T, 2 * Fs), dtype=BF16, device=dev)
            s_h = torch.empty((T, Fs), dtype=BF16, device=dev)
            shared_expert_x = torch.empty((T, H), dtype=BF16, device=dev)
            moe_grouped_ffn(ss, x, shared_w_gate, shared_w_up, shared_w_down, s_counts, s_gus, s_h,
                            shared_expert_x)
            ctx.s_shape = ss
            s_saved = (shared_w_gate, shared_w_up, shared_w_down, s_counts, s_gus, s_h)
        out = torch.empty((T, H), dtype=BF16, device=dev)
        moe_combine(shape, y, topk_idx, topk_weights, d.assist_info_for_combine, d.ep_recv_counts,
                    mask, shared_expert_x, x, const_alpha_1, const_alpha_2, const_v, out)
        ctx.shape = shape
        ctx.has_shared_x = shared_expert_x is not None and not ctx.shared_ffn
        ctx.save_for_backward(x, topk_weights, w_gate, w_up, w_down, topk_idx, mask, const_alpha_1,
                              const_alpha_2, const_v, d.expand_x if fp8 else None, d.assist_info_for_combine,
                              d.ep_recv_counts, gus, h, y, *s_saved)
        # the transposed weight codes of the data-gradient GEMMs (not tensors
        # of the graph, so kept on ctx)
        ctx.wq = tuple((q.codes_t, q.scales_t) if ctx.mx else (q.codes_t, q.scales) for q in wq)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        saved = ctx.saved_tensors
        (x, topk_weights, w_gate, w_up, w_down, topk_idx, mask, a1, a2, cv, expand_x, assist,
         recv, gus, h, y) = saved[:16]
        shape = ctx.shape
        grad_out = grad_out.contiguous()
        cap, H, F, T, K = shape.capacity, shape.H, shape.F, shape.T, shape.K
        dev = x.device
        # grad_y rows exist on the 8-bit paths only (the bf16 down GEMMs read
        # grad_out through the map)
        gy = torch.empty((cap, H), dtype=BF16, device=dev) if ctx.fp8 or not fold_combine_bwd(F) else None
        # routing weights that need no gradient: the combine backward reads no y row
        # and writes only grad_y or the row weights (the fp8 variant always writes both)
        need_gw = ctx.needs_input_grad[1] or ctx.fused8
        gw = torch.empty((T, K), dtype=F32, device=dev) if need_gw else None
        if ctx.fused8:
            gyq = torch.empty((cap, H), dtype=U8T, device=dev)
            gys = torch.empty((H // 128, cap), dtype=F32T, device=dev)
            moe_combine_bwd_fp8(shape, grad_out, y, topk_idx, topk_weights, assist, recv, mask, x, a1, a2, cv,
                                gy, gyq, gys, gw)
        elif not ctx.fp8 and fold_combine_bwd(F):
            # bf16, narrow FFN: the combine backward folded into the down GEMMs
            # (grad_out rows read through the map, each row's routing weight
            # applied in the GEMM)
            roww = torch.empty((cap,), dtype=F32, device=dev)
            moe_combine_bwd_weights(shape, grad_out, y if need_gw else None, topk_idx, topk_weights, assist, recv,
                                    mask, x, a1, a2, cv, gw, roww)
        else:
            moe_combine_bwd(shape, grad_out, y, topk_idx, topk_weights, assist, recv, mask, x, a1, a2, cv,
                            gy, gw)
        # the fp8 weight gradients need no bf16 dG/dU (its codes come out of the
        # down data gradient)
        ggu = None if ctx.fp8_wgrad else torch.empty((cap, 2 * F), dtype=BF16, device=dev)
        gx_exp = torch.empty((cap, H), dtype=BF16, device=dev)
        gwg = torch.empty(w_gate.shape, dtype=F32, device=dev)
        gwu = torch.empty(w_up.shape, dtype=F32, device=dev)
        gwd = torch.empty(w_down.shape, dtype=F32, device=dev)
        # data gradients first, the gate/up weight gradient after dispatch
        # backward (each gather right after the kernel that wrote its input)
        if ctx.fused8:
            moe_grouped_ffn_bwd_fp8(shape, gy, gyq, gys, expand_x, gus, h, ctx.wq8, recv, ggu, gx_exp, gwg, gwu, gwd,
                                    torch.empty(moe_ffn_fp8_workspace_size(shape), dtype=torch.uint8, device=dev))
            del gyq, gys
            ctx.wq8 = None
        elif ctx.mx:
            (wgt, wgs), (wut, wus), (wdt, wds) = ctx.wq
            nrows = recv[-1:]
            dyq, dys = quant_rows_mx(gy, nrows)
            dgq = torch.empty((cap, 2 * F), dtype=U8T, device=dev)
            dgs = torch.empty((cap, 2 * F // 32), dtype=U8T, device=dev)
            moe_ffn_down_bwd_data_mx(shape, dyq, dys, wdt, wds, gus, recv, ggu, (dgq, dgs))
            del dyq, dys
            moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)
            moe_ffn_gate_up_bwd_data_mx(shape, dgq, dgs, wgt, wgs, wut, wus, recv, gx_exp)
            del dgq, dgs
        elif ctx.fp8:
            (wgt, wgs), (wut, wus), (wdt, wds) = ctx.wq
            nrows = recv[-1:]
            dyq, dys = quant_rows_fp8(gy, nrows)
            dgq = torch.empty((cap, 2 * F), dtype=U8T, device=dev)
            dgs = torch.empty((2 * F // 128, cap), dtype=F32T, device=dev)
            if ctx.fp8_wgrad:
                ns = cols_fp8_slots(cap, shape.num_experts)
                dg_cols = (torch.empty((2 * F, 128 * ns), dtype=U8T, device=dev),
                           torch.empty((ns, 2 * F), dtype=F32T, device=dev))
                moe_ffn_down_bwd_data_fp8_quant(shape, dyq, dys, wdt, wds, gus, recv, None, (dgq, dgs), dg_cols)
            else:
                moe_ffn_down_bwd_data_fp8_quant(shape, dyq, dys, wdt, wds, gus, recv, ggu, (dgq, dgs))
            del dyq, dys
            if ctx.fp8_wgrad:
                dyq_t, dys_t = quant_cols_fp8(gy, recv)
                moe_ffn_down_bwd_weight_fp8(shape, dyq_t, dys_t, *ctx.h_cols, recv, gwd)
                del dyq_t, dys_t
                ctx.h_cols = None
            else:
                moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)
            moe_ffn_gate_up_bwd_data_fp8(shape, dgq, dgs, wgt, wgs, wut, wus, recv, gx_exp)
            del dgq, dgs
        elif fold_combine_bwd(F):
            moe_ffn_down_bwd_data_gather(shape, grad_out, assist, roww, w_down, gus, recv, ggu)
            moe_ffn_down_bwd_weight_gather(shape, grad_out, assist, roww, h, recv, gwd)
            moe_ffn_gate_up_bwd_data(shape, ggu, w_gate, w_up, recv, gx_exp)
        else:
            moe_ffn_down_bwd_data(shape, gy, w_down, gus, recv, ggu)
            moe_ffn_down_bwd_weight(shape, gy, h, recv, gwd)
            moe_ffn_gate_up_bwd_data(shape, ggu, w_gate, w_up, recv, gx_exp)
        accum = None
        s_grads = (None, None, None)
        if ctx.shared_ffn:
            swg, swu, swd, s_counts, s_gus, s_h = saved[16:]
            ss = ctx.s_shape
            Fs = ss.F
            s_ggu = torch.empty((T, 2 * Fs), dtype=BF16, device=dev)
            accum = torch.empty((T, H), dtype=BF16, device=dev)
            s_gwg = torch.empty(swg.shape, dtype=F32, device=dev)
            s_gwu = torch.empty(swu.shape, dtype=F32, device=dev)
            s_gwd = torch.empty(swd.shape, dtype=F32, device=dev)
            # the shared expert's output gradient is grad_out itself
            moe_grouped_ffn_bwd(ss, grad_out, x, s_gus, s_h, swg, swu, swd, s_counts, s_ggu, accum,
                                s_gwg, s_gwu, s_gwd)
            s_grads = (s_gwg.to(swg.dtype), s_gwu.to(swu.dtype), s_gwd.to(swd.dtype))
        gx = torch.empty((T, H), dtype=BF16, device=dev)
        moe_dispatch_bwd(shape, gx_exp, assist, topk_idx, topk_weights, mask, grad_out, a1, accum, gx)
        if ctx.fp8_wgrad:
            xq_t, xs_t = quant_cols_fp8(expand_x, recv)
            moe_ffn_gate_up_bwd_weight_fp8(shape, *dg_cols, xq_t, xs_t, recv, gwg, gwu)
            del dg_cols, xq_t, xs_t
        elif ctx.fused8:
            pass  # in moe_grouped_ffn_bwd_fp8
        elif ctx.fp8:
            moe_ffn_gate_up_bwd_weight(shape, ggu, expand_x, recv, gwg, gwu)
        else:
            moe_ffn_gate_up_bwd_weight_gather(shape, ggu, x, assist, recv, gwg, gwu)
        g_shared = grad_out if ctx.has_shared_x else None
        return (gx, gw, gwg.to(w_gate.dtype), gwu.to(w_up.dtype), gwd.to(w_down.dtype), g_shared,
                *s_grads, None, None, None, None, None, None, None, None, None, None, None, None)


@dataclass
class Int8Weights:
    """int8 codes (E, N, K) with one fp32 scale per output channel (E, N) of one weight tensor."""
    codes: torch.Tensor
    scales: torch.Tensor

    @staticmethod
    def quantize(w, stream=None):
        c, s = quant_rows_int8(w.contiguous(), stream=stream)
        return Int8Weights(c, s)


@torch.no_grad()
def moe_layer_int8(x, topk_idx, topk_weights, wq_gate, wq_up, wq_down, *, smooth_scales=None,
                   x_active_mask=None, shared_expert_x=None, const_alpha_1=None, const_alpha_2=None,
                   const_v=None, zero_expert_num=0, copy_expert_num=0, const_expert_num=0, stream=None):
    """Forward of one MoE layer on the decode regime's int8 path (inference, no autograd):
    int8 dispatch (optionally smooth-scaled per expert), w8a8 gate/up GEMM with the SwiGLU
    epilogue, per-row int8 requantisation of h, w8a8 down GEMM, bf16 combine.
    wq_*: Int8Weights of w_gate, w_up (E, F, H) and w_down (E, H, F)."""
    T, H = x.shape
    K = topk_idx.shape[1]
    E, F, _ = wq_gate.codes.shape
    dev = x.device
    mask_ndim = 0 if x_active_mask is None else x_active_mask.dim()
    shape = make_shape(T, H, K, E, F=F, zero_expert_num=zero_expert_num, copy_expert_num=copy_expert_num,
                       const_expert_num=const_expert_num, mask_ndim=mask_ndim)
    mask = None if x_active_mask is None else x_active_mask.view(torch.uint8)
    d, dyn = dispatch_int8(shape, x, topk_idx, mask, smooth_scales, stream=stream)
    cap = shape.capacity
    gus = torch.empty((cap, 2 * F), dtype=BF16, device=dev)
    h = torch.empty((cap, F), dtype=BF16, device=dev)
    y = torch.empty((cap, H), dtype=BF16, device=dev)
    recv = d.ep_recv_counts
    moe_ffn_gate_up_fwd_int8(shape, d.expand_x, dyn, wq_gate.codes, wq_gate.scales, wq_up.codes, wq_up.scales,
                             recv, gus, h, stream)
    hq = torch.empty((cap, F), dtype=I8T, device=dev)
    hs = torch.empty(cap, dtype=F32, device=dev)
    moe_quant_rows_int8(h, hq, hs, recv[-1:], stream)
    moe_ffn_down_fwd_int8(shape, hq, hs, wq_down.codes, wq_down.scales, recv, y, stream)
    out = torch.empty((T, H), dtype=BF16, device=dev)
    moe_combine(shape, y, topk_idx, topk_weights, d.assist_info_for_combine, recv, mask, shared_expert_x, x,
                const_alpha_1, const_alpha_2, const_v, out, stream)
    return out


def moe_layer(x, topk_idx, topk_weights, w_gate, w_up, w_down, *, x_active_mask=None,
              shared_expert_x=None, shared_w_gate=None, shared_w_up=None, shared_w_down=None,
              const_alpha_1=None, const_alpha_2=None, const_v=None,
              zero_expert_num=0, copy_expert_num=0, const_expert_num=0, fp8=False,
              comm_quant_mode=0, fp8_wgrad=False, mx=False):
    """One MoE layer (ori_x is x itself).

    The shared-expert term of combine is either given (shared_expert_x) or
    computed here by a SwiGLU shared expert (shared_w_gate, shared_w_up of shape
    (1, Fs, H), shared_w_down of shape (1, H, Fs)).  Differentiable in x,
    topk_weights, all expert weights and shared_expert_x.  Weight gradients are
    computed in fp32 and returned in the weights' dtype; use the C entries
    directly to keep fp32.

    fp8=True runs the routed experts' forward and data-gradient GEMMs on
    block-scaled e4m3 operands (H and F multiples of 128), and with
    fp8_wgrad=True its weight gradients too, on operands requantised per 128
    tokens of each expert; mx=True (with fp8=True) uses microscaled e4m3 (E8M0
    scale per 32 values, applied by the block-scaled MFMA) instead of fp32 block
    scales for the forward and data-gradient GEMMs; comm_quant_mode=2 sends the
    expert outputs through the int8 combine payload."""
    return _MoELayerFn.apply(x, topk_weights, w_gate, w_up, w_down, shared_expert_x, shared_w_gate,
                             shared_w_up, shared_w_down, topk_idx, x_active_mask, const_alpha_1,
                             const_alpha_2, const_v, zero_expert_num, copy_expert_num,
                             const_expert_num, fp8, comm_quant_mode, fp8_wgrad, mx)
