// The fp8 grouped FFN and its backward as one entry each, the way the bf16
// moe_grouped_ffn / moe_grouped_ffn_bwd chain their GEMMs: block-scaled e4m3
// operands (weights per 128 x 128 block, activations per (row, 128 columns) of
// the contraction; the Megatron-LM MoE performance-test page lists FP8 as a
// precision of its tests, section Added Test Cases), bf16 storage of G, U, h, y,
// dG|dU and dX, bf16 weight gradients.
//
// Forward: gate/up GEMM on the e4m3 rows of moe_dispatch_fp8, h's e4m3 codes
// (its 128-column scale blocks span two of the gate/up GEMM's 64-column h
// tiles, so they are taken by the row quantiser over the finished h), down GEMM.
// Backward (dY codes from moe_combine_bwd_fp8): down data gradient with the
// SwiGLU backward and the codes of dG|dU fused into its epilogue, bf16 down
// weight gradient, gate/up data gradient on those codes, bf16 gate/up weight
// gradient.  Every step is one of the library's single-GEMM entries; the
// workspace holds the codes and scales passed between them.
#include "common.hpp"

namespace {
constexpr size_t kAlign = 256;
size_t up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }
// codes (capacity, C) then scales (C/128, capacity)
size_t rows_bytes(const moe_shape* s, int64_t C) {
  return up((size_t)s->capacity * C) + up((size_t)s->capacity * (C / 128) * sizeof(float));
}
}  // namespace

extern "C" moe_status moe_ffn_fp8_workspace_size(const moe_shape* s, size_t* bytes) {
  moe_status st = moe::check_fp8_shape(s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL_ARG;
  const size_t f = rows_bytes(s, s->F), b = rows_bytes(s, 2 * s->F);
  *bytes = f > b ? f : b;
  return MOE_OK;
}

extern "C" moe_status moe_grouped_ffn_fp8(const moe_shape* s, const uint8_t* expand_xq, const float* x_scales,
                                          const moe_fp8_weight* w, const int32_t* ep_recv_counts,
                                          void* gate_up_save, void* h_act, void* y, void* workspace,
                                          size_t ws_bytes, void* stream) {
  size_t need = 0;
  moe_status st = moe_ffn_fp8_workspace_size(s, &need);
  if (st != MOE_OK) return st;
  if (!w || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  uint8_t* hq = static_cast<uint8_t*>(workspace);
  float* hs = reinterpret_cast<float*>(hq + up((size_t)s->capacity * s->F));
  const int32_t* nrows = ep_recv_counts + (s->num_experts - 1);  // only routed rows
  st = moe_ffn_gate_up_fwd_fp8(s, expand_xq, x_scales, w[0].codes, w[0].scales, w[1].codes, w[1].scales,
                               ep_recv_counts, gate_up_save, h_act, stream);
  if (st != MOE_OK) return st;
  st = moe_quant_rows_fp8(s->capacity, s->F, h_act, nrows, hq, hs, stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_fwd_fp8(s, hq, hs, w[2].codes, w[2].scales, ep_recv_counts, y, stream);
}

extern "C" moe_status moe_grouped_ffn_bwd_fp8(const moe_shape* s, const void* grad_y, const uint8_t* grad_yq,
                                              const float* grad_y_scales, const void* expand_x,
                                              const void* gate_up_save, const void* h_act,
                                              const moe_fp8_weight* w, const int32_t* ep_recv_counts,
                                              void* grad_gate_up, void* grad_expand_x, float* grad_w_gate,
                                              float* grad_w_up, float* grad_w_down, void* workspace,
                                              size_t ws_bytes, void* stream) {
  size_t need = 0;
  moe_status st = moe_ffn_fp8_workspace_size(s, &need);
  if (st != MOE_OK) return st;
  if (!w || !ep_recv_counts || !grad_w_gate || !grad_w_up || !grad_w_down) return MOE_ERR_NULL_ARG;
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  uint8_t* dq = static_cast<uint8_t*>(workspace);
  float* ds = reinterpret_cast<float*>(dq + up((size_t)s->capacity * 2 * s->F));
  if (s->capacity > 0) {
    st = moe_ffn_down_bwd_data_fp8_quant(s, grad_yq, grad_y_scales, w[2].codes_t, w[2].scales, gate_up_save,
                                         ep_recv_counts, grad_gate_up, dq, ds, nullptr, nullptr, stream);
    if (st != MOE_OK) return st;
  }
  st = moe_ffn_down_bwd_weight(s, grad_y, h_act, ep_recv_counts, grad_w_down, stream);
  if (st != MOE_OK) return st;
  if (s->capacity > 0) {
    st = moe_ffn_gate_up_bwd_data_fp8(s, dq, ds, w[0].codes_t, w[0].scales, w[1].codes_t, w[1].scales,
                                      ep_recv_counts, grad_expand_x, stream);
    if (st != MOE_OK) return st;
  }
  return moe_ffn_gate_up_bwd_weight(s, grad_gate_up, expand_x, ep_recv_counts, grad_w_gate, grad_w_up, stream);
}
