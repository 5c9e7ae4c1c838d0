// Combine (forward and backward) and the gradient of dispatch: token-parallel,
// HBM-bound gather-reduce kernels.
//
// Combine follows the low_latency_combine API page, "Function" (Formula and the
// special-expert cases) and "Parameters" (topk_weights, shared_expert_x, ori_x,
// const_expert_alpha_1/_2, const_expert_v, zero/copy/const id ranges):
//   out[t] = sum_k w[t,k] * v(t,k) + shared_expert_x[t]
// with v = y[row] (routed), 0 (zero expert or masked slot), ori_x[t] (copy),
// alpha_1[j]*ori_x[t] + alpha_2[j]*v[j] (constant expert j).
//
// Layout: one 64-lane wave per token, four tokens per 256-thread block; each
// lane owns 16-byte (8 x bf16) column vectors, so every row read or written by
// a wave is a run of fully coalesced 1 KiB transactions.  The K slot codes and
// weights of the token are read once by lanes 0..K-1 and broadcast with
// readlane.  Sums run in k order with separately rounded products and adds (this
// file is compiled without floating-point contraction), so results do not
// depend on the launch shape and are bit-reproducible.
#include <type_traits>

#include "combine_token.hpp"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

template <int KMAX, bool ONE_PASS>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int64_t t = gw / a.split;
  const int part = (int)(gw - t * a.split);
  if (t >= a.T) return;
  combine_token<KMAX, ONE_PASS>(a, t, part, lane);
}

struct CombineBwdArgs {
  const uint4* dout;
  const uint4* y;
  const float* w;
  const int32_t* slot2row;
  const uint4* ori;
  const uint4* a1;
  const uint4* a2;
  const uint4* cv;
  uint4* dy;
  float* dw;
  int64_t T;
  int K;
  int64_t Hv;
  int qpay;
  // Q8: e4m3 codes of every dY row (8 per 16-byte vector) with one fp32 scale
  // per 128 columns, stored (H/128, capacity) like moe_quant_rows_fp8's
  uint2* dyq;
  float* dys;
  int64_t capacity;
  // optional: the routing weight of every routed row, roww[row] = w[slot] (the
  // per-row scales of the gathered down-backward GEMMs)
  float* roww;
};

// Q8: also the e4m3 codes of the bf16 dY rows, by the rule of the row quantiser
// on the stored bf16 values (the 16 lanes of an aligned group hold one
// 128-column block: H is a multiple of 128); dy may then be NULL.
// PART: 0 both outputs; 1 grad_y only (no y row is read); 2 grad_topk_weights
// only (no grad_y row is written); 3 neither (the row weights alone).  Each part
// computes its outputs exactly as the whole kernel does.
template <int KMAX, bool ONE_PASS, bool Q8 = false, int PART = 0>
__global__ __launch_bounds__(256) void k_combine_bwd(CombineBwdArgs a) {
  constexpr bool kDY = PART == 0 || PART == 1, kDW = PART == 0 || PART == 2;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (t >= a.T) return;
  SlotInfo<KMAX> si;
  load_slots(a.slot2row, a.w, t, a.K, lane, si);
  if (a.roww)
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (lane == k && si.code[k] >= 0) a.roww[si.code[k]] = si.w[k];
  if constexpr (PART == 3) return;
  const int64_t Hv = a.Hv;
  const uint4* __restrict__ y = a.y;
  const uint4* __restrict__ dout = a.dout;
  uint4* __restrict__ dy = a.dy;
  float qinv[KMAX], qsc[KMAX];
  constexpr int U = kChunk<KMAX>;
  // int8 payload: one read of the rows when they fit in one chunk (as in combine)
  constexpr bool one_pass = ONE_PASS;
  uint4 pre[ONE_PASS ? U : 1][KMAX];
  if constexpr (ONE_PASS && kDW) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane + u * kWave < Hv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (si.code[k] >= 0) pre[u][k] = ld_row(&y[(int64_t)si.code[k] * Hv + lane + u * kWave]);
      }
    int8_params_regs<KMAX, U>(pre, si, lane, Hv, qinv, qsc);
  } else if (kDW && a.qpay) {
    int8_params(y, si, Hv, lane, qinv, qsc);
  }
  float dot[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) dot[k] = 0.f;
  for (int64_t v0 = lane; v0 < Hv; v0 += U * kWave) {
    uint4 raw[U][KMAX], dr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < Hv) {
        dr[u] = dout[t * Hv + v];
        if constexpr (kDW)
#pragma unroll
          for (int k = 0; k < KMAX; ++k)
            if (si.code[k] >= 0) {
              if constexpr (one_pass) raw[u][k] = pre[u][k];
              else raw[u][k] = ld_row(&y[(int64_t)si.code[k] * Hv + v]);
            }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * kWave;
      if (v < Hv) {
        float d[8];
        unpack8(dr[u], d);
        float ox[8];
        if (kDW && si.any_ori) unpack8(a.ori[t * Hv + v], ox);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int c = si.code[k];
          if (c == MOE_SLOT_NONE) continue;
          if constexpr (kDW) {
            float f[8];
            if (c >= 0) {
              unpack8(raw[u][k], f);
              if (a.qpay) int8_qdq(f, qinv[k], qsc[k]);
            } else {
              special_value(c, ox, a.a1, a.a2, a.cv, Hv, v, f);
            }
            float p = dot[k];
#pragma unroll
            for (int i = 0; i < 8; ++i) p = p + f[i] * d[i];
            dot[k] = p;
          }
          if (kDY && c >= 0) {
            float g[8];
            const float wk = si.w[k];
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = wk * d[i];
            const uint4 gp = pack8(g);
            if (!Q8 || dy) dy[(int64_t)c * Hv + v] = gp;
            if constexpr (Q8) {
              float q[8];
              unpack8(gp, q);
              float amax = 0.f;
#pragma unroll
              for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(q[i]));
#pragma unroll
              for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
              const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
              a.dyq[(int64_t)c * Hv + v] = make_uint2(
                  e4m3x4(__fmul_rn(q[0], inv), __fmul_rn(q[1], inv), __fmul_rn(q[2], inv), __fmul_rn(q[3], inv)),
                  e4m3x4(__fmul_rn(q[4], inv), __fmul_rn(q[5], inv), __fmul_rn(q[6], inv), __fmul_rn(q[7], inv)));
              if ((v & 15) == 0) a.dys[(v >> 4) * a.capacity + c] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
            }
          }
        }
      }
    }
  }
  // fixed-shape butterfly over the wave: the same order for every launch
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (kDW && k < a.K) {
      float p = dot[k];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) p = p + __shfl_xor(p, o, kWave);
      if (lane == 0) a.dw[t * a.K + k] = (si.code[k] == MOE_SLOT_NONE) ? 0.f : p;
    }
  }
}

struct DispatchBwdArgs {
  const uint4* dx_exp;
  const int32_t* slot2row;
  const float* w;
  const uint4* dout;
  const uint4* a1;
  const uint4* accum;
  uint4* dx;
  int64_t T;
  int K;
  int64_t Hv;
  int split;  // waves per token
};

template <int KMAX>
__global__ __launch_bounds__(256) void k_dispatch_bwd(DispatchBwdArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int64_t t = gw / a.split;
  const int part = (int)(gw - t * a.split);
  if (t >= a.T) return;
  SlotInfo<KMAX> si;
  load_slots(a.slot2row, a.w, t, a.K, lane, si);
  const int64_t Hv = a.Hv;
  const uint4* __restrict__ dx_exp = a.dx_exp;
  const uint4* __restrict__ accum = a.accum;
  uint4* __restrict__ dx = a.dx;
  constexpr int U = kChunk<KMAX>;
  const int64_t vs = (int64_t)a.split * kWave;  // stride between a wave's column blocks
  for (int64_t v0 = lane + part * kWave; v0 < Hv; v0 += U * vs) {
    uint4 raw[U][KMAX], ac[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * vs;
      if (v < Hv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (si.code[k] >= 0) raw[u][k] = ld_row(&dx_exp[(int64_t)si.code[k] * Hv + v]);
        if (accum) ac[u] = accum[t * Hv + v];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * vs;
      if (v < Hv) {
        float d[8];
        if (si.any_ori) unpack8(a.dout[t * Hv + v], d);
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int c = si.code[k];
          if (c == MOE_SLOT_NONE) continue;
          float f[8];
          if (c >= 0) {
            unpack8(raw[u][k], f);
          } else if (c == MOE_SLOT_COPY) {
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = si.w[k] * d[i];
          } else {
            float p[8];
            unpack8(a.a1[(int64_t)(-c - 3) * Hv + v], p);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = si.w[k] * (p[i] * d[i]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = acc[i] + f[i];
        }
        if (accum) {
          float sv[8];
          unpack8(ac[u], sv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = acc[i] + sv[i];
        }
        dx[t * Hv + v] = pack8(acc);
      }
    }
  }
}

// Calls f with std::integral_constant<int, KMAX> for the smallest KMAX >= K.
template <typename Fn>
inline void launch_k(int K, Fn f) {
  if (K <= 2) f(std::integral_constant<int, 2>{});
  else if (K <= 4) f(std::integral_constant<int, 4>{});
  else if (K <= 8) f(std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{});
}

// Waves per token of the combine: when the row's 64-vector column blocks split
// evenly into one pass of kChunk blocks per wave (H = 7168, K = 8: 14 blocks,
// seven waves of two), that many; otherwise the split the gradient of dispatch
// uses (at H = 7168, K = 8 seven waves measured 2-3% faster than four).
inline int combine_split(int64_t Hv, int K) {
  if (K >= 4 && Hv % kWave == 0) {
    const int km = K <= 4 ? 4 : (K <= 8 ? 8 : 16);
    const int64_t u = km >= 16 ? 1 : 16 / km;  // kChunk<km>
    const int64_t blocks = Hv / kWave;
    if (blocks % u == 0 && blocks / u >= 4 && blocks / u <= 16) return (int)(blocks / u);
  }
  return token_split(Hv, K);
}

inline dim3 token_grid(int64_t T) {
  return dim3((unsigned)((T + kWavesPerBlock - 1) / kWavesPerBlock));
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_shape* s, const void* y, const int32_t* topk_idx,
                                  const float* topk_weights, const int32_t* assist,
                                  const int32_t* ep_send_counts, const uint8_t* x_active_mask,
                                  const void* shared_expert_x, const void* ori_x,
                                  const void* const_alpha_1, const void* const_alpha_2,
                                  const void* const_v, void* out, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  MOE_NEED(y, s->capacity * s->H);
  if (!topk_idx || !topk_weights || !assist || !ep_send_counts || !out) return MOE_ERR_NULL_ARG;
  if (s->mask_ndim > 0 && !x_active_mask) return MOE_ERR_NULL_ARG;
  st = check_special(s, ori_x, const_alpha_1, const_alpha_2, const_v);
  if (st != MOE_OK) return st;
  CombineArgs a{static_cast<const uint4*>(y),     topk_weights,
                assist,                            static_cast<const uint4*>(shared_expert_x),
                static_cast<const uint4*>(ori_x), static_cast<const uint4*>(const_alpha_1),
                static_cast<const uint4*>(const_alpha_2), static_cast<const uint4*>(const_v),
                static_cast<uint4*>(out),          s->T,
                s->K,                              s->H / 8,
                s->comm_quant_mode == 2,
                // the int8 payload needs every row's amax, which one wave per
                // token computes once
                s->comm_quant_mode == 2 ? 1 : combine_split(s->H / 8, s->K)};
  launch_k(s->K, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    if (a.qpay && a.Hv <= (int64_t)kChunk<KM> * kWave)
      hipLaunchKernelGGL((k_combine<KM, true>), token_grid(s->T * a.split), dim3(256), 0, as_stream(stream), a);
    else
      hipLaunchKernelGGL((k_combine<KM, false>), token_grid(s->T * a.split), dim3(256), 0, as_stream(stream), a);
  });
  return launch_status();
}

namespace {
moe_status combine_bwd_impl(const moe_shape* s, const void* grad_out, const void* y, const int32_t* topk_idx,
                            const float* topk_weights, const int32_t* assist, const int32_t* ep_send_counts,
                            const uint8_t* x_active_mask, const void* ori_x, const void* const_alpha_1,
                            const void* const_alpha_2, const void* const_v, void* grad_y, uint8_t* grad_yq,
                            float* grad_y_scales, float* grad_topk_weights, void* stream,
                            float* row_weights = nullptr) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const bool q8 = grad_yq != nullptr;
  if (q8 && s->H % 128 != 0) return MOE_ERR_BAD_SHAPE;
  if (q8 && s->capacity * (s->H / 128) * 4 >= (int64_t)0x7ffffff0) return MOE_ERR_UNSUPPORTED;
  // bf16: either output may be left out (NULL), not both; the fp8 variant
  // writes grad_topk_weights always
  const int part = q8 ? 0 : (!grad_y ? (grad_topk_weights ? 2 : 3) : (!grad_topk_weights ? 1 : 0));
  if (!q8 && !grad_y && !grad_topk_weights && !row_weights) return MOE_ERR_NULL_ARG;
  if (s->T == 0) return MOE_OK;
  if (part == 0 || part == 2) MOE_NEED(y, s->capacity * s->H);
  if (q8) MOE_NEED(grad_y_scales, s->capacity * (s->H / 128));
  if (!grad_out || !topk_idx || !topk_weights || !assist || !ep_send_counts || (q8 && !grad_topk_weights))
    return MOE_ERR_NULL_ARG;
  if (s->mask_ndim > 0 && !x_active_mask) return MOE_ERR_NULL_ARG;
  st = check_special(s, ori_x, const_alpha_1, const_alpha_2, const_v);
  if (st != MOE_OK) return st;
  CombineBwdArgs a{static_cast<const uint4*>(grad_out),
                   static_cast<const uint4*>(y),
                   topk_weights,
                   assist,
                   static_cast<const uint4*>(ori_x),
                   static_cast<const uint4*>(const_alpha_1),
                   static_cast<const uint4*>(const_alpha_2),
                   static_cast<const uint4*>(const_v),
                   static_cast<uint4*>(grad_y),
                   grad_topk_weights,
                   s->T,
                   s->K,
                   s->H / 8,
                   s->comm_quant_mode == 2,
                   reinterpret_cast<uint2*>(grad_yq),
                   grad_y_scales,
                   s->capacity,
                   row_weights};
  launch_k(s->K, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    const bool one = a.qpay && a.Hv <= (int64_t)kChunk<KM> * kWave;
    if (q8 && one)
      hipLaunchKernelGGL((k_combine_bwd<KM, true, true>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
    else if (q8)
      hipLaunchKernelGGL((k_combine_bwd<KM, false, true>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
    else if (part == 3)  // the row weights alone
      hipLaunchKernelGGL((k_combine_bwd<KM, false, false, 3>), token_grid(s->T), dim3(256), 0, as_stream(stream),
                         a);
    else if (part == 1)  // grad_y alone reads no y row, so it needs no int8 amax either
      hipLaunchKernelGGL((k_combine_bwd<KM, false, false, 1>), token_grid(s->T), dim3(256), 0, as_stream(stream),
                         a);
    else if (part == 2 && one)
      hipLaunchKernelGGL((k_combine_bwd<KM, true, false, 2>), token_grid(s->T), dim3(256), 0, as_stream(stream),
                         a);
    else if (part == 2)
      hipLaunchKernelGGL((k_combine_bwd<KM, false, false, 2>), token_grid(s->T), dim3(256), 0, as_stream(stream),
                         a);
    else if (one)
      hipLaunchKernelGGL((k_combine_bwd<KM, true>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
    else
      hipLaunchKernelGGL((k_combine_bwd<KM, false>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
  });
  return launch_status();
}
}  // namespace

extern "C" moe_status moe_combine_bwd(const moe_shape* s, const void* grad_out, const void* y,
                                      const int32_t* topk_idx, const float* topk_weights,
                                      const int32_t* assist, const int32_t* ep_send_counts,
                                      const uint8_t* x_active_mask, const void* ori_x,
                                      const void* const_alpha_1, const void* const_alpha_2,
                                      const void* const_v, void* grad_y, float* grad_topk_weights,
                                      void* stream) {
  return combine_bwd_impl(s, grad_out, y, topk_idx, topk_weights, assist, ep_send_counts, x_active_mask, ori_x,
                          const_alpha_1, const_alpha_2, const_v, grad_y, nullptr, nullptr, grad_topk_weights,
                          stream);
}

extern "C" moe_status moe_combine_bwd_fp8(const moe_shape* s, const void* grad_out, const void* y,
                                          const int32_t* topk_idx, const float* topk_weights,
                                          const int32_t* assist, const int32_t* ep_send_counts,
                                          const uint8_t* x_active_mask, const void* ori_x,
                                          const void* const_alpha_1, const void* const_alpha_2,
                                          const void* const_v, void* grad_y, uint8_t* grad_yq,
                                          float* grad_y_scales, float* grad_topk_weights, void* stream) {
  if (!grad_yq) return MOE_ERR_NULL_ARG;
  return combine_bwd_impl(s, grad_out, y, topk_idx, topk_weights, assist, ep_send_counts, x_active_mask, ori_x,
                          const_alpha_1, const_alpha_2, const_v, grad_y, grad_yq, grad_y_scales,
                          grad_topk_weights, stream);
}

extern "C" moe_status moe_combine_bwd_weights(const moe_shape* s, const void* grad_out, const void* y,
                                              const int32_t* topk_idx, const float* topk_weights,
                                              const int32_t* assist, const int32_t* ep_send_counts,
                                              const uint8_t* x_active_mask, const void* ori_x,
                                              const void* const_alpha_1, const void* const_alpha_2,
                                              const void* const_v, float* grad_topk_weights, float* row_weights,
                                              void* stream) {
  if (!row_weights) return MOE_ERR_NULL_ARG;
  return combine_bwd_impl(s, grad_out, y, topk_idx, topk_weights, assist, ep_send_counts, x_active_mask, ori_x,
                          const_alpha_1, const_alpha_2, const_v, nullptr, nullptr, nullptr, grad_topk_weights,
                          stream, row_weights);
}

extern "C" moe_status moe_dispatch_bwd(const moe_shape* s, const void* grad_expand_x,
                                       const int32_t* assist, const int32_t* topk_idx,
                                       const float* topk_weights, const uint8_t* x_active_mask,
                                       const void* grad_out, const void* const_alpha_1,
                                       const void* grad_x_accum, void* grad_x, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  MOE_NEED(grad_expand_x, s->capacity * s->H);
  if (!assist || !topk_idx || !topk_weights || !grad_x) return MOE_ERR_NULL_ARG;
  if (s->mask_ndim > 0 && !x_active_mask) return MOE_ERR_NULL_ARG;
  if ((s->copy_expert_num > 0 || s->const_expert_num > 0) && !grad_out) return MOE_ERR_NULL_ARG;
  if (s->const_expert_num > 0 && !const_alpha_1) return MOE_ERR_NULL_ARG;
  DispatchBwdArgs a{static_cast<const uint4*>(grad_expand_x),
                    assist,
                    topk_weights,
                    static_cast<const uint4*>(grad_out),
                    static_cast<const uint4*>(const_alpha_1),
                    static_cast<const uint4*>(grad_x_accum),
                    static_cast<uint4*>(grad_x),
                    s->T,
                    s->K,
                    s->H / 8,
                    token_split(s->H / 8, s->K)};
  launch_k(s->K, [&](auto km) {
    hipLaunchKernelGGL(k_dispatch_bwd<decltype(km)::value>, token_grid(s->T * a.split), dim3(256), 0,
                       as_stream(stream), a);
  });
  return launch_status();
}
