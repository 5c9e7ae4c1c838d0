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

#include "common.hpp"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

// The per-token slot arrays are sized by a compile-time bound KMAX >= K (2, 4,
// 8 or 16), so a kernel only holds the row registers its K needs.
template <int KMAX>
struct SlotInfo {
  int code[KMAX];
  float w[KMAX];
  bool any_ori;
};

template <int KMAX>
__device__ __forceinline__ void load_slots(const int32_t* slot2row, const float* w, int64_t t,
                                           int K, int lane, SlotInfo<KMAX>& si) {
  const int my = lane < K ? slot2row[t * K + lane] : MOE_SLOT_NONE;
  const float mw = lane < K ? w[t * K + lane] : 0.f;
  bool any = false;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    si.code[k] = k < K ? __builtin_amdgcn_readlane(my, k) : MOE_SLOT_NONE;
    si.w[k] = k < K ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mw), k)) : 0.f;
    any |= si.code[k] <= MOE_SLOT_COPY;
  }
  si.any_ori = any;
}

// Value of a copy or constant slot for one 8-column vector.
__device__ __forceinline__ void special_value(int code, const float* ox, const uint4* a1,
                                              const uint4* a2, const uint4* cv, int64_t Hv,
                                              int64_t v, float* f) {
  if (code == MOE_SLOT_COPY) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = ox[i];
    return;
  }
  const int64_t j = -code - 3;
  float p[8], q[8], c[8];
  unpack8(a1[j * Hv + v], p);
  unpack8(a2[j * Hv + v], q);
  unpack8(cv[j * Hv + v], c);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = p[i] * ox[i] + q[i] * c[i];
}

// int8 payload (comm_quant_mode 2, Parameters of the low_latency_combine page):
// every routed slot's expert-output row is quantised symmetrically per row,
// q = clamp(rint(y * (127/amax)), -127, 127), and used as q * (amax/127).  The
// row's amax comes from a first pass over the row (wave max).
template <int KMAX>
__device__ __forceinline__ void int8_params(const uint4* y, const SlotInfo<KMAX>& si, int64_t Hv,
                                            int lane, float* qinv, float* qsc) {
  float mx[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) mx[k] = 0.f;
  for (int64_t v = lane; v < Hv; v += kWave) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (si.code[k] >= 0) {
        float f[8];
        unpack8(y[(int64_t)si.code[k] * Hv + v], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[k] = fmaxf(mx[k], fabsf(f[i]));
      }
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    float m = mx[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    qinv[k] = m > 0.f ? __fdiv_rn(127.0f, m) : 0.f;
    qsc[k] = m > 0.f ? __fdiv_rn(m, 127.0f) : 1.0f;
  }
}

__device__ __forceinline__ void int8_qdq(float* f, float inv, float sc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(rintf(f[i] * inv), -127.0f), 127.0f) * sc;
}

// int8 parameters from rows already in registers: the token's whole rows are
// one chunk of U vectors per lane (all lanes take part in the butterfly).
template <int KMAX, int U>
__device__ __forceinline__ void int8_params_regs(const uint4 (&raw)[U][KMAX], const SlotInfo<KMAX>& si,
                                                 int lane, int64_t Hv, float* qinv, float* qsc) {
  float mx[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) mx[k] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (lane + u * kWave < Hv) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (si.code[k] >= 0) {
          float f[8];
          unpack8(raw[u][k], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) mx[k] = fmaxf(mx[k], fabsf(f[i]));
        }
    }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    float m = mx[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    qinv[k] = m > 0.f ? __fdiv_rn(127.0f, m) : 0.f;
    qsc[k] = m > 0.f ? __fdiv_rn(m, 127.0f) : 1.0f;
  }
}

struct CombineArgs {
  const uint4* y;
  const float* w;
  const int32_t* slot2row;
  const uint4* shared;
  const uint4* ori;
  const uint4* a1;
  const uint4* a2;
  const uint4* cv;
  uint4* out;
  int64_t T;
  int K;
  int64_t Hv;
  int qpay;  // comm_quant_mode 2: int8 round trip of every expert-output row
  int split;  // waves per token (each takes every split-th 64-vector column block)
};

// A gathered expert-row vector, loaded non-temporally: each row is read once
// (by its token's wave), so the load should not displace cached data (measured
// on MI355X: 3.1 -> 4.0 TB/s for combine and 3.2 -> 4.5 TB/s for dispatch
// backward with the inputs in HBM).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_row(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Vectors per lane whose row loads are issued together before any of them is
// used: U * KMAX 16-byte registers (at most 16), so a wave keeps up to 16 KiB of
// row reads in flight.
template <int KMAX>
constexpr int kChunk = KMAX >= 16 ? 1 : 16 / KMAX;

template <int KMAX, bool ONE_PASS>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int64_t t = gw / a.split;
  const int part = (int)(gw - t * a.split);
  if (t >= a.T) return;
  SlotInfo<KMAX> si;
  load_slots(a.slot2row, a.w, t, a.K, lane, si);
  const int64_t Hv = a.Hv;
  const uint4* __restrict__ y = a.y;
  const uint4* __restrict__ shared = a.shared;
  uint4* __restrict__ out = a.out;
  float qinv[KMAX], qsc[KMAX];
  constexpr int U = kChunk<KMAX>;
  const int64_t vs = (int64_t)a.split * kWave;  // stride between a wave's column blocks
  // int8 payload: when the token's rows fit in one chunk (ONE_PASS; split is 1
  // with the payload), the rows are read once and the amax comes from the
  // registers; otherwise a first pass over the rows finds it
  constexpr bool one_pass = ONE_PASS;
  uint4 pre[ONE_PASS ? U : 1][KMAX];
  if constexpr (ONE_PASS) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane + u * kWave < Hv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (si.code[k] >= 0) pre[u][k] = ld_row(&y[(int64_t)si.code[k] * Hv + lane + u * kWave]);
      }
    int8_params_regs<KMAX, U>(pre, si, lane, Hv, qinv, qsc);
  } else if (a.qpay) {
    int8_params(y, si, Hv, lane, qinv, qsc);
  }
  for (int64_t v0 = lane + part * kWave; v0 < Hv; v0 += U * vs) {
    uint4 raw[U][KMAX], sh[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * vs;
      if (v < Hv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (si.code[k] >= 0) {
            if constexpr (one_pass) raw[u][k] = pre[u][k];
            else raw[u][k] = ld_row(&y[(int64_t)si.code[k] * Hv + v]);
          }
        if (shared) sh[u] = shared[t * Hv + v];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + u * vs;
      if (v < Hv) {
        float ox[8];
        if (si.any_ori) unpack8(a.ori[t * Hv + v], ox);
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
            if (a.qpay) int8_qdq(f, qinv[k], qsc[k]);
          } else {
            special_value(c, ox, a.a1, a.a2, a.cv, Hv, v, f);
          }
          const float wk = si.w[k];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = acc[i] + wk * f[i];
        }
        if (shared) {
          float sv[8];
          unpack8(sh[u], sv);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = acc[i] + sv[i];
        }
        out[t * Hv + v] = pack8(acc);
      }
    }
  }
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
};

template <int KMAX, bool ONE_PASS>
__global__ __launch_bounds__(256) void k_combine_bwd(CombineBwdArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (t >= a.T) return;
  SlotInfo<KMAX> si;
  load_slots(a.slot2row, a.w, t, a.K, lane, si);
  const int64_t Hv = a.Hv;
  const uint4* __restrict__ y = a.y;
  const uint4* __restrict__ dout = a.dout;
  uint4* __restrict__ dy = a.dy;
  float qinv[KMAX], qsc[KMAX];
  constexpr int U = kChunk<KMAX>;
  // int8 payload: one read of the rows when they fit in one chunk (as in combine)
  constexpr bool one_pass = ONE_PASS;
  uint4 pre[ONE_PASS ? U : 1][KMAX];
  if constexpr (ONE_PASS) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane + u * kWave < Hv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (si.code[k] >= 0) pre[u][k] = ld_row(&y[(int64_t)si.code[k] * Hv + lane + u * kWave]);
      }
    int8_params_regs<KMAX, U>(pre, si, lane, Hv, qinv, qsc);
  } else if (a.qpay) {
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
        if (si.any_ori) unpack8(a.ori[t * Hv + v], ox);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int c = si.code[k];
          if (c == MOE_SLOT_NONE) continue;
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
          if (c >= 0) {
            float g[8];
            const float wk = si.w[k];
#pragma unroll
            for (int i = 0; i < 8; ++i) g[i] = wk * d[i];
            dy[(int64_t)c * Hv + v] = pack8(g);
          }
        }
      }
    }
  }
  // fixed-shape butterfly over the wave: the same order for every launch
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < a.K) {
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

inline dim3 token_grid(int64_t T) {
  return dim3((unsigned)((T + kWavesPerBlock - 1) / kWavesPerBlock));
}

// Pointers needed by the special experts (Parameters: ori_x required when
// copy_expert_num or const_expert_num is not 0; the const tensors when
// const_expert_num is not 0).
inline moe_status check_special(const moe_shape* s, const void* ori_x, const void* a1,
                                const void* a2, const void* cv) {
  if ((s->copy_expert_num > 0 || s->const_expert_num > 0) && !ori_x) return MOE_ERR_NULL_ARG;
  if (s->const_expert_num > 0 && (!a1 || !a2 || !cv)) return MOE_ERR_NULL_ARG;
  return MOE_OK;
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
                s->comm_quant_mode == 2 ? 1 : token_split(s->H / 8, s->K)};
  launch_k(s->K, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    if (a.qpay && a.Hv <= (int64_t)kChunk<KM> * kWave)
      hipLaunchKernelGGL((k_combine<KM, true>), token_grid(s->T * a.split), dim3(256), 0, as_stream(stream), a);
    else
      hipLaunchKernelGGL((k_combine<KM, false>), token_grid(s->T * a.split), dim3(256), 0, as_stream(stream), a);
  });
  return launch_status();
}

extern "C" moe_status moe_combine_bwd(const moe_shape* s, const void* grad_out, const void* y,
                                      const int32_t* topk_idx, const float* topk_weights,
                                      const int32_t* assist, const int32_t* ep_send_counts,
                                      const uint8_t* x_active_mask, const void* ori_x,
                                      const void* const_alpha_1, const void* const_alpha_2,
                                      const void* const_v, void* grad_y, float* grad_topk_weights,
                                      void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  MOE_NEED(y, s->capacity * s->H);
  MOE_NEED(grad_y, s->capacity * s->H);
  if (!grad_out || !topk_idx || !topk_weights || !assist || !ep_send_counts ||
      !grad_topk_weights)
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
                   s->comm_quant_mode == 2};
  launch_k(s->K, [&](auto km) {
    constexpr int KM = decltype(km)::value;
    if (a.qpay && a.Hv <= (int64_t)kChunk<KM> * kWave)
      hipLaunchKernelGGL((k_combine_bwd<KM, true>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
    else
      hipLaunchKernelGGL((k_combine_bwd<KM, false>), token_grid(s->T), dim3(256), 0, as_stream(stream), a);
  });
  return launch_status();
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
