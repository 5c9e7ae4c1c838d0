// The per-token combine (low_latency_combine API page, "Function": the Formula
// and the special-expert cases; "Parameters": topk_weights, shared_expert_x,
// ori_x, const_expert_alpha_1/_2, const_expert_v, the int8 payload of
// comm_quant_mode 2), shared by the combine kernel and the fused decode kernel.
// Sums run in k order with separately rounded products and adds (floating-point
// contraction is off in these functions), so a token's result does not depend
// on the kernel that computes it.
#pragma once

#include "common.hpp"

namespace moe {

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
#pragma clang fp contract(off)
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

// Combine of token t (the column vectors of part `part` of its row, every
// split-th block of 64 vectors), one wave, lane `lane`; UC vectors per lane in
// flight per slot (the result does not depend on it).
template <int KMAX, bool ONE_PASS, int UC = kChunk<KMAX>>
__device__ __forceinline__ void combine_token(const CombineArgs& a, int64_t t, int part, int lane) {
#pragma clang fp contract(off)
  SlotInfo<KMAX> si;
  load_slots(a.slot2row, a.w, t, a.K, lane, si);
  const int64_t Hv = a.Hv;
  const uint4* __restrict__ y = a.y;
  const uint4* __restrict__ shared = a.shared;
  uint4* __restrict__ out = a.out;
  float qinv[KMAX], qsc[KMAX];
  constexpr int U = ONE_PASS ? kChunk<KMAX> : UC;
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

// Pointers needed by the special experts (Parameters: ori_x required when
// copy_expert_num or const_expert_num is not 0; the const tensors when
// const_expert_num is not 0).
inline moe_status check_special(const moe_shape* s, const void* ori_x, const void* a1,
                                const void* a2, const void* cv) {
  if ((s->copy_expert_num > 0 || s->const_expert_num > 0) && !ori_x) return MOE_ERR_NULL_ARG;
  if (s->const_expert_num > 0 && (!a1 || !a2 || !cv)) return MOE_ERR_NULL_ARG;
  return MOE_OK;
}

}  // namespace moe
