// Router: softmax top-K gating of each token over its n expert ids, and its
// backward to the logits.
//
// The low_latency_combine page takes topk_idx (K distinct ids per token) and
// topk_weights (a float per token and choice) as inputs ("Parameters") and
// prints no router; this is plain softmax top-K gating: the K ids of the
// largest logits in descending order (equal logits by increasing id), weights
// softmax(logits) at those ids, or renormalised over the K (a softmax over the
// selected logits).
//
// One wave per token, 64 lanes x NPL logits (lane l holds ids q*64 + l), so a
// row is read with coalesced loads once and kept in registers.  Selection: K
// rounds of a wave argmax over the ids not yet taken, (larger logit, then
// smaller id) winning; the owner lane marks its id taken.  Lane k keeps choice
// k; the weights follow from one more wave reduction (the sum of the K
// exponentials, or of all n for the plain softmax).  NaN logits are read as
// -inf.  Memory: 4n bytes read and 8K written per token; the kernel is bound
// by latency, not bandwidth.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int NPL>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_router(const float* __restrict__ logits, int64_t T,
                                                                 int n, int K, int renorm,
                                                                 int32_t* __restrict__ topk_idx,
                                                                 float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // a whole wave leaves together
  const float* row = logits + t * n;
  float v[NPL];
  uint64_t taken = 0;  // bit q: id q*64 + lane already chosen (or past n)
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int id = q * 64 + lane;
    if (id < n) {
      const float x = row[id];
      v[q] = x != x ? -INFINITY : x;
    } else {
      v[q] = -INFINITY;
      taken |= 1ull << q;
    }
  }
  int my_id = 0;
  float my_v = 0.f;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NPL; ++q)
      if (!((taken >> q) & 1) && better(v[q], q * 64 + lane, bv, bi)) { bv = v[q]; bi = q * 64 + lane; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    // K <= n, so an untaken id always exists and bi is a real id
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == k) { my_id = bi; my_v = bv; }
  }
  float w;
  if (renorm) {
    const float top = __shfl(my_v, 0, 64);
    const float e = lane < K ? expf(my_v - top) : 0.f;
    w = e / wave_sum(e);
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < NPL; ++q) m = fmaxf(m, v[q]);
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NPL; ++q)
      if (q * 64 + lane < n) s += expf(v[q] - m);
    w = expf(my_v - m) / wave_sum(s);
  }
  if (lane < K) {
    topk_idx[t * K + lane] = my_id;
    topk_w[t * K + lane] = w;
  }
}

template <int NPL>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_router_bwd(
    const float* __restrict__ logits, int64_t T, int n, int K, int renorm, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ grad_w, float* __restrict__ grad_logits) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  // choice k lives in lane k: its id, weight and incoming gradient
  const int my_id = lane < K ? topk_idx[t * K + lane] : -1;
  const float my_w = lane < K ? topk_w[t * K + lane] : 0.f;
  const float my_dw = lane < K ? grad_w[t * K + lane] : 0.f;
  const float s = wave_sum(my_w * my_dw);  // sum_k w_k dw_k
  // the softmax of the row (plain gating only)
  float p[NPL];
  if (!renorm) {
    const float* row = logits + t * n;
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      const int id = q * 64 + lane;
      float x = -INFINITY;
      if (id < n) {
        x = row[id];
        if (x != x) x = -INFINITY;
      }
      p[q] = x;
      m = fmaxf(m, x);
    }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < NPL; ++q) {
      p[q] = q * 64 + lane < n ? expf(p[q] - m) : 0.f;
      z += p[q];
    }
    z = wave_sum(z);
#pragma unroll
    for (int q = 0; q < NPL; ++q) p[q] /= z;
  }
  // every lane gets the K choices (lanes past K carry id -1, which matches nothing)
  int sid[16];
  float sw[16], sdw[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    sid[k] = __shfl(my_id, k, 64);
    sw[k] = __shfl(my_w, k, 64);
    sdw[k] = __shfl(my_dw, k, 64);
  }
  float* out = grad_logits + t * n;
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int id = q * 64 + lane;
    float wk = 0.f, dwk = 0.f;
    bool sel = false;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (sid[k] == id) { sel = true; wk = sw[k]; dwk = sdw[k]; }
    if (id < n) out[id] = renorm ? (sel ? wk * (dwk - s) : 0.f) : p[q] * ((sel ? dwk : 0.f) - s);
  }
}

int npl_of(int64_t n) {
  int npl = 1;
  while (npl * 64 < n) npl *= 2;
  return npl;
}

}  // namespace
}  // namespace moe

using namespace moe;

namespace {
constexpr int64_t kMaxIds = 64 * 64;  // 64 logits per lane

moe_status check_router(int64_t T, int64_t n, int32_t K, int32_t renorm) {
  if (T < 0 || n < 1 || n > kMaxIds || K < 1 || K > 16 || K > n) return MOE_ERR_BAD_SHAPE;
  if (renorm != 0 && renorm != 1) return MOE_ERR_BAD_RANGE;
  if (T * n > ((int64_t)1 << 40) || (T + kWavesPerBlock - 1) / kWavesPerBlock > 0x7fffffff)
    return MOE_ERR_BAD_SHAPE;
  return MOE_OK;
}
}  // namespace

#define ROUTER_DISPATCH(KERNEL, ...)                                                       \
  do {                                                                                      \
    const dim3 grid((unsigned)((T + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock); \
    switch (npl_of(n)) {                                                                    \
      case 1: hipLaunchKernelGGL(KERNEL<1>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;   \
      case 2: hipLaunchKernelGGL(KERNEL<2>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;   \
      case 4: hipLaunchKernelGGL(KERNEL<4>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;   \
      case 8: hipLaunchKernelGGL(KERNEL<8>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;   \
      case 16: hipLaunchKernelGGL(KERNEL<16>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;  \
      case 32: hipLaunchKernelGGL(KERNEL<32>, grid, block, 0, as_stream(stream), __VA_ARGS__); break;  \
      default: hipLaunchKernelGGL(KERNEL<64>, grid, block, 0, as_stream(stream), __VA_ARGS__); break; \
    }                                                                                       \
  } while (0)

extern "C" moe_status moe_router(int64_t T, int64_t n_ids, int32_t K, int32_t renorm, const float* logits,
                                 int32_t* topk_idx, float* topk_weights, void* stream) {
  const moe_status st = check_router(T, n_ids, K, renorm);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_weights) return MOE_ERR_NULL_ARG;
  const int n = (int)n_ids;
  ROUTER_DISPATCH(k_router, logits, T, n, (int)K, (int)renorm, topk_idx, topk_weights);
  return launch_status();
}

extern "C" moe_status moe_router_bwd(int64_t T, int64_t n_ids, int32_t K, int32_t renorm, const float* logits,
                                     const int32_t* topk_idx, const float* topk_weights,
                                     const float* grad_topk_weights, float* grad_logits, void* stream) {
  const moe_status st = check_router(T, n_ids, K, renorm);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !topk_weights || !grad_topk_weights || !grad_logits || (!renorm && !logits))
    return MOE_ERR_NULL_ARG;
  const int n = (int)n_ids;
  ROUTER_DISPATCH(k_router_bwd, logits, T, n, (int)K, (int)renorm, topk_idx, topk_weights, grad_topk_weights,
                  grad_logits);
  return launch_status();
}
