// Slot classification and wave-level multisplit of the routing, shared by the
// dispatch kernels and the fused decode kernel.
//
// Follows the low_latency_combine API page, "Parameters": topk_idx (ids in
// range, no duplicate in a row), x_active_mask (1-D prefix of trues or 2-D per
// slot) and the zero/copy/const expert id ranges.
#pragma once

#include "common.hpp"

namespace moe {

struct RouteArgs {
  const int32_t* idx;
  const uint8_t* mask;
  int64_t T;
  int K, E, Z, C, Q, mask_ndim;
};

// Class of slot s = base + lane (the wave's 64 consecutive slots from base; slots
// at or past s1 are not slots): >= 0 routed expert id; MOE_SLOT_NONE;
// MOE_SLOT_COPY; -(3+j).  ORs MOE_FLAG_ID_RANGE / MOE_FLAG_ID_DUPLICATE (and,
// with a 1-D mask, MOE_FLAG_MASK_NOT_PREFIX) into err.  Invalid and duplicate
// slots (the later occurrence) are inactive.  When K divides 64 the wave's
// slots are whole tokens (base is a multiple of K), so a slot's earlier ids of
// its token sit in the lanes just below it: the duplicate test is K-1 lane
// shuffles instead of K-1 loads.
__device__ __forceinline__ int classify_wave(const RouteArgs& a, int64_t base, int64_t s1, uint32_t& err) {
  const int lane = threadIdx.x % kWave;
  const int64_t s = base + lane;
  const bool valid = s < s1;
  const int64_t t = s / a.K;
  const int k = (int)(s - t * a.K);
  const int id = valid ? a.idx[s] : -1;
  bool act = true;
  if (valid && a.mask_ndim == 1) {
    act = a.mask[t] != 0;
    if (k == 0 && t > 0 && act && a.mask[t - 1] == 0) err |= MOE_FLAG_MASK_NOT_PREFIX;
  } else if (valid && a.mask_ndim == 2) {
    act = a.mask[s] != 0;
  }
  bool dup = false;
  if (kWave % a.K == 0) {
    for (int j = 1; j < a.K; ++j) {
      const int o = __shfl_up(id, (unsigned)j, kWave);
      dup |= (j <= k) && (o == id);
    }
  } else if (valid) {
    const int32_t* row = a.idx + t * a.K;
    for (int kk = 0; kk < k; ++kk) dup |= row[kk] == id;
  }
  if (!valid) return MOE_SLOT_NONE;
  const int etot = a.E + a.Z + a.C + a.Q;
  if (id < 0 || id >= etot) {
    err |= MOE_FLAG_ID_RANGE;
    return MOE_SLOT_NONE;
  }
  if (dup) {
    err |= MOE_FLAG_ID_DUPLICATE;
    return MOE_SLOT_NONE;
  }
  if (!act) return MOE_SLOT_NONE;
  if (id < a.E) return id;
  if (id < a.E + a.Z) return MOE_SLOT_NONE;
  if (id < a.E + a.Z + a.C) return MOE_SLOT_COPY;
  return -(3 + (id - a.E - a.Z - a.C));
}

__device__ __forceinline__ uint32_t wave_or_bits(uint32_t v) {
  uint32_t r = 0;
  if (__ballot(v & MOE_FLAG_ID_RANGE)) r |= MOE_FLAG_ID_RANGE;
  if (__ballot(v & MOE_FLAG_ID_DUPLICATE)) r |= MOE_FLAG_ID_DUPLICATE;
  if (__ballot(v & MOE_FLAG_MASK_NOT_PREFIX)) r |= MOE_FLAG_MASK_NOT_PREFIX;
  return r;
}

// Lanes of the wave whose slot is routed to the same expert as this lane's (a
// wave-level multisplit: one ballot per bit of the expert id).  0 when not routed.
__device__ __forceinline__ uint64_t same_expert(int cls, int nbits) {
  const bool routed = cls >= 0;
  uint64_t peers = __ballot(routed);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = routed && ((cls >> b) & 1);
    const uint64_t bb = __ballot(bit);
    peers &= bit ? bb : ~bb;
  }
  return routed ? peers : 0ull;
}

}  // namespace moe
