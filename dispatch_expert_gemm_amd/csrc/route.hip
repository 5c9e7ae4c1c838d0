// Dispatch: classify every (token, choice) slot, count tokens per expert,
// prefix-sum the counts and lay the active routed slots out by expert in
// increasing slot order, then copy each token's row to its expert rows.
//
// Follows the low_latency_combine API page, "Parameters": topk_idx (ids in
// range, no duplicate in a row), x_active_mask (1-D prefix of trues or 2-D per
// slot), zero/copy/const expert id ranges, and ep_send_counts as a prefix sum of
// per-expert counts.  With one device the all-to-all of low_latency_dispatch is
// the permutation built here.
//
// Kernels (all on the caller's stream, no host synchronisation):
//   k_route_count  one wave per chunk of 64*R slots: classify, per-chunk expert
//                  histogram in LDS, chunk error bits
//   k_route_scan   one block: per-expert sums over chunks (each expert's column
//                  split across thread groups), scan over experts, exclusive
//                  per-(chunk, expert) row offsets, outputs
//   k_route_rank   one wave per chunk: stable rank of each routed slot among
//                  the slots of its expert in the chunk (wave ballots), writes
//                  slot->row and row->slot
//   k_permute      one wave (or 2-4 for wide rows) per token: read x[t] once,
//                  write it to its rows
#include "common.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
// Slot chunks: one wave takes 64 R slots, R >= kMinSlotsPerLane, and R grows
// once the chunk count would pass kMaxChunks (measured on MI355X at 65536 and
// 32768 slots: 2 slots per lane and up to 512 chunks beat 4 and 256 by 5%).
constexpr int kMaxChunks = 512;
constexpr int kMinSlotsPerLane = 2;

struct RouteArgs {
  const int32_t* idx;
  const uint8_t* mask;
  int64_t T;
  int K, E, Z, C, Q, mask_ndim;
};

// Class of slot s: >= 0 routed expert id; MOE_SLOT_NONE; MOE_SLOT_COPY; -(3+j).
// ORs MOE_FLAG_ID_RANGE / MOE_FLAG_ID_DUPLICATE into err.  Invalid and duplicate
// slots (the later occurrence) are inactive.
__device__ __forceinline__ int classify(const RouteArgs& a, int64_t s, uint32_t& err) {
  const int64_t t = s / a.K;
  const int k = (int)(s - t * a.K);
  const int id = a.idx[s];
  const int etot = a.E + a.Z + a.C + a.Q;
  if (id < 0 || id >= etot) {
    err |= MOE_FLAG_ID_RANGE;
    return MOE_SLOT_NONE;
  }
  const int32_t* row = a.idx + t * a.K;
  for (int kk = 0; kk < k; ++kk)
    if (row[kk] == id) {
      err |= MOE_FLAG_ID_DUPLICATE;
      return MOE_SLOT_NONE;
    }
  bool act = true;
  if (a.mask_ndim == 1) act = a.mask[t] != 0;
  else if (a.mask_ndim == 2) act = a.mask[s] != 0;
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

__global__ __launch_bounds__(256) void k_route_count(RouteArgs a, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ chunk_err,
                                                     int64_t nslots, int nchunks, int R) {
  extern __shared__ int32_t sh[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int chunk = blockIdx.x * kWavesPerBlock + wave;
  int32_t* h = sh + wave * a.E;
  for (int e = lane; e < a.E; e += kWave) h[e] = 0;
  __syncthreads();
  uint32_t err = 0;
  if (chunk < nchunks) {
    for (int r = 0; r < R; ++r) {
      const int64_t s = ((int64_t)chunk * R + r) * kWave + lane;
      if (s < nslots) {
        const int cls = classify(a, s, err);
        if (cls >= 0) atomicAdd(&h[cls], 1);
        if (a.mask_ndim == 1 && (s % a.K) == 0) {
          const int64_t t = s / a.K;
          if (t > 0 && a.mask[t] != 0 && a.mask[t - 1] == 0) err |= MOE_FLAG_MASK_NOT_PREFIX;
        }
      }
    }
  }
  __syncthreads();
  if (chunk < nchunks) {
    for (int e = lane; e < a.E; e += kWave) hist[(int64_t)chunk * a.E + e] = h[e];
    const uint32_t we = wave_or_bits(err);
    if (lane == 0) chunk_err[chunk] = (int32_t)we;
  }
}

// One block of 1024 threads.  Thread (e, grp) with e = tid % Ep, grp = tid / Ep
// (Ep = E rounded up to a power of two, G = 1024 / Ep groups) owns the chunks
// [grp*per, (grp+1)*per) of expert e's column: it sums them, the group sums
// are scanned in LDS, the expert totals are scanned over experts, and each
// thread rewrites its chunks as exclusive row offsets.
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ hist,
                                                     const int32_t* __restrict__ chunk_err,
                                                     int nchunks, int E, int Ep,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ prefix,
                                                     int32_t* __restrict__ err_flag) {
  __shared__ int32_t part[1024];  // [grp][e] partial sums
  __shared__ int32_t tot[1024];   // expert totals, then their inclusive scan
  __shared__ int32_t errsh;
  const int tid = threadIdx.x;
  const int G = 1024 / Ep;
  const int e = tid % Ep, grp = tid / Ep;
  const int per = (nchunks + G - 1) / G;
  const int c0 = grp * per, c1 = (c0 + per < nchunks) ? c0 + per : nchunks;
  if (tid == 0) errsh = 0;
  int32_t sum = 0;
  if (e < E) {
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hist[(int64_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
    for (; c < c1; ++c) sum += hist[(int64_t)c * E + e];
  }
  part[grp * Ep + e] = sum;
  __syncthreads();
  uint32_t er = 0;
  for (int c = tid; c < nchunks; c += 1024) er |= (uint32_t)chunk_err[c];
  if (er) atomicOr(&errsh, (int32_t)er);
  // exclusive prefix of this thread's group within its expert, and the expert total
  int32_t before = 0, total = 0;
  for (int q = 0; q < G; ++q) {
    const int32_t v = part[q * Ep + e];
    before += q < grp ? v : 0;
    total += v;
  }
  tot[tid] = tid < Ep ? total : 0;  // thread tid < Ep is (expert tid, group 0)
  __syncthreads();
  // inclusive scan of the expert totals (Hillis-Steele over 1024 entries)
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (e < E) {
    if (grp == 0) {
      counts[e] = total;
      prefix[e] = tot[e];
    }
    int32_t run = tot[e] - total + before;  // exclusive base of (expert e, chunk c0)
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = hist[(int64_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hist[(int64_t)(c + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; c < c1; ++c) {
      const int32_t v = hist[(int64_t)c * E + e];
      hist[(int64_t)c * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  if (tid == 0) *err_flag = errsh;
}

__global__ __launch_bounds__(256) void k_route_rank(RouteArgs a, const int32_t* __restrict__ offs,
                                                    int64_t nslots, int nchunks, int R, int nbits,
                                                    int32_t* __restrict__ slot2row,
                                                    int32_t* __restrict__ row2slot) {
  extern __shared__ int32_t sh[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int chunk = blockIdx.x * kWavesPerBlock + wave;
  int32_t* h = sh + wave * a.E;
  if (chunk < nchunks)
    for (int e = lane; e < a.E; e += kWave) h[e] = offs[(int64_t)chunk * a.E + e];
  __syncthreads();
  if (chunk >= nchunks) return;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < R; ++r) {
    const int64_t s = ((int64_t)chunk * R + r) * kWave + lane;
    uint32_t unused = 0;
    const int cls = s < nslots ? classify(a, s, unused) : MOE_SLOT_NONE;
    const bool routed = cls >= 0;
    // lanes routed to the same expert: match every bit of the expert id
    uint64_t peers = __ballot(routed);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = routed && ((cls >> b) & 1);
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    int base = 0;
    if (routed) base = h[cls];
    if (routed) {
      const int row = base + __popcll(peers & below);
      slot2row[s] = row;
      row2slot[row] = (int32_t)s;
      if ((peers & below) == 0) h[cls] = base + __popcll(peers);
    } else if (s < nslots) {
      slot2row[s] = cls;
    }
  }
}

__global__ __launch_bounds__(256) void k_permute(const uint4* __restrict__ x,
                                                 const int32_t* __restrict__ slot2row, int64_t T,
                                                 int K, int64_t Hv, int split, uint4* __restrict__ ex) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const int64_t t = gw / split;
  const int part = (int)(gw - t * split);
  if (t >= T) return;
  const int my = lane < K ? slot2row[t * K + lane] : -1;
  int rows[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) rows[k] = k < K ? __builtin_amdgcn_readlane(my, k) : -1;
  const uint4* xr = x + t * Hv;
  // the wave's column blocks are part, part + split, ...
  for (int64_t v = lane + part * kWave; v < Hv; v += (int64_t)split * kWave) {
    const uint4 val = xr[v];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (rows[k] >= 0) ex[(int64_t)rows[k] * Hv + v] = val;
  }
}

// int8 dispatch (quant_mode 2): one wave per slot (token, choice), so a decode
// batch of a few hundred tokens still gives thousands of waves; the wave reads
// the token's row (NV 16-byte vectors per lane, H <= 64 * 8 * NV, kept packed
// in registers), multiplies it by the smooth-scale row of the slot's expert when
// given, and writes the int8 row with one dynamic scale: codes clamp(rint(v *
// (127/amax)), -127, 127), scale amax/127 (all-zero: codes 0, scale 1).
template <int NV>
__global__ __launch_bounds__(256) void k_permute_i8(const uint4* __restrict__ x, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ slot2row, int64_t nslots, int K,
                                                    int64_t Hv, const float* __restrict__ smooth,
                                                    uint2* __restrict__ exq, float* __restrict__ dyn) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t sl = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (sl >= nslots) return;
  const int row = slot2row[sl];
  if (row < 0) return;  // the whole wave: not a routed slot
  const int64_t t = sl / K;
  const float4* sr = smooth ? reinterpret_cast<const float4*>(smooth + (int64_t)idx[sl] * Hv * 8) : nullptr;
  uint4 xr[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int64_t v = lane + (int64_t)q * kWave;
    xr[q] = v < Hv ? x[t * Hv + v] : make_uint4(0u, 0u, 0u, 0u);
  }
  // the 8 values of vector q, times the smooth-scale row when given
  auto vals = [&](int q, float (&f)[8]) {
    unpack8(xr[q], f);
    if (sr) {
      const int64_t v = lane + (int64_t)q * kWave;
      const float4 s0 = sr[2 * v], s1 = sr[2 * v + 1];
      f[0] = __fmul_rn(f[0], s0.x); f[1] = __fmul_rn(f[1], s0.y);
      f[2] = __fmul_rn(f[2], s0.z); f[3] = __fmul_rn(f[3], s0.w);
      f[4] = __fmul_rn(f[4], s1.x); f[5] = __fmul_rn(f[5], s1.y);
      f[6] = __fmul_rn(f[6], s1.z); f[7] = __fmul_rn(f[7], s1.w);
    }
  };
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    if (lane + (int64_t)q * kWave >= Hv) continue;
    float f[8];
    vals(q, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  }
  m = wave_max64(m);
  const float inv = m > 0.f ? __fdiv_rn(127.0f, m) : 0.f;
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int64_t v = lane + (int64_t)q * kWave;
    if (v >= Hv) continue;
    float f[8];
    vals(q, f);
    exq[(int64_t)row * Hv + v] = make_uint2(i8x4(f[0], f[1], f[2], f[3], inv), i8x4(f[4], f[5], f[6], f[7], inv));
  }
  if (lane == 0) dyn[row] = m > 0.f ? __fdiv_rn(m, 127.0f) : 1.0f;
}

struct RouteGeom {
  int64_t nslots;
  int R;
  int nchunks;
};

RouteGeom route_geom(const moe_shape* s) {
  RouteGeom g;
  g.nslots = s->T * s->K;
  const int64_t per = (int64_t)kWave * kMaxChunks;
  int64_t R = (g.nslots + per - 1) / per;
  g.R = (int)(R < kMinSlotsPerLane ? kMinSlotsPerLane : R);
  g.nchunks = (int)((g.nslots + (int64_t)kWave * g.R - 1) / ((int64_t)kWave * g.R));
  return g;
}

size_t route_ws_bytes(const moe_shape* s) {
  const RouteGeom g = route_geom(s);
  const size_t b = ((size_t)g.nchunks * s->num_experts + g.nchunks + 1) * sizeof(int32_t);
  return (b + 255) & ~(size_t)255;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "a size is out of range or misaligned";
    case MOE_ERR_BAD_RANGE: return "an enumerated field has an unknown value";
    case MOE_ERR_CAPACITY: return "capacity is below T * min(num_experts, K)";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" moe_status moe_assist_info_size(const moe_shape* s, int64_t* n) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!n) return MOE_ERR_NULL_ARG;
  *n = s->T * s->K + s->capacity;
  return MOE_OK;
}

extern "C" moe_status moe_workspace_size(const moe_shape* s, size_t* bytes) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL_ARG;
  *bytes = route_ws_bytes(s);
  return MOE_OK;
}

namespace {
// argument checks shared by the two dispatch entries (the expanded-row buffer is
// checked by each)
moe_status check_dispatch(const moe_shape* s, const int32_t* topk_idx,
                          const uint8_t* x_active_mask, int32_t* assist, int32_t* expert_token_nums,
                          int32_t* ep_recv_counts, int32_t* err_flag, void* workspace, size_t ws_bytes) {
  const int64_t TK = s->T * s->K;
  MOE_NEED(topk_idx, TK);
  MOE_NEED(x_active_mask, s->mask_ndim == 0 ? 0 : (s->mask_ndim == 1 ? s->T : TK));
  MOE_NEED(assist, TK + s->capacity);
  if (!expert_token_nums || !ep_recv_counts || !err_flag) return MOE_ERR_NULL_ARG;
  const size_t need = route_ws_bytes(s);
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// the routing kernels of both dispatch entries: counts, scan, rank (maps)
void launch_route(const moe_shape* s, const int32_t* topk_idx, const uint8_t* x_active_mask,
                  int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                  int32_t* err_flag, void* workspace, hipStream_t strm) {
  const RouteGeom g = route_geom(s);
  RouteArgs a{topk_idx, x_active_mask, s->T, s->K, s->num_experts, s->zero_expert_num,
              s->copy_expert_num, s->const_expert_num, s->mask_ndim};
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* cerr = hist + (size_t)g.nchunks * s->num_experts;
  int32_t* slot2row = assist;
  int32_t* row2slot = assist + s->T * s->K;
  const size_t lds = (size_t)kWavesPerBlock * s->num_experts * sizeof(int32_t);
  const int blocks = (g.nchunks + kWavesPerBlock - 1) / kWavesPerBlock;
  if (g.nchunks > 0)
    hipLaunchKernelGGL(k_route_count, dim3(blocks), dim3(256), lds, strm, a, hist, cerr,
                       g.nslots, g.nchunks, g.R);
  int Ep = 1;
  while (Ep < s->num_experts) Ep <<= 1;
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, strm, hist, cerr, g.nchunks,
                     s->num_experts, Ep, expert_token_nums, ep_recv_counts, err_flag);
  if (g.nchunks > 0) {
    int nbits = 0;
    while ((1 << nbits) < s->num_experts) ++nbits;
    hipLaunchKernelGGL(k_route_rank, dim3(blocks), dim3(256), lds, strm, a, hist, g.nslots,
                       g.nchunks, g.R, nbits, slot2row, row2slot);
  }
}
}  // namespace

extern "C" moe_status moe_route(const moe_shape* s, const int32_t* topk_idx, const uint8_t* x_active_mask,
                                int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                                int32_t* err_flag, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_dispatch(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag,
                      workspace, ws_bytes);
  if (st != MOE_OK) return st;
  launch_route(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag, workspace,
               as_stream(stream));
  return launch_status();
}

extern "C" moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                   const uint8_t* x_active_mask, void* expand_x,
                                   int32_t* assist, int32_t* expert_token_nums,
                                   int32_t* ep_recv_counts, int32_t* err_flag, void* workspace,
                                   size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_dispatch(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag,
                      workspace, ws_bytes);
  if (st != MOE_OK) return st;
  MOE_NEED(x, s->T * s->H);
  MOE_NEED(expand_x, s->capacity * s->H);
  hipStream_t strm = as_stream(stream);
  launch_route(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag, workspace, strm);
  const int32_t* slot2row = assist;
  if (s->T > 0) {
    const int split = token_split(s->H / 8, s->K);
    const int64_t pb = (s->T * split + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_permute, dim3((unsigned)pb), dim3(256), 0, strm,
                       static_cast<const uint4*>(x), slot2row, s->T, s->K, s->H / 8, split,
                       static_cast<uint4*>(expand_x));
  }
  return launch_status();
}

extern "C" moe_status moe_dispatch_int8(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                        const uint8_t* x_active_mask, const float* smooth_scales,
                                        int8_t* expand_x, float* dynamic_scales, int32_t* assist,
                                        int32_t* expert_token_nums, int32_t* ep_recv_counts,
                                        int32_t* err_flag, void* workspace, size_t ws_bytes,
                                        void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  // the row lives in registers: at most 16 vectors of 8 per lane
  if (s->H > 64 * 8 * 16) return MOE_ERR_UNSUPPORTED;
  st = check_dispatch(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag,
                      workspace, ws_bytes);
  if (st != MOE_OK) return st;
  MOE_NEED(x, s->T * s->H);
  MOE_NEED(expand_x, s->capacity * s->H);
  MOE_NEED(dynamic_scales, s->capacity);
  hipStream_t strm = as_stream(stream);
  launch_route(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag, workspace, strm);
  if (s->T > 0) {
    const int64_t Hv = s->H / 8;
    const int nv = (int)((Hv + kWave - 1) / kWave);
    const int64_t nslots = s->T * s->K;
    const dim3 grid((unsigned)((nslots + kWavesPerBlock - 1) / kWavesPerBlock)), block(256);
    const uint4* xv = static_cast<const uint4*>(x);
    uint2* out = reinterpret_cast<uint2*>(expand_x);
#define PERMUTE_I8(N)                                                                                        \
  hipLaunchKernelGGL(k_permute_i8<N>, grid, block, 0, strm, xv, topk_idx, assist, nslots, s->K, Hv, smooth_scales, \
                     out, dynamic_scales)
    if (nv <= 1) PERMUTE_I8(1);
    else if (nv <= 2) PERMUTE_I8(2);
    else if (nv <= 4) PERMUTE_I8(4);
    else if (nv <= 8) PERMUTE_I8(8);
    else PERMUTE_I8(16);
#undef PERMUTE_I8
  }
  return launch_status();
}
