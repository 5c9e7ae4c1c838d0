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
// Two kernels, on the caller's stream, no host synchronisation.  The slots are
// cut into chunks of whole tokens (about 512 slots, more when there are many
// tokens, so that there are at most 256 chunks and at most 32768 (chunk,
// expert) counts):
//   k_route_count  one workgroup per chunk: classify every slot, count the
//                  chunk's slots per expert with wave ballots (lanes with the
//                  same expert are found by ballots over the bits of its id;
//                  the lowest of them adds their number), chunk error bits
//   k_route_place  P workgroups per chunk: each sums the counts of the chunks
//                  before its own and of all chunks per expert (16-byte loads
//                  spread over the workgroup), scans the expert totals, gives
//                  every routed slot of the chunk its row (stable rank among
//                  the chunk's slots of its expert, by the same ballots) and
//                  writes both maps; then, for dispatch, the P workgroups of
//                  the chunk each copy 1/P of the chunk's tokens to their rows.
//                  The first workgroup also writes the counts, the prefix sums
//                  and the error flag.
#include "route_wave.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

// Chunks of whole tokens: chunk c holds tokens [c tpc, (c+1) tpc), its slots
// t K + k in 64-slot rounds.  Counts are stored per chunk in rows of Ep = E
// rounded up to a multiple of 4 (16-byte loads).
struct RouteGeom {
  int64_t nslots, tpc;
  int nchunks, rounds, Ep, P;
};

__global__ __launch_bounds__(256) void k_route_count(RouteArgs a, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ chunk_err, int64_t tpc, int rounds,
                                                     int Ep, int nbits) {
  extern __shared__ int32_t sh[];  // [4][Ep] per-wave counts
  __shared__ uint32_t errsh;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t c = blockIdx.x;
  for (int i = threadIdx.x; i < 4 * Ep; i += 256) sh[i] = 0;
  if (threadIdx.x == 0) errsh = 0;
  __syncthreads();
  const int64_t t1 = (c + 1) * tpc < a.T ? (c + 1) * tpc : a.T;
  const int64_t s0 = c * tpc * a.K, s1 = t1 * a.K;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* h = sh + wave * Ep;
  uint32_t err = 0;
  for (int r = wave; r < rounds; r += 4) {
    const int cls = classify_wave(a, s0 + (int64_t)r * kWave, s1, err);
    const uint64_t peers = same_expert(cls, nbits);
    // one lane per expert present in the round adds the round's count
    if (peers && (peers & below) == 0) h[cls] += __popcll(peers);
  }
  const uint32_t we = wave_or_bits(err);
  if (lane == 0 && we) atomicOr(&errsh, we);
  __syncthreads();
  for (int e = threadIdx.x; e < Ep; e += 256) hist[c * Ep + e] = sh[e] + sh[Ep + e] + sh[2 * Ep + e] + sh[3 * Ep + e];
  if (threadIdx.x == 0) chunk_err[c] = (int32_t)errsh;
}

// Inclusive scan of v over the 256 threads of a block (wave scans with lane
// shuffles, then the wave totals).
__device__ __forceinline__ int32_t block_scan(int32_t v, int32_t* wtot) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wtot[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += wtot[w];
  __syncthreads();
  return v;
}

// COPY: 0 maps only; 1 bf16 token rows to their rows; 2 e4m3 codes of the
// token rows (one fp32 scale per 128 columns, the rule of moe_quant_rows_fp8,
// taken once per token) to their rows, and the bf16 rows too when ex is given.
template <int COPY>
__global__ __launch_bounds__(256) void k_route_place(RouteArgs a, const int32_t* __restrict__ hist,
                                                     const int32_t* __restrict__ chunk_err, int64_t tpc, int nchunks,
                                                     int rounds, int Ep, int nbits, int P,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ prefix,
                                                     int32_t* __restrict__ err_flag, int32_t* __restrict__ slot2row,
                                                     int32_t* __restrict__ row2slot, const uint4* __restrict__ x,
                                                     int64_t Hv, uint4* __restrict__ ex, uint2* __restrict__ exq,
                                                     float* __restrict__ exs, int64_t capacity) {
  constexpr bool PERMUTE = COPY != 0;
  // LDS: off[4][Ep] running row offsets of each wave's rounds, cnt[4][Ep] their
  // counts, red[2][G][Ep] partial sums (G * Ep <= 1024), rows of this
  // workgroup's tokens [tokens of the part][K]
  extern __shared__ int32_t sh[];
  int32_t* off = sh;
  int32_t* cnt = sh + 4 * Ep;
  int32_t* red = sh + 8 * Ep;
  int32_t* rows = sh + 8 * Ep + 2048;
  __shared__ int32_t wtot[4];
  __shared__ uint32_t errsh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t c = blockIdx.x / P;
  const int p = (int)(blockIdx.x % P);
  for (int i = tid; i < 4 * Ep; i += 256) cnt[i] = 0;
  // counts of chunks before c (pre) and of all chunks (tot), per expert: thread
  // tid sums four experts (one 16-byte load per chunk) over every G-th chunk
  const int q4 = Ep / 4;                       // 16-byte columns per row
  const int G = q4 >= 256 ? 1 : 256 / q4;      // chunk groups
  for (int col = tid % (q4 < 256 ? q4 : 256); col < q4; col += 256) {
    int4 pre4 = {0, 0, 0, 0}, tot4 = {0, 0, 0, 0};
    const int g = q4 >= 256 ? 0 : tid / q4;
    if (g < G) {
      // eight independent loads in flight per round of the loop
      for (int cc0 = g; cc0 < nchunks; cc0 += 8 * G) {
        int4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int cc = cc0 + u * G;
          v[u] = cc < nchunks ? *reinterpret_cast<const int4*>(hist + (int64_t)cc * Ep + 4 * col) : int4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int cc = cc0 + u * G;
          tot4.x += v[u].x; tot4.y += v[u].y; tot4.z += v[u].z; tot4.w += v[u].w;
          if (cc < c) { pre4.x += v[u].x; pre4.y += v[u].y; pre4.z += v[u].z; pre4.w += v[u].w; }
        }
      }
      *reinterpret_cast<int4*>(red + g * Ep + 4 * col) = pre4;
      *reinterpret_cast<int4*>(red + 1024 + g * Ep + 4 * col) = tot4;
    }
  }
  if (tid == 0) errsh = 0;
  // the chunk's slots: wave w takes the contiguous rounds [w rw, (w+1) rw); it
  // classifies them and counts them per expert (same ballots as the count kernel)
  const int64_t t0 = c * tpc;
  const int64_t t1 = (c + 1) * tpc < a.T ? (c + 1) * tpc : a.T;
  const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
  const int rw = (rounds + 3) / 4;
  const int r0 = wave * rw, r1 = (r0 + rw) < rounds ? r0 + rw : rounds;
  constexpr int kKeep = 8;  // classes kept in registers between the two passes
  int keep[kKeep];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();  // cnt zeroed, red written
  auto count_round = [&](int r) -> int {
    uint32_t unused = 0;
    const int cls = classify_wave(a, s0 + (int64_t)r * kWave, s1, unused);
    const uint64_t peers = same_expert(cls, nbits);
    if (peers && (peers & below) == 0) cnt[wave * Ep + cls] += __popcll(peers);
    return cls;
  };
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    if (r0 + i < r1) keep[i] = count_round(r0 + i);
  for (int r = r0 + kKeep; r < r1; ++r) count_round(r);
  // expert totals, their exclusive scan (each thread a run of consecutive
  // experts), and each wave's first row per expert
  const int per = (Ep + 255) / 256;
  int32_t mine[4] = {0, 0, 0, 0};  // per <= 4 (Ep <= 1024)
  int32_t run = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    int32_t t = 0;
    if (e < Ep)
      for (int g = 0; g < G; ++g) t += red[1024 + g * Ep + e];
    mine[i] = t;
    run += t;
  }
  const int32_t incl = block_scan(run, wtot);  // (its barriers also order the cnt updates)
  int32_t ex0 = incl - run;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < a.E) {
      int32_t o = ex0;
      for (int g = 0; g < G; ++g) o += red[g * Ep + e];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        off[w * Ep + e] = o;
        o += cnt[w * Ep + e];
      }
      if (blockIdx.x == 0) {
        counts[e] = mine[i];
        prefix[e] = ex0 + mine[i];
      }
    }
    ex0 += mine[i];
  }
  if (blockIdx.x == 0) {
    uint32_t er = 0;
    for (int cc = tid; cc < nchunks; cc += 256) er |= (uint32_t)chunk_err[cc];
    if (er) atomicOr(&errsh, er);
  }
  // this workgroup's tokens for the copy
  const int64_t nt = t1 - t0;
  const int64_t pt0 = t0 + nt * p / P, pt1 = t0 + nt * (p + 1) / P;
  const int64_t ps0 = pt0 * a.K, ps1 = pt1 * a.K;
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *err_flag = (int32_t)errsh;
  // rows: every wave ranks its rounds in slot order (stable ranks)
  int32_t* o = off + wave * Ep;
  auto place_round = [&](int r, int cls) {
    const int64_t s = s0 + (int64_t)r * kWave + lane;
    const uint64_t peers = same_expert(cls, nbits);
    int row = cls;
    if (peers) {
      const int base = o[cls];
      row = base + __popcll(peers & below);
      if ((peers & below) == 0) o[cls] = base + __popcll(peers);
    }
    if (p == 0 && s < s1) {
      slot2row[s] = row;
      if (peers) row2slot[row] = (int32_t)s;
    }
    if (PERMUTE && s >= ps0 && s < ps1) rows[s - ps0] = peers ? row : -1;
  };
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    if (r0 + i < r1) place_round(r0 + i, keep[i]);
  for (int r = r0 + kKeep; r < r1; ++r) {
    uint32_t unused = 0;
    place_round(r, classify_wave(a, s0 + (int64_t)r * kWave, s1, unused));
  }
  if constexpr (PERMUTE) {
    __syncthreads();
    // copy: thread tid takes vectors tid, tid + 256, ... of the part's token rows
    // (token-major), four loads in flight before their K stores
    const int64_t nv = (pt1 - pt0) * Hv;
    for (int64_t v0 = tid; v0 < nv; v0 += 4 * 256) {
      uint4 val[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t v = v0 + q * 256;
        if (v < nv) val[q] = x[(pt0 + v / Hv) * Hv + v % Hv];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t v = v0 + q * 256;
        if constexpr (COPY == 2) {
          // the 16 lanes of an aligned group hold one 128-column block of a token
          // row (H is a multiple of 128): all of them valid or all past the end
          float f[8];
          if (v < nv) unpack8(val[q], f);
          else
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = 0.f;
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
          if (v >= nv) continue;
          const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
          const uint2 code = make_uint2(
              e4m3x4(__fmul_rn(f[0], inv), __fmul_rn(f[1], inv), __fmul_rn(f[2], inv), __fmul_rn(f[3], inv)),
              e4m3x4(__fmul_rn(f[4], inv), __fmul_rn(f[5], inv), __fmul_rn(f[6], inv), __fmul_rn(f[7], inv)));
          const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
          const int64_t lt = v / Hv, col = v % Hv;
          for (int k = 0; k < a.K; ++k) {
            const int rr = rows[lt * a.K + k];
            if (rr < 0) continue;
            if (ex) ex[(int64_t)rr * Hv + col] = val[q];
            exq[(int64_t)rr * Hv + col] = code;
            if ((col & 15) == 0) exs[(col >> 4) * capacity + rr] = scale;
          }
        } else {
          if (v >= nv) continue;
          const int64_t lt = v / Hv, col = v % Hv;
          for (int k = 0; k < a.K; ++k) {
            const int rr = rows[lt * a.K + k];
            if (rr >= 0) ex[(int64_t)rr * Hv + col] = val[q];
          }
        }
      }
    }
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

RouteGeom route_geom(const moe_shape* s) {
  RouteGeom g;
  g.nslots = s->T * s->K;
  g.Ep = (s->num_experts + 3) / 4 * 4;
  int64_t cmax = 32768 / g.Ep;  // at most 32768 (chunk, expert) counts
  cmax = cmax < 4 ? 4 : (cmax > 256 ? 256 : cmax);
  const int64_t by_slots = (512 + s->K - 1) / s->K, by_count = (s->T + cmax - 1) / cmax;
  g.tpc = by_slots > by_count ? by_slots : by_count;
  g.nchunks = (int)(s->T > 0 ? (s->T + g.tpc - 1) / g.tpc : 0);
  g.rounds = (int)((g.tpc * s->K + kWave - 1) / kWave);
  // about 1024 copying workgroups, each of at least one token
  int64_t P = (1024 + (g.nchunks > 0 ? g.nchunks : 1) - 1) / (g.nchunks > 0 ? g.nchunks : 1);
  g.P = (int)(P < 1 ? 1 : (P > g.tpc ? g.tpc : P));
  return g;
}

size_t route_ws_bytes(const moe_shape* s) {
  const RouteGeom g = route_geom(s);
  const size_t b = ((size_t)g.nchunks * g.Ep + g.nchunks + 1) * sizeof(int32_t);
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

// the routing kernels: counts, then rows and maps, and, given x, the copy of
// every token row to its rows (bf16 into expand_x, and with expand_xq the e4m3
// codes and scales too)
void launch_route(const moe_shape* s, const int32_t* topk_idx, const uint8_t* x_active_mask,
                  int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                  int32_t* err_flag, void* workspace, hipStream_t strm, const void* x = nullptr,
                  void* expand_x = nullptr, uint8_t* expand_xq = nullptr, float* dynamic_scales = nullptr) {
  const RouteGeom g = route_geom(s);
  RouteArgs a{topk_idx, x_active_mask, s->T, s->K, s->num_experts, s->zero_expert_num,
              s->copy_expert_num, s->const_expert_num, s->mask_ndim};
  int32_t* hist = static_cast<int32_t*>(workspace);
  int32_t* cerr = hist + (size_t)g.nchunks * g.Ep;
  int32_t* slot2row = assist;
  int32_t* row2slot = assist + s->T * s->K;
  int nbits = 0;
  while ((1 << nbits) < s->num_experts) ++nbits;
  if (g.nchunks > 0)
    hipLaunchKernelGGL(k_route_count, dim3(g.nchunks), dim3(256), (size_t)4 * g.Ep * sizeof(int32_t), strm, a, hist,
                       cerr, g.tpc, g.rounds, g.Ep, nbits);
  const int copy = (x == nullptr || g.nchunks == 0) ? 0 : (expand_xq ? 2 : 1);
  const int P = copy ? g.P : 1;
  const int64_t part_tokens = (g.tpc + P - 1) / P;
  const size_t lds = ((size_t)8 * g.Ep + 2048 + (copy ? part_tokens * s->K : 0)) * sizeof(int32_t);
  const dim3 grid((unsigned)(g.nchunks > 0 ? (int64_t)g.nchunks * P : 1));
  const uint4* xv = static_cast<const uint4*>(x);
  uint4* ev = static_cast<uint4*>(expand_x);
  uint2* qv = reinterpret_cast<uint2*>(expand_xq);
#define PLACE(C)                                                                                                    \
  hipLaunchKernelGGL(k_route_place<C>, grid, dim3(256), lds, strm, a, hist, cerr, g.tpc, g.nchunks, g.rounds, g.Ep, \
                     nbits, P, expert_token_nums, ep_recv_counts, err_flag, slot2row, row2slot, xv, s->H / 8, ev, qv, \
                     dynamic_scales, s->capacity)
  if (copy == 2) PLACE(2);
  else if (copy == 1) PLACE(1);
  else PLACE(0);
#undef PLACE
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

namespace moe {
// moe_dispatch after its argument checks: routing, then the permute (declared in
// common.hpp for the other dispatch entries)
moe_status dispatch_impl(const moe_shape* s, const void* x, const int32_t* topk_idx,
                         const uint8_t* x_active_mask, void* expand_x, int32_t* assist,
                         int32_t* expert_token_nums, int32_t* ep_recv_counts, int32_t* err_flag,
                         void* workspace, hipStream_t strm) {
  launch_route(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag, workspace, strm, x,
               expand_x);
  return launch_status();
}

size_t dispatch_ws_bytes(const moe_shape* s) { return route_ws_bytes(s); }

moe_status dispatch_check(const moe_shape* s, const void* x, const int32_t* topk_idx, const uint8_t* x_active_mask,
                          void* expand_x, int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                          int32_t* err_flag, void* workspace, size_t ws_bytes) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_dispatch(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag,
                      workspace, ws_bytes);
  if (st != MOE_OK) return st;
  MOE_NEED(x, s->T * s->H);
  MOE_NEED(expand_x, s->capacity * s->H);
  return MOE_OK;
}
}  // namespace moe

extern "C" moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                   const uint8_t* x_active_mask, void* expand_x,
                                   int32_t* assist, int32_t* expert_token_nums,
                                   int32_t* ep_recv_counts, int32_t* err_flag, void* workspace,
                                   size_t ws_bytes, void* stream) {
  const moe_status st = dispatch_check(s, x, topk_idx, x_active_mask, expand_x, assist, expert_token_nums,
                                       ep_recv_counts, err_flag, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  return dispatch_impl(s, x, topk_idx, x_active_mask, expand_x, assist, expert_token_nums, ep_recv_counts,
                       err_flag, workspace, as_stream(stream));
}

extern "C" moe_status moe_dispatch_fp8(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                       const uint8_t* x_active_mask, void* expand_x, uint8_t* expand_xq,
                                       float* dynamic_scales, int32_t* assist, int32_t* expert_token_nums,
                                       int32_t* ep_recv_counts, int32_t* err_flag, void* workspace,
                                       size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->H % 128 != 0) return MOE_ERR_BAD_SHAPE;
  // the scales of all rows are addressed with 32-bit offsets like the fp8 GEMMs'
  if (s->capacity * (s->H / 128) * 4 >= (int64_t)0x7ffffff0) return MOE_ERR_UNSUPPORTED;
  st = check_dispatch(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag,
                      workspace, ws_bytes);
  if (st != MOE_OK) return st;
  MOE_NEED(x, s->T * s->H);
  MOE_NEED(expand_xq, s->capacity * s->H);
  MOE_NEED(dynamic_scales, s->capacity * (s->H / 128));
  launch_route(s, topk_idx, x_active_mask, assist, expert_token_nums, ep_recv_counts, err_flag, workspace,
               as_stream(stream), x, expand_x, expand_xq, dynamic_scales);
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
