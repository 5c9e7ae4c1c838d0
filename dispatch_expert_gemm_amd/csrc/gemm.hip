// Grouped GEMMs of the expert SwiGLU FFN, forward and backward, on gfx950 MFMA.
//
// The expert FFN (SwiGLU with intermediate size F: the --ffn_dim of the
// Triton-distributed ep_moe_fused benchmark page) runs as one grouped GEMM per
// projection over the expert-sorted rows built by dispatch.  Six GEMM kinds:
//
//   mode               C (M x N)            A (M x K)             B (N x K)
//   GATE_UP_FWD        [G|U] rows x F       expand_x  (K-contig)  Wg_e, Wu_e (K-contig)
//   DOWN_FWD           y rows x H           h_act     (K-contig)  Wd_e       (K-contig)
//   DOWN_BWD_DATA      dH rows x F          grad_y    (K-contig)  Wd_e       (N-contig)
//   GATE_UP_BWD_DATA   dX rows x H          grad_gu   (K-contig)  [Wg_e;Wu_e](N-contig)
//   DOWN_BWD_W         dWd_e H x F          grad_y    (M-contig)  h_act      (N-contig)
//   GATE_UP_BWD_W      [dWg_e;dWu_e] 2F x H grad_gu   (M-contig)  expand_x   (N-contig)
//
// The first four are grouped over M (each expert owns a contiguous row range of
// the expanded buffers); the last two are grouped over K (the contraction runs
// over the expert's rows, which may be none).
//
// Tiling: 128 x 128 output tile per 256-thread workgroup, four waves in a 2 x 2
// arrangement, each wave 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16 tiles; K step
// 32 staged through double-buffered LDS (one barrier per step), the next step's
// global loads in flight in registers while the current step's MFMAs issue.  In
// LDS both operands are stored K-contiguous (row pitch 40 elements), so every
// MFMA operand is one 16-byte LDS read; operands that are K-strided in memory
// are transposed on their way into LDS.
//
// Expert counts stay on the device: the grid covers floor(capacity/128) + E row
// tiles per column tile, and each workgroup finds its expert from the prefix
// counts with one wave ballot (expert e owns row-tile slots starting at
// prefix[e-1]/128 + e); surplus workgroups exit at once.  Workgroup ids are
// remapped so that consecutive tiles (sharing A rows and expert weights) land on
// the same XCD and its L2.
#include "common.hpp"

namespace moe {
namespace {

enum Mode : int {
  GATE_UP_FWD = 0,
  DOWN_FWD = 1,
  DOWN_BWD_DATA = 2,
  GATE_UP_BWD_DATA = 3,
  DOWN_BWD_W = 4,
  GATE_UP_BWD_W = 5
};

constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;
constexpr int kThreads = 256;

struct GemmArgs {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B0;
  const bf16_t* B1;
  int64_t ldb;
  int64_t bstride;  // elements between consecutive experts' B0/B1 matrices
  const int32_t* prefix;
  int E;
  int64_t M, N, Kd, F;
  int64_t n_tiles, m_tiles, tiles;
  bf16_t* C0;
  bf16_t* C1;
  const bf16_t* aux;
  float* W0;
  float* W1;
};

__device__ __forceinline__ int find_expert(const int32_t* __restrict__ prefix, int E, int64_t mt) {
  const int lane = threadIdx.x & 63;
  int found = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    bool le = false;
    if (e < E) {
      const int64_t P = e ? prefix[e - 1] : 0;
      le = (P / BM + e) <= mt;
    }
    const uint64_t m = __ballot(le);
    if (m) found = base + 63 - __clzll(m);
    if (m != ~0ull) break;
  }
  return found;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void k_gemm(GemmArgs g) {
  constexpr bool KGROUP = MODE == DOWN_BWD_W || MODE == GATE_UP_BWD_W;
  constexpr bool B_KC = MODE == GATE_UP_FWD || MODE == DOWN_FWD;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t nb = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= g.tiles) return;

  int e;
  int64_t row0, n0, kbeg, kend;
  int rows_valid;
  if constexpr (!KGROUP) {
    const int64_t mt = logical / g.n_tiles;
    const int64_t nt = logical % g.n_tiles;
    e = find_expert(g.prefix, g.E, mt);
    const int64_t p0 = e ? g.prefix[e - 1] : 0, p1 = g.prefix[e];
    row0 = p0 + (mt - (p0 / BM + e)) * BM;
    if (row0 >= p1) return;
    rows_valid = (int)((p1 - row0) < BM ? (p1 - row0) : BM);
    n0 = nt * (MODE == GATE_UP_FWD ? BN / 2 : BN);
    kbeg = 0;
    kend = g.Kd;
  } else {
    const int64_t per = g.m_tiles * g.n_tiles;
    e = (int)(logical / per);
    const int64_t rem = logical % per;
    row0 = (rem / g.n_tiles) * BM;  // first output row (weight row)
    n0 = (rem % g.n_tiles) * BN;
    kbeg = e ? g.prefix[e - 1] : 0;
    kend = g.prefix[e];
    rows_valid = (int)((g.M - row0) < BM ? (g.M - row0) : BM);
  }
  const int64_t klen = kend - kbeg;

  // ---- global -> register loads of one K step
  uint4 ra[2], rb[2];
  auto load_a = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + kThreads * j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (!KGROUP) {
        const int r = i >> 2, c = (i & 3) * 8;
        const int64_t src = row0 + (r < rows_valid ? r : rows_valid - 1);
        if (k0 + c < kend) v = *reinterpret_cast<const uint4*>(g.A + src * g.lda + k0 + c);
      } else {
        const int kr = i >> 4, x8 = (i & 15) * 8;
        if (k0 + kr < klen && row0 + x8 < g.M)
          v = *reinterpret_cast<const uint4*>(g.A + (kbeg + k0 + kr) * g.lda + row0 + x8);
      }
      ra[j] = v;
    }
  };
  auto load_b = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + kThreads * j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if constexpr (B_KC) {
        const int r = i >> 2, c = (i & 3) * 8;
        if (k0 + c < kend) {
          const bf16_t* base;
          int64_t n;
          if constexpr (MODE == GATE_UP_FWD) {
            base = (r < BN / 2 ? g.B0 : g.B1) + (int64_t)e * g.bstride;
            n = n0 + (r & (BN / 2 - 1));
            if (n >= g.F) n = g.F - 1;
          } else {
            base = g.B0 + (int64_t)e * g.bstride;
            n = n0 + r;
            if (n >= g.N) n = g.N - 1;
          }
          v = *reinterpret_cast<const uint4*>(base + n * g.ldb + k0 + c);
        }
      } else {
        const int kr = i >> 4, x8 = (i & 15) * 8;
        const int64_t k = k0 + kr;
        if (k < klen && n0 + x8 < g.N) {
          const bf16_t* p;
          if constexpr (MODE == DOWN_BWD_DATA) {
            p = g.B0 + (int64_t)e * g.bstride + k * g.ldb;
          } else if constexpr (MODE == GATE_UP_BWD_DATA) {
            p = (k < g.F ? g.B0 + k * g.ldb : g.B1 + (k - g.F) * g.ldb) + (int64_t)e * g.bstride;
          } else {
            p = g.B0 + (kbeg + k) * g.ldb;
          }
          v = *reinterpret_cast<const uint4*>(p + n0 + x8);
        }
      }
      rb[j] = v;
    }
  };
  // ---- register -> LDS (K-contiguous rows)
  auto store_kc = [&](bf16_t* S, const uint4* r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + kThreads * j;
      *reinterpret_cast<uint4*>(S + (i >> 2) * LDK + (i & 3) * 8) = r[j];
    }
  };
  auto store_tr = [&](bf16_t* S, const uint4* r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + kThreads * j;
      const int kr = i >> 4, x8 = (i & 15) * 8;
      const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        S[(x8 + 2 * q) * LDK + kr] = (bf16_t)(w[q] & 0xffffu);
        S[(x8 + 2 * q + 1) * LDK + kr] = (bf16_t)(w[q] >> 16);
      }
    }
  };
  auto store_a = [&](int s) {
    if constexpr (!KGROUP) store_kc(As[s], ra);
    else store_tr(As[s], ra);
  };
  auto store_b = [&](int s) {
    if constexpr (B_KC) store_kc(Bs[s], rb);
    else store_tr(Bs[s], rb);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto brow = [&](int j) -> int {
    if constexpr (MODE == GATE_UP_FWD) return j * (BN / 2) + wn * 32;
    else return wn * 64 + j * 32;
  };

  const int64_t nk = (klen + BK - 1) / BK;
  if (nk > 0) {
    load_a(0);
    load_b(0);
    store_a(0);
    store_b(0);
    __syncthreads();
  }
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int s = (int)(kt & 1);
    if (kt + 1 < nk) {
      load_a((kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
    const bf16_t* as = As[s];
    const bf16_t* bs = Bs[s];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ko = kk * 16 + (lane >> 5) * 8;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(as + (wm * 64 + i * 32 + (lane & 31)) * LDK + ko);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(bs + (brow(j) + (lane & 31)) * LDK + ko);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_a(s ^ 1);
      store_b(s ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue.  acc[i][j][r] holds C(m, n) with
  //   m = wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,  n = brow(j) + lane%32
  const int ln = lane & 31, lh = lane >> 5;
  if constexpr (MODE == GATE_UP_FWD) {
    const int64_t f = n0 + wn * 32 + ln;
    if (f < g.F) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
          if (m < rows_valid) {
            const float gv = acc[i][0][r], uv = acc[i][1][r];
            const int64_t row = row0 + m;
            g.C0[row * g.F + f] = (bf16_t)f2bf(silu_f(gv) * uv);
            g.C1[row * 2 * g.F + f] = (bf16_t)f2bf(gv);
            g.C1[row * 2 * g.F + g.F + f] = (bf16_t)f2bf(uv);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + brow(j) + ln;
      if (n >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * 64 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
          if (m >= rows_valid) continue;
          const float c = acc[i][j][r];
          if constexpr (MODE == DOWN_FWD || MODE == GATE_UP_BWD_DATA) {
            g.C0[(row0 + m) * g.N + n] = (bf16_t)f2bf(c);
          } else if constexpr (MODE == DOWN_BWD_DATA) {
            const int64_t row = row0 + m;
            const float gv = bf2f(g.aux[row * 2 * g.F + n]);
            const float uv = bf2f(g.aux[row * 2 * g.F + g.F + n]);
            const float sg = 1.0f / (1.0f + __expf(-gv));
            const float dg = c * uv * sg * (1.0f + gv * (1.0f - sg));
            const float du = c * (gv * sg);
            g.C0[row * 2 * g.F + n] = (bf16_t)f2bf(dg);
            g.C0[row * 2 * g.F + g.F + n] = (bf16_t)f2bf(du);
          } else if constexpr (MODE == DOWN_BWD_W) {
            g.W0[(int64_t)e * g.M * g.N + (row0 + m) * g.N + n] = c;
          } else {  // GATE_UP_BWD_W: rows [0, F) -> dWg, [F, 2F) -> dWu
            const int64_t jrow = row0 + m;
            if (jrow < g.F) g.W0[(int64_t)e * g.F * g.N + jrow * g.N + n] = c;
            else g.W1[(int64_t)e * g.F * g.N + (jrow - g.F) * g.N + n] = c;
          }
        }
    }
  }
}

template <int MODE>
moe_status launch(GemmArgs& g, const moe_shape* s, hipStream_t strm) {
  if (MODE == DOWN_BWD_W || MODE == GATE_UP_BWD_W) {
    g.m_tiles = (g.M + BM - 1) / BM;
    g.tiles = (int64_t)s->num_experts * g.m_tiles * g.n_tiles;
  } else {
    g.m_tiles = s->capacity / BM + s->num_experts;
    g.tiles = g.m_tiles * g.n_tiles;
  }
  if (g.tiles == 0) return MOE_OK;
  const int64_t grid = (g.tiles + 7) / 8 * 8;
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_gemm<MODE>, dim3((unsigned)grid), dim3(kThreads), 0, strm, g);
  return launch_status();
}

GemmArgs base_args(const moe_shape* s, const int32_t* prefix) {
  GemmArgs g{};
  g.prefix = prefix;
  g.E = s->num_experts;
  g.F = s->F;
  return g;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_ffn_gate_up_fwd(const moe_shape* s, const void* expand_x,
                                          const void* w_gate, const void* w_up,
                                          const int32_t* ep_recv_counts, void* gate_up_save,
                                          void* h_act, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!expand_x || !gate_up_save || !h_act) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(expand_x);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_gate);
  g.B1 = static_cast<const bf16_t*>(w_up);
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->F;
  g.Kd = s->H;
  g.n_tiles = (s->F + BN / 2 - 1) / (BN / 2);
  g.C0 = static_cast<bf16_t*>(h_act);
  g.C1 = static_cast<bf16_t*>(gate_up_save);
  return launch<GATE_UP_FWD>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_fwd(const moe_shape* s, const void* h_act, const void* w_down,
                                       const int32_t* ep_recv_counts, void* y, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!h_act || !y) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(h_act);
  g.lda = s->F;
  g.B0 = static_cast<const bf16_t*>(w_down);
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->H;
  g.Kd = s->F;
  g.n_tiles = (s->H + BN - 1) / BN;
  g.C0 = static_cast<bf16_t*>(y);
  return launch<DOWN_FWD>(g, s, as_stream(stream));
}

extern "C" moe_status moe_grouped_ffn(const moe_shape* s, const void* expand_x,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const int32_t* ep_recv_counts, void* gate_up_save,
                                      void* h_act, void* y, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!expand_x || !gate_up_save || !h_act || !y)) return MOE_ERR_NULL_ARG;
  st = moe_ffn_gate_up_fwd(s, expand_x, w_gate, w_up, ep_recv_counts, gate_up_save, h_act,
                           stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_fwd(s, h_act, w_down, ep_recv_counts, y, stream);
}

extern "C" moe_status moe_ffn_down_bwd_data(const moe_shape* s, const void* grad_y,
                                            const void* w_down, const void* gate_up_save,
                                            const int32_t* ep_recv_counts, void* grad_gate_up,
                                            void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_down || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!grad_y || !gate_up_save || !grad_gate_up) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_y);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(w_down);
  g.ldb = s->F;
  g.bstride = s->H * s->F;
  g.N = s->F;
  g.Kd = s->H;
  g.n_tiles = (s->F + BN - 1) / BN;
  g.aux = static_cast<const bf16_t*>(gate_up_save);
  g.C0 = static_cast<bf16_t*>(grad_gate_up);
  return launch<DOWN_BWD_DATA>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_down_bwd_weight(const moe_shape* s, const void* grad_y,
                                              const void* h_act, const int32_t* ep_recv_counts,
                                              float* grad_w_down, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_down) return MOE_ERR_NULL_ARG;
  MOE_NEED(grad_y, s->capacity * s->H);
  MOE_NEED(h_act, s->capacity * s->F);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_y);
  g.lda = s->H;
  g.B0 = static_cast<const bf16_t*>(h_act);
  g.ldb = s->F;
  g.M = s->H;
  g.N = s->F;
  g.n_tiles = (s->F + BN - 1) / BN;
  g.W0 = grad_w_down;
  return launch<DOWN_BWD_W>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_data(const moe_shape* s, const void* grad_gate_up,
                                               const void* w_gate, const void* w_up,
                                               const int32_t* ep_recv_counts,
                                               void* grad_expand_x, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (s->capacity == 0) return MOE_OK;
  if (!grad_gate_up || !grad_expand_x) return MOE_ERR_NULL_ARG;
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_gate_up);
  g.lda = 2 * s->F;
  g.B0 = static_cast<const bf16_t*>(w_gate);
  g.B1 = static_cast<const bf16_t*>(w_up);
  g.ldb = s->H;
  g.bstride = s->F * s->H;
  g.N = s->H;
  g.Kd = 2 * s->F;
  g.n_tiles = (s->H + BN - 1) / BN;
  g.C0 = static_cast<bf16_t*>(grad_expand_x);
  return launch<GATE_UP_BWD_DATA>(g, s, as_stream(stream));
}

extern "C" moe_status moe_ffn_gate_up_bwd_weight(const moe_shape* s, const void* grad_gate_up,
                                                 const void* expand_x,
                                                 const int32_t* ep_recv_counts,
                                                 float* grad_w_gate, float* grad_w_up,
                                                 void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!ep_recv_counts || !grad_w_gate || !grad_w_up) return MOE_ERR_NULL_ARG;
  MOE_NEED(grad_gate_up, s->capacity * 2 * s->F);
  MOE_NEED(expand_x, s->capacity * s->H);
  GemmArgs g = base_args(s, ep_recv_counts);
  g.A = static_cast<const bf16_t*>(grad_gate_up);
  g.lda = 2 * s->F;
  g.B0 = static_cast<const bf16_t*>(expand_x);
  g.ldb = s->H;
  g.M = 2 * s->F;
  g.N = s->H;
  g.n_tiles = (s->H + BN - 1) / BN;
  g.W0 = grad_w_gate;
  g.W1 = grad_w_up;
  return launch<GATE_UP_BWD_W>(g, s, as_stream(stream));
}

extern "C" moe_status moe_grouped_ffn_bwd(const moe_shape* s, const void* grad_y,
                                          const void* expand_x, const void* gate_up_save,
                                          const void* h_act, const void* w_gate, const void* w_up,
                                          const void* w_down, const int32_t* ep_recv_counts,
                                          void* grad_gate_up, void* grad_expand_x,
                                          float* grad_w_gate, float* grad_w_up,
                                          float* grad_w_down, void* stream) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !w_down || !ep_recv_counts || !grad_w_gate || !grad_w_up ||
      !grad_w_down)
    return MOE_ERR_NULL_ARG;
  if (s->capacity > 0 && (!grad_y || !expand_x || !gate_up_save || !h_act || !grad_gate_up ||
                          !grad_expand_x))
    return MOE_ERR_NULL_ARG;
  st = moe_ffn_down_bwd_data(s, grad_y, w_down, gate_up_save, ep_recv_counts, grad_gate_up,
                             stream);
  if (st != MOE_OK) return st;
  st = moe_ffn_down_bwd_weight(s, grad_y, h_act, ep_recv_counts, grad_w_down, stream);
  if (st != MOE_OK) return st;
  st = moe_ffn_gate_up_bwd_data(s, grad_gate_up, w_gate, w_up, ep_recv_counts, grad_expand_x,
                                stream);
  if (st != MOE_OK) return st;
  return moe_ffn_gate_up_bwd_weight(s, grad_gate_up, expand_x, ep_recv_counts, grad_w_gate,
                                    grad_w_up, stream);
}
