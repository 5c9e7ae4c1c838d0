// fp8 e4m3 quantisers of the fp8 FFN path.
//
//  * rows: one scale per (row, 128 consecutive columns), codes = e4m3(x * (448/amax)),
//    scale = amax/448 (both fp32, correctly rounded); an all-zero block gets codes 0
//    and scale 1.  Scales are stored column-block major, (C/128, R), so a GEMM K
//    step reads the scales of consecutive rows from consecutive words.  16 lanes own one block (8 columns each) of four consecutive
//    rows, so the block's amax is a 16-lane butterfly and every load and store is
//    a full vector.
//  * weights: one scale per 128 x 128 block of each expert's (out, in) matrix, same
//    rule; the kernel also writes the codes transposed, so the data-gradient GEMMs
//    read their fp8 weights K-contiguous like the forward ones.  The block scales
//    serve both layouts (the transposed GEMM indexes them with swapped block
//    coordinates).
//
//  * columns per 128 tokens (the weight-gradient operands, which contract over
//    an expert's rows): each expert's rows are cut into 128-row slots from its
//    first row, and each (slot, column) gets one scale, same rule.  The codes
//    are written transposed, column by column, with slot s at codes s*128 ..
//    s*128+127 of every column, so the weight-gradient GEMMs read them
//    K-contiguous; a slot's rows past the expert's end get code 0.
//
// The pages name FP8 only as a precision of the MoE layer performance tests
// (Megatron-LM page, "Added Test Cases"); the block recipe is this library's.
#include "common.hpp"

namespace moe {
namespace {

// 16 lanes own one (row, 128-column) block, 8 columns each, and take the same
// block of kRowsPerGroup consecutive rows, all loads issued before the first
// amax, so each lane keeps several row reads in flight.
constexpr int kRowsPerGroup = 4;

__global__ __launch_bounds__(256) void k_quant_rows_fp8(const uint4* __restrict__ src, int64_t R,
                                                        int64_t C, const int32_t* __restrict__ nrows,
                                                        uint2* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int64_t nb = C / 128;  // blocks per row
  const int64_t g = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // 16-lane group id
  const int sub = threadIdx.x & 15;
  const int64_t rg = g / nb, blk = g % nb;
  int64_t rows = nrows ? (int64_t)*nrows : R;
  if (rows > R) rows = R;
  const int64_t r0 = rg * kRowsPerGroup;
  if (r0 >= rows) return;  // a whole 16-lane group leaves together
  uint4 raw[kRowsPerGroup];
#pragma unroll
  for (int i = 0; i < kRowsPerGroup; ++i)
    if (r0 + i < rows) raw[i] = src[(r0 + i) * (C / 8) + blk * 16 + sub];
#pragma unroll
  for (int i = 0; i < kRowsPerGroup; ++i) {
    const int64_t row = r0 + i;
    float f[8];
    if (row < rows) unpack8(raw[i], f);
    else
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] = 0.f;
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(f[q]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    if (row >= rows) continue;
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
    const uint32_t lo = e4m3x4(__fmul_rn(f[0], inv), __fmul_rn(f[1], inv), __fmul_rn(f[2], inv), __fmul_rn(f[3], inv));
    const uint32_t hi = e4m3x4(__fmul_rn(f[4], inv), __fmul_rn(f[5], inv), __fmul_rn(f[6], inv), __fmul_rn(f[7], inv));
    codes[row * (C / 8) + blk * 16 + sub] = make_uint2(lo, hi);
    if (sub == 0) scales[blk * R + row] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  }
}

// One 256-thread block per (slot, 128 columns).  Thread t loads rows
// 8 (t/16) .. +7, columns 8 (t%16) .. +7; the column amax is a reduction over
// the 16 row groups (two shuffles in a wave, then LDS across the four waves).
// The codes go through LDS transposed (column-major, 144-byte pitch) and leave
// as 16-byte stores, eight lanes per column.
__global__ __launch_bounds__(256) void k_quant_cols_fp8(const uint4* __restrict__ src, int64_t D, int E,
                                                        const int32_t* __restrict__ prefix, int64_t ldc,
                                                        uint8_t* __restrict__ codes_t,
                                                        float* __restrict__ scales) {
  const int64_t nb = D / 128;
  const int64_t slot = blockIdx.x / nb, cb = blockIdx.x % nb;
  const int e = find_expert<128>(prefix, E, slot);
  const int64_t p0 = e ? prefix[e - 1] : 0, p1 = prefix[e];
  const int64_t row0 = p0 + (slot - (p0 / 128 + e)) * 128;
  if (row0 >= p1) return;  // a slot no expert row falls in: never read
  const int rows = (int)((p1 - row0) < 128 ? (p1 - row0) : 128);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, c = t & 15, rg = t >> 4;
  float v[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * rg + i;
    if (r < rows) unpack8(src[(row0 + r) * (D / 8) + cb * 16 + c], v[i]);
    else
#pragma unroll
      for (int q = 0; q < 8; ++q) v[i][q] = 0.f;
  }
  __shared__ float red[4][128];
  __shared__ __attribute__((aligned(16))) uint8_t ct[128 * 144];
  float m[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i][q]));
    a = fmaxf(a, __shfl_xor(a, 16, 64));
    a = fmaxf(a, __shfl_xor(a, 32, 64));
    m[q] = a;
  }
  if (lane < 16)
#pragma unroll
    for (int q = 0; q < 8; ++q) red[wave][8 * c + q] = m[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int col = 8 * c + q;
    const float amax = fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
    const uint32_t lo = e4m3x4(__fmul_rn(v[0][q], inv), __fmul_rn(v[1][q], inv), __fmul_rn(v[2][q], inv),
                               __fmul_rn(v[3][q], inv));
    const uint32_t hi = e4m3x4(__fmul_rn(v[4][q], inv), __fmul_rn(v[5][q], inv), __fmul_rn(v[6][q], inv),
                               __fmul_rn(v[7][q], inv));
    *reinterpret_cast<uint2*>(ct + col * 144 + 8 * rg) = make_uint2(lo, hi);
    if (rg == 0) scales[slot * D + cb * 128 + col] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = t + 256 * k, col = idx >> 3, ch = idx & 7;
    *reinterpret_cast<uint4*>(codes_t + (cb * 128 + col) * ldc + slot * 128 + ch * 16) =
        *reinterpret_cast<const uint4*>(ct + col * 144 + ch * 16);
  }
}

// One 256-thread block per 128 x 128 weight block.  Thread t owns rows
// t/16 + 16j (j < 8), columns 8*(t%16) .. +7.
__global__ __launch_bounds__(256) void k_quant_weights_fp8(const uint4* __restrict__ w, int64_t N,
                                                           int64_t Kd, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ codes_t,
                                                           float* __restrict__ scales) {
  __shared__ float wmax[4];
  __shared__ __attribute__((aligned(16))) uint8_t tr[128 * 144];  // transposed tile, padded rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nbn = N / 128, nbk = Kd / 128;
  const int64_t e = blockIdx.x / (nbn * nbk);
  const int64_t rem = blockIdx.x % (nbn * nbk);
  const int64_t bn = rem / nbk, bk = rem % nbk;
  const int64_t n0 = bn * 128, k0 = bk * 128;
  const int c8 = (tid & 15) * 8;
  float f[8][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 4) + 16 * j;
    unpack8(w[((e * N + n0 + r) * Kd + k0 + c8) / 8], f[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[j][i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 4) + 16 * j;
    const uint2 pk = make_uint2(
        e4m3x4(__fmul_rn(f[j][0], inv), __fmul_rn(f[j][1], inv), __fmul_rn(f[j][2], inv), __fmul_rn(f[j][3], inv)),
        e4m3x4(__fmul_rn(f[j][4], inv), __fmul_rn(f[j][5], inv), __fmul_rn(f[j][6], inv), __fmul_rn(f[j][7], inv)));
    *reinterpret_cast<uint2*>(codes + (e * N + n0 + r) * Kd + k0 + c8) = pk;
    if (codes_t) {
#pragma unroll
      for (int i = 0; i < 8; ++i) tr[(c8 + i) * 144 + r] = (uint8_t)((i < 4 ? pk.x : pk.y) >> (8 * (i & 3)));
    }
  }
  if (tid == 0) scales[(e * nbn + bn) * nbk + bk] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (codes_t) {
    __syncthreads();
    // row c of the transposed block = column c of the block: 128 bytes = 8 x 16
    for (int v = tid; v < 128 * 8; v += 256) {
      const int c = v >> 3, part = (v & 7) * 16;
      *reinterpret_cast<uint4*>(codes_t + (e * Kd + k0 + c) * N + n0 + part) =
          *reinterpret_cast<const uint4*>(tr + c * 144 + part);
    }
  }
}

// int8 rows (the per-token requantisation of h on the int8 path, and int8
// weights with one scale per output channel): one wave per row, an amax pass
// and a code pass over 16-byte vectors, codes clamp(rint(v * (127/amax)),
// -127, 127), scale amax/127 (all-zero: codes 0, scale 1).
__global__ __launch_bounds__(256) void k_quant_rows_int8(const uint4* __restrict__ src, int64_t R, int64_t C,
                                                         const int32_t* __restrict__ nrows,
                                                         uint2* __restrict__ codes, float* __restrict__ scales) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  int64_t rows = nrows ? (int64_t)*nrows : R;
  if (rows > R) rows = R;
  if (r >= rows) return;  // a whole wave leaves together
  const int64_t Cv = C / 8;
  const uint4* row = src + r * Cv;
  float m = 0.f;
  for (int64_t v = lane; v < Cv; v += 64) {
    float f[8];
    unpack8(row[v], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  }
  m = wave_max64(m);
  const float inv = m > 0.f ? __fdiv_rn(127.0f, m) : 0.f;
  for (int64_t v = lane; v < Cv; v += 64) {
    float f[8];
    unpack8(row[v], f);
    codes[r * Cv + v] = make_uint2(i8x4(f[0], f[1], f[2], f[3], inv), i8x4(f[4], f[5], f[6], f[7], inv));
  }
  if (lane == 0) scales[r] = m > 0.f ? __fdiv_rn(m, 127.0f) : 1.0f;
}

// rows: 4 lanes per 32-value block, 8 values each (one 16-byte load, one 8-byte store)
__global__ __launch_bounds__(256) void k_quant_rows_mx(const uint4* __restrict__ src, int64_t R, int64_t C,
                                                       const int32_t* __restrict__ nrows, uint2* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // vector of 8 values
  const int64_t Cv = C / 8;
  const int64_t r = i / Cv;
  int64_t rows = nrows ? (int64_t)*nrows : R;
  if (rows > R) rows = R;
  // C is a multiple of 32, so the 4 lanes of a block are in one row and leave together
  if (r >= rows) return;
  float f[8];
  unpack8(src[i], f);
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(f[q]));
  m = fmaxf(m, __shfl_xor(m, 1, 4));
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  const int e = mx_exponent(m);
  const float inv = mx_inv(e);
  codes[i] = make_uint2(e4m3x4(__fmul_rn(f[0], inv), __fmul_rn(f[1], inv), __fmul_rn(f[2], inv), __fmul_rn(f[3], inv)),
                        e4m3x4(__fmul_rn(f[4], inv), __fmul_rn(f[5], inv), __fmul_rn(f[6], inv), __fmul_rn(f[7], inv)));
  // scale layout: the four 32-value blocks of one 128-value column block of one
  // row are one 4-byte word, words ordered (column block, row), so a GEMM K step
  // reads the scales of consecutive rows from consecutive words
  if ((i & 3) == 0) {
    const int64_t b = (i % Cv) / 4;  // 32-block within the row
    scales[((b / 4) * R + r) * 4 + (b & 3)] = (uint8_t)(e + 127);
  }
}

// transposed weights: one workgroup per (expert, 32 rows n, 128 columns k) of W
// (E, N, K); thread t takes column k = t/2 and rows 16 (t%2) .. +15 of the tile,
// writes the 16 codes of W^T row k (the 32-block n0 .. n0+31 is shared with its
// neighbour lane) and the block's scale
__global__ __launch_bounds__(256) void k_quant_weights_mx_t(const uint4* __restrict__ w, int64_t E, int64_t N,
                                                            int64_t K, uint8_t* __restrict__ codes_t,
                                                            uint8_t* __restrict__ scales_t) {
  const int64_t nbk = K / 128, nbn = N / 32;
  const int64_t b = blockIdx.x;
  const int64_t e = b / (nbn * nbk), rem = b % (nbn * nbk);
  const int64_t n0 = (rem / nbk) * 32, k0 = (rem % nbk) * 128;
  const int t = threadIdx.x;
  __shared__ __attribute__((aligned(16))) bf16_t tile[32][136];
  // 32 rows x 16 vectors of 8: two per thread
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = t + 256 * j, row = v / 16, c8 = (v % 16) * 8;
    *reinterpret_cast<uint4*>(&tile[row][c8]) = w[((e * N + n0 + row) * K + k0 + c8) / 8];
  }
  __syncthreads();
  const int col = t >> 1, h = t & 1;
  float f[16];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[i] = bf2f(tile[16 * h + i][col]);
    m = fmaxf(m, fabsf(f[i]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  const int ex = mx_exponent(m);
  const float inv = mx_inv(ex);
  uint32_t wd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wd[q] = e4m3x4(__fmul_rn(f[4 * q], inv), __fmul_rn(f[4 * q + 1], inv), __fmul_rn(f[4 * q + 2], inv),
                   __fmul_rn(f[4 * q + 3], inv));
  const int64_t rowt = e * K + k0 + col;  // row of W^T
  *reinterpret_cast<uint4*>(codes_t + rowt * N + n0 + 16 * h) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  // words ordered (128-column block of W^T, row of W^T over all experts), as the
  // row quantiser orders them for the E*K rows of W^T
  if (h == 0) {
    const int64_t bn = n0 / 32;
    scales_t[((bn / 4) * (E * K) + rowt) * 4 + (bn & 3)] = (uint8_t)(ex + 127);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_quant_rows_fp8(int64_t R, int64_t C, const void* src,
                                         const int32_t* nrows, uint8_t* codes, float* scales,
                                         void* stream) {
  if (R < 0 || C <= 0 || C % 128 != 0 || R * (C / 128) > ((int64_t)1 << 35))
    return MOE_ERR_BAD_SHAPE;
  if (R == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_NULL_ARG;
  const int64_t groups = (R + kRowsPerGroup - 1) / kRowsPerGroup * (C / 128);  // 16 lanes each
  const int64_t blocks = (groups * 16 + 255) / 256;
  hipLaunchKernelGGL(k_quant_rows_fp8, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), R, C, nrows, reinterpret_cast<uint2*>(codes),
                     scales);
  return launch_status();
}

extern "C" moe_status moe_quant_cols_fp8(int64_t capacity, int64_t D, int32_t num_experts,
                                         const void* src, const int32_t* ep_recv_counts,
                                         uint8_t* codes_t, float* scales, void* stream) {
  if (capacity < 0 || D <= 0 || D % 128 != 0 || num_experts < 1) return MOE_ERR_BAD_SHAPE;
  const int64_t slots = capacity / 128 + num_experts;
  const int64_t blocks = slots * (D / 128);
  if (blocks > 0x7fffffff || D * slots * 128 >= ((int64_t)1 << 40)) return MOE_ERR_BAD_SHAPE;
  if (!ep_recv_counts) return MOE_ERR_NULL_ARG;
  if (capacity == 0) return MOE_OK;
  if (!src || !codes_t || !scales) return MOE_ERR_NULL_ARG;
  hipLaunchKernelGGL(k_quant_cols_fp8, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), D, (int)num_experts, ep_recv_counts, slots * 128,
                     codes_t, scales);
  return launch_status();
}

extern "C" moe_status moe_quantize_weights_fp8(int64_t E, int64_t N, int64_t Kdim, const void* w,
                                               uint8_t* codes, uint8_t* codes_t, float* scales,
                                               void* stream) {
  if (E <= 0 || N <= 0 || Kdim <= 0 || N % 128 != 0 || Kdim % 128 != 0) return MOE_ERR_BAD_SHAPE;
  if (E * N * Kdim >= ((int64_t)1 << 40)) return MOE_ERR_BAD_SHAPE;
  if (!w || !codes || !scales) return MOE_ERR_NULL_ARG;
  const int64_t blocks = E * (N / 128) * (Kdim / 128);
  if (blocks > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_quant_weights_fp8, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(w), N, Kdim, codes, codes_t, scales);
  return launch_status();
}

extern "C" moe_status moe_quant_rows_int8(int64_t R, int64_t C, const void* src, const int32_t* nrows,
                                          int8_t* codes, float* scales, void* stream) {
  if (R < 0 || C <= 0 || C % 8 != 0 || R * C >= ((int64_t)1 << 40)) return MOE_ERR_BAD_SHAPE;
  if (R == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_NULL_ARG;
  const int64_t blocks = (R + 3) / 4;
  if (blocks > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_quant_rows_int8, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), R, C, nrows, reinterpret_cast<uint2*>(codes), scales);
  return launch_status();
}

extern "C" moe_status moe_quant_rows_mx(int64_t R, int64_t C, const void* src, const int32_t* nrows,
                                        uint8_t* codes, uint8_t* scales, void* stream) {
  if (R < 0 || C <= 0 || C % 32 != 0 || R * C >= ((int64_t)1 << 40)) return MOE_ERR_BAD_SHAPE;
  if (R == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_NULL_ARG;
  const int64_t blocks = (R * (C / 8) + 255) / 256;
  if (blocks > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_quant_rows_mx, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), R, C, nrows, reinterpret_cast<uint2*>(codes), scales);
  return launch_status();
}

extern "C" moe_status moe_quantize_weights_mx(int64_t E, int64_t N, int64_t K, const void* w, uint8_t* codes,
                                              uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                                              void* stream) {
  if (E <= 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_BAD_SHAPE;
  if (E * N * K >= ((int64_t)1 << 40)) return MOE_ERR_BAD_SHAPE;
  if (!w || !codes || !scales) return MOE_ERR_NULL_ARG;
  if (!codes_t != !scales_t) return MOE_ERR_NULL_ARG;
  moe_status st = moe_quant_rows_mx(E * N, K, w, nullptr, codes, scales, stream);
  if (st != MOE_OK || !codes_t) return st;
  const int64_t blocks = E * (N / 32) * (K / 128);
  if (blocks > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_quant_weights_mx_t, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(w), E, N, K, codes_t, scales_t);
  return launch_status();
}
