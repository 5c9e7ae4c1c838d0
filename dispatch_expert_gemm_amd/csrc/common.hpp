// Shared helpers of the libmoe HIP sources: bf16 storage conversions, vector
// types, host-side argument validation and launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // storage of an IEEE bfloat16

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Exact widening of a bf16 bit pattern.
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// Narrowing float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> one 32-bit word of two bf16 (lo in the low half).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// Two floats -> two bf16 (lo in the low half) with the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack the 8 bf16 of a 16-byte vector to floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 v;
  v.x = pack_bf2(f[0], f[1]); v.y = pack_bf2(f[2], f[3]);
  v.z = pack_bf2(f[4], f[5]); v.w = pack_bf2(f[6], f[7]);
  return v;
}

// float -> OCP fp8 e4m3 code (1-4-3, bias 7, largest finite 448, S.1111.111 = NaN),
// round to nearest with ties to the even code, saturating at +-448; NaN gives
// 0x7F; the sign of zero is kept.  Written from the format definition: below
// 2^-6 the code is the subnormal count m * 2^-9, above it the 23-bit fp32
// mantissa is rounded to 3 bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  const float af = __uint_as_float(a);
  if (af >= 448.0f) return sign | 0x7eu;
  const int e = (int)(a >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    code = (uint32_t)rintf(af * 512.0f);  // exact product, rint = ties to even
  } else {
    const uint32_t mant = a & 0x7fffffu;
    uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    uint32_t ee = (uint32_t)(e + 7);
    if (q == 8u) {
      q = 0u;
      ++ee;
    }
    code = (ee << 3) | q;
  }
  return sign | code;
}

// Four codes packed into a word (byte i = code of the i-th value), through the
// hardware conversion (v_cvt_pk_fp8_f32: OCP e4m3 on gfx950, round to nearest
// even) of the inputs clamped to +-448.  That agrees with f32_to_e4m3 on every
// one of the 2^32 float inputs except NaN, which the clamp turns into -448
// (compared exhaustively on MI355X); a word with a NaN input takes
// f32_to_e4m3.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), (int)w, true);
  if (a != a || b != b || c != c || d != d)
    w = f32_to_e4m3(a) | f32_to_e4m3(b) << 8 | f32_to_e4m3(c) << 16 | f32_to_e4m3(d) << 24;
  return w;
}

// Four int8 codes packed into a word: clamp(rint(v * inv), -127, 127) each (the
// product rounded to fp32 first, ties to even), byte i = the i-th value.
__device__ __forceinline__ uint32_t i8x4(float a, float b, float c, float d, float inv) {
  auto q = [inv](float v) { return (uint32_t)(int)fminf(fmaxf(rintf(__fmul_rn(v, inv)), -127.0f), 127.0f) & 0xffu; };
  return q(a) | q(b) << 8 | q(c) << 16 | q(d) << 24;
}

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Microscaled e4m3 (E8M0 scale per 32 values): the scale is the smallest power of
// two 2^e with amax / 2^e <= 448; with amax = M * 2^E (1 <= M < 2) that is e = E - 8,
// or E - 7 when M > 1.75 (mantissa bits above 0x600000), clamped to [-127, 127]
// (zero and subnormal amax give -127).  Scale byte e + 127.
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int biased = (int)(b >> 23);
  int e = biased - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  if (biased == 0) e = -127;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^-e as a float (e in [-126, 126]; -127 gives 2^127)
__device__ __forceinline__ float mx_inv(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

constexpr int kWave = 64;

// ----------------------------------------------------------------------------- host side

// Expert of row-tile slot mt when expert e owns BM-row slots starting at
// prefix[e-1]/BM + e (prefix = inclusive row counts): the largest e whose first
// slot is <= mt, by one wave ballot per 64 experts.  Every lane of the wave
// gets the same answer.
template <int BM>
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

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t e_total(const moe_shape* s) {
  return (int64_t)s->num_experts + s->zero_expert_num + s->copy_expert_num + s->const_expert_num;
}

// Rules shared by every entry point (low_latency_combine page, Constraints:
// 0 < K <= 16 and K <= E+Z+C+Q; num_experts in [1, 1024]; special expert counts
// non-negative with a total below 2^31; A >= BS * min(local_expert_num, K)).
inline moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL_ARG;
  if (s->comm_quant_mode != 0 && s->comm_quant_mode != 2) return MOE_ERR_BAD_RANGE;
  if (s->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->mask_ndim < 0 || s->mask_ndim > 2) return MOE_ERR_BAD_RANGE;
  if (s->T < 0 || s->H <= 0 || (s->H % 8) != 0) return MOE_ERR_BAD_SHAPE;
  if (s->K < 1 || s->K > 16) return MOE_ERR_BAD_SHAPE;
  if (s->num_experts < 1 || s->num_experts > 1024) return MOE_ERR_BAD_SHAPE;
  if (s->zero_expert_num < 0 || s->copy_expert_num < 0 || s->const_expert_num < 0)
    return MOE_ERR_BAD_SHAPE;
  if (e_total(s) >= (int64_t)0x7fffffff) return MOE_ERR_BAD_SHAPE;
  if ((int64_t)s->K > e_total(s)) return MOE_ERR_BAD_SHAPE;
  const int64_t need = s->T * (int64_t)(s->num_experts < s->K ? s->num_experts : s->K);
  if (s->capacity < need) return MOE_ERR_CAPACITY;
  if (s->capacity > (int64_t)0x7fffffff || s->T * (int64_t)s->K > (int64_t)0x7fffffff)
    return MOE_ERR_BAD_SHAPE;
  if (s->H > (int64_t)1 << 20) return MOE_ERR_BAD_SHAPE;
  return MOE_OK;
}

inline moe_status check_ffn_shape(const moe_shape* s) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->F <= 0 || (s->F % 32) != 0 || s->F > (int64_t)1 << 20) return MOE_ERR_BAD_SHAPE;
  // the GEMMs address one expert's weight matrix through a buffer resource
  // with 32-bit offsets and a byte range below 2^31
  if (s->F * s->H * 2 >= (int64_t)0x7ffffff0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// A pointer may be NULL only when the tensor it stands for has no elements.
#define MOE_NEED(p, n) \
  do {                                          \
    if (!(p) && (int64_t)(n) > 0) return MOE_ERR_NULL_ARG; \
  } while (0)

// fp8 GEMMs: the 128-wide scale blocks must tile H and F exactly.
inline moe_status check_fp8_shape(const moe_shape* s) {
  moe_status st = check_ffn_shape(s);
  if (st != MOE_OK) return st;
  if (s->H % 128 != 0 || s->F % 128 != 0) return MOE_ERR_BAD_SHAPE;
  // the fp8 GEMMs keep one B block scale per 128-wide K block in LDS: K = H or
  // 2F at most 32768
  if (s->H > 32768 || 2 * s->F > 32768) return MOE_ERR_UNSUPPORTED;
  // the activation scales of all rows are read with 32-bit byte offsets
  const int64_t kmax = s->H > 2 * s->F ? s->H : 2 * s->F;
  if (s->capacity * (kmax / 128) * 4 >= (int64_t)0x7ffffff0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Waves per token for the column-parallel row kernels (permute, combine,
// dispatch backward) over rows of Hv 16-byte vectors and K slots per token:
// wide rows of tokens with many slots are split over several waves so that
// more row accesses are in flight (measured on MI355X at H = 7168, K = 8:
// 4.1 -> 4.6 TB/s for combine with the inputs in HBM); with K = 2 the split
// measured slower.
inline int token_split(int64_t Hv, int K) {
  if (K < 4) return 1;
  return Hv >= 512 ? 4 : (Hv >= 256 ? 2 : 1);
}

inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// moe_dispatch in parts (route.hip): its workspace size, its argument checks
// and its launches, for entries that bring the workspace from elsewhere.
size_t dispatch_ws_bytes(const moe_shape* s);
moe_status dispatch_check(const moe_shape* s, const void* x, const int32_t* topk_idx, const uint8_t* x_active_mask,
                          void* expand_x, int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                          int32_t* err_flag, void* workspace, size_t ws_bytes);
moe_status dispatch_impl(const moe_shape* s, const void* x, const int32_t* topk_idx, const uint8_t* x_active_mask,
                         void* expand_x, int32_t* assist, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                         int32_t* err_flag, void* workspace, hipStream_t strm);

}  // namespace moe
