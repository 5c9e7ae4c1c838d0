// A streaming kernel that measures how fast this GPU's HBM moves data in the
// access patterns of the gather-reduce kernels: a plain copy (every byte read
// once and written once), a read-only sweep and a write-only fill.  It is the
// measured ceiling the dispatch, combine and dispatch-backward kernels are
// compared with; it computes nothing of the layer.
//
// Each workgroup streams one contiguous range of the buffer, its lanes taking
// consecutive 16-byte vectors, eight loads in flight per lane before their
// stores (of the layouts measured on MI355X -- grid-strided or per-workgroup
// ranges, 4 to 16 vectors in flight, plain or non-temporal accesses, 1024 to
// 8192 workgroups -- per-workgroup ranges with plain accesses moved the most).
#include "common.hpp"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamBlocks = 4096;
constexpr int kUnroll = 8;

template <int MODE>  // 0 copy, 1 read, 2 write
__global__ __launch_bounds__(256) void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                int64_t nvec, int64_t per, u32x4* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < nvec ? b0 + per : nvec;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = b0 + threadIdx.x; i < b1; i += kUnroll * 256) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t j = i + q * 256;
      if (MODE == 2) v[q] = u32x4{(unsigned)j, 1u, 2u, 3u};
      else if (j < b1) v[q] = src[j];
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t j = i + q * 256;
      if (j >= b1) continue;
      if (MODE == 1) acc ^= v[q];
      else dst[j] = v[q];
    }
  }
  // the read sweep leaves one vector per thread that depends on every load
  if (MODE == 1) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_hbm_stream(int32_t mode, const void* src, void* dst, int64_t bytes, void* sink,
                                     void* stream) {
  if (mode < 0 || mode > 2) return MOE_ERR_BAD_RANGE;
  if (bytes < 0 || bytes % 16 != 0) return MOE_ERR_BAD_SHAPE;
  if ((mode != 2 && !src) || (mode != 1 && !dst) || (mode == 1 && !sink)) return MOE_ERR_NULL_ARG;
  const int64_t nvec = bytes / 16;
  if (nvec == 0) return MOE_OK;
  const int64_t per = (nvec + kStreamBlocks - 1) / kStreamBlocks;
  hipStream_t strm = as_stream(stream);
  const dim3 grid(kStreamBlocks), block(256);
  const auto* s = static_cast<const u32x4*>(src);
  auto* d = static_cast<u32x4*>(dst);
  auto* k = static_cast<u32x4*>(sink);
  if (mode == 0) hipLaunchKernelGGL(k_stream<0>, grid, block, 0, strm, s, d, nvec, per, k);
  else if (mode == 1) hipLaunchKernelGGL(k_stream<1>, grid, block, 0, strm, s, d, nvec, per, k);
  else hipLaunchKernelGGL(k_stream<2>, grid, block, 0, strm, s, d, nvec, per, k);
  return launch_status();
}
