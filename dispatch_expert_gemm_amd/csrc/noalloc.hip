// moe_dispatch_noalloc: moe_dispatch for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  The routing scratch that moe_dispatch takes as a workspace
// argument lives here in a fixed device array of the library instead; every
// other buffer is the caller's, as for moe_dispatch, and the kernels are the
// same ones.
#include <mutex>

#include "common.hpp"

namespace moe {

// Routing scratch of the allocation-free dispatch: per-chunk expert histograms
// and chunk error words (the layout moe_workspace_size describes).  The routing
// cuts the slots into at most 256 chunks and at most 32768 (chunk, expert)
// counts, so every valid shape needs at most 129 KiB; the array is 256 KiB.
// Each GPU holds its own copy for the life of the process.  Its name in host
// code is only a host-side handle: the device address comes from
// hipGetSymbolAddress.
constexpr size_t kScratchBytes = 256u << 10;
__device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up once per device (with
// that device current) on its first call.
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                           const uint8_t* x_active_mask, void* expand_x, int32_t* assist,
                                           int32_t* expert_token_nums, int32_t* ep_recv_counts,
                                           int32_t* err_flag, void* stream) {
  const moe_status sst = check_shape(s);
  if (sst != MOE_OK) return sst;
  // the shape's routing scratch must fit the fixed array
  if (dispatch_ws_bytes(s) > kScratchBytes) return MOE_ERR_WORKSPACE;
  // argument checks before any device call (the workspace is the array, of its size)
  const uintptr_t stand_in = 1;  // non-null placeholder: only its presence is checked
  moe_status st = dispatch_check(s, x, topk_idx, x_active_mask, expand_x, assist, expert_token_nums,
                                 ep_recv_counts, err_flag, reinterpret_cast<void*>(stand_in), kScratchBytes);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return dispatch_impl(s, x, topk_idx, x_active_mask, expand_x, assist, expert_token_nums, ep_recv_counts,
                       err_flag, ws, as_stream(stream));
}
