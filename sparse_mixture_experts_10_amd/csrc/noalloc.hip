// moe_route_noalloc: the fused routing pass with its scratch in a static
// device array instead of a caller workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The array lives in this file's device code; every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is a host-side
// stand-in, not a device address): the first call on each device looks the
// address up with hipGetSymbolAddress, with that device current, and keeps
// it; kernels take that pointer exactly as they take a caller workspace.
// The routing kernels need no cleared scratch (each pass writes what it later
// reads), so nothing is cleared.  Calls that overlap on one GPU share the
// array and race: order them on one stream.

#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "internal.h"

namespace moe {

constexpr size_t kScratchBytes = MOE_ROUTE_NOALLOC_MAX_BYTES;  // a device
constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// This device's address of the array (looked up once per device).
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev]() {
    g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr) return MOE_ERR_HIP;
  *ptr = g_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_route_noalloc(const void* x, int x_dtype, int64_t T, int32_t d, const float* W_g,
                      const float* b_g, const float* b_sel, int32_t E, int32_t k, const float* noise,
                      float noise_std, float temperature, int64_t capacity, float alpha, float beta,
                      float* logits, float* lse, int32_t* topk_idx, float* topk_gate,
                      int32_t* expert_count, int32_t* expert_offset, int32_t* slot, int32_t* row,
                      int32_t* row_token, float* f, float* P, float* losses, hipStream_t stream) {
  const RouteCall c{x, x_dtype, T, d, W_g, b_g, b_sel, E, k, noise, noise_std, temperature, capacity, alpha,
                    beta, logits, lse, topk_idx, topk_gate, expert_count, expert_offset, slot, row, row_token,
                    f, P, losses};
  size_t need = 0;
  if (int rc = route_check(c, &need)) return rc;
  if (need > kScratchBytes) return MOE_ERR_SCRATCH;
  void* ptr = nullptr;
  if (int rc = scratch_address(&ptr)) return rc;
  return route_run(c, ptr, stream);
}

}  // extern "C"
