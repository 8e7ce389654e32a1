// libroutedfp4: moe_layer_fwd for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops that must not call the
// allocator).  The workspace moe_layer_fwd takes from its caller is, here, the
// library's own device array `scratch` (one copy per GPU, held until the
// process ends).  Host code never passes the array's name to a kernel: its
// device address is looked up once per device with hipGetSymbolAddress and
// kept, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = size_t(40) << 20;   // 40 MiB: every call of up to 16 tokens
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];      // device address of `scratch` per device, once looked up

// The error word of the single-launch decode kernel (byte 16 of its
// workspace) to the caller's int32, then cleared.
__global__ void k_take_error(uint32_t* word, int32_t* out) {
  *out = (int32_t)*word;
  *word = 0u;
}

// The array's device address on the current device; the first call on a
// device also zero-fills the array on `st` (a fill kernel, no memset node),
// which the single-launch kernel's call counter needs.
moe_status scratch_for_device(hipStream_t st, void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
    const moe_status s = moe_workspace_init(p, kScratchBytes, st);
    if (s != MOE_OK) return s;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_fwd_noalloc(const moe_bank* bank, const float* w_router, const float* x,
                                 int32_t C, int32_t k, float* out, int32_t* topk_idx_out,
                                 float* topk_w_out, int32_t* error_out, void* stream) {
  const moe_status bs = rf4::bank_status(bank);
  if (bs != MOE_OK) return bs;
  const size_t need = moe_workspace_size(bank->num_experts, bank->hidden, bank->inter, k, C);
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  moe_status s = scratch_for_device(st, &ws);
  if (s != MOE_OK) return s;
  s = moe_layer_fwd(bank, w_router, x, C, k, out, topk_idx_out, topk_w_out, ws, kScratchBytes, stream);
  if (s != MOE_OK || !error_out) return s;
  hipLaunchKernelGGL(k_take_error, dim3(1), dim3(1), 0, st,
                     reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + 16), error_out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

}  // extern "C"
