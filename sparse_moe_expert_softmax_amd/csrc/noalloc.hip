// Route + forward for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// workspace of ft_moe_route_forward lives in a fixed device array of this
// library instead of a caller buffer.
//
// The array is a file-scope __device__ variable, so each GPU holds its own
// copy from module load until the process ends.  In host code its name is
// only a host-side stand-in: the device address of each GPU's copy is taken
// once per device with hipGetSymbolAddress (that device current) and kept
// here, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/ft_moe.h"
#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)FT_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up once
// per device.  Returns nullptr (and the HIP error in *err) on failure.
void* scratch_address(int dev, hipError_t* err) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  *err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || q == nullptr) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int ft_moe_route_forward_noalloc(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const void* w_router,
                                 const float* sel_bias, int32_t* topk_ids, float* topk_gates, const void* pool_base,
                                 const uint32_t* expert_mask, float* out, void* stream) {
  if (!desc) return ft::report(FT_EINVAL, "desc is NULL");
  if (n_tokens < 0) return ft::report(FT_EINVAL, "n_tokens < 0");
  if (n_tokens == 0) return FT_OK;
  const size_t need = ft_moe_route_forward_workspace_bytes(desc, n_tokens);
  if (need == 0)  // invalid desc: the full call reports which check failed, before any launch
    return ft_moe_route_forward(desc, x, n_tokens, w_router, sel_bias, topk_ids, topk_gates, pool_base, expert_mask,
                                out, nullptr, 0, stream);
  if (need > kScratchBytes)
    return ft::report(FT_EWORKSPACE, "this call needs %zu workspace bytes; the allocation-free entry point holds %zu",
                      need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ft::report(FT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return ft::report(FT_EINVAL, "device %d beyond %d", dev, kMaxDevices);
  void* ws = scratch_address(dev, &e);
  if (!ws) return ft::report(FT_EHIP, "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
  return ft_moe_route_forward(desc, x, n_tokens, w_router, sel_bias, topk_ids, topk_gates, pool_base, expert_mask,
                              out, ws, kScratchBytes, stream);
}

}  // extern "C"
