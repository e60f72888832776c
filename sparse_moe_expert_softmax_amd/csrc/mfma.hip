// Large-batch (prefill) MXFP4 expert GEMM on gfx950 scaled MFMA.
#include "common.hpp"
#include "internal.hpp"

namespace ft {

hipError_t launch_mfma_forward(const ft_moe_desc&, const FwdPlan&, const void*, const int32_t*, const void*,
                               const float*, float*, char*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace ft
