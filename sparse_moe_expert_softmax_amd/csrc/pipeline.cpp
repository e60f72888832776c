// Full-layer double buffering at prefill: while layer n computes from one
// device layer buffer, layer n+1's whole expert set is copied from pinned
// host memory into the other buffer on a second stream (FreeToken explainer
// page, "how" section; architecture guide, prefill passage).  The state is
// caller-owned (ft_prefill_pipeline); this file only sequences the copies,
// the events and the route + forward calls on the two streams.
#include <hip/hip_runtime.h>

#include "../../include/ft_moe.h"
#include "internal.hpp"

namespace {

int check_pipeline(const ft_prefill_pipeline* p) {
  if (!p) return ft::report(FT_EINVAL, "pipeline is NULL");
  if (!p->layer_buf[0] || !p->layer_buf[1] || p->layer_buf[0] == p->layer_buf[1])
    return ft::report(FT_EINVAL, "two distinct layer buffers are needed");
  if (!p->ready[0] || !p->ready[1] || !p->freed[0] || !p->freed[1])
    return ft::report(FT_EINVAL, "the four pipeline events are needed");
  if (p->compute_stream == p->copy_stream)
    return ft::report(FT_EINVAL, "copy_stream must differ from compute_stream (the copies would not overlap)");
  if (p->n_experts <= 0 || p->record_bytes <= 0 || p->expert_stride < p->record_bytes)
    return ft::report(FT_EINVAL, "n_experts, record_bytes and expert_stride");
  if (p->n_done < 0 || p->n_uploaded < 0) return ft::report(FT_EINVAL, "negative layer count");
  return FT_OK;
}

// slots 0 .. E-1: the layer buffer holds expert e at e * expert_stride
int upload_layer(ft_prefill_pipeline* p, int b, const void* const* records) {
  const int E = p->n_experts;
  if (E > 1024) return ft::report(FT_EINVAL, "n_experts %d > 1024", E);
  int32_t slots[1024];
  for (int e = 0; e < E; ++e) slots[e] = e;
  return ft_expert_upload(p->layer_buf[b], p->expert_stride, p->record_bytes, slots, records, E, p->copy_stream,
                          p->ready[b]);
}

}  // namespace

extern "C" {

int ft_prefill_pipeline_start(ft_prefill_pipeline* p, const void* const* first_layer) {
  int rc = check_pipeline(p);
  if (rc) return rc;
  if (!first_layer) return ft::report(FT_EINVAL, "first_layer is NULL");
  p->n_done = 0;
  p->n_uploaded = 0;
  rc = upload_layer(p, 0, first_layer);
  if (rc) return rc;
  p->n_uploaded = 1;
  return FT_OK;
}

int ft_prefill_pipeline_layer(ft_prefill_pipeline* p, const void* const* next_layer, const ft_moe_desc* desc,
                              const void* x, int32_t n_tokens, const void* w_router, int32_t* topk_ids,
                              float* topk_gates, float* out, void* workspace, size_t ws_bytes) {
  int rc = check_pipeline(p);
  if (rc) return rc;
  if (!desc) return ft::report(FT_EINVAL, "desc is NULL");
  if (desc->expert_stride != p->expert_stride)
    return ft::report(FT_EINVAL, "desc->expert_stride differs from the pipeline's");
  if (desc->n_experts != p->n_experts) return ft::report(FT_EINVAL, "desc->n_experts differs from the pipeline's");
  // the forward's own checks, before anything is enqueued, so that a refused
  // call leaves the pipeline as it was
  const size_t need = ft_moe_route_forward_workspace_bytes(desc, n_tokens);
  if (need == 0 || n_tokens <= 0) return ft::report(FT_EINVAL, "invalid desc or n_tokens %d", n_tokens);
  if (!x || !w_router || !topk_ids || !topk_gates || !out) return ft::report(FT_EINVAL, "NULL x / router / output");
  if (!workspace || ws_bytes < need) return ft::report(FT_EWORKSPACE, "route + forward needs %zu workspace bytes", need);
  const int n = p->n_done, b = n & 1;
  if (p->n_uploaded != n + 1)
    return ft::report(FT_EINVAL, "layer %d was not uploaded (the previous call passed no next layer, or the pipeline "
                      "was not started)", n);
  hipStream_t comp = reinterpret_cast<hipStream_t>(p->compute_stream);
  hipStream_t copy = reinterpret_cast<hipStream_t>(p->copy_stream);
  // 1. the next layer's copy into the other buffer, once the previous layer's
  //    compute (the last reader of that buffer) is done with it
  if (next_layer) {
    if (n >= 1) {
      hipError_t e = hipStreamWaitEvent(copy, reinterpret_cast<hipEvent_t>(p->freed[b ^ 1]), 0);
      if (e != hipSuccess) return ft::report(FT_EHIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    }
    rc = upload_layer(p, b ^ 1, next_layer);
    if (rc) return rc;
    p->n_uploaded = n + 2;
  }
  // 2. this layer's compute, after its own copy landed
  hipError_t e = hipStreamWaitEvent(comp, reinterpret_cast<hipEvent_t>(p->ready[b]), 0);
  if (e != hipSuccess) return ft::report(FT_EHIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
  rc = ft_moe_route_forward(desc, x, n_tokens, w_router, nullptr, topk_ids, topk_gates, p->layer_buf[b], nullptr, out,
                            workspace, ws_bytes, p->compute_stream);
  if (rc) return rc;
  e = hipEventRecord(reinterpret_cast<hipEvent_t>(p->freed[b]), comp);
  if (e != hipSuccess) return ft::report(FT_EHIP, "hipEventRecord: %s", hipGetErrorString(e));
  p->n_done = n + 1;
  return FT_OK;
}

}  // extern "C"
