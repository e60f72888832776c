// C ABI of the MoE-layer library: host-side validation, workspace planning,
// and launches.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/ft_moe.h"
#include "common.hpp"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(FT_EHIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_desc(const ft_moe_desc* d) {
  if (!d) return fail(FT_EINVAL, "desc is NULL");
  if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0)
    return fail(FT_EINVAL, "non-positive size in desc");
  if (d->top_k > d->n_experts) return fail(FT_EINVAL, "top_k %d > n_experts %d", d->top_k, d->n_experts);
  if (d->top_k > 32) return fail(FT_EINVAL, "top_k %d > 32", d->top_k);
  if (d->n_experts > 1024) return fail(FT_EINVAL, "n_experts %d > 1024", d->n_experts);
  if (d->act_dtype != FT_F32 && d->act_dtype != FT_BF16)
    return fail(FT_EUNSUPPORTED, "act_dtype %d (need F32 or BF16)", d->act_dtype);
  if (d->router_dtype != FT_F32 && d->router_dtype != FT_BF16)
    return fail(FT_EUNSUPPORTED, "router_dtype %d (need F32 or BF16)", d->router_dtype);
  if (d->w_dtype < FT_F32 || d->w_dtype > FT_NVFP4) return fail(FT_EUNSUPPORTED, "w_dtype %d", d->w_dtype);
  if (d->hidden % 32 || d->inter % 32) return fail(FT_EINVAL, "hidden and inter must be multiples of 32");
  if (d->act_terms < 0 || d->act_terms > 2) return fail(FT_EINVAL, "act_terms %d (need 0, 1 or 2)", d->act_terms);
  return FT_OK;
}

}  // namespace

namespace ft {

int report(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

FwdPlan plan_forward(const ft_moe_desc& d, int T) {
  FwdPlan p{};
  p.T = T;
  p.P = T * d.top_k;
  p.E = d.n_experts;
  p.H = d.hidden;
  p.I = d.inter;
  p.nb = (p.P + PERM_CHUNK - 1) / PERM_CHUNK;
  if (p.nb < 1) p.nb = 1;
  const bool mx = mfma_supported(d, T), bf = !mx && mfma_bf16_supported(d, T);
  p.mfma = mx || bf;
  p.mfma_w = mx ? FT_MXFP4 : (bf ? FT_BF16 : -1);
  p.path = p.mfma ? PATH_MFMA : (dec_supported(d, T) ? PATH_DEC : PATH_GEMV);
  p.terms = (mx && d.act_terms != 1) ? 2 : 1;
  p.max_tiles = p.P / (256 / p.terms) + p.E + 1;
  size_t o = 0;
  p.off_hist = o;    o = align256(o + sizeof(int32_t) * (size_t)p.nb * p.E);
  p.off_offsets = o; o = align256(o + sizeof(int32_t) * (size_t)(p.E + 2));
  p.off_active = o;  o = align256(o + sizeof(int32_t) * (size_t)p.E);
  p.off_perm = o;    o = align256(o + sizeof(int32_t) * (size_t)p.P);
  p.off_pos = o;     o = align256(o + sizeof(int32_t) * (size_t)p.P);
  p.off_cnt = o;     o = align256(o + sizeof(uint32_t) * (size_t)(p.H / 16 + 1));
  p.off_h = o;       o = align256(o + sizeof(float) * (size_t)p.P * p.I);   // fp32 h, bf16 (hi/lo), or MXFP8 codes
  p.off_y = o;       o = align256(o + (p.mfma ? 2 : 4) * (size_t)p.P * p.H);  // bf16 y on the matrix-core paths
  p.off_dtab = o;    o = align256(o + (p.path == PATH_DEC ? DEC_DTAB_BYTES : 0));
  if (bf) {
    p.off_xq = p.off_xs = p.off_hs = o;
    p.off_tiles = o; o = align256(o + sizeof(int32_t) * ((size_t)2 * p.max_tiles + 1 +
                                                          (size_t)p.max_tiles * (p.I / 128 + p.H / 256)));
  } else if (mx) {
    p.off_xq = o;    o = align256(o + (size_t)p.terms * T * p.H);             // MXFP8 x codes (per term)
    p.off_xs = o;    o = align256(o + (size_t)p.terms * T * p.H / 32);        // and scales
    p.off_hs = o;    o = align256(o + (size_t)p.terms * p.P * p.I / 32);      // h scales (h codes: off_h)
    p.off_tiles = o; o = align256(o + sizeof(int32_t) * ((size_t)2 * p.max_tiles + 1 +
                                                          (size_t)p.max_tiles * (p.I / 128 + p.H / 256)));
  } else {
    p.off_xq = p.off_xs = p.off_hs = p.off_tiles = o;
  }
  p.bytes = o;
  return p;
}

}  // namespace ft

extern "C" {

const char* ft_last_error(void) { return g_err; }

size_t ft_record_bytes(int32_t hidden, int32_t inter, int32_t w_dtype) {
  if (hidden <= 0 || inter <= 0 || w_dtype < FT_F32 || w_dtype > FT_NVFP4) return 0;
  return (size_t)ft::record_layout(hidden, inter, w_dtype).bytes;
}

size_t ft_route_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens) {
  if (!desc || n_tokens < 0) return 0;
  // fp64 logits [T, E]; also room for the bounded prefill path's fp32
  // approximate logits [T, E] and its fp64 norm bounds (|w| [E], with room
  // for [T] more)
  const size_t te = (size_t)n_tokens * desc->n_experts;
  const size_t a = sizeof(double) * te;
  const size_t b = sizeof(float) * (te + 64) + sizeof(double) * ((size_t)n_tokens + 32 + desc->n_experts);
  return 256 + align256(a > b ? a : b);
}

int ft_moe_route(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const void* w_router,
                 const float* sel_bias, int32_t* topk_ids, float* topk_gates, double* logits, void* workspace,
                 size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n_tokens < 0) return fail(FT_EINVAL, "n_tokens < 0");
  if (n_tokens == 0) return FT_OK;
  if (!x || !w_router || !topk_ids || !topk_gates) return fail(FT_EINVAL, "NULL x / w_router / output");
  if (!aligned(x, 16) || !aligned(w_router, 16)) return fail(FT_EINVAL, "x and w_router must be 16-byte aligned");
  if (desc->hidden % 8) return fail(FT_EINVAL, "hidden must be a multiple of 8");
  if (!workspace || ws_bytes < ft_route_workspace_bytes(desc, n_tokens))
    return fail(FT_EWORKSPACE, "route needs %zu workspace bytes", ft_route_workspace_bytes(desc, n_tokens));
  if (!aligned(workspace, 256)) return fail(FT_EINVAL, "workspace must be 256-byte aligned");
  double* lg = logits ? logits : reinterpret_cast<double*>(reinterpret_cast<char*>(workspace) + 256);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (n_tokens <= ft::ROUTE_DECODE_MAX_T)
                     ? ft::launch_route_decode(*desc, x, n_tokens, w_router, sel_bias, topk_ids, topk_gates, lg, st)
                     : ft::launch_route(*desc, x, n_tokens, w_router, sel_bias, topk_ids, topk_gates, lg,
                                        logits != nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "ft_moe_route launch");
  return FT_OK;
}

size_t ft_slot_table_bytes(int32_t n_layers, int32_t n_experts, int32_t n_slots) {
  if (n_layers <= 0 || n_experts <= 0 || n_slots <= 0) return 0;
  return ft::slot_table_bytes(n_layers, n_experts, n_slots);
}

int ft_slot_table_init(void* table, int32_t n_layers, int32_t n_experts, int32_t n_slots, void* stream) {
  if (!table) return fail(FT_EINVAL, "table is NULL");
  if (n_layers <= 0 || n_experts <= 0 || n_slots <= 0) return fail(FT_EINVAL, "non-positive table size");
  if (n_slots > ft::slot_max_slots()) return fail(FT_EINVAL, "n_slots %d > %d", n_slots, ft::slot_max_slots());
  if (n_experts > ft::slot_max_experts())
    return fail(FT_EINVAL, "n_experts %d > %d", n_experts, ft::slot_max_experts());
  if ((int64_t)n_layers * n_experts >= (int64_t)1 << 31) return fail(FT_EINVAL, "too many keys");
  if (!aligned(table, 8)) return fail(FT_EINVAL, "table must be 8-byte aligned");
  hipError_t e = ft::launch_slot_table_init(table, n_layers, n_experts, n_slots, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ft_slot_table_init launch");
  return FT_OK;
}

int ft_slot_lookup(void* table, int32_t layer, const int32_t* topk_ids, int32_t n_pairs, int32_t* slot_ids,
                   uint8_t* miss_flags, int32_t* miss_list, int32_t* n_miss, void* stream) {
  if (!table || !topk_ids || !slot_ids || !miss_flags || !miss_list || !n_miss)
    return fail(FT_EINVAL, "NULL argument to ft_slot_lookup");
  if (n_pairs < 1 || n_pairs > 1024) return fail(FT_EINVAL, "n_pairs %d outside [1, 1024]", n_pairs);
  if (layer < 0) return fail(FT_EINVAL, "layer %d < 0", layer);
  // the layer bound lives in the device header; the kernel ignores ids >= E and
  // the host wrapper keeps the layer count, so check it there
  hipError_t e = ft::launch_slot_lookup(table, layer, topk_ids, n_pairs, slot_ids, miss_flags, miss_list, n_miss,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ft_slot_lookup launch");
  return FT_OK;
}

int ft_slot_probe(const void* table, int32_t layer, const int32_t* ids, int32_t n, uint8_t* resident, void* stream) {
  if (!table || !ids || !resident) return fail(FT_EINVAL, "NULL argument to ft_slot_probe");
  if (n < 0) return fail(FT_EINVAL, "n < 0");
  if (layer < 0) return fail(FT_EINVAL, "layer %d < 0", layer);
  if (n == 0) return FT_OK;
  hipError_t e = ft::launch_slot_probe(table, layer, ids, n, resident, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ft_slot_probe launch");
  return FT_OK;
}

int ft_moe_add_partial(float* out, const float* part, int64_t n, void* stream) {
  if (n < 0) return fail(FT_EINVAL, "n < 0");
  if (n == 0) return FT_OK;
  if (!out || !part) return fail(FT_EINVAL, "NULL argument to ft_moe_add_partial");
  hipError_t e = ft::launch_add_partial(out, part, n, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ft_moe_add_partial launch");
  return FT_OK;
}

int ft_expert_upload(void* pool_base, int64_t expert_stride, int64_t record_bytes, const int32_t* slots,
                     const void* const* host_src, int32_t n, void* stream, void* done_event) {
  if (n < 0) return fail(FT_EINVAL, "n < 0");
  if (n > 0 && (!pool_base || !slots || !host_src)) return fail(FT_EINVAL, "NULL argument to ft_expert_upload");
  if (record_bytes <= 0 || expert_stride < record_bytes) return fail(FT_EINVAL, "record_bytes / stride");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0) return fail(FT_EINVAL, "slot %d < 0", slots[i]);
    if (!host_src[i]) return fail(FT_EINVAL, "host_src[%d] is NULL", i);
    hipPointerAttribute_t at;
    hipError_t pe = hipPointerGetAttributes(&at, host_src[i]);
    if (pe != hipSuccess || at.type != hipMemoryTypeHost) {
      (void)hipGetLastError();  // clear a sticky "invalid value" from the query
      return fail(FT_EINVAL, "host_src[%d] is not pinned host memory", i);
    }
  }
  for (int i = 0; i < n; ++i) {
    char* dst = reinterpret_cast<char*>(pool_base) + (int64_t)slots[i] * expert_stride;
    hipError_t e = hipMemcpyAsync(dst, host_src[i], (size_t)record_bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "ft_expert_upload copy");
  }
  if (done_event) {
    hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(done_event), st);
    if (e != hipSuccess) return hip_fail(e, "ft_expert_upload event");
  }
  return FT_OK;
}

int ft_expert_fetch(void* pool_base, int64_t expert_stride, int64_t record_bytes, int32_t n_experts,
                    int32_t n_slots, const uint64_t* layer_src, const int32_t* miss_list, const int32_t* n_miss,
                    int32_t max_miss, void* stream) {
  if (max_miss < 0) return fail(FT_EINVAL, "max_miss < 0");
  if (max_miss == 0) return FT_OK;
  if (!pool_base || !layer_src || !miss_list || !n_miss) return fail(FT_EINVAL, "NULL argument to ft_expert_fetch");
  if (n_experts <= 0 || n_slots <= 0) return fail(FT_EINVAL, "n_experts and n_slots must be positive");
  if (record_bytes <= 0 || record_bytes % 16 || expert_stride < record_bytes || expert_stride % 16)
    return fail(FT_EINVAL, "record_bytes and expert_stride must be positive multiples of 16, stride >= record");
  if (!aligned(pool_base, 16)) return fail(FT_EINVAL, "pool_base must be 16-byte aligned");
  if ((int64_t)max_miss * ((record_bytes + 65535) / 65536) > (int64_t)INT32_MAX)
    return fail(FT_EINVAL, "max_miss too large");
  hipError_t e = ft::launch_fetch(pool_base, expert_stride, record_bytes, n_experts, n_slots, layer_src, miss_list,
                                  n_miss, max_miss, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ft_expert_fetch launch");
  return FT_OK;
}

size_t ft_moe_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens) {
  if (check_desc(desc) || n_tokens < 0) return 0;
  return ft::plan_forward(*desc, n_tokens).bytes;
}

int ft_moe_forward(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const int32_t* topk_ids,
                   const float* topk_gates, const int32_t* slot_ids, const void* pool_base,
                   const uint32_t* expert_mask, float* out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n_tokens < 0) return fail(FT_EINVAL, "n_tokens < 0");
  if (n_tokens == 0) return FT_OK;
  if (!x || !topk_ids || !topk_gates || !pool_base || !out) return fail(FT_EINVAL, "NULL argument to ft_moe_forward");
  const size_t rec = ft_record_bytes(desc->hidden, desc->inter, desc->w_dtype);
  if (desc->expert_stride < (int64_t)rec || desc->expert_stride % 256)
    return fail(FT_EINVAL, "expert_stride %lld must be >= %zu and a multiple of 256", (long long)desc->expert_stride, rec);
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(pool_base, 256))
    return fail(FT_EINVAL, "x/out must be 16-byte aligned, pool_base 256-byte aligned");
  if ((int64_t)n_tokens * desc->top_k > (1 << 30)) return fail(FT_EINVAL, "too many pairs");
  const ft::FwdPlan pl = ft::plan_forward(*desc, n_tokens);
  if (!workspace || ws_bytes < pl.bytes) return fail(FT_EWORKSPACE, "forward needs %zu workspace bytes", pl.bytes);
  if (!aligned(workspace, 256)) return fail(FT_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  hipError_t e;
  if (pl.path == ft::PATH_DEC) {
    e = ft::launch_dec_forward(*desc, pl, x, topk_ids, expert_mask, slot_ids, pool_base, topk_gates, out, ws, st);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return FT_OK;
  }
  e = ft::launch_permute(pl, topk_ids, expert_mask, ws, st);
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  if (pl.mfma && pl.mfma_w == FT_BF16)
    e = ft::launch_mfma_bf16_forward(*desc, pl, x, slot_ids, pool_base, topk_gates, out, ws, st);
  else if (pl.mfma)
    e = ft::launch_mfma_forward(*desc, pl, x, slot_ids, pool_base, topk_gates, out, ws, st);
  else
    e = ft::launch_gemv_forward(*desc, pl, x, slot_ids, pool_base, topk_gates, out, ws, st);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return FT_OK;
}

size_t ft_moe_route_forward_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens) {
  if (check_desc(desc) || n_tokens < 0) return 0;
  return align256(ft_route_workspace_bytes(desc, n_tokens)) + ft_moe_workspace_bytes(desc, n_tokens);
}

int ft_moe_route_forward(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const void* w_router,
                         const float* sel_bias, int32_t* topk_ids, float* topk_gates, const void* pool_base,
                         const uint32_t* expert_mask, float* out, void* workspace, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n_tokens < 0) return fail(FT_EINVAL, "n_tokens < 0");
  if (n_tokens == 0) return FT_OK;
  const size_t need = ft_moe_route_forward_workspace_bytes(desc, n_tokens);
  if (!workspace || ws_bytes < need) return fail(FT_EWORKSPACE, "route + forward needs %zu workspace bytes", need);
  if (!aligned(workspace, 256)) return fail(FT_EINVAL, "workspace must be 256-byte aligned");
  char* rws = reinterpret_cast<char*>(workspace);
  const size_t rbytes = align256(ft_route_workspace_bytes(desc, n_tokens));
  char* fws = rws + rbytes;
  const size_t fbytes = ws_bytes - rbytes;
  const ft::FwdPlan pl = ft::plan_forward(*desc, n_tokens);
  // selection inside the gate/up kernel saves a launch but runs once per
  // workgroup: bf16 2048/768/128 top-8 measured 1.108 against 1.152 ms per
  // 40 layers at 1 token (768 workgroups), and 1.762 against 1.726 ms at 2
  // tokens, 3.097 against 2.867 ms at 4 (1,536 and 3,072 workgroups)
  const bool fuse = pl.path == ft::PATH_DEC && n_tokens <= ft::ROUTE_DECODE_MAX_T &&
                    desc->n_experts <= ft::DEC_FUSE_MAX_E &&
                    ft::dec_gateup_shape(*desc, n_tokens).grid <= ft::DEC_FUSE_MAX_GRID;
  if (!fuse) {
    rc = ft_moe_route(desc, x, n_tokens, w_router, sel_bias, topk_ids, topk_gates, nullptr, rws, rbytes, stream);
    if (rc) return rc;
    return ft_moe_forward(desc, x, n_tokens, topk_ids, topk_gates, nullptr, pool_base, expert_mask, out, fws, fbytes,
                          stream);
  }
  // the argument checks of both calls
  if (!x || !w_router || !topk_ids || !topk_gates || !pool_base || !out)
    return fail(FT_EINVAL, "NULL argument to ft_moe_route_forward");
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(out, 16) || !aligned(pool_base, 256))
    return fail(FT_EINVAL, "x/w_router/out must be 16-byte aligned, pool_base 256-byte aligned");
  const size_t rec = ft_record_bytes(desc->hidden, desc->inter, desc->w_dtype);
  if (desc->expert_stride < (int64_t)rec || desc->expert_stride % 256)
    return fail(FT_EINVAL, "expert_stride %lld must be >= %zu and a multiple of 256", (long long)desc->expert_stride, rec);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  double* lg = reinterpret_cast<double*>(rws + 256);
  hipError_t e = ft::launch_route_logits_decode(*desc, x, n_tokens, w_router, lg, st);
  if (e != hipSuccess) return hip_fail(e, "ft_moe_route_forward logits launch");
  e = ft::launch_dec_forward(*desc, pl, x, nullptr, expert_mask, nullptr, pool_base, nullptr, out, fws, st, lg, sel_bias,
                             topk_ids, topk_gates);
  if (e != hipSuccess) return hip_fail(e, "ft_moe_route_forward launch");
  return FT_OK;
}

}  // extern "C"
