/* ft_moe.h -- C ABI of the MI355X (gfx950) exact MoE-layer forward over a
 * global expert cache.
 *
 * The operation (FreeToken pages): a MoE layer routes each token to a few of
 * its experts without changing or approximating the router (explainer page,
 * "how" and "who" sections); the full expert pool lives in host memory and
 * free device memory is one least-recently-used expert cache shared by all
 * MoE layers (explainer page, "how" section; LRU as defined in its
 * glossary); at prefill the next layer's whole expert set is copied while
 * the current layer computes (explainer page, "how" section; architecture
 * guide, prefill/decode section); the experts of a token may be computed
 * in different places and the partial outputs summed, which leaves the MoE
 * output mathematically identical (explainer page, "how" section).  Shapes
 * come from the same page's "why now" section (256 experts, 6 active).
 * The pages give no formula: the layer is the textbook one, softmax router,
 * top-k with renormalised gates, SwiGLU experts, gate-weighted sum.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked (host).  Nothing here
 *    allocates: callers own every buffer and size workspaces with the
 *    *_bytes queries.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream) unless its comment says otherwise.
 *  - Host-side argument checks run before any launch; a failed check returns
 *    a negative ft_status and launches nothing.  A failed HIP launch returns
 *    FT_EHIP.  ft_last_error() gives a thread-local message for the last
 *    non-OK status.  No C++ exception crosses this boundary.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders, so two identical calls give bitwise identical outputs.
 */
#ifndef FT_MOE_H
#define FT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FT_OK = 0,
  FT_EINVAL = -1,        /* bad argument (null, size, alignment, pageable host memory) */
  FT_EUNSUPPORTED = -2,  /* valid but not implemented combination (e.g. dtype pair) */
  FT_EPOOL = -3,         /* slot pool exhausted by one lookup (see ft_slot_lookup) */
  FT_EHIP = -4,          /* a HIP runtime call failed */
  FT_EWORKSPACE = -5     /* workspace too small */
} ft_status;

typedef enum { FT_F32 = 0, FT_BF16 = 1, FT_MXFP4 = 2, FT_NVFP4 = 3 } ft_dtype;

/* One MoE layer's shape and formats.
 *  hidden H, inter I (SwiGLU width per expert), n_experts E, top_k k.
 *  act_dtype: x is FT_F32 or FT_BF16 (row-major [T, H]).
 *  router_dtype: W_r is FT_F32 or FT_BF16 ([E, H] row-major).
 *  w_dtype: expert record format, see "packed expert record" below.
 *  renormalize: 1 = gates are the softmax over the k selected logits (the
 *    full softmax renormalised over the selection); 0 = full-softmax probs.
 *  expert_stride: bytes between consecutive expert records in a pool
 *    (>= ft_record_bytes(), multiple of 256). */
typedef struct {
  int32_t hidden, inter, n_experts, top_k;
  int32_t act_dtype, w_dtype, router_dtype, renormalize;
  int64_t expert_stride;
} ft_moe_desc;

/* Packed expert record (the offline pre-converted weight format the pages
 * describe as skipping start-up conversion, explainer "how" section):
 * gate [I,H], up [I,H], down [H,I], each row-major with the reduction
 * dimension contiguous.
 *  FT_F32 / FT_BF16: the three matrices' elements back to back.
 *  FT_MXFP4: E2M1 codes of gate, up, down (2 per byte, low nibble = even
 *    element), then E8M0 scales of gate, up, down, [rows, K/32] each
 *    (OCP MX v1.0; value = e2m1 * 2^(scale-127)).
 *  FT_NVFP4: E2M1 codes as above, then E4M3 block scales [rows, K/16] of
 *    gate, up, down, then 3 little-endian fp32 per-tensor scales;
 *    value = e2m1 * e4m3 * tensor_scale.
 * Requirements: H and I multiples of 32 (of 8 for F32/BF16). */
size_t ft_record_bytes(int32_t hidden, int32_t inter, int32_t w_dtype);

/* ---------------------------------------------------------------- route --
 * l[t,e] = sum_h x[t,h] W_r[e,h], accumulated from exact products in fp64;
 * score s = l + sel_bias[t,e] (fp64; sel_bias nullable = 0, selection only);
 * topk_ids[t,:] = the k experts with largest s in order (s desc, id asc);
 * topk_gates[t,j] = softmax of the selected l (renormalize=1) or the full
 * softmax probability (renormalize=0), computed in fp64, stored fp32.
 * logits (nullable): l as fp64 [T, E].
 * With more than 16 tokens, bf16 x and W_r, renormalize = 1 and logits
 * NULL, l is computed in fp64 only for the experts that a rounding bound on
 * bf16 matrix-core scores cannot rule out; ids and gates are the same as
 * above (the excluded experts provably score below the k-th).
 * workspace: ft_route_workspace_bytes(desc, T) bytes, 256-byte aligned
 * (holds the logits when `logits` is NULL; calls sharing it must not overlap).
 * Its contents need not be initialised; every workspace in this header is
 * fully written before it is read, so one buffer can serve call after call,
 * also from a replayed graph.
 * Errors: FT_EINVAL on null x/w_router/outputs, n_tokens < 0, k > E,
 * E > 1024, k > 32; FT_EUNSUPPORTED on other dtypes.  n_tokens = 0 is a no-op. */
size_t ft_route_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens);
int ft_moe_route(const ft_moe_desc* desc, const void* x, int32_t n_tokens,
                 const void* w_router, const float* sel_bias,
                 int32_t* topk_ids, float* topk_gates, double* logits,
                 void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ global slot table --
 * One LRU table of n_slots expert slots shared by n_layers layers of
 * n_experts experts each; key = (layer, expert).  Device-resident layout:
 * header {tick u32, status i32, L, E, S} then key_slot i32 [L*E] (-1 absent),
 * slot_key i32 [S] (layer*E+e, -1 free), last_use u32 [S] (0 never).
 * ft_slot_table_init fills it with the cold state (all slots free). */
size_t ft_slot_table_bytes(int32_t n_layers, int32_t n_experts, int32_t n_slots);
int ft_slot_table_init(void* table, int32_t n_layers, int32_t n_experts, int32_t n_slots,
                       void* stream);

/* One lookup of the ids one layer selected (any order, repeats allowed):
 * distinct ids ascending; hits are stamped with the new tick; if the misses
 * outnumber the slots not stamped by this call, nothing changes, *n_miss =
 * -1 and the header status = FT_EPOOL; else the i-th miss (ascending id)
 * takes the i-th slot in (last_use asc, slot asc) order among slots not
 * stamped by this call, evicting its key.
 * Outputs (device): slot_ids i32 [n_pairs], miss_flags u8 [n_pairs] (1 on
 * every occurrence of a missed id), miss_list i32 [2*n_pairs] as (expert,
 * slot) pairs in ascending expert order, n_miss i32 [1].
 * Errors: FT_EINVAL on nulls, layer out of range, n_pairs < 1 or > 1024. */
int ft_slot_lookup(void* table, int32_t layer, const int32_t* topk_ids, int32_t n_pairs,
                   int32_t* slot_ids, uint8_t* miss_flags, int32_t* miss_list,
                   int32_t* n_miss, void* stream);

/* --------------------------------------------------------------- upload --
 * Copy n packed expert records from pinned host memory into pool slots:
 * host_src[i] (host array of host pointers, each pinned) -> pool_base +
 * slots[i] * expert_stride, record_bytes bytes each, as hipMemcpyAsync on
 * `stream`; `done_event` (hipEvent_t as void*, nullable) is recorded after
 * the last copy.  Errors: FT_EINVAL on nulls, n < 0, a negative slot, or a
 * source that is not pinned host memory (a pageable copy would serialise). */
int ft_expert_upload(void* pool_base, int64_t expert_stride, int64_t record_bytes,
                     const int32_t* slots, const void* const* host_src, int32_t n,
                     void* stream, void* done_event);

/* ---------------------------------------------------- device-side fetch --
 * The copy step after ft_slot_lookup without a host round trip: the pages
 * keep the per-layer control inside one captured graph (FreeToken blog
 * page, architecture section); here the miss list and its count never leave
 * the device.  Copies, for i < *n_miss, the record of expert miss_list[2i]
 * from host memory layer_src[e] to pool_base + miss_list[2i+1] *
 * expert_stride.  A negative *n_miss (exhausted pool) copies nothing.
 *  layer_src: device array [n_experts] of addresses of this layer's records
 *    in pinned host memory (hipHostMalloc, torch pin_memory), which the GPU
 *    reads directly over the host link; 16-byte aligned.  The caller
 *    guarantees that every address is pinned host memory (pageable memory
 *    cannot be read by the GPU).
 *  miss_list, n_miss: device, as ft_slot_lookup wrote them.
 *  max_miss: upper bound on *n_miss; sizes the grid.  Pass the lookup's
 *    n_pairs (a lookup never reports more misses than ids): misses past
 *    max_miss would not be copied, and the call cannot see *n_miss on the
 *    host to report it.
 *  Entries with e outside [0, n_experts) or a slot outside [0, n_slots) are
 *  skipped.  Asynchronous on `stream`, after the lookup on the same stream.
 * Errors: FT_EINVAL on nulls, non-positive sizes, record_bytes or stride not
 * a multiple of 16, misaligned pool.  max_miss = 0 is a no-op. */
int ft_expert_fetch(void* pool_base, int64_t expert_stride, int64_t record_bytes, int32_t n_experts,
                    int32_t n_slots, const uint64_t* layer_src, const int32_t* miss_list,
                    const int32_t* n_miss, int32_t max_miss, void* stream);

/* -------------------------------------------------------------- forward --
 * out[t,:] = sum_j [expert_mask has e_tj] * topk_gates[t,j] * y_tj with
 * y_tj = D (silu(G x_t) * (U x_t)) of expert e_tj, summed over j in order.
 * The record of expert e is at pool_base + slot * expert_stride where slot =
 * slot_ids[t*k+j] (slot_ids nullable -> slot = e).  Masked-out experts are
 * never read.  expert_mask: bitset u32 [ceil(E/32)], nullable = all.
 * out: fp32 [T, H], fully overwritten; it must not overlap any input.
 * Decode-sized calls (few pairs per expert) run as bandwidth-bound grouped
 * GEMV; large MXFP4 calls run on gfx950 scaled MFMA with activations
 * quantised to MXFP8 (E4M3, E8M0 per 32) first.
 * Errors: FT_EINVAL on nulls / sizes, FT_EUNSUPPORTED on dtype pairs,
 * FT_EWORKSPACE if ws_bytes < ft_moe_workspace_bytes(desc, T). */
size_t ft_moe_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens);
int ft_moe_forward(const ft_moe_desc* desc, const void* x, int32_t n_tokens,
                   const int32_t* topk_ids, const float* topk_gates,
                   const int32_t* slot_ids, const void* pool_base,
                   const uint32_t* expert_mask, float* out,
                   void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ route + forward --
 * One call doing ft_moe_route followed by ft_moe_forward with every expert
 * resident at its own slot (slot = expert id), for callers whose pool holds
 * all experts: the results (topk_ids, topk_gates, out) are bitwise those of
 * the two calls.  For decode-sized calls (at most 16 tokens on the grouped
 * GEMV path, at most 256 experts, a gate/up grid of at most 1,024
 * workgroups: min(T k, E) experts x I/8 row tiles, halved where two tiles
 * share a workgroup) the selection runs inside the gate/up kernel instead of
 * as a launch of its own (the routing rule itself is unchanged: pages,
 * explainer "how" and "who" sections); other sizes run the two calls in
 * sequence.
 * workspace: ft_moe_route_forward_workspace_bytes(desc, T) bytes, 256-byte
 * aligned; calls sharing it must not overlap.  out must not overlap any
 * input.  Errors: those of ft_moe_route and ft_moe_forward. */
size_t ft_moe_route_forward_workspace_bytes(const ft_moe_desc* desc, int32_t n_tokens);
int ft_moe_route_forward(const ft_moe_desc* desc, const void* x, int32_t n_tokens,
                         const void* w_router, const float* sel_bias,
                         int32_t* topk_ids, float* topk_gates,
                         const void* pool_base, const uint32_t* expert_mask, float* out,
                         void* workspace, size_t ws_bytes, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* ft_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FT_MOE_H */
