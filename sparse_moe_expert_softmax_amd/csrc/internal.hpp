// Internal launchers shared by the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ft_moe.h"

namespace ft {

// record a non-OK status and its message for ft_last_error(); returns code
int report(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// router
// logits: [T, E] fp64 (the caller's when want_logits, else workspace, which
// the bounded prefill path also uses for its own arrays)
hipError_t launch_route(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                        int32_t* ids, float* gates, double* logits, bool want_logits, hipStream_t st);
constexpr int ROUTE_DECODE_MAX_T = 16;
hipError_t launch_route_decode(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                               int32_t* ids, float* gates, double* logits, hipStream_t st);
// the fp64 logit kernel of the decode router alone (T <= ROUTE_DECODE_MAX_T)
hipError_t launch_route_logits_decode(const ft_moe_desc& d, const void* x, int T, const void* wr, double* logits,
                                      hipStream_t st);

// slot table
size_t slot_table_bytes(int L, int E, int S);
hipError_t launch_slot_table_init(void* table, int L, int E, int S, hipStream_t st);
hipError_t launch_slot_lookup(void* table, int layer, const int32_t* ids, int n_pairs, int32_t* slot_ids,
                              uint8_t* miss_flags, int32_t* miss_list, int32_t* n_miss, hipStream_t st);
int slot_max_slots();
hipError_t launch_slot_probe(const void* table, int layer, const int32_t* ids, int n, uint8_t* resident,
                             hipStream_t st);
hipError_t launch_fetch(void* pool, int64_t stride, int64_t rec_bytes, int E, int S, const uint64_t* layer_src,
                        const int32_t* miss_list, const int32_t* n_miss, int max_miss, hipStream_t st);
int slot_max_experts();

// forward paths
enum FwdPath { PATH_DEC = 0, PATH_GEMV = 1, PATH_MFMA = 2 };
constexpr int DEC_MAX_PAIRS = 64;  // decode path: T*k pairs grouped inside the kernels
constexpr size_t DEC_DTAB_BYTES = 8192;  // decode path: the down kernel's (expert, token) table, built by gate/up

// forward workspace: every region 256-byte aligned
struct FwdPlan {
  int T, P, E, H, I, nb;       // tokens, pairs, experts, hidden, inter, permute blocks
  int path;                    // FwdPath
  bool mfma;                   // large-batch matrix-core path (PATH_MFMA)
  int mfma_w;                  // its weight format: FT_MXFP4 (scaled MFMA) or FT_BF16 (bf16 MFMA)
  int terms;                   // MXFP8 terms per activation on the MXFP4 path (1 or 2); 1 on the bf16 path
  size_t off_hist, off_offsets, off_active, off_perm, off_pos, off_h, off_y, off_xq, off_xs, off_hs, off_cnt;
  size_t off_tiles;            // MFMA path: tile list (2 ints per tile) + count
  size_t off_dtab;             // decode path: DEC_DTAB_BYTES
  int max_tiles;               // upper bound of (expert, row chunk) tiles: P/(256/terms) + E + 1
  size_t bytes;
};
typedef FwdPlan DecPlan;
FwdPlan plan_forward(const ft_moe_desc& d, int T);

// decode path (matrix-core GEMV, in-kernel grouping, fused combine)
bool dec_supported(const ft_moe_desc& d, int T);
// launch shape of the decode gate/up kernel: staged-activation loop, 8-row
// tiles per workgroup, workgroups (sized for min(P, E) distinct experts)
struct DecGateupShape { bool xl; int ntw; unsigned grid; };
DecGateupShape dec_gateup_shape(const ft_moe_desc& d, int T);
// the fused route + forward selects inside the gate/up kernel, once per
// workgroup: worth it only while the grid runs in about one round
constexpr unsigned DEC_FUSE_MAX_GRID = 1024;
// in-kernel selection up to this many experts: every gate/up workgroup ranks
// them, E^2 compares in all; at 256 experts (one token) that took 4.6 us in
// each workgroup, and the two separate calls measured 3 us faster per layer
constexpr int DEC_FUSE_MAX_E = 128;
// route_logits != nullptr: the gate/up kernel selects the top-k from these
// fp64 logits itself (ids and gates are then ignored) and stores the
// selection in ids_out / gates_out.
hipError_t launch_dec_forward(const ft_moe_desc& d, const DecPlan& pl, const void* x, const int32_t* ids,
                              const uint32_t* mask, const int32_t* slot_ids, const void* pool, const float* gates,
                              float* out, char* ws, hipStream_t st, const double* route_logits = nullptr,
                              const float* sel_bias = nullptr, int32_t* ids_out = nullptr,
                              float* gates_out = nullptr);

// permutation (grouping pairs by expert, stable in pair order)
hipError_t launch_permute(const FwdPlan& pl, const int32_t* ids, const uint32_t* mask, char* ws,
                          hipStream_t st);

// decode-sized grouped GEMV: gate/up + SwiGLU, then down, then combine
hipError_t launch_gemv_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                               const void* pool, const float* gates, float* out, char* ws, hipStream_t st);

// large-batch paths on gfx950 matrix cores: MXFP4 weights on the scaled
// fp8 x fp4 MFMA, bf16 weights on the bf16 MFMA
constexpr int MFMA_MIN_TOKENS = 256;
bool mfma_supported(const ft_moe_desc& d, int T);
bool mfma_bf16_supported(const ft_moe_desc& d, int T);
// tile list and work items of the grouped GEMMs (one workgroup per expert)
hipError_t launch_build_tiles(const int32_t* offsets, int E, int32_t* tiles, int32_t* n_tiles, int32_t* work_a,
                              int n_nt_a, int32_t* work_b, int n_nt_b, int chunk, hipStream_t st);
// out += part over n floats
hipError_t launch_add_partial(float* out, const float* part, int64_t n, hipStream_t st);
// fixed-j-order fp32 combine over the bf16 expert outputs y [P, H] at off_y
hipError_t launch_combine(const FwdPlan& pl, const int32_t* pos, const float* gates, float* out, char* ws,
                          hipStream_t st);
hipError_t launch_mfma_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                               const void* pool, const float* gates, float* out, char* ws, hipStream_t st);
hipError_t launch_mfma_bf16_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                                    const void* pool, const float* gates, float* out, char* ws, hipStream_t st);

constexpr int PERM_CHUNK = 1024;  // pairs per permute block (one per thread)

}  // namespace ft
