// Decode-batch grouped expert GEMV on gfx950 matrix cores.
//
// At decode (a handful of tokens) the expert FFN is a bandwidth-bound
// matrix-vector product: every byte of each routed expert is read once.
// The reduction along K is done by v_mfma_f32_16x16x32_bf16 with the 16
// weight rows of a tile as the A operand and up to 16 routed tokens as the
// B columns, so no cross-lane reduction is needed and the VALU only decodes
// weights.  Weights stay in their stored format in HBM and are expanded to
// bf16 in registers: bf16 as is, MXFP4 with the hardware fp4 conversion
// (the E8M0 scale is a power of two, so the bf16 values are exact), the
// NVFP4-like format through fp32 (e2m1 * e4m3 has at most 6 significant
// bits, exact in bf16) with the fp32 tensor scale applied to the
// accumulators.  Activations are bf16 inputs (exact).  The down projection
// reads h as two bf16 terms h = hi + lo (|h - hi - lo| <= 2^-18 |h|).
//
// Two kernels per layer:
//  1. gate/up: grid = (distinct expert d) x (pair of 8-row tiles of I).
//     Each workgroup derives the expert grouping of the <= 64 (token, rank)
//     pairs itself (no separate permutation launch), and per tile splits K
//     over 4 waves (the two tiles in turn, or side by side on 8 waves),
//     sums the wave partials in LDS in a fixed order, applies SwiGLU and
//     stores g * h (gate of the pair folded in).
//  2. down + combine: work items = 16-row tiles of H x 2 halves of the
//     expert list, at most one workgroup per CU; a workgroup's items
//     (several at hidden sizes above 2048) run side by side, sharing h.
//     The gate is folded into h (h' = g_tj * h_tj), so the part of
//     out[t] = sum over routed experts of D_e h'_t that one workgroup owns is
//     one accumulation: every (expert, K chunk) job of the tile adds into the
//     same 16 x 16 (rows x tokens) accumulator.  Jobs are dealt to the 16
//     waves round-robin and the wave partials are summed in LDS in a fixed
//     order; the two halves are added into the output, which the gate/up
//     kernel zeroed.  Two addends onto zero commute exactly in IEEE
//     arithmetic, so the result does not depend on which half lands first.
// The combine is the weighted sum of partial expert outputs that the pages
// rely on for exactness (FreeToken explainer page, "how" section).
#include "common.hpp"
#include "internal.hpp"
#include "topk.hpp"

namespace ft {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int DM_WAVES = 4;
constexpr int DM_MERGE_MIN = 768;  // gate/up workgroups: merge tile pairs only if this many remain
constexpr int DM_THREADS = DM_WAVES * 64;
constexpr int DEC_RED8_BYTES = 2 * DM_WAVES * 64 * 16;  // eight waves' partials (f32x4 per lane)

// Pairs routed to this workgroup's expert, derived from the ids in LDS.
struct PairInfo {
  int n_distinct;   // distinct (kept) experts among the pairs
  int expert;       // expert handled by this workgroup (valid if d < n_distinct)
  int npairs;       // pairs routed to it
  int ntok;         // distinct tokens among them (<= T)
  // bytes, not ints: the table sits beside up to 16 staged activation rows in
  // LDS, and at hidden 6144 with 4 tokens 768 more bytes per workgroup cost a
  // third resident workgroup per CU (NVFP4 decode measured 14% slower)
  uint8_t pair[DEC_MAX_PAIRS];  // their pair indices t*k + j, ascending
  uint8_t rank[DEC_MAX_PAIRS];  // rank of each pair's token among the distinct tokens
  uint8_t tok[DEC_MAX_PAIRS];   // token of each rank
};
static_assert(DEC_MAX_PAIRS <= 256, "pair table entries are bytes");

__device__ __forceinline__ bool dm_in_mask(const uint32_t* mask, int e) {
  return mask == nullptr || ((mask[e >> 5] >> (e & 31)) & 1u);
}

// Wave 0: group the P <= 64 pairs by expert; the d-th group in order of first
// appearance goes to this workgroup.  Any fixed order works: d only chooses
// which workgroup computes which expert.  A pair starts a group when it is
// its expert's lowest pair: an LDS atomic minimum per expert (in `scr`, room
// for scr_n expert ids the caller does not need meanwhile) finds that in
// three LDS round trips, where one ballot round per distinct expert took up
// to 32 rounds; layers with more experts than scr_n take the rounds.
__device__ __forceinline__ void dm_group_pairs(const int32_t* __restrict__ ids, const uint32_t* __restrict__ mask,
                                               int P, int k, int E, int d, PairInfo* pi, int* scr, int scr_n) {
  const int lane = threadIdx.x & 63;
  int e = -1;
  bool valid = false;
  if (lane < P) {
    e = ids[lane];
    valid = e >= 0 && e < E && dm_in_mask(mask, e);
  }
  int n = 0;
  uint64_t mine = 0;
  int my_e = -1;
  if (E <= scr_n) {
    if (valid) scr[e] = 64;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stores land before the minima
    __builtin_amdgcn_wave_barrier();
    if (valid) atomicMin(&scr[e], lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const bool lead = valid && scr[e] == lane;
    const uint64_t fm = __ballot(lead);
    const uint64_t blw = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    n = __popcll(fm);
    const uint64_t ld = __ballot(lead && __popcll(fm & blw) == d);  // the lane that starts group d
    if (ld) {
      my_e = __builtin_amdgcn_readlane(e, __builtin_ctzll(ld));
      mine = __ballot(valid && e == my_e);
    }
  } else {
    uint64_t todo = __ballot(valid);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int el = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(valid && e == el);
      if (n == d) { mine = m; my_e = el; }
      todo &= ~m;
      ++n;
    }
  }
  // pairs ascend, so their tokens do not decrease; a pair is its token's
  // first when no pair of the same token sits below it (a token lists an
  // expert more than once only if the caller's ids repeat it)
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int t0 = (lane / k) * k;  // first pair of this lane's token
  const uint64_t same_below = below & ~((t0 == 0) ? 0ull : (~0ull >> (64 - t0)));
  const bool in = (mine >> lane) & 1ull;
  const uint64_t first = __ballot(in && (mine & same_below) == 0ull);
  if (in) {
    const int q = __popcll(mine & below), r = __popcll(first & below);
    pi->pair[q] = (uint8_t)lane;
    pi->rank[q] = (uint8_t)(r - (((first >> lane) & 1ull) ? 0 : 1));
    if ((first >> lane) & 1ull) pi->tok[r] = (uint8_t)(lane / k);
  }
  if (lane == 0) {
    pi->n_distinct = n;
    pi->expert = my_e;
    pi->npairs = __popcll(mine);
    pi->ntok = __popcll(first);
  }
}

constexpr int DD_WAVES = 16;
constexpr int DD_THREADS = DD_WAVES * 64;
constexpr int DD_MAXT = 16;  // token columns of the accumulator
constexpr int DD_MAX_GRID = 256;  // down-projection workgroups at most (one per CU)

struct DownInfo {
  int n_distinct;
  int slot[DEC_MAX_PAIRS];                 // record slot of each distinct expert (-1: failed lookup)
  int pair[DEC_MAX_PAIRS][DD_MAXT];        // pair index of (expert d, token t), -1 if t not routed to d
};

// One wave: every kept (expert, token) pair, grouped by (expert, occurrence)
// in order of first appearance.  A group holds at most one pair per token:
// a token that lists an expert twice puts its second pair in a group of its
// own (same expert and slot), so every pair's term reaches the output.
__device__ __forceinline__ void dd_group_all(const int32_t* __restrict__ ids, const uint32_t* __restrict__ mask,
                                             const int32_t* __restrict__ slot_ids, int P, int k, int E,
                                             DownInfo* di) {
  const int lane = threadIdx.x & 63;
  int e = -1;
  bool valid = false;
  if (lane < P) {
    e = ids[lane];
    valid = e >= 0 && e < E && dm_in_mask(mask, e);
  }
  // occurrence of e among this token's earlier ranks
  const int j = lane % k;
  int occ = 0;
  for (int jj = 1; jj < k; ++jj) {
    const int prev = __shfl(e, lane - jj, 64);
    occ += (jj <= j && prev == e) ? 1 : 0;
  }
  const int key = valid ? (e | (occ << 16)) : -1;
  for (int q = lane; q < DEC_MAX_PAIRS * DD_MAXT; q += 64) (&di->pair[0][0])[q] = -1;
  uint64_t todo = __ballot(valid);
  int n = 0;
  int my_d = -1;
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int el = __builtin_amdgcn_readlane(e, leader);
    const int kl = __builtin_amdgcn_readlane(key, leader);
    const uint64_t m = __ballot(valid && key == kl);
    if ((m >> lane) & 1ull) my_d = n;
    if (lane == leader) di->slot[n] = slot_ids ? slot_ids[leader] : el;
    todo &= ~m;
    ++n;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (valid) di->pair[my_d][lane / k] = lane;
  if (lane == 0) di->n_distinct = n;
}

// ------------------------------------------------------------ weight tiles --
// Chunk = the K extent one lane group covers per step: 64 for bf16 (two
// MFMAs, 8 contiguous K each), 128 for the fp4 formats (one 32-element block
// per lane group, four MFMAs).  Actual k of MFMA j, lane group g, element e:
//   bf16: c*64  + 32*j + 8*g + e        fp4: c*128 + 32*g + 8*j + e
template <int WD> struct Chunk { static constexpr int K = (WD == FT_BF16) ? 64 : 128; static constexpr int NM = (WD == FT_BF16) ? 2 : 4; };

template <int WD>
__device__ __forceinline__ int kofs(int c, int j, int g) {
  if constexpr (WD == FT_BF16) return c * 64 + 32 * j + 8 * g;
  else return c * 128 + 32 * g + 8 * j;
}

// Raw bytes of one lane's share of a chunk, loaded before any decode so that
// the loads of several chunks can be in flight together.
template <int WD> struct RawW;
template <> struct RawW<FT_BF16> { uint4 q[2]; };
template <> struct RawW<FT_MXFP4> { uint4 q; uint32_t s; };
template <> struct RawW<FT_NVFP4> { uint4 q; uint32_t s; };

struct WMat {
  const uint8_t* codes;
  const uint8_t* scales;
  float tscale;
  int K;
};

template <int WD>
__device__ __forceinline__ WMat wmat(const uint8_t* rec, const RecordLayout& L, int m, int K) {
  WMat w;
  w.codes = rec + L.code_off[m];
  w.scales = rec + L.scale_off[m];
  w.K = K;
  w.tscale = 1.0f;
  if constexpr (WD == FT_NVFP4) w.tscale = reinterpret_cast<const float*>(rec + L.tscale_off)[m];
  return w;
}

template <int WD>
__device__ __forceinline__ void load_raw(const WMat& w, int row, int c, int g, RawW<WD>& r) {
  if constexpr (WD == FT_BF16) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(w.codes) + (int64_t)row * w.K;
    r.q[0] = *reinterpret_cast<const uint4*>(base + kofs<WD>(c, 0, g));
    r.q[1] = *reinterpret_cast<const uint4*>(base + kofs<WD>(c, 1, g));
  } else {
    const int k0 = c * 128 + 32 * g;  // 32 elements = 16 bytes of codes
    r.q = *reinterpret_cast<const uint4*>(w.codes + ((int64_t)row * w.K + k0) / 2);
    if constexpr (WD == FT_MXFP4) {
      r.s = w.scales[(int64_t)row * (w.K / 32) + k0 / 32];
    } else {  // two E4M3 block scales, blocks of 16 (adjacent, 2-byte aligned: one 16-bit load)
      r.s = *reinterpret_cast<const uint16_t*>(w.scales + (int64_t)row * (w.K / 16) + k0 / 16);
    }
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// 8 E2M1 codes (one dword) -> 8 bf16, each times `scale` (a power of two).
__device__ __forceinline__ bf16x8_t fp4x8_bf16(uint32_t q, float scale) {
  union { bf16x2_t h[4]; bf16x8_t v; } u;
  u.h[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  u.h[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q >> 8, scale, 0);
  u.h[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q >> 16, scale, 0);
  u.h[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q >> 24, scale, 0);
  return u.v;
}

// 8 E2M1 codes times an arbitrary fp32 block scale (exact products, so the
// bf16 conversion, one v_cvt_pk_bf16_f32 per pair, does not round) -> bf16.
__device__ __forceinline__ bf16x8_t fp4x8_bf16_mul(uint32_t q, float s) {
  bf16x8_t r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q >> (8 * b), 1.0f, 0);
    r[2 * b] = (__bf16)(v[0] * s);
    r[2 * b + 1] = (__bf16)(v[1] * s);
  }
  return r;
}

// A lane's block scale(s) for one chunk, converted once before the chunk's
// products (MXFP4: one E8M0 scale; NVFP4: the E4M3 scales of its two blocks
// of 16), not once per product.
struct ChunkScale { float s0, s1; };
template <int WD>
__device__ __forceinline__ ChunkScale chunk_scale(const RawW<WD>& r) {
  if constexpr (WD == FT_MXFP4) {
    const float s = e8m0_to_f32(r.s);
    return {s, s};
  } else if constexpr (WD == FT_NVFP4) {
    return {e4m3_to_f32(r.s & 0xFFu), e4m3_to_f32(r.s >> 8)};
  } else {
    return {1.f, 1.f};
  }
}

// A operand (weights) of MFMA j of a chunk.
template <int WD>
__device__ __forceinline__ bf16x8_t decode_a(const RawW<WD>& r, int j, ChunkScale cs) {
  if constexpr (WD == FT_BF16) {
    return as_bf16x8(r.q[j]);
  } else if constexpr (WD == FT_MXFP4) {
    const uint32_t q = (j == 0) ? r.q.x : (j == 1) ? r.q.y : (j == 2) ? r.q.z : r.q.w;
    return fp4x8_bf16(q, cs.s0);
  } else {
    const uint32_t q = (j == 0) ? r.q.x : (j == 1) ? r.q.y : (j == 2) ? r.q.z : r.q.w;
    return fp4x8_bf16_mul(q, (j < 2) ? cs.s0 : cs.s1);
  }
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 round-to-nearest-even of a finite fp32 value
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// -------------------------------------------------------------- gate / up --
// A workgroup covers 8 rows of h for one expert: the 16 A-operand rows are the
// 8 gate rows (tile rows 0-7) and the same 8 up rows (tile rows 8-15), so one
// accumulator chain carries both and the grid has I/8 tiles per expert.
//
// Two options for the fp4 formats, where a chunk's codes are only 16 bytes
// per lane and every further small load per chunk costs as much L1 work:
//  XL:  the token group's activation rows are staged once in LDS (dynamic
//       shared memory, row stride H + 8) and the MFMA's B operand is read
//       from there, instead of loading it from memory for every chunk;
//  GRP: each wave takes a contiguous quarter of the chunks, four at a time,
//       and loads the block scales of those four chunks with one 16-byte
//       (MXFP4) or two 16-byte (NVFP4) loads per lane instead of one or two
//       byte loads per chunk.
// Weight scales of MXFP4 for chunk c, lane group g: byte 4c + g of the row;
// NVFP4: bytes 8c + 2g and 8c + 2g + 1.
// In-kernel routing for the fused route + forward call (at most 128
// experts): the fp64 logits come from the router's logit kernel; every
// gate/up workgroup selects the top-k of each token itself instead of waiting
// for a separate selection launch (one token with renormalised gates: all
// four waves rank the experts; otherwise one wave per token), and workgroup 0
// stores the selection as the call's outputs.  logits == nullptr: ids and
// gates are inputs.  The kernel is instantiated per logits-per-lane count
// (E <= 64 * RPER) so that the selection code does not raise the register
// count of the streaming loop.
struct DecRoute {
  const double* logits;   // [T, E] fp64
  const float* sel_bias;  // [T, E] selection-only bias, nullable
  int32_t* ids_out;       // [T, k]
  float* gates_out;       // [T, k]
  int renormalize;
};

// NW: waves per workgroup.  4: the workgroup's tiles run one after the other
// on all four waves.  8 (staged activations, two tiles): each tile runs on
// its own four waves, side by side, so the one staged copy of the
// activation rows serves twice the waves (NVFP4 at hidden 6144 and four
// tokens stages 49 KB per workgroup, which caps a CU at three workgroups).
template <int WD, int UNROLL, bool XL, bool GRP, int RPER, int NW>
__global__ void __launch_bounds__(NW * 64) dec_gateup_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, const uint32_t* __restrict__ mask, int P,
    int k, const void* __restrict__ pool, int64_t stride, const int32_t* __restrict__ slot_ids,
    const float* __restrict__ gates, uint16_t* __restrict__ hbuf, float* __restrict__ out, int T, int H, int I,
    int E, DecRoute route, int ntw, DownInfo* __restrict__ dtab) {
  static_assert(NW == DM_WAVES || (NW == 2 * DM_WAVES && XL && GRP && RPER == 0), "eight waves: staged loop");
  constexpr int NTH = NW * 64;
  __shared__ PairInfo pi;
  // wave partials: their own array on four waves; on eight they take the
  // place of the staged activations once every wave is done with those (the
  // dynamic LDS is then at least RED8_BYTES), so the workgroup needs no more
  // LDS than the staged rows and three fit on a CU at NVFP4's 49 KB
  __shared__ f32x4_t red_s[NW == DM_WAVES ? DM_WAVES : 1][64];
  extern __shared__ uint4 xs_dyn[];
  f32x4_t(*red)[64] = (NW == DM_WAVES) ? red_s : reinterpret_cast<f32x4_t(*)[64]>(xs_dyn);
  const int scr_bytes = (NW == DM_WAVES) ? (int)sizeof(red_s) : DEC_RED8_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, col = lane & 15;
  const int wl = wv & (DM_WAVES - 1), tsub = wv / DM_WAVES;  // wave within its tile's group, the group
  // out starts at zero: the down kernel adds its two halves into it
  for (int i = blockIdx.x * NTH + tid; i < T * H / 4; i += gridDim.x * NTH)
    reinterpret_cast<float4*>(out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  // workgroup: distinct expert d, 8-row tiles rt0 .. rt0 + ntw - 1 of I
  // (several tiles only where the activations are staged in LDS: elsewhere
  // the loop would cost the register-fed loop a wave of occupancy)
  if constexpr (!XL) ntw = 1;
  const int n_rtg = I / 8 / ntw;
  const int d = blockIdx.x / n_rtg, rt0 = (blockIdx.x % n_rtg) * ntw;
  bool ranked = false;  // one token ranked by the whole workgroup (below)
  if constexpr (RPER > 0) {
    __shared__ int32_t s_ids[DEC_MAX_PAIRS];
    __shared__ float s_gates[DEC_MAX_PAIRS];
    // one token with renormalised gates: the whole workgroup ranks the
    // experts (its LDS scratch is the reduction buffer, unused until the
    // streaming loop ends); else, or where high halves tie, a wave per token
    static_assert(sizeof(red_s) >= 3364, "selection scratch");
    ranked = (T == 1 && route.renormalize) &&
             topk_wg_one_token<RPER, DM_THREADS>(route.logits, route.sel_bias, E, k, s_ids, s_gates,
                                                 reinterpret_cast<unsigned char*>(&red[0][0]));
    if (!ranked)
      for (int t = wv; t < T; t += DM_WAVES)
        topk_one_token<RPER>(route.logits + (int64_t)t * E, route.sel_bias ? route.sel_bias + (int64_t)t * E : nullptr,
                             E, k, route.renormalize, s_ids + t * k, s_gates + t * k);
    __syncthreads();
    if (blockIdx.x == 0)
      for (int q = tid; q < P; q += NTH) {
        route.ids_out[q] = s_ids[q];
        route.gates_out[q] = s_gates[q];
      }
    ids = s_ids;
    gates = s_gates;
  }
  if (ranked && mask == nullptr) {
    // one token, no mask: pair j is rank j, and the k ranked experts are
    // distinct, so group d is pair d alone (what dm_group_pairs would find,
    // without its serial ballot rounds)
    if (tid == 0) {
      pi.n_distinct = k;
      pi.expert = (d < k) ? ids[d] : -1;
      pi.npairs = 1;
      pi.ntok = 1;
      pi.pair[0] = (uint8_t)d;
      pi.rank[0] = 0;
      pi.tok[0] = 0;
    }
  } else if (wv == 0) {
    dm_group_pairs(ids, mask, P, k, E, d, &pi, reinterpret_cast<int*>(&red[0][0]), scr_bytes / (int)sizeof(int));
  }
  // the down kernel's grouping, built here beside wave 0's so that the down
  // kernel starts its weight loads after one table copy instead of a
  // dependent load of the ids and the grouping rounds
  if (blockIdx.x == 0 && wv == 1) dd_group_all(ids, mask, slot_ids, P, k, E, dtab);
  __syncthreads();
  if (d >= pi.n_distinct) return;
  const int e = pi.expert, np = pi.npairs;
  const int slot = slot_ids ? slot_ids[pi.pair[0]] : e;
  if (slot < 0) {  // failed lookup: poison this expert's h, never read out of bounds
    if (wv == 0)
      for (int q = lane; q < np * 8 * ntw; q += 64) {
        const int p = pi.pair[q / (8 * ntw)], r = rt0 * 8 + q % (8 * ntw);
        hbuf[(int64_t)p * 2 * I + r] = 0x7FC0u;
        hbuf[(int64_t)p * 2 * I + I + r] = 0u;
      }
    return;
  }
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(pool) + (int64_t)slot * stride;
  const RecordLayout L = record_layout(H, I, WD);
  const WMat Gm = wmat<WD>(rec, L, 0, H), Um = wmat<WD>(rec, L, 1, H);
  const WMat& Wl = (col < 8) ? Gm : Um;   // this lane's A-operand matrix
  const int row0 = rt0 * 8 + (col & 7);  // and row in the first tile
  constexpr int CK = Chunk<WD>::K, NM = Chunk<WD>::NM;
  const int nchunk = H / CK;

  uint16_t* xs = reinterpret_cast<uint16_t*>(xs_dyn);
  const int XS = H + 8;  // LDS row stride of the staged activations (elements)
  // chunk of pass c0, step u: strided over the waves, or (GRP) a contiguous
  // quarter per wave taken four chunks at a time
  const int cpw = nchunk / DM_WAVES;
  const int cbeg = GRP ? wl * cpw : wv, cend = GRP ? cbeg + cpw : nchunk;
  const int cstep = GRP ? UNROLL : DM_WAVES * UNROLL, ustep = GRP ? 1 : DM_WAVES;
  bool staged = false;  // activation rows of the expert's distinct tokens (at most 16) in LDS, once
  for (int tg = 0; tg < np; tg += 16) {
    const bool tok_ok = tg + col < np;
    const int t = tok_ok ? pi.pair[tg + col] / k : 0;
    const int xrow = tok_ok ? pi.rank[tg + col] : 0;  // LDS row of this column's token
    const float gate = (tok_ok && wl == 0) ? gates[pi.pair[tg + col]] : 0.f;  // issued before the stream
    const uint16_t* xr = x + (int64_t)t * H;
    // this workgroup's tiles, activations staged once: one after the other,
    // or (eight waves) tile rt0 + tsub on this wave's group
    const int rt_beg = (NW == DM_WAVES) ? rt0 : rt0 + tsub, rt_end = (NW == DM_WAVES) ? rt0 + ntw : rt_beg + 1;
    for (int rt = rt_beg; rt < rt_end; ++rt) {
      const int row = row0 + 8 * (rt - rt0);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!XL && !GRP) {
        for (int c0 = wv; c0 < nchunk; c0 += DM_WAVES * UNROLL) {
          RawW<WD> rw[UNROLL];
          uint4 xb[UNROLL][NM];
  #pragma unroll
          for (int u = 0; u < UNROLL; ++u) {
            const int c = c0 + u * DM_WAVES;
            if (c < nchunk) {
              load_raw<WD>(Wl, row, c, g, rw[u]);
  #pragma unroll
              for (int j = 0; j < NM; ++j)
                xb[u][j] = tok_ok ? *reinterpret_cast<const uint4*>(xr + kofs<WD>(c, j, g)) : make_uint4(0, 0, 0, 0);
            }
          }
  #pragma unroll
          for (int u = 0; u < UNROLL; ++u) {
            const int c = c0 + u * DM_WAVES;
            if (c < nchunk) {
              const ChunkScale cs = chunk_scale<WD>(rw[u]);
  #pragma unroll
              for (int j = 0; j < NM; ++j) acc = mfma(decode_a<WD>(rw[u], j, cs), as_bf16x8(xb[u][j]), acc);
            }
          }
        }
      } else {
        // every wave runs the first pass (its chunks are guarded), so the barrier
        // that publishes the staged activations is reached by all waves
        int c0 = cbeg;
        do {
          RawW<WD> rw[UNROLL];
          uint4 xb[XL ? 1 : UNROLL][NM];
          if constexpr (GRP && WD != FT_BF16) {  // four consecutive chunks, scales in one go
            const WMat& W = Wl;
            uint4 sg[(WD == FT_MXFP4) ? 1 : 2];
            if constexpr (WD == FT_MXFP4) {
              sg[0] = *reinterpret_cast<const uint4*>(W.scales + (int64_t)row * (W.K / 32) + 4 * c0);
            } else {
              const uint4* sp = reinterpret_cast<const uint4*>(W.scales + (int64_t)row * (W.K / 16) + 8 * c0);
              sg[0] = sp[0];
              sg[1] = sp[1];
            }
            uint32_t sw[8];  // the group's scale words (constant indices only: stays in registers)
            sw[0] = sg[0].x; sw[1] = sg[0].y; sw[2] = sg[0].z; sw[3] = sg[0].w;
            if constexpr (WD == FT_NVFP4) { sw[4] = sg[1].x; sw[5] = sg[1].y; sw[6] = sg[1].z; sw[7] = sg[1].w; }
    #pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              const int c = c0 + u;
              rw[u].q = *reinterpret_cast<const uint4*>(W.codes + ((int64_t)row * W.K + c * 128 + 32 * g) / 2);
              if constexpr (WD == FT_MXFP4) {
                rw[u].s = (sw[u] >> (8 * g)) & 0xFFu;
              } else {
                const uint32_t lo = sw[2 * u], hi = sw[2 * u + 1];
                rw[u].s = (((g >> 1) ? hi : lo) >> (16 * (g & 1))) & 0xFFFFu;
              }
            }
          } else {
    #pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              const int c = c0 + u * ustep;
              if (c < cend) load_raw<WD>(Wl, row, c, g, rw[u]);
            }
          }
          if constexpr (!XL) {
    #pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              const int c = c0 + u * ustep;
              if (c < cend) {
    #pragma unroll
                for (int j = 0; j < NM; ++j)
                  xb[u][j] = tok_ok ? *reinterpret_cast<const uint4*>(xr + kofs<WD>(c, j, g)) : make_uint4(0, 0, 0, 0);
              }
            }
          } else {
            if (c0 == cbeg) {
              if (!staged) {  // after the first pass's weight loads are issued: the two latencies overlap
                for (int q = tid; q < pi.ntok * (H / 8); q += NTH) {
                  const int r = q / (H / 8), c8 = q % (H / 8);
                  *reinterpret_cast<uint4*>(xs + r * XS + 8 * c8) =
                      *reinterpret_cast<const uint4*>(x + (int64_t)pi.tok[r] * H + 8 * c8);
                }
                staged = true;
              }
              __syncthreads();  // staged activations visible (first pass only)
            }
          }
    #pragma unroll
          for (int u = 0; u < UNROLL; ++u) {
            const int c = c0 + u * ustep;
            if (c < cend) {
              const ChunkScale cs = chunk_scale<WD>(rw[u]);
    #pragma unroll
              for (int j = 0; j < NM; ++j) {
                uint4 xv;
                if constexpr (XL) xv = tok_ok ? *reinterpret_cast<const uint4*>(xs + xrow * XS + kofs<WD>(c, j, g)) : make_uint4(0, 0, 0, 0);
                else xv = xb[u][j];
                acc = mfma(decode_a<WD>(rw[u], j, cs), as_bf16x8(xv), acc);
              }
            }
          }
          c0 += cstep;
        } while (c0 < cend);
      }
      if constexpr (NW != DM_WAVES) __syncthreads();  // every wave is done with the staged rows
      red[wv][lane] = acc;
      __syncthreads();
      const int w0 = tsub * DM_WAVES;  // first wave of this tile's group
      if (wl == 0) {
        f32x4_t s = red[w0][lane];
  #pragma unroll
        for (int w = 1; w < DM_WAVES; ++w) s += red[w0 + w][lane];
        red[w0][lane] = s;  // lanes 32-63 (tile rows 8-15) hold the up rows of lanes 0-31
      }
      __syncthreads();
      if (wl == 0 && g < 2 && tok_ok) {
        const f32x4_t sg = red[w0][lane], su = red[w0][lane + 32];
        const int p = pi.pair[tg + col];
        uint16_t hi[4], lo[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = sg[i] * Gm.tscale, uv = su[i] * Um.tscale;
          const float h = gate * (gv / (1.0f + expf(-gv)) * uv);
          const uint32_t hb = bf16_rne_bits(h);
          hi[i] = (uint16_t)hb;
          lo[i] = (uint16_t)bf16_rne_bits(h - __uint_as_float(hb << 16));
        }
        // h rows of this lane: rt*8 + 4*g + i
        uint16_t* hp = hbuf + (int64_t)p * 2 * I + rt * 8 + 4 * g;
        *reinterpret_cast<uint2*>(hp) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2*>(hp + I) = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
      }
      __syncthreads();
      // eight waves: the partials overwrote the staged rows, so a further
      // group of 16 pairs (an expert listed more than 16 times) stages again
      if constexpr (NW != DM_WAVES) staged = false;
    }
  }
}

// ---------------------------------------------------------- down + combine --
// PACK (T <= 8): the MFMA's 16 token columns carry h's hi terms in columns
// 0 .. T-1 and its lo terms in columns T .. 2T-1, so one product per K slice
// covers both (and every h load fills twice the lanes); the two column
// groups are added once at the end.  Otherwise hi and lo take a product each.
// MI > 1 (packed columns; every workgroup holds at most MI items, all of
// one half, so they share their jobs' experts, chunks and h): a wave takes
// job (expert, chunk) for all of the workgroup's items at once, loading h
// once for them and the weight rows of each item's tile, with an
// accumulator per item.  The items then run side by side instead of one
// after the other, and h, which costs a job 16 VGPRs against the weights'
// 5, is loaded once per MI jobs.  Each accumulator adds the same jobs in
// the same order as the item loop below, so the results are the same.
template <int WD, int UNROLL, bool PACK, int MI>
__global__ void __launch_bounds__(DD_THREADS) dec_down_kernel(
    const uint16_t* __restrict__ hbuf, const DownInfo* __restrict__ dtab, const void* __restrict__ pool,
    int64_t stride, float* __restrict__ out, int T, int H, int I) {
  __shared__ DownInfo di;
  __shared__ f32x4_t red[DD_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, col = lane & 15;
  // the grouping the gate/up kernel's first workgroup stored
  static_assert(sizeof(DownInfo) % 4 == 0 && sizeof(DownInfo) <= DEC_DTAB_BYTES, "down table");
  for (int q = tid; q < (int)(sizeof(DownInfo) / 4); q += DD_THREADS)
    reinterpret_cast<int32_t*>(&di)[q] = reinterpret_cast<const int32_t*>(dtab)[q];
  __syncthreads();
  const int nd = di.n_distinct;
  constexpr int CK = Chunk<WD>::K, NM = Chunk<WD>::NM;
  const int nchunk = I / CK;
  const RecordLayout L = record_layout(H, I, WD);
  if constexpr (MI > 1) {
    static_assert(PACK, "items side by side: packed columns");
    const int n_items = (H / 16) * 2;
    const int half = blockIdx.x & 1;  // the grid is even: every item of this workgroup has this half
    const int ndh = (nd - half + 1) / 2;
    const int njobs = ndh * nchunk;
    bool ok[MI];
    int rowi[MI];
  #pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int item = (int)blockIdx.x + i * (int)gridDim.x;
      ok[i] = item < n_items;
      rowi[i] = (item >> 1) * 16 + col;
    }
    const bool lo = col >= T, cok = col < 2 * T;
    const int tk = lo ? col - T : col;
    f32x4_t acc[MI];
  #pragma unroll
    for (int i = 0; i < MI; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    bool poisoned = false;
    for (int j0 = wv; j0 < njobs; j0 += DD_WAVES * UNROLL) {
      RawW<WD> rw[UNROLL][MI];
      uint4 bh[UNROLL][NM];
      float ts[UNROLL];
  #pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int job = j0 + u * DD_WAVES;
        ts[u] = 0.f;
        if (job < njobs) {
          const int d = half + 2 * (job / nchunk), c = job % nchunk;
          const int slot = di.slot[d];
          const int p = cok ? di.pair[d][tk] : -1;
          if (slot < 0) {
            poisoned = true;
          } else {
            const uint8_t* rec = reinterpret_cast<const uint8_t*>(pool) + (int64_t)slot * stride;
            const WMat Dm = wmat<WD>(rec, L, 2, I);
            ts[u] = Dm.tscale;
  #pragma unroll
            for (int i = 0; i < MI; ++i)
              if (ok[i]) load_raw<WD>(Dm, rowi[i], c, g, rw[u][i]);
          }
          const uint16_t* hh = hbuf + (int64_t)(p < 0 ? 0 : p) * 2 * I + (lo ? I : 0);
  #pragma unroll
          for (int jj = 0; jj < NM; ++jj)
            bh[u][jj] = p >= 0 ? *reinterpret_cast<const uint4*>(hh + kofs<WD>(c, jj, g)) : make_uint4(0, 0, 0, 0);
        }
      }
  #pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (ts[u] != 0.f) {
  #pragma unroll
          for (int i = 0; i < MI; ++i) {
            if (!ok[i]) continue;
            f32x4_t part = {0.f, 0.f, 0.f, 0.f};
            const ChunkScale cs = chunk_scale<WD>(rw[u][i]);
  #pragma unroll
            for (int jj = 0; jj < NM; ++jj) part = mfma(decode_a<WD>(rw[u][i], jj, cs), as_bf16x8(bh[u][jj]), part);
            if constexpr (WD == FT_NVFP4) acc[i] += part * ts[u];
            else acc[i] += part;
          }
        }
      }
    }
  #pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (!ok[i]) break;
      red[wv][lane] = poisoned ? acc[i] * __builtin_nanf("") : acc[i];
      __syncthreads();
      if (wv == 0) {
        f32x4_t s = red[0][lane];
  #pragma unroll
        for (int w = 1; w < DD_WAVES; ++w) s += red[w][lane];
        const int src = (lane & ~15) | ((col + T) & 15);  // the lo column of this token
  #pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += __shfl(s[q], src, 64);
        if (col < T) {
          // exactly two addends land on each zeroed output element (one per
          // half), and (0 + a) + b == (0 + b) + a: the sum is deterministic
          float* o = out + (int64_t)col * H + (rowi[i] - col) + 4 * g;
  #pragma unroll
          for (int q = 0; q < 4; ++q) unsafeAtomicAdd(o + q, s[q]);
        }
      }
      __syncthreads();  // red is reused by the next item
    }
    return;
  }
  // work items: (16-row tile rt, half) with half s taking the distinct experts
  // d = s, s+2, ...; a workgroup takes items blockIdx.x, + gridDim.x, ... (the
  // grid is capped, so the grouping above is done once per workgroup)
  for (int item = blockIdx.x; item < (H / 16) * 2; item += gridDim.x) {
    const int rt = item >> 1, half = item & 1;
    const int ndh = (nd - half + 1) / 2;  // experts of this half
    const int row = rt * 16 + col;
    const int njobs = ndh * nchunk;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    bool poisoned = false;
    for (int j0 = wv; j0 < njobs; j0 += DD_WAVES * UNROLL) {
      RawW<WD> rw[UNROLL];
      uint4 bh[UNROLL][NM], bl[UNROLL][NM];
      float ts[UNROLL];
  #pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int job = j0 + u * DD_WAVES;
        ts[u] = 0.f;
        if (job < njobs) {
          const int d = half + 2 * (job / nchunk), c = job % nchunk;
          const int slot = di.slot[d];
          // this lane's B column: token col (hi), or token col - T (lo) when packed
          const int tk = (PACK && col >= T) ? col - T : col;
          const int p = (tk < T && col < (PACK ? 2 * T : T)) ? di.pair[d][tk] : -1;
          if (slot < 0) {
            poisoned = true;
          } else {
            const uint8_t* rec = reinterpret_cast<const uint8_t*>(pool) + (int64_t)slot * stride;
            const WMat Dm = wmat<WD>(rec, L, 2, I);
            ts[u] = Dm.tscale;
            load_raw<WD>(Dm, row, c, g, rw[u]);
          }
          const uint16_t* hh = hbuf + (int64_t)(p < 0 ? 0 : p) * 2 * I + ((PACK && col >= T) ? I : 0);
  #pragma unroll
          for (int jj = 0; jj < NM; ++jj) {
            const int ko = kofs<WD>(c, jj, g);
            bh[u][jj] = p >= 0 ? *reinterpret_cast<const uint4*>(hh + ko) : make_uint4(0, 0, 0, 0);
            if constexpr (!PACK) bl[u][jj] = p >= 0 ? *reinterpret_cast<const uint4*>(hh + I + ko) : make_uint4(0, 0, 0, 0);
          }
        }
      }
  #pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (ts[u] != 0.f) {
          f32x4_t part = {0.f, 0.f, 0.f, 0.f};
          const ChunkScale cs = chunk_scale<WD>(rw[u]);
  #pragma unroll
          for (int jj = 0; jj < NM; ++jj) {
            const bf16x8_t a = decode_a<WD>(rw[u], jj, cs);
            part = mfma(a, as_bf16x8(bh[u][jj]), part);
            if constexpr (!PACK) part = mfma(a, as_bf16x8(bl[u][jj]), part);
          }
          if constexpr (WD == FT_NVFP4) acc += part * ts[u];
          else acc += part;
        }
      }
    }
    if (poisoned) acc = acc * __builtin_nanf("");
    red[wv][lane] = acc;
    __syncthreads();
    if (wv == 0) {
      f32x4_t s = red[0][lane];
  #pragma unroll
      for (int w = 1; w < DD_WAVES; ++w) s += red[w][lane];
      if constexpr (PACK) {  // add the lo column group (col + T of the same 16-lane row group)
        const int src = (lane & ~15) | ((col + T) & 15);
  #pragma unroll
        for (int i = 0; i < 4; ++i) s[i] += __shfl(s[i], src, 64);
      }
      if (col < T) {
        // exactly two addends land on each zeroed output element, and
        // (0 + a) + b == (0 + b) + a in IEEE arithmetic: the sum is deterministic
        float* o = out + (int64_t)col * H + rt * 16 + 4 * g;
  #pragma unroll
        for (int i = 0; i < 4; ++i) unsafeAtomicAdd(o + i, s[i]);
      }
    }
    __syncthreads();  // red is reused by the next item
  }
}

static size_t dec_xl_bytes(int T, int H) {
  const int tmax = T < 16 ? T : 16;
  return (size_t)tmax * (H + 8) * 2;
}

DecGateupShape dec_gateup_shape(const ft_moe_desc& d, int T) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, P = T * d.top_k;
  const int nd_max = P < E ? P : E;
  const int nchunk = H / ((d.w_dtype == FT_BF16) ? 64 : 128);
  // Staged activations (XL: the expert's token rows in LDS, each wave a
  // contiguous quarter of the chunks) with two 8-row tiles per workgroup when
  // at least 2 * DM_MERGE_MIN tiles exist (each workgroup groups the pairs,
  // and stages activations, once for both).  Measured, same box: MXFP4 and
  // NVFP4 layers with 1,536 and more tiles 10-15% faster; the bf16 layer at
  // 2 and 4 tokens (1,536 and 3,072 tiles) 3% and 7% faster than its strided
  // register-fed loop, which it keeps at one token (768 tiles, equal there).
  DecGateupShape sh;
  const bool many = (int64_t)nd_max * (I / 8) >= 2 * DM_MERGE_MIN && (I / 8) % 2 == 0;
  if (d.w_dtype == FT_BF16)
    sh.xl = many && dec_xl_bytes(T, H) <= 56 * 1024 && nchunk % 16 == 0;
  else
    sh.xl = dec_xl_bytes(T, H) <= 56 * 1024 && nchunk % 16 == 0;
  sh.ntw = (sh.xl && many) ? 2 : 1;
  sh.grid = (unsigned)(nd_max * (I / 8 / sh.ntw));
  return sh;
}

template <int WD>
static hipError_t dec_forward_t(const ft_moe_desc& d, const DecPlan& pl, const void* x, const int32_t* ids,
                                const uint32_t* mask, const int32_t* slot_ids, const void* pool, const float* gates,
                                float* out, char* ws, const DecRoute& route, hipStream_t st) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k;
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + pl.off_h);
  DownInfo* dtab = reinterpret_cast<DownInfo*>(ws + pl.off_dtab);
  const size_t xl_bytes = dec_xl_bytes(pl.T, H);
  const DecGateupShape shp = dec_gateup_shape(d, pl.T);
  const bool xl = shp.xl;
  const int ntw = shp.ntw;
  const unsigned grid = shp.grid;
  const int rper = !route.logits ? 0 : (E <= 64 ? 1 : (E <= 128 ? 2 : 4));
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
#define DM_GATEUP(UN, XL_, GRP_, SH)                                                                   \
  do {                                                                                               \
    if (rper == 0)                                                                                   \
      dec_gateup_kernel<WD, UN, XL_, GRP_, 0, DM_WAVES><<<grid, DM_THREADS, SH, st>>>(               \
          xb, ids, mask, pl.P, k, pool, d.expert_stride, slot_ids, gates, hbuf, out, pl.T, H, I, E, route, ntw, dtab); \
    else if (rper == 1)                                                                              \
      dec_gateup_kernel<WD, UN, XL_, GRP_, 1, DM_WAVES><<<grid, DM_THREADS, SH, st>>>(               \
          xb, ids, mask, pl.P, k, pool, d.expert_stride, slot_ids, gates, hbuf, out, pl.T, H, I, E, route, ntw, dtab); \
    else                                                                                             \
      dec_gateup_kernel<WD, UN, XL_, GRP_, 2, DM_WAVES><<<grid, DM_THREADS, SH, st>>>(               \
          xb, ids, mask, pl.P, k, pool, d.expert_stride, slot_ids, gates, hbuf, out, pl.T, H, I, E, route, ntw, dtab); \
  } while (0)
  // staged loop: four chunks per wave and pass (bf16 at H 2048: two passes
  // at 74 VGPRs, six waves per SIMD, measured 0.5-1% faster than one pass of
  // eight at 110 VGPRs, four waves per SIMD)
  // fp4, staged activations, two tiles per workgroup, no in-kernel selection:
  // the two tiles on eight waves side by side where four-wave workgroups
  // would leave few waves resident, i.e. where the staged rows cap a CU at
  // three workgroups (above 40 KB) or the grid gives each of the 256 CUs at
  // most four.
  // Measured against four waves, same box: NVFP4 6144/2048/256 at four
  // tokens 213 -> 199 us per forward (49 KB staged), MXFP4 4096/2048/256 at
  // one token 33.4 -> 32.9 us (768 workgroups); MXFP4 at four tokens (33 KB,
  // ~2,700 workgroups) 92.2 us on four waves against 92.7 on eight.
  const bool eight = WD != FT_BF16 && xl && ntw == 2 && rper == 0 && (xl_bytes > 40 * 1024 || grid <= 4u * 256u);
  if (eight) {
    if constexpr (WD != FT_BF16)
      dec_gateup_kernel<WD, 4, true, true, 0, 2 * DM_WAVES>
          <<<grid, 2 * DM_THREADS, xl_bytes > (size_t)DEC_RED8_BYTES ? xl_bytes : DEC_RED8_BYTES, st>>>(
              xb, ids, mask, pl.P, k, pool, d.expert_stride, slot_ids, gates, hbuf, out, pl.T, H, I, E, route, ntw,
              dtab);
  } else if (xl)
    DM_GATEUP(4, true, true, xl_bytes);
  else
    DM_GATEUP((WD == FT_BF16) ? 6 : 4, false, false, 0);
#undef DM_GATEUP
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // one workgroup of 16 waves per CU: cap the grid at the CU count and let
  // each workgroup loop over its (tile, half) items
  const unsigned dgrid = (H / 16) * 2 < DD_MAX_GRID ? (H / 16) * 2 : DD_MAX_GRID;
  // three jobs' loads per wave and pass (fp4, per-call forwards: two 40.4 /
  // 232.7 us, three 39.7 / 229.6, four 39.8 / 232.7, five spill; MXFP4
  // 4096/2048/256 at one token, NVFP4 6144/2048/256 at four); two for fp4
  // without the packed h columns (its separate lo loads spill at three)
  constexpr int DU = 3, DUL = (WD == FT_BF16) ? 3 : 2;
#ifndef FT_DD_MI
#define FT_DD_MI 1
#endif
  const int itw = ((H / 16) * 2 + (int)dgrid - 1) / (int)dgrid;  // items per workgroup
  if (FT_DD_MI && pl.T <= 8 && itw == 2)
    dec_down_kernel<WD, 3, true, 2><<<dgrid, DD_THREADS, 0, st>>>(hbuf, dtab, pool, d.expert_stride, out, pl.T, H, I);
  else if (FT_DD_MI && pl.T <= 8 && itw == 3)
    dec_down_kernel<WD, 2, true, 3><<<dgrid, DD_THREADS, 0, st>>>(hbuf, dtab, pool, d.expert_stride, out, pl.T, H, I);
  else if (pl.T <= 8)
    dec_down_kernel<WD, DU, true, 1><<<dgrid, DD_THREADS, 0, st>>>(hbuf, dtab, pool, d.expert_stride, out, pl.T, H, I);
  else
    dec_down_kernel<WD, DUL, false, 1><<<dgrid, DD_THREADS, 0, st>>>(hbuf, dtab, pool, d.expert_stride, out, pl.T, H,
                                                                    I);
  return hipGetLastError();
}

bool dec_supported(const ft_moe_desc& d, int T) {
  if (d.act_dtype != FT_BF16) return false;
  if (d.w_dtype != FT_BF16 && d.w_dtype != FT_MXFP4 && d.w_dtype != FT_NVFP4) return false;
  const int64_t P = (int64_t)T * d.top_k;
  if (P < 1 || P > DEC_MAX_PAIRS || T > DD_MAXT) return false;
  const int ck = (d.w_dtype == FT_BF16) ? 64 : 128;
  return d.hidden % ck == 0 && d.inter % ck == 0 && d.hidden % 16 == 0 && d.inter % 16 == 0;
}

hipError_t launch_dec_forward(const ft_moe_desc& d, const DecPlan& pl, const void* x, const int32_t* ids,
                              const uint32_t* mask, const int32_t* slot_ids, const void* pool, const float* gates,
                              float* out, char* ws, hipStream_t st, const double* route_logits,
                              const float* sel_bias, int32_t* ids_out, float* gates_out) {
  const DecRoute route{route_logits, sel_bias, ids_out, gates_out, d.renormalize};
  switch (d.w_dtype) {
    case FT_BF16: return dec_forward_t<FT_BF16>(d, pl, x, ids, mask, slot_ids, pool, gates, out, ws, route, st);
    case FT_MXFP4: return dec_forward_t<FT_MXFP4>(d, pl, x, ids, mask, slot_ids, pool, gates, out, ws, route, st);
    default: return dec_forward_t<FT_NVFP4>(d, pl, x, ids, mask, slot_ids, pool, gates, out, ws, route, st);
  }
}

}  // namespace ft
