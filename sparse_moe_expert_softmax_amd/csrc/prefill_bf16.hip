// Prefill-sized grouped expert GEMM on gfx950 bf16 matrix cores, for layers
// whose expert weights are stored in bf16 or in the NVFP4-like format.
//
// At prefill every expert sees hundreds of tokens, so its FFN is a dense
// contraction C_e = A_e . W_e^T.  Activations x are bf16 inputs; bf16
// weights are used as stored, and NVFP4 weights (E2M1 codes, an E4M3 scale
// per 16 along K, an fp32 scale per matrix) are expanded to bf16 on their way
// into LDS: code x block scale has at most 6 significant bits, so the bf16
// value is exact, and the per-matrix fp32 scale multiplies the accumulators.
// Both operands then feed v_mfma_f32_16x16x32_bf16 exactly, with fp32
// accumulation; nothing is quantised on the way in.  h = silu(gate) * up is
// rounded once to bf16 (nearest even) for the down projection, and each
// expert output y is rounded to bf16 before the fp32 combine, as on the
// MXFP4 prefill path.
//
// Operand layout of that instruction (lane l, group g = l / 16):
//   A: row l % 16, k = 8 g .. 8 g + 7 (eight bf16, 16 bytes)
//   B: column l % 16, the same k
//   result: D[4 g + i][l % 16], i = 0..3
// A is the activation rows (pair rows), B the weight rows, so a lane's
// accumulator holds four pair rows of one weight row.
//
// Tiles: a workgroup (8 waves) computes up to 256 pair rows of one expert x
// 256 weight rows; K advances 32 per step (64 bytes per row).  Operands go
// global -> LDS through the buffer unit's LDS-DMA path, four stages deep
// (while step q computes, the loads of steps q+1 .. q+3 are in flight), so
// no registers are spent on staging.  NVFP4 weights take a detour: each wave
// DMAs the raw codes and scales of its own 32 weight rows two steps ahead
// into a small ring, and expands the next step's rows into the stage right
// after its own products.  Tile list and work items are the ones the MXFP4
// path uses (one tile list per expert chunk, weight tiles of one chunk side
// by side on one XCD).
//   gate/up: weight rows = 128 gate rows + the same 128 up rows; epilogue
//            h = silu(gate) * up in bf16, staged through LDS for 16-byte stores.
//   down:    weight rows = 256 rows of D; epilogue stores y rounded to bf16.
// The combine (fixed j order, fp32) is the MXFP4 path's kernel.
#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace ft {

typedef __bf16 bfx8_t __attribute__((ext_vector_type(8)));
typedef float fx4_t __attribute__((ext_vector_type(4)));
typedef float fx2_t __attribute__((ext_vector_type(2)));

constexpr int BF_BM = 256;               // pair rows per tile
constexpr int BF_BN = 256;               // weight rows per tile
constexpr int BF_BK = 32;                // K per step
constexpr int BF_ROWB = 2 * BF_BK;       // bytes of one row per step
constexpr int BF_OPB = BF_BM * BF_ROWB;  // bytes of one operand per step (16 KB)
constexpr int BF_STG = 2 * BF_OPB;       // A + B per stage
constexpr int BF_NSTG = 4;               // stages
constexpr int BF_HSTR = 72;              // row stride (bf16) of the h staging tile
constexpr int BF_RAW = 768;              // NVFP4 raw bytes per wave and step: 32 rows x 16 B codes + 256 B scales

enum { BF_GATEUP = 0, BF_DOWN = 1 };

struct BfGemmArgs {
  const uint8_t* a;        // A rows: x [T, H] (gate/up) or h [P, I] (down), bf16
  int64_t a_bytes;         // size of that array (< 2^31)
  const int32_t* perm;     // sorted position -> pair index
  const int32_t* offsets;  // [E+2]
  const int32_t* tiles;    // tile list
  const int32_t* n_tiles;
  const int32_t* work;     // work items of this GEMM
  const int32_t* slot_ids; // per pair (nullable)
  const uint8_t* pool;
  int64_t stride;
  __bf16* h;               // gate/up out: [P, I]
  __bf16* y;               // down out: [P, H]
  int H, I, k, n_ntiles;
};

__device__ __forceinline__ bfx8_t bf_as_x8(uint4 v) {
  bfx8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Buffer load of 4 bytes per lane straight into LDS (lane l at lds + 4 l); see bg_dma16.
__device__ __forceinline__ void bf_dma4(bg_i32x4_t rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// 8 E2M1 codes (one dword, low nibble first) times an E4M3 block scale s ->
// 8 bf16 packed in 16 bytes.  Each product has at most 6 significant bits, so
// the bf16 conversion is exact.
__device__ __forceinline__ uint4 nv8_bf16(uint32_t q, float s) {
  uint32_t w[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const fx2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q >> (8 * b), 1.0f, 0);
    const uint32_t lo = __float_as_uint(v[0] * s) >> 16, hi = __float_as_uint(v[1] * s) & 0xFFFF0000u;
    w[b] = lo | hi;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Wave w: row blocks 16 (wm + 4 i), i = 0..3, wm = w & 3 (every wave holds a
// quarter of any prefix of rows); weight rows 128 (w >> 2) .. +127 of the
// tile (gate/up: 64 gate + the same 64 up rows).
// LDS (A and B alike): row r (64 B) at r * 64, 16-byte chunk c at
// 16 (c ^ ((r >> 1) & 3)); the operand reads (16 rows x 4 chunks per
// instruction) then spread over all banks.
template <int MODE, int WD>
__global__ void __launch_bounds__(512, 1) bf_gemm256_kernel(BfGemmArgs ga) {
  constexpr bool NV = WD == FT_NVFP4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[BF_NSTG * BF_STG + (NV ? 2 * 8 * BF_RAW : 0)];
  // workgroups map XCD-major over the actual work items (the grid is sized
  // for the most tiles possible): consecutive items run on one XCD
  const int n_items = *ga.n_tiles * ga.n_ntiles;
  const int per_xcd = (n_items + 7) / 8;
  const int xk = blockIdx.x / 8;
  if (xk >= per_xcd) return;
  const int w = (blockIdx.x % 8) * per_xcd + xk;
  if (w >= n_items) return;
  const int item = ga.work[w];
  const int tile = item & 0xFFFFF, ntile = item >> 20;
  const int e = ga.tiles[2 * tile], m0 = ga.tiles[2 * tile + 1];
  const int m_lim = ga.offsets[e + 1];
  const int nv = (m_lim - m0 < BF_BM) ? m_lim - m0 : BF_BM;  // valid pair rows of this tile
  const int K = (MODE == BF_GATEUP) ? ga.H : ga.I;
  const int nks = K / BF_BK;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 3, wn = wv >> 2;

  // a failed lookup (negative slot) reads no weights (a buffer of zero bytes
  // returns zeros) and the down epilogue stores NaN for the expert's rows
  const int slot = ga.slot_ids ? ga.slot_ids[ga.perm[m0]] : e;
  const bool poisoned = slot < 0;
  const uint8_t* rec = ga.pool + (poisoned ? 0 : (int64_t)slot * ga.stride);
  const RecordLayout L = record_layout(ga.H, ga.I, WD);
  const bg_i32x4_t rA = bg_rsrc(ga.a, ga.a_bytes);
  const bg_i32x4_t rB = bg_rsrc(rec, poisoned ? 0 : L.bytes);

  // ---- LDS-DMA sources: instruction t of this wave fills rows 16 j .. 16 j + 15
  // of an operand, j = wv + 8 t; lane -> row 16 j + lane / 4, physical chunk
  // lane % 4, logical chunk (lane % 4) ^ ((row >> 1) & 3).  The K step rides
  // in the scalar offset.  A rows past the tile's valid rows read the array's
  // first row (results discarded).  Row sources come from clamped indices
  // first (a guarded load per row would be a load and a full wait each).
  const int cl = (lane & 3) ^ ((lane >> 3) & 3);
  int voA[2], voB[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 16 * (wv + 8 * t) + (lane >> 2);
    const int rr = r < nv ? r : 0;
    const int src = (MODE == BF_GATEUP) ? ga.perm[m0 + rr] / ga.k : m0 + rr;
    voA[t] = (r < nv ? src * (2 * K) : 0) + 16 * cl;
  }
  // tile weight row n -> matrix and row within it
  auto wmat = [&](int n) { return (MODE == BF_GATEUP) ? (n < 128 ? 0 : 1) : 2; };
  auto wrow = [&](int n) { return (MODE == BF_GATEUP) ? ntile * 128 + (n & 127) : ntile * 256 + n; };
  int voS = 0;
  if constexpr (!NV) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = 16 * (wv + 8 * t) + (lane >> 2);
      voB[t] = (int)(L.code_off[wmat(n)] + (int64_t)wrow(n) * (2 * K)) + 16 * cl;
    }
  } else {
    // raw NVFP4 bytes of this wave's weight rows 32 wv .. 32 wv + 31, per step:
    // codes as two dword loads (lane -> row 32 wv + 16 t + lane / 4, dword
    // lane % 4 of the row's 16 bytes), block scales as one dword load per row
    // (lane % 32; the dword holds the scales of an even step and the next one)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = 32 * wv + 16 * t + (lane >> 2);
      voB[t] = (int)(L.code_off[wmat(n)] + (int64_t)wrow(n) * (K / 2)) + 4 * (lane & 3);
    }
    const int n = 32 * wv + (lane & 31);
    voS = (int)(L.scale_off[wmat(n)] + (int64_t)wrow(n) * (K / 16));
  }

  const uint32_t lbase = bg_lds_addr(smem);
  // bf16 weights: both operands of step s into stage STG (four loads)
#define BF_DMA(STG, s)                                                                              \
  do {                                                                                              \
    const uint32_t l_ = lbase + (STG) * BF_STG;                                                     \
    const int ko_ = (s) * BF_ROWB;                                                                  \
    bg_dma16(rA, l_ + 1024 * wv, voA[0], ko_);                                                      \
    bg_dma16(rA, l_ + 1024 * (wv + 8), voA[1], ko_);                                                \
    bg_dma16(rB, l_ + BF_OPB + 1024 * wv, voB[0], ko_);                                             \
    bg_dma16(rB, l_ + BF_OPB + 1024 * (wv + 8), voB[1], ko_);                                       \
  } while (0)
  // NVFP4 weights: the activations of step s into stage STG (two loads) ...
#define BF_DMA_A(STG, s)                                                                            \
  do {                                                                                              \
    const uint32_t l_ = lbase + (STG) * BF_STG;                                                     \
    const int ko_ = (s) * BF_ROWB;                                                                  \
    bg_dma16(rA, l_ + 1024 * wv, voA[0], ko_);                                                      \
    bg_dma16(rA, l_ + 1024 * (wv + 8), voA[1], ko_);                                                \
  } while (0)
  // ... and this wave's raw weight bytes of step s into ring slot SL (three loads)
  const uint32_t rawb = lbase + BF_NSTG * BF_STG + wv * BF_RAW;
#define BF_DMA_RAW(SL, s)                                                                           \
  do {                                                                                              \
    const uint32_t r_ = rawb + (SL) * (8 * BF_RAW);                                                 \
    bf_dma4(rB, r_, voB[0], (s) * 16);                                                              \
    bf_dma4(rB, r_ + 256, voB[1], (s) * 16);                                                        \
    bf_dma4(rB, r_ + 512, voS, ((s) & ~1) * 2);                                                     \
  } while (0)
  // expand this wave's 32 weight rows of step s (raw ring slot SL) to bf16 in
  // stage STG: lane -> row 32 wv + lane / 2, codes 16 (lane % 2) .. + 15
#define BF_CONV(STG, SL, s)                                                                         \
  do {                                                                                              \
    const uint8_t* r_ = smem + BF_NSTG * BF_STG + ((SL) * 8 + wv) * BF_RAW;                         \
    const int rl_ = lane >> 1, hh_ = lane & 1;                                                      \
    const uint2 q_ = *reinterpret_cast<const uint2*>(r_ + 16 * rl_ + 8 * hh_);                      \
    const uint32_t sb_ = (*reinterpret_cast<const uint32_t*>(r_ + 512 + 4 * rl_) >>                 \
                          (8 * (2 * ((s) & 1) + hh_))) & 0xFFu;                                     \
    const float sv_ = e4m3_to_f32(sb_);                                                             \
    const int n_ = 32 * wv + rl_;                                                                   \
    uint8_t* d_ = smem + (STG) * BF_STG + BF_OPB + n_ * BF_ROWB;                                    \
    const int sz_ = (n_ >> 1) & 3;                                                                  \
    *reinterpret_cast<uint4*>(d_ + 16 * ((2 * hh_) ^ sz_)) = nv8_bf16(q_.x, sv_);                   \
    *reinterpret_cast<uint4*>(d_ + 16 * ((2 * hh_ + 1) ^ sz_)) = nv8_bf16(q_.y, sv_);               \
  } while (0)

  fx4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (fx4_t){0.f, 0.f, 0.f, 0.f};

  // per-lane LDS read offsets: A row block i at stage + lA + 4096 i; B
  // sub-tile s (weight rows nB0 + bsrow(s) .. + 15) at stage + BF_OPB + lB + 64 bsrow(s)
  const int sw = 16 * (g ^ ((c16 >> 1) & 3));
  const int lA = (16 * wm + c16) * BF_ROWB + sw;
  const int nB0 = (MODE == BF_GATEUP) ? 64 * wn : 128 * wn;
  const int lB = BF_OPB + (nB0 + c16) * BF_ROWB + sw;
#define BF_BSROW(s) ((MODE == BF_GATEUP) ? ((s) < 4 ? 16 * (s) : 128 + 16 * ((s) - 4)) : 16 * (s))

#define BF_STEP(STG, NB)                                                                            \
  do {                                                                                              \
    bfx8_t fa_[4], fb_[4];                                                                          \
    _Pragma("unroll") for (int i = 0; i < (NB); ++i)                                                \
      fa_[i] = bf_as_x8(*reinterpret_cast<const uint4*>(smem + (STG) * BF_STG + 4096 * i + lA));    \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                            \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                                                 \
        fb_[s] = bf_as_x8(*reinterpret_cast<const uint4*>(smem + (STG) * BF_STG + lB +              \
                                                           64 * BF_BSROW(4 * h + s)));              \
      _Pragma("unroll") for (int i = 0; i < (NB); ++i)                                              \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                                                 \
        acc[i][4 * h + s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa_[i], fb_[s], acc[i][4 * h + s], \
                                                                     0, 0, 0);                      \
    }                                                                                               \
  } while (0)
#define BF_PIN_ACC()                                                                                \
  do {                                                                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                                \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) asm volatile("" : "+v"(acc[i_][j_]));           \
  } while (0)
  // iteration for step q = q0 + J, computed from stage J; the loads of step
  // q+3 go to stage (J+3)%4, the stage every wave finished reading before
  // this iteration's barrier.  Every iteration issues four loads (past the
  // last step they repeat it into a stage nobody reads), so at the top the
  // loads of steps q+1 and q+2 may be in flight: eight.
#define BF_ITER(J, NB)                                                                              \
  do {                                                                                              \
    const int q = q0 + (J);                                                                         \
    BG_VMWAIT(8);                                                                                   \
    BG_BARRIER();                                                                                   \
    BF_DMA(((J) + 3) & 3, (q + 3 < nks ? q + 3 : nks - 1));                                         \
    BF_STEP(J, NB);                                                                                 \
    BF_PIN_ACC();                                                                                   \
  } while (0)
  // NVFP4 iteration for step q: every iteration issues three raw loads (step
  // q+2) then two activation loads (step q+3), so at the top the loads of
  // the two iterations before may be in flight (ten) and this wave's
  // expansions of step q must have reached LDS; after the products, step
  // q+1's raw loads must have landed (seven younger loads in flight) before
  // they are expanded into stage J+1, which every wave finished reading
  // three iterations ago.
#define BF_ITER_NV(J, NB)                                                                           \
  do {                                                                                              \
    const int q = q0 + (J);                                                                         \
    __builtin_amdgcn_s_waitcnt(0x0070 | 10);                                                        \
    BG_BARRIER();                                                                                   \
    BF_DMA_RAW((J) & 1, (q + 2 < nks ? q + 2 : nks - 1));                                           \
    BF_DMA_A(((J) + 3) & 3, (q + 3 < nks ? q + 3 : nks - 1));                                       \
    BF_STEP(J, NB);                                                                                 \
    BF_PIN_ACC();                                                                                   \
    BG_VMWAIT(7);                                                                                   \
    BF_CONV(((J) + 1) & 3, ((J) + 1) & 1, (q + 1 < nks ? q + 1 : nks - 1));                         \
  } while (0)
#define BF_KLOOP(NB)                                                                                \
  do {                                                                                              \
    int q0 = 0;                                                                                     \
    for (; q0 + 4 <= nks; q0 += 4) {                                                                \
      if constexpr (NV) {                                                                           \
        BF_ITER_NV(0, NB);                                                                          \
        BF_ITER_NV(1, NB);                                                                          \
        BF_ITER_NV(2, NB);                                                                          \
        BF_ITER_NV(3, NB);                                                                          \
      } else {                                                                                      \
        BF_ITER(0, NB);                                                                             \
        BF_ITER(1, NB);                                                                             \
        BF_ITER(2, NB);                                                                             \
        BF_ITER(3, NB);                                                                             \
      }                                                                                             \
    }                                                                                               \
    if constexpr (NV) {                                                                             \
      if (q0 < nks) BF_ITER_NV(0, NB);                                                              \
      if (q0 + 1 < nks) BF_ITER_NV(1, NB);                                                          \
      if (q0 + 2 < nks) BF_ITER_NV(2, NB);                                                          \
    } else {                                                                                        \
      if (q0 < nks) BF_ITER(0, NB);                                                                 \
      if (q0 + 1 < nks) BF_ITER(1, NB);                                                             \
      if (q0 + 2 < nks) BF_ITER(2, NB);                                                             \
    }                                                                                               \
  } while (0)

  if constexpr (NV) {
    // the activations of step 0, then raw step 0 and activations 1, raw 1 and
    // activations 2 (the order of iterations -2 and -1), then step 0's
    // expansion once its raw loads have landed
    BF_DMA_A(0, 0);
    BF_DMA_RAW(0, 0);
    BF_DMA_A(1, (nks > 1 ? 1 : 0));
    BF_DMA_RAW(1, (nks > 1 ? 1 : 0));
    BF_DMA_A(2, (nks > 2 ? 2 : nks - 1));
    BG_VMWAIT(7);
    BF_CONV(0, 0, 0);
  } else {
    BF_DMA(0, 0);
    BF_DMA(1, (nks > 1 ? 1 : 0));
    BF_DMA(2, (nks > 2 ? 2 : nks - 1));
  }
  {
    // row blocks 16 (wm + 4 i) of this wave that hold valid rows (at least one is run)
    const int nbr = (nv - 16 * wm + 63) / 64;
    const int nbv = nbr < 1 ? 1 : (nbr > 4 ? 4 : nbr);
    if (nbv == 4) BF_KLOOP(4);
    else if (nbv == 3) BF_KLOOP(3);
    else if (nbv == 2) BF_KLOOP(2);
    else BF_KLOOP(1);
  }
#undef BF_KLOOP
#undef BF_ITER
#undef BF_ITER_NV
#undef BF_STEP
#undef BF_PIN_ACC
#undef BF_DMA
#undef BF_DMA_A
#undef BF_DMA_RAW
#undef BF_CONV
  // NVFP4: the fp32 scale of each matrix multiplies its accumulators
  float ts0 = 1.f, ts1 = 1.f, ts2 = 1.f;
  if constexpr (NV) {
    if (!poisoned) {
      const float* tsp = reinterpret_cast<const float*>(rec + L.tscale_off);
      ts0 = tsp[0];
      ts1 = tsp[1];
      ts2 = tsp[2];
    }
  }
  BG_VMWAIT(0);     // no LDS-DMA load may still be landing in the stage buffers
  __syncthreads();  // all operand reads done: the stage buffers now hold the epilogue tiles

  // ---- epilogue: accumulator element k of (i, s) is tile row
  // 16 (wm + 4 i) + 4 g + k, weight row nB0 + bsrow(s) + c16
  if (MODE == BF_GATEUP) {
    // h columns 64 wn + 16 s + c16 of the tile's 128 (gate sub-tile s with up
    // sub-tile 4 + s), staged per wave as [wave row][64 columns] so that lane
    // l stores wave row l (tile row 16 (wm + 4 (l / 16)) + l % 16) as 128
    // contiguous bytes
    __bf16* sh = reinterpret_cast<__bf16*>(smem) + wv * 64 * BF_HSTR;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float gv = acc[i][s][k] * ts0, uv = acc[i][4 + s][k] * ts1;
          sh[(16 * i + 4 * g + k) * BF_HSTR + 16 * s + c16] = (__bf16)(gv / (1.0f + expf(-gv)) * uv);
        }
    __syncthreads();
    const int tr = 16 * (wm + 4 * (lane >> 4)) + (lane & 15);
    if (tr < nv) {
      const uint4* src = reinterpret_cast<const uint4*>(sh + lane * BF_HSTR);
      uint4* dst = reinterpret_cast<uint4*>(ga.h + (int64_t)(m0 + tr) * ga.I + ntile * 128 + 64 * wn);
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = src[q];
    }
  } else {
    __bf16* yb = ga.y + ntile * 256 + nB0 + c16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tr = 16 * (wm + 4 * i) + 4 * g + k;
        if (tr < nv) {
          __bf16* yr = yb + (int64_t)(m0 + tr) * ga.H;
#pragma unroll
          for (int s = 0; s < 8; ++s) yr[16 * s] = (__bf16)(poisoned ? __builtin_nanf("") : acc[i][s][k] * ts2);
        }
      }
  }
}

hipError_t launch_mfma_bf16_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                                    const void* pool, const float* gates, float* out, char* ws, hipStream_t st) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, T = pl.T;
  __bf16* h = reinterpret_cast<__bf16*>(ws + pl.off_h);
  __bf16* y = reinterpret_cast<__bf16*>(ws + pl.off_y);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.off_tiles);
  int32_t* n_tiles = tiles + 2 * pl.max_tiles;
  int32_t* work_a = n_tiles + 1;                                // gate/up work items
  int32_t* work_b = work_a + (size_t)pl.max_tiles * (I / 128);  // down work items
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + pl.off_offsets);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + pl.off_perm);
  const int32_t* pos = reinterpret_cast<const int32_t*>(ws + pl.off_pos);

  hipError_t err = launch_build_tiles(offsets, E, tiles, n_tiles, work_a, I / 128, work_b, H / 256, BF_BM, st);
  if (err != hipSuccess) return err;
  BfGemmArgs ga{};
  ga.perm = perm;
  ga.offsets = offsets;
  ga.tiles = tiles;
  ga.n_tiles = n_tiles;
  ga.slot_ids = slot_ids;
  ga.pool = reinterpret_cast<const uint8_t*>(pool);
  ga.stride = d.expert_stride;
  ga.H = H;
  ga.I = I;
  ga.k = d.top_k;
  // gate/up: A = x gathered by token, N = I in 128-column tiles (gate + up rows)
  ga.a = reinterpret_cast<const uint8_t*>(x);
  ga.a_bytes = (int64_t)2 * T * H;
  ga.h = h;
  ga.n_ntiles = I / 128;
  ga.work = work_a;
  // the grid covers the most items possible; surplus workgroups exit at once
  const unsigned grid_a = (unsigned)((pl.max_tiles * ga.n_ntiles + 7) / 8 * 8);
  if (d.w_dtype == FT_NVFP4) bf_gemm256_kernel<BF_GATEUP, FT_NVFP4><<<grid_a, 512, 0, st>>>(ga);
  else bf_gemm256_kernel<BF_GATEUP, FT_BF16><<<grid_a, 512, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // down: A = h by sorted position, N = H in 256-row tiles
  ga.a = reinterpret_cast<const uint8_t*>(h);
  ga.a_bytes = (int64_t)2 * pl.P * I;
  ga.y = y;
  ga.n_ntiles = H / 256;
  ga.work = work_b;
  const unsigned grid_b = (unsigned)((pl.max_tiles * ga.n_ntiles + 7) / 8 * 8);
  if (d.w_dtype == FT_NVFP4) bf_gemm256_kernel<BF_DOWN, FT_NVFP4><<<grid_b, 512, 0, st>>>(ga);
  else bf_gemm256_kernel<BF_DOWN, FT_BF16><<<grid_b, 512, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(pl, pos, gates, out, ws, st);
}

bool mfma_bf16_supported(const ft_moe_desc& d, int T) {
  return (d.w_dtype == FT_BF16 || d.w_dtype == FT_NVFP4) && d.act_dtype == FT_BF16 && T >= MFMA_MIN_TOKENS &&
         d.hidden % 256 == 0 && d.inter % 128 == 0 && (int64_t)2 * T * d.hidden < (1ll << 31) &&
         (int64_t)2 * T * d.top_k * d.inter < (1ll << 31) &&
         record_layout(d.hidden, d.inter, d.w_dtype).bytes < (1ll << 31);
}

}  // namespace ft
