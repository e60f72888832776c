// Prefill-sized grouped expert GEMM on gfx950 scaled matrix cores.
//
// At prefill every expert sees hundreds of tokens, so the expert FFN is a
// dense contraction per expert: C_e = A_e . W_e^T.  MXFP4 weights go to the
// matrix cores as they are stored (E2M1 codes with an E8M0 scale per 32
// along K); bf16 activations cannot feed the fp8/fp6/fp4 instruction, so
// they are quantised once to MXFP8 (E4M3 elements, E8M0 scale per 32 along
// K, OCP MX v1.0 rule: shared exponent floor(log2 amax) - 8, nearest-even,
// saturating at 448).  h is quantised the same way before the down
// projection.  One instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with
// A = activations (fp8), B = weights (fp4), fp32 accumulation.
//
// Operand layout of that instruction, as measured on the device (lane l,
// group g = l / 16, row/column l % 16):
//   fp8 operand: byte p < 16 holds k = 16 g + p, byte p >= 16 holds
//                k = 64 + 16 g + (p - 16)
//   fp4 operand: nibble p (low nibble first, dwords 0-3) holds k = 32 g + p
//   scale operand: E8M0 of row/column l % 16, K block g (32 wide)
//   result: D[4 g + i][l % 16], i = 0..3
//
// Tiles: a workgroup (8 waves) computes all rows of one expert (in chunks of
// up to 256 pair rows) x 256 weight rows; K advances 128 per step.  Both
// operands and their block scales go global -> LDS through the buffer
// unit's LDS-DMA path, three steps deep, so no registers are spent on staging
// and every weight byte crosses L2 -> LDS once per expert chunk.  The tile
// list (expert, 256-row chunk) comes from the permutation; work items are
// ordered expert chunk, weight tile and mapped so that the weight tiles of
// one expert run side by side on one XCD (its L2 then serves the expert's
// activation rows to all of them).
//   gate/up: weight rows = 128 gate rows + the same 128 up rows; epilogue
//            h = silu(gate) * up, quantised to MXFP8 through LDS.
//   down:    weight rows = 256 rows of D; epilogue stores y rounded to bf16.
// The combine (fixed j order, fp32) runs as its own kernel afterwards.
#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace ft {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GM_BK = 128;     // K per step (one scaled MFMA)

// -------------------------------------------------------- E4M3 rounding --
// |v| (already divided by the block scale, finite) -> E4M3 code, nearest
// with ties to even, saturating at 448 (0x7E); sign from v.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                   // below 2^-6: subnormal grid of step 2^-9
    code = (uint32_t)rintf(a * 512.0f);  // 0..8 (8 = 2^-6, the smallest normal, code 0x08)
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);    // round the mantissa to 3 bits, ties to even
    const uint32_t e = (b >> 23) - 127u + 7u;
    code = (e << 3) | ((b >> 20) & 7u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Shared exponent of a block from its amax: floor(log2 amax) - 8, in [-127, 127];
// a zero block takes -127.  Returns the biased E8M0 byte.
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  if (!(amax > 0.0f)) return 0u;
  const uint32_t b = __float_as_uint(amax);
  int e = (int)((b >> 23) & 0xFFu) - 127;
  if (((b >> 23) & 0xFFu) == 0u) e = -118 - __builtin_clz(b & 0x7FFFFFu);  // subnormal: floor(log2(m * 2^-149))
  int x = e - 8;
  x = x < -127 ? -127 : (x > 127 ? 127 : x);
  return (uint32_t)(x + 127);
}

__device__ __forceinline__ float e8m0_f32(uint32_t s) {
  if (s == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(s << 23);
}

// Quantise 32 fp32 values to MXFP8: 32 code bytes (written to dst) and the scale byte.
__device__ __forceinline__ uint32_t quant_block32(const float* v, uint8_t* dst) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = mx8_scale_byte(amax);
  const float inv = (amax > 0.0f) ? 1.0f / e8m0_f32(sb) : 0.0f;  // exact power of two
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    w[q] = f32_to_e4m3(v[4 * q] * inv) | (f32_to_e4m3(v[4 * q + 1] * inv) << 8) |
           (f32_to_e4m3(v[4 * q + 2] * inv) << 16) | (f32_to_e4m3(v[4 * q + 3] * inv) << 24);
  }
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(w[0], w[1], w[2], w[3]);
  d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  return sb;
}

// E4M3 code -> its value (finite codes)
__device__ __forceinline__ float e4m3_val(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = (e == 0u) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// Two MXFP8 terms of 32 fp32 values: the first as quant_block32, the second
// the same quantisation of the residual v - q1 (exact in fp32: q1 is within
// a factor of two of v, or zero).  Codes to dst_hi / dst_lo, scale bytes
// returned in *s_hi / *s_lo.
__device__ __forceinline__ void quant_block32_2t(const float* v, uint8_t* dst_hi, uint8_t* dst_lo, uint32_t* s_hi,
                                                 uint32_t* s_lo) {
  *s_hi = quant_block32(v, dst_hi);
  const float sc = e8m0_f32(*s_hi);
  const uint4* c = reinterpret_cast<const uint4*>(dst_hi);
  const uint4 c0 = c[0], c1 = c[1];
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  float r[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) r[i] = v[i] - e4m3_val((w[i >> 2] >> (8 * (i & 3))) & 0xFFu) * sc;
  *s_lo = quant_block32(r, dst_lo);
}

// x [T, H] bf16 -> xq [TERMS*T, H] E4M3 + xs [TERMS*T, H/32] E8M0 (two
// terms: row 2t holds the first term of token t, row 2t+1 the second); one
// thread per 32-block.
template <int TERMS>
__global__ void __launch_bounds__(256) quant_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xs, int64_t nblocks, int bpr) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = src[q];
    const uint32_t a[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_lo(a[j]);
      v[8 * q + 2 * j + 1] = bf16_hi(a[j]);
    }
  }
  if constexpr (TERMS == 1) {
    xs[b] = (uint8_t)quant_block32(v, xq + b * 32);
  } else {
    const int64_t t = b / bpr, c = b % bpr;   // token, block within the row
    const int64_t b0 = (2 * t) * bpr + c, b1 = b0 + bpr;
    uint32_t s0, s1;
    quant_block32_2t(v, xq + b0 * 32, xq + b1 * 32, &s0, &s1);
    xs[b0] = (uint8_t)s0;
    xs[b1] = (uint8_t)s1;
  }
}

// Tile geometry of the expert GEMM (below).
constexpr int BG_BM = 256;                    // A rows per tile (pair rows x activation terms)
constexpr int BG_BN = 256;                    // weight rows per tile
constexpr int BG_ASZ = BG_BM * 128;           // A bytes per step
constexpr int BG_STG = BG_ASZ + BG_BN * 64;   // A + B bytes per step
constexpr int BG_SCL = BG_BM * 16;            // bytes of one scale group of A (or B): 16-byte row slots
constexpr int BG_HSTR = 33;                   // row stride (floats) of the h staging tile

// ------------------------------------------------------------ tile list --
// tiles[2*i] = expert, tiles[2*i+1] = first row (sorted position) of tile i
// (chunks of up to BG_BM rows);
// tiles are grouped by expert; count in *n_tiles.  Work lists (one per GEMM,
// n_nt weight tiles each): item = tile | (ntile << 20), ordered by row
// chunk, then weight tile, so that the weight tiles of one chunk run side by
// side and its activation rows stay in one L2.
// One workgroup per expert.
__global__ void __launch_bounds__(1024) build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                           int32_t* __restrict__ work_a, int n_nt_a,
                                                           int32_t* __restrict__ work_b, int n_nt_b, int chunk) {
  // Workgroup b writes expert b's entries; every workgroup first forms the
  // exclusive prefix sum of the per-expert tile counts (E <= 1024): wave scans
  // of 64 lanes, then a scan of the wave totals.
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_start, s_mt;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, eb = blockIdx.x;
  const int cnt = (t < E) ? offsets[t + 1] - offsets[t] : 0;
  const int mt_own = (cnt + chunk - 1) / chunk;
  int incl = mt_own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) { const int v = wsum[i]; wsum[i] = run; run += v; }
  }
  __syncthreads();
  if (t == eb) { s_start = wsum[w] + incl - mt_own; s_mt = mt_own; }
  if (eb == 0 && t == E - 1) *n_tiles = wsum[w] + incl;
  __syncthreads();
  const int st = s_start, mt = s_mt, o0 = offsets[eb];
  for (int i = t; i < mt; i += blockDim.x) {
    tiles[2 * (st + i)] = eb;
    tiles[2 * (st + i) + 1] = o0 + i * chunk;
  }
  for (int j = t; j < mt * n_nt_a; j += blockDim.x) work_a[st * n_nt_a + j] = (st + j % mt) | ((j / mt) << 20);
  for (int j = t; j < mt * n_nt_b; j += blockDim.x) work_b[st * n_nt_b + j] = (st + j % mt) | ((j / mt) << 20);
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int32_t* tiles, int32_t* n_tiles, int32_t* work_a,
                              int n_nt_a, int32_t* work_b, int n_nt_b, int chunk, hipStream_t st) {
  build_tiles_kernel<<<E, 1024, 0, st>>>(offsets, E, tiles, n_tiles, work_a, n_nt_a, work_b, n_nt_b, chunk);
  return hipGetLastError();
}

// -------------------------------------------------------------- the GEMM --
enum { GM_GATEUP = 0, GM_DOWN = 1 };

struct GemmArgs {
  const uint8_t* aq;       // A codes: x_q [T, K] (gate/up) or h_q [P, K] (down)
  const uint8_t* as;       // A scales [rows, K/32]
  const int32_t* perm;     // sorted position -> pair index
  const int32_t* offsets;  // [E+2]
  const int32_t* tiles;    // tile list
  const int32_t* n_tiles;
  const int32_t* work;     // work items of this GEMM
  const int32_t* slot_ids; // per pair (nullable)
  const uint8_t* pool;
  int64_t stride;
  uint8_t* hq;             // gate/up out: h codes [P, I]
  uint8_t* hs;             // gate/up out: h scales [P, I/32]
  __bf16* y;               // down out: [P, H], bf16
  int64_t a_bytes;         // size of the A code array (< 2^31)
  int H, I, k, n_ntiles;
};

// A workgroup of eight waves computes up to 256 pair rows (one expert's rows,
// or a 256-row chunk of them) x 256 weight rows; K advances 128 per step.
// All operand traffic goes global -> LDS by the buffer unit's LDS-DMA path
// (no registers held), three stages deep: while step q computes, the loads of
// steps q+1 and q+2 are in flight.  Block scales travel the same way in groups
// of three steps (12 bytes per row, landing in 16-byte slots), double-buffered.
//   wave w: row blocks wm + 4i (16 rows each, i = 0..3), wm = w & 3, so every
//           wave holds a quarter of any prefix of rows; weight rows 128*(w>>2)
//           .. +127 of the tile (gate/up: 64 gate + the same 64 up rows).
// LDS layouts (16-byte chunks XOR-swizzled against bank conflicts):
//   A: row r (128 B) at r*128, chunk c at 16*(c ^ ((r >> 1) & 7))
//   B: weight row n (64 B) at n*64, chunk c at 16*(c ^ ((n >> 1) & 3))
//   (both measured free of bank conflicts for the operand reads on gfx950)
//   scales: row r of a group at r*16 (12 bytes used), byte 4*j + g for step j, block g.
template <int MODE, int TERMS>
__global__ void __launch_bounds__(512, 1) mx_gemm256_kernel(GemmArgs ga) {
  // LDS: three operand stages, then two scale-group buffers (A rows, B rows each)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * BG_STG + 4 * BG_SCL];
  // map workgroups XCD-major over the actual work items (the grid is sized
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
  constexpr int BMP = BG_BM / TERMS;  // pair rows per tile
  const int nvp = (m_lim - m0 < BMP) ? m_lim - m0 : BMP;  // valid pair rows of this tile
  const int nv = nvp * TERMS;                              // valid A rows
  const int K = (MODE == GM_GATEUP) ? ga.H : ga.I;
  const int nks = K / GM_BK;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 3, wn = wv >> 2;

  // a failed lookup (negative slot) reads no weights (a buffer of zero bytes
  // returns zeros) and the down epilogue stores NaN for the expert's rows
  const int slot = ga.slot_ids ? ga.slot_ids[ga.perm[m0]] : e;
  const bool poisoned = slot < 0;
  const uint8_t* rec = ga.pool + (poisoned ? 0 : (int64_t)slot * ga.stride);
  const RecordLayout L = record_layout(ga.H, ga.I, FT_MXFP4);
  const bg_i32x4_t rA = bg_rsrc(ga.aq, ga.a_bytes);
  const bg_i32x4_t rAs = bg_rsrc(ga.as, ga.a_bytes / 32);
  const bg_i32x4_t rB = bg_rsrc(rec, poisoned ? 0 : L.bytes);

  // activation row of tile row r (valid rows only); with two terms, tile
  // rows 2i and 2i+1 are the first and second term of pair row i
  auto arow = [&](int r) -> int {
    if constexpr (TERMS == 1) {
      const int m = m0 + r;
      return (MODE == GM_GATEUP) ? ga.perm[m] / ga.k : m;
    } else {
      const int m = m0 + (r >> 1);
      return 2 * ((MODE == GM_GATEUP) ? ga.perm[m] / ga.k : m) + (r & 1);
    }
  };
  // tile weight row n -> matrix, row within it
  auto wmat = [&](int n) { return (MODE == GM_GATEUP) ? (n < 128 ? 0 : 1) : 2; };
  auto wrow = [&](int n) { return (MODE == GM_GATEUP) ? ntile * 128 + (n & 127) : ntile * 256 + n; };

  // ---- LDS-DMA sources (per-lane offsets fixed over K; the K step rides in
  // the scalar offset).  A: instruction t of this wave fills tile rows
  // 8j .. 8j+7, j = wv + 8t, lane -> row 8j + lane/8, physical chunk lane%8.
  // Rows past the tile's valid rows read row 0's line (results discarded).
  // the rows' sources first, from clamped indices (a guarded load per row
  // would be a load and a full wait each), then the offsets
  int srcA[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 8 * (wv + 8 * t) + (lane >> 3);
    srcA[t] = arow(r < nv ? r : 0);
  }
  int voA[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = wv + 8 * t;
    const int r = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ (((lane >> 4) + 4 * (j & 1)) & 7);
    voA[t] = (r < nv ? srcA[t] * K : 0) + 16 * c;
  }
  // B: instruction t fills tile weight rows 16j .. 16j+15, j = wv + 8t,
  // lane -> row 16j + lane/4, physical chunk lane%4.
  int voB[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = 16 * (wv + 8 * t) + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 3) & 3);
    voB[t] = (int)(L.code_off[wmat(n)] + (int64_t)wrow(n) * (K / 2)) + 16 * c;
  }
  // scales: waves 0-3 fill A rows 64*wv + lane, waves 4-7 B rows 64*(wv-4) + lane
  // (one buffer descriptor and LDS offset per wave, so a single load serves both halves)
  const bg_i32x4_t rS = (wv < 4) ? rAs : rB;
  const uint32_t lsS = (wv < 4) ? 1024 * wv : BG_SCL + 1024 * (wv - 4);
  int voS;
  {
    const int r = 64 * (wv & 3) + lane;
    if (wv < 4) voS = arow(r < nv ? r : 0) * (K / 32);
    else voS = (int)(L.scale_off[wmat(r)] + (int64_t)wrow(r) * (K / 32));
  }
  const int ngroups = (nks + 2) / 3;

  const uint32_t lbase = bg_lds_addr(smem);
  const uint32_t la0 = lbase, la1 = lbase + BG_STG, la2 = lbase + 2 * BG_STG;
  const uint32_t ls0 = lbase + 3 * BG_STG, ls1 = ls0 + 2 * BG_SCL;
#define BG_DMA(lbuf, s)                                                                             \
  do {                                                                                              \
    const int ka_ = (s) * GM_BK, kb_ = (s) * (GM_BK / 2);                                           \
    bg_dma16(rA, (lbuf) + 1024 * wv, voA[0], ka_);                                                  \
    bg_dma16(rA, (lbuf) + 1024 * (wv + 8), voA[1], ka_);                                            \
    bg_dma16(rA, (lbuf) + 1024 * (wv + 16), voA[2], ka_);                                           \
    bg_dma16(rA, (lbuf) + 1024 * (wv + 24), voA[3], ka_);                                           \
    bg_dma16(rB, (lbuf) + BG_ASZ + 1024 * wv, voB[0], kb_);                                         \
    bg_dma16(rB, (lbuf) + BG_ASZ + 1024 * (wv + 8), voB[1], kb_);                                   \
  } while (0)
  // scale group G (clamped) into a group buffer: 12 bytes per lane, landing
  // in 16-byte slots (lane l at 16*l), i.e. row 64*(wv&3) + l of the A or B half
#define BG_SDMA(lsbuf, G)                                                                           \
  do {                                                                                              \
    const int gg_ = ((G) < ngroups ? (G) : ngroups - 1) * 12;                                       \
    bg_dma12(rS, (lsbuf) + lsS, voS, gg_);                                                          \
  } while (0)

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // per-lane LDS read offsets (the rest of every address is a constant):
  //   A row block i, half h:  stage + lA[h] + 8192 i
  //   B sub-tile s:           stage + lB + bsub(s)
  //   scales (group buffer):  A: lSA + 1024 i + 4 j;  B: lSB + 16 bsrow(s) + 4 j
  const int swa = (c16 >> 1) & 7;
  const int lA0 = (16 * wm + c16) * 128 + 16 * (g ^ swa);
  const int lA1 = (16 * wm + c16) * 128 + 16 * ((g + 4) ^ swa);
  const int nB0 = (MODE == GM_GATEUP) ? 64 * wn : 128 * wn;  // first tile weight row of the wave
  const int lB = BG_ASZ + (nB0 + c16) * 64 + 16 * (g ^ ((c16 >> 1) & 3));
  const int lSA = (16 * wm + c16) * 16 + g;
  const int lSB = BG_SCL + (nB0 + c16) * 16 + g;
  // sub-tile s of the wave: weight rows nB0 + bsrow(s) .. + 15
#define BG_BSROW(s) ((MODE == GM_GATEUP) ? ((s) < 4 ? 16 * (s) : 128 + 16 * ((s) - 4)) : 16 * (s))
  auto nB = [&](int s) { return nB0 + BG_BSROW(s); };

#define BG_STEP(SOFF, SCOFF, j, NB)                                                                 \
  do {                                                                                              \
    i32x8_t fa_[4], fb_[4];                                                                         \
    int fas_[4], fbs_[4];                                                                           \
    _Pragma("unroll") for (int i = 0; i < (NB); ++i) {                                              \
      const uint4 lo_ = *reinterpret_cast<const uint4*>(smem + (SOFF) + 8192 * i + lA0);            \
      const uint4 hi_ = *reinterpret_cast<const uint4*>(smem + (SOFF) + 8192 * i + lA1);            \
      fa_[i] = (i32x8_t){(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w,                            \
                         (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w};                           \
      fas_[i] = smem[(SCOFF) + 1024 * i + 4 * (j) + lSA];                                            \
    }                                                                                               \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                            \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                               \
        const uint4 b_ = *reinterpret_cast<const uint4*>(smem + (SOFF) + 64 * BG_BSROW(4 * h + s) + lB); \
        fb_[s] = (i32x8_t){(int)b_.x, (int)b_.y, (int)b_.z, (int)b_.w, 0, 0, 0, 0};                 \
        fbs_[s] = smem[(SCOFF) + 16 * BG_BSROW(4 * h + s) + 4 * (j) + lSB];                         \
      }                                                                                             \
      _Pragma("unroll") for (int i = 0; i < (NB); ++i)                                              \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                                                 \
        acc[i][4 * h + s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                       \
            fa_[i], fb_[s], acc[i][4 * h + s], 0, 4, 0, fas_[i], 0, fbs_[s]);                       \
    }                                                                                               \
  } while (0)
#define BG_PIN_ACC()                                                                                \
  do {                                                                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                                \
    _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) asm volatile("" : "+v"(acc[i_][j_]));           \
  } while (0)
  // iteration for step q = q0 + J (stage buffer cur = st[J], the loads of
  // step q+2 go to st[(J+2)%3]; scale group q0/3 in scur, the next group is
  // loaded into snxt at J = 0).  Loads per iteration, in issue order: [J = 0:
  // one scale load] then six operand loads (while q+2 < nks).  At the top
  // this wave's loads of step q must have landed: allowed in flight are the
  // loads of step q+1 and, at J = 1, the scale load issued just before them.
#define BG_ITER(J, QO, CUR, lnxt2, SCUR, lsnxt, NB)                                                 \
  do {                                                                                              \
    const int q = q0 + (QO);                                                                        \
    if ((J) == 1) BG_VMWAIT(7); else BG_VMWAIT(6);                                                  \
    BG_BARRIER();                                                                                   \
    if ((J) == 0) BG_SDMA(lsnxt, q / 3 + 1);                                                        \
    BG_DMA(lnxt2, (q + 2 < nks ? q + 2 : nks - 1));                                                 \
    BG_STEP((CUR) * BG_STG, 3 * BG_STG + (SCUR) * 2 * BG_SCL, J, NB);                               \
    BG_PIN_ACC();                                                                                   \
  } while (0)
  // steps q0 .. q0+5: stage buffers 0 1 2 0 1 2, scale groups in buffer 0
  // then 1.  Every iteration issues the same loads (past the last step they
  // repeat it into a buffer nobody reads), so the wait counts are the same
  // everywhere.  NB = row blocks this wave computes (the rest are padding).
#define BG_KLOOP(NB)                                                                                \
  do {                                                                                              \
    int q0 = 0;                                                                                     \
    for (; q0 + 6 <= nks; q0 += 6) {                                                                \
      BG_ITER(0, 0, 0, la2, 0, ls1, NB);                                                            \
      BG_ITER(1, 1, 1, la0, 0, ls1, NB);                                                            \
      BG_ITER(2, 2, 2, la1, 0, ls1, NB);                                                            \
      BG_ITER(0, 3, 0, la2, 1, ls0, NB);                                                            \
      BG_ITER(1, 4, 1, la0, 1, ls0, NB);                                                            \
      BG_ITER(2, 5, 2, la1, 1, ls0, NB);                                                            \
    }                                                                                               \
    if (q0 < nks) BG_ITER(0, 0, 0, la2, 0, ls1, NB);                                                \
    if (q0 + 1 < nks) BG_ITER(1, 1, 1, la0, 0, ls1, NB);                                            \
    if (q0 + 2 < nks) BG_ITER(2, 2, 2, la1, 0, ls1, NB);                                            \
    if (q0 + 3 < nks) BG_ITER(0, 3, 0, la2, 1, ls0, NB);                                            \
    if (q0 + 4 < nks) BG_ITER(1, 4, 1, la0, 1, ls0, NB);                                            \
  } while (0)

  BG_SDMA(ls0, 0);
  BG_DMA(la0, 0);
  BG_DMA(la1, (nks > 1 ? 1 : 0));
  {
    // row blocks 16 (wm + 4 i) of this wave that hold valid rows (at least one is run)
    const int nbr = (nv - 16 * wm + 63) / 64;
    const int nbv = nbr < 1 ? 1 : (nbr > 4 ? 4 : nbr);
    if (nbv == 4) BG_KLOOP(4);
    else if (nbv == 3) BG_KLOOP(3);
    else if (nbv == 2) BG_KLOOP(2);
    else BG_KLOOP(1);
  }
#undef BG_KLOOP
#undef BG_ITER
#undef BG_STEP
#undef BG_PIN_ACC
#undef BG_DMA
#undef BG_SDMA
  BG_VMWAIT(0);     // no LDS-DMA load may still be landing in the stage buffers
  __syncthreads();  // all operand reads done: the stage buffers now hold the epilogue tiles

  // ---- epilogue: accumulator element k of (i, s) is tile row
  // 16 (wm + 4 i) + 4 g + k, weight row nB(s) + c16
  if (MODE == GM_GATEUP) {
    // two MX blocks of h per row: h columns 64 wn + 32 hb .. + 31 of the
    // tile's 128 (gate sub-tiles 2hb, 2hb+1 with up sub-tiles 4+2hb, 5+2hb);
    // staged per wave in LDS so that lane l quantises wave row l (with two
    // terms, the pair row's value is the sum of its two tile rows, and lanes
    // 0-31 quantise the wave's 32 pair rows, into two term rows each)
    constexpr int WR = 64 / TERMS;  // pair rows per wave
    float* sh = reinterpret_cast<float*>(smem) + wv * (BG_BM / 4) * BG_HSTR;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
#pragma unroll
          for (int k = 0; k < 4 / TERMS; ++k) {
            float gv, uv;
            if constexpr (TERMS == 1) {
              gv = acc[i][2 * hb + ss][k];
              uv = acc[i][4 + 2 * hb + ss][k];
            } else {
              gv = acc[i][2 * hb + ss][2 * k] + acc[i][2 * hb + ss][2 * k + 1];
              uv = acc[i][4 + 2 * hb + ss][2 * k] + acc[i][4 + 2 * hb + ss][2 * k + 1];
            }
            sh[(WR / 4 * i + 4 / TERMS * g + k) * BG_HSTR + 16 * ss + c16] = gv / (1.0f + expf(-gv)) * uv;
          }
      __syncthreads();
      // wave pair row l -> tile pair row (16 / TERMS) (wm + 4 (l / (16 / TERMS))) + l % (16 / TERMS)
      constexpr int RB = 16 / TERMS;
      const int tr = RB * (wm + 4 * (lane / RB)) + (lane % RB);
      if (lane < WR && tr < nvp) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sh[lane * BG_HSTR + i];
        const int m = m0 + tr;
        const int i0 = ntile * 128 + 64 * wn + 32 * hb;
        if constexpr (TERMS == 1) {
          const uint32_t sb = quant_block32(v, ga.hq + (int64_t)m * ga.I + i0);
          ga.hs[(int64_t)m * (ga.I / 32) + i0 / 32] = (uint8_t)sb;
        } else {
          uint32_t s0, s1;
          quant_block32_2t(v, ga.hq + (int64_t)(2 * m) * ga.I + i0, ga.hq + (int64_t)(2 * m + 1) * ga.I + i0, &s0,
                           &s1);
          ga.hs[(int64_t)(2 * m) * (ga.I / 32) + i0 / 32] = (uint8_t)s0;
          ga.hs[(int64_t)(2 * m + 1) * (ga.I / 32) + i0 / 32] = (uint8_t)s1;
        }
      }
      __syncthreads();
    }
  } else {
    __bf16* yb = ga.y + ntile * 256 + c16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4 / TERMS; ++k) {
        const int tr = (16 / TERMS) * (wm + 4 * i) + (4 / TERMS) * g + k;  // tile pair row
        if (tr < nvp) {
          __bf16* yr = yb + (int64_t)(m0 + tr) * ga.H;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float yv = (TERMS == 1) ? acc[i][s][k] : acc[i][s][2 * k] + acc[i][s][2 * k + 1];
            yr[nB(s)] = (__bf16)(poisoned ? __builtin_nanf("") : yv);
          }
        }
      }
  }
}

hipError_t launch_mfma_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                               const void* pool, const float* gates, float* out, char* ws, hipStream_t st) {
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k, T = pl.T;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + pl.off_xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + pl.off_xs);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + pl.off_h);
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + pl.off_hs);
  __bf16* y = reinterpret_cast<__bf16*>(ws + pl.off_y);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.off_tiles);
  int32_t* n_tiles = tiles + 2 * pl.max_tiles;
  int32_t* work_a = n_tiles + 1;                            // gate/up work items
  int32_t* work_b = work_a + (size_t)pl.max_tiles * (I / 128);  // down work items
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + pl.off_offsets);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + pl.off_perm);
  const int32_t* pos = reinterpret_cast<const int32_t*>(ws + pl.off_pos);

  const int64_t nblk = (int64_t)T * H / 32;
  const bool two = pl.terms == 2;
  if (two)
    quant_x_kernel<2><<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x), xq, xs,
                                                                      nblk, H / 32);
  else
    quant_x_kernel<1><<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x), xq, xs,
                                                                      nblk, H / 32);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if ((err = launch_build_tiles(offsets, E, tiles, n_tiles, work_a, I / 128, work_b, H / 256, BG_BM / pl.terms,
                                st)) != hipSuccess)
    return err;

  GemmArgs ga{};
  ga.perm = perm;
  ga.offsets = offsets;
  ga.tiles = tiles;
  ga.n_tiles = n_tiles;
  ga.slot_ids = slot_ids;
  ga.pool = reinterpret_cast<const uint8_t*>(pool);
  ga.stride = d.expert_stride;
  ga.H = H;
  ga.I = I;
  ga.k = k;
  // gate/up: A = x_q gathered by token, N = I in 128-column tiles (gate + up rows)
  ga.aq = xq;
  ga.as = xs;
  ga.a_bytes = (int64_t)pl.terms * T * H;
  ga.hq = hq;
  ga.hs = hs;
  ga.n_ntiles = I / 128;
  ga.work = work_a;
  // the grid covers the most items possible; surplus workgroups exit at once
  const unsigned grid_a = (unsigned)((pl.max_tiles * ga.n_ntiles + 7) / 8 * 8);
  if (two) mx_gemm256_kernel<GM_GATEUP, 2><<<grid_a, 512, 0, st>>>(ga);
  else mx_gemm256_kernel<GM_GATEUP, 1><<<grid_a, 512, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // down: A = h_q by sorted position, N = H in 256-row tiles
  ga.aq = hq;
  ga.as = hs;
  ga.a_bytes = (int64_t)pl.terms * pl.P * I;
  ga.y = y;
  ga.n_ntiles = H / 256;
  ga.work = work_b;
  const unsigned grid_b = (unsigned)((pl.max_tiles * ga.n_ntiles + 7) / 8 * 8);
  if (two) mx_gemm256_kernel<GM_DOWN, 2><<<grid_b, 512, 0, st>>>(ga);
  else mx_gemm256_kernel<GM_DOWN, 1><<<grid_b, 512, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(pl, pos, gates, out, ws, st);
}

bool mfma_supported(const ft_moe_desc& d, int T) {
  return d.w_dtype == FT_MXFP4 && d.act_dtype == FT_BF16 && T >= MFMA_MIN_TOKENS && d.hidden % 256 == 0 &&
         d.inter % 128 == 0 && (int64_t)2 * T * d.hidden < (1ll << 31) &&
         (int64_t)2 * T * d.top_k * d.inter < (1ll << 31) &&
         record_layout(d.hidden, d.inter, FT_MXFP4).bytes < (1ll << 31);
}

}  // namespace ft
