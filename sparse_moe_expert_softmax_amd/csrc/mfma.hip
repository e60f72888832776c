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
// Tiles: a workgroup (4 waves) computes 64 pair rows x 256 weight rows, each
// wave all 64 rows x 64 weight rows; K advances 128 per step.  Activations go
// through double-buffered LDS, weights straight from memory into the MFMA
// operand registers, block scales in groups of three steps through LDS; the
// loads of two steps are in flight while a step computes.  The tile list
// (expert, 64-row block) comes from the permutation; work items are ordered
// expert, weight tile, row tile and mapped so that consecutive items run on
// one XCD (its L2 then serves a weight tile to all row tiles of the expert).
//   gate/up: weight rows = 128 gate rows + the same 128 up rows; epilogue
//            h = silu(gate) * up, quantised to MXFP8 through LDS.
//   down:    weight rows = 256 rows of D; epilogue stores y rounded to bf16.
// The combine (fixed j order, fp32) runs as its own kernel afterwards.
#include "common.hpp"
#include "internal.hpp"

namespace ft {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GM_BM = 64;      // pair rows per tile
constexpr int GM_BN = 256;     // weight rows per tile (gate/up: 128 gate rows + the same 128 up rows)
constexpr int GM_BK = 128;     // K per step
constexpr int GM_ASTR = 144;   // LDS row stride of A (bytes), padded: conflict-free 16-byte fragment reads
constexpr int GM_HSTR = 33;    // LDS row stride of the h epilogue tile (floats)

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

// x [T, H] bf16 -> xq [T, H] E4M3 + xs [T, H/32] E8M0; one thread per 32-block.
__global__ void __launch_bounds__(256) quant_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xs, int64_t nblocks) {
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
  xs[b] = (uint8_t)quant_block32(v, xq + b * 32);
}

// ------------------------------------------------------------ tile list --
// tiles[2*i] = expert, tiles[2*i+1] = first row (sorted position) of tile i;
// tiles are grouped by expert; count in *n_tiles.  Work lists (one per GEMM,
// n_nt weight tiles each): item = tile | (ntile << 20), ordered by expert,
// then weight tile, then row tile, so that the row tiles sharing a weight
// tile run side by side and an expert's activation rows stay in one L2.
// One workgroup per expert.
__global__ void __launch_bounds__(1024) build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                           int32_t* __restrict__ work_a, int n_nt_a,
                                                           int32_t* __restrict__ work_b, int n_nt_b) {
  // Workgroup b writes expert b's entries; every workgroup first forms the
  // exclusive prefix sum of the per-expert tile counts (E <= 1024): wave scans
  // of 64 lanes, then a scan of the wave totals.
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_start, s_mt;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, eb = blockIdx.x;
  const int cnt = (t < E) ? offsets[t + 1] - offsets[t] : 0;
  const int mt_own = (cnt + GM_BM - 1) / GM_BM;
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
    tiles[2 * (st + i) + 1] = o0 + i * GM_BM;
  }
  for (int j = t; j < mt * n_nt_a; j += blockDim.x) work_a[st * n_nt_a + j] = (st + j % mt) | ((j / mt) << 20);
  for (int j = t; j < mt * n_nt_b; j += blockDim.x) work_b[st * n_nt_b + j] = (st + j % mt) | ((j / mt) << 20);
}

// -------------------------------------------------------------- the GEMM --
enum { GM_GATEUP = 0, GM_DOWN = 1 };

// Buffer descriptor word 3 for untyped 32-bit accesses on gfx9-family parts.
constexpr int GM_RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ uint3 gm_ld96(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef int i32x3_t __attribute__((ext_vector_type(3)));
  const i32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
  return make_uint3((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z);
}

__device__ __forceinline__ uint4 gm_ld128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

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
  int H, I, k, n_ntiles, total_wg;
};

// Workgroup tile: 64 pair rows x 256 weight rows, K advancing 128 per step.
// The four waves split the weight rows: each wave owns all 64 pair rows and
// 64 weight rows (4 x 4 MFMAs per K step, 16 independent accumulators).
//   A (activations, shared by the waves) goes global -> registers -> LDS,
//     double-buffered; each wave reads its fragments from LDS.
//   B (weights, private to one wave) goes global -> registers straight into
//     the MFMA operand: lane l loads the 16 bytes (one MX block of 32 E2M1
//     codes) of weight row l % 16, K block l / 16, and the matching scale byte.
// A ring of three register slots keeps the loads of two K steps in flight;
// every step issues the same loads unconditionally (the step index is
// clamped at the end), so the compiler's wait counts stay exact.
template <int MODE>
__global__ void __launch_bounds__(256, 2) grouped_mx_gemm_kernel(GemmArgs ga) {
  constexpr int A_STAGE = GM_BM * GM_ASTR;
  constexpr int LDS_MAIN = 2 * A_STAGE + 2 * GM_BM * 12 + 2 * GM_BN * 12;
  constexpr int LDS_EPI = 4 * GM_BM * GM_HSTR * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI];
  // map workgroups XCD-major: consecutive work items run on one XCD
  const int G = ga.total_wg;
  const int per_xcd = (G + 7) / 8;
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int nt = *ga.n_tiles;
  if (w >= nt * ga.n_ntiles) return;
  const int item = ga.work[w];
  const int tile = item & 0xFFFFF, ntile = item >> 20;
  const int e = ga.tiles[2 * tile], m0 = ga.tiles[2 * tile + 1];
  const int m_end = ga.offsets[e + 1];
  const int K = (MODE == GM_GATEUP) ? ga.H : ga.I;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, c16 = lane & 15;

  const int slot = ga.slot_ids ? ga.slot_ids[ga.perm[m0]] : e;
  const uint8_t* rec = ga.pool + (int64_t)slot * ga.stride;
  const RecordLayout L = record_layout(ga.H, ga.I, FT_MXFP4);

  // ---- A sources: 2 x 16 B per thread (tile rows tid/8 and tid/8 + 32,
  // 16-byte chunk tid%8) and one scale word per thread (row tid%64; only
  // threads < 64 store theirs)
  int ma0 = m0 + tid / 8, ma1 = m0 + tid / 8 + 32, mas = m0 + 16 * wv + c16;
  if (ma0 >= m_end) ma0 = m_end - 1;  // padding rows repeat the last row (results discarded)
  if (ma1 >= m_end) ma1 = m_end - 1;
  if (mas >= m_end) mas = m_end - 1;
  const int64_t ar0 = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[ma0] / ga.k) : (int64_t)ma0;
  const int64_t ar1 = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[ma1] / ga.k) : (int64_t)ma1;
  const int64_t ars = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[mas] / ga.k) : (int64_t)mas;
  // Loads go through buffer descriptors: a per-lane 32-bit offset that stays
  // fixed over the K loop plus a scalar K offset, so the loop keeps no 64-bit
  // addresses in vector registers.
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ga.aq, (short)0, (int)ga.a_bytes, GM_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rAs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ga.as, (short)0, (int)(ga.a_bytes / 32), GM_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)rec, (short)0, (int)L.bytes, GM_RSRC_WORD3);
  const int oa0 = (int)(ar0 * K) + (tid % 8) * 16;
  const int oa1 = (int)(ar1 * K) + (tid % 8) * 16;
  // scales travel in groups of three K steps (12 blocks, 12 bytes per row):
  // lane l of wave w loads dword min(l/16, 2) of A row 16w + l%16, and the 12
  // bytes of its wave's weight row 16*(l/16) + l%16 (sub-tile l/16)
  const int oas = (int)(ars * (K / 32)) + 4 * (g < 3 ? g : 2);

  // ---- B sources: weight row of sub-tile ns for this lane, K block g
  // gate/up: ns 0,1 = gate rows, ns 2,3 = the same up rows
  //          (ntile*128 + 32*wave + 16*(ns&1) + lane%16)
  // down:    rows ntile*256 + 64*wave + 16*ns + lane%16
  auto brow = [&](int ns) {
    return (MODE == GM_GATEUP) ? ntile * 128 + 32 * wv + 16 * (ns & 1) + c16 : ntile * 256 + 64 * wv + 16 * ns + c16;
  };
  auto bmat = [&](int ns) { return (MODE == GM_GATEUP) ? (ns < 2 ? 0 : 1) : 2; };
  // one per-lane offset (sub-tile 0) for all four sub-tiles; the others
  // differ by a uniform amount that rides in the scalar offset
  const int ob = (int)L.code_off[bmat(0)] + brow(0) * (K / 2) + 16 * g;
  auto bdelta = [&](int ns) {
    return (int)(L.code_off[bmat(ns)] - L.code_off[bmat(0)]) + (brow(ns) - brow(0)) * (K / 2);
  };
  const int db1 = bdelta(1), db2 = bdelta(2), db3 = bdelta(3);
  int obs;  // this lane's weight-scale row: sub-tile g, row lane%16
  {
    const int ns = g;
    const int row = (MODE == GM_GATEUP) ? ntile * 128 + 32 * wv + 16 * (ns & 1) + c16 : ntile * 256 + 64 * wv + 16 * ns + c16;
    const int mat = (MODE == GM_GATEUP) ? (ns < 2 ? 0 : 1) : 2;
    obs = (int)L.scale_off[mat] + row * (K / 32);
  }

  uint8_t* const s_a = smem + (tid / 8) * GM_ASTR + (tid % 8) * 16;  // this thread's A store address
  // scale groups, double-buffered: A [2][64 rows][3 dwords], weights [2][4 waves][64 rows][3 dwords]
  uint32_t* const s_as = reinterpret_cast<uint32_t*>(smem + 2 * A_STAGE);
  uint32_t* const s_bs = s_as + 2 * GM_BM * 3;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nks = K / GM_BK;
#define GM_DECL(r) uint4 ra0_##r, ra1_##r, rb0_##r, rb1_##r, rb2_##r, rb3_##r;
  GM_DECL(0) GM_DECL(1) GM_DECL(2)
#undef GM_DECL
  uint32_t gsa;  // A-scale dword of the group in flight
  uint3 gsb;     // weight-scale bytes (12) of the group in flight
#define GM_LOAD(r, st)                                                              \
  do {                                                                              \
    const int kb_ = ((st) < nks ? (st) : nks - 1) * GM_BK;                          \
    ra0_##r = gm_ld128(rA, oa0, kb_);                                               \
    ra1_##r = gm_ld128(rA, oa1, kb_);                                               \
    rb0_##r = gm_ld128(rB, ob, kb_ / 2);                                            \
    rb1_##r = gm_ld128(rB, ob, db1 + kb_ / 2);                                      \
    rb2_##r = gm_ld128(rB, ob, db2 + kb_ / 2);                                      \
    rb3_##r = gm_ld128(rB, ob, db3 + kb_ / 2);                                      \
  } while (0)
#define GM_STORE(r, buf)                                                            \
  do {                                                                              \
    *reinterpret_cast<uint4*>(s_a + (buf) * A_STAGE) = ra0_##r;                     \
    *reinterpret_cast<uint4*>(s_a + (buf) * A_STAGE + 32 * GM_ASTR) = ra1_##r;      \
  } while (0)
  // scale group G covers K steps 3G .. 3G+2 (clamped at the end; the bytes of
  // a partial last group past the row are never used)
#define GM_GLOAD(G)                                                                 \
  do {                                                                              \
    const int gg_ = ((G) <= (nks - 1) / 3 ? (G) : (nks - 1) / 3) * 12;              \
    gsa = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rAs, oas, gg_, 0);         \
    gsb = gm_ld96(rB, obs, gg_);                                                    \
  } while (0)
#define GM_GSTORE(buf)                                                              \
  do {                                                                              \
    if (g < 3) s_as[(buf) * GM_BM * 3 + (16 * wv + c16) * 3 + g] = gsa;             \
    uint32_t* d_ = s_bs + (buf) * GM_BN * 3 + (64 * wv + lane) * 3;                 \
    d_[0] = gsb.x; d_[1] = gsb.y; d_[2] = gsb.z;                                    \
  } while (0)
#define GM_BOP(v_) ((i32x8_t){(int)(v_).x, (int)(v_).y, (int)(v_).z, (int)(v_).w, 0, 0, 0, 0})
#define GM_STEP(r, buf, sbuf, j)                                                                  \
  do {                                                                                            \
    const uint8_t* sa_ = smem + (buf) * A_STAGE;                                                  \
    const uint8_t* sas_ = reinterpret_cast<const uint8_t*>(s_as + (sbuf) * GM_BM * 3) + 4 * (j) + g; \
    const uint8_t* sbs_ = reinterpret_cast<const uint8_t*>(s_bs + (sbuf) * GM_BN * 3 + 64 * wv * 3) + 4 * (j) + g; \
    const i32x8_t b0_ = GM_BOP(rb0_##r), b1_ = GM_BOP(rb1_##r);                                   \
    const i32x8_t b2_ = GM_BOP(rb2_##r), b3_ = GM_BOP(rb3_##r);                                   \
    const int bs0_ = sbs_[(c16) * 12], bs1_ = sbs_[(16 + c16) * 12];                              \
    const int bs2_ = sbs_[(32 + c16) * 12], bs3_ = sbs_[(48 + c16) * 12];                         \
    _Pragma("unroll") for (int ms = 0; ms < 4; ++ms) {                                            \
      const int row_ = 16 * ms + c16;                                                             \
      const uint4 lo_ = *reinterpret_cast<const uint4*>(sa_ + row_ * GM_ASTR + 16 * g);           \
      const uint4 hi_ = *reinterpret_cast<const uint4*>(sa_ + row_ * GM_ASTR + 64 + 16 * g);      \
      const i32x8_t a_ = (i32x8_t){(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w,                \
                                   (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w};               \
      const int as_ = sas_[row_ * 12];                                                            \
      acc[ms][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_, b0_, acc[ms][0], 0, 4, 0, as_, 0, bs0_); \
      acc[ms][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_, b1_, acc[ms][1], 0, 4, 0, as_, 0, bs1_); \
      acc[ms][2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_, b2_, acc[ms][2], 0, 4, 0, as_, 0, bs2_); \
      acc[ms][3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_, b3_, acc[ms][3], 0, 4, 0, as_, 0, bs3_); \
    }                                                                                             \
  } while (0)
  // An empty asm that reads and writes every accumulator ends each K step:
  // without it the compiler sinks a step's MFMAs past the barrier into the
  // next steps, keeping several steps' operands live at once (and spilling).
#define GM_PIN_ACC()                                                                \
  do {                                                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                \
    _Pragma("unroll") for (int j_ = 0; j_ < 4; ++j_) asm volatile("" : "+v"(acc[i_][j_])); \
  } while (0)
  // iteration for K step q = q0 + J (ring slot J = q % 3, scale group q0 / 3):
  // A of step q+1 goes to LDS, the loads of step q+2 refill the slot that held
  // step q-1, step q computes.  The next scale group is loaded at J = 0 and
  // stored at J = 2, before the barrier that precedes its first step.
#define GM_ITER(J, JN, JL)                                                          \
  do {                                                                              \
    const int q = q0 + J;                                                           \
    const int cur = q & 1;                                                          \
    GM_STORE(JN, cur ^ 1);                                                          \
    GM_LOAD(JL, q + 2);                                                             \
    if (J == 0) GM_GLOAD(q0 / 3 + 1);                                               \
    GM_STEP(J, cur, gb, J);                                                         \
    if (J == 2) GM_GSTORE(gb ^ 1);                                                  \
    GM_PIN_ACC();                                                                   \
    __syncthreads();                                                                \
  } while (0)

  GM_GLOAD(0);
  GM_LOAD(0, 0);
  GM_LOAD(1, 1);
  GM_GSTORE(0);
  GM_STORE(0, 0);
  __syncthreads();
  int q0 = 0, gb = 0;
  for (; q0 + 3 <= nks; q0 += 3, gb ^= 1) {
    GM_ITER(0, 1, 2);
    GM_ITER(1, 2, 0);
    GM_ITER(2, 0, 1);
  }
  // K-step tail: the ring is back at slot 0 here.
  const int rem = nks - q0;
  if (rem >= 1) GM_ITER(0, 1, 2);
  if (rem >= 2) GM_ITER(1, 2, 0);
#undef GM_ITER
#undef GM_STEP
#undef GM_GLOAD
#undef GM_GSTORE
#undef GM_PIN_ACC
#undef GM_BOP
#undef GM_LOAD
#undef GM_STORE

  // ---- epilogue (accumulator element i of sub-tile (ms, ns) is row
  // 16 ms + 4 g + i, weight row 16 ns + lane%16 of the wave's 64)
  if (MODE == GM_GATEUP) {
    // The wave's 32 h columns (i0 = ntile*128 + 32*wave) are one MX block per
    // row: stage h = silu(gate) * up in the wave's own LDS area, then lane r
    // quantises row r.  (The loop's last barrier freed the A buffers.)
    float* sh = reinterpret_cast<float*>(smem) + wv * GM_BM * GM_HSTR;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int nsub = 0; nsub < 2; ++nsub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[ms][nsub][i], uv = acc[ms][nsub + 2][i];
          sh[(16 * ms + 4 * g + i) * GM_HSTR + 16 * nsub + c16] = gv / (1.0f + expf(-gv)) * uv;
        }
    __syncthreads();
    const int m = m0 + lane;
    if (m < m_end) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = sh[lane * GM_HSTR + i];
      const int i0 = ntile * 128 + 32 * wv;
      const uint32_t sb = quant_block32(v, ga.hq + (int64_t)m * ga.I + i0);
      ga.hs[(int64_t)m * (ga.I / 32) + i0 / 32] = (uint8_t)sb;
    }
  } else {
    // y rows straight from the accumulators, rounded to bf16 (nearest even):
    // 16 lanes store 32 contiguous bytes
    __bf16* yb = ga.y + ntile * 256 + 64 * wv + c16;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * ms + 4 * g + i;
        if (m < m_end) {
          __bf16* yr = yb + (int64_t)m * ga.H;
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) yr[16 * ns] = (__bf16)acc[ms][ns][i];
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
  quant_x_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x), xq, xs, nblk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  build_tiles_kernel<<<E, 1024, 0, st>>>(offsets, E, tiles, n_tiles, work_a, I / 128, work_b, H / 256);
  if ((err = hipGetLastError()) != hipSuccess) return err;

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
  ga.a_bytes = (int64_t)T * H;
  ga.hq = hq;
  ga.hs = hs;
  ga.n_ntiles = I / 128;
  ga.work = work_a;
  ga.total_wg = (pl.max_tiles * ga.n_ntiles + 7) / 8 * 8;  // a multiple of 8 keeps the XCD mapping a bijection
  grouped_mx_gemm_kernel<GM_GATEUP><<<ga.total_wg, 256, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // down: A = h_q by sorted position, N = H in 256-row tiles
  ga.aq = hq;
  ga.as = hs;
  ga.a_bytes = (int64_t)pl.P * I;
  ga.y = y;
  ga.n_ntiles = H / 256;
  ga.work = work_b;
  ga.total_wg = (pl.max_tiles * ga.n_ntiles + 7) / 8 * 8;
  grouped_mx_gemm_kernel<GM_DOWN><<<ga.total_wg, 256, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(pl, pos, gates, out, ws, st);
}

bool mfma_supported(const ft_moe_desc& d, int T) {
  return d.w_dtype == FT_MXFP4 && d.act_dtype == FT_BF16 && T >= MFMA_MIN_TOKENS && d.hidden % 256 == 0 &&
         d.inter % 128 == 0 && (int64_t)T * d.hidden < (1ll << 31) &&
         (int64_t)T * d.top_k * d.inter < (1ll << 31) &&
         record_layout(d.hidden, d.inter, FT_MXFP4).bytes < (1ll << 31);
}

}  // namespace ft
