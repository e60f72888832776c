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
// Tiles: a workgroup (4 waves, 2 x 2) computes 64 pair-rows x 128 weight
// rows; K advances 128 per step through double-buffered LDS (global loads
// for step s+1 are in flight while step s computes).  The tile list (expert,
// 64-row block) comes from the permutation; workgroups are mapped so that all
// tiles of one expert land on one XCD (its L2 keeps the A rows and the weight
// tiles), with the eight XCDs taking workgroups round-robin.
//   gate/up: weight rows = 64 gate rows + the same 64 up rows; epilogue
//            h = silu(gate) * up, quantised to MXFP8 through LDS.
//   down:    weight rows = 128 rows of D; epilogue stores y (fp32) through LDS.
// The combine (fixed j order, fp32) runs as its own kernel afterwards.
#include "common.hpp"
#include "internal.hpp"

namespace ft {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GM_BM = 64;      // pair rows per tile
constexpr int GM_BN = 128;     // weight rows per tile
constexpr int GM_BK = 128;     // K per step
constexpr int GM_ASTR = 144;   // LDS row stride of A (bytes), padded
constexpr int GM_BSTR = 80;    // LDS row stride of B (bytes), padded

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
// tiles are grouped by expert; count in *n_tiles.  One workgroup.
__global__ void __launch_bounds__(1024) build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int32_t start[1025];
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      start[e] = run;
      const int cnt = offsets[e + 1] - offsets[e];
      run += (cnt + GM_BM - 1) / GM_BM;
    }
    start[E] = run;
    *n_tiles = run;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int cnt = offsets[e + 1] - offsets[e];
    for (int i = 0; i * GM_BM < cnt; ++i) {
      tiles[2 * (start[e] + i)] = e;
      tiles[2 * (start[e] + i) + 1] = offsets[e] + i * GM_BM;
    }
  }
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
  const int32_t* slot_ids; // per pair (nullable)
  const uint8_t* pool;
  int64_t stride;
  uint8_t* hq;             // gate/up out: h codes [P, I]
  uint8_t* hs;             // gate/up out: h scales [P, I/32]
  float* y;                // down out: [P, H]
  int H, I, k, n_ntiles, total_wg;
};

template <int MODE>
__global__ void __launch_bounds__(256) grouped_mx_gemm_kernel(GemmArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (GM_BM * GM_ASTR + GM_BN * GM_BSTR) + 2 * (GM_BM + GM_BN) * 4];
  // map workgroups XCD-major: consecutive work items run on one XCD
  const int G = ga.total_wg;
  const int per_xcd = (G + 7) / 8;
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int nt = *ga.n_tiles;
  if (w >= nt * ga.n_ntiles) return;
  const int tile = w / ga.n_ntiles, ntile = w % ga.n_ntiles;
  const int e = ga.tiles[2 * tile], m0 = ga.tiles[2 * tile + 1];
  const int m_end = ga.offsets[e + 1];
  const int K = (MODE == GM_GATEUP) ? ga.H : ga.I;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wm = wv >> 1, wn = wv & 1;

  const int slot = ga.slot_ids ? ga.slot_ids[ga.perm[m0]] : e;
  const uint8_t* rec = ga.pool + (int64_t)slot * ga.stride;
  const RecordLayout L = record_layout(ga.H, ga.I, FT_MXFP4);

  // ---- per-thread global sources for the loads of one K step (kept in scalar
  // registers: no local arrays, no captures, nothing goes to scratch)
  // A: 2 x 16 B per thread: tile rows tid/8 and tid/8 + 32, 16-byte chunk tid%8
  int ma0 = m0 + tid / 8, ma1 = m0 + tid / 8 + 32;
  if (ma0 >= m_end) ma0 = m_end - 1;  // padding rows repeat the last row (results discarded)
  if (ma1 >= m_end) ma1 = m_end - 1;
  const int64_t ar0 = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[ma0] / ga.k) : (int64_t)ma0;
  const int64_t ar1 = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[ma1] / ga.k) : (int64_t)ma1;
  const uint8_t* pa0 = ga.aq + ar0 * K + (tid % 8) * 16;
  const uint8_t* pa1 = ga.aq + ar1 * K + (tid % 8) * 16;
  // B: 2 x 16 B per thread: tile rows tid/4 and tid/4 + 64, chunk tid%4
  // (gate/up: tile rows 0-63 are gate rows, 64-127 the same up rows)
  const int br0 = tid / 4, br1 = tid / 4 + 64;
  const int mat0 = (MODE == GM_GATEUP) ? 0 : 2, mat1 = (MODE == GM_GATEUP) ? 1 : 2;
  const int row0 = (MODE == GM_GATEUP) ? ntile * 64 + br0 : ntile * 128 + br0;
  const int row1 = (MODE == GM_GATEUP) ? ntile * 64 + (br1 - 64) : ntile * 128 + br1;
  const uint8_t* pb0 = rec + L.code_off[mat0] + (int64_t)row0 * (K / 2) + (tid % 4) * 16;
  const uint8_t* pb1 = rec + L.code_off[mat1] + (int64_t)row1 * (K / 2) + (tid % 4) * 16;
  // scales: thread t < 64 -> A row t; 64 <= t < 192 -> B tile row t - 64
  const uint8_t* psc = ga.as;
  if (tid < 64) {
    int m = m0 + tid;
    if (m >= m_end) m = m_end - 1;
    const int64_t ar = (MODE == GM_GATEUP) ? (int64_t)(ga.perm[m] / ga.k) : (int64_t)m;
    psc = ga.as + ar * (K / 32);
  } else if (tid < 192) {
    const int br = tid - 64;
    const int mat = (MODE == GM_GATEUP) ? (br < 64 ? 0 : 1) : 2;
    const int row = (MODE == GM_GATEUP) ? ntile * 64 + (br & 63) : ntile * 128 + br;
    psc = rec + L.scale_off[mat] + (int64_t)row * (K / 32);
  }

  // stage b: A at b*STAGE, B at b*STAGE + A bytes; scales after both stages
  constexpr int STAGE = GM_BM * GM_ASTR + GM_BN * GM_BSTR;
  uint8_t* const s_a0 = smem + (tid / 8) * GM_ASTR + (tid % 8) * 16;
  uint8_t* const s_b0 = smem + GM_BM * GM_ASTR + (tid / 4) * GM_BSTR + (tid % 4) * 16;
  uint32_t* const s_sc = reinterpret_cast<uint32_t*>(smem + 2 * STAGE);

  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nks = K / GM_BK;
  uint4 ra0, ra1, rb0, rb1;
  uint32_t rs = 0;
  // prologue: stage 0
  ra0 = *reinterpret_cast<const uint4*>(pa0);
  ra1 = *reinterpret_cast<const uint4*>(pa1);
  rb0 = *reinterpret_cast<const uint4*>(pb0);
  rb1 = *reinterpret_cast<const uint4*>(pb1);
  if (tid < 192) rs = *reinterpret_cast<const uint32_t*>(psc);
  *reinterpret_cast<uint4*>(s_a0) = ra0;
  *reinterpret_cast<uint4*>(s_a0 + 32 * GM_ASTR) = ra1;
  *reinterpret_cast<uint4*>(s_b0) = rb0;
  *reinterpret_cast<uint4*>(s_b0 + 64 * GM_BSTR) = rb1;
  if (tid < 192) s_sc[tid] = rs;
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {  // next stage's global loads, in flight during this stage's MFMAs
      const int kb = (ks + 1) * GM_BK;
      ra0 = *reinterpret_cast<const uint4*>(pa0 + kb);
      ra1 = *reinterpret_cast<const uint4*>(pa1 + kb);
      rb0 = *reinterpret_cast<const uint4*>(pb0 + kb / 2);
      rb1 = *reinterpret_cast<const uint4*>(pb1 + kb / 2);
      if (tid < 192) rs = *reinterpret_cast<const uint32_t*>(psc + kb / 32);
    }
    const uint8_t* sa = smem + cur * STAGE;
    const uint8_t* sb = smem + cur * STAGE + GM_BM * GM_ASTR;
    const uint32_t* ss = s_sc + cur * (GM_BM + GM_BN);
    i32x8_t af0, af1;
    int asc0, asc1;
    {
      const int row = wm * 32 + c16;
      const uint4 lo = *reinterpret_cast<const uint4*>(sa + row * GM_ASTR + 16 * g);
      const uint4 hi = *reinterpret_cast<const uint4*>(sa + row * GM_ASTR + 64 + 16 * g);
      af0 = (i32x8_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      asc0 = (int)((ss[row] >> (8 * g)) & 0xFFu);
      const int row2 = row + 16;
      const uint4 lo2 = *reinterpret_cast<const uint4*>(sa + row2 * GM_ASTR + 16 * g);
      const uint4 hi2 = *reinterpret_cast<const uint4*>(sa + row2 * GM_ASTR + 64 + 16 * g);
      af1 = (i32x8_t){(int)lo2.x, (int)lo2.y, (int)lo2.z, (int)lo2.w, (int)hi2.x, (int)hi2.y, (int)hi2.z, (int)hi2.w};
      asc1 = (int)((ss[row2] >> (8 * g)) & 0xFFu);
    }
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      int brow;
      if (MODE == GM_GATEUP) brow = (ns < 2) ? (32 * wn + 16 * ns + c16) : (64 + 32 * wn + 16 * (ns - 2) + c16);
      else brow = 64 * wn + 16 * ns + c16;
      const uint4 q = *reinterpret_cast<const uint4*>(sb + brow * GM_BSTR + 16 * g);
      const i32x8_t bf = (i32x8_t){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      const int bsc = (int)((ss[GM_BM + brow] >> (8 * g)) & 0xFFu);
      acc[0][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af0, bf, acc[0][ns], 0, 4, 0, asc0, 0, bsc);
      acc[1][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af1, bf, acc[1][ns], 0, 4, 0, asc1, 0, bsc);
    }
    if (more) {
      const int nb = cur ^ 1;
      *reinterpret_cast<uint4*>(s_a0 + nb * STAGE) = ra0;
      *reinterpret_cast<uint4*>(s_a0 + nb * STAGE + 32 * GM_ASTR) = ra1;
      *reinterpret_cast<uint4*>(s_b0 + nb * STAGE) = rb0;
      *reinterpret_cast<uint4*>(s_b0 + nb * STAGE + 64 * GM_BSTR) = rb1;
      if (tid < 192) s_sc[nb * (GM_BM + GM_BN) + tid] = rs;
    }
    __syncthreads();
  }

  // ---- epilogue through LDS (reuses the operand buffers)
  float* sh = reinterpret_cast<float*>(smem);
  if (MODE == GM_GATEUP) {
    // h tile: 64 rows x 64 columns (i0 = ntile*64), row stride 68 floats
    constexpr int HS = 68;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int nsub = 0; nsub < 2; ++nsub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[ms][nsub][i], uv = acc[ms][nsub + 2][i];
          const int r = wm * 32 + ms * 16 + 4 * g + i;
          const int c = 32 * wn + 16 * nsub + c16;
          sh[r * HS + c] = gv / (1.0f + expf(-gv)) * uv;
        }
    __syncthreads();
    if (tid < 128) {  // one 32-block per thread: row tid/2, block tid%2
      const int r = tid / 2, b = tid % 2;
      const int m = m0 + r;
      if (m < m_end) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = sh[r * HS + 32 * b + i];
        const int i0 = ntile * 64 + 32 * b;
        const uint32_t sb = quant_block32(v, ga.hq + (int64_t)m * ga.I + i0);
        ga.hs[(int64_t)m * (ga.I / 32) + i0 / 32] = (uint8_t)sb;
      }
    }
  } else {
    // y tile: 64 rows x 128 columns, row stride 132 floats
    constexpr int YS = 132;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 32 + ms * 16 + 4 * g + i;
          const int c = 64 * wn + 16 * ns + c16;
          sh[r * YS + c] = acc[ms][ns][i];
        }
    __syncthreads();
    // 64 rows x 32 float4 = 2048 stores, 8 per thread
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = q * 256 + tid;
      const int r = idx / 32, c4 = idx % 32;
      const int m = m0 + r;
      if (m < m_end)
        *reinterpret_cast<float4*>(ga.y + (int64_t)m * ga.H + ntile * 128 + 4 * c4) =
            *reinterpret_cast<const float4*>(sh + r * YS + 4 * c4);
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
  float* y = reinterpret_cast<float*>(ws + pl.off_y);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + pl.off_tiles);
  int32_t* n_tiles = tiles + 2 * pl.max_tiles;
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + pl.off_offsets);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + pl.off_perm);
  const int32_t* pos = reinterpret_cast<const int32_t*>(ws + pl.off_pos);

  const int64_t nblk = (int64_t)T * H / 32;
  quant_x_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x), xq, xs, nblk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  build_tiles_kernel<<<1, 1024, 0, st>>>(offsets, E, tiles, n_tiles);
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
  // gate/up: A = x_q gathered by token, N = I in 64-column tiles (gate + up rows)
  ga.aq = xq;
  ga.as = xs;
  ga.hq = hq;
  ga.hs = hs;
  ga.n_ntiles = I / 64;
  ga.total_wg = (pl.max_tiles * ga.n_ntiles + 7) / 8 * 8;  // a multiple of 8 keeps the XCD mapping a bijection
  grouped_mx_gemm_kernel<GM_GATEUP><<<ga.total_wg, 256, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // down: A = h_q by sorted position, N = H in 128-row tiles
  ga.aq = hq;
  ga.as = hs;
  ga.y = y;
  ga.n_ntiles = H / 128;
  ga.total_wg = (pl.max_tiles * ga.n_ntiles + 7) / 8 * 8;
  grouped_mx_gemm_kernel<GM_DOWN><<<ga.total_wg, 256, 0, st>>>(ga);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_combine(pl, pos, gates, out, ws, st);
}

bool mfma_supported(const ft_moe_desc& d, int T) {
  return d.w_dtype == FT_MXFP4 && d.act_dtype == FT_BF16 && T >= MFMA_MIN_TOKENS && d.hidden % 128 == 0 &&
         d.inter % 128 == 0;
}

}  // namespace ft
