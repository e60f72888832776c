// Router: fp64 logits from exact products, then wave64 top-k with
// lowest-index tie-break and renormalised softmax gates.
//
// The pages require that routing is neither changed nor approximated (FreeToken
// explainer page, "how" and "who" sections).  Selection is an integer
// decision taken on floating-point logits, so the logits are accumulated in
// fp64 from exact products (bf16*bf16 and fp32*fp32 products are exact in
// fp64): the result is within ~1e-13 of the exactly rounded dot product, far
// below any gap between distinct logits of real inputs.  Every expert row is
// reduced in the same fixed order, so bitwise-equal rows give bitwise-equal
// logits and the tie goes to the lower expert id.
#include "common.hpp"
#include "internal.hpp"
#include "topk.hpp"

namespace ft {

// Load 8 consecutive elements (fp32 or bf16) at element index i as doubles.
template <int DT>
__device__ __forceinline__ void load8_f64(const void* base, int64_t i, double (&v)[8]) {
  if constexpr (DT == FT_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (double)bf16_lo(w[j]);
      v[2 * j + 1] = (double)bf16_hi(w[j]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ---------------------------------------------------------------- decode --
// Few tokens: workgroup e computes the logits of expert e for all T <= 16
// tokens (its 4 waves split H; fp64 partial sums reduced across the wave with
// a multi-value butterfly, then across waves in LDS, in a fixed order that is
// the same for every expert).  A second launch of one workgroup (one wave per
// token) runs the top-k.  Two launches rather than a last-workgroup handoff:
// a device-scope release per workgroup costs an L2 write-back on this chip.
constexpr int RD_MAXT = 16;

// Reduce v[N] (N a power of two <= 16) over the 64 lanes; afterwards lane l
// holds the total of index (l >> (6 - log2 N)).
template <int N>
__device__ __forceinline__ double multi_reduce(double (&v)[N]) {
  const int lane = threadIdx.x & 63;
  int n = N;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    if (n > 1) {
      const bool upper = (lane & o) != 0;
      const int h = n / 2;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        if (i < h) {
          const double send = upper ? v[i] : v[i + h];
          const double keep = upper ? v[i + h] : v[i];
          v[i] = keep + __shfl_xor(send, o, 64);
        }
      }
      n = h;
    } else {
      v[0] += __shfl_xor(v[0], o, 64);
    }
  }
  return v[0];
}

template <int XDT, int WDT, int NT>
__global__ void __launch_bounds__(256) route_decode_kernel(const void* __restrict__ x, const void* __restrict__ wr,
                                                           double* __restrict__ logits, int T, int H, int E) {
  __shared__ double part[4][RD_MAXT];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x;
  double acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0;
  const int hq = H / 4;  // this wave's quarter of H (H % 32 == 0)
  if (XDT == FT_BF16 && WDT == FT_BF16 && NT <= 4 && hq <= 4 * 512) {
    // bf16, few tokens, H <= 8192: the loads of every pass are issued before
    // any is used (passes past the quarter read its first element and are
    // skipped); same products in the same order as the loop below
    const int h0 = wv * hq + lane * 8, hend = (wv + 1) * hq;
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(wr) + (int64_t)e * H;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    uint4 wq[4], xq[4][NT];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int h = h0 + 512 * it, hc = h < hend ? h : wv * hq;
      wq[it] = *reinterpret_cast<const uint4*>(wb + hc);
#pragma unroll
      for (int t = 0; t < NT; ++t) xq[it][t] = *reinterpret_cast<const uint4*>(xb + (int64_t)(t < T ? t : 0) * H + hc);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (h0 + 512 * it >= hend) continue;
      const uint32_t ww[4] = {wq[it].x, wq[it].y, wq[it].z, wq[it].w};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= T) continue;
        const uint32_t xx[4] = {xq[it][t].x, xq[it][t].y, xq[it][t].z, xq[it][t].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[t] = fma((double)bf16_lo(xx[j]), (double)bf16_lo(ww[j]), acc[t]);
          acc[t] = fma((double)bf16_hi(xx[j]), (double)bf16_hi(ww[j]), acc[t]);
        }
      }
    }
  } else {
    for (int h = wv * hq + lane * 8; h < (wv + 1) * hq; h += 64 * 8) {
      double w[8];
      load8_f64<WDT>(wr, (int64_t)e * H + h, w);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < T) {
          double xv[8];
          load8_f64<XDT>(x, (int64_t)t * H + h, xv);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[t] = fma(xv[j], w[j], acc[t]);
        }
      }
    }
  }
  // one token: a fixed-order wave sum by DPP row operations (a few cycles
  // per step) instead of six dependent LDS permutes
  double r;
  if constexpr (NT == 1) r = tk_wave_sum_f64(acc[0]);
  else r = multi_reduce<NT>(acc);
  constexpr int SH = (NT == 1) ? 6 : (NT == 2) ? 5 : (NT == 4) ? 4 : (NT == 8) ? 3 : 2;
  if ((lane & ((1 << SH) - 1)) == 0) part[wv][lane >> SH] = r;
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    logits[(int64_t)t * E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
  }
}

// One wave per token, PER = ceil(E / 64) logits per lane.
template <int PER>
__global__ void __launch_bounds__(1024) route_topk_decode_kernel(const double* __restrict__ logits,
                                                                 const float* __restrict__ sel_bias,
                                                                 int32_t* __restrict__ ids, float* __restrict__ gates,
                                                                 int T, int E, int k, int renormalize) {
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * (blockDim.x >> 6) + w;
  if (t >= T) return;
  topk_one_token<PER>(logits + (int64_t)t * E, sel_bias ? sel_bias + (int64_t)t * E : nullptr, E, k, renormalize,
                      ids + (int64_t)t * k, gates + (int64_t)t * k);
}

template <int XDT, int WDT>
static void launch_route_logits_decode_t(const ft_moe_desc& d, const void* x, int T, const void* wr, double* logits,
                                         hipStream_t st) {
  const int H = d.hidden, E = d.n_experts;
  if (T <= 1) route_decode_kernel<XDT, WDT, 1><<<E, 256, 0, st>>>(x, wr, logits, T, H, E);
  else if (T <= 2) route_decode_kernel<XDT, WDT, 2><<<E, 256, 0, st>>>(x, wr, logits, T, H, E);
  else if (T <= 4) route_decode_kernel<XDT, WDT, 4><<<E, 256, 0, st>>>(x, wr, logits, T, H, E);
  else if (T <= 8) route_decode_kernel<XDT, WDT, 8><<<E, 256, 0, st>>>(x, wr, logits, T, H, E);
  else route_decode_kernel<XDT, WDT, 16><<<E, 256, 0, st>>>(x, wr, logits, T, H, E);
}

template <int XDT, int WDT>
static void launch_route_decode_t(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                                  int32_t* ids, float* gates, double* logits, hipStream_t st) {
  const int E = d.n_experts, k = d.top_k, rn = d.renormalize;
  launch_route_logits_decode_t<XDT, WDT>(d, x, T, wr, logits, st);
  const int threads = 64 * T;
  if (E <= 64) route_topk_decode_kernel<1><<<1, threads, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 128) route_topk_decode_kernel<2><<<1, threads, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 256) route_topk_decode_kernel<4><<<1, threads, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 512) route_topk_decode_kernel<8><<<1, threads, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else route_topk_decode_kernel<16><<<1, threads, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
}

hipError_t launch_route_logits_decode(const ft_moe_desc& d, const void* x, int T, const void* wr, double* logits,
                                      hipStream_t st) {
  const int xd = d.act_dtype, wd = d.router_dtype;
  if (xd == FT_BF16 && wd == FT_BF16) launch_route_logits_decode_t<FT_BF16, FT_BF16>(d, x, T, wr, logits, st);
  else if (xd == FT_F32 && wd == FT_F32) launch_route_logits_decode_t<FT_F32, FT_F32>(d, x, T, wr, logits, st);
  else if (xd == FT_BF16 && wd == FT_F32) launch_route_logits_decode_t<FT_BF16, FT_F32>(d, x, T, wr, logits, st);
  else launch_route_logits_decode_t<FT_F32, FT_BF16>(d, x, T, wr, logits, st);
  return hipGetLastError();
}

hipError_t launch_route_decode(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                               int32_t* ids, float* gates, double* logits, hipStream_t st) {
  const int xd = d.act_dtype, wd = d.router_dtype;
  if (xd == FT_BF16 && wd == FT_BF16) launch_route_decode_t<FT_BF16, FT_BF16>(d, x, T, wr, sel_bias, ids, gates, logits, st);
  else if (xd == FT_F32 && wd == FT_F32) launch_route_decode_t<FT_F32, FT_F32>(d, x, T, wr, sel_bias, ids, gates, logits, st);
  else if (xd == FT_BF16 && wd == FT_F32) launch_route_decode_t<FT_BF16, FT_F32>(d, x, T, wr, sel_bias, ids, gates, logits, st);
  else launch_route_decode_t<FT_F32, FT_BF16>(d, x, T, wr, sel_bias, ids, gates, logits, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- prefill --
// Many tokens, hidden size not a multiple of 32 (the matrix-core kernel
// below needs 32-element chunks): logits as a tiled fp64 GEMM on the vector
// ALUs.  A workgroup computes 128 tokens x 64 experts; each thread holds
// 8 x 4 fp64 accumulators; K advances 16 per step through double-buffered
// LDS holding the operands already widened to fp64 (exact).  Each
// accumulator adds its products in ascending h order, the same order for
// every expert.
constexpr int RL_TT = 128, RL_TE = 64, RL_KB = 16;

template <int XDT, int WDT>
__global__ void __launch_bounds__(256) route_logits_tiled_kernel(const void* __restrict__ x, const void* __restrict__ wr,
                                                                 double* __restrict__ logits, int T, int H, int E) {
  __shared__ double xs[2][RL_KB][RL_TT];
  __shared__ double wsm[2][RL_KB][RL_TE];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RL_TT, e0 = blockIdx.y * RL_TE;
  const int ty = tid / 16, tx = tid % 16;  // thread owns tokens ty*8.. and experts tx*4..
  double acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  // loaders: x: token tid/2, 8 consecutive k at (tid%2)*8; w: threads < 128: expert tid/2, same k split
  const int xt = t0 + tid / 2, xk = (tid % 2) * 8;
  const int we = e0 + tid / 2;
  double lx[8], lw[8];
  auto gload = [&](int kb) {
    if (xt < T) load8_f64<XDT>(x, (int64_t)xt * H + kb + xk, lx);
    else for (int j = 0; j < 8; ++j) lx[j] = 0.0;
    if (tid < 128) {
      if (we < E) load8_f64<WDT>(wr, (int64_t)we * H + kb + xk, lw);
      else for (int j = 0; j < 8; ++j) lw[j] = 0.0;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[buf][xk + j][tid / 2] = lx[j];
    if (tid < 128)
#pragma unroll
      for (int j = 0; j < 8; ++j) wsm[buf][xk + j][tid / 2] = lw[j];
  };
  const int nk = H / RL_KB;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    if (s + 1 < nk) gload((s + 1) * RL_KB);
#pragma unroll 2
    for (int kk = 0; kk < RL_KB; ++kk) {
      double a[8], b[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = xs[cur][kk][ty * 8 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = wsm[cur][kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    if (s + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + ty * 8 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

// Many tokens on the fp64 matrix cores: v_mfma_f64_16x16x4_f64 multiplies
// 16 tokens x 4 h by 4 h x 16 experts into a 16 x 16 fp64 tile (lane l holds
// A[l%16][l/16] and B[l/16][l%16]; D[l/16 + 4i][l%16] in its 4 results, as
// measured on the device).
// Products of widened bf16 / fp32 operands are exact in fp64; only the sums
// round.  A workgroup (2 x 2 waves) computes 64 tokens x 64 experts, each
// wave 32 x 32 (2 x 2 tiles).  Along h, 32-element chunks are consumed in 8
// MFMA steps with lane group g taking h = 8g + s at step s, so every lane
// loads 8 consecutive elements of its token row and of its expert row per
// chunk (16 B of bf16); the next chunk's raw loads are in flight while the
// current one computes.  Every expert column goes through the same sequence
// of operations, so bitwise-equal expert rows give bitwise-equal logits.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int RM_T = 64, RM_E = 64;

template <int DT> struct Raw8;
template <> struct Raw8<FT_BF16> { uint4 q; };
template <> struct Raw8<FT_F32> { uint4 q[2]; };

template <int DT>
__device__ __forceinline__ void raw8_load(const void* base, int64_t i, Raw8<DT>& r) {
  if constexpr (DT == FT_BF16) {
    r.q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + i);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + i);
    r.q[0] = p[0];
    r.q[1] = p[1];
  }
}

template <int DT>
__device__ __forceinline__ double raw8_get(const Raw8<DT>& r, int j) {
  if constexpr (DT == FT_BF16) {
    const uint32_t w = (j < 2) ? r.q.x : (j < 4) ? r.q.y : (j < 6) ? r.q.z : r.q.w;
    return (double)((j & 1) ? bf16_hi(w) : bf16_lo(w));
  } else {
    const uint4 q = r.q[j >> 2];
    const uint32_t w = ((j & 3) == 0) ? q.x : ((j & 3) == 1) ? q.y : ((j & 3) == 2) ? q.z : q.w;
    return (double)__uint_as_float(w);
  }
}

template <int XDT, int WDT>
__global__ void __launch_bounds__(256) route_logits_mfma_kernel(const void* __restrict__ x, const void* __restrict__ wr,
                                                                double* __restrict__ logits, int T, int H, int E) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int tw = blockIdx.x * RM_T + (wv >> 1) * 32, ew = blockIdx.y * RM_E + (wv & 1) * 32;
  int64_t xrow[2], wrow[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    int t = tw + 16 * m + c;
    if (t >= T) t = T - 1;  // rows past the end repeat the last row (never stored)
    int e = ew + 16 * m + c;
    if (e >= E) e = E - 1;
    xrow[m] = (int64_t)t * H + 8 * g;
    wrow[m] = (int64_t)e * H + 8 * g;
  }
  f64x4_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = (f64x4_t){0.0, 0.0, 0.0, 0.0};
  Raw8<XDT> ax[2];
  Raw8<WDT> bw[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    raw8_load<XDT>(x, xrow[m], ax[m]);
    raw8_load<WDT>(wr, wrow[m], bw[m]);
  }
  const int nch = H / 32;
  for (int ch = 0; ch < nch; ++ch) {
    Raw8<XDT> cx[2] = {ax[0], ax[1]};
    Raw8<WDT> cw[2] = {bw[0], bw[1]};
    if (ch + 1 < nch) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        raw8_load<XDT>(x, xrow[m] + 32 * (ch + 1), ax[m]);
        raw8_load<WDT>(wr, wrow[m] + 32 * (ch + 1), bw[m]);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const double a0 = raw8_get<XDT>(cx[0], s), a1 = raw8_get<XDT>(cx[1], s);
      const double b0 = raw8_get<WDT>(cw[0], s), b1 = raw8_get<WDT>(cw[1], s);
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int e = ew + 16 * n + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tw + 16 * m + g + 4 * i;
        if (t < T && e < E) logits[(int64_t)t * E + e] = acc[m][n][i];
      }
    }
}

// ------------------------------------------------ prefill, bounded path --
// Many tokens with bf16 x and W_r: the fp64 logits of every (token, expert)
// are more work than the selection needs.  Approximate logits L~ come from
// bf16 matrix cores with fp32 accumulation; every product of two bf16
// values is exact in fp32, and any fp32 summation of the H products (each
// addition faithfully rounded or better, plus one accumulator addition per
// 32 products) is within 2^-23 * (H + H/32) * sum|x_h w_eh| of the exact
// logit, and sum|x_h w_eh| <= |x| |w| (Cauchy-Schwarz).  So with
// B = 2^-23 * 1.125 H * |x| |w| (each norm replaced by an upper bound taken
// from an fp32 sum of squares, ra_norm_upper) the exact score lies in
// [s~ - B, s~ + B]; the two K halves of the matrix-core sum add one more
// rounding, inside the slack of 1.125 H.  Experts whose upper end lies below the
// k-th largest lower end cannot be selected; the rest (the k certain ones and
// the few near the boundary) get their logits recomputed exactly in fp64, and
// the selection and the gates are taken on those exact values.  Non-finite
// bounds (non-finite inputs) recompute every expert.
constexpr int RA_T = 64;   // tokens per workgroup
constexpr int RA_E = 128;  // experts per workgroup
constexpr int RA_K = 128;  // K per LDS stage (two halves of 64, one per wave group)
constexpr int RF_Q = 8;    // refine: 16-byte pieces per lane held in registers (H <= 4096)

typedef __bf16 ra_bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 ra_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float ra_f32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes from a valid address, zeroed where ok is false (an unconditional
// load and a select: no branch around the load)
__device__ __forceinline__ uint4 ra_ld16(const uint16_t* p, bool ok) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t m = 0u - (uint32_t)ok;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

__device__ __forceinline__ ra_bf16x8_t ra_as_bf16x8(uint4 v) {
  ra_bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// s + the squares of the eight bf16 values in v, fp32 (v_dot2c_f32_bf16)
__device__ __forceinline__ float ra_sq8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra_bf16x2_t p;
    __builtin_memcpy(&p, &w[j], 4);
    s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
  }
  return s;
}

// Upper bound on sqrt(sum of squares) from its fp32 accumulation over n
// terms: every square of a bf16 value is exact in fp32, each two-term step
// rounds at most twice (relative error below 2^-23 per step even for a
// directed rounding), so the exact sum is below q (1 + n 2^-21); squares
// flushed below the normal range add at most n 2^-126.
__device__ __forceinline__ double ra_norm_upper(float q, int n) {
  return sqrt((double)q * (1.0 + (double)n * 0x1p-21) + (double)n * 0x1p-120) * (1.0 + 0x1p-50);
}

// L~ [T, E] fp32 and |w_e| [E] (an upper bound, fp64).  Grid (T/64, E/128),
// eight waves: wave (wt, kh) takes tokens 16 wt .. 16 wt + 15 and all 128
// experts of the tile (8 blocks of v_mfma_f32_16x16x32_bf16) over the K half
// kh of every 128-K stage; the two halves are added once at the end in a
// fixed order.  W_r goes through double-buffered LDS, one 128 x 64
// sub-buffer per K half, rows of 128 bytes with 16-byte chunks XOR-swizzled
// by (row >> 1) & 7; x goes straight to registers, four stages ahead.
// |w_e|^2 is summed by one wave per group of rows, in the first eight
// workgroups of a column only.  (A 2 x 4 block per wave, which halves the
// LDS reads per product, measured slower: it doubles the x loads.)
__global__ void __launch_bounds__(512) route_approx_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr, float* __restrict__ la,
                                                           double* __restrict__ rw, int T,
                                                           int H, int E) {
  constexpr int HALF = RA_E * 64 * 2;  // bytes of one K-half sub-buffer
  __shared__ __attribute__((aligned(16))) uint8_t ws[2][2 * HALF];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, wt = wv & 3, kh = wv >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = blockIdx.x * RA_T, e0 = blockIdx.y * RA_E;
  const int ta = t0 + 16 * wt + c16;
  const bool tok_ok = ta < T;
  const uint16_t* xr = x + (int64_t)(tok_ok ? ta : T - 1) * H + 64 * kh + 8 * g;
  // stage pieces j < 4: K half j / 2, row (tid >> 3) + 64 (j & 1), chunk tid & 7
  const int prow = tid >> 3, pc = tid & 7;
  const uint16_t* wa = wr + (int64_t)min(e0 + prow, E - 1) * H + 8 * pc;
  const uint16_t* wb = wr + (int64_t)min(e0 + prow + 64, E - 1) * H + 8 * pc;
  const bool oka = e0 + prow < E, okb = e0 + prow + 64 < E;
  const int gx = gridDim.x;
  const bool do_nw = (gx >= 8) ? ((int)blockIdx.x == wv) : (wv % gx == (int)blockIdx.x);
  // Rows past T or E, and stages past the last one, are read at a clamped
  // (valid) place and zeroed after the load, so the loop below has no
  // branches: it runs a multiple of four stages, the extra ones all zeros
  // (both operands zero: they add exactly +0).
  const int nkc = H / RA_K, nkc4 = (nkc + 3) & ~3;
  auto wload = [&](int kc, uint4 (&r)[4]) {
    const int k0 = min(kc, nkc - 1) * RA_K;
    const bool ks = kc < nkc;
    r[0] = ra_ld16(wa + k0, oka && ks);
    r[1] = ra_ld16(wb + k0, okb && ks);
    r[2] = ra_ld16(wa + k0 + 64, oka && ks);
    r[3] = ra_ld16(wb + k0 + 64, okb && ks);
  };
  auto xload = [&](int kc, uint4 (&xa)[2]) {
    const int k0 = min(kc, nkc - 1) * RA_K;
    const bool ks = kc < nkc;
    xa[0] = ra_ld16(xr + k0, tok_ok && ks);
    xa[1] = ra_ld16(xr + k0 + 32, tok_ok && ks);
  };
  float nwa = 0.f, nwb = 0.f;
  // |w|^2 of the stage in r, then r into LDS buffer buf
  auto lstore = [&](int buf, const uint4 (&r)[4]) {
    if (do_nw) {
      nwa = ra_sq8(r[0], nwa);
      nwb = ra_sq8(r[1], nwb);
      nwa = ra_sq8(r[2], nwa);
      nwb = ra_sq8(r[3], nwb);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = prow + 64 * (j & 1);
      *reinterpret_cast<uint4*>(&ws[buf][(j >> 1) * HALF + row * 128 + 16 * (pc ^ ((row >> 1) & 7))]) = r[j];
    }
  };
  ra_f32x4_t acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = (ra_f32x4_t){0.f, 0.f, 0.f, 0.f};
  // x of stages kc .. kc + 3 in flight in xs[kc % 4]; W of stage kc + 1 in wq[(kc + 1) % 2]
  uint4 xs[4][2], wq[2][4];
  wload(0, wq[0]);
  wload(1, wq[1]);
#pragma unroll
  for (int u = 0; u < 4; ++u) xload(u, xs[u]);
  lstore(0, wq[0]);
  __syncthreads();
  for (int kc4 = 0; kc4 < nkc4; kc4 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = kc4 + u;
      wload(kc + 2, wq[u & 1]);
      const uint8_t* wsb = &ws[u & 1][kh * HALF];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 bv[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const int row = 16 * b + c16;
          bv[b] = *reinterpret_cast<const uint4*>(&wsb[row * 128 + 16 * ((4 * ks + g) ^ ((row >> 1) & 7))]);
        }
        const ra_bf16x8_t av = ra_as_bf16x8(xs[u][ks]);
#pragma unroll
        for (int b = 0; b < 8; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ra_as_bf16x8(bv[b]), acc[b], 0, 0, 0);
      }
      xload(kc + 4, xs[u]);
      lstore((u + 1) & 1, wq[(u + 1) & 1]);
      __syncthreads();
    }
  }
  // the K half 1 waves hand their partial sums over through LDS
  float* red = reinterpret_cast<float*>(&ws[0][0]);  // [4 wt][8 b][4 i][64 lanes]
  if (kh == 1) {
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wt * 8 + b) * 4 + i) * 64 + lane] = acc[b][i];
  }
  __syncthreads();
  if (kh == 0) {
    // D[4 g + i][c16]: token t0 + 16 wt + 4 g + i, expert e0 + 16 b + c16
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int e = e0 + 16 * b + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * wt + 4 * g + i;
        const float v = acc[b][i] + red[((wt * 8 + b) * 4 + i) * 64 + lane];
        if (t < T && e < E) la[(int64_t)t * E + e] = v;
      }
    }
  }
  // |w|: the eight lanes of a row hold disjoint chunks of every stage
  nwa += __shfl_xor(nwa, 1, 64);
  nwa += __shfl_xor(nwa, 2, 64);
  nwa += __shfl_xor(nwa, 4, 64);
  nwb += __shfl_xor(nwb, 1, 64);
  nwb += __shfl_xor(nwb, 2, 64);
  nwb += __shfl_xor(nwb, 4, 64);
  if (do_nw && pc == 0) {
    if (oka) rw[e0 + prow] = ra_norm_upper(nwa, H + 8);
    if (okb) rw[e0 + prow + 64] = ra_norm_upper(nwb, H + 8);
  }
}

// One wave per token: |x_t|, bounds, candidates, exact fp64 logits of the
// candidates, selection and gates.  Lane l owns the 16-byte pieces of a row
// at elements 8 l + 512 q.  Short rows (H <= 512 RF_Q, LONG false) keep the
// x row in registers; long rows go through it in chunks of 512 RF_Q.
template <int PER, bool LONG>
__global__ void __launch_bounds__(256) route_refine_kernel(const float* __restrict__ la,
                                                           const double* __restrict__ rw,
                                                           const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ sel_bias,
                                                           int32_t* __restrict__ ids, float* __restrict__ gates, int T,
                                                           int H, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  auto load_row = [&](const uint16_t* row, int q0, uint4 (&r)[RF_Q]) {  // row points at element 8 lane
#pragma unroll
    for (int q = 0; q < RF_Q; ++q) {
      const int off = 512 * (q0 + q), ok = 8 * lane + off < H;
      r[q] = ra_ld16(row + (ok ? off : -8 * lane), ok);  // pieces past H read the row's start
    }
  };
  const uint16_t* xr = x + (int64_t)t * H + 8 * lane;
  uint4 xq[RF_Q], wq[RF_Q];
  // |x_t|^2: fp32 partial sums per lane, then a fixed butterfly (H + 64 roundings at most)
  float q2 = 0.f;
  for (int q0 = 0; q0 == 0 || (LONG && 512 * q0 < H); q0 += RF_Q) {
    load_row(xr, q0, xq);
#pragma unroll
    for (int q = 0; q < RF_Q; ++q) q2 = ra_sq8(xq[q], q2);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q2 += __shfl_xor(q2, o, 64);
  const double rxt = ra_norm_upper(q2, H + 64);
  const double cB = 1.125 * (double)H * 0x1p-23;
  uint32_t lhi[PER], llo[PER];
  double ub[PER];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i, ec = min(e, E - 1);  // lanes past E read expert E - 1, then drop it
    const bool ok = e < E;
    double s = (double)la[(int64_t)t * E + ec];
    if (sel_bias) s += (double)sel_bias[(int64_t)t * E + ec];
    const double bnd = cB * (rxt * rw[ec]) * (1.0 + 1e-12) + 1e-30 + fabs(s) * 1e-15;
    if (ok && !(fabs(s) <= 1e300 && bnd <= 1e300)) bad = true;
    const uint64_t lk = ok ? dkey(s - bnd) + 1ull : 0ull;
    lhi[i] = (uint32_t)(lk >> 32);
    llo[i] = (uint32_t)lk;
    ub[i] = s + bnd;
  }
  const bool full = __ballot(bad) != 0ull;
  uint64_t cand[PER];
  if (full) {
#pragma unroll
    for (int i = 0; i < PER; ++i) cand[i] = __ballot(lane + 64 * i < E);
  } else {
    const uint64_t kth = tk_kth_largest<PER>(lhi, llo, k);  // k-th largest lower end (key + 1)
#pragma unroll
    for (int i = 0; i < PER; ++i) cand[i] = __ballot(lane + 64 * i < E && dkey(ub[i]) + 1ull >= kth);
  }
  // exact logits of the candidates (lowest id first); everything else cannot
  // win.  Sixteen independent fp64 chains per lane (piece parity x element
  // slot), folded in a fixed order, then the wave's fixed tree.
  double lv[PER], sv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) { lv[i] = -__builtin_inf(); sv[i] = -__builtin_inf(); }
  auto next_cand = [&]() -> int {  // lowest remaining candidate, removed; -1 when none
    int e = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (e < 0 && cand[i] != 0ull) {
        e = 64 * i + __builtin_ctzll(cand[i]);
        cand[i] &= cand[i] - 1;
      }
    return e;
  };
  auto dot = [](const uint4 (&a)[RF_Q], const uint4 (&b)[RF_Q], double (&acc)[16]) {
#pragma unroll
    for (int q = 0; q < RF_Q; ++q) {
      const uint32_t xa[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
      const uint32_t wa[4] = {b[q].x, b[q].y, b[q].z, b[q].w};
      const int c = 8 * (q & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[c + j] = fma((double)bf16_lo(xa[j]), (double)bf16_lo(wa[j]), acc[c + j]);
        acc[c + 4 + j] = fma((double)bf16_hi(xa[j]), (double)bf16_hi(wa[j]), acc[c + 4 + j]);
      }
    }
  };
  auto record = [&](int e, const double (&acc)[16]) {
    double f[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) f[c] = acc[c] + acc[c + 8];
    const double l = tk_wave_sum_f64(((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7])));
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (e == lane + 64 * i) {
        lv[i] = l;
        sv[i] = sel_bias ? l + (double)sel_bias[(int64_t)t * E + e] : l;
      }
  };
  if (!LONG) {
    for (int e = next_cand(); e >= 0; e = next_cand()) {
      double acc[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = 0.0;
      load_row(wr + (int64_t)e * H + 8 * lane, 0, wq);
      // keep the x row packed: converting it once outside this loop would
      // take 128 more registers per lane
#pragma unroll
      for (int q = 0; q < RF_Q; ++q) asm volatile("" : "+v"(xq[q].x), "+v"(xq[q].y), "+v"(xq[q].z), "+v"(xq[q].w));
      dot(xq, wq, acc);
      record(e, acc);
    }
  } else {
    for (int e = next_cand(); e >= 0; e = next_cand()) {
      const uint16_t* wrow = wr + (int64_t)e * H + 8 * lane;
      double acc[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = 0.0;
      for (int q0 = 0; 512 * q0 < H; q0 += RF_Q) {
        load_row(xr, q0, xq);
        load_row(wrow, q0, wq);
        dot(xq, wq, acc);
      }
      record(e, acc);
    }
  }
  topk_core<PER>(lv, sv, sel_bias != nullptr, E, k, 1, ids + (int64_t)t * k, gates + (int64_t)t * k);
}

template <bool LONG>
static void launch_refine(int nb, hipStream_t st, const float* la, const double* rw, const uint16_t* x,
                          const uint16_t* wr, const float* sel_bias, int32_t* ids, float* gates, int T, int H, int E,
                          int k) {
  if (E <= 64) route_refine_kernel<1, LONG><<<nb, 256, 0, st>>>(la, rw, x, wr, sel_bias, ids, gates, T, H, E, k);
  else if (E <= 128) route_refine_kernel<2, LONG><<<nb, 256, 0, st>>>(la, rw, x, wr, sel_bias, ids, gates, T, H, E, k);
  else if (E <= 256) route_refine_kernel<4, LONG><<<nb, 256, 0, st>>>(la, rw, x, wr, sel_bias, ids, gates, T, H, E, k);
  else if (E <= 512) route_refine_kernel<8, LONG><<<nb, 256, 0, st>>>(la, rw, x, wr, sel_bias, ids, gates, T, H, E, k);
  else route_refine_kernel<16, LONG><<<nb, 256, 0, st>>>(la, rw, x, wr, sel_bias, ids, gates, T, H, E, k);
}

hipError_t launch_route(const ft_moe_desc& d, const void* x, int T, const void* wr,
                        const float* sel_bias, int32_t* ids, float* gates, double* logits,
                        bool want_logits, hipStream_t st) {
  dim3 grid((T + RL_TT - 1) / RL_TT, (d.n_experts + RL_TE - 1) / RL_TE);
  const int xd = d.act_dtype, wd = d.router_dtype, H = d.hidden, E = d.n_experts;
  if (xd == FT_BF16 && wd == FT_BF16 && !want_logits && d.renormalize && H % RA_K == 0 && E <= 1024) {
    // bounded path; the logits buffer [T, E] fp64 holds L~ [T, E] fp32, then |w| [E] fp64
    float* la = reinterpret_cast<float*>(logits);
    double* rw = reinterpret_cast<double*>(la + (((int64_t)T * E + 63) / 64) * 64);
    route_approx_kernel<<<dim3((T + RA_T - 1) / RA_T, (E + RA_E - 1) / RA_E), 512, 0, st>>>(
        reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(wr), la, rw, T, H, E);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nb = (T + 3) / 4, k = d.top_k;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(wr);
    if (H <= 512 * RF_Q) launch_refine<false>(nb, st, la, rw, xb, wb, sel_bias, ids, gates, T, H, E, k);
    else launch_refine<true>(nb, st, la, rw, xb, wb, sel_bias, ids, gates, T, H, E, k);
    return hipGetLastError();
  }
  dim3 mgrid((T + RM_T - 1) / RM_T, (E + RM_E - 1) / RM_E);
  if (H % 32 == 0) {  // matrix-core path
    if (xd == FT_BF16 && wd == FT_BF16)
      route_logits_mfma_kernel<FT_BF16, FT_BF16><<<mgrid, 256, 0, st>>>(x, wr, logits, T, H, E);
    else if (xd == FT_F32 && wd == FT_F32)
      route_logits_mfma_kernel<FT_F32, FT_F32><<<mgrid, 256, 0, st>>>(x, wr, logits, T, H, E);
    else if (xd == FT_BF16 && wd == FT_F32)
      route_logits_mfma_kernel<FT_BF16, FT_F32><<<mgrid, 256, 0, st>>>(x, wr, logits, T, H, E);
    else
      route_logits_mfma_kernel<FT_F32, FT_BF16><<<mgrid, 256, 0, st>>>(x, wr, logits, T, H, E);
  } else if (xd == FT_BF16 && wd == FT_BF16)
    route_logits_tiled_kernel<FT_BF16, FT_BF16><<<grid, 256, 0, st>>>(x, wr, logits, T, H, E);
  else if (xd == FT_F32 && wd == FT_F32)
    route_logits_tiled_kernel<FT_F32, FT_F32><<<grid, 256, 0, st>>>(x, wr, logits, T, H, E);
  else if (xd == FT_BF16 && wd == FT_F32)
    route_logits_tiled_kernel<FT_BF16, FT_F32><<<grid, 256, 0, st>>>(x, wr, logits, T, H, E);
  else
    route_logits_tiled_kernel<FT_F32, FT_BF16><<<grid, 256, 0, st>>>(x, wr, logits, T, H, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int k = d.top_k, rn = d.renormalize;
  const int nb = (T + 3) / 4;
  if (E <= 64) route_topk_decode_kernel<1><<<nb, 256, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 128) route_topk_decode_kernel<2><<<nb, 256, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 256) route_topk_decode_kernel<4><<<nb, 256, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else if (E <= 512) route_topk_decode_kernel<8><<<nb, 256, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  else route_topk_decode_kernel<16><<<nb, 256, 0, st>>>(logits, sel_bias, ids, gates, T, E, k, rn);
  return hipGetLastError();
}

}  // namespace ft
