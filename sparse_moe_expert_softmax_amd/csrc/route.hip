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

// One wave per (expert, tile of RT tokens); lanes stride over H, 8 elements each.
template <int XDT, int WDT, int RT>
__global__ void __launch_bounds__(256) route_logits_kernel(const void* __restrict__ x,
                                                           const void* __restrict__ wr,
                                                           double* __restrict__ logits, int T, int H,
                                                           int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * RT;
  if (e >= E) return;
  double acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = 0.0;
  for (int h = lane * 8; h < H; h += 64 * 8) {
    double w[8];
    load8_f64<WDT>(wr, (int64_t)e * H + h, w);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (t0 + r < T) {
        double xv[8];
        load8_f64<XDT>(x, (int64_t)(t0 + r) * H + h, xv);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r] = fma(xv[j], w[j], acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const double s = wave_sum(acc[r]);
    if (lane == 0 && t0 + r < T) logits[(int64_t)(t0 + r) * E + e] = s;
  }
}

// Candidate order: a beats b if a's score is larger, or equal with lower id;
// NaN ranks below every number.
__device__ __forceinline__ bool beats(double a, int ea, double b, int eb) {
  const bool na = a != a, nb = b != b;
  if (na || nb) {
    if (!na) return true;
    if (!nb) return false;
    return ea < eb;
  }
  return a > b || (a == b && ea < eb);
}

constexpr int MAX_E_PER_LANE = 16;  // E <= 1024

// One wave per token.
__global__ void __launch_bounds__(256) route_topk_kernel(const double* __restrict__ logits,
                                                         const float* __restrict__ sel_bias,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ gates, int T, int E,
                                                         int k, int renormalize) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double* lt = logits + (int64_t)t * E;
  double s[MAX_E_PER_LANE];
  uint32_t taken = 0;
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < MAX_E_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    double v = __longlong_as_double(0x7FF8000000000000LL);  // NaN = empty
    if (i < per && e < E) {
      v = lt[e];
      if (sel_bias) v += (double)sel_bias[(int64_t)t * E + e];
    } else {
      taken |= 1u << i;
    }
    s[i] = v;
  }
  int my_id = -1;  // lane j < k ends up holding the j-th selected id
  for (int j = 0; j < k; ++j) {
    double best = __longlong_as_double(0x7FF8000000000000LL);
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < MAX_E_PER_LANE; ++i) {
      if (!(taken >> i & 1u) && beats(s[i], lane + 64 * i, best, be)) {
        best = s[i];
        be = lane + 64 * i;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ob = __shfl_xor(best, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (beats(ob, oe, best, be)) { best = ob; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) my_id = be;
  }
  // gates in fp64
  const bool sel = lane < k;
  const double l = sel ? lt[my_id] : 0.0;
  double g;
  if (renormalize) {
    double m = sel ? l : -__builtin_inf();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
    const double ex = sel ? exp(l - m) : 0.0;
    const double den = wave_sum(ex);
    g = ex / den;
  } else {
    double m = -__builtin_inf();
    for (int e = lane; e < E; e += 64) m = fmax(m, lt[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp(lt[e] - m);
    const double den = wave_sum(part);
    g = sel ? exp(l - m) / den : 0.0;
  }
  if (sel) {
    ids[(int64_t)t * k + lane] = my_id;
    gates[(int64_t)t * k + lane] = (float)g;
  }
}

hipError_t launch_route(const ft_moe_desc& d, const void* x, int T, const void* wr,
                        const float* sel_bias, int32_t* ids, float* gates, double* logits,
                        hipStream_t st) {
  constexpr int RT = 4;
  dim3 grid((d.n_experts + 3) / 4, (T + RT - 1) / RT);
  const int xd = d.act_dtype, wd = d.router_dtype;
  if (xd == FT_BF16 && wd == FT_BF16)
    route_logits_kernel<FT_BF16, FT_BF16, RT><<<grid, 256, 0, st>>>(x, wr, logits, T, d.hidden, d.n_experts);
  else if (xd == FT_F32 && wd == FT_F32)
    route_logits_kernel<FT_F32, FT_F32, RT><<<grid, 256, 0, st>>>(x, wr, logits, T, d.hidden, d.n_experts);
  else if (xd == FT_BF16 && wd == FT_F32)
    route_logits_kernel<FT_BF16, FT_F32, RT><<<grid, 256, 0, st>>>(x, wr, logits, T, d.hidden, d.n_experts);
  else
    route_logits_kernel<FT_F32, FT_BF16, RT><<<grid, 256, 0, st>>>(x, wr, logits, T, d.hidden, d.n_experts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  route_topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, sel_bias, ids, gates, T, d.n_experts,
                                                 d.top_k, d.renormalize);
  return hipGetLastError();
}

}  // namespace ft
