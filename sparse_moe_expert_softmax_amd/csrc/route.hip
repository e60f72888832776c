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

// ---------------------------------------------------------------- decode --
// One launch for few tokens: workgroup e computes the logits of expert e for
// all T <= 16 tokens (its 4 waves split H; fp64 partial sums reduced across
// the wave with a multi-value butterfly, then across waves in LDS, in a fixed
// order identical for every expert).  The workgroup that finishes last (a
// device-scope counter in the workspace, reset after use) runs the top-k.
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

// orderable key of a double: larger key = larger value; NaN lowest
__device__ __forceinline__ uint64_t dkey(double s) {
  if (s != s) return 0ull;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int PER>
__device__ void topk_one_token(const double* __restrict__ lt, const float* __restrict__ bias_t, int E, int k,
                               int renormalize, int32_t* __restrict__ ids_t, float* __restrict__ gates_t) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      double v = lt[e];
      if (bias_t) v += (double)bias_t[e];
      key[i] = dkey(v) | 0ull;
    } else {
      key[i] = 0ull;
    }
  }
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;
  int my_id = -1;
  for (int j = 0; j < k; ++j) {
    uint64_t bk = 0ull;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (!((taken >> i) & 1u) && (key[i] > bk || (key[i] == bk && e < be))) { bk = key[i]; be = e; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t ok = __shfl_xor(bk, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) my_id = be;
  }
  const bool sel = lane < k;
  const double l = sel ? lt[my_id] : 0.0;
  double gsel;
  if (renormalize) {
    double m = sel ? l : -__builtin_inf();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
    const double ex = sel ? exp(l - m) : 0.0;
    gsel = ex / wave_sum(ex);
  } else {
    double m = -__builtin_inf();
    for (int e = lane; e < E; e += 64) m = fmax(m, lt[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp(lt[e] - m);
    const double den = wave_sum(part);
    gsel = sel ? exp(l - m) / den : 0.0;
  }
  if (sel) {
    ids_t[lane] = my_id;
    gates_t[lane] = (float)gsel;
  }
}

template <int XDT, int WDT, int NT>
__global__ void __launch_bounds__(256) route_decode_kernel(const void* __restrict__ x, const void* __restrict__ wr,
                                                           const float* __restrict__ sel_bias,
                                                           double* __restrict__ logits, int32_t* __restrict__ ids,
                                                           float* __restrict__ gates, uint32_t* __restrict__ counter,
                                                           int T, int H, int E, int k, int renormalize) {
  __shared__ double part[4][RD_MAXT];
  __shared__ int last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x;
  double acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0;
  const int hq = H / 4;  // this wave's quarter of H (H % 32 == 0)
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
  const double r = multi_reduce<NT>(acc);
  constexpr int SH = (NT == 1) ? 6 : (NT == 2) ? 5 : (NT == 4) ? 4 : (NT == 8) ? 3 : 2;
  if ((lane & ((1 << SH) - 1)) == 0) part[wv][lane >> SH] = r;
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    logits[(int64_t)t * E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = (atomicAdd(counter, 1u) == (uint32_t)(gridDim.x - 1));
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int t = wv; t < T; t += 4) {
    const double* lt = logits + (int64_t)t * E;
    const float* bt = sel_bias ? sel_bias + (int64_t)t * E : nullptr;
    if (E <= 64) topk_one_token<1>(lt, bt, E, k, renormalize, ids + (int64_t)t * k, gates + (int64_t)t * k);
    else if (E <= 128) topk_one_token<2>(lt, bt, E, k, renormalize, ids + (int64_t)t * k, gates + (int64_t)t * k);
    else if (E <= 256) topk_one_token<4>(lt, bt, E, k, renormalize, ids + (int64_t)t * k, gates + (int64_t)t * k);
    else if (E <= 512) topk_one_token<8>(lt, bt, E, k, renormalize, ids + (int64_t)t * k, gates + (int64_t)t * k);
    else topk_one_token<16>(lt, bt, E, k, renormalize, ids + (int64_t)t * k, gates + (int64_t)t * k);
  }
  if (threadIdx.x == 0) *counter = 0u;
}

template <int XDT, int WDT>
static void launch_route_decode_t(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                                  int32_t* ids, float* gates, double* logits, uint32_t* counter, hipStream_t st) {
  const int H = d.hidden, E = d.n_experts, k = d.top_k, rn = d.renormalize;
  if (T <= 1)
    route_decode_kernel<XDT, WDT, 1><<<E, 256, 0, st>>>(x, wr, sel_bias, logits, ids, gates, counter, T, H, E, k, rn);
  else if (T <= 2)
    route_decode_kernel<XDT, WDT, 2><<<E, 256, 0, st>>>(x, wr, sel_bias, logits, ids, gates, counter, T, H, E, k, rn);
  else if (T <= 4)
    route_decode_kernel<XDT, WDT, 4><<<E, 256, 0, st>>>(x, wr, sel_bias, logits, ids, gates, counter, T, H, E, k, rn);
  else if (T <= 8)
    route_decode_kernel<XDT, WDT, 8><<<E, 256, 0, st>>>(x, wr, sel_bias, logits, ids, gates, counter, T, H, E, k, rn);
  else
    route_decode_kernel<XDT, WDT, 16><<<E, 256, 0, st>>>(x, wr, sel_bias, logits, ids, gates, counter, T, H, E, k, rn);
}

hipError_t launch_route_decode(const ft_moe_desc& d, const void* x, int T, const void* wr, const float* sel_bias,
                               int32_t* ids, float* gates, double* logits, uint32_t* counter, hipStream_t st) {
  const int xd = d.act_dtype, wd = d.router_dtype;
  if (xd == FT_BF16 && wd == FT_BF16) launch_route_decode_t<FT_BF16, FT_BF16>(d, x, T, wr, sel_bias, ids, gates, logits, counter, st);
  else if (xd == FT_F32 && wd == FT_F32) launch_route_decode_t<FT_F32, FT_F32>(d, x, T, wr, sel_bias, ids, gates, logits, counter, st);
  else if (xd == FT_BF16 && wd == FT_F32) launch_route_decode_t<FT_BF16, FT_F32>(d, x, T, wr, sel_bias, ids, gates, logits, counter, st);
  else launch_route_decode_t<FT_F32, FT_BF16>(d, x, T, wr, sel_bias, ids, gates, logits, counter, st);
  return hipGetLastError();
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
