// Decode-sized grouped expert GEMV: for every active expert, the tokens
// routed to it (few at decode batch 1-4) are multiplied with that expert's
// weights, streamed once from HBM.
//   gate/up : h[p, i] = silu(G_i . x_t) * (U_i . x_t)      (p = sorted pair)
//   down    : y[p, r] = D_r . h[p, :]
//   combine : out[t, :] = sum_j [mask] g_tj * y[pos(t, j), :]   (j in order)
// SwiGLU with silu(z) = z / (1 + exp(-z)); the pages give no FFN formula
// (plain reading).  Accumulation is fp32 in a fixed order; weights are
// dequantised in registers (bf16 shift, E2M1 * E8M0, E2M1 * E4M3 * fp32).
#include "common.hpp"
#include "internal.hpp"

namespace ft {

constexpr int GV_ROWS = 4;     // rows per wave
constexpr int GV_WAVES = 4;    // waves per workgroup
constexpr int GV_TOK = 4;      // tokens per pass over the weights

// elements per lane per K step: 16 B of f32/bf16, 4 B of fp4 codes
template <int WD> struct Epl { static constexpr int v = (WD == FT_F32) ? 4 : 8; };

// Matrix view inside one expert record.
struct MatView {
  const uint8_t* codes;   // row-major elements / codes
  const uint8_t* scales;  // block scales (fp4 formats)
  float tscale;           // NVFP4 tensor scale
  int K;                  // reduction length (row length)
};

template <int WD>
__device__ __forceinline__ MatView mat_view(const uint8_t* rec, const RecordLayout& L, int m, int K) {
  MatView v;
  v.codes = rec + L.code_off[m];
  v.scales = rec + L.scale_off[m];
  v.K = K;
  v.tscale = 1.0f;
  if constexpr (WD == FT_NVFP4) v.tscale = reinterpret_cast<const float*>(rec + L.tscale_off)[m];
  return v;
}

// Dequantise the lane's chunk c (elements [c*EPL, c*EPL+EPL)) of row `row`.
template <int WD>
__device__ __forceinline__ void load_w(const MatView& v, int row, int c, float (&w)[Epl<WD>::v]) {
  constexpr int E = Epl<WD>::v;
  if constexpr (WD == FT_F32) {
    const float4 q = *reinterpret_cast<const float4*>(v.codes + ((int64_t)row * v.K + (int64_t)c * E) * 4);
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
  } else if constexpr (WD == FT_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(v.codes + ((int64_t)row * v.K + (int64_t)c * E) * 2);
    const uint32_t a[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) { w[2 * j] = bf16_lo(a[j]); w[2 * j + 1] = bf16_hi(a[j]); }
  } else {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(v.codes + ((int64_t)row * v.K + (int64_t)c * E) / 2);
    float s;
    if constexpr (WD == FT_MXFP4) {
      s = e8m0_to_f32(v.scales[(int64_t)row * (v.K / 32) + (c * E) / 32]);
    } else {
      s = e4m3_to_f32(v.scales[(int64_t)row * (v.K / 16) + (c * E) / 16]) * v.tscale;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = e2m1_to_f32((q >> (4 * j)) & 0xFu) * s;
  }
}

template <int N, typename XT>
__device__ __forceinline__ void load_x(const XT* row, int64_t off, float (&xv)[N]) {
  if constexpr (sizeof(XT) == 2) {  // bf16 bits
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row) + off;
    if constexpr (N == 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(p);
      const uint32_t a[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) { xv[2 * j] = bf16_lo(a[j]); xv[2 * j + 1] = bf16_hi(a[j]); }
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      xv[0] = bf16_lo(q.x); xv[1] = bf16_hi(q.x); xv[2] = bf16_lo(q.y); xv[3] = bf16_hi(q.y);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(row) + off;
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      const float4 q = *reinterpret_cast<const float4*>(p + j);
      xv[j] = q.x; xv[j + 1] = q.y; xv[j + 2] = q.z; xv[j + 3] = q.w;
    }
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Expert of unit d and its record.
// A negative slot (a failed lookup) yields nullptr: the expert is skipped and
// its outputs are NaN, never an out-of-bounds read.
__device__ __forceinline__ const uint8_t* expert_record_ptr(const void* pool, int64_t stride, const int32_t* slot_ids,
                                                           const int32_t* perm, int off, int e) {
  const int slot = slot_ids ? slot_ids[perm[off]] : e;
  if (slot < 0) return nullptr;
  return reinterpret_cast<const uint8_t*>(pool) + (int64_t)slot * stride;
}

template <int WD, typename XT>
__global__ void __launch_bounds__(GV_WAVES * 64) gateup_gemv_kernel(
    const XT* __restrict__ x, const void* __restrict__ pool, int64_t stride, const int32_t* __restrict__ slot_ids,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active, const int32_t* __restrict__ perm,
    float* __restrict__ hbuf, int H, int I, int E, int k, int row_blocks) {
  constexpr int EPL = Epl<WD>::v;
  const int d = blockIdx.x / row_blocks, rb = blockIdx.x % row_blocks;
  if (d >= offsets[E + 1]) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = active[d];
  const int off = offsets[e], cnt = offsets[e + 1] - off;
  const uint8_t* rec = expert_record_ptr(pool, stride, slot_ids, perm, off, e);
  const int row0 = rb * (GV_WAVES * GV_ROWS) + wv * GV_ROWS;
  if (rec == nullptr) {
    for (int q = lane; q < cnt * GV_ROWS; q += 64) {
      const int row = row0 + q % GV_ROWS;
      if (row < I) hbuf[(int64_t)(off + q / GV_ROWS) * I + row] = __builtin_nanf("");
    }
    return;
  }
  const RecordLayout L = record_layout(H, I, WD);
  const MatView G = mat_view<WD>(rec, L, 0, H), U = mat_view<WD>(rec, L, 1, H);
  const int nchunk = H / EPL;
  for (int tg = 0; tg < cnt; tg += GV_TOK) {
    const int nt = min(GV_TOK, cnt - tg);
    int tok[GV_TOK];
#pragma unroll
    for (int q = 0; q < GV_TOK; ++q) tok[q] = (q < nt) ? perm[off + tg + q] / k : 0;
    float ag[GV_ROWS][GV_TOK], au[GV_ROWS][GV_TOK];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) { ag[r][q] = 0.f; au[r][q] = 0.f; }
    for (int c = lane; c < nchunk; c += 64) {
      float xv[GV_TOK][EPL];
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) load_x<EPL>(x + (int64_t)tok[q] * H, (int64_t)c * EPL, xv[q]);
#pragma unroll
      for (int r = 0; r < GV_ROWS; ++r) {
        const int row = row0 + r;
        if (row < I) {
          float wg[EPL], wu[EPL];
          load_w<WD>(G, row, c, wg);
          load_w<WD>(U, row, c, wu);
#pragma unroll
          for (int q = 0; q < GV_TOK; ++q)
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
              ag[r][q] = fmaf(wg[j], xv[q][j], ag[r][q]);
              au[r][q] = fmaf(wu[j], xv[q][j], au[r][q]);
            }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) {
        const float g = wave_sum(ag[r][q]);
        const float u = wave_sum(au[r][q]);
        const int row = row0 + r;
        if (lane == 0 && q < nt && row < I) hbuf[(int64_t)(off + tg + q) * I + row] = silu_f(g) * u;
      }
  }
}

template <int WD>
__global__ void __launch_bounds__(GV_WAVES * 64) down_gemv_kernel(
    const float* __restrict__ hbuf, const void* __restrict__ pool, int64_t stride,
    const int32_t* __restrict__ slot_ids, const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ perm, float* __restrict__ ybuf, int H, int I, int E, int row_blocks) {
  constexpr int EPL = Epl<WD>::v;
  const int d = blockIdx.x / row_blocks, rb = blockIdx.x % row_blocks;
  if (d >= offsets[E + 1]) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = active[d];
  const int off = offsets[e], cnt = offsets[e + 1] - off;
  const uint8_t* rec = expert_record_ptr(pool, stride, slot_ids, perm, off, e);
  const int row0 = rb * (GV_WAVES * GV_ROWS) + wv * GV_ROWS;
  if (rec == nullptr) {
    for (int q = lane; q < cnt * GV_ROWS; q += 64) {
      const int row = row0 + q % GV_ROWS;
      if (row < H) ybuf[(int64_t)(off + q / GV_ROWS) * H + row] = __builtin_nanf("");
    }
    return;
  }
  const RecordLayout L = record_layout(H, I, WD);
  const MatView D = mat_view<WD>(rec, L, 2, I);
  const int nchunk = I / EPL;
  for (int tg = 0; tg < cnt; tg += GV_TOK) {
    const int nt = min(GV_TOK, cnt - tg);
    float acc[GV_ROWS][GV_TOK];
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) acc[r][q] = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      float hv[GV_TOK][EPL];
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) {
        const int pq = off + tg + ((q < nt) ? q : 0);
        load_x<EPL>(hbuf + (int64_t)pq * I, (int64_t)c * EPL, hv[q]);
      }
#pragma unroll
      for (int r = 0; r < GV_ROWS; ++r) {
        const int row = row0 + r;
        if (row < H) {
          float w[EPL];
          load_w<WD>(D, row, c, w);
#pragma unroll
          for (int q = 0; q < GV_TOK; ++q)
#pragma unroll
            for (int j = 0; j < EPL; ++j) acc[r][q] = fmaf(w[j], hv[q][j], acc[r][q]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < GV_ROWS; ++r)
#pragma unroll
      for (int q = 0; q < GV_TOK; ++q) {
        const float s = wave_sum(acc[r][q]);
        const int row = row0 + r;
        if (lane == 0 && q < nt && row < H) ybuf[(int64_t)(off + tg + q) * H + row] = s;
      }
  }
}

// out[t, :] = sum_j [pair kept] g[t,j] * y[pos(t,j), :], j ascending, fp32.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ ybuf, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ gates, float* __restrict__ out, int T,
                                                      int H, int k) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (t >= T || h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int p = pos[(int64_t)t * k + j];
    if (p < 0) continue;
    const float g = gates[(int64_t)t * k + j];
    const float4 y = *reinterpret_cast<const float4*>(ybuf + (int64_t)p * H + h);
    acc.x = fmaf(g, y.x, acc.x);
    acc.y = fmaf(g, y.y, acc.y);
    acc.z = fmaf(g, y.z, acc.z);
    acc.w = fmaf(g, y.w, acc.w);
  }
  *reinterpret_cast<float4*>(out + (int64_t)t * H + h) = acc;
}

// The same combine over expert outputs stored in bf16 (the matrix-core path):
// 8 columns per thread, fp32 accumulation in the same fixed j order.
__global__ void __launch_bounds__(256) combine_bf16_kernel(const uint16_t* __restrict__ ybuf,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ gates, float* __restrict__ out,
                                                           int T, int H, int k) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (t >= T || h >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // up to eight pairs at a time with all their loads in flight (positions and
  // gates first, then the y rows; a masked-out pair reads row 0 and adds 0),
  // summed in rank order
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pj[8];
    float gj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, k - 1);
      pj[u] = pos[(int64_t)t * k + j];
      gj[u] = gates[(int64_t)t * k + j];
    }
    uint4 yj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) yj[u] = *reinterpret_cast<const uint4*>(ybuf + (int64_t)max(pj[u], 0) * H + h);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u >= k || pj[u] < 0) continue;
      const uint32_t w[4] = {yj[u].x, yj[u].y, yj[u].z, yj[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(gj[u], bf16_lo(w[q]), acc[2 * q]);
        acc[2 * q + 1] = fmaf(gj[u], bf16_hi(w[q]), acc[2 * q + 1]);
      }
    }
  }
  float4* o = reinterpret_cast<float4*>(out + (int64_t)t * H + h);
  o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// out += part, elementwise (the sum of two partial outputs over disjoint
// expert sets)
__global__ void __launch_bounds__(256) add_partial_kernel(float* __restrict__ out, const float* __restrict__ part,
                                                          int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] += part[i];
}

hipError_t launch_add_partial(float* out, const float* part, int64_t n, hipStream_t st) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  add_partial_kernel<<<(unsigned)blocks, 256, 0, st>>>(out, part, n);
  return hipGetLastError();
}

hipError_t launch_combine(const FwdPlan& pl, const int32_t* pos, const float* gates, float* out, char* ws,
                          hipStream_t st) {
  const uint16_t* ybuf = reinterpret_cast<const uint16_t*>(ws + pl.off_y);
  dim3 cg((pl.H / 8 + 255) / 256, pl.T);
  combine_bf16_kernel<<<cg, 256, 0, st>>>(ybuf, pos, gates, out, pl.T, pl.H, pl.P / pl.T);
  return hipGetLastError();
}

template <int WD>
static hipError_t gemv_forward_t(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                                 const void* pool, const float* gates, float* out, char* ws, hipStream_t st) {
  const int32_t* offsets = reinterpret_cast<const int32_t*>(ws + pl.off_offsets);
  const int32_t* active = reinterpret_cast<const int32_t*>(ws + pl.off_active);
  const int32_t* perm = reinterpret_cast<const int32_t*>(ws + pl.off_perm);
  const int32_t* pos = reinterpret_cast<const int32_t*>(ws + pl.off_pos);
  float* hbuf = reinterpret_cast<float*>(ws + pl.off_h);
  float* ybuf = reinterpret_cast<float*>(ws + pl.off_y);
  const int H = d.hidden, I = d.inter, E = d.n_experts, k = d.top_k;
  const int max_active = pl.P < E ? pl.P : E;
  const int rows_per_wg = GV_WAVES * GV_ROWS;
  const int rb_gu = (I + rows_per_wg - 1) / rows_per_wg;
  const int rb_dn = (H + rows_per_wg - 1) / rows_per_wg;
  if (d.act_dtype == FT_BF16)
    gateup_gemv_kernel<WD, uint16_t><<<max_active * rb_gu, GV_WAVES * 64, 0, st>>>(
        reinterpret_cast<const uint16_t*>(x), pool, d.expert_stride, slot_ids, offsets, active, perm, hbuf, H, I, E,
        k, rb_gu);
  else
    gateup_gemv_kernel<WD, float><<<max_active * rb_gu, GV_WAVES * 64, 0, st>>>(
        reinterpret_cast<const float*>(x), pool, d.expert_stride, slot_ids, offsets, active, perm, hbuf, H, I, E, k,
        rb_gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  down_gemv_kernel<WD><<<max_active * rb_dn, GV_WAVES * 64, 0, st>>>(hbuf, pool, d.expert_stride, slot_ids, offsets,
                                                                     active, perm, ybuf, H, I, E, rb_dn);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 cg((H / 4 + 255) / 256, pl.T);
  combine_kernel<<<cg, 256, 0, st>>>(ybuf, pos, gates, out, pl.T, H, k);
  return hipGetLastError();
}

hipError_t launch_gemv_forward(const ft_moe_desc& d, const FwdPlan& pl, const void* x, const int32_t* slot_ids,
                               const void* pool, const float* gates, float* out, char* ws, hipStream_t st) {
  switch (d.w_dtype) {
    case FT_F32: return gemv_forward_t<FT_F32>(d, pl, x, slot_ids, pool, gates, out, ws, st);
    case FT_BF16: return gemv_forward_t<FT_BF16>(d, pl, x, slot_ids, pool, gates, out, ws, st);
    case FT_MXFP4: return gemv_forward_t<FT_MXFP4>(d, pl, x, slot_ids, pool, gates, out, ws, st);
    default: return gemv_forward_t<FT_NVFP4>(d, pl, x, slot_ids, pool, gates, out, ws, st);
  }
}

}  // namespace ft
