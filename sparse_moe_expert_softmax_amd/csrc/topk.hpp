// Top-k selection of one token's expert scores by one wave: the routing
// rule of the pages (softmax gates over the k highest-scoring experts,
// neither changed nor approximated; FreeToken explainer page, "how" and
// "who" sections), shared by the router and the fused decode path.
#pragma once
#include "common.hpp"

namespace ft {

// orderable key of a double: larger key = larger value; NaN lowest
__device__ __forceinline__ uint64_t dkey(double s) {
  if (s != s) return 0ull;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Top-k of one token's E <= 64*PER scores by one wave: k rounds of a
// wave-wide maximum over the orderable 64-bit keys of the experts not yet
// taken (the high halves; the low halves only where several keys share the
// highest high half), the lowest expert id winning among equal keys.  Round j
// yields the expert of rank j, so the order is (score desc, id asc) by
// construction.  Keys are stored plus one, so 0 marks an expert that is
// taken or does not exist while a NaN score (key 0) stays selectable, below
// every number.  The gates are formed afterwards with the softmax
// denominator summed over the winners in ascending id order.  No LDS is used.

// wave-wide unsigned 32-bit maximum, returned as a uniform value: six DPP
// steps (quads, rows of 16, then across rows), the result in lane 63; each
// step waits the two wait states a DPP read of a just-written VGPR needs
__device__ __forceinline__ uint32_t tk_wave_max_u32(uint32_t v) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// one DPP step of a wave-wide fp64 sum: a + (a moved by the DPP control)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double tk_dpp_add_f64(double a) {
  const uint64_t u = (uint64_t)__double_as_longlong(a);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  return a + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// wave-wide fp64 sum in a fixed order (quads, rows, then across rows; the
// total lands in lane 63), returned as a uniform value
__device__ __forceinline__ double tk_wave_sum_f64(double v) {
  v = tk_dpp_add_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = tk_dpp_add_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = tk_dpp_add_f64<0x124, 0xF>(v);  // row_ror:4
  v = tk_dpp_add_f64<0x128, 0xF>(v);  // row_ror:8
  v = tk_dpp_add_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = tk_dpp_add_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double tk_readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The selection from values in registers: lane l holds expert l + 64 i as
// logit lv[i] and score sv[i] (logit plus any selection bias).
template <int PER>
__device__ void topk_core(const double (&lv)[PER], const double (&sv)[PER], bool has_bias, int E, int k,
                          int renormalize, int32_t* __restrict__ ids_t, float* __restrict__ gates_t) {
  const int lane = threadIdx.x & 63;
  uint32_t khi[PER], klo[PER];  // key + 1 of the experts not yet taken, else 0
  int rank[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool ok = lane + 64 * i < E;
    const uint64_t key = ok ? dkey(sv[i]) + 1ull : 0ull;  // dkey <= dkey(+inf) < 2^64 - 1
    khi[i] = (uint32_t)(key >> 32);
    klo[i] = (uint32_t)key;
    rank[i] = 0;
  }
  double mx = -__builtin_inf();  // largest logit among the winners
  for (int j = 0; j < k; ++j) {
    uint32_t h = khi[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) h = max(h, khi[i]);
    const uint32_t mh = tk_wave_max_u32(h);
    // experts holding that high half; the low halves decide only among several
    uint64_t mt[PER];
    int nt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mt[i] = __ballot(khi[i] == mh && (khi[i] | klo[i]) != 0u);
      nt += __popcll(mt[i]);
    }
    if (nt > 1) {
      uint32_t l = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((mt[i] >> lane) & 1ull) l = max(l, klo[i]);
      const uint32_t ml = tk_wave_max_u32(l);
#pragma unroll
      for (int i = 0; i < PER; ++i) mt[i] = __ballot(((mt[i] >> lane) & 1ull) && klo[i] == ml);
    }
    int w = -1, iw = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (w < 0 && mt[i] != 0ull) { w = __builtin_ctzll(mt[i]); iw = i; }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == iw) {
        if (lane == w) { rank[i] = j; khi[i] = 0u; klo[i] = 0u; }
        // without a selection bias the first winner holds the largest logit
        if (j == 0 || has_bias) mx = fmax(mx, tk_readlane_f64(lv[i], w));
      }
  }
  // winners: the experts that exist and were taken
  uint64_t sel[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sel[i] = __ballot(lane + 64 * i < E && (khi[i] | klo[i]) == 0u);
  if (renormalize) {
    double ex[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) ex[i] = ((sel[i] >> lane) & 1ull) ? exp(lv[i] - mx) : 0.0;
    double den = 0.0;
#pragma unroll
    for (int iw = 0; iw < PER; ++iw) {
      uint64_t m = sel[iw];
      while (m) {
        const int lw = __builtin_ctzll(m);
        m &= m - 1;
        den += tk_readlane_f64(ex[iw], lw);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((sel[i] >> lane) & 1ull) {
        ids_t[rank[i]] = lane + 64 * i;
        gates_t[rank[i]] = (float)(ex[i] / den);
      }
  } else {
    double mxa = -__builtin_inf();
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < E) mxa = fmax(mxa, lv[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mxa = fmax(mxa, __shfl_xor(mxa, o, 64));
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < E) part += exp(lv[i] - mxa);
    const double den = wave_sum(part);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((sel[i] >> lane) & 1ull) {
        ids_t[rank[i]] = lane + 64 * i;
        gates_t[rank[i]] = (float)(exp(lv[i] - mxa) / den);
      }
  }
}

template <int PER>
__device__ __forceinline__ void topk_one_token(const double* __restrict__ lt, const float* __restrict__ bias_t, int E, int k,
                               int renormalize, int32_t* __restrict__ ids_t, float* __restrict__ gates_t) {
  const int lane = threadIdx.x & 63;
  double lv[PER], sv[PER];
  // unconditional loads from clamped indices (lanes past E read expert E - 1
  // and drop it), so all of them are in flight at once
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const double l = lt[e < E ? e : E - 1];
    lv[i] = e < E ? l : 0.0;
    sv[i] = lv[i];
  }
  if (bias_t) {
    float b[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) b[i] = bias_t[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < E) sv[i] += (double)b[i];
  }
  topk_core<PER>(lv, sv, bias_t != nullptr, E, k, renormalize, ids_t, gates_t);
}

// Top-k of ONE token by a whole workgroup of NTHR threads (E <= 64 * PER),
// with renormalised gates.  Each expert's rank is the number of experts whose
// key has a larger high half, counted by NTHR / (64 PER) threads, each over
// an equal share of the experts, from high halves broadcast out of LDS: a
// few hundred cycles of independent compares instead of k dependent rounds.
// Where the high halves within the top k are distinct, the ranks below k name
// k different experts in the order of topk_core's rounds.  Where one is shared
// (scores equal, or equal to about one part in a million, or NaN scores and
// absent experts needed to fill k), two experts claim one rank and another
// rank stays empty; the function then returns false with nothing stored, and
// the caller runs topk_one_token, which breaks such ties exactly.  The gates
// are topk_core's: the same exponentials, summed in ascending expert id order,
// so every result is bitwise that of topk_one_token.  `scr`: 3,364 bytes of
// LDS the caller does not need meanwhile.  All NTHR threads call it together.
template <int PER, int NTHR>
__device__ __forceinline__ bool topk_wg_one_token(const double* __restrict__ lt, const float* __restrict__ bias_t, int E, int k,
                                  int32_t* __restrict__ ids_t, float* __restrict__ gates_t, unsigned char* scr) {
  constexpr int EP = 64 * PER, NT = NTHR / EP, SPAN = EP / NT;
  static_assert(NT * EP == NTHR && SPAN % 4 == 0 && EP <= 256, "workgroup shape");
  uint32_t* s_hi = reinterpret_cast<uint32_t*>(scr);          // [EP]   high halves of the keys
  int* s_cnt = reinterpret_cast<int*>(scr + 1024);             // [NTHR] partial counts
  double* s_ex = reinterpret_cast<double*>(scr + 2048);        // [k]    exponentials, ascending id
  double* s_lw = reinterpret_cast<double*>(scr + 2560);        // [k]    winners' logits by rank
  int* s_win = reinterpret_cast<int*>(scr + 3072);             // [k]    winner of each rank
  uint64_t* s_wm = reinterpret_cast<uint64_t*>(scr + 3328);    // [PER]  winners, one word per 64 ids
  int* s_bad = reinterpret_cast<int*>(scr + 3360);
  const int tid = threadIdx.x, lane = tid & 63, i = tid % EP, part = tid / EP;
  const int ic = i < E ? i : E - 1;  // clamped: every load issues at once
  const double l = lt[ic];
  const float b = bias_t ? bias_t[ic] : 0.f;
  double sc = l;
  if (bias_t) sc += (double)b;
  const uint32_t hi = (i < E) ? (uint32_t)((dkey(sc) + 1ull) >> 32) : 0u;
  if (part == 0) s_hi[i] = hi;
  if (tid < k) s_win[tid] = -1;
  if (tid == 0) *s_bad = 0;
  __syncthreads();
  // eight 16-byte broadcast reads in flight, then their compares (left to
  // itself the compiler waited for each read before the next one: 64
  // serialised LDS round trips at 256 experts)
  constexpr int NQ = SPAN / 4, QB = NQ < 8 ? NQ : 8;
  static_assert(NQ % QB == 0, "batches");
  int cnt = 0;
  const uint4* h4 = reinterpret_cast<const uint4*>(s_hi + part * SPAN);
#pragma unroll
  for (int q0 = 0; q0 < NQ; q0 += QB) {
    uint4 v[QB];
#pragma unroll
    for (int u = 0; u < QB; ++u) v[u] = h4[q0 + u];
#pragma unroll
    for (int u = 0; u < QB; ++u)
      cnt += (v[u].x > hi ? 1 : 0) + (v[u].y > hi ? 1 : 0) + (v[u].z > hi ? 1 : 0) + (v[u].w > hi ? 1 : 0);
  }
  s_cnt[tid] = cnt;
  __syncthreads();
  int rank = 0;
  bool win = false;
  if (part == 0) {
#pragma unroll
    for (int p = 0; p < NT; ++p) rank += s_cnt[i + p * EP];
    win = i < E && rank < k;
    if (win) {
      s_win[rank] = i;
      s_lw[rank] = l;
    }
  }
  const uint64_t wm = __ballot(win);  // part 0 is waves 0 .. PER-1, expert i = tid
  if (part == 0 && lane == 0) s_wm[tid >> 6] = wm;
  __syncthreads();
  // two claimants of one rank: one of them reads the other's id; an empty rank reads -1
  if ((win && s_win[rank] != i) || (tid < k && s_win[tid] < 0)) *s_bad = 1;
  __syncthreads();
  if (*s_bad) return false;
  double ex = 0.0;
  if (win) {
    double mx = -__builtin_inf();  // topk_core: the rank-0 logit, or the largest winner logit with a bias
    if (bias_t) {
      for (int q = 0; q < k; ++q) mx = fmax(mx, s_lw[q]);
    } else {
      mx = fmax(mx, s_lw[0]);
    }
    ex = exp(l - mx);
    const int w = tid >> 6;
    int pos = __popcll(s_wm[w] & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    for (int q = 0; q < w; ++q) pos += __popcll(s_wm[q]);
    s_ex[pos] = ex;
  }
  __syncthreads();
  if (win) {
    double den = 0.0;
    for (int q = 0; q < k; ++q) den += s_ex[q];
    ids_t[rank] = i;
    gates_t[rank] = (float)(ex / den);
  }
  return true;
}

// The k-th largest of the wave's keys (key + 1 per expert, 0 = absent),
// by the same rounds of wave maxima.
template <int PER>
__device__ uint64_t tk_kth_largest(uint32_t (&khi)[PER], uint32_t (&klo)[PER], int k) {
  const int lane = threadIdx.x & 63;
  uint64_t last = 0ull;
  for (int j = 0; j < k; ++j) {
    uint32_t h = khi[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) h = max(h, khi[i]);
    const uint32_t mh = tk_wave_max_u32(h);
    uint64_t mt[PER];
    int nt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mt[i] = __ballot(khi[i] == mh && (khi[i] | klo[i]) != 0u);
      nt += __popcll(mt[i]);
    }
    uint32_t ml;
    {
      uint32_t l = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((mt[i] >> lane) & 1ull) l = max(l, klo[i]);
      ml = (nt > 1) ? tk_wave_max_u32(l) : (uint32_t)0;
      if (nt == 1) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (mt[i]) ml = (uint32_t)__builtin_amdgcn_readlane((int)klo[i], __builtin_ctzll(mt[i]));
      }
    }
    last = ((uint64_t)mh << 32) | ml;
    // remove one expert holding that key (the lowest id; which one does not matter)
    int w = -1, iw = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint64_t m = __ballot(((mt[i] >> lane) & 1ull) && klo[i] == ml);
      if (w < 0 && m != 0ull) { w = __builtin_ctzll(m); iw = i; }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == iw && lane == w) { khi[i] = 0u; klo[i] = 0u; }
  }
  return last;
}

}  // namespace ft
