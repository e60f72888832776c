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

// Top-k of one token's E <= 64*PER scores by one wave, without a serial
// chain of cross-lane shuffles: a radix select over the orderable 64-bit
// keys (one ballot per held value and bit, most significant bit first,
// stopping as soon as the candidate set is exactly the number still needed),
// then the k winners are ranked by (score desc, id asc) through LDS.
// Equal scores at the boundary go to the lowest ids.  Scratch: 32 entries
// per wave in LDS.
struct TopkScratch {
  uint64_t key[32];
  double l[32];
  double ex[32];
  int id[32];
};

template <int PER>
__device__ void topk_one_token(const double* __restrict__ lt, const float* __restrict__ bias_t, int E, int k,
                               int renormalize, int32_t* __restrict__ ids_t, float* __restrict__ gates_t,
                               TopkScratch* sc) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PER];
  double lv[PER];
  bool cand[PER], sel[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const bool ok = e < E;
    lv[i] = ok ? lt[e] : 0.0;
    double s = lv[i];
    if (ok && bias_t) s += (double)bias_t[e];
    key[i] = ok ? dkey(s) : 0ull;
    cand[i] = ok;
    sel[i] = false;
  }
  int need = k;
  for (int b = 63; b >= 0 && need > 0; --b) {
    int n_cand = 0, c1 = 0;
    uint64_t m1[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool one = cand[i] && ((key[i] >> b) & 1ull);
      m1[i] = __ballot(one);
      c1 += __popcll(m1[i]);
      n_cand += __popcll(__ballot(cand[i]));
    }
    if (n_cand == need) break;  // every candidate is selected
    const bool take_ones = c1 >= need;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool one = (m1[i] >> lane) & 1ull;
      if (take_ones) {
        cand[i] = cand[i] && one;
      } else {
        if (cand[i] && one) sel[i] = true;  // strictly above the threshold
        cand[i] = cand[i] && !one;
      }
    }
    if (!take_ones) need -= c1;
  }
  // remaining candidates share the threshold key (or fit exactly): take the
  // `need` lowest ids, i.e. first in (i, lane) order
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint64_t m = __ballot(cand[i]);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int before = __popcll(m & below);
    if (cand[i] && before < need) sel[i] = true;
    need -= __popcll(m);
    if (need < 0) need = 0;
  }
  // compact the winners into LDS in (i, lane) = ascending id order
  int base = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint64_t m = __ballot(sel[i]);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (sel[i]) {
      const int pos = base + __popcll(m & below);
      sc->key[pos] = key[i];
      sc->l[pos] = lv[i];
      sc->id[pos] = lane + 64 * i;
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const bool mine = lane < k;
  uint64_t kk = 0ull;
  int id = 0;
  double l = 0.0;
  int rank = 0;
  if (mine) {
    kk = sc->key[lane];
    id = sc->id[lane];
    l = sc->l[lane];
    for (int m = 0; m < k; ++m) {
      const uint64_t km = sc->key[m];
      rank += (km > kk || (km == kk && sc->id[m] < id)) ? 1 : 0;
    }
  }
  double g = 0.0;
  if (renormalize) {
    double mx = -__builtin_inf();
    for (int m = 0; m < k; ++m) mx = fmax(mx, sc->l[m]);
    const double ex = mine ? exp(l - mx) : 0.0;
    if (mine) sc->ex[lane] = ex;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    double den = 0.0;
    for (int m = 0; m < k; ++m) den += sc->ex[m];
    g = ex / den;
  } else {
    double mx = -__builtin_inf();
    for (int e = lane; e < E; e += 64) mx = fmax(mx, lt[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp(lt[e] - mx);
    const double den = wave_sum(part);
    g = mine ? exp(l - mx) / den : 0.0;
  }
  if (mine) {
    ids_t[rank] = id;
    gates_t[rank] = (float)g;
  }
}

}  // namespace ft
