// Token permutation by expert: count the (token, rank) pairs each expert
// receives, exclusive prefix sums over experts (LDS scans), then a stable
// scatter so that pairs are grouped by expert and kept in pair order
// (t*k + j) inside each group.  Pairs whose expert is masked out are left
// out entirely (their expert's weights are never read).  The grouping is the
// usual way a MoE kernel aggregates the tokens of each active expert; the
// pages describe one kernel that aggregates all active experts (FreeToken
// blog page, architecture section) without giving its layout.
#include "common.hpp"
#include "internal.hpp"

namespace ft {

__device__ __forceinline__ bool in_mask(const uint32_t* mask, int e) {
  return mask == nullptr || ((mask[e >> 5] >> (e & 31)) & 1u);
}

// Per-block expert histogram of masked-in pairs.
__global__ void __launch_bounds__(1024) perm_count_kernel(const int32_t* __restrict__ ids,
                                                          const uint32_t* __restrict__ mask, int P, int E,
                                                          int32_t* __restrict__ block_hist) {
  __shared__ int32_t hist[1024];
  for (int e = threadIdx.x; e < E; e += 1024) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * PERM_CHUNK;
  for (int i = threadIdx.x; i < PERM_CHUNK; i += 1024) {
    const int p = base + i;
    if (p < P) {
      const int e = ids[p];
      if (e >= 0 && e < E && in_mask(mask, e)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) block_hist[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of v over the block's 1024 threads (one value each).
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) { const int c = tmp[i]; tmp[i] = run; run += c; }
    *total = run;
  }
  __syncthreads();
  const int r = tmp[w] + incl - v;
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024) perm_scatter_kernel(
    const int32_t* __restrict__ ids, const uint32_t* __restrict__ mask, int P, int E, int nb,
    const int32_t* __restrict__ block_hist, int32_t* __restrict__ offsets, int32_t* __restrict__ active,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos_of_pair) {
  __shared__ int32_t base_e[1024];        // where this block's pairs of expert e start
  __shared__ uint16_t wcnt[16][1024];     // per-wave counts, then per-wave prefixes
  __shared__ int32_t tmp[16];
  __shared__ int32_t tot;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  // per-expert totals and this block's prefix over earlier blocks (E <= 1024)
  int total = 0, before = 0;
  if (tid < E) {
    // sixteen rows in flight at a time (clamped rows, dropped after the load)
    for (int bb0 = 0; bb0 < nb; bb0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = block_hist[(int64_t)min(bb0 + u, nb - 1) * E + tid];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int bb = bb0 + u;
        const int cv = bb < nb ? c[u] : 0;
        total += cv;
        before += bb < b ? cv : 0;
      }
    }
  }
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
  const int eoff = block_exclusive_scan(tid < E ? total : 0, tmp, &tot);
  const int aoff = block_exclusive_scan((tid < E && total > 0) ? 1 : 0, tmp, &tot);
  if (tid < E) {
    base_e[tid] = eoff + before;
    if (b == 0) {
      offsets[tid] = eoff;
      if (total > 0) active[aoff] = tid;
    }
  }
  if (b == 0 && tid == E - 1) offsets[E] = eoff + total;  // pairs kept
  if (b == 0 && tid == 0) offsets[E + 1] = tot;             // number of active experts
  // one pair per thread: rank among earlier lanes of the wave with the same expert
  const int p = b * PERM_CHUNK + tid;
  int e = -1;
  bool valid = false;
  if (p < P) {
    e = ids[p];
    valid = e >= 0 && e < E && in_mask(mask, e);
    if (!valid) pos_of_pair[p] = -1;
  }
  uint64_t todo = __ballot(valid);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int el = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == el);
    if (valid && e == el) rank = __popcll(m & below);
    if (lane == leader) wcnt[wv][el] = (uint16_t)__popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  // exclusive prefix of the per-wave counts, wave order, for every expert
  if (tid < E) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = (uint16_t)run;
      run += c;
    }
  }
  __syncthreads();
  if (valid) {
    const int pos = base_e[e] + wcnt[wv][e] + rank;
    perm[pos] = p;
    pos_of_pair[p] = pos;
  }
}

hipError_t launch_permute(const FwdPlan& pl, const int32_t* ids, const uint32_t* mask, char* ws, hipStream_t st) {
  int32_t* hist = reinterpret_cast<int32_t*>(ws + pl.off_hist);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + pl.off_offsets);
  int32_t* active = reinterpret_cast<int32_t*>(ws + pl.off_active);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + pl.off_perm);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + pl.off_pos);
  perm_count_kernel<<<pl.nb, 1024, 0, st>>>(ids, mask, pl.P, pl.E, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  perm_scatter_kernel<<<pl.nb, 1024, 0, st>>>(ids, mask, pl.P, pl.E, pl.nb, hist, offsets, active, perm, pos);
  return hipGetLastError();
}

}  // namespace ft
