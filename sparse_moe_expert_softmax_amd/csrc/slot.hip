// Global LRU expert-slot table, resident in HBM and updated on the device.
//
// The pages keep every expert in host memory and use free device memory as
// one least-recently-used expert cache shared by all MoE layers (FreeToken
// explainer page, "how" section; LRU per its glossary: at capacity the entry
// unreferenced for longest goes).  Key = (layer, expert).  One lookup call
// takes the ids one layer selected for a batch:
//   distinct ids ascending; hits stamped with the new tick; if the misses
//   outnumber the slots this call did not stamp -> no change, FT_EPOOL;
//   else the i-th miss (ascending id) takes the i-th slot in (last_use asc,
//   slot asc) order among the unstamped slots, evicting its key.
// One workgroup does the whole call: the state is small
// and the call is a strict sequence of dependent steps.  Limits: S <= 8192
// slots, E <= 4096 experts per layer, <= 1024 ids per call.
#include "common.hpp"
#include "internal.hpp"

namespace ft {

constexpr int SLOT_THREADS = 1024;
constexpr int SLOT_MAX_S = 8192;
constexpr int SLOT_MAX_E = 4096;

struct TableView {
  uint32_t* tick;
  int32_t* status;
  int32_t* key_slot;   // [L*E]
  int32_t* slot_key;   // [S]
  uint32_t* last_use;  // [S]
  int L, E, S;
};

__host__ __device__ inline TableView table_view(void* base) {
  int32_t* h = reinterpret_cast<int32_t*>(base);
  TableView v;
  v.tick = reinterpret_cast<uint32_t*>(h);
  v.status = h + 1;
  v.L = h[2];
  v.E = h[3];
  v.S = h[4];
  int32_t* p = h + 16;  // 64-byte header
  v.key_slot = p;
  v.slot_key = p + (int64_t)v.L * v.E;
  v.last_use = reinterpret_cast<uint32_t*>(v.slot_key + v.S);
  return v;
}

size_t slot_table_bytes(int L, int E, int S) {
  return 64 + sizeof(int32_t) * ((size_t)L * E + S) + sizeof(uint32_t) * (size_t)S;
}

__global__ void slot_table_init_kernel(int32_t* base, int L, int E, int S) {
  const int64_t n_keys = (int64_t)L * E;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid == 0) {
    base[0] = 0;  // tick
    base[1] = FT_OK;
    base[2] = L;
    base[3] = E;
    base[4] = S;
    for (int i = 5; i < 16; ++i) base[i] = 0;
  }
  int32_t* key_slot = base + 16;
  int32_t* slot_key = key_slot + n_keys;
  uint32_t* last_use = reinterpret_cast<uint32_t*>(slot_key + S);
  for (int64_t i = tid; i < n_keys; i += (int64_t)gridDim.x * blockDim.x) key_slot[i] = -1;
  for (int64_t i = tid; i < S; i += (int64_t)gridDim.x * blockDim.x) {
    slot_key[i] = -1;
    last_use[i] = 0u;
  }
}

hipError_t launch_slot_table_init(void* table, int L, int E, int S, hipStream_t st) {
  const int64_t n = (int64_t)L * E + S;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  slot_table_init_kernel<<<blocks, 256, 0, st>>>(reinterpret_cast<int32_t*>(table), L, E, S);
  return hipGetLastError();
}

// 64-bit victim key: (last_use, slot); ~0 = not eligible.
__device__ __forceinline__ uint64_t vkey(uint32_t lu, int s) { return ((uint64_t)lu << 32) | (uint32_t)s; }

__global__ void __launch_bounds__(SLOT_THREADS) slot_lookup_kernel(
    void* table, int layer, const int32_t* __restrict__ ids, int n_pairs, int32_t* __restrict__ slot_ids,
    uint8_t* __restrict__ miss_flags, int32_t* __restrict__ miss_list, int32_t* __restrict__ n_miss_out) {
  __shared__ uint32_t lu_s[SLOT_MAX_S];          // last_use copy
  __shared__ uint8_t present[SLOT_MAX_E];        // per expert of this layer: 1 if selected
  __shared__ uint8_t umiss[SLOT_MAX_E];          // 1 if missed
  __shared__ int32_t uslot[SLOT_MAX_E];          // slot after the call (for selected experts)
  __shared__ int32_t ulist[SLOT_THREADS];        // distinct ids ascending
  __shared__ int32_t n_u, n_hit, n_mis;
  __shared__ uint64_t wave_best[SLOT_THREADS / 64];
  __shared__ int32_t victims[SLOT_THREADS];
  __shared__ int32_t vold[SLOT_THREADS];         // key held by each victim before this call

  TableView tv = table_view(table);
  const int tid = threadIdx.x;
  const int E = tv.E, S = tv.S;
  if (layer >= tv.L || S > SLOT_MAX_S || E > SLOT_MAX_E) {  // bad call: report, touch nothing
    if (tid == 0) { *tv.status = FT_EINVAL; *n_miss_out = -1; }
    for (int p = tid; p < n_pairs; p += SLOT_THREADS) { slot_ids[p] = -1; miss_flags[p] = 0; }
    return;
  }
  const int32_t* ks_layer = tv.key_slot + (int64_t)layer * E;

  for (int e = tid; e < E; e += SLOT_THREADS) { present[e] = 0; umiss[e] = 0; }
  if (tid == 0) { n_u = 0; n_hit = 0; n_mis = 0; }
  __syncthreads();
  for (int p = tid; p < n_pairs; p += SLOT_THREADS) {
    const int e = ids[p];
    if (e >= 0 && e < E) present[e] = 1;
  }
  __syncthreads();
  // current slot of every selected expert (-1: absent), fetched in parallel
  // so that the serial steps below read only LDS
  for (int e = tid; e < E; e += SLOT_THREADS)
    if (present[e]) uslot[e] = ks_layer[e];
  __syncthreads();
  // distinct ids in ascending order: wave 0 compacts 64 experts per step
  // (a ballot of the present flags, each lane's place from the set bits below it)
  if (tid < 64) {
    int n = 0, h = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + tid, ec = e < E ? e : E - 1;  // lanes past E read a valid entry and drop it
      const bool pr = e < E && present[ec];
      const bool hit = pr && uslot[ec] >= 0;
      const uint64_t m = __ballot(pr);
      const uint64_t below = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
      if (pr) ulist[n + __popcll(m & below)] = e;
      n += __popcll(m);
      h += __popcll(__ballot(hit));
    }
    if (tid == 0) {
      n_u = n;
      n_hit = h;
      n_mis = n - h;
    }
  }
  __syncthreads();
  const int nu = n_u, nm = n_mis, nh = n_hit;
  if (nm > S - nh) {  // exhaustion: report, change nothing
    if (tid == 0) { *tv.status = FT_EPOOL; *n_miss_out = -1; }
    for (int p = tid; p < n_pairs; p += SLOT_THREADS) { slot_ids[p] = -1; miss_flags[p] = 0; }
    return;
  }
  const uint32_t tick = *tv.tick + 1u;
  // last_use into LDS, all passes' loads in flight together (S <= 8 passes)
  {
    uint32_t v[SLOT_MAX_S / SLOT_THREADS];
#pragma unroll
    for (int u = 0; u < SLOT_MAX_S / SLOT_THREADS; ++u) {
      const int s = tid + u * SLOT_THREADS;
      v[u] = tv.last_use[s < S ? s : S - 1];
    }
#pragma unroll
    for (int u = 0; u < SLOT_MAX_S / SLOT_THREADS; ++u) {
      const int s = tid + u * SLOT_THREADS;
      if (s < S) lu_s[s] = v[u];
    }
  }
  __syncthreads();
  // stamp hits (in the LDS copy and in the table)
  for (int i = tid; i < nu; i += SLOT_THREADS) {
    const int s = uslot[ulist[i]];
    if (s >= 0) { tv.last_use[s] = tick; lu_s[s] = tick; }
  }
  __syncthreads();
  // pick nm victims, smallest (last_use, slot) among slots with last_use < tick
  const int lane = tid & 63, wv = tid >> 6;
  for (int r = 0; r < nm; ++r) {
    uint64_t best = ~0ull;
    for (int s = tid; s < S; s += SLOT_THREADS) {
      const uint32_t lu = lu_s[s];
      if (lu < tick) {
        const uint64_t kk = vkey(lu, s);
        best = kk < best ? kk : best;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t ob = __shfl_xor(best, o, 64);
      best = ob < best ? ob : best;
    }
    if (lane == 0) wave_best[wv] = best;
    __syncthreads();
    if (tid < 64) {  // the minimum of the wave minima, in wave 0
      uint64_t b = (tid < SLOT_THREADS / 64) ? wave_best[tid] : ~0ull;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        const uint64_t ob = __shfl_xor(b, o, 64);
        b = ob < b ? ob : b;
      }
      if (tid == 0) {
        const int s = (int)(uint32_t)(b & 0xFFFFFFFFu);
        victims[r] = s;
        lu_s[s] = tick;  // now stamped by this call
      }
    }
    __syncthreads();
  }
  // the victims' current keys, fetched in parallel.  A victim was not
  // stamped by this call, so its key is none of this call's ids: the
  // evictions below cannot touch a key that this call reads.
  for (int r = tid; r < nm; r += SLOT_THREADS) vold[r] = tv.slot_key[victims[r]];
  __syncthreads();
  // assign misses (ascending id) to victims in order (thread 0; LDS reads only)
  if (tid == 0) {
    int r = 0;
    for (int i = 0; i < nu; ++i) {
      const int e = ulist[i];
      if (uslot[e] >= 0) continue;
      const int s = victims[r];
      const int old = vold[r];
      if (old >= 0) tv.key_slot[old] = -1;
      tv.slot_key[s] = layer * E + e;
      tv.key_slot[(int64_t)layer * E + e] = s;
      tv.last_use[s] = tick;
      uslot[e] = s;
      umiss[e] = 1;
      miss_list[2 * r] = e;
      miss_list[2 * r + 1] = s;
      ++r;
    }
    *tv.tick = tick;
    *tv.status = FT_OK;
    *n_miss_out = nm;
  }
  __syncthreads();
  for (int p = tid; p < n_pairs; p += SLOT_THREADS) {
    const int e = ids[p];
    const bool ok = e >= 0 && e < E;
    slot_ids[p] = ok ? uslot[e] : -1;
    miss_flags[p] = ok ? umiss[e] : (uint8_t)0;
  }
}

// ------------------------------------------------------ device-side fetch --
// The copy that follows a lookup, driven by the miss list the lookup wrote,
// so no host round trip sits between the lookup and the forward.  Records
// are read straight from pinned host memory (the GPU addresses it directly)
// with 16-byte loads.  Workgroup b copies 64 KB chunk b % cpr of miss
// b / cpr; workgroups past the reported count (or a negative count, from an
// exhausted pool) copy nothing, and entries with an expert or slot out of
// range are skipped.
constexpr int FETCH_THREADS = 256;
constexpr int64_t FETCH_CHUNK = 64 * 1024;

__global__ void __launch_bounds__(FETCH_THREADS) fetch_kernel(uint8_t* __restrict__ pool, int64_t stride,
                                                             int64_t rec_bytes, int E, int S,
                                                             const uint64_t* __restrict__ layer_src,
                                                             const int32_t* __restrict__ miss_list,
                                                             const int32_t* __restrict__ n_miss, int cpr) {
  const int m = blockIdx.x / cpr, c = blockIdx.x % cpr;
  if (m >= *n_miss) return;  // also every workgroup when the count is negative
  const int e = miss_list[2 * m], s = miss_list[2 * m + 1];
  if (e < 0 || e >= E || s < 0 || s >= S) return;
  const uint4* src = reinterpret_cast<const uint4*>(layer_src[e] + c * FETCH_CHUNK);
  uint4* dst = reinterpret_cast<uint4*>(pool + (int64_t)s * stride + c * FETCH_CHUNK);
  const int64_t rem = rec_bytes - c * FETCH_CHUNK;
  const int n16 = (int)((rem < FETCH_CHUNK ? rem : FETCH_CHUNK) / 16);
  // four 16-byte pieces per thread in flight, then their stores
  for (int i0 = threadIdx.x; i0 < n16; i0 += 4 * FETCH_THREADS) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * FETCH_THREADS;
      v[u] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * FETCH_THREADS;
      if (i < n16) dst[i] = v[u];
    }
  }
}

hipError_t launch_fetch(void* pool, int64_t stride, int64_t rec_bytes, int E, int S, const uint64_t* layer_src,
                        const int32_t* miss_list, const int32_t* n_miss, int max_miss, hipStream_t st) {
  const int cpr = (int)((rec_bytes + FETCH_CHUNK - 1) / FETCH_CHUNK);
  fetch_kernel<<<(unsigned)(max_miss * cpr), FETCH_THREADS, 0, st>>>(reinterpret_cast<uint8_t*>(pool), stride,
                                                                      rec_bytes, E, S, layer_src, miss_list, n_miss,
                                                                      cpr);
  return hipGetLastError();
}

// Residency of each id in one layer, without changing the table.
__global__ void slot_probe_kernel(const int32_t* __restrict__ table, int layer, const int32_t* __restrict__ ids,
                                  int n, uint8_t* __restrict__ resident) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n) return;
  const int L = table[2], E = table[3];
  const int e = ids[p];
  const bool ok = layer < L && e >= 0 && e < E;
  const int32_t* key_slot = table + 16;
  resident[p] = (ok && key_slot[(int64_t)layer * E + (ok ? e : 0)] >= 0) ? 1 : 0;
}

hipError_t launch_slot_probe(const void* table, int layer, const int32_t* ids, int n, uint8_t* resident,
                             hipStream_t st) {
  slot_probe_kernel<<<(n + 255) / 256, 256, 0, st>>>(reinterpret_cast<const int32_t*>(table), layer, ids, n,
                                                    resident);
  return hipGetLastError();
}

hipError_t launch_slot_lookup(void* table, int layer, const int32_t* ids, int n_pairs, int32_t* slot_ids,
                              uint8_t* miss_flags, int32_t* miss_list, int32_t* n_miss, hipStream_t st) {
  slot_lookup_kernel<<<1, SLOT_THREADS, 0, st>>>(table, layer, ids, n_pairs, slot_ids, miss_flags, miss_list,
                                                 n_miss);
  return hipGetLastError();
}

int slot_max_slots() { return SLOT_MAX_S; }
int slot_max_experts() { return SLOT_MAX_E; }

}  // namespace ft
