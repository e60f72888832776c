// Host-side checks of the library's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only and run on a machine
// without a GPU: workspace planning, every argument refusal that returns
// before a launch, and the host forward (pure CPU).  Any memory error or
// undefined behaviour aborts the run; a failed expectation exits with 1.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../include/ft_moe.h"

static int g_fail = 0;

#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n",     \
              __FILE__, __LINE__, #cond, ft_last_error());                    \
      g_fail = 1;                                                             \
    }                                                                         \
  } while (0)

static ft_moe_desc make_desc(int H, int I, int E, int k, int wd, int act = FT_BF16) {
  ft_moe_desc d;
  memset(&d, 0, sizeof d);
  d.hidden = H;
  d.inter = I;
  d.n_experts = E;
  d.top_k = k;
  d.act_dtype = act;
  d.w_dtype = wd;
  d.router_dtype = FT_BF16;
  d.renormalize = 1;
  size_t rb = ft_record_bytes(H, I, wd);
  d.expert_stride = (int64_t)((rb + 4095) / 4096 * 4096);
  return d;
}

// xorshift64*: the driver's own deterministic bytes
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return (uint32_t)((g_rng * 2685821657736338717ull) >> 32);
}
static uint16_t bf16_of(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  return (uint16_t)(b >> 16);
}
static float small_normalish() { return ((int)(rnd() % 2001) - 1000) * 2e-5f; }

// A record with finite values for each format: bf16 values of small
// magnitude; fp4 codes of any value with E8M0 scales near 2^0 or E4M3 scales
// of moderate size, tensor scales 1.
static std::vector<uint8_t> make_record(int H, int I, int wd) {
  const size_t n = ft_record_bytes(H, I, wd);
  std::vector<uint8_t> r(n);
  const size_t nel = (size_t)3 * H * I;
  if (wd == FT_BF16) {
    for (size_t i = 0; i < nel; ++i) {
      const uint16_t b = bf16_of(small_normalish());
      memcpy(&r[2 * i], &b, 2);
    }
    return r;
  }
  const size_t codes = nel / 2, blk = (wd == FT_MXFP4) ? 32 : 16, nsc = nel / blk;
  for (size_t i = 0; i < codes; ++i) r[i] = (uint8_t)rnd();
  for (size_t i = 0; i < nsc; ++i) r[codes + i] = (wd == FT_MXFP4) ? (uint8_t)(120 + rnd() % 8) : (uint8_t)(0x20 + rnd() % 0x30);
  if (wd == FT_NVFP4) {
    const float one = 1.0f;
    for (int m = 0; m < 3; ++m) memcpy(&r[codes + nsc + 4 * m], &one, 4);
  }
  return r;
}

static void check_planning() {
  const int wds[4] = {FT_F32, FT_BF16, FT_MXFP4, FT_NVFP4};
  const int Ts[8] = {0, 1, 4, 16, 17, 255, 256, 8192};
  for (int wd : wds)
    for (int T : Ts)
      for (int terms = 0; terms <= 2; ++terms) {
        ft_moe_desc d = make_desc(2048, 768, 128, 8, wd, wd == FT_F32 ? FT_F32 : FT_BF16);
        d.act_terms = terms;
        const size_t f = ft_moe_workspace_bytes(&d, T), r = ft_route_workspace_bytes(&d, T);
        const size_t rf = ft_moe_route_forward_workspace_bytes(&d, T);
        EXPECT(f % 256 == 0);
        EXPECT(rf >= f + r);
      }
  ft_moe_desc big = make_desc(4096, 2048, 256, 6, FT_MXFP4);
  EXPECT(ft_moe_workspace_bytes(&big, 16384) > ft_moe_workspace_bytes(&big, 8192));
  EXPECT(ft_record_bytes(0, 768, FT_BF16) == 0);
  EXPECT(ft_record_bytes(2048, 768, 7) == 0);
  EXPECT(ft_record_bytes(2048, 768, FT_BF16) == (size_t)3 * 2048 * 768 * 2);
  EXPECT(ft_moe_workspace_bytes(nullptr, 4) == 0);
  EXPECT(ft_slot_table_bytes(0, 1, 1) == 0);
  EXPECT(ft_slot_table_bytes(43, 256, 2752) > 0);
}

static void check_refusals() {
  ft_moe_desc d = make_desc(256, 256, 8, 2, FT_BF16);
  alignas(256) static uint8_t buf[1 << 16];
  int32_t ids[8] = {0};
  float gates[8] = {0};
  float out[1024];
  // descriptors
  EXPECT(ft_moe_forward(nullptr, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  ft_moe_desc bad = d;
  bad.top_k = 9;
  EXPECT(ft_moe_forward(&bad, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  bad = d;
  bad.w_dtype = 9;
  EXPECT(ft_moe_forward(&bad, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) ==
         FT_EUNSUPPORTED);
  bad = d;
  bad.act_terms = 3;
  EXPECT(ft_moe_forward(&bad, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  bad = d;
  bad.hidden = 250;
  EXPECT(ft_moe_forward(&bad, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  bad = d;
  bad.expert_stride = 100;
  EXPECT(ft_moe_forward(&bad, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  // arguments and workspace
  EXPECT(ft_moe_forward(&d, buf, -1, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_forward(&d, buf, 0, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_OK);
  EXPECT(ft_moe_forward(&d, nullptr, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_forward(&d, buf + 1, 4, ids, gates, nullptr, buf, nullptr, out, buf, sizeof buf, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_forward(&d, buf, 4, ids, gates, nullptr, buf, nullptr, out, buf, 16, nullptr) == FT_EWORKSPACE);
  EXPECT(strlen(ft_last_error()) > 0);
  EXPECT(ft_moe_route(&d, buf, 4, buf, nullptr, ids, gates, nullptr, buf, 8, nullptr) == FT_EWORKSPACE);
  EXPECT(ft_moe_route(&d, buf, 4, nullptr, nullptr, ids, gates, nullptr, buf, sizeof buf, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_route(&d, buf, 0, buf, nullptr, ids, gates, nullptr, buf, sizeof buf, nullptr) == FT_OK);
  EXPECT(ft_moe_route_forward(&d, buf, 4, buf, nullptr, ids, gates, buf, nullptr, out, buf, 8, nullptr) ==
         FT_EWORKSPACE);
  // slot table, lookup, probe
  EXPECT(ft_slot_table_init(nullptr, 1, 8, 4, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_table_init(buf, 1, 8, 1 << 30, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_table_init(buf, 1, 1 << 20, 4, nullptr) == FT_EINVAL);
  int32_t slots[8], miss[32], nmiss[1];
  uint8_t flags[8];
  EXPECT(ft_slot_lookup(buf, 0, ids, 0, slots, flags, miss, nmiss, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_lookup(buf, 0, ids, 2000, slots, flags, miss, nmiss, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_lookup(buf, -1, ids, 4, slots, flags, miss, nmiss, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_lookup(nullptr, 0, ids, 4, slots, flags, miss, nmiss, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_probe(buf, 0, ids, -1, flags, nullptr) == FT_EINVAL);
  EXPECT(ft_slot_probe(buf, 0, ids, 0, flags, nullptr) == FT_OK);
  // uploads and fetches
  const void* src[2] = {buf, nullptr};
  int32_t up_slots[2] = {0, -1};
  EXPECT(ft_expert_upload(buf, 4096, 1024, up_slots, src, -1, nullptr, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_upload(buf, 1024, 4096, up_slots, src, 1, nullptr, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_upload(buf, 4096, 1024, up_slots + 1, src, 1, nullptr, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_upload(buf, 4096, 1024, up_slots, src + 1, 1, nullptr, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_upload(buf, 4096, 1024, up_slots, src, 0, nullptr, nullptr) == FT_OK);
  uint64_t lsrc[8] = {0};
  EXPECT(ft_expert_fetch(buf, 4096, 1000, 8, 4, lsrc, miss, nmiss, 4, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_fetch(buf, 1024, 4096, 8, 4, lsrc, miss, nmiss, 4, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_fetch(buf, 4096, 1024, 0, 4, lsrc, miss, nmiss, 4, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_fetch(buf, 4096, 1024, 8, 4, lsrc, miss, nmiss, -1, nullptr) == FT_EINVAL);
  EXPECT(ft_expert_fetch(buf, 4096, 1024, 8, 4, lsrc, miss, nmiss, 0, nullptr) == FT_OK);
  // prefill pipeline
  ft_prefill_pipeline p;
  memset(&p, 0, sizeof p);
  EXPECT(ft_prefill_pipeline_start(nullptr, src) == FT_EINVAL);
  EXPECT(ft_prefill_pipeline_start(&p, src) == FT_EINVAL);
  EXPECT(ft_prefill_pipeline_layer(&p, nullptr, &d, buf, 4, buf, ids, gates, out, buf, sizeof buf) == FT_EINVAL);
  // partial sums
  EXPECT(ft_moe_add_partial(out, out, -1, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_add_partial(nullptr, out, 4, nullptr) == FT_EINVAL);
  EXPECT(ft_moe_add_partial(out, out, 0, nullptr) == FT_OK);
  // the allocation-free entry point refuses sizes beyond its scratch
  ft_moe_desc huge = make_desc(4096, 2048, 256, 8, FT_MXFP4);
  EXPECT(ft_moe_route_forward_noalloc(&huge, buf, 16384, buf, nullptr, ids, gates, buf, nullptr, out, nullptr) ==
         FT_EWORKSPACE);
  EXPECT(ft_moe_route_forward_noalloc(nullptr, buf, 4, buf, nullptr, ids, gates, buf, nullptr, out, nullptr) ==
         FT_EINVAL);
}

// The host forward on a small layer of each format: thread counts agree bit
// for bit; a mask and its complement add up to the unmasked output; repeated
// ids; a needed NULL record is refused.
static void check_host_forward(int wd) {
  const int H = 64, I = 96, E = 6, k = 3, T = 5;
  ft_moe_desc d = make_desc(H, I, E, k, wd);
  std::vector<std::vector<uint8_t>> recs;
  std::vector<const void*> ptrs;
  for (int e = 0; e < E; ++e) recs.push_back(make_record(H, I, wd));
  for (int e = 0; e < E; ++e) ptrs.push_back(recs[e].data());
  std::vector<uint16_t> x(T * H);
  for (auto& v : x) v = bf16_of(small_normalish() * 50);
  std::vector<int32_t> ids(T * k);
  std::vector<float> gates(T * k);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      ids[t * k + j] = (t == 2 && j == 2) ? ids[t * k] : (int32_t)(rnd() % E);  // token 2 repeats an expert
      gates[t * k + j] = 1.0f / k;
    }
  std::vector<float> ref(T * H), got(T * H), a(T * H), b(T * H);
  EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), ptrs.data(), nullptr, ref.data(), 1) == FT_OK);
  for (float v : ref) EXPECT(isfinite(v));
  // thread counts on one kind of loop agree bit for bit; the portable loops
  // (negative counts) and the AVX2 rows (MXFP4 on an AVX2 CPU) sum in
  // another order, so across the two only to fp32 rounding
  std::vector<float> port(T * H);
  EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), ptrs.data(), nullptr, port.data(), -1) ==
         FT_OK);
  const int threads[4] = {3, 0, -2, -3};
  for (int nt : threads) {
    EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), ptrs.data(), nullptr, got.data(), nt) ==
           FT_OK);
    EXPECT(memcmp(got.data(), nt > 0 || nt == 0 ? ref.data() : port.data(), sizeof(float) * T * H) == 0);
  }
  {
    float pmax = 0.f, pd = 0.f;
    for (int i = 0; i < T * H; ++i) {
      pmax = fmaxf(pmax, fabsf(ref[i]));
      pd = fmaxf(pd, fabsf(port[i] - ref[i]));
    }
    EXPECT(pd <= 1e-5f * (pmax > 0 ? pmax : 1.f));
  }
  const uint32_t m = 0b010110u, c = (~m) & ((1u << E) - 1);
  EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), ptrs.data(), &m, a.data(), 2) == FT_OK);
  EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), ptrs.data(), &c, b.data(), 2) == FT_OK);
  float amax = 0.f, dmax = 0.f;
  for (int i = 0; i < T * H; ++i) {
    amax = fmaxf(amax, fabsf(ref[i]));
    dmax = fmaxf(dmax, fabsf(a[i] + b[i] - ref[i]));
  }
  EXPECT(dmax <= 1e-5f * (amax > 0 ? amax : 1.f));
  // a record the mask does not keep may be NULL; one it keeps may not
  std::vector<const void*> holes = ptrs;
  int absent = -1;
  for (int e = 0; e < E && absent < 0; ++e) {
    bool used = false;
    for (int i = 0; i < T * k; ++i) used |= ids[i] == e;
    if (!used) absent = e;
  }
  if (absent >= 0) {
    holes[absent] = nullptr;
    EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), holes.data(), nullptr, got.data(), 2) ==
           FT_OK);
    EXPECT(memcmp(got.data(), ref.data(), sizeof(float) * T * H) == 0);
  }
  holes = ptrs;
  holes[ids[0]] = nullptr;
  EXPECT(ft_moe_forward_host(&d, x.data(), T, ids.data(), gates.data(), holes.data(), nullptr, got.data(), 2) ==
         FT_EINVAL);
  EXPECT(ft_moe_forward_host(&d, x.data(), -1, ids.data(), gates.data(), ptrs.data(), nullptr, got.data(), 2) ==
         FT_EINVAL);
}

int main() {
  check_planning();
  check_refusals();
  check_host_forward(FT_BF16);
  check_host_forward(FT_MXFP4);
  check_host_forward(FT_NVFP4);
  printf(g_fail ? "host checks FAILED\n" : "host checks passed\n");
  return g_fail;
}
