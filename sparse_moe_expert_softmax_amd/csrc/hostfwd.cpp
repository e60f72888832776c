// The host leg of decode co-execution: the experts a step does not copy to
// the device are computed in place on the host's cores from the pinned host
// records, and their partial output is added to the device's partial output
// over the other experts.  The pages split a step's missed experts between a
// transfer over the host link and computation on the host CPU, run both at
// once, and sum the partial outputs, which keeps the MoE output exact
// (FreeToken explainer page, "how" section, decode passage; architecture
// guide, decode passage).
//
// fp32 arithmetic: weights decoded from the packed record (bf16, MXFP4,
// NVFP4-like, fp32) exactly to fp32, activations bf16/fp32 to fp32, fp32
// accumulation in index order, SwiGLU in fp32, combine in rank order.  Work
// is spread over std::threads: first the gate/up rows of every computed
// expert (16-row items), then the down rows, each phase pulled from an
// atomic counter; the combine is sequential.
#include <hip/hip_runtime.h>

#include <immintrin.h>

#include <atomic>
#include <exception>
#include <cmath>
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/ft_moe.h"
#include "common.hpp"
#include "internal.hpp"

namespace {

constexpr int ROWS_PER_ITEM = 16;

float bf16_f32(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// E2M1 magnitudes by code (sign in bit 3)
const float kE2M1[16] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f, -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

float e8m0_f32(uint8_t v) {
  if (v == 255) return NAN;
  return std::ldexp(1.0f, (int)v - 127);
}

float e4m3_f32(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  float mag;
  if (e == 0) mag = std::ldexp((float)m, -9);
  else if (e == 15 && m == 7) mag = NAN;
  else mag = std::ldexp(1.0f + m / 8.0f, e - 7);
  return (c & 0x80) ? -mag : mag;
}

struct Pair {
  int t, j;
};

struct Expert {
  int e;
  const uint8_t* rec;
  std::vector<Pair> pairs;
  std::vector<float> h;  // [n_pairs, I]
  std::vector<float> y;  // [n_pairs, H]
};

// Row `r` of matrix m (0 gate, 1 up: K = H; 2 down: K = I) decoded to fp32.
void decode_row(const uint8_t* rec, const ft::RecordLayout& L, int wd, int m, int r, int K, float* dst) {
  if (wd == FT_F32) {
    std::memcpy(dst, rec + L.code_off[m] + (int64_t)r * K * 4, (size_t)K * 4);
  } else if (wd == FT_BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(rec + L.code_off[m]) + (int64_t)r * K;
    for (int k = 0; k < K; ++k) dst[k] = bf16_f32(p[k]);
  } else {
    const uint8_t* codes = rec + L.code_off[m] + (int64_t)r * K / 2;
    const int blk = (wd == FT_MXFP4) ? 32 : 16;
    const uint8_t* sc = rec + L.scale_off[m] + (int64_t)r * (K / blk);
    float ts = 1.0f;
    if (wd == FT_NVFP4) std::memcpy(&ts, rec + L.tscale_off + 4 * m, 4);
    for (int b = 0; b < K / blk; ++b) {
      const float s = (wd == FT_MXFP4 ? e8m0_f32(sc[b]) : e4m3_f32(sc[b]) * ts);
      const uint8_t* q = codes + b * blk / 2;
      float* d = dst + b * blk;
      for (int i = 0; i < blk / 2; ++i) {
        d[2 * i] = kE2M1[q[i] & 15] * s;
        d[2 * i + 1] = kE2M1[q[i] >> 4] * s;
      }
    }
  }
}

float dot(const float* a, const float* b, int K) {
  // eight partial sums, combined in a fixed order
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int k = 0;
  for (; k + 8 <= K; k += 8)
    for (int u = 0; u < 8; ++u) s[u] += a[k + u] * b[k + u];
  for (; k < K; ++k) s[0] += a[k] * b[k];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// AVX2 dot products of one MXFP4 row with n vectors: decode and multiply in
// one pass, no decoded row stored.  2 * E2M1 is an integer in
// {0, 1, 2, 3, 4, 6, 8, 12} (with sign), so each nibble maps to an int8 by a
// byte shuffle, widened to int32 and converted to fp32 exactly; every block
// sum is scaled by 2^(s - 127) / 2.  Sums per block run in a fixed order.
__attribute__((target("avx2,fma"))) void dot_mxfp4_avx2(const uint8_t* codes, const uint8_t* scales, int K,
                                                        const float* const* vec, int n, float* res) {
  const __m128i lut = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
  const __m128i lo4 = _mm_set1_epi8(0x0F);
  __m256 acc[8];
  for (int p = 0; p < n; ++p) acc[p] = _mm256_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    const __m128i q = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b));
    const __m128i lo = _mm_and_si128(q, lo4), hi = _mm_and_si128(_mm_srli_epi16(q, 4), lo4);
    const __m128i v0 = _mm_shuffle_epi8(lut, _mm_unpacklo_epi8(lo, hi));  // elements 0..15
    const __m128i v1 = _mm_shuffle_epi8(lut, _mm_unpackhi_epi8(lo, hi));  // elements 16..31
    const __m256 w0 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v0));
    const __m256 w1 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v0, 8)));
    const __m256 w2 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v1));
    const __m256 w3 = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v1, 8)));
    const uint8_t sv = scales[b];
    const float s = (sv == 255) ? NAN : std::ldexp(0.5f, (int)sv - 127);
    const __m256 vs = _mm256_set1_ps(s);
    for (int p = 0; p < n; ++p) {
      const float* x = vec[p] + 32 * b;
      __m256 t = _mm256_mul_ps(w0, _mm256_loadu_ps(x));
      t = _mm256_fmadd_ps(w1, _mm256_loadu_ps(x + 8), t);
      t = _mm256_fmadd_ps(w2, _mm256_loadu_ps(x + 16), t);
      t = _mm256_fmadd_ps(w3, _mm256_loadu_ps(x + 24), t);
      acc[p] = _mm256_fmadd_ps(vs, t, acc[p]);
    }
  }
  for (int p = 0; p < n; ++p) {
    alignas(32) float f[8];
    _mm256_store_ps(f, acc[p]);
    res[p] = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
  }
}

bool have_avx2() {
  static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
  return ok;
}

}  // namespace

extern "C" {

static int forward_host(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const int32_t* topk_ids,
                        const float* topk_gates, const void* const* records, const uint32_t* expert_mask,
                        float* out, int32_t n_threads, bool no_simd) {
  if (!desc) return ft::report(FT_EINVAL, "desc is NULL");
  const int H = desc->hidden, I = desc->inter, E = desc->n_experts, k = desc->top_k, T = n_tokens;
  if (H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E || H % 32 || I % 32)
    return ft::report(FT_EINVAL, "bad sizes in desc");
  if (desc->act_dtype != FT_F32 && desc->act_dtype != FT_BF16) return ft::report(FT_EUNSUPPORTED, "act_dtype");
  if (desc->w_dtype < FT_F32 || desc->w_dtype > FT_NVFP4) return ft::report(FT_EUNSUPPORTED, "w_dtype");
  if (T < 0) return ft::report(FT_EINVAL, "n_tokens < 0");
  if (T == 0) return FT_OK;
  if (!x || !topk_ids || !topk_gates || !records || !out) return ft::report(FT_EINVAL, "NULL argument");
  const int wd = desc->w_dtype;
  const ft::RecordLayout L = ft::record_layout(H, I, wd);

  // activations to fp32
  std::vector<float> xf((size_t)T * H);
  if (desc->act_dtype == FT_F32) std::memcpy(xf.data(), x, xf.size() * 4);
  else
    for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_f32(reinterpret_cast<const uint16_t*>(x)[i]);

  // the computed experts and their pairs, in order of first appearance
  std::vector<int> slot_of(E, -1);
  std::vector<Expert> ex;
  std::vector<int> pair_expert((size_t)T * k, -1), pair_index((size_t)T * k, -1);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int e = topk_ids[t * k + j];
      if (e < 0 || e >= E) continue;
      if (expert_mask && !((expert_mask[e >> 5] >> (e & 31)) & 1u)) continue;
      if (slot_of[e] < 0) {
        if (!records[e]) return ft::report(FT_EINVAL, "records[%d] is NULL but expert %d is computed", e, e);
        slot_of[e] = (int)ex.size();
        ex.push_back(Expert{e, reinterpret_cast<const uint8_t*>(records[e]), {}, {}, {}});
      }
      Expert& X = ex[slot_of[e]];
      pair_expert[t * k + j] = slot_of[e];
      pair_index[t * k + j] = (int)X.pairs.size();
      X.pairs.push_back(Pair{t, j});
    }
  for (Expert& X : ex) {
    X.h.assign(X.pairs.size() * (size_t)I, 0.f);
    X.y.assign(X.pairs.size() * (size_t)H, 0.f);
  }

  // work items: phase A (gate/up rows), then phase B (down rows)
  const int items_a_per = (I + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
  const int items_b_per = (H + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
  const int n_a = (int)ex.size() * items_a_per, n_b = (int)ex.size() * items_b_per;
  std::atomic<int> next_a{0}, next_b{0}, done_a{0};
  int nt = n_threads > 0 ? n_threads : (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > 256) nt = 256;

  const bool fast = wd == FT_MXFP4 && have_avx2() && !no_simd;
  auto worker = [&]() {
    std::vector<float> wg(H > I ? H : I), wu(H > I ? H : I);
    for (;;) {
      const int it = next_a.fetch_add(1);
      if (it >= n_a) break;
      Expert& X = ex[it / items_a_per];
      const int r0 = (it % items_a_per) * ROWS_PER_ITEM;
      for (int r = r0; r < r0 + ROWS_PER_ITEM && r < I; ++r) {
        if (fast) {  // MXFP4 rows, pairs in groups of up to 8
          for (size_t p0 = 0; p0 < X.pairs.size(); p0 += 8) {
            const int n = (int)std::min<size_t>(8, X.pairs.size() - p0);
            const float* v[8];
            float a[8], b[8];
            for (int i = 0; i < n; ++i) v[i] = xf.data() + (size_t)X.pairs[p0 + i].t * H;
            dot_mxfp4_avx2(X.rec + L.code_off[0] + (int64_t)r * H / 2, X.rec + L.scale_off[0] + (int64_t)r * (H / 32),
                           H, v, n, a);
            dot_mxfp4_avx2(X.rec + L.code_off[1] + (int64_t)r * H / 2, X.rec + L.scale_off[1] + (int64_t)r * (H / 32),
                           H, v, n, b);
            for (int i = 0; i < n; ++i) X.h[(p0 + i) * I + r] = a[i] / (1.0f + std::exp(-a[i])) * b[i];
          }
          continue;
        }
        decode_row(X.rec, L, wd, 0, r, H, wg.data());
        decode_row(X.rec, L, wd, 1, r, H, wu.data());
        for (size_t p = 0; p < X.pairs.size(); ++p) {
          const float* xr = xf.data() + (size_t)X.pairs[p].t * H;
          const float a = dot(wg.data(), xr, H), b = dot(wu.data(), xr, H);
          X.h[p * I + r] = a / (1.0f + std::exp(-a)) * b;
        }
      }
      done_a.fetch_add(1, std::memory_order_release);
    }
    // phase B needs every h: wait until all phase-A items are finished
    while (done_a.load(std::memory_order_acquire) < n_a) std::this_thread::yield();
    for (;;) {
      const int it = next_b.fetch_add(1);
      if (it >= n_b) break;
      Expert& X = ex[it / items_b_per];
      const int r0 = (it % items_b_per) * ROWS_PER_ITEM;
      for (int r = r0; r < r0 + ROWS_PER_ITEM && r < H; ++r) {
        if (fast) {
          for (size_t p0 = 0; p0 < X.pairs.size(); p0 += 8) {
            const int n = (int)std::min<size_t>(8, X.pairs.size() - p0);
            const float* v[8];
            float y[8];
            for (int i = 0; i < n; ++i) v[i] = X.h.data() + (p0 + i) * I;
            dot_mxfp4_avx2(X.rec + L.code_off[2] + (int64_t)r * I / 2, X.rec + L.scale_off[2] + (int64_t)r * (I / 32),
                           I, v, n, y);
            for (int i = 0; i < n; ++i) X.y[(p0 + i) * H + r] = y[i];
          }
          continue;
        }
        decode_row(X.rec, L, wd, 2, r, I, wg.data());
        for (size_t p = 0; p < X.pairs.size(); ++p) X.y[p * H + r] = dot(wg.data(), X.h.data() + p * I, I);
      }
    }
  };
  std::vector<std::thread> pool;
  try {
    pool.reserve(nt - 1);
    for (int i = 1; i < nt; ++i) pool.emplace_back(worker);
  } catch (const std::exception&) {
    // fewer threads than asked: the work counters still hand out every item
  }
  worker();
  for (std::thread& th : pool) th.join();

  // combine in rank order
  for (int t = 0; t < T; ++t) {
    float* o = out + (size_t)t * H;
    for (int c = 0; c < H; ++c) o[c] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int xi = pair_expert[t * k + j];
      if (xi < 0) continue;
      const float g = topk_gates[t * k + j];
      const float* y = ex[xi].y.data() + (size_t)pair_index[t * k + j] * H;
      for (int c = 0; c < H; ++c) o[c] += g * y[c];
    }
  }
  return FT_OK;
}

int ft_moe_forward_host(const ft_moe_desc* desc, const void* x, int32_t n_tokens, const int32_t* topk_ids,
                        const float* topk_gates, const void* const* records, const uint32_t* expert_mask,
                        float* out, int32_t n_threads) {
  try {
    const bool no_simd = n_threads < 0;  // negative: the portable loops (tests compare the two)
    return forward_host(desc, x, n_tokens, topk_ids, topk_gates, records, expert_mask, out,
                        n_threads < 0 ? -n_threads : n_threads, no_simd);
  } catch (const std::exception& ex) {
    return ft::report(FT_EINVAL, "host forward: %s", ex.what());
  }
}

}  // extern "C"
