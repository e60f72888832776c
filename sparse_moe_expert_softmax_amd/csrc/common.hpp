// Shared device helpers for the gfx950 MoE kernels: element decoders for the
// packed expert record, wave64 reductions, and the record layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ft_moe.h"

#define FT_WAVE 64

namespace ft {

// ---------------------------------------------------------------- layout ---
// Record of one expert: gate [I,H], up [I,H], down [H,I] (reduction dim
// contiguous).  F32/BF16: elements back to back.  MXFP4/NVFP4: the three
// code blocks (2 per byte, low nibble first), then three scale blocks
// (E8M0 per 32 / E4M3 per 16 along K), then (NVFP4) 3 fp32 tensor scales.
struct RecordLayout {
  int64_t code_off[3];   // byte offset of each matrix's elements / codes
  int64_t scale_off[3];  // byte offset of each matrix's block scales (fp4 formats)
  int64_t tscale_off;    // NVFP4: byte offset of the 3 fp32 tensor scales
  int64_t bytes;         // total bytes used
};

__host__ __device__ inline RecordLayout record_layout(int H, int I, int w_dtype) {
  RecordLayout L{};
  const int64_t n1 = (int64_t)I * H;  // every matrix has H*I elements
  if (w_dtype == FT_F32 || w_dtype == FT_BF16) {
    const int64_t esz = (w_dtype == FT_F32) ? 4 : 2;
    for (int m = 0; m < 3; ++m) { L.code_off[m] = m * n1 * esz; L.scale_off[m] = 0; }
    L.tscale_off = 0;
    L.bytes = 3 * n1 * esz;
  } else {
    const int64_t blk = (w_dtype == FT_MXFP4) ? 32 : 16;
    for (int m = 0; m < 3; ++m) L.code_off[m] = m * (n1 / 2);
    const int64_t s0 = 3 * (n1 / 2);
    for (int m = 0; m < 3; ++m) L.scale_off[m] = s0 + m * (n1 / blk);
    L.tscale_off = s0 + 3 * (n1 / blk);
    L.bytes = L.tscale_off + ((w_dtype == FT_NVFP4) ? 12 : 0);
  }
  return L;
}

// --------------------------------------------------------------- decoders ---
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// E2M1 nibble -> fp32 (OCP MX FP4: sign, 2-bit exponent with bias 1, 1 mantissa bit;
// exponent 0 is subnormal 0.5*m).  Built from the bit fields, no table.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t mag = c & 7u;
  uint32_t bits;
  if (mag >= 2u) bits = (mag << 22) + 0x3F000000u;   // (1 + m/2) * 2^(e-1)
  else bits = mag ? 0x3F000000u : 0u;                // 0.5 or 0
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// E8M0 -> fp32: 2^(v-127); 0 -> 2^-127 (fp32 subnormal); 255 -> NaN.
// Selects on values, not branches: per-lane branches here compile to
// exec-mask blocks of a dozen scalar instructions at every use.
__device__ __forceinline__ float e8m0_to_f32(uint32_t v) {
  uint32_t b = v << 23;
  b = (v == 0u) ? 0x00400000u : b;
  b = (v == 255u) ? 0x7FC00000u : b;
  return __uint_as_float(b);
}

// E4M3 (OCP FN: bias 7, no inf, S.1111.111 = NaN) -> fp32, by selects.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t sub = __float_as_uint((float)m * 0.001953125f);   // e == 0: m/8 * 2^-6
  const uint32_t nrm = ((e + 120u) << 23) | (m << 20);             // (1+m/8) * 2^(e-7)
  const uint32_t keep = 0u - (uint32_t)(e != 0u);                  // a mask blend, not a branch
  uint32_t mag = (nrm & keep) | (sub & ~keep);
  mag = (e == 15u && m == 7u) ? 0x7FC00000u : mag;
  return __uint_as_float(mag | ((c & 0x80u) << 24));
}

// ------------------------------------------------------------ reductions ---
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, FT_WAVE);
  return v;
}

}  // namespace ft
