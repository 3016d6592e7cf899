// Shared device helpers for the latent-MoE kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 lm_bf16x8;
typedef __attribute__((ext_vector_type(16))) float lm_f32x16;
typedef __attribute__((ext_vector_type(4))) float lm_f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t lm_u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t lm_u32x2;

#define LM_DEV __device__ __forceinline__

constexpr int kWave = 64;

LM_DEV float lm_bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even to bfloat16 (quiet NaN stays NaN).
LM_DEV uint16_t lm_f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// silu(g) = g * sigma(g), with the hardware reciprocal (about one ulp) in
// place of an IEEE division: the result is rounded to BF16 or an MX code.
LM_DEV float lm_silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Deterministic wave-wide sums (fixed butterfly order).
LM_DEV float lm_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Sum over the 32 lanes sharing bit 5 of the lane id (lanes 0-31 / 32-63).
LM_DEV float lm_half_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
