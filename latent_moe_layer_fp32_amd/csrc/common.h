// Shared device helpers for the latent-MoE kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 lm_bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 lm_f16x8;
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

// Nearest-even FP16, saturating at the largest finite value (65504); NaN
// stays NaN.
LM_DEV _Float16 lm_f32_to_f16_sat(float f) {
  return (_Float16)(fabsf(f) > 65504.0f ? copysignf(65504.0f, f) : f);
}

// Power of two 2^s (|s| <= 126) and the shift s of such a power, by their
// exponent bits.
LM_DEV float lm_pow2(int s) { return __uint_as_float((uint32_t)(127 + s) << 23); }
LM_DEV int lm_log2_of_pow2(float p) { return (int)(__float_as_uint(p) >> 23) - 127; }

// silu(g) = g * sigma(g), with the hardware reciprocal (about one ulp) in
// place of an IEEE division: the result is rounded to FP16 or an MX code.
LM_DEV float lm_silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// v from the lane that a DPP control word names (quad_perm, row mirrors).
template <int CTRL>
LM_DEV float lm_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// v from lane xor 16 within each group of 32 (ds_swizzle, bit mode: and
// mask 0x1F, xor mask 0x10; no memory access).
LM_DEV float lm_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Reduction over the 32 lanes sharing bit 5 of the lane id of N values per
// lane at once, each step applied to all N before the next (so a value's
// cross-lane moves are N instructions apart, with no wait states): lanes
// xor 1 and xor 2 (DPP quad_perm), then the mirrored partner in the group of
// 8 and of 16 (DPP row mirrors; each group already holds its result in every
// lane), then lane xor 16. Every lane ends with the same result: each step
// combines a lane with one partner, and max and + commute.
template <int N, class Op>
LM_DEV void lm_half_reduce(float (&v)[N], Op op) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = op(v[i], lm_dpp<0xB1>(v[i]));   // quad_perm [1,0,3,2]
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = op(v[i], lm_dpp<0x4E>(v[i]));   // quad_perm [2,3,0,1]
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = op(v[i], lm_dpp<0x141>(v[i]));  // row_half_mirror
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = op(v[i], lm_dpp<0x140>(v[i]));  // row_mirror
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = op(v[i], lm_xor16(v[i]));       // lane xor 16
}
