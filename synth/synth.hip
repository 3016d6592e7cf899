// Seeded synthetic inputs for the latent-MoE layer: one counter-based generator,
// evaluated either on host cores or on the GPU, producing identical bytes.
//
// This module holds no arithmetic of the layer itself. It only draws numbers:
//   bits(i)  = SplitMix64 output function applied to key + (i+1)*golden-gamma
//              (Steele, Lea & Flood, "Fast splittable pseudorandom number
//              generators", OOPSLA 2014; the 64-bit finaliser constants are
//              the ones Vigna publishes for splitmix64).
//   z        = a standard normal variate by inverse-CDF table lookup: the top
//              16 bits pick one of 65536 equal-probability segments of a
//              piecewise-linear inverse normal CDF (segment s spans the
//              quantiles s/2^16 to (s+1)/2^16), the next 16 bits place the
//              sample inside that segment. The two end segments (the normal's
//              tails beyond 4.17 sigma) are split again by the remaining 32
//              bits: 16 pick one of 65536 equal-probability sub-segments of
//              the lower tail (sub-segment t spans the quantiles t/2^32 to
//              (t+1)/2^32; the first starts at 2^-33, so |z| <= 6.36), 16
//              place the sample inside it, and the upper end segment takes the
//              mirror image. The knot tables are computed on the host from
//              scipy's ndtri and passed in, so host and device read the same
//              floats and use only exactly-rounded operations (fmaf, one
//              multiply, integer rounding), which makes both sides
//              bit-identical.
//   value    = z * scale               (weights, x)
//            = 1 + 0.1 * z             (RMSNorm gammas)
// Outputs: FP32, BF16 (round-to-nearest-even of the FP32 value) or MXFP4
// (OCP Microscaling v1.0: E2M1 elements, one E8M0 scale per 32 consecutive
// elements along the contiguous axis, scale exponent floor(log2 amax) - 2,
// elements rounded to nearest even on the E2M1 grid and saturated at +-6).
// The MXFP4 path is how a quantised checkpoint is produced; the layer only
// ever decodes it.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <thread>
#include <vector>
#include <algorithm>

#define SYN_HD __host__ __device__ __forceinline__

enum { SYN_F32 = 0, SYN_BF16 = 1, SYN_MXFP4 = 2 };
enum { SYN_MODE_SCALED = 0, SYN_MODE_GAMMA = 1 };

SYN_HD uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYN_HD uint64_t syn_key(uint64_t seed, uint32_t tensor_id, uint32_t chunk) {
  uint64_t k = syn_mix(seed + 0x9E3779B97F4A7C15ULL);
  k ^= (uint64_t)(tensor_id + 1) * 0xD1B54A32D192ED03ULL;
  k = syn_mix(k);
  k ^= (uint64_t)(chunk + 1) * 0x8CB92BA72F3D8DD7ULL;
  return syn_mix(k);
}

SYN_HD uint64_t syn_bits(uint64_t key, uint64_t i) {
  return syn_mix(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

// knots / slopes: 2 x 65536 entries, the interior segments at [s] (s = 1 ..
// 65534) and the lower tail's sub-segments at [65536 + t].
SYN_HD float syn_normal(const float* knots, const float* slopes, uint64_t bits) {
  const uint32_t seg = (uint32_t)(bits >> 48);
  const uint32_t frac = (uint32_t)(bits >> 32) & 0xFFFFu;
  if (seg != 0u && seg != 0xFFFFu) return fmaf(slopes[seg], (float)frac * (1.0f / 65536.0f), knots[seg]);
  const uint32_t t = 65536u + ((uint32_t)(bits >> 16) & 0xFFFFu);
  const uint32_t tfrac = (uint32_t)bits & 0xFFFFu;
  const float z = fmaf(slopes[t], (float)tfrac * (1.0f / 65536.0f), knots[t]);
  return seg == 0u ? z : -z;
}

SYN_HD float syn_value(const float* knots, const float* slopes, uint64_t key, uint64_t i,
                       int mode, float scale) {
  float z = syn_normal(knots, slopes, syn_bits(key, i));
  return mode == SYN_MODE_GAMMA ? fmaf(0.1f, z, 1.0f) : z * scale;
}

SYN_HD uint32_t syn_f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

SYN_HD uint16_t syn_bf16_rne(float f) {
  uint32_t u = syn_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E2M1 code (sign in bit 3) of v, already divided by the block scale.
SYN_HD uint8_t syn_e2m1_rne(float v) {
  uint8_t s = (syn_f32_bits(v) >> 31) ? 8 : 0;
  float a = fabsf(v);
  uint8_t m;
  // Midpoints between neighbouring grid values {0,.5,1,1.5,2,3,4,6}; a tie
  // goes to the neighbour whose mantissa bit is 0 (even).
  if (a <= 0.25f) m = 0;
  else if (a < 0.75f) m = 1;
  else if (a <= 1.25f) m = 2;
  else if (a < 1.75f) m = 3;
  else if (a <= 2.5f) m = 4;
  else if (a < 3.5f) m = 5;
  else if (a <= 5.0f) m = 6;
  else m = 7;
  return (uint8_t)(s | m);
}

// One 32-element block: values -> 16 packed bytes (element 2i low nibble) + scale code.
SYN_HD void syn_mx_block(const float* v, uint8_t* packed, uint8_t* scale_code) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int code;
  int e;
  if (amax == 0.0f) {
    code = 0;
    e = -127;
  } else {
    uint32_t bexp = (syn_f32_bits(amax) >> 23) & 0xFFu;  // values here are normal floats
    e = (int)bexp - 127 - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    code = e + 127;
  }
  // Division by 2^e is exact; build 2^-e directly from its exponent bits.
  int ie = -e;
  float inv = 1.0f;
  if (ie > 0) { for (int i = 0; i < ie; ++i) inv *= 2.0f; }
  else { for (int i = 0; i < -ie; ++i) inv *= 0.5f; }
  for (int i = 0; i < 16; ++i) {
    uint8_t lo = syn_e2m1_rne(v[2 * i] * inv);
    uint8_t hi = syn_e2m1_rne(v[2 * i + 1] * inv);
    packed[i] = (uint8_t)(lo | (hi << 4));
  }
  *scale_code = (uint8_t)code;
}

struct SynArgs {
  uint64_t key;
  int kind, mode;
  float scale;
  uint64_t start, count;  // elements
  const float* knots;
  const float* slopes;
  void* out;
  uint8_t* out_scales;
};

SYN_HD void syn_fill_one(const SynArgs& a, uint64_t j) {
  // j: element index (F32/BF16) or block index (MXFP4), relative to start.
  if (a.kind == SYN_F32) {
    ((float*)a.out)[j] = syn_value(a.knots, a.slopes, a.key, a.start + j, a.mode, a.scale);
  } else if (a.kind == SYN_BF16) {
    ((uint16_t*)a.out)[j] =
        syn_bf16_rne(syn_value(a.knots, a.slopes, a.key, a.start + j, a.mode, a.scale));
  } else {
    float v[32];
    uint64_t e0 = a.start + j * 32;
    for (int i = 0; i < 32; ++i) v[i] = syn_value(a.knots, a.slopes, a.key, e0 + i, a.mode, a.scale);
    syn_mx_block(v, (uint8_t*)a.out + j * 16, a.out_scales + j);
  }
}

__global__ void syn_fill_kernel(SynArgs a, uint64_t units) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < units; j += stride)
    syn_fill_one(a, j);
}

static int syn_make_args(SynArgs* a, uint64_t seed, uint32_t tensor_id, uint32_t chunk, int kind,
                         int mode, float scale, uint64_t start, uint64_t count, const float* knots,
                         const float* slopes, void* out, void* out_scales, uint64_t* units) {
  if (!out || !knots || !slopes) return -1;
  if (kind < SYN_F32 || kind > SYN_MXFP4) return -1;
  if (kind == SYN_MXFP4 && ((start % 32) || (count % 32) || !out_scales)) return -1;
  a->key = syn_key(seed, tensor_id, chunk);
  a->kind = kind;
  a->mode = mode;
  a->scale = scale;
  a->start = start;
  a->count = count;
  a->knots = knots;
  a->slopes = slopes;
  a->out = out;
  a->out_scales = (uint8_t*)out_scales;
  *units = kind == SYN_MXFP4 ? count / 32 : count;
  return 0;
}

extern "C" {

// Fill `count` elements starting at linear element index `start` of tensor
// (seed, tensor_id, chunk) into host memory, using up to `nthreads` threads
// (<= 0: all hardware threads). Returns 0, or -1 on a bad argument.
int synth_fill_cpu(uint64_t seed, uint32_t tensor_id, uint32_t chunk, int kind, int mode,
                   float scale, uint64_t start, uint64_t count, const float* knots,
                   const float* slopes, void* out, void* out_scales, int nthreads) {
  SynArgs a;
  uint64_t units;
  if (syn_make_args(&a, seed, tensor_id, chunk, kind, mode, scale, start, count, knots, slopes,
                    out, out_scales, &units))
    return -1;
  int nt = nthreads > 0 ? nthreads : (int)std::max(1u, std::thread::hardware_concurrency());
  if ((uint64_t)nt > units / 4096 + 1) nt = (int)(units / 4096 + 1);
  if (nt <= 1) {
    for (uint64_t j = 0; j < units; ++j) syn_fill_one(a, j);
    return 0;
  }
  std::vector<std::thread> pool;
  uint64_t per = (units + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    uint64_t lo = per * t, hi = std::min(units, lo + per);
    if (lo >= hi) break;
    pool.emplace_back([&a, lo, hi]() {
      for (uint64_t j = lo; j < hi; ++j) syn_fill_one(a, j);
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

// Same fill into device memory on `stream` (a hipStream_t; 0 = null stream).
// `knots`/`slopes` must be device pointers here. Returns 0, -1 on a bad
// argument, -4 on a HIP error.
int synth_fill_gpu(uint64_t seed, uint32_t tensor_id, uint32_t chunk, int kind, int mode,
                   float scale, uint64_t start, uint64_t count, const float* knots,
                   const float* slopes, void* out, void* out_scales, void* stream) {
  SynArgs a;
  uint64_t units;
  if (syn_make_args(&a, seed, tensor_id, chunk, kind, mode, scale, start, count, knots, slopes,
                    out, out_scales, &units))
    return -1;
  if (units == 0) return 0;
  int threads = 256;
  uint64_t blocks = (units + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(syn_fill_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, a, units);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
