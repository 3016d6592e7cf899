// Kernels of the latent-MoE layer forward (gfx950).
//
// Step order (web page "SGLang and Miles Add Day-0 Support for Muse Spark
// Open", section "MoE with Pooler, Unpooler and Per-Expert Normalization"):
//   optional boundary RMSNorm of the residual     lm_input_norm_kernel
//   router logits (FP32)  -> top-k + softmax      lm_topk_kernel
//   grouping by expert    (LDS histogram per block, then a stable scatter:
//                          the "LDS kernel" replacing an atomic-add expert
//                          sort, section "AMD Support / Day-0 Enablement")
//   pooler GEMM + pre-expert RMSNorm statistics  PoolerProb, lm_rowscale_kernel
//   gate/up GEMM per expert + SwiGLU             GateUpProb
//   down GEMM per expert + per-row sum of squares partials (section "The
//     Fused Post-per-expert Norm": each second-GEMM tile contributes a partial
//     sum of squares; here written per tile and summed in a fixed order)
//   per-expert RMSNorm, routing weight, FP32 sum  lm_combine_kernel
//   unpooler GEMM                                 UnpoolerProb
#pragma once
#include "gemm.h"

// ------------------------------------------------------------ boundary norm
// Exact three-piece BF16 split of an FP32 value: f = b1 + b2 + b3 with each
// piece the nearest-even BF16 of what remains (exact for normal floats: 8
// significant bits per piece, and each remainder is exact in FP32).
LM_DEV void lm_split3(float f, uint16_t& b1, uint16_t& b2, uint16_t& b3) {
  b1 = lm_f32_to_bf16(f);
  const float r1 = f - lm_bf16_to_f32(b1);
  b2 = lm_f32_to_bf16(r1);
  const float r2 = r1 - lm_bf16_to_f32(b2);
  b3 = lm_f32_to_bf16(r2);
}

// One token row per workgroup: x = r * (1 / sqrt(mean(r^2) + eps)) * gamma
// (the block's sandwich pre-norm; the router reads its FP32 output), with the
// sum of squares, the root and each product in FP64 and one rounding to FP32
// per element. FP32 layers write x to xn [T, H]. BF16 layers write its exact
// three-piece BF16 split to xs [T, 3H] (pieces side by side): the first piece
// is x's nearest-even BF16 rounding, the pooler's input, and the router forms
// the FP32 products from the pieces on the matrix cores. Each thread owns
// 8-element chunks (H % 64 == 0); sum order: per-thread chunk partials, wave
// butterfly, then the four waves in order. The second pass re-reads the row
// (16 KB at H = 8192, from L2).
template <typename Et>
__global__ __launch_bounds__(256) void lm_input_norm_kernel(const Et* r, int H, const float* gamma,
                                                            float eps, float* xn, uint16_t* xs) {
  __shared__ double red[4];
  // 8 elements = one 16-byte load (BF16) or two (FP32)
  const lm_u32x4* row = (const lm_u32x4*)(r + (size_t)blockIdx.x * H);
  const int nch = H / 8;
  auto elems = [&](int c, float (&v)[8]) {
    if constexpr (sizeof(Et) == 2) {
      const lm_u32x4 q = row[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(q[j] << 16);
        v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
      }
    } else {
      const lm_u32x4 q0 = row[2 * c], q1 = row[2 * c + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = __uint_as_float(q0[j]);
        v[4 + j] = __uint_as_float(q1[j]);
      }
    }
  };
  // Four chunks per thread in flight (indices clamped, all loads issued
  // before the arithmetic), processed in chunk order.
  constexpr int kU = 4;
  double s = 0.0;
  for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * kU) {
    float v[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u) elems(min(c0 + 256 * u, nch - 1), v[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (c0 + 256 * u < nch) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s += (double)v[u][j] * (double)v[u][j];
      }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const double inv = 1.0 / sqrt((((red[0] + red[1]) + red[2]) + red[3]) / H + (double)eps);
  for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * kU) {
    float vv[kU][8];
    float4 gg[kU][2];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(c0 + 256 * u, nch - 1);
      elems(c, vv[u]);
      gg[u][0] = ((const float4*)gamma)[2 * c];
      gg[u][1] = ((const float4*)gamma)[2 * c + 1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 256 * u;
      if (c >= nch) break;
      const float* v = vv[u];
      const float g[8] = {gg[u][0].x, gg[u][0].y, gg[u][0].z, gg[u][0].w,
                          gg[u][1].x, gg[u][1].y, gg[u][1].z, gg[u][1].w};
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (float)((double)v[j] * inv * (double)g[j]);
      if (xn) {
        float4* dst = (float4*)(xn + (size_t)blockIdx.x * H) + 2 * c;
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
      if (xs) {
        lm_u32x4 p[3];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint16_t a1, a2, a3, b1, b2, b3;
          lm_split3(o[2 * j], a1, a2, a3);
          lm_split3(o[2 * j + 1], b1, b2, b3);
          p[0][j] = (uint32_t)a1 | ((uint32_t)b1 << 16);
          p[1][j] = (uint32_t)a2 | ((uint32_t)b2 << 16);
          p[2][j] = (uint32_t)a3 | ((uint32_t)b3 << 16);
        }
        lm_u32x4* dst = (lm_u32x4*)(xs + (size_t)blockIdx.x * 3 * H);
        dst[c] = p[0];
        dst[nch + c] = p[1];
        dst[2 * nch + c] = p[2];
      }
    }
  }
}

// --------------------------------------------------- matrix-core B layout
// Weights read by the streaming kernel are repacked once (at create) so that
// one 16-byte load per lane fetches exactly the B fragment of a 32x32x16
// MFMA step, and the 64 lanes of that load read 1 KB of contiguous memory.
// For a row-major [R, K] matrix of 16-bit elements (R % 256 == 0, K % 64 ==
// 0), 16-byte chunk c of row n, in row group g = n/32 (block gb = g/8, gi =
// g%8) and k-tile kt = c/8, lands at chunk index
//   (((gb * K/64 + kt) * 8 + gi) * 4 + s) * 64 + h * 32 + n%32
// with MFMA step s = (c%8)%4 and lane half h = (c%8)/4: 4 KB per group and
// k-tile, the eight groups of a block side by side for each k-tile. A
// workgroup reading 4 or 8 consecutive groups (its waves' weight rows) thus
// reads 16 or 32 KB of contiguous memory per k-tile and tensor, not 4 KB
// pieces 256 KB apart.
template <typename E>
LM_DEV const lm_u32x4* lm_packed_group(const E* base, int64_t row0, int K) {
  const int64_t g = row0 / 32;
  return (const lm_u32x4*)base +
         ((g / kLmPackGroups) * (int64_t)(K / 64) * kLmPackGroups + g % kLmPackGroups) * 256;
}

// ds == nullptr: BF16 copied as is. Otherwise the BF16 source is written as
// FP16, each row times 2^s, with 2^-s = ds[row] from lm_row_descale_bf16_kernel,
// and (kc != nullptr) each 32-column block of a row times 2^c as well, c =
// kc[(row / rows_per_set) * K/32 + block] (the down weights of expert e: the
// shifts of the SwiGLU output's blocks, see lm_a_shift_kernel).
__global__ void lm_pack_mfma_kernel(const lm_u32x4* src, lm_u32x4* dst, int64_t rows, int K,
                                    const float* ds, const int* kc, int64_t rows_per_set) {
  const int64_t n = rows * (K / 8);
  const int ktiles = K / 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63), s = (int)((i >> 6) & 3);
    const int gi = (int)((i >> 8) % kLmPackGroups);
    const int64_t rest = (i >> 8) / kLmPackGroups;  // gb * K/64 + kt
    const int64_t gb = rest / ktiles;
    const int kt = (int)(rest - gb * ktiles);
    const int64_t row = (gb * kLmPackGroups + gi) * 32 + (lane & 31);
    lm_u32x4 v = src[row * (K / 8) + kt * 8 + 4 * (lane >> 5) + s];
    if (ds) {
      const float m = lm_pow2(-lm_log2_of_pow2(ds[row]));
      // the chunk's 8 columns lie in 32-column block 2 kt + h
      const float mc = kc ? lm_pow2(kc[(row / rows_per_set) * (K / 32) + 2 * kt + (lane >> 5)]) : 1.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const _Float16 lo = (_Float16)(lm_bf16_to_f32((uint16_t)(v[q] & 0xffffu)) * mc * m);
        const _Float16 hi = (_Float16)(lm_bf16_to_f32((uint16_t)(v[q] >> 16)) * mc * m);
        v[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
    }
    dst[i] = v;
  }
}

// FP16 copies of BF16 weights: each weight row (an output column of its
// GEMM) is scaled by a power of two 2^s before the conversion, so that its
// largest magnitude lands in [2^14, 2^15): s = 141 - the biased exponent of
// that magnitude. A BF16 value has 8 significant bits and FP16 reaches down
// to multiples of 2^-24, so every value of the row within 2^31 of the
// largest converts exactly (a smaller one rounds, by at most 2^-39 of the
// largest). The epilogue multiplies the output
// column by ds[row] = 2^-s (exact). s is clamped to [-100, 100] (an all-zero
// row gets 2^-100). With kc, each 32-column block counts times its 2^c (as
// lm_pack_mfma_kernel scales it). One wavefront per row.
__global__ __launch_bounds__(256) void lm_row_descale_bf16_kernel(const uint16_t* w, int64_t rows,
                                                                  int K, float* ds, const int* kc,
                                                                  int64_t rows_per_set) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += waves) {
    const lm_u32x4* row = (const lm_u32x4*)(w + r * K);
    uint32_t m = 0;
    for (int c = lane; c < K / 8; c += 64) {
      const lm_u32x4 q = row[c];
      // magnitude bits; a block shift adds c to the exponent field of non-zero values
      const uint32_t add = kc ? (uint32_t)kc[(r / rows_per_set) * (K / 32) + c / 4] << 7 : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = q[j] & 0x7fffu, hi = (q[j] >> 16) & 0x7fffu;
        m = max(m, max(lo ? lo + add : 0u, hi ? hi + add : 0u));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    if (lane == 0) ds[r] = lm_pow2(-min(max(141 - (int)(m >> 7), -100), 100));
  }
}

// Euclidean norm of each row of a BF16 [rows, K] matrix (FP32 sums), one
// wavefront per row.
__global__ __launch_bounds__(256) void lm_row_norm_bf16_kernel(const uint16_t* w, int64_t rows, int K,
                                                               float* out) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += waves) {
    const lm_u32x4* row = (const lm_u32x4*)(w + r * K);
    float s = 0.0f;
    for (int c = lane; c < K / 8; c += 64) {
      const lm_u32x4 q = row[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __uint_as_float(q[j] << 16), b = __uint_as_float(q[j] & 0xffff0000u);
        s += a * a + b * b;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    if (lane == 0) out[r] = sqrtf(s);
  }
}

// The same for MXFP4 [rows, K] (codes [rows, K/2], E8M0 scales [rows, K/32]);
// each lane decodes one 32-element block at a time.
__global__ __launch_bounds__(256) void lm_row_norm_mx_kernel(const uint8_t* codes, const uint8_t* sc,
                                                             int64_t rows, int K, float* out) {
  const float e2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += waves) {
    float s = 0.0f;
    for (int b = lane; b < K / 32; b += 64) {
      const lm_u32x4 q = ((const lm_u32x4*)(codes + r * (K / 2)))[b];
      const uint32_t code = sc[r * (K / 32) + b];
      const float x = code == 255 ? __uint_as_float(0x7fc00000u) : ldexpf(1.0f, (int)code - 127);
      float t = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float v = e2m1[(q[j >> 3] >> (4 * (j & 7))) & 7u];
        t += v * v;
      }
      s += t * x * x;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    if (lane == 0) out[r] = sqrtf(s);
  }
}

// Shifts of the FP16 SwiGLU output a: for expert e and intermediate index i,
// |a_i| = |silu(g_i) v_i| <= |g_i| |v_i| <= ||Wg_i|| ||Wu_i|| ||u||^2
// (Cauchy-Schwarz, |silu(g)| <= |g|), and ||u||^2 <= u2 = P max(gamma_p)^2
// (an RMS-normed row). Per block of 32 consecutive i (one MX scale block of
// the down weights' reduction axis): c = the smallest shift >= 0 with the
// block's largest bound times 2^-c within 2^15 (at most 60). The gate/up
// epilogue stores a times a_down = 2^-c; the down weights' copies carry 2^c
// on those 32 columns, so the products are unchanged.
__global__ void lm_a_shift_kernel(const float* ng, const float* nu, int64_t nblk, float u2, int* kc,
                                  float* a_down) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * blockDim.x) {
    float m = 0.0f;
    for (int i = 0; i < 32; ++i) m = fmaxf(m, ng[b * 32 + i] * nu[b * 32 + i]);
    const float bound = m * u2;
    int c = 0;
    if (bound > 32768.0f && bound <= 3.0e38f) {
      int e;
      frexpf(bound / 32768.0f, &e);  // bound / 2^15 <= 2^e
      c = min(e, 60);
    } else if (!(bound <= 32768.0f)) {
      c = 60;  // infinite (or NaN) bound: the largest shift
    }
    kc[b] = c;
    a_down[b] = lm_pow2(-c);
  }
}

// Powers of two of the FP16 expert outputs, which hold o times the expert's
// gamma, one per expert: |o_p| = |Wd_p . a| <= ||Wd_p|| ||a|| and ||a|| <=
// ||u||^2 sqrt(sum_i (||Wg_i|| ||Wu_i||)^2) (each |a_i| <= ||Wg_i|| ||Wu_i||
// ||u||^2, as for lm_a_shift_kernel), with ||u||^2 <= u2; the bound on
// |o_p gamma_p| takes max_p |gamma_p| as well; amp (1, or 2 where a is
// MX-quantised: a code can exceed its value by at most a factor 1.5) scales
// it. o_down = the largest 2^-c, 0 <= c <= 100, keeping the bound within
// 2^15; o_up = 2^c. One workgroup per expert: ng, nu [E, I] (gate / up row
// norms), nd [E, P] (down row norms), gamma [E, P].
__global__ __launch_bounds__(256) void lm_o_shift_kernel(const float* ng, const float* nu, const float* nd,
                                                         const float* gamma, int I, int P, float u2, float amp,
                                                         float* o_down, float* o_up) {
  __shared__ double red[256];
  __shared__ float redm[256], redg[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  double s = 0.0;
  for (int i = tid; i < I; i += 256) {
    const double q = (double)ng[(size_t)e * I + i] * (double)nu[(size_t)e * I + i];
    s += q * q;
  }
  float m = 0.0f, gm = 0.0f;
  for (int p = tid; p < P; p += 256) {
    m = fmaxf(m, nd[(size_t)e * P + p]);
    gm = fmaxf(gm, fabsf(gamma[(size_t)e * P + p]));
  }
  red[tid] = s;
  redm[tid] = m;
  redg[tid] = gm;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      red[tid] += red[tid + o];
      redm[tid] = fmaxf(redm[tid], redm[tid + o]);
      redg[tid] = fmaxf(redg[tid], redg[tid + o]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double bound = (double)redm[0] * (double)u2 * sqrt(red[0]) * (double)amp * (double)redg[0];
    int c = 0;
    if (!(bound <= 32768.0)) {  // above 2^15, infinite or NaN
      if (bound <= 1e300) {
        int ex;
        frexp(bound / 32768.0, &ex);  // bound / 2^15 <= 2^ex
        c = min(ex, 100);
      } else {
        c = 100;
      }
    }
    o_down[e] = lm_pow2(-c);
    o_up[e] = lm_pow2(c);
  }
}

// The same for MXFP4 weights, from their E8M0 scales [rows, K/32]: with emax
// the row's largest scale code (255, NaN, ignored), s = 139 - emax puts the
// row's largest decoded magnitude (at most 6 x 2^(emax - 127)) in [2^14,
// 24576]; every E2M1 value of a block whose scale is within 2^35 of emax is
// then an FP16 number. One thread per row.
__global__ void lm_row_descale_mx_kernel(const uint8_t* sc, int64_t rows, int K, float* ds,
                                         const int* kc, int64_t rows_per_set) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x) {
    const lm_u32x4* row = (const lm_u32x4*)(sc + r * (K / 32));
    const int* rc = kc ? kc + (r / rows_per_set) * (K / 32) : nullptr;
    int m = 0;
    for (int c = 0; c < K / 512; ++c) {
      const lm_u32x4 q = row[c];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int b = (int)((q[j >> 2] >> (8 * (j & 3))) & 0xffu);
        const int bc = rc ? min(b + rc[c * 16 + j], 254) : b;  // as lm_pack_mx_kernel stores it
        m = b != 255 ? max(m, bc) : m;
      }
    }
    ds[r] = lm_pow2(-min(max(139 - m, -100), 100));
  }
}

// MXFP4 weights use the same 32-row blocks: for k-tile kt (64 columns) of a
// 32-row group, lane L = 32h + r holds the 32 E2M1 codes of row r, columns
// [64kt + 32h, 64kt + 32h + 32) as 16 bytes (element 2i in the low nibble):
// exactly one 32-element scale block, and bytes 4s..4s+3 are the B fragment
// of MFMA step s. The 64 lanes of a k-tile are 1 KB contiguous. Scales: one
// byte per lane and k-tile, packed as a dword per lane for four k-tiles:
//   scale byte of (group g, k-tile kt, lane L) at ((g*K/256 + kt/4)*64 + L)*4 + kt%4.
LM_DEV const lm_u32x4* lm_packed_mx_group(const void* base, int64_t row0, int K) {
  return (const lm_u32x4*)base + (row0 / 32) * (int64_t)(K / 64) * 64;
}
LM_DEV const uint32_t* lm_packed_mx_scales(const void* base, int64_t row0, int K) {
  return (const uint32_t*)base + (row0 / 32) * (int64_t)(K / 256) * 64;
}

// kc != nullptr: each 32-column block's scale code is raised by its shift c
// (lm_a_shift_kernel; codes stay at most 254).
__global__ void lm_pack_mx_kernel(const lm_u32x4* src, const uint8_t* src_scales, lm_u32x4* dst,
                                  uint8_t* dst_scales, int64_t rows, int K, const int* kc,
                                  int64_t rows_per_set) {
  const int64_t n = rows * (K / 32);  // 16-byte chunks (32 codes each)
  const int ktiles = K / 64;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = i >> 6;
    const int lane = (int)(i & 63);
    const int64_t g = blk / ktiles;
    const int kt = (int)(blk - g * ktiles);
    const int h = lane >> 5;
    const int64_t row = g * 32 + (lane & 31);
    const int64_t sidx = row * (K / 32) + 2 * kt + h;  // source chunk == source scale index
    dst[i] = src[sidx];
    int code = src_scales[sidx];
    if (kc && code != 255) code = min(code + kc[(row / rows_per_set) * (K / 32) + 2 * kt + h], 254);
    dst_scales[((g * (K / 256) + kt / 4) * 64 + lane) * 4 + (kt & 3)] = (uint8_t)code;
  }
}

// ----------------------------------------------------------------- router
// Partial logits over k-splits: part[s][t][e] = sum over split s of x[t,k] W[e,k],
// accumulated as FP64 sums of per-k-tile FP32 matrix-core chains.
// FP32 layers: x and W FP32, one k-tile per 32 columns.
// BF16 activations: W is [E, 3H] holding the exact three-piece BF16 split
// W1|W2|W3 of the FP32 router. x BF16 (pieces = 1): x is read three times
// (a_ktile wraps), so the matrix cores see exact products x*Wj. x given as
// its own three-piece split X1|X2|X3 [T, 3H] (pieces = 3, the boundary norm's
// FP32 output): the logical K runs over six segments X1W1, X1W2, X1W3, X2W1,
// X2W2, X3W1, every product exact. The dropped cross terms X2W3, X3W2 and
// X3W3 are each at most 2^-24 of |x||W| (X2, W2 within 2^-8 and X3, W3 within
// 2^-16 of the whole), about 2^-26 on average, and of random sign, so their
// sum over a row stays far below the FP32 rounding of the logit.
template <class Cfg_>
struct RouterProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  const E* x;
  const E* w;
  double* part;
  int T, Ew, H, Kw, kta, mt, nt, splits, kt_per;
  int lda = 0;     // row stride of x in elements (0: H)
  int pieces = 1;  // BF16: pieces of x (1 or 3)
  lm_u32x4* counters = nullptr;  // the top-k kernel's expert counters, cleared here
  int counter_chunks = 0;        // their size in 16-byte chunks

  LM_DEV void clear(int bid, int nb, int tid) const {
    for (int i = bid * 256 + tid; i < counter_chunks; i += nb * 256) counters[i] = lm_u32x4{0u, 0u, 0u, 0u};
  }
  LM_DEV int ktot() const { return pieces == 3 ? 6 * kta : Kw / Cfg::KT; }
  LM_DEV bool tile(int bid, LmTile& t) const {
    int L;
    if (!lm_xcd_map(bid, mt * nt * splits, L)) return false;
    const int s = L / (mt * nt);
    int m, n;
    lm_dense_order(L - s * mt * nt, mt, nt, 8, m, n);
    t.m0 = m * Cfg::BM;
    t.rows = min(Cfg::BM, T - t.m0);
    t.n0 = n * Cfg::BN;
    t.nt = n;
    t.e = s;
    t.kt0 = s * kt_per;
    t.kt1 = min(ktot(), t.kt0 + kt_per);
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(x + (size_t)(t.m0 + min(r, t.rows - 1)) * (lda ? lda : H));
  }
  LM_DEV const lm_u32x4* b_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(w + (size_t)min(t.n0 + r, Ew - 1) * Kw);
  }
  // segment g of the six-product K: x piece (0,0,0,1,1,2), W piece (0,1,2,0,1,0)
  LM_DEV int a_ktile(int kt) const {
    if (pieces != 3) return kt % kta;
    const int g = kt / kta;
    return (g < 3 ? 0 : g < 5 ? 1 : 2) * kta + kt % kta;
  }
  LM_DEV int b_ktile(int kt) const {
    if (pieces != 3) return kt;
    const int g = kt / kta;
    return (g < 3 ? g : g - 3 - (g == 5 ? 2 : 0)) * kta + kt % kta;
  }
  LM_DEV void epilogue_f64(const LmTile& t, const double (&acc)[Cfg::TM][Cfg::TN][16], int wm,
                           int wn, int lane) const {
    double* dst = part + ((size_t)t.e * T + t.m0) * Ew + t.n0;
#pragma unroll
    for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn) {
        const int col = lm_acc_col<Cfg>(wn, tn, lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
          if (row < t.rows && t.n0 + col < Ew) dst[(size_t)row * Ew + col] = acc[tm][tn][i];
        }
      }
  }
};

// ----------------------------------------------------------------- pooler
// h = x Wp^T. Writes gamma_p * h (FP32 layers: to pooled; BF16 layers: in
// FP32 to pooled32) and, per row and n-tile, the partial sum of h^2 used by
// the pre-expert RMSNorm.
template <class Cfg_>
struct PoolerProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  const E* x;
  const E* w;
  const float* gamma;
  E* pooled;
  float* ssq;  // [T, nt]
  int T, H, P, mt, nt;
  float* pooled32 = nullptr;  // if set, gamma_p * h is written here in FP32 instead

  LM_DEV bool tile(int bid, LmTile& t) const {
    int L;
    if (!lm_xcd_map(bid, mt * nt, L)) return false;
    int m, n;
    lm_dense_order(L, mt, nt, 8, m, n);
    t.m0 = m * Cfg::BM;
    t.rows = min(Cfg::BM, T - t.m0);
    t.n0 = n * Cfg::BN;
    t.nt = n;
    t.e = 0;
    t.kt0 = 0;
    t.kt1 = H / Cfg::KT;
    return true;
  }
  int lda = 0;  // row stride of x in elements (0: H)
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(x + (size_t)(t.m0 + min(r, t.rows - 1)) * (lda ? lda : H));
  }
  LM_DEV const lm_u32x4* b_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(w + (size_t)min(t.n0 + r, P - 1) * H);
  }
  LM_DEV const lm_u32x4* b_group(const LmTile& t, int wv, int j) const {
    return lm_packed_group(w, min(t.n0 + (wv * Cfg::TN + j) * 32, P - 32), H);
  }
  LM_DEV int a_ktile(int kt) const { return kt; }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void* smem) const {
    float* red = (float*)smem;
    lm_tile_row_ssq<Cfg>(acc, wm, wn, lane, P - t.n0, red, [](float v, int, int) { return v; });
    if ((int)threadIdx.x < t.rows)
      ssq[(size_t)(t.m0 + threadIdx.x) * nt + t.nt] = red[Cfg::WN * Cfg::BM + threadIdx.x];
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int col = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
      if (col >= P) continue;
      const float g = gamma[col];
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
          if (row < t.rows) {
            const float v = acc[tm][tn][i] * g;
            if (pooled32) pooled32[(size_t)(t.m0 + row) * P + col] = v;
            else pooled[(size_t)(t.m0 + row) * P + col] = LmElem<E>::from_f32(v);
          }
        }
    }
  }
};

// ------------------------------------------------------ grouped tile lookup
// Tiles of all experts form one list: expert e owns tiles
// [tile_off[e], tile_off[e+1]) (ceil(count_e / BM) of them), each walked over
// all nt column tiles. Logical index L -> (expert, m-tile, n-tile): within an
// expert, groups of up to 8 m-tiles walk all n-tiles together, the m-tiles of
// a group adjacent, so they share each weight tile in L2 while the group's
// rows are reused across the n-tiles (an expert of a few m-tiles is one
// group; a hot expert's rows are not streamed again for every n-tile).
LM_DEV bool lm_group_tile(const int* tile_off, const int* offsets, const int* counts, int E, int BM,
                          int nt, int cols, int bid, LmTile& t) {
  const int total = tile_off[E] * nt;
  int L;
  if (!lm_xcd_map(bid, total, L)) return false;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] * nt <= L) lo = mid;
    else hi = mid;
  }
  const int e = lo;
  const int mte = tile_off[e + 1] - tile_off[e];
  int mi, n;
  lm_dense_order(L - tile_off[e] * nt, mte, nt, 8, mi, n);
  t.e = e;
  t.m0 = offsets[e] + mi * BM;
  t.rows = min(BM, counts[e] - mi * BM);
  t.n0 = n * cols;
  t.nt = n;
  return true;
}

// --------------------------------------------------------------- gate / up
// For the rows (routed pairs) of expert e: g = u Wg_e^T, v = u Wu_e^T,
// act = silu(g) * v. FP16 operands: u is the normed FP16 row and the weights
// the FP16 copies scaled per row by 2^s, so g and v are the accumulators
// times the rows' 2^-s. FP32 layers: pooled holds gamma_p * h and the token's
// RMSNorm row scale r multiplies the accumulators (the norm is linear in its
// input, so it is applied after the GEMM).
// B tile rows: wave column wn owns rows [64 wn, 64 wn + 64): the first 32 are
// gate rows, the next 32 the up rows of the same 32 output columns, so each
// lane holds g and v of the same element.
template <class Cfg_, bool MX_ = false>
struct GateUpProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  static_assert(Cfg::TN == 2, "gate/up pairs");
  static constexpr int kCols = Cfg::WN * 32;
  static constexpr bool kMx = MX_;  // weights in the packed MXFP4 layout
  static constexpr bool kWeightsOnce = true;
  static constexpr bool kPairedB = true;  // B tile: WN gate groups, then the WN up groups
  static constexpr bool kScaledW = std::is_same_v<E, _Float16>;  // per-row 2^s weight copies
  static constexpr bool kRowValue = !kScaledW;                    // r applied in the epilogue
  const void* sg = nullptr;  // packed scales (MXFP4)
  const void* su = nullptr;
  const float* dsg = nullptr;  // FP16 operands: 2^-s per gate / up weight row [E*I]
  const float* dsu = nullptr;
  float u_up = 1.0f;           // FP16 operands: u is stored times 1 / u_up (a power of two)
  const float* a_down = nullptr;  // FP16 operands: a is stored times a_down[e][i / 32]
  const E* pooled;  // FP16 operands: the normed u [T, P]; FP32 layers: gamma_p * h
  const E* wg;
  const E* wu;
  const float* row_scale;
  const int* perm_token;
  const int* counts;
  const int* offsets;
  const int* tile_off;
  E* act;  // [pairs, I]
  int P, I, Ex, nt;

  LM_DEV bool tile(int bid, LmTile& t) const {
    if (!lm_group_tile(tile_off, offsets, counts, Ex, Cfg::BM, nt, kCols, bid, t)) return false;
    t.kt0 = 0;
    t.kt1 = P / Cfg::KT;
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    const int tok = perm_token[t.m0 + min(r, t.rows - 1)];
    return (const lm_u32x4*)(pooled + (size_t)tok * P);
  }
  LM_DEV const lm_u32x4* b_row(const LmTile& t, int r) const {
    const int within = r & 63;
    const int col = t.n0 + (r >> 6) * 32 + (within & 31);
    const E* base = within >= 32 ? wu : wg;
    return (const lm_u32x4*)(base + ((size_t)t.e * I + col) * P);
  }
  LM_DEV const lm_u32x4* b_group(const LmTile& t, int wv, int j) const {
    if constexpr (kMx) return lm_packed_mx_group(j ? wu : wg, (int64_t)t.e * I + t.n0 + wv * 32, P);
    else return lm_packed_group(j ? wu : wg, (int64_t)t.e * I + t.n0 + wv * 32, P);
  }
  LM_DEV const uint32_t* b_scales(const LmTile& t, int wv, int j) const {
    return lm_packed_mx_scales(j ? su : sg, (int64_t)t.e * I + t.n0 + wv * 32, P);
  }
  LM_DEV const float* b_descale(const LmTile& t, int wv, int j) const {
    return (j ? dsu : dsg) + (int64_t)t.e * I + t.n0 + wv * 32;
  }
  LM_DEV int a_ktile(int kt) const { return kt; }
  // the token's RMSNorm row scale (gathered), one per tile row
  LM_DEV float row_value(const LmTile& t, int r) const {
    return row_scale[perm_token[t.m0 + min(r, t.rows - 1)]];
  }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void* smem) const {
    const float* rs = (const float*)smem;  // row_value() of each tile row
    const int col = t.n0 + wn * 32 + (lane & 31);
    float dg = 1.0f, du = 1.0f, ad = 1.0f;
    if constexpr (kScaledW) {
      dg = dsg[(size_t)t.e * I + col] * u_up;
      du = dsu[(size_t)t.e * I + col] * u_up;
      ad = a_down[(size_t)t.e * (I / 32) + (col >> 5)];
    }
    auto put = [&](int tm, int i) {
      const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
      float g, v;
      if constexpr (kScaledW) {
        g = acc[tm][0][i] * dg;
        v = acc[tm][1][i] * du;
      } else {
        g = rs[row] * acc[tm][0][i];
        v = rs[row] * acc[tm][1][i];
      }
      act[(size_t)(t.m0 + row) * I + col] = LmElem<E>::from_f32(lm_silu(g) * v * ad);
    };
    if (t.rows == Cfg::BM) {
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) put(tm, i);
    } else {
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (lm_acc_row<Cfg>(wm, tm, i, lane) < t.rows) put(tm, i);
    }
  }
};

// -------------------------------------------------------------------- down
// o = act Wd_e^T for the rows of expert e; writes o (FP32 layers) or
// gamma_e * o in FP16 (BF16 layers, out16), and per row and n-tile the
// partial sum of o^2 for the per-expert RMSNorm. FP16 operands: o is the
// accumulator times the weight row's 2^-s.
template <class Cfg_, bool MX_ = false>
struct DownProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  static constexpr bool kMx = MX_;  // weights in the packed MXFP4 layout
  static constexpr bool kWeightsOnce = true;
  static constexpr bool kScaledW = std::is_same_v<E, _Float16>;
  const void* sd = nullptr;         // packed scales (MXFP4)
  const float* dsd = nullptr;       // FP16 operands: 2^-s per down weight row [E*P]
  const E* act;
  const E* wd;
  const int* counts;
  const int* offsets;
  const int* tile_off;
  float* out;  // [pairs, P] FP32, or
  _Float16* out16 = nullptr;      // [pairs, P] FP16: o times gamma_e times o_down[e] (a power of two)
  const float* o_down = nullptr;  // [E], with out16
  const float* gamma = nullptr;   // [E, P] per-expert norm gamma, with out16
  float* ssq;  // [pairs, nt]
  int P, I, Ex, nt;

  LM_DEV bool tile(int bid, LmTile& t) const {
    if (!lm_group_tile(tile_off, offsets, counts, Ex, Cfg::BM, nt, Cfg::BN, bid, t)) return false;
    t.kt0 = 0;
    t.kt1 = I / Cfg::KT;
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(act + (size_t)(t.m0 + min(r, t.rows - 1)) * I);
  }
  LM_DEV const lm_u32x4* b_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(wd + ((size_t)t.e * P + min(t.n0 + r, P - 1)) * I);
  }
  LM_DEV const lm_u32x4* b_group(const LmTile& t, int wv, int j) const {
    const int64_t row0 = (int64_t)t.e * P + min(t.n0 + (wv * Cfg::TN + j) * 32, P - 32);
    if constexpr (kMx) return lm_packed_mx_group(wd, row0, I);
    else return lm_packed_group(wd, row0, I);
  }
  LM_DEV const uint32_t* b_scales(const LmTile& t, int wv, int j) const {
    return lm_packed_mx_scales(sd, (int64_t)t.e * P + min(t.n0 + (wv * Cfg::TN + j) * 32, P - 32), I);
  }
  LM_DEV const float* b_descale(const LmTile& t, int wv, int j) const {
    return dsd + (int64_t)t.e * P + min(t.n0 + (wv * Cfg::TN + j) * 32, P - 32);
  }
  LM_DEV int a_ktile(int kt) const { return kt; }
  // Prefill-sized tiles (one row band, 128 rows): the FP16 outputs go out in
  // whole 128-byte lines. Each wave stages 16 rows x its 64 columns (2 KB of
  // its own LDS region; the caller's LDS holds at least WN x 2 KB) as 4-byte
  // column pairs (lanes 2m, 2m + 1 swap one value of each row pair with a DPP
  // quad permutation, so each writes two columns of one row), then reads it
  // back as 16-byte row segments and writes 8 rows of 128 bytes per store.
  // A wave reads only what it wrote, and a wave's LDS operations complete in
  // order, so no barrier is needed between the two phases.
  LM_DEV void store16_staged(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wn, int lane,
                             const float (&dd)[Cfg::TN], void* smem) const {
    static_assert(Cfg::TN == 2, "64 columns per wave");
    __syncthreads();  // every thread has read the row sums of squares out of the LDS
    const float od = o_down[t.e];
    float gg[Cfg::TN];  // the lane's column of the expert's gamma
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int c = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
      gg[tn] = c < P ? gamma[(size_t)t.e * P + c] : 0.0f;
    }
    const bool odd = lane & 1;
    uint32_t* st = (uint32_t*)smem + wn * 512;  // 16 rows x 32 column pairs
    const lm_u32x4* ld = (const lm_u32x4*)st;
    const int col = t.n0 + wn * 64 + (lane & 7) * 8;  // the lane's 8 columns when reading back
#pragma unroll
    for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn)
#pragma unroll
          for (int i = 8 * h; i < 8 * h + 8; i += 2) {
            const uint32_t h0 =
                __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[tm][tn][i] * dd[tn] * gg[tn] * od));
            const uint32_t h1 =
                __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[tm][tn][i + 1] * dd[tn] * gg[tn] * od));
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, true);
            const int lr = 8 * ((i >> 2) & 1) + 4 * (lane >> 5) + (i & 3) + (odd ? 1 : 0);  // row in the 16
            st[lr * 32 + tn * 16 + ((lane & 31) >> 1)] = odd ? (other | (h1 << 16)) : (h0 | (other << 16));
          }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const lm_u32x4 v = ld[j * 64 + lane];
          const int row = tm * 32 + h * 16 + j * 8 + (lane >> 3);
          if (row < t.rows && col < P) *(lm_u32x4*)(out16 + (size_t)(t.m0 + row) * P + col) = v;
        }
        __builtin_amdgcn_wave_barrier();
      }
  }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void* smem) const {
    float* red = (float*)smem;
    float dd[Cfg::TN];
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn)
      dd[tn] = kScaledW ? dsd[(size_t)t.e * P + min(t.n0 + lm_acc_col<Cfg>(wn, tn, lane), P - 1)] : 1.0f;
    lm_tile_row_ssq<Cfg>(acc, wm, wn, lane, P - t.n0, red, [&](float v, int tn, int) { return v * dd[tn]; });
    if ((int)threadIdx.x < t.rows)
      ssq[(size_t)(t.m0 + threadIdx.x) * nt + t.nt] = red[Cfg::WN * Cfg::BM + threadIdx.x];
    // the sums of squares come from the FP32 o; FP16 O rounds o times gamma_e
    // times o_down[e]
    if constexpr (Cfg::WM == 1 && Cfg::TM == 4) {
      if (out16) {
        store16_staged(t, acc, wn, lane, dd, smem);
        return;
      }
    }
    if (out16) {
      // Two columns per 4-byte store: lanes 2m and 2m + 1 hold columns c, c + 1
      // of the same rows; they swap one of each row pair (i, i + 1) (DPP quad
      // permutation 1,0,3,2), so the even lane stores row i and the odd lane
      // row i + 1, both at columns c, c + 1. P is even, so a pair's columns are
      // both inside or both beyond P; every lane takes part in the swap.
      const float od = o_down[t.e];
      const bool odd = lane & 1;
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn) {
        const int col = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
        const bool cok = col < P;
        const float g = cok ? gamma[(size_t)t.e * P + col] : 0.0f;
        _Float16* dst = out16 + (size_t)t.m0 * P + (col & ~1);
#pragma unroll
        for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const uint32_t h0 = __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[tm][tn][i] * dd[tn] * g * od));
            const uint32_t h1 = __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[tm][tn][i + 1] * dd[tn] * g * od));
            const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, true);
            const int row = lm_acc_row<Cfg>(wm, tm, i, lane) + (odd ? 1 : 0);
            if (cok && row < t.rows)
              *(uint32_t*)(dst + (size_t)row * P) = odd ? (other | (h1 << 16)) : (h0 | (other << 16));
          }
      }
      return;
    }
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int col = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
      if (col >= P) continue;
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
          if (row >= t.rows) continue;
          out[(size_t)(t.m0 + row) * P + col] = acc[tm][tn][i] * dd[tn];
        }
    }
  }
};

// ---------------------------------------------------------------- unpooler
// out = y Wun^T. FP16 operands (ds set): W is the FP16 copy scaled per row by
// 2^s and out the accumulator times ds[col] = 2^-s.
template <class Cfg_>
struct UnpoolerProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  const E* y;
  const E* w;
  const float* ds = nullptr;  // [H] or none
  float y_up = 1.0f;          // y is stored times 1 / y_up (a power of two)
  float* out;  // [T, H]
  int T, H, P, mt, nt;

  LM_DEV bool tile(int bid, LmTile& t) const {
    int L;
    if (!lm_xcd_map(bid, mt * nt, L)) return false;
    int m, n;
    lm_dense_order(L, mt, nt, 8, m, n);
    t.m0 = m * Cfg::BM;
    t.rows = min(Cfg::BM, T - t.m0);
    t.n0 = n * Cfg::BN;
    t.nt = n;
    t.e = 0;
    t.kt0 = 0;
    t.kt1 = P / Cfg::KT;
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(y + (size_t)(t.m0 + min(r, t.rows - 1)) * P);
  }
  LM_DEV const lm_u32x4* b_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(w + (size_t)min(t.n0 + r, H - 1) * P);
  }
  LM_DEV const lm_u32x4* b_group(const LmTile& t, int wv, int j) const {
    return lm_packed_group(w, min(t.n0 + (wv * Cfg::TN + j) * 32, H - 32), P);
  }
  LM_DEV int a_ktile(int kt) const { return kt; }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void*) const {
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int col = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
      if (col >= H) continue;
      const float d = (ds ? ds[col] : 1.0f) * y_up;
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
          if (row < t.rows) out[(size_t)(t.m0 + row) * H + col] = acc[tm][tn][i] * d;
        }
    }
  }
};

// ------------------------------------------- split-K dense projections
// For few tokens the pooler / unpooler have too few output tiles to keep the
// chip streaming weights, so K is split and each split writes FP32 partial
// sums part[s][row][col] (times ds[col] where the weights are a per-row
// scaled FP16 copy); a finish kernel adds them in split order.
template <class Cfg_>
struct DenseSplitProb {
  using Cfg = Cfg_;
  using E = typename Cfg::E;
  const E* a;   // [T, K]
  const E* w;   // packed [N, K]
  const float* ds = nullptr;  // [N] or none
  float a_up = 1.0f;          // a is stored times 1 / a_up (a power of two)
  float* part;  // [splits, T, N]
  int T, N, K, mt, nt, splits, kt_per;

  LM_DEV bool tile(int bid, LmTile& t) const {
    int L;
    if (!lm_xcd_map(bid, mt * nt * splits, L)) return false;
    const int s = L / (mt * nt);
    int m, n;
    lm_dense_order(L - s * mt * nt, mt, nt, 8, m, n);
    t.m0 = m * Cfg::BM;
    t.rows = min(Cfg::BM, T - t.m0);
    t.n0 = n * Cfg::BN;
    t.nt = n;
    t.e = s;
    t.kt0 = s * kt_per;
    t.kt1 = min(K / Cfg::KT, t.kt0 + kt_per);
    return true;
  }
  int lda = 0;  // row stride of a in elements (0: K)
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(a + (size_t)(t.m0 + min(r, t.rows - 1)) * (lda ? lda : K));
  }
  LM_DEV const lm_u32x4* b_group(const LmTile& t, int wv, int j) const {
    return lm_packed_group(w, min(t.n0 + (wv * Cfg::TN + j) * 32, N - 32), K);
  }
  LM_DEV int a_ktile(int kt) const { return kt; }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void*) const {
    float* dst = part + ((size_t)t.e * T + t.m0) * N;
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int col = t.n0 + lm_acc_col<Cfg>(wn, tn, lane);
      if (col >= N) continue;
      const float d = (ds ? ds[col] : 1.0f) * a_up;
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
          if (row < t.rows) dst[(size_t)row * N + col] = acc[tm][tn][i] * d;
        }
    }
  }
};

// Sum of p[0], p[stride], ..., p[(splits - 1) stride] in index order, with
// eight loads in flight at a time.
LM_DEV float lm_sum_splits(const float* p, size_t stride, int splits) {
  float v = 0.0f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = p[(size_t)(sp + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) v += x[i];
  }
  for (; sp < splits; ++sp) v += p[(size_t)sp * stride];
  return v;
}

// Pooler finish, one workgroup per (token, 256 columns): h = sum of the
// split partials in split order; pooled32 = gamma_p * h (FP32); the chunk's
// sum of h^2 (fixed tree over the workgroup) goes to ssq[t][chunk], from
// which the row scale is formed exactly as on the unsplit path.
__global__ __launch_bounds__(256) void lm_pool_finish_kernel(const float* part, int splits, int T,
                                                             int P, const float* gamma, float* ssq,
                                                             float* pooled32) {
  __shared__ float red[256];
  const int t = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  const int c = chunk * 256 + tid;
  float h = 0.0f;
  if (c < P) {
    h = lm_sum_splits(part + (size_t)t * P + c, (size_t)T * P, splits);
    pooled32[(size_t)t * P + c] = h * gamma[c];
  }
  red[tid] = h * h;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) ssq[(size_t)t * gridDim.y + chunk] = red[0];
}

// Unpooler finish: out = sum of the split partials, in split order.
__global__ void lm_unpool_finish_kernel(const float* part, int splits, int64_t n, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    out[i] = lm_sum_splits(part + i, (size_t)n, splits);
  }
}

// ------------------------------------------------------------ small kernels

// Largest |v| over n FP32 values (NaN ignored) into out[0]; one workgroup
// (used once, at create, on the norm gammas).
__global__ __launch_bounds__(256) void lm_absmax_kernel(const float* v, int64_t n, float* out) {
  __shared__ float red[256];
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf(v[i]));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
}

// Exact split of FP32 router weights into three BF16 pieces (w = b1 + b2 + b3
// exactly for normal inputs: each remainder is exactly representable and the
// third piece holds at most 8 significant bits). Layout [E, 3H]: piece q of
// row e at columns [q H, (q+1) H).
__global__ void lm_split_router_kernel(const float* w, uint16_t* w3, int E, int H) {
  const size_t n = (size_t)E * H;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t e = i / H, h = i - e * H;
    uint16_t b1, b2, b3;
    lm_split3(w[i], b1, b2, b3);
    uint16_t* row = w3 + e * 3 * (size_t)H;
    row[h] = b1;
    row[H + h] = b2;
    row[2 * H + h] = b3;
  }
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
LM_DEV uint32_t lm_ord(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
LM_DEV float lm_unord(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
LM_DEV uint64_t lm_wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// Router logits and top-k, TPB tokens per workgroup. Phase 1: the k-split
// partial logits of each (token, expert) are summed in a fixed order (FP64),
// the bias added and the sum rounded once to FP32. Four tokens per workgroup
// (256 threads): one thread per (token, expert), splits in index order. One
// token per workgroup (decode sizes, many splits; 1024 threads): Q = 1024 /
// (64 NV) threads per expert, thread q summing the q-th contiguous range of
// splits in index order, then the Q range sums added in q order, so that
// each thread has few loads to wait for. Phase 2: one wavefront per token
// picks the top k by (logit desc, index asc) and takes the softmax over
// them. Routed pairs per expert are counted in an LDS histogram, then one
// integer atomic per expert and workgroup into cpad, where each expert's
// counter sits alone in a 128-byte line (cpad[e * kLmCountStride]) so that
// the atomics of different experts do not queue on a few lines.
constexpr int kLmCountStride = 32;  // ints per padded expert counter
constexpr int kLmMaxK = 32;         // largest top-k the kernels take

// Sum of src[sp * stride] for sp in [lo, hi), in index order, up to 32 loads
// in flight: batches of up to 32 splits, each issued as 32 loads with the
// index clamped to the batch's last split (no load sits behind a branch,
// which would make the compiler wait for all of them at the join) and all
// issued before the first addition (a scheduling barrier; left to itself the
// compiler interleaved the additions and kept a few loads in flight), the
// clamped repeats left out of the sum; a rest of at most four one by one.
LM_DEV double lm_sum_splits_f64(const double* src, size_t stride, int lo, int hi) {
  double sd = 0.0;
  int sp = lo;
  while (hi - sp > 4) {
    const int n = min(32, hi - sp);
    const double* q = src + (size_t)sp * stride;
    double v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = q[(size_t)min(i, n - 1) * stride];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) sd = i < n ? sd + v[i] : sd;
    sp += n;
  }
  for (; sp < hi; ++sp) sd += src[(size_t)sp * stride];
  return sd;
}

template <int NV, int TPB>
__global__ __launch_bounds__((TPB == 1 ? 1024 : 256)) void lm_topk_kernel(
    const double* part, int splits, int T, int E, const float* bias, int k, float* logits, int* ids,
    float* wts, int* cpad) {
  static_assert(TPB == 1 || TPB == 4, "one or four tokens per workgroup");
  constexpr int NTH = TPB == 1 ? 1024 : 256;  // threads (the launch uses the same count)
  constexpr int ES = NV * 64;                         // expert slots (E <= ES)
  constexpr int Q = TPB == 1 ? (NTH / ES > 1 ? NTH / ES : 1) : 1;  // threads per expert
  __shared__ int hist[1024];
  __shared__ float sl[TPB][ES];
  __shared__ double red[TPB == 1 ? NTH : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int t0 = blockIdx.x * TPB;
  const size_t stride = (size_t)T * E;
  for (int i = tid; i < E; i += NTH) hist[i] = 0;
  if constexpr (TPB == 1) {
    const int q = tid / ES, e = tid - q * ES;
    if (e < E && t0 < T)
      red[tid] = lm_sum_splits_f64(part + (size_t)t0 * E + e, stride, q * splits / Q, (q + 1) * splits / Q);
    __syncthreads();
    if (tid < E && t0 < T) {
      double sd = red[tid];
#pragma unroll
      for (int r = 1; r < Q; ++r) sd += red[r * ES + tid];
      if (bias) sd += (double)bias[tid];
      const float v = (float)sd + 0.0f;  // one rounding to FP32; -0 -> +0
      logits[(size_t)t0 * E + tid] = v;
      sl[0][tid] = v;
    }
  } else {
    for (int i = tid; i < TPB * E; i += NTH) {
      const int tt = i / E, e = i - tt * E, t = t0 + tt;
      if (t >= T) continue;
      double sd = lm_sum_splits_f64(part + (size_t)t * E + e, stride, 0, splits);
      if (bias) sd += (double)bias[e];
      const float v = (float)sd + 0.0f;
      logits[(size_t)t * E + e] = v;
      sl[tt][e] = v;
    }
  }
  __syncthreads();
  const int tt = tid >> 6, t = t0 + tt;
  if (tt < TPB && t < T) {
    uint64_t key[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = lane + 64 * v;
      key[v] = e < E ? ((uint64_t)lm_ord(sl[tt][e]) << 32) | (uint32_t)(~(uint32_t)e) : 0;
    }
    // lane j keeps the j-th selection
    float v0 = 0.0f, myv = 0.0f;
    int myi = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < NV; ++v) best = key[v] > best ? key[v] : best;
      best = lm_wave_max_u64(best);
      const int e = (int)(~(uint32_t)best);
      const float val = lm_unord((uint32_t)(best >> 32));
      if (j == 0) v0 = val;
      if (j == lane) {
        myv = val;
        myi = e;
      }
      if ((e & 63) == lane) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (v == (e >> 6)) key[v] = 0;
      }
    }
    // softmax over the selection, the exponentials summed in selection order
    const float ex = expf(myv - v0);
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += __shfl(ex, j, kWave);
    if (lane < k) {
      ids[(size_t)t * k + lane] = myi;
      wts[(size_t)t * k + lane] = ex / sum;
      atomicAdd(&hist[myi], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < E; i += NTH)
    if (hist[i]) atomicAdd(&cpad[i * kLmCountStride], hist[i]);
}

// Exclusive block-wide prefix sum over 256 threads (deterministic).
LM_DEV int lm_block_exscan(int v, int* sbuf, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == 63) sbuf[wave] = inc;
  __syncthreads();
  int woff = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int s = sbuf[w];
    woff += w < wave ? s : 0;
    total += s;
  }
  __syncthreads();
  return woff + inc - v;
}

// One workgroup per expert: its offset and first tile index (prefix over
// lower experts), then a stable scatter of its routed pairs, in (t, j) order,
// into the grouped order. Writes perm_token (grouped row -> token) and
// pair_row (pair t*k+j -> grouped row), and the per-expert counts, from the
// padded counters cpad of the top-k kernel, compactly to counts [E].
__global__ __launch_bounds__(256) void lm_permute_kernel(const int* ids, int npairs, int k,
                                                         const int* cpad, int E, int bm,
                                                         int* counts, int* offsets, int* tile_off,
                                                         int* perm_token, int* pair_row) {
  __shared__ int sbuf[8];
  const int e = blockIdx.x, tid = threadIdx.x;
  int a = 0, b = 0;
  for (int i = tid; i < e; i += 256) {
    const int c = cpad[(size_t)i * kLmCountStride];
    a += c;
    b += (c + bm - 1) / bm;
  }
  int ta, tb;
  lm_block_exscan(a, sbuf, ta);
  lm_block_exscan(b, sbuf, tb);
  const int off = ta, tbase = tb;
  const int cnt = cpad[(size_t)e * kLmCountStride];
  if (tid == 0) {
    counts[e] = cnt;
    offsets[e] = off;
    tile_off[e] = tbase;
    if (e == E - 1) {
      offsets[E] = off + cnt;
      tile_off[E] = tbase + (cnt + bm - 1) / bm;
    }
  }
  if (cnt == 0) return;
  int base = 0;
  for (int start = 0; start < npairs; start += 256 * 16) {
    const int p0 = start + tid * 16;
    // this thread's 16 consecutive ids: four 16-byte loads (ids is 256-byte
    // aligned and p0 a multiple of 16) when all are in range
    int iv[16];
    if (p0 + 16 <= npairs) {
      const lm_u32x4* q = (const lm_u32x4*)(ids + p0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const lm_u32x4 w = q[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) iv[4 * v + i] = (int)w[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) iv[i] = p0 + i < npairs ? ids[p0 + i] : -1;
    }
    unsigned mask = 0;
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool m = iv[i] == e;
      mask |= (unsigned)m << i;
      c += m;
    }
    int total;
    int pos = off + base + lm_block_exscan(c, sbuf, total);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((mask >> i) & 1u) {
        const int p = p0 + i;
        perm_token[pos] = p / k;
        pair_row[p] = pos;
        ++pos;
      }
    }
    base += total;
    if (base >= cnt) break;
  }
}

// p[0] + p[1] + ... + p[n - 1] in FP32, in index order, 16 loads in flight at
// a time (indices clamped to n - 1 so that no load sits behind a branch, and
// all issued before the first addition).
LM_DEV float lm_sum_in_order(const float* p, int n) {
  float s = 0.0f;
  for (int i0 = 0; i0 < n; i0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = p[min(i0 + i, n - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) s = i0 + i < n ? s + v[i] : s;
  }
  return s;
}

// r_t = 1 / sqrt(sum of the row's pooled partial sums of squares / P + eps).
LM_DEV float lm_row_rms_scale(const float* ssq, int nparts, int t, int P, float eps) {
  const float s = lm_sum_in_order(ssq + (size_t)t * nparts, nparts);
  return 1.0f / sqrtf(s / (float)P + eps);
}
__global__ void lm_rowscale_kernel(const float* ssq, int nparts, int T, int P, float eps,
                                   float* rs) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  rs[t] = lm_row_rms_scale(ssq, nparts, t, P, eps);
}

// Pre-expert RMSNorm for FP16 expert inputs, one token row per workgroup: the
// row scale r_t as above, then u = FP16(r_t * pooled32 * down), pooled32 =
// gamma_p * h in FP32. |r_t * pooled32| <= sqrt(P) max|gamma_p|, and down (a
// power of two chosen at create) keeps that bound within 2^15.
__global__ __launch_bounds__(256) void lm_norm_u_kernel(const float* pooled32, const float* ssq,
                                                        int nparts, int P, float eps, float down,
                                                        float* rs, _Float16* u) {
  __shared__ float sr;
  const int t = blockIdx.x;
  if (threadIdx.x == 0) {
    const float r = lm_row_rms_scale(ssq, nparts, t, P, eps);
    sr = r;
    rs[t] = r;
  }
  __syncthreads();
  const float r = sr;
  const float rd = r * down;  // exact: down is a power of two
  const float* src = pooled32 + (size_t)t * P;
  for (int c = threadIdx.x * 8; c < P; c += 256 * 8) {
    const lm_f32x4 a = *(const lm_f32x4*)(src + c) * rd;
    const lm_f32x4 b = *(const lm_f32x4*)(src + c + 4) * rd;
    lm_u32x4 o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(a[2 * q])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(a[2 * q + 1])) << 16);
      o[2 + q] = (uint32_t)__builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(b[2 * q])) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(b[2 * q + 1])) << 16);
    }
    *(lm_u32x4*)(u + (size_t)t * P + c) = o;
  }
}

// One workgroup per token: y = sum over slots j (in order) of
// w_j / sqrt(mean(o_j^2) + eps) * gamma_{e_j} * o_j, in FP32. O is FP32
// (FP32 layers; gamma read here) or FP16 holding gamma_e * o times
// o_down[e] (BF16 layers: the down GEMM applied gamma; o_up[e] = 1 /
// o_down[e] is folded into the slot's coefficient, exactly: a power of two);
// the sums of squares are those of the FP32 o. FP32 layers store y
// [T, P] in FP32, BF16 layers the nearest-even FP16 rounding of y * down, the
// unpooler's operand: |y| <= sqrt(P) max|gamma_e|, and down (a power of two
// chosen at create) keeps that bound within 2^15.
template <typename OT, typename Y>
__global__ __launch_bounds__(256) void lm_combine_kernel(const OT* O, const float* ossq, int nparts,
                                                         const int* pair_row, const int* ids, const float* wts,
                                                         const float* gamma, const float* o_up, int k, int P,
                                                         float eps, float down, Y* y) {
  __shared__ float s_coef[kLmMaxK];
  __shared__ int s_row[kLmMaxK], s_e[kLmMaxK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    const int p = pair_row[(size_t)t * k + tid];
    const int e = ids[(size_t)t * k + tid];
    const float s = lm_sum_in_order(ossq + (size_t)p * nparts, nparts);
    s_coef[tid] = wts[(size_t)t * k + tid] * (1.0f / sqrtf(s / (float)P + eps)) * (o_up ? o_up[e] : 1.0f);
    s_row[tid] = p;
    s_e[tid] = e;
  }
  __syncthreads();
  // Eight-column chunks, two per thread (2048 columns apart) at a time;
  // every column sums its slots in order.
  constexpr int kC = 2;
  for (int c0 = tid * 8; c0 < P; c0 += kC * 2048) {
    lm_f32x4 acc[kC][2];
#pragma unroll
    for (int q = 0; q < kC; ++q) acc[q][0] = acc[q][1] = lm_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (sizeof(OT) == 2) {
      // FP16 O: the chunks of eight slots loaded together (slot and column
      // clamped, so that no load sits behind a branch, and all issued before
      // the first addition), then added in slot order
      constexpr int kS = 8;
      for (int j0 = 0; j0 < k; j0 += kS) {
        lm_u32x4 hv[kS][kC];
#pragma unroll
        for (int jj = 0; jj < kS; ++jj) {
          const OT* orow = O + (size_t)s_row[min(j0 + jj, k - 1)] * P;
#pragma unroll
          for (int q = 0; q < kC; ++q)
            // each expert-output row is read once: streaming (non-temporal) loads
            hv[jj][q] = __builtin_nontemporal_load((const lm_u32x4*)(orow + min(c0 + q * 2048, P - 8)));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < kS; ++jj) {
          if (j0 + jj >= k) break;
          const float cf = s_coef[j0 + jj];
#pragma unroll
          for (int q = 0; q < kC; ++q) {
            lm_f32x4 o[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              o[i >> 1][2 * (i & 1)] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[jj][q][i] & 0xffffu));
              o[i >> 1][2 * (i & 1) + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[jj][q][i] >> 16));
            }
            acc[q][0] += cf * o[0];  // gamma is in O
            acc[q][1] += cf * o[1];
          }
        }
      }
    } else {
    for (int j = 0; j < k; ++j) {
      const OT* orow = O + (size_t)s_row[j] * P;
      const float* grow = gamma + (size_t)s_e[j] * P;
      lm_f32x4 o[kC][2], g[kC][2];
#pragma unroll
      for (int q = 0; q < kC; ++q) {
        const int c = c0 + q * 2048;
        if (c < P) {
          // each expert-output row is read once: streaming (non-temporal) loads
          if constexpr (sizeof(OT) == 4) {
            o[q][0] = __builtin_nontemporal_load((const lm_f32x4*)(orow + c));
            o[q][1] = __builtin_nontemporal_load((const lm_f32x4*)(orow + c + 4));
          } else {
            const lm_u32x4 hv = __builtin_nontemporal_load((const lm_u32x4*)(orow + c));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              o[q][i >> 1][2 * (i & 1)] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[i] & 0xffffu));
              o[q][i >> 1][2 * (i & 1) + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[i] >> 16));
            }
          }
          if constexpr (sizeof(OT) == 4) {
            g[q][0] = *(const lm_f32x4*)(grow + c);
            g[q][1] = *(const lm_f32x4*)(grow + c + 4);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kC; ++q)
        if (c0 + q * 2048 < P) {
          if constexpr (sizeof(OT) == 4) {
            acc[q][0] += s_coef[j] * (g[q][0] * o[q][0]);
            acc[q][1] += s_coef[j] * (g[q][1] * o[q][1]);
          } else {  // gamma is in O
            acc[q][0] += s_coef[j] * o[q][0];
            acc[q][1] += s_coef[j] * o[q][1];
          }
        }
    }
    }
#pragma unroll
    for (int q = 0; q < kC; ++q) {
      const int c = c0 + q * 2048;
      if (c >= P) continue;
      if constexpr (sizeof(Y) == 4) {
        *(lm_f32x4*)((float*)y + (size_t)t * P + c) = acc[q][0];
        *(lm_f32x4*)((float*)y + (size_t)t * P + c + 4) = acc[q][1];
      } else {
        static_assert(std::is_same_v<Y, _Float16>, "FP32 or FP16 y");
        lm_u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t lo = __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[q][i >> 1][2 * (i & 1)] * down));
          const uint16_t hi = __builtin_bit_cast(uint16_t, lm_f32_to_f16_sat(acc[q][i >> 1][2 * (i & 1) + 1] * down));
          v[i] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
        *(lm_u32x4*)((uint16_t*)y + (size_t)t * P + c) = v;
      }
    }
  }
}
