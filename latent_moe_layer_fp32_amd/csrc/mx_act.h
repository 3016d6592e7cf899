// MX activations for the expert GEMMs (gfx950 scaled matrix cores).
//
// The "fp8 x fp4" and "mxfp4 x mxfp4" MMA kinds (web page "SGLang and Miles
// Add Day-0 Support for Muse Spark Open", section "NVFP4 as a third MMA
// kind"): the expert GEMMs read their activations as OCP MX FP8 (E4M3
// elements) or MX FP4 (E2M1 elements, two per byte), one E8M0 scale per 32
// consecutive elements along the reduction axis, against MXFP4 weights, on
// v_mfma_scale_f32_32x32x64_f8f6f4. The pre-expert norm is applied by the
// quantiser (section "Fuse normalization and remove routing conversions"):
// u = r * (gamma_p * h) is formed in FP32 and quantised; a = silu(g) * v is
// quantised in the gate/up epilogue.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 on gfx950 (measured with
// one-hot probes): with K split into two 32-element blocks g = 0, 1,
//   FP4 operand (B, or A with cbsz = 4; 16 bytes per lane): lane 32g + n
//     holds row / column n, block g, element p in nibble p (low nibble
//     first), and supplies that block's scale;
//   FP8 A (32 bytes per lane): lane 32h + m holds row m, bytes 16g .. 16g+15
//     = block g, elements 16h .. 16h+15; the scale of (row m, block g) comes
//     from lane 32g + m whatever lane holds the data.
// The scale operands are dwords; an immediate selects the byte.
// The MXFP4 weight layout (lm_packed_mx_group) already gives each lane one
// 32-element block per 64-wide k-tile; A is staged through LDS in row
// segments of one 128-element k-tile (two MFMA steps): 128 bytes of FP8, of
// which lane half h reads the 16-byte chunks 4s + h and 4s + 2 + h for step s,
// or 64 bytes of FP4, of which it reads chunk 2s + h. Either way lane half h
// supplies the scale of block 2s + h: byte 2s + h of its row's scale dword.
#pragma once
#include "kernels.h"

// ------------------------------------------------------------- MX codecs
// E8M0 exponent of a block: floor(log2(amax)) - emax (the element format's
// largest exponent: 8 for E4M3, 2 for E2M1), clamped to [-127, 127]; an
// all-zero block takes -127.
template <int EMAX>
LM_DEV int lm_mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  (void)frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
  const int s = e - 1 - EMAX;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E4M3 code of q (already divided by the block scale): nearest value, ties to
// the even code, saturating at 448.
LM_DEV uint32_t lm_e4m3_rne(float q) {
  const uint32_t sgn = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (!(a < 448.0f)) return sgn | 0x7Eu;
  uint32_t code;
  if (a < 0.015625f) {  // subnormal: m * 2^-9, m = 8 is the smallest normal
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    int e;
    const float m = frexpf(a, &e);  // a = (2m) * 2^(e-1), 2m in [1, 2)
    uint32_t mm = (uint32_t)rintf((2.0f * m - 1.0f) * 8.0f);
    int be = e - 1 + 7;
    if (mm == 8) {
      mm = 0;
      ++be;
    }
    code = ((uint32_t)be << 3) | mm;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sgn | code;
}

// E2M1 code (sign in bit 3) of q (already divided by the block scale): the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code, saturating
// at 6. Below 1 the grid is the multiples of 0.5 (codes 0, 1, 2: nearest-even
// rounding of 2|q|); from 1 up it is every FP32 value with one mantissa bit,
// so the FP32 bits are rounded to one mantissa bit (nearest, ties to even:
// add just under half a unit, plus the kept bit), clamped at 6.0, and the
// code is the exponent (1 -> 1, 2 -> 2, 4 -> 3) and that bit. No compares:
// a compare's mask feeding a select costs wait states on this chip.
LM_DEV uint32_t lm_e2m1_rne(float q) {
  const float a = fabsf(q);
  const uint32_t lo = (uint32_t)rintf(a * 2.0f);
  uint32_t b = __float_as_uint(a);
  b = (b + 0x1FFFFFu + ((b >> 22) & 1u)) & ~0x3FFFFFu;
  b = min(b, 0x40C00000u);
  const uint32_t hi = (((b >> 23) - 126u) << 1) | ((b >> 22) & 1u);
  return ((__float_as_uint(q) >> 28) & 0x8u) | (a < 1.0f ? lo : hi);
}

// u = r_t * u'_t (u' = gamma_p * Wp x, FP32 [T, P]) quantised to MX FP8
// (BITS = 8: codes [T, P] bytes) or MX FP4 (BITS = 4: codes [T, P/2] bytes,
// element 2i in the low nibble), scales [T, P/32] E8M0 bytes. Eight threads
// per block of 32, four elements each.
template <int BITS>
__global__ __launch_bounds__(256) void lm_quant_u_kernel(const float* pooled, const float* row_scale,
                                                         int T, int P, uint8_t* uq, uint8_t* us) {
  const int64_t nblk = (int64_t)T * (P / 32);
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = gid >> 3;
  const int sub = (int)(gid & 7);
  const bool live = b < nblk;
  const int64_t bb = live ? b : nblk - 1;
  const int64_t t = bb / (P / 32);
  const float r = row_scale[t];
  const float* src = pooled + bb * 32 + sub * 4;
  const lm_f32x4 v = *(const lm_f32x4*)src * r;
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const int se = lm_mx_scale_exp<BITS == 8 ? 8 : 2>(amax);
  uint32_t w = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (BITS == 8) w |= lm_e4m3_rne(ldexpf(v[q], -se)) << (8 * q);
    else w |= lm_e2m1_rne(ldexpf(v[q], -se)) << (4 * q);
  }
  if (live) {
    if constexpr (BITS == 8) *(uint32_t*)(uq + bb * 32 + sub * 4) = w;
    else *(uint16_t*)(uq + bb * 16 + sub * 2) = (uint16_t)w;
    if (sub == 0) us[bb] = (uint8_t)(se + 127);
  }
}

// ------------------------------------------------------------ GEMM problems
// Gate/up on MX u (gathered rows; BITS 8: E4M3 codes [T, P], 4: E2M1 codes
// [T, P/2]) against MXFP4 weights; the epilogue forms a = silu(g) * v in FP32
// and writes it in the same format (codes [pairs, I * BITS / 8], scales
// [pairs, I/32]): the 32 columns of one block are the 32 lanes of a
// half-wave, so the block maximum is a half-wave reduction.
template <class Cfg_, int BITS>
struct GateUpMxaProb : GateUpProb<Cfg_, true> {
  using Base = GateUpProb<Cfg_, true>;
  using Cfg = Cfg_;
  static constexpr int kBits = BITS;
  // FP4 A, 128-row tiles: B one k-tile ahead (the step-ahead A fragments
  // leave no registers for more); see lm_gemm_stream_mxa_kernel
  static constexpr bool kDeepB = false;
  const uint8_t* uq = nullptr;  // [T, P * BITS / 8]
  const uint8_t* us = nullptr;  // [T, P/32] E8M0
  uint8_t* aq = nullptr;        // [pairs, I * BITS / 8]
  uint8_t* as = nullptr;        // [pairs, I/32] E8M0

  LM_DEV bool tile(int bid, LmTile& t) const {
    if (!Base::tile(bid, t)) return false;
    t.kt1 = this->P / 128;  // 128-element k-tiles
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    const int tok = this->perm_token[t.m0 + min(r, t.rows - 1)];
    return (const lm_u32x4*)(uq + (size_t)tok * this->P * BITS / 8);
  }
  // a row's scales sit at 1 / (4 BITS) of its code offset from the bases
  LM_DEV const uint8_t* a_base() const { return uq; }
  LM_DEV const uint8_t* a_scale_base() const { return us; }
  LM_DEV void epilogue(const LmTile& t, const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn,
                       int lane, void*) const {
    const int I = this->I;
    const int col = t.n0 + wn * 32 + (lane & 31);
    // One row block (16 values per lane) at a time, each step applied to all
    // 16 values before the next.
    auto block = [&](int tm, bool full) __attribute__((always_inline)) {
      float a[16], m[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a[i] = lm_silu(acc[tm][0][i]) * acc[tm][1][i];
        m[i] = fabsf(a[i]);
      }
      lm_half_reduce(m, [](float x, float y) { return fmaxf(x, y); });
      uint32_t code[16];
      int se[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        se[i] = lm_mx_scale_exp<BITS == 8 ? 8 : 2>(m[i]);
        code[i] = BITS == 8 ? lm_e4m3_rne(ldexpf(a[i], -se[i])) : lm_e2m1_rne(ldexpf(a[i], -se[i]));
      }
      if constexpr (BITS == 4) {  // columns 2c and 2c+1 (neighbouring lanes) share a byte
#pragma unroll
        for (int i = 0; i < 16; ++i)
          code[i] |= __builtin_bit_cast(uint32_t, lm_dpp<0xB1>(__builtin_bit_cast(float, code[i]))) << 4;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = lm_acc_row<Cfg>(wm, tm, i, lane);
        if (!full && row >= t.rows) continue;
        const size_t pr = (size_t)(t.m0 + row);
        if constexpr (BITS == 8) aq[pr * I + col] = (uint8_t)code[i];
        else if ((lane & 1) == 0) aq[pr * (I / 2) + (col >> 1)] = (uint8_t)code[i];
        if ((lane & 31) == 0) as[pr * (I / 32) + (col >> 5)] = (uint8_t)(se[i] + 127);
      }
    };
    // full tiles store without a row test
    if (t.rows == Cfg::BM) {
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm) block(tm, true);
    } else {
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm) block(tm, false);
    }
  }
};

// Down on MX act (grouped rows) against MXFP4 weights; epilogue as DownProb.
template <class Cfg_, int BITS>
struct DownMxaProb : DownProb<Cfg_, true> {
  using Base = DownProb<Cfg_, true>;
  using Cfg = Cfg_;
  static constexpr int kBits = BITS;
  // FP4 A, 128-row tiles: B three k-tiles ahead (measured 10% faster)
  static constexpr bool kDeepB = true;
  const uint8_t* aq = nullptr;  // [pairs, I * BITS / 8]
  const uint8_t* as = nullptr;  // [pairs, I/32] E8M0

  LM_DEV bool tile(int bid, LmTile& t) const {
    if (!Base::tile(bid, t)) return false;
    t.kt1 = this->I / 128;
    return true;
  }
  LM_DEV const lm_u32x4* a_row(const LmTile& t, int r) const {
    return (const lm_u32x4*)(aq + (size_t)(t.m0 + min(r, t.rows - 1)) * this->I * BITS / 8);
  }
  LM_DEV const uint8_t* a_base() const { return aq; }
  LM_DEV const uint8_t* a_scale_base() const { return as; }
};

// ------------------------------------------------------------------ kernel
// Streaming-B GEMM with MX FP8 or FP4 A and MXFP4 B, four or eight waves side
// by side along N as in lm_gemm_stream_kernel. A k-tile is 128 elements: 128 (FP8) or
// 64 (FP4) bytes per A row (LDS, double buffered, with each row's E8M0 scale
// dword of the k-tile next to it) and two 64-wide MXFP4 k-tiles of B per wave
// group (1 KB each, loaded straight into the MFMA registers); two scaled MFMA
// steps of K = 64.
// Iteration kt:
//   step 0: MFMA(kt,0), each A fragment re-read for step 1 right after its
//           MFMAs | global loads of B(kt+kDistB)
//   barrier: stage (kt+1)&1 (stored in the previous iteration) is visible,
//           every wave has read stage kt&1
//   step 1: MFMA(kt,1) | fragments and A scales of (kt+1, 0) from stage (kt+1)&1
//   store A(kt+2) and its scales into stage kt&1; load A(kt+3); every other
//   k-tile, the B scale dword of the pair of k-tiles starting at kt+kDistB
// The k-tile count is a multiple of 4 (validated on the host) so the ring
// slots and scale byte selectors are compile-time.
template <class Prob>
__global__ __launch_bounds__(64 * Prob::Cfg::WN) __attribute__((amdgpu_waves_per_eu(LM_WAVES_MAX, LM_WAVES_MAX)))
void lm_gemm_stream_mxa_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM == 1 && (Cfg::WN == 4 || Cfg::WN == 8), "streaming-B layout: four or eight waves along N");
  constexpr int TM = Cfg::TM, TN = Cfg::TN, BM = Cfg::BM;
  constexpr bool kA4 = Prob::kBits == 4;
  constexpr int kCh = kA4 ? 4 : 8;     // 16-byte A chunks per row and k-tile
  constexpr int kRows = 64 * Cfg::WN / kCh;  // A rows covered by one load pass
  // B one k-tile ahead (ring of two) for TM = 4; three ahead (ring of four)
  // for decode-sized tiles, whose time goes to streaming the weights.
  // With FP4 A a k-tile holds half the matrix work of an FP8 one, too little
  // to cover a load's latency in one iteration: B then runs three k-tiles
  // ahead and A two iterations ahead of its LDS store (a ring of two slots).
  constexpr bool kLean = TM >= 4 && !(kA4 && Prob::kDeepB);
  constexpr int kRingB = kLean ? 2 : 4, kDistB = kLean ? 1 : 3;
  constexpr bool kNT = TM == 1 && LmWeightsOnce<Prob>::value;  // streaming weight loads
  constexpr int kRingA = 1;
  constexpr int kStage = BM * kCh;  // 16-byte chunks per A stage
  // A chunks per thread per k-tile; with fewer rows than one pass covers
  // (FP4, 32-row tiles) two threads load and store the same chunk
  constexpr int QA = BM >= kRows ? BM / kRows : 1;
  __shared__ lm_u32x4 sa[2 * kStage];
  __shared__ uint32_t ssc[2 * BM];

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int lc = tid % kCh, lr = tid / kCh;
  auto arow = [&](int q) { return (lr + kRows * q) % BM; };
  // LDS row of kCh 16-byte chunks, chunk index XORed so that 16 consecutive
  // rows read at one logical chunk (and the stores of one load pass) fall in
  // 16 distinct 16-byte bank groups
  auto swz = [](int row, int c) {
    if constexpr (kA4) return row * 4 + (c ^ ((row >> 2) & 3));
    else return lm_swz(row, c);
  };

  // A rows; a row's E8M0 scales sit at 1 / (4 BITS) of its code offset from
  // the scale base (K * BITS / 8 bytes of codes, K/32 of scales per row)
  const lm_u32x4* asrc[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) asrc[q] = p.a_row(t, arow(q));
  const uint8_t* const abase = p.a_base();
  const uint8_t* const asbase = p.a_scale_base();
  const lm_u32x4* bsrc[TN];
  const uint32_t* bscl[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    bsrc[j] = p.b_group(t, w, j) + lane;
    bscl[j] = p.b_scales(t, w, j) + lane;
  }

  const int kt0 = t.kt0, kt1 = t.kt1, klast = kt1 - 1;
  lm_u32x4 ra[kRingA][QA];
  uint32_t rsa[kRingA][QA];
  lm_u32x4 rb[kRingB][TN][2];
  uint32_t rsb[2][TN];
  auto load_a = [&](int aslot, int kt) __attribute__((always_inline)) {
    const int ka = min(kt, klast);
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      ra[aslot][q] = asrc[q][ka * kCh + lc];
      const size_t off = (size_t)((const uint8_t*)asrc[q] - abase) >> (kA4 ? 4 : 5);
      rsa[aslot][q] = ((const uint32_t*)(asbase + off))[ka];
    }
  };
  auto store_a = [&](int aslot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      sa[buf * kStage + swz(arow(q), lc)] = ra[aslot][q];
      // the threads of a row hold the same dword: an unconditional store
      // keeps the loop free of branches (which would let the compiler move
      // MFMAs across iterations)
      ssc[buf * BM + arow(q)] = rsa[aslot][q];
    }
  };
  auto load_b = [&](int slot, int kt) __attribute__((always_inline)) {
    const int kc = min(kt, klast);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      rb[slot][j][0] = lm_wload<kNT>(&bsrc[j][(2 * kc) * 64]);
      rb[slot][j][1] = lm_wload<kNT>(&bsrc[j][(2 * kc + 1) * 64]);
    }
  };
  // B scale dword of 64-wide k-tiles 4m .. 4m+3 = 128-wide k-tiles 2m, 2m+1
  auto load_bs = [&](int sslot, int kt) __attribute__((always_inline)) {
    const int kc = min(kt, klast);
#pragma unroll
    for (int j = 0; j < TN; ++j) rsb[sslot][j] = lm_wload<kNT>(&bscl[j][(kc >> 1) * 64]);
  };

  // A fragments, two in flight: fragment (s, i+1) is read while the MFMAs of
  // (s, i) run (ping-pong on i over the whole k-tile sequence); the A scale
  // dwords of the current and next k-tile.
  typedef __attribute__((ext_vector_type(8))) int v8i;
  // FP8: 32 bytes, block 0 elements 16h.., block 1 elements 16h..;
  // FP4: 16 bytes, block h (upper half unused)
  v8i fa[2];
  uint32_t asd[2][TM];
  auto read_frag = [&](int fb, int i, int buf, int s) __attribute__((always_inline)) {
    const lm_u32x4* st = sa + buf * kStage;
    if constexpr (kA4) {
      const lm_u32x4 c = st[swz(i * 32 + r, 2 * s + h)];
      fa[fb] = __builtin_bit_cast(v8i, __builtin_shufflevector(c, c, 0, 1, 2, 3, -1, -1, -1, -1));
    } else {
      const lm_u32x4 c0 = st[swz(i * 32 + r, 4 * s + h)];
      const lm_u32x4 c1 = st[swz(i * 32 + r, 4 * s + 2 + h)];
      fa[fb] = __builtin_bit_cast(v8i, __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // FP4 A: the TM fragments of a whole step are read one step ahead (an FP4
  // step's MFMAs take half the time of an FP8 one, too short to cover an LDS
  // read issued one fragment ahead): f4[step parity][i].
  lm_u32x4 f4[kA4 ? 2 : 1][TM];
  auto read_step4 = [&](int fs, int buf, int s) __attribute__((always_inline)) {
    const lm_u32x4* st = sa + buf * kStage;
#pragma unroll
    for (int i = 0; i < TM; ++i) f4[fs][i] = st[swz(i * 32 + r, 2 * s + h)];
  };
  auto read_scales = [&](int sb, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) asd[sb][i] = ssc[buf * BM + i * 32 + r] >> (8 * h);
  };

  lm_f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto mma = [&](auto sc, auto ob, int fb, int i, int j, int slot, int sbsl, int asl) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    constexpr int opb = decltype(ob)::value;
    const lm_u32x4 b4 = rb[slot][j][s];
    const v8i bv = __builtin_bit_cast(v8i, __builtin_shufflevector(b4, b4, 0, 1, 2, 3, -1, -1, -1, -1));
    v8i av;
    if constexpr (kA4)
      av = __builtin_bit_cast(v8i, __builtin_shufflevector(f4[fb][i], f4[fb][i], 0, 1, 2, 3, -1, -1, -1, -1));
    else
      av = fa[fb];
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], kA4 ? 4 : 0, 4, 2 * s,
                                                                (int)asd[asl][i], opb,
                                                                (int)rsb[sbsl][j]);
  };

  // Prologue: A(kt0), A(kt0+1) in the two stages, B in flight, fragments and
  // scales of (kt0, 0) in registers.
  load_a(0, kt0);
#pragma unroll
  for (int d = 0; d < kDistB; ++d) load_b(d, kt0 + d);
  load_bs(0, kt0);
  if (kDistB >= 2) load_bs(1, kt0 + 2);
  store_a(0, 0);
  load_a(0, kt0 + 1);
  store_a(0, 1);
  load_a(0, kt0 + 2);
  if constexpr (kRingA == 2) load_a(1, kt0 + 3);
  __syncthreads();
  if constexpr (kA4) read_step4(0, 0, 0);
  else read_frag(0, 0, 0, 0);
  read_scales(0, 0);

  // Fragment (s, i) of k-tile kt sits in fa[(2 * TM * kt + s * TM + i) & 1];
  // TM is even or 1, so the parity depends on (s, i) (and, for TM = 1, on s).
  auto iter = [&](int kt, auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;  // kt % 4
    constexpr int cur = q & 1, nxt = cur ^ 1, slot = q % kRingB;
    constexpr int sbs = (q >> 1) & 1;        // B scale slot of this k-tile
    constexpr int ob0 = 2 * (q & 1), ob1 = ob0 + 1;  // B scale bytes of steps 0, 1
    load_b((q + kDistB) % kRingB, kt + kDistB);
    if constexpr (kA4) {
      // step 0: MFMAs of step 0 (f4[0]) while step 1 is read from this stage
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          mma(std::integral_constant<int, 0>{}, std::integral_constant<int, ob0>{}, 0, i, j, slot, sbs, cur);
        f4[1][i] = sa[cur * kStage + swz(i * 32 + r, 2 + h)];
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x020, (TN * 2 + TM - 1) / TM, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
      // barrier: every wave has read this stage (it is overwritten below) and
      // the next stage, stored in the previous iteration, is visible
      __syncthreads();
      read_scales(nxt, nxt);
      // step 1: MFMAs of step 1 (f4[1]) while step 0 of kt+1 is read
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          mma(std::integral_constant<int, 1>{}, std::integral_constant<int, ob1>{}, 1, i, j, slot, sbs, cur);
        f4[0][i] = sa[nxt * kStage + swz(i * 32 + r, h)];
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
    // step 0: MFMAs of (0, i) while (0, i+1), then (1, 0), are read
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int fb = i & 1;
#pragma unroll
      for (int j = 0; j < TN; ++j)
        mma(std::integral_constant<int, 0>{}, std::integral_constant<int, ob0>{}, fb, i, j, slot, sbs, cur);
      if (i + 1 < TM) read_frag(fb ^ 1, i + 1, cur, 0);
      else read_frag(fb ^ 1, 0, cur, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);            // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, kA4 ? 1 : 2, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x020, (TN * 2 + TM - 1) / TM, 0);  // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 1: MFMAs of (1, i) while (1, i+1) are read; the last fragment of
    // the k-tile and the scales of kt+1 come from the next stage, after the
    // barrier (which also frees this stage for the store below)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int fb = (TM + i) & 1;
      if (i + 1 == TM) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        read_scales(nxt, nxt);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
        mma(std::integral_constant<int, 1>{}, std::integral_constant<int, ob1>{}, fb, i, j, slot, sbs, cur);
      if (i + 1 < TM) read_frag(fb ^ 1, i + 1, cur, 1);
      else read_frag(fb ^ 1, 0, nxt, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kA4 ? 1 : 2, 0);
    }
    }
    __builtin_amdgcn_sched_barrier(0);
    // A(kt+2) (slot cur with a ring of two) into the stage just consumed; the
    // next load into that slot is A(kt + 2 + kRingA)
    store_a(kRingA == 2 ? cur : 0, cur);
    load_a(kRingA == 2 ? cur : 0, kt + 2 + kRingA);
    // B scales of the pair starting at k-tile kt+kDistB; its slot's previous
    // pair (k-tiles up to kt) is done with
    if constexpr (((q + kDistB) & 1) == 0) load_bs(((q + kDistB) >> 1) & 1, kt + kDistB);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = kt0; kt < kt1; kt += 4) {
    iter(kt, std::integral_constant<int, 0>{});
    iter(kt + 1, std::integral_constant<int, 1>{});
    iter(kt + 2, std::integral_constant<int, 2>{});
    iter(kt + 3, std::integral_constant<int, 3>{});
  }
  __syncthreads();
  p.epilogue(t, acc, 0, w, lane, (void*)sa);
}
