// Streaming-B matrix-core GEMM for gfx950 (BF16 or FP16 operands, FP32
// accumulation).
//
// Same problem interface and accumulator layout as lm_gemm_kernel, with all
// four (or eight) wavefronts side by side along N (WM = 1): every wave needs
// the whole A tile and its own 32*TN rows of B, so
//   * A (activations) is staged through LDS: loaded into registers four
//     k-tiles ahead, written to the LDS double buffer two k-tiles ahead, and
//     read into fragment registers one MFMA step ahead;
//   * B (weights) is loaded from global memory straight into the registers
//     the MFMA reads, one or three k-tiles ahead, and never touches LDS. The
//     weights are stored in a matrix-core packed layout (lm_packed_group,
//     lm_packed_mx_group), so each such load reads 1 KB of contiguous memory
//     per wave: loading the row-major layout straight into MFMA registers
//     would touch 32 cache lines per instruction and throttle the vector
//     memory path. MXFP4 weights arrive as E2M1 codes plus E8M0 scales and
//     are decoded exactly to FP16 in registers right before their MFMA, each
//     weight row times its power of two 2^s (chosen at create so that the
//     row's largest value lands in [2^14, 2^15)); the epilogue multiplies
//     the row's output column by 2^-s.
// Per 64-wide k-tile a wave issues TM*TN*4 32x32x16 MFMAs and reads
// only A from LDS: with TM = 4 that is about 64 B/clk/CU of LDS reads at full
// matrix rate, against ~135 B/clk measured on MI355X, where a 64x64 wave tile
// reading both operands from LDS needs twice that and becomes LDS-bound. Eight
// waves along N share each A tile twice as widely: the same LDS reads per
// MFMA, half the A loads per MFMA.
//
// The K bijection: lane half h (lane / 32) at step s consumes the 16-byte
// chunk 4h + s of the 128-byte k-tile row, for A and B alike, so each lane
// streams 64 contiguous bytes of its B row per k-tile.
#pragma once
#include <type_traits>

#include "gemm.h"

#ifndef LM_WAVES_MAX
#define LM_WAVES_MAX 2
#endif

// Problems whose expert weights are MXFP4 declare kMx = true.
template <class P, class = void>
struct LmIsMx : std::false_type {};
template <class P>
struct LmIsMx<P, std::void_t<decltype(P::kMx)>> : std::integral_constant<bool, P::kMx> {};

// E8M0 scale code times 2^s as FP32: 2^(code - 127 + s) (code 0 is 2^-127,
// code 255 is NaN). The callers keep code + s <= 254; below the normal range
// the scale is 0 (such a block is over 2^100 below its row's largest).
LM_DEV float lm_e8m0_shifted(uint32_t code, int s) {
  const int ex = (int)code + s;
  return code == 255 ? __uint_as_float(0x7fc00000u) : ex >= 1 ? __uint_as_float((uint32_t)ex << 23) : 0.0f;
}

// The register budget allows two waves per SIMD: two four-wave workgroups
// per CU, or one eight-wave workgroup (see kLeanA, kLeanB below).
// Decode-sized tiles with MXFP4 weights need fewer registers (a quarter of
// the B bytes per k-tile) and run LM_MX_NARROW_WAVES waves per SIMD (three
// measured about 1% faster at decode than two, four no faster than three).
#ifndef LM_MX_NARROW_WAVES
#define LM_MX_NARROW_WAVES 3
#endif
template <class Prob>
struct LmWavesPerEu
    : std::integral_constant<int, Prob::Cfg::TM == 1 && LmIsMx<Prob>::value ? LM_MX_NARROW_WAVES : LM_WAVES_MAX> {};

template <class Prob>
__global__ __launch_bounds__(64 * Prob::Cfg::WN)
__attribute__((amdgpu_waves_per_eu(LmWavesPerEu<Prob>::value, LmWavesPerEu<Prob>::value)))
void lm_gemm_stream_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM == 1 && (Cfg::WN == 4 || Cfg::WN == 8), "streaming-B layout: four or eight waves along N");
  static_assert(sizeof(typename Cfg::E) == 2, "16-bit operands");
  constexpr bool kMx = LmIsMx<Prob>::value;
  static_assert(!kMx || std::is_same_v<typename Cfg::E, _Float16>, "MXFP4 weights decode to FP16");
  constexpr int TM = Cfg::TM, TN = Cfg::TN, BM = Cfg::BM;
  // A (TM = 4): one register slot; A(kt+3) is loaded right after A(kt+2)
  // has been written to LDS at the end of iteration kt, so it has a whole
  // iteration in flight, and since vmcnt retires in issue order, the store
  // that waits for it does not also wait for the B loads issued after it.
  // A (TM < 4, decode-sized tiles): loaded four k-tiles ahead into a ring of
  // four; A(kt+2) is written to LDS at iteration kt and waits only on loads
  // issued two iterations earlier. B: one k-tile ahead in a ring of two for
  // 16-bit weights with TM = 4 (small enough for two waves per SIMD to hide
  // each other's latency); otherwise (few B registers: narrow tiles, MXFP4
  // codes) three ahead in a ring of four.
  constexpr bool kLeanA = TM >= 4;
  constexpr bool kLeanB = kLeanA && !kMx;
  constexpr int kRingA = kLeanA ? 2 : 4, kRingB = kLeanB ? 2 : 4;
  constexpr int kDistB = kLeanB ? 1 : 3, kDistA = kLeanA ? 2 : 4;
  constexpr int kBq = kMx ? 1 : 4;  // 16-byte B loads per 32-row group and k-tile
  constexpr bool kNT = TM == 1 && LmWeightsOnce<Prob>::value;  // streaming weight loads
  constexpr int NT = 64 * Cfg::WN;  // threads
  constexpr int RS = NT / 8;        // A rows per pass of the workgroup (8 chunks per row)
  constexpr int kStage = BM * 8;    // 16-byte chunks per A stage
  constexpr int QA = BM * 8 / NT;   // A chunks per thread per k-tile
  __shared__ lm_u32x4 sa[2 * kStage];

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  float rowv = 0.0f;
  if constexpr (LmHasRowValue<Prob>::value)
    if (tid < BM) rowv = p.row_value(t, tid);
  const int lc = tid & 7, lr = tid >> 3;

  // A: thread loads chunk lc of tile rows lr + RS q.
  const lm_u32x4* asrc[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) asrc[q] = p.a_row(t, lr + RS * q);
  // B: wave w's j-th 32-row group in the packed layout. 16-bit weights: the
  // fragment of step s of k-tile kt is 1 KB at (kt*4*8 + s)*64 chunks (eight
  // groups interleaved per k-tile). MXFP4: all four
  // steps of k-tile kt are 1 KB at kt*64 chunks, scales a dword per lane per
  // four k-tiles.
  const lm_u32x4* bsrc[TN];
  const uint32_t* ssrc[TN];
  int bsh[TN];  // MXFP4: the shift s of the lane's weight row (from its 2^-s)
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    bsrc[j] = p.b_group(t, w, j) + lane;
    if constexpr (kMx) {
      ssrc[j] = p.b_scales(t, w, j) + lane;
      bsh[j] = -lm_log2_of_pow2(p.b_descale(t, w, j)[lane & 31]);
    }
  }

  const int kt0 = t.kt0, kt1 = t.kt1, klast = kt1 - 1;
  // Register rings: slot q holds A / B of the k-tile with kt % ring == q
  // (A with TM = 4 uses slot 0 past the prologue); MXFP4 scale dwords
  // alternate per four k-tiles.
  lm_u32x4 ra[kRingA][QA], rb[kRingB][TN][kBq];
  uint32_t rsc[2][TN];
  auto load_a = [&](int slot, int kt) {
    const int ka = p.a_ktile(min(kt, klast));
#pragma unroll
    for (int q = 0; q < QA; ++q) ra[slot][q] = asrc[q][ka * 8 + lc];
  };
  auto store_a = [&](int slot, int buf) {
#pragma unroll
    for (int q = 0; q < QA; ++q) sa[buf * kStage + lm_swz(lr + RS * q, lc)] = ra[slot][q];
  };
  auto load_b = [&](int slot, int kt) {
    const int kc = lm_b_ktile(p, min(kt, klast));
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (kMx) {
        rb[slot][j][0] = lm_wload<kNT>(&bsrc[j][kc * 64]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          rb[slot][j][s] = lm_wload<kNT>(&bsrc[j][(kc * 4 * kLmPackGroups + s) * 64]);
      }
    }
  };
  auto load_scales = [&](int sslot, int kt) {
    if constexpr (kMx) {
      const int kc4 = min(kt, klast) >> 2;
#pragma unroll
      for (int j = 0; j < TN; ++j) rsc[sslot][j] = lm_wload<kNT>(&ssrc[j][kc4 * 64]);
    }
  };
  // A fragments of one MFMA step, double-buffered across steps.
  lm_u32x4 fa[2][TM];
  auto read_frag = [&](int fb, int buf, int s) {
    const lm_u32x4* st = sa + buf * kStage;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[fb][i] = st[lm_swz(i * 32 + r, 4 * h + s)];
  };

  lm_f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // B fragment of step s: 16-bit weights straight from the ring; MXFP4
  // decoded here to FP16, exactly (every E2M1 value x 2^(e - 127 + s) is an
  // FP16 number unless the block's scale is over 2^35 below the row's
  // largest), one code pair per conversion (v_cvt_scalef32_pk_f16_fp4).
  auto b_frag = [&](int slot, int j, int s, int sq, int kb) -> lm_u32x4 {
    if constexpr (kMx) {
      const uint32_t codes = rb[slot][j][0][s];
      const float scale = lm_e8m0_shifted((rsc[sq][j] >> (8 * kb)) & 0xffu, bsh[j]);
      lm_u32x4 f;
      f[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0));
      f[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1));
      f[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2));
      f[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3));
      return f;
    } else {
      return rb[slot][j][s];
    }
  };
  auto mma_step = [&](int fb, int slot, int s, int sq, int kb) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const lm_u32x4 bf = b_frag(slot, j, s, sq, kb);
#pragma unroll
      for (int i = 0; i < TM; ++i) LmElem<typename Cfg::E>::mma(acc[i][j], fa[fb][i], bf);
    }
  };
  // Interleave within a step: the step's TM*TN MFMAs with the TM LDS reads
  // of the next step (and, where given, global loads), so LDS and memory
  // latency hide behind the matrix pipe instead of in front of it.
  auto pattern = [&](auto with_vmem) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      if constexpr (decltype(with_vmem)::value)
        __builtin_amdgcn_sched_group_barrier(0x020, ((kLeanA ? 0 : QA) + TN * kBq + TM - 1) / TM, 0);  // VMEM read
    }
  };

  // Prologue: the first k-tiles in flight, A(kt0) and A(kt0+1) in the two LDS
  // stages, step 0 of kt0 in registers.
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if (d < kDistB) load_b(d, kt0 + d);
    if (d < (kLeanA ? 2 : kDistA)) load_a(d, kt0 + d);
  }
  load_scales(0, kt0);
  store_a(0, 0);
  store_a(1, 1);
  if constexpr (kLeanA) load_a(0, kt0 + 2);
  __syncthreads();
  read_frag(0, 0, 0);

  // Iteration kt (q = kt % 8). On entry LDS stage kt&1 holds A(kt), stage
  // (kt+1)&1 holds A(kt+1), fa[0] holds the fragments of (kt, step 0).
  //   step 0: MFMA(kt,0) | LDS reads (kt,1) | global loads of B(kt+kDistB),
  //           A(kt+4) (TM < 4) and, every fourth k-tile, MXFP4 scales
  //   step 1: MFMA(kt,1) | LDS reads (kt,2)
  //   step 2: MFMA(kt,2) | LDS reads (kt,3)
  //   barrier: every wave's reads of stage kt&1 are done, and A(kt+1)
  //            (stored in the previous iteration) is visible
  //   step 3: MFMA(kt,3) | LDS reads (kt+1,0) from stage (kt+1)&1
  //   store A(kt+2) into stage kt&1 (published by the next iteration's
  //   barrier, before its step 3 reads it); TM = 4: load A(kt+3)
  // One barrier per k-tile, and the matrix pipe never waits for LDS data
  // issued in the same step. The k-tile count is a multiple of 8 and kt0 a
  // multiple of 8 (validated on the host), so ring slots are compile-time;
  // indices past the end are clamped: those loads are issued but unused.
  auto iter = [&](int kt, auto qc) {
    constexpr int q = decltype(qc)::value;
    constexpr int cur = q & 1, nxt = cur ^ 1, slot = q % kRingB;
    constexpr int sq = (q >> 2) & 1, kb = q & 3;
    read_frag(1, cur, 1);
    load_b((q + kDistB) % kRingB, kt + kDistB);
    if constexpr ((q + kDistB) % 4 == 0) load_scales(((q + kDistB) >> 2) & 1, kt + kDistB);
    if constexpr (!kLeanA) load_a((q + kDistA) % kRingA, kt + kDistA);
    mma_step(0, slot, 0, sq, kb);
    pattern(std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    read_frag(0, cur, 2);
    mma_step(1, slot, 1, sq, kb);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    read_frag(1, cur, 3);
    mma_step(0, slot, 2, sq, kb);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frag(0, nxt, 0);
    mma_step(1, slot, 3, sq, kb);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    store_a(kLeanA ? 0 : (q + 2) % kRingA, cur);
    if constexpr (kLeanA) load_a(0, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = kt0; kt < kt1; kt += 8) {
    iter(kt, std::integral_constant<int, 0>{});
    iter(kt + 1, std::integral_constant<int, 1>{});
    iter(kt + 2, std::integral_constant<int, 2>{});
    iter(kt + 3, std::integral_constant<int, 3>{});
    iter(kt + 4, std::integral_constant<int, 4>{});
    iter(kt + 5, std::integral_constant<int, 5>{});
    iter(kt + 6, std::integral_constant<int, 6>{});
    iter(kt + 7, std::integral_constant<int, 7>{});
  }
  __syncthreads();
  if constexpr (LmHasRowValue<Prob>::value) {
    if (tid < BM) ((float*)sa)[tid] = rowv;
    __syncthreads();
  }
  p.epilogue(t, acc, 0, w, lane, (void*)sa);
}
