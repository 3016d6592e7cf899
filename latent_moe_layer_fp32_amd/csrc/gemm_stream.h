// Streaming-B matrix-core GEMM for gfx950 (BF16 operands, FP32 accumulation).
//
// Same problem interface and accumulator layout as lm_gemm_kernel, with all
// four wavefronts side by side along N (WM = 1): every wave needs the whole
// A tile and its own 32*TN rows of B, so
//   * A (activations) is staged through LDS: loaded into registers four
//     k-tiles ahead, written to the LDS double buffer two k-tiles ahead, and
//     read into fragment registers one MFMA step ahead;
//   * B (weights) is loaded from global memory straight into the registers
//     the MFMA reads, three k-tiles ahead, and never touches LDS. The weights are
//     stored in a matrix-core packed layout (lm_packed_group), so each such
//     load reads 1 KB of contiguous memory per wave: loading the row-major
//     layout straight into MFMA registers would touch 32 cache lines per
//     instruction and throttle the vector memory path.
// Per 64-wide k-tile a wave issues TM*TN*4 v_mfma_f32_32x32x16_bf16 and reads
// only A from LDS: with TM = 4 that is about 64 B/clk/CU of LDS reads at full
// matrix rate, against ~135 B/clk measured on MI355X, where a 64x64 wave tile
// reading both operands from LDS needs twice that and becomes LDS-bound.
//
// The K bijection: lane half h (lane / 32) at step s consumes the 16-byte
// chunk 4h + s of the 128-byte k-tile row, for A and B alike, so each lane
// streams 64 contiguous bytes of its B row per k-tile.
#pragma once
#include <type_traits>

#include "gemm.h"

// Global prefetch distances in k-tiles. Deep (TM < 4, few accumulators: the
// decode-sized tiles that only stream weights): B 3 ahead, A 4 ahead (A(kt+2)
// is written to LDS at iteration kt; since vmcnt retires in issue order, that
// store then waits only on loads issued two iterations earlier), register
// rings of four k-tiles. Lean (TM = 4): B 1 ahead, A loaded and written
// within the iteration, rings of two, small enough for two workgroups per CU
// to hide each other's latency.
#ifndef LM_WAVES_MAX
#define LM_WAVES_MAX 2
#endif

// One workgroup per CU is intended (the accumulators alone take 128 AGPRs at
// TM = 4), so let the compiler use the whole register file.
template <class Prob>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LM_WAVES_MAX, LM_WAVES_MAX)))
void lm_gemm_stream_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM == 1 && Cfg::WN == 4, "streaming-B layout: four waves along N");
  static_assert(sizeof(typename Cfg::E) == 2, "BF16 operands");
  constexpr int TM = Cfg::TM, TN = Cfg::TN, BM = Cfg::BM;
  constexpr bool kLean = TM >= 4;
  constexpr int kRing = kLean ? 2 : 4;
  constexpr int kDistB = kLean ? 1 : 3, kDistA = kLean ? 2 : 4;
  constexpr int kStage = BM * 8;  // 16-byte chunks per A stage
  constexpr int QA = BM * 8 / 256;  // A chunks per thread per k-tile (= TM)
  __shared__ lm_u32x4 sa[2 * kStage];

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int lc = tid & 7, lr = tid >> 3;

  // A: thread loads chunk lc of tile rows lr + 32 q.
  const lm_u32x4* asrc[QA];
#pragma unroll
  for (int q = 0; q < QA; ++q) asrc[q] = p.a_row(t, lr + 32 * q);
  // B: wave w's j-th 32-row group in the matrix-core packed layout; the
  // fragment of step s of k-tile kt is 1 KB at (kt*4 + s)*64 chunks.
  const lm_u32x4* bsrc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bsrc[j] = p.b_group(t, w, j) + lane;

  const int kt0 = t.kt0, kt1 = t.kt1, klast = kt1 - 1;
  // Register rings: slot q holds A / B of the k-tile with kt % kRing == q
  // (lean: A uses slot 0 only).
  lm_u32x4 ra[kRing][QA], rb[kRing][TN][4];
  auto load_a = [&](int slot, int kt) {
    const int ka = p.a_ktile(min(kt, klast));
#pragma unroll
    for (int q = 0; q < QA; ++q) ra[slot][q] = asrc[q][ka * 8 + lc];
  };
  auto store_a = [&](int slot, int buf) {
#pragma unroll
    for (int q = 0; q < QA; ++q) sa[buf * kStage + lm_swz(lr + 32 * q, lc)] = ra[slot][q];
  };
  auto load_b = [&](int slot, int kt) {
    const int kc = min(kt, klast);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) rb[slot][j][s] = bsrc[j][(kc * 4 + s) * 64];
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

  auto mma_step = [&](int fb, int slot, int s) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) LmElem<uint16_t>::mma(acc[i][j], fa[fb][i], rb[slot][j][s]);
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
        __builtin_amdgcn_sched_group_barrier(0x020, (QA + 4 * TN) / TM, 0);  // VMEM read
    }
  };

  // Prologue: B(kt0 .. kt0+2) and A(kt0 .. kt0+3) in flight, A(kt0) and
  // A(kt0+1) in the two LDS stages, step 0 of kt0 in registers.
  if constexpr (kLean) {
    load_b(0, kt0);
    load_a(0, kt0);
    load_a(1, kt0 + 1);
  } else {
#pragma unroll
    for (int d = 0; d < kDistA; ++d) {
      if (d < kDistB) load_b(d, kt0 + d);
      load_a(d, kt0 + d);
    }
  }
  store_a(0, 0);
  store_a(1, 1);
  __syncthreads();
  read_frag(0, 0, 0);

  // Iteration kt. On entry LDS stage kt&1 holds A(kt), stage (kt+1)&1 holds
  // A(kt+1), fa[0] holds the fragments of (kt, step 0).
  //   step 0: MFMA(kt,0) | LDS reads (kt,1) | global loads B(kt+3), A(kt+4)
  //   step 1: MFMA(kt,1) | LDS reads (kt,2)
  //   step 2: MFMA(kt,2) | LDS reads (kt,3)
  //   barrier: every wave's reads of stage kt&1 are done, and A(kt+1)
  //            (stored in the previous iteration) is visible
  //   step 3: MFMA(kt,3) | LDS reads (kt+1,0) from stage (kt+1)&1
  //   store A(kt+2) into stage kt&1 (published by the next iteration's
  //   barrier, before its step 3 reads it)
  // One barrier per k-tile, and the matrix pipe never waits for LDS data
  // issued in the same step.
  auto iter = [&](int kt, int q) {
    const int cur = q & 1, nxt = cur ^ 1;
    read_frag(1, cur, 1);
    load_b((q + kDistB) % kRing, kt + kDistB);
    load_a(kLean ? 0 : (q + kDistA) % kRing, kt + kDistA);
    mma_step(0, q % kRing, 0);
    pattern(std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    read_frag(0, cur, 2);
    mma_step(1, q % kRing, 1);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    read_frag(1, cur, 3);
    mma_step(0, q % kRing, 2);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frag(0, nxt, 0);
    mma_step(1, q % kRing, 3);
    pattern(std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    store_a(kLean ? 0 : (q + 2) % kRing, cur);
  };
  for (int kt = kt0; kt < kt1; kt += 4) {
    iter(kt, 0);
    iter(kt + 1, 1);
    iter(kt + 2, 2);
    iter(kt + 3, 3);
  }
  __syncthreads();
  p.epilogue(t, acc, 0, w, lane, (void*)sa);
}
