// LDS-staged matrix-core GEMM for gfx950 with direct global->LDS loads
// (16-bit operands, FP32 accumulation): the prefill-sized expert and dense
// projection GEMMs.
//
// One workgroup of eight wavefronts per CU computes a 256 x 256 output tile:
// two row bands (wm) of four waves (wn), each wave 128 x 64 (TM = 4 row
// blocks x TN = 2 column blocks of 32 x 32). Both operands of a tile are
// shared: every A byte serves four waves and every B byte two, so per
// multiply-add the tile moves a fifth fewer bytes from L2 than a 128 x 512
// tile whose waves each stream their own weight rows, and none of it through
// vector registers.
//
// Operands go global -> LDS with global_load_lds_dwordx4: each instruction
// moves 1 KB per wave, lane L's 16 bytes landing at byte 16 L of the
// destination, from any per-lane global address. A stage is one 64-wide
// k-tile (128 bytes of every row):
//   * A: 256 rows x 128 bytes, row-major with the chunks of row R permuted by
//     (R / 2) % 8 (lm_swz: conflict-free fragment reads). An instruction loads
//     8 whole rows, 8 lanes per row, so each gathered row is one coalesced
//     128-byte line (fetching fragments lane-wise instead touches 32 lines per
//     instruction and re-fetches each line from L2 four times).
//   * B: from the packed weight layout, where the fragment of one MFMA step
//     of a 32-row group is already 1 KB of contiguous memory; stored in that
//     order, so lane L reads its operand at 16 L.
//
// Pipeline: two stages (2 x 64 KB of LDS) in two distinct LDS arrays. At
// k-tile i a wave waits for its own loads of k-tile i (s_waitcnt vmcnt), a
// barrier makes every wave's loads visible and frees the buffer read at
// k-tile i - 1, the loads of k-tile i + 1 go into that buffer, and the
// k-tile's MFMAs run with their fragments read one step ahead. The barrier is
// the bare s_barrier: __syncthreads' fence would also wait for the loads
// still in flight. Distinct arrays per stage let the compiler see that the
// loads in flight never alias the buffer being read, so it adds no waits of
// its own.
//
// A row band whose rows all lie beyond the tile's valid rows (the last tile
// of an expert with at most 128 rows) skips its reads and MFMAs; its waves
// still load their share of the operands and join every barrier.
//
// Built only with LM_LDS_GEMM=1. On the 16384-token prefill it runs the
// gate/up GEMM in 9.4 ms against 8.8 ms for the streaming kernel: the clock
// it holds is higher (1.6 against 1.5 GHz) but the matrix cores are busy
// 59% of the time against 65-70%, the barrier per k-tile and the LDS
// fragment reads costing more than the L2 bytes it saves.
#pragma once
#include <type_traits>

#include "gemm.h"

// Problems whose B tile holds paired rows (gate/up: LDS groups 0..WN-1 gate
// rows, WN..2WN-1 the up rows of the same columns) declare kPairedB.
template <class P, class = void>
struct LmPairedB : std::false_type {};
template <class P>
struct LmPairedB<P, std::void_t<decltype(P::kPairedB)>> : std::integral_constant<bool, P::kPairedB> {};

#define LM_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt at their
// maxima, i.e. not waited on): gfx9 encoding, vmcnt in bits 3:0 and 15:14.
template <int N>
LM_DEV void lm_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <class Prob>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lm_gemm_lds_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM == 2 && Cfg::WN == 4 && Cfg::TM == 4 && Cfg::TN == 2, "256 x 256 tiles of eight waves");
  static_assert(sizeof(typename Cfg::E) == 2, "16-bit operands");
  static_assert(!LmHasRowValue<Prob>::value, "row values are not staged by this kernel");
  constexpr int TM = Cfg::TM, TN = Cfg::TN, WN = Cfg::WN;
  constexpr bool kPaired = LmPairedB<Prob>::value;
  constexpr int kFrag = 64;           // 16-byte chunks per fragment (1 KB)
  constexpr int kHalf = 256 * 8;      // chunks of A (or B) per stage: 256 rows x 8 chunks
  constexpr int kDma = 8;             // loads per wave per stage: 4 of A, 4 of B
  __shared__ lm_u32x4 st0[2 * kHalf];
  __shared__ lm_u32x4 st1[2 * kHalf];

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WN, wn = w % WN;
  const int h = lane >> 5, r = lane & 31;
  // loads: wave w fetches A rows 32 w .. 32 w + 31 (8 rows per instruction,
  // lane L: row 8 j + L / 8, LDS slot L % 8 holding chunk (L % 8) ^ swz) and
  // the four step fragments of B group w
  const lm_u32x4* arow[4];
  int achunk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = w * 32 + 8 * j + (lane >> 3);
    arow[j] = p.a_row(t, row);
    achunk[j] = (lane & 7) ^ ((row >> 1) & 7);
  }
  const lm_u32x4* bgrp = (kPaired ? p.b_group(t, w % WN, w / WN) : p.b_group(t, w / TN, w % TN)) + lane;
  // compute: wave (wm, wn) reads A blocks 4 wm + i and B groups lg[j]
  int lg[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) lg[j] = kPaired ? j * WN + wn : wn * TN + j;
  // this band holds valid rows (wave-uniform: a scalar branch, not an exec mask)
  const bool live = __builtin_amdgcn_readfirstlane((int)(wm * TM * 32 < t.rows)) != 0;

  const int kt0 = t.kt0;
  const int nkt = t.kt1 - t.kt0;  // k-tiles (a multiple of 2)

  auto stage_buf = [&](auto qc) -> lm_u32x4* {
    if constexpr (decltype(qc)::value == 0) return st0;
    else return st1;
  };
  // loads of k-tile i (clamped to the last: a load past the end refetches it
  // into a buffer nobody reads again, so every stage issues the same count),
  // in four parts of two (A rows 8 j.., B step j) so that they can be spread
  // between the MFMAs of the k-tile before
  auto issue_part = [&](auto qc, int i, int j) {
    lm_u32x4* buf = stage_buf(qc);
    const int kt = kt0 + min(i, nkt - 1);
    const int ka = p.a_ktile(kt), kb = lm_b_ktile(p, kt);
    __builtin_amdgcn_global_load_lds((const void*)(arow[j] + ka * 8 + achunk[j]),
                                     LM_LDS_PTR(buf + (w * 32 + 8 * j) * 8), 16, 0, 0);
    // the packed fragment of step j (eight groups interleaved per k-tile)
    __builtin_amdgcn_global_load_lds((const void*)(bgrp + (kb * 4 * kLmPackGroups + j) * kFrag),
                                     LM_LDS_PTR(buf + kHalf + (w * 4 + j) * kFrag), 16, 0, 0);
  };
  auto issue = [&](auto qc, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_part(qc, i, j);
  };

  lm_f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Fragments alternate between two register sets by step parity. The MFMAs
  // run one step behind the reads: the first reads of a k-tile go out right
  // after its barrier together with the MFMAs of the previous k-tile's last
  // step (whose fragments were read before the barrier), so the matrix pipe
  // has work while they are in flight.
  lm_u32x4 fa[2][TM], fb[2][TN];
  auto read_frags = [&](const lm_u32x4* buf, int fbuf, int s) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[fbuf][i] = buf[lm_swz((wm * TM + i) * 32 + r, 4 * h + s)];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[fbuf][j] = buf[kHalf + (lg[j] * 4 + s) * kFrag + lane];
  };
  auto mma = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) LmElem<typename Cfg::E>::mma(acc[i][j], fa[fbuf][i], fb[fbuf][j]);
  };
  // one step: this step's TM + TN fragment reads and two loads of the next
  // k-tile between the previous step's TM * TN MFMAs
  auto pattern = [&]() {
#pragma unroll
    for (int i = 0; i < TM + TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
  };
  // Step s: the fragment reads and MFMAs of a live band, then (every wave)
  // two of the next k-tile's loads. The loads sit outside the branch: with
  // loads on one side of a branch only, the compiler's wait tracking merges
  // the two paths and adds a full vmcnt(0) before the next fragment read.
  auto block = [&](auto qc, int i) {
    const lm_u32x4* buf = stage_buf(qc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (live) {
        read_frags(buf, s & 1, s);
        if (s > 0 || i > 0) mma((s - 1) & 1);
        pattern();
      }
      issue_part(std::integral_constant<int, decltype(qc)::value ^ 1>{}, i + 1, s);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  issue(std::integral_constant<int, 0>{}, 0);  // k-tile 0 in flight
  // K-tile i: this wave's fragment reads of k-tile i-1 have completed and its
  // loads of k-tile i have landed; the barrier makes that true of every wave,
  // so k-tile i is visible and the buffer of k-tile i-1 free for k-tile i+1,
  // whose loads go out two per MFMA step.
  auto iter = [&](auto qc, int i) {
    constexpr int q = decltype(qc)::value;
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0), lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    block(qc, i);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int i = 0; i < nkt; i += 2) {
    iter(std::integral_constant<int, 0>{}, i);
    iter(std::integral_constant<int, 1>{}, i + 1);
  }
  if (live) mma(1);  // the last k-tile's last step
  // the surplus loads of the last iteration land before the buffers are reused
  lm_wait_vmcnt<0>();
  __syncthreads();
  p.epilogue(t, acc, wm, wn, lane, (void*)st0);
}

