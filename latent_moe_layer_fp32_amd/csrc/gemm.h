// Tiled matrix-core GEMM core for gfx950: C[M,N] = A[M,K] * B[N,K]^T.
//
// One workgroup = 4 wavefronts of 64 lanes computes a BM x BN output tile.
// A and B k-tiles of 128 bytes per row (64 BF16 or 32 FP32 elements) are
// staged through LDS in two buffers: while the matrix cores consume one
// buffer, the next k-tile is already in flight from global memory into
// registers. LDS rows are 8 chunks of 16 bytes with the chunk index XORed by
// (row / 2) % 8: a 16-byte LDS access is served 16 lanes (256 bytes) per
// pass, and with that swizzle any 16 consecutive rows read at one logical
// chunk, as well as the 16-byte stores of two consecutive rows, fall into 16
// distinct 16-byte bank groups. (XOR by row % 8 leaves rows r and r+8 on
// the same banks: a measured 2-way conflict on the operand reads.)
//
// Matrix instructions: BF16 uses v_mfma_f32_32x32x16_bf16, FP16
// v_mfma_f32_32x32x16_f16, FP32 v_mfma_f32_32x32x2_f32. A lane reads one 16-byte chunk of its A row and its
// B row per step; any assignment of k to (lane, step) is valid as long as A
// and B use the same one, which lets every lane read whole chunks.
//
// A problem type supplies: Cfg (tile shape), tile() mapping a block to a
// tile, a_row()/b_row() row pointers (gathers and expert offsets live there),
// a_ktile() (k-tile index into A; lets the router reuse x across the three
// BF16 pieces of its FP32 weights) and epilogue().
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"

template <typename E>
struct LmElem;

template <>
struct LmElem<uint16_t> {  // bfloat16 bits
  static constexpr int kPerChunk = 8;
  LM_DEV static void mma(lm_f32x16& acc, lm_u32x4 a, lm_u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lm_bf16x8, a),
                                                  __builtin_bit_cast(lm_bf16x8, b), acc, 0, 0, 0);
  }
  LM_DEV static uint16_t from_f32(float v) { return lm_f32_to_bf16(v); }
  LM_DEV static float to_f32(uint16_t v) { return lm_bf16_to_f32(v); }
};

template <>
struct LmElem<_Float16> {  // IEEE half: same matrix rate as BF16, three more mantissa bits
  static constexpr int kPerChunk = 8;
  LM_DEV static void mma(lm_f32x16& acc, lm_u32x4 a, lm_u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(lm_f16x8, a),
                                                 __builtin_bit_cast(lm_f16x8, b), acc, 0, 0, 0);
  }
  LM_DEV static _Float16 from_f32(float v) { return lm_f32_to_f16_sat(v); }
  LM_DEV static float to_f32(_Float16 v) { return (float)v; }
};

template <>
struct LmElem<float> {
  static constexpr int kPerChunk = 4;
  LM_DEV static void mma(lm_f32x16& acc, lm_u32x4 a, lm_u32x4 b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc,
                                                 0, 0, 0);
  }
  LM_DEV static float from_f32(float v) { return v; }
  LM_DEV static float to_f32(float v) { return v; }
};

// WM x WN waves, each wave TM x TN tiles of 32x32. FLUSH > 0 folds the running
// FP32 accumulator into an FP64 one every FLUSH k-tiles and hands the FP64
// sums to the epilogue (short FP32 addition chains: the router's logits must
// be accurate to a few 1e-7 for the top-k selection).
template <typename E_, int WM_, int WN_, int TM_, int TN_, int FLUSH_ = 0>
struct LmGemmCfg {
  using E = E_;
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  static constexpr int FLUSH = FLUSH_;
  static constexpr int KT = 8 * LmElem<E>::kPerChunk;  // elements per k-tile
  static_assert(WM * WN == 4 || (WM == 1 && WN == 8) || (WM == 2 && WN == 4),
                "four wavefronts per workgroup, or eight (along N, or 2 x 4)");
};

struct LmTile {
  int m0;    // first row of the tile in the problem's row space
  int rows;  // valid rows (<= BM)
  int n0;    // first output column
  int nt;    // n-tile index
  int kt0, kt1;  // k-tile range
  int e;     // expert (grouped problems) or k-split index
};

// Problems whose epilogue needs one value per tile row (gathered from memory)
// declare row_value() (and may switch it off with kRowValue = false); it is
// loaded at the start of the tile, so its latency hides behind the main loop,
// and handed to the epilogue through LDS.
template <class P, class = void>
struct LmRowValueOn : std::true_type {};
template <class P>
struct LmRowValueOn<P, std::void_t<decltype(P::kRowValue)>> : std::integral_constant<bool, P::kRowValue> {};
template <class P, class = void>
struct LmHasRowValue : std::false_type {};
template <class P>
struct LmHasRowValue<P, std::void_t<decltype(std::declval<const P&>().row_value(std::declval<const LmTile&>(), 0))>>
    : LmRowValueOn<P> {};

// Problems whose B k-tiles are not read in order declare b_ktile() (the
// router's six-product split); the others read B k-tile kt at step kt.
template <class P, class = void>
struct LmHasBKtile : std::false_type {};
template <class P>
struct LmHasBKtile<P, std::void_t<decltype(std::declval<const P&>().b_ktile(0))>> : std::true_type {};
template <class P>
LM_DEV int lm_b_ktile(const P& p, int kt) {
  if constexpr (LmHasBKtile<P>::value) return p.b_ktile(kt);
  else return kt;
}

LM_DEV int lm_swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Row groups of 32 rows interleaved per k-tile in the packed weight layout
// (lm_packed_group).
constexpr int kLmPackGroups = 8;

// Weight loads. NT: a non-temporal load, for weights read once and never
// again (the streaming hint measured 7.07 against 6.34 TB/s for plain
// 16-byte loads on MI355X); otherwise a plain load, where other m-tiles reuse
// the weight tile from L2.
//
// Grouped expert problems declare kWeightsOnce: with decode-sized tiles an
// expert's few rows fit one m-tile, so each weight tile is read once.
template <class P, class = void>
struct LmWeightsOnce : std::false_type {};
template <class P>
struct LmWeightsOnce<P, std::void_t<decltype(P::kWeightsOnce)>>
    : std::integral_constant<bool, P::kWeightsOnce> {};

// Problems that clear a small counter array before the kernels after them
// count into it declare clear(block, blocks, thread); every block of the
// launch runs it first (the router clears the top-k kernel's expert counters,
// so no separate fill kernel runs between the two).
template <class P, class = void>
struct LmHasClear : std::false_type {};
template <class P>
struct LmHasClear<P, std::void_t<decltype(std::declval<const P&>().clear(0, 0, 0))>> : std::true_type {};

template <bool NT, class T>
LM_DEV T lm_wload(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <class Cfg>
struct LmGemmSmem {
  lm_u32x4 a[2][Cfg::BM * 8];
  lm_u32x4 b[2][Cfg::BN * 8];
};

// Accumulator coordinates of the 32x32 MFMA result: register i of lane l
// holds row 8*(i/4) + 4*(l/32) + i%4, column l%32.
template <class Cfg>
LM_DEV int lm_acc_row(int wm, int tm, int i, int lane) {
  return wm * Cfg::TM * 32 + tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}
template <class Cfg>
LM_DEV int lm_acc_col(int wn, int tn, int lane) {
  return wn * Cfg::TN * 32 + tn * 32 + (lane & 31);
}

// Blocks are dispatched round-robin over the 8 XCDs (block b on XCD b % 8).
// Give each XCD a contiguous range of the logical order so that neighbours in
// that order (tiles sharing weights or activations) share an L2.
LM_DEV bool lm_xcd_map(int bid, int total, int& L) {
  const int per = (total + 7) >> 3;
  const int s = bid >> 3;
  if (s >= per) return false;
  L = (bid & 7) * per + s;
  return L < total;
}

// Dense tile order: groups of GM m-tiles walk all n-tiles together.
LM_DEV void lm_dense_order(int L, int mt, int nt, int GM, int& m, int& n) {
  const int per_group = GM * nt;
  const int g = L / per_group;
  const int first = g * GM;
  const int gsz = min(GM, mt - first);
  const int r = L - g * per_group;
  m = first + r % gsz;
  n = r / gsz;
}

template <class Prob>
__global__ __launch_bounds__(256) void lm_gemm_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM * Cfg::WN == 4, "four wavefronts");
  using El = LmElem<typename Cfg::E>;
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  constexpr int QA = Cfg::BM / 32, QB = Cfg::BN / 32;
  __shared__ LmGemmSmem<Cfg> sm;
  if constexpr (LmHasClear<Prob>::value) p.clear(blockIdx.x, gridDim.x, threadIdx.x);

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int lc = tid & 7, lr = tid >> 3;
  float rowv = 0.0f;
  if constexpr (LmHasRowValue<Prob>::value)
    if (tid < Cfg::BM) rowv = p.row_value(t, tid);

  const lm_u32x4* ap[QA];
  const lm_u32x4* bp[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) ap[q] = p.a_row(t, lr + 32 * q);
#pragma unroll
  for (int q = 0; q < QB; ++q) bp[q] = p.b_row(t, lr + 32 * q);

  lm_u32x4 ra[QA], rb[QB];
  lm_f32x16 acc[TM][TN];
  double acc2[Cfg::FLUSH ? TM : 1][Cfg::FLUSH ? TN : 1][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if constexpr (Cfg::FLUSH) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.0;
  }

  auto gload = [&](int kt) {
    const int ka = p.a_ktile(kt);
#pragma unroll
    for (int q = 0; q < QA; ++q) ra[q] = ap[q][ka * 8 + lc];
    const int kb = lm_b_ktile(p, kt);
#pragma unroll
    for (int q = 0; q < QB; ++q) rb[q] = bp[q][kb * 8 + lc];
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < QA; ++q) sm.a[buf][lm_swz(lr + 32 * q, lc)] = ra[q];
#pragma unroll
    for (int q = 0; q < QB; ++q) sm.b[buf][lm_swz(lr + 32 * q, lc)] = rb[q];
  };

  gload(t.kt0);
  sstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = t.kt0; kt < t.kt1; ++kt) {
    const bool more = kt + 1 < t.kt1;
    if (more) gload(kt + 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + (lane >> 5);
      lm_u32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = sm.a[buf][lm_swz(wm * TM * 32 + i * 32 + (lane & 31), ch)];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = sm.b[buf][lm_swz(wn * TN * 32 + j * 32 + (lane & 31), ch)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) El::mma(acc[i][j], fa[i], fb[j]);
    }
    if constexpr (Cfg::FLUSH) {
      if (((kt - t.kt0 + 1) % Cfg::FLUSH) == 0 || !more) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc2[i][j][r] += (double)acc[i][j][r];
              acc[i][j][r] = 0.0f;
            }
      }
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if constexpr (LmHasRowValue<Prob>::value) {
    if (tid < Cfg::BM) ((float*)&sm)[tid] = rowv;
    __syncthreads();
  }
  if constexpr (Cfg::FLUSH)
    p.epilogue_f64(t, acc2, wm, wn, lane);
  else
    p.epilogue(t, acc, wm, wn, lane, (void*)&sm);
}

// Short k ranges with FP64 folding (the router at decode sizes: four k-tiles
// per k-split): every k-tile of the block's range is loaded into registers at
// the start, so the block waits for memory once instead of once per k-tile
// (with cold caches each wait is a whole HBM round trip); the k-tiles then
// pass through the two LDS buffers in turn, with the same fragment reads,
// matrix instructions and FP64 folds as lm_gemm_kernel, so the two kernels
// produce identical sums. Requires t.kt1 - t.kt0 <= KD (checked on the host).
template <class Prob, int KD>
__global__ __launch_bounds__(256) void lm_gemm_kdeep_kernel(const Prob p) {
  using Cfg = typename Prob::Cfg;
  static_assert(Cfg::WM * Cfg::WN == 4, "four wavefronts");
  static_assert(Cfg::FLUSH > 0, "problems folding into FP64");
  using El = LmElem<typename Cfg::E>;
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  constexpr int QA = Cfg::BM / 32, QB = Cfg::BN / 32;
  __shared__ LmGemmSmem<Cfg> sm;
  if constexpr (LmHasClear<Prob>::value) p.clear(blockIdx.x, gridDim.x, threadIdx.x);

  LmTile t;
  if (!p.tile(blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int lc = tid & 7, lr = tid >> 3;
  const int nk = t.kt1 - t.kt0;

  lm_u32x4 ra[KD][QA], rb[KD][QB];
  {
    const lm_u32x4* ap[QA];
    const lm_u32x4* bp[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) ap[q] = p.a_row(t, lr + 32 * q);
#pragma unroll
    for (int q = 0; q < QB; ++q) bp[q] = p.b_row(t, lr + 32 * q);
#pragma unroll
    for (int d = 0; d < KD; ++d) {
      if (d < nk) {
        const int ka = p.a_ktile(t.kt0 + d), kb = lm_b_ktile(p, t.kt0 + d);
#pragma unroll
        for (int q = 0; q < QA; ++q) ra[d][q] = ap[q][ka * 8 + lc];
#pragma unroll
        for (int q = 0; q < QB; ++q) rb[d][q] = bp[q][kb * 8 + lc];
      }
    }
  }

  lm_f32x16 acc[TM][TN];
  double acc2[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[i][j][r] = 0.0f;
        acc2[i][j][r] = 0.0;
      }

  // k-tile d goes through LDS buffer d & 1. The store of k-tile d + 2 into
  // the same buffer comes after the barrier of k-tile d + 1, which every wave
  // reaches only once its reads of k-tile d are done.
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    if (d < nk) {
      const int buf = d & 1;
#pragma unroll
      for (int q = 0; q < QA; ++q) sm.a[buf][lm_swz(lr + 32 * q, lc)] = ra[d][q];
#pragma unroll
      for (int q = 0; q < QB; ++q) sm.b[buf][lm_swz(lr + 32 * q, lc)] = rb[d][q];
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = 2 * s + (lane >> 5);
        lm_u32x4 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = sm.a[buf][lm_swz(wm * TM * 32 + i * 32 + (lane & 31), ch)];
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = sm.b[buf][lm_swz(wn * TN * 32 + j * 32 + (lane & 31), ch)];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) El::mma(acc[i][j], fa[i], fb[j]);
      }
      if (((d + 1) % Cfg::FLUSH) == 0 || d + 1 == nk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc2[i][j][r] += (double)acc[i][j][r];
              acc[i][j][r] = 0.0f;
            }
      }
    }
  }
  p.epilogue_f64(t, acc2, wm, wn, lane);
}

// Per-row sum over the tile's valid columns of v(acc)^2, reduced in a fixed
// order (lanes, then waves). `red` must hold (Cfg::WN + 1) * Cfg::BM floats;
// the sum for tile row r is left in red[Cfg::WN * Cfg::BM + r], and all
// threads are synchronised on return.
template <class Cfg, class F>
LM_DEV void lm_tile_row_ssq(const lm_f32x16 (&acc)[Cfg::TM][Cfg::TN], int wm, int wn, int lane,
                            int ncols_valid, float* red, F value) {
#pragma unroll
  for (int tm = 0; tm < Cfg::TM; ++tm) {
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.0f;
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn) {
        const int col = lm_acc_col<Cfg>(wn, tn, lane);
        const float v = value(acc[tm][tn][i], tn, col);
        s[i] += col < ncols_valid ? v * v : 0.0f;
      }
    }
    lm_half_reduce(s, [](float x, float y) { return x + y; });
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((lane & 31) == 0) red[wn * Cfg::BM + lm_acc_row<Cfg>(wm, tm, i, lane)] = s[i];
  }
  __syncthreads();
  if (threadIdx.x < Cfg::BM) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < Cfg::WN; ++w) s += red[w * Cfg::BM + threadIdx.x];
    red[Cfg::WN * Cfg::BM + threadIdx.x] = s;
  }
  __syncthreads();
}
