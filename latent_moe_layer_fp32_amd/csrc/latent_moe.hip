// Host runtime and C ABI of the latent-MoE layer forward (see include/latent_moe.h).
//
// create(): validate, allocate one workspace sized by max_tokens, split the
// FP32 router into three BF16 pieces and repack the weights into the
// matrix-core layout (BF16 activations: the pooler in BF16, the expert and
// unpooler weights as FP16 copies scaled per row by a power of two, or
// MXFP4 codes with that power of two per row, so that the expert and
// unpooler GEMMs run on FP16 operands u, a and y). forward(): enqueue
// the kernel sequence on the caller's stream with no host synchronisation and
// no allocation; per-expert tile counts stay on the device and the grouped
// GEMMs are launched with upper-bound grids whose surplus blocks exit.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>

#include "../../include/latent_moe.h"
#include "gemm_lds.h"
#include "gemm_stream.h"
#include "kernels.h"
#include "mx_act.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define LM_HIP(call)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess) return fail(LMOE_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Test hooks, read from the environment at create:
//   LATENT_MOE_FAULT=alloc    the first device allocation of create fails (as
//   LATENT_MOE_FAULT=alloc:N  out of memory), or the N-th (1-based)
//   LATENT_MOE_DEBUG=poison   the workspace is filled with 0xFF bytes (NaN
//                             floats, -1 integers) at create and before every
//                             forward, so a stage reading a value no earlier
//                             stage of the same forward wrote shows up as NaN;
//                             guard words after the workspace are checked by
//                             destroy (LMOE_ERR_CORRUPT if any was overwritten).
struct AllocCtl {
  int fail_at = 0;  // 0: no injected failure
  int n = 0;        // allocations so far
};
AllocCtl alloc_ctl_from_env() {
  AllocCtl c;
  const char* e = getenv("LATENT_MOE_FAULT");
  if (e && strncmp(e, "alloc", 5) == 0) c.fail_at = e[5] == ':' ? atoi(e + 6) : 1;
  return c;
}
hipError_t lm_malloc(AllocCtl& c, void** p, size_t bytes) {
  if (++c.n == c.fail_at) return hipErrorOutOfMemory;
  return hipMalloc(p, bytes);
}
bool debug_poison() {
  const char* e = getenv("LATENT_MOE_DEBUG");
  return e && strstr(e, "poison") != nullptr;
}
constexpr size_t kGuardBytes = 65536;
constexpr uint32_t kGuardWord = 0x5A17C0DEu;

__global__ void lm_fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}
// Fill `bytes` (a multiple of 4) with a 32-bit word, by a kernel (no memset
// node, so the call is safe inside a captured stream).
hipError_t lm_fill_launch(void* p, size_t bytes, uint32_t v, hipStream_t s) {
  const size_t n = bytes / 4;
  if (!n) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256 < 16384 ? (n + 255) / 256 : 16384);
  hipLaunchKernelGGL(lm_fill_u32_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, n, v);
  return hipGetLastError();
}

// Tile configurations: "wide" for many rows per expert (prefill-sized),
// "narrow" for few (decode-sized). 16-bit operands run the streaming-B kernel
// (four or eight waves along N, 64 output columns each); FP32 runs the
// LDS-staged kernel.
#ifndef LM_WIDE_TM
#define LM_WIDE_TM 4
#endif
#ifndef LM_EXPERT_WN
#define LM_EXPERT_WN 8
#endif
// FP16 operands (expert and unpooler GEMMs), prefill-sized: one workgroup of
// LM_EXPERT_WN waves along N per CU (128 x 512 tiles: each gathered A row is
// read once per 256 output columns of gate/up instead of per 128, and the
// L2 bytes per MFMA drop by a sixth against two 128 x 256 workgroups).
template <typename E>
using CfgWide = std::conditional_t<
    std::is_same_v<E, _Float16>, LmGemmCfg<E, 1, LM_EXPERT_WN, LM_WIDE_TM, 2>,
    std::conditional_t<sizeof(E) == 2, LmGemmCfg<E, 1, 4, LM_WIDE_TM, 2>, LmGemmCfg<E, 2, 2, 2, 2>>>;
template <typename E> using CfgNarrow = LmGemmCfg<E, 1, 4, 1, 2>;
// Prefill-sized 16-bit GEMMs with both operands staged in LDS by direct loads
// (lm_gemm_lds_kernel): 256 x 256 tiles of eight waves, two k-tile stages.
// BF16 experts and the dense projections; MXFP4 experts keep the streaming
// kernel.
// Expert outputs O of BF16 layers in FP16 (o times a per-expert power of two)
// or, with 0, in FP32.
#ifndef LM_O_F16
#define LM_O_F16 1
#endif
// Off by default: slower than the streaming kernel on the prefill shapes.
#ifndef LM_LDS_GEMM
#define LM_LDS_GEMM 0
#endif
template <typename E> using CfgLds = LmGemmCfg<E, 2, 4, 4, 2>;
// Router: FP32 chains of one k-tile (64 BF16 products per lane pair), FP64 beyond.
template <typename E> using CfgRouterWide = LmGemmCfg<E, 2, 2, 1, 2, 1>;
template <typename E> using CfgRouterNarrow = LmGemmCfg<E, 1, 4, 1, 2, 1>;

constexpr int kNarrowRowsPerExpert = 64;  // mean rows per expert below which "narrow" tiles run
constexpr int kMinBN = 128;  // smallest BN of the tile configurations (sizes the ssq partials)

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

struct Layout {
  size_t part, logits, ids, wts, cpad, counts, offsets, tile_off, perm_token, pair_row, pooled, pssq,
      row_scale, act, O, ossq, y, kpart, xn, xna, uq, us, acts, u16, total;
};

// Split-K plan for a dense BF16 projection: split only when the output tiles
// cannot cover the chip; each split a multiple of 8 k-tiles (the streaming
// kernel's unroll).
void dense_split(int64_t T, int64_t N, int64_t K, int BM, int BN, int& splits, int& kt_per) {
  const int64_t tiles = ceil_div(T, BM) * (int64_t)ceil_div(N, BN);
  const int ktiles = (int)(K / 64);
  splits = 1;
  kt_per = ktiles;
  if (tiles >= 256) return;
  int want = ceil_div(512, tiles);
  if (want > ktiles / 8) want = ktiles / 8;
  if (want <= 1) return;
  kt_per = (ceil_div(ktiles, want) + 7) / 8 * 8;
  splits = ceil_div(ktiles, kt_per);
}

}  // namespace

constexpr int kStages = LMOE_NUM_STAGES;

struct latent_moe {
  latent_moe_config cfg;
  latent_moe_weights w;            // points into `owned` after create (nothing is borrowed)
  int device;
  char* ws;                        // workspace (+ guard words in poison mode)
  Layout lay;
  size_t part_floats;
  char* owned;                     // library-owned copies of every weight the forward reads
  size_t owned_bytes;
  const void* pk_pooler;           // BF16 layers: weights in the matrix-core layout
  const void* pk_unpooler;
  const void* pk_gate;
  const void* pk_up;
  const void* pk_down;
  const void* pk_sgate;  // MXFP4: packed scales
  const void* pk_sup;
  const void* pk_sdown;
  const void* wr3;       // BF16 layers: the router's exact three-piece BF16 split [E, 3H]
  const float* ds_gate;  // 2^-s per weight row of the FP16 / MXFP4 copies
  const float* ds_up;
  const float* ds_down;
  const float* ds_unpooler;
  float u_down = 1.0f;  // FP16 u and y are stored times these powers of two (see create)
  float y_down = 1.0f;
  const float* a_down;  // FP16 a is stored times a_down[e][i / 32] (see lm_a_shift_kernel)
  const float* o_down = nullptr;  // FP16 expert outputs are stored times o_down[e] (lm_o_shift_kernel)
  const float* o_up = nullptr;    // 1 / o_down[e]
  bool side_ok = false;            // the side stream and its events exist
  hipStream_t side = nullptr;      // the pooler steps run here, beside routing on the caller's stream
  hipEvent_t fork = nullptr, join = nullptr;  // order the side stream after the caller's and back
  bool poison = false;             // debug: workspace refilled with 0xFF bytes before each forward
  bool prof = false;               // record stage events in forward
  bool prof_valid = false;         // a forward has recorded a full set
  hipEvent_t ev[kStages + 1] = {};  // created by latent_moe_set_profiling
};

namespace {

int esize_act(const latent_moe_config& c) { return c.act_dtype == LMOE_F32 ? 4 : 2; }
int esize_exp(const latent_moe_config& c) { return c.expert_dtype == LMOE_F32 ? 4 : 2; }

bool narrow_for(const latent_moe_config& c, int64_t T) {
  return T * c.top_k < (int64_t)kNarrowRowsPerExpert * c.experts;
}

// Routers whose k-splits span at most this many k-tiles run lm_gemm_kdeep_kernel.
constexpr int kRouterDeep = 4;

// Router k-splits: enough blocks to cover the chip, each split at least 4
// k-tiles, all splits non-empty. FP32 layers: K = H in 32-column k-tiles.
// BF16 layers: x against the three-piece BF16 split of the router (K = 3H),
// or, with the boundary norm, the six exact piece products (K = 6H).
void router_split(const latent_moe_config& c, int64_t T, int& splits, int& kt_per, int& mt,
                  int& nt) {
  const bool f32 = c.act_dtype == LMOE_F32;
  const bool nar = narrow_for(c, T);
  const int BM = nar ? 32 : 64, BN = nar ? 256 : 128;  // router tile shapes
  const int KT = f32 ? 32 : 64;
  const int64_t Kw = f32 ? c.hidden : (c.input_norm ? 6 : 3) * c.hidden;
  const int ktot = (int)(Kw / KT);
  mt = ceil_div(T, BM);
  nt = ceil_div(c.experts, BN);
  int want = ceil_div(512, (int64_t)mt * nt);
  int maxs = ktot / 4 > 0 ? ktot / 4 : 1;
  splits = want < 1 ? 1 : (want > maxs ? maxs : want);
  kt_per = ceil_div(ktot, splits);
  splits = ceil_div(ktot, kt_per);
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

int validate_config(const latent_moe_config* c) {
  if (!c) return fail(LMOE_ERR_INVALID_ARG, "config is NULL");
  if (c->hidden <= 0 || c->pooled <= 0 || c->intermediate <= 0 || c->hidden % 64 ||
      c->pooled % 64 || c->intermediate % 128)
    return fail(LMOE_ERR_INVALID_ARG,
                "hidden and pooled must be positive multiples of 64, intermediate of 128");
  if (c->hidden > (1 << 20) || c->pooled > (1 << 20) || c->intermediate > (1 << 20))
    return fail(LMOE_ERR_INVALID_ARG, "dimension too large");
  if (c->experts < 1 || c->experts > 1024)
    return fail(LMOE_ERR_INVALID_ARG, "experts must be in [1, 1024]");
  if (c->top_k < 1 || c->top_k > kLmMaxK || c->top_k > c->experts)
    return fail(LMOE_ERR_INVALID_ARG, "top_k must be in [1, min(experts, %d)]", kLmMaxK);
  if (!std::isfinite(c->eps) || c->eps < 0.0f)
    return fail(LMOE_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (c->max_tokens < 1 || c->max_tokens * c->top_k > (1 << 28))
    return fail(LMOE_ERR_INVALID_ARG, "max_tokens must be in [1, 2^28 / top_k]");
  const bool act_ok = c->act_dtype == LMOE_F32 || c->act_dtype == LMOE_BF16;
  const bool exp_ok = c->expert_dtype == LMOE_F32 || c->expert_dtype == LMOE_BF16 ||
                      c->expert_dtype == LMOE_MXFP4;
  if (!act_ok || !exp_ok) return fail(LMOE_ERR_INVALID_ARG, "unknown dtype code");
  if ((c->act_dtype == LMOE_F32) != (c->expert_dtype == LMOE_F32))
    return fail(LMOE_ERR_UNSUPPORTED, "FP32 experts need FP32 activations and vice versa");
  if (c->act_dtype == LMOE_BF16 && (c->hidden % 512 || c->pooled % 512 || c->intermediate % 512))
    return fail(LMOE_ERR_UNSUPPORTED,
                "BF16 layers are built for hidden, pooled and intermediate multiples of 512");
  if (c->input_norm != 0 && c->input_norm != 1)
    return fail(LMOE_ERR_INVALID_ARG, "input_norm must be 0 or 1");
  if (c->expert_act != 0 && c->expert_act != LMOE_MXFP8 && c->expert_act != LMOE_MXFP4)
    return fail(LMOE_ERR_INVALID_ARG, "expert_act must be 0, LMOE_MXFP8 or LMOE_MXFP4");
  if (c->expert_act != 0 && (c->expert_dtype != LMOE_MXFP4 || c->act_dtype != LMOE_BF16))
    return fail(LMOE_ERR_UNSUPPORTED, "MX expert activations need MXFP4 experts and BF16 activations");
  if ((size_t)c->pooled * c->intermediate * c->experts > ((size_t)1 << 40))
    return fail(LMOE_ERR_INVALID_ARG, "expert tensors too large");
  return LMOE_OK;
}

Layout make_layout(const latent_moe_config& c, size_t* part_floats) {
  const int64_t Tm = c.max_tokens, k = c.top_k, E = c.experts, P = c.pooled, I = c.intermediate;
  const int64_t Mp = Tm * k;
  // largest router partial buffer over T in [1, Tm]; beyond 65536 tokens a
  // single split covers the chip, so T = Tm bounds the rest
  size_t pf = 0;
  const int64_t scan = Tm < 65536 ? Tm : 65536;
  for (int64_t T = 1; T <= scan + 1; ++T) {
    const int64_t TT = T <= scan ? T : Tm;
    int s, kp, mt, nt;
    router_split(c, TT, s, kp, mt, nt);
    const size_t need = (size_t)s * TT * E;
    if (need > pf) pf = need;
  }
  *part_floats = pf;
  const int parts = ceil_div(P, kMinBN);  // n-tiles of the pooler / down GEMMs
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.part = take(pf * 8);
  L.logits = take((size_t)Tm * E * 4);
  L.ids = take((size_t)Mp * 4);
  L.wts = take((size_t)Mp * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.tile_off = take((size_t)(E + 1) * 4);
  L.perm_token = take((size_t)Mp * 4);
  L.pair_row = take((size_t)Mp * 4);
  const bool mxa = c.expert_act != 0;
  const size_t abits = c.expert_act == LMOE_MXFP8 ? 8 : 4;
  L.pooled = take((size_t)Tm * P * 4);  // gamma_p * h, FP32
  L.pssq = take((size_t)Tm * parts * 4);
  L.row_scale = take((size_t)Tm * 4);
  L.act = take((size_t)Mp * I * esize_exp(c));
  L.O = take((size_t)Mp * P * (c.act_dtype == LMOE_BF16 && LM_O_F16 ? 2 : 4));  // expert outputs: FP16 (BF16 layers) or FP32
  L.ossq = take((size_t)Mp * parts * 4);
  L.y = take((size_t)Tm * P * esize_act(c));  // FP32 or FP16 [T, P]
  size_t kp = 0;
  if (c.act_dtype == LMOE_BF16) {
    for (int64_t T = 1; T <= (Tm < 65536 ? Tm : 65536); ++T) {
      // the tile shapes forward uses: pooler on BF16, unpooler on FP16 operands
      const bool nar = narrow_for(c, T);
      const int BM = nar ? CfgNarrow<uint16_t>::BM : CfgWide<uint16_t>::BM;
      const int BNp = nar ? CfgNarrow<uint16_t>::BN : CfgWide<uint16_t>::BN;
      const int BNu = nar ? CfgNarrow<_Float16>::BN : CfgWide<_Float16>::BN;
      int sp, kpt;
      dense_split(T, P, c.hidden, BM, BNp, sp, kpt);
      if (sp > 1 && (size_t)sp * T * P > kp) kp = (size_t)sp * T * P;
      dense_split(T, c.hidden, P, BM, BNu, sp, kpt);
      if (sp > 1 && (size_t)sp * T * c.hidden > kp) kp = (size_t)sp * T * c.hidden;
    }
  }
  L.kpart = take(kp * 4);
  L.uq = take(mxa ? (size_t)Tm * P * abits / 8 : 0);  // MX u codes
  L.us = take(mxa ? (size_t)Tm * P / 32 : 0);          // and E8M0 scales
  L.acts = take(mxa ? (size_t)Mp * I / 32 : 0);        // E8M0 scales of the MX act codes (in act)
  L.xn = take(c.input_norm && c.act_dtype == LMOE_F32 ? (size_t)Tm * c.hidden * 4 : 0);
  L.xna = take(c.input_norm && c.act_dtype == LMOE_BF16 ? (size_t)Tm * 3 * c.hidden * 2 : 0);
  L.u16 = take(c.act_dtype == LMOE_BF16 && !mxa ? (size_t)Tm * P * 2 : 0);  // FP16 u
  L.cpad = take((size_t)E * kLmCountStride * 4);  // padded per-expert counters
  L.total = o;
  return L;
}

template <class Prob>
hipError_t launch(const Prob& p, int64_t units, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  const int64_t g = (units + 7) / 8 * 8;
  if constexpr (Prob::Cfg::WM * Prob::Cfg::WN == 8 && Prob::Cfg::WM == 2)
    hipLaunchKernelGGL(lm_gemm_lds_kernel<Prob>, dim3((unsigned)g), dim3(512), 0, s, p);
  else if constexpr (sizeof(typename Prob::Cfg::E) == 2 && Prob::Cfg::WM == 1 && !Prob::Cfg::FLUSH)
    hipLaunchKernelGGL(lm_gemm_stream_kernel<Prob>, dim3((unsigned)g), dim3(64 * Prob::Cfg::WN), 0, s, p);
  else
    hipLaunchKernelGGL(lm_gemm_kernel<Prob>, dim3((unsigned)g), dim3(256), 0, s, p);
  return hipGetLastError();
}

#define LM_MARK(i)                                       \
  do {                                                   \
    if (h->prof) LM_HIP(hipEventRecord(h->ev[(i)], s));  \
  } while (0)

template <class Prob>
hipError_t launch_mxa(const Prob& p, int64_t units, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  const int64_t g = (units + 7) / 8 * 8;
  hipLaunchKernelGGL(lm_gemm_stream_mxa_kernel<Prob>, dim3((unsigned)g), dim3(64 * Prob::Cfg::WN), 0, s, p);
  return hipGetLastError();
}

// MX: MXFP4 expert weights; AB: expert GEMM inputs as MX FP8 (8) or MX FP4
// (4) codes, or in the activation type (0).
template <typename Et, template <typename> class CW, template <typename> class CR, bool MX = false,
          int AB = 0>
int forward_impl(latent_moe* h, const void* x, int64_t T, float* out, hipStream_t s) {
  constexpr bool MXA = AB != 0;
  const latent_moe_config& c = h->cfg;
  const latent_moe_weights& w = h->w;
  const Layout& L = h->lay;
  char* ws = h->ws;
  const int E = (int)c.experts, k = c.top_k, H = (int)c.hidden, P = (int)c.pooled,
            I = (int)c.intermediate;
  const int npairs = (int)(T * k);
  const bool packed = sizeof(Et) == 2;  // BF16 matrices read from the packed copies
  const void* Wpool = packed ? h->pk_pooler : w.pooler;
  const void* Wunpool = packed ? h->pk_unpooler : w.unpooler;
  const void* Wgate = packed ? h->pk_gate : w.w_gate;
  const void* Wup = packed ? h->pk_up : w.w_up;
  const void* Wdown = packed ? h->pk_down : w.w_down;
  using Cw = CW<Et>;
  using Cr = CR<Et>;
  // expert and unpooler operands: FP16 in BF16 layers, FP32 in FP32 layers
  constexpr bool F16 = sizeof(Et) == 2;
  using Eh = std::conditional_t<F16, _Float16, Et>;
  using Ch = CW<Eh>;
  // MX expert inputs, prefill-sized down GEMM: as many waves along N as the FP16
  // GEMMs (measured faster; the MX gate/up kernel measured slower on eight waves)
  using Cx = std::conditional_t<MXA && Cw::TM == 4, LmGemmCfg<Et, 1, Ch::WN, Cw::TM, 2>, Cw>;
  // prefill-sized BF16 layers with BF16 experts: the LDS-staged 256 x 256 kernel
  // for the pooler, gate/up, down and unpooler
  constexpr bool kLds = LM_LDS_GEMM && F16 && !MX && !MXA && Cw::TM == 4;
  using Cp = std::conditional_t<kLds, CfgLds<Et>, Cw>;  // pooler
  using Ce = std::conditional_t<kLds, CfgLds<Eh>, Ch>;  // gate/up, down, unpooler
  constexpr int kBmGroup = kLds ? Ce::BM : Cw::BM;      // rows per grouped-GEMM tile
  double* part = (double*)(ws + L.part);
  float* logits = (float*)(ws + L.logits);
  int* ids = (int*)(ws + L.ids);
  float* wts = (float*)(ws + L.wts);
  int* cpad = (int*)(ws + L.cpad);
  int* counts = (int*)(ws + L.counts);
  int* offsets = (int*)(ws + L.offsets);
  int* tile_off = (int*)(ws + L.tile_off);
  int* perm_token = (int*)(ws + L.perm_token);
  int* pair_row = (int*)(ws + L.pair_row);
  Et* pooled = (Et*)(ws + L.pooled);  // FP32 layers: gamma_p * h; BF16 layers: unused
  float* pooled32 = (float*)(ws + L.pooled);  // BF16 layers: gamma_p * h in FP32
  float* pssq = (float*)(ws + L.pssq);
  float* row_scale = (float*)(ws + L.row_scale);
  Eh* u16 = (Eh*)(ws + L.u16);  // BF16 layers without MX inputs: the FP16 u
  Eh* act = (Eh*)(ws + L.act);
  float* O = (float*)(ws + L.O);  // FP32 layers: o; BF16 layers: FP16 gamma_e * o times o_down[e]
  float* ossq = (float*)(ws + L.ossq);
  Eh* y = (Eh*)(ws + L.y);

  if (h->poison) LM_HIP(lm_fill_launch(ws, L.total, 0xFFFFFFFFu, s));
  LM_MARK(0);
  // 0. boundary norm (optional): x is the pre-norm residual. FP32 layers: the
  // router and pooler read the FP32 norm. BF16 layers: its exact three-piece
  // BF16 split [T, 3H]; the router forms the FP32 products from the pieces,
  // the pooler reads the first piece (the BF16 rounding) at row stride 3H.
  const Et* xp = (const Et*)x;  // pooler input
  int xp_ld = 0;                // its row stride (0: H)
  const void* xr = x;           // router input
  if (c.input_norm) {
    float* xn = sizeof(Et) == 4 ? (float*)(ws + L.xn) : nullptr;
    uint16_t* xs = sizeof(Et) == 2 ? (uint16_t*)(ws + L.xna) : nullptr;
    hipLaunchKernelGGL(lm_input_norm_kernel<Et>, dim3((unsigned)T), dim3(256), 0, s, (const Et*)x, H,
                       w.input_gamma, c.eps, xn, xs);
    LM_HIP(hipGetLastError());
    xr = sizeof(Et) == 4 ? (const void*)xn : (const void*)xs;
    xp = (const Et*)xr;
    xp_ld = sizeof(Et) == 4 ? 0 : 3 * H;
  }
  LM_MARK(1);
  // Steps 1-3 (routing) depend only on x, as do the pooler and its norm
  // statistics (step 4): outside stage profiling, the pooler steps run on the
  // handle's side stream, forked from and joined back into the caller's
  // stream, so the two overlap. Routing, the longer of the two at decode
  // sizes, stays on the caller's stream: it reaches the join after the side
  // stream has finished, and the join then costs only the runtime's own
  // cross-stream wait, about 8 us measured (the other way round, the
  // caller's stream also idled until the side stream's routing ended, 12-13
  // us at the join in all). With stage profiling on, every step runs in
  // order on the caller's stream so the per-stage times are separable.
  const bool fork = !h->prof && h->side_ok;
  const hipStream_t sr = s;  // routing
  hipStream_t sp = s;        // pooler and the steps that read only its output
  if (fork) {
    LM_HIP(hipEventRecord(h->fork, s));
    LM_HIP(hipStreamWaitEvent(h->side, h->fork, 0));
    sp = h->side;
  }
  // 1. router: partial logits over k-splits
  {
    int splits, kt_per, mt, nt;
    router_split(c, T, splits, kt_per, mt, nt);
    RouterProb<Cr> p;
    p.x = (const Et*)xr;
    p.w = sizeof(Et) == 2 ? (const Et*)h->wr3 : (const Et*)w.router;
    p.part = part;
    p.T = (int)T;
    p.Ew = E;
    p.H = H;
    p.Kw = sizeof(Et) == 2 ? 3 * H : H;
    p.kta = H / Cr::KT;
    p.mt = mt;
    p.nt = nt;
    p.splits = splits;
    p.kt_per = kt_per;
    if (sizeof(Et) == 2 && c.input_norm) {
      p.lda = 3 * H;
      p.pieces = 3;
    }
    // the router's blocks also clear the expert counters the top-k kernel counts into
    p.counters = (lm_u32x4*)cpad;
    p.counter_chunks = E * kLmCountStride / 4;
    if (kt_per <= kRouterDeep) {  // decode sizes: each block's k-tiles all in flight at once
      const int64_t g = ((int64_t)mt * nt * splits + 7) / 8 * 8;
      hipLaunchKernelGGL((lm_gemm_kdeep_kernel<RouterProb<Cr>, kRouterDeep>), dim3((unsigned)g), dim3(256), 0,
                         sr, p);
      LM_HIP(hipGetLastError());
    } else {
      LM_HIP(launch(p, (int64_t)mt * nt * splits, sr));
    }
    LM_MARK(2);
    // 2. top-k + softmax + per-expert counts
    // few tokens with many k-splits: one token per workgroup spreads the
    // split sums over all threads; otherwise four tokens per workgroup
    const bool one = splits > 4;
    const dim3 g(one ? (unsigned)T : (unsigned)ceil_div(T, 4));
#define LM_TOPK(NV)                                                                             \
  do {                                                                                          \
    if (one)                                                                                    \
      hipLaunchKernelGGL((lm_topk_kernel<NV, 1>), g, dim3(1024), 0, sr, part, splits, (int)T, E, \
                         w.router_bias, k, logits, ids, wts, cpad);                             \
    else                                                                                        \
      hipLaunchKernelGGL((lm_topk_kernel<NV, 4>), g, dim3(256), 0, sr, part, splits, (int)T, E, \
                         w.router_bias, k, logits, ids, wts, cpad);                             \
  } while (0)
    if (E <= 64) LM_TOPK(1);
    else if (E <= 128) LM_TOPK(2);
    else if (E <= 256) LM_TOPK(4);
    else if (E <= 512) LM_TOPK(8);
    else LM_TOPK(16);
#undef LM_TOPK
    LM_HIP(hipGetLastError());
  }
  LM_MARK(3);
  // 3. grouping by expert
  hipLaunchKernelGGL(lm_permute_kernel, dim3(E), dim3(256), 0, sr, ids, npairs, k, cpad, E, kBmGroup,
                     counts, offsets, tile_off, perm_token, pair_row);
  LM_HIP(hipGetLastError());
  LM_MARK(4);
  // 4. pooler + norm statistics
  const int pnt = ceil_div(P, Cp::BN);
  int psplits = 1, pkt = 0;
  // the split decision on the split kernel's tiles (Cw), as the workspace
  // layout sizes its partials
  if (packed) dense_split(T, P, H, Cw::BM, Cw::BN, psplits, pkt);
  if (psplits > 1) {
    if constexpr (sizeof(Et) == 2) {
    DenseSplitProb<Cw> p;
    p.a = xp;
    p.lda = xp_ld;
    p.w = (const Et*)Wpool;
    p.part = (float*)(ws + L.kpart);
    p.T = (int)T;
    p.N = P;
    p.K = H;
    p.mt = ceil_div(T, Cw::BM);
    p.nt = ceil_div(P, Cw::BN);
    p.splits = psplits;
    p.kt_per = pkt;
    LM_HIP(launch(p, (int64_t)p.mt * p.nt * psplits, sp));
    LM_MARK(5);
    const int chunks = ceil_div(P, 256);
    hipLaunchKernelGGL(lm_pool_finish_kernel, dim3((unsigned)T, (unsigned)chunks), dim3(256), 0, sp,
                       (const float*)(ws + L.kpart), psplits, (int)T, P, w.pool_gamma, pssq, pooled32);
    LM_HIP(hipGetLastError());
    if (MXA) {
      hipLaunchKernelGGL(lm_rowscale_kernel, dim3(ceil_div(T, 256)), dim3(256), 0, sp, pssq, chunks,
                         (int)T, P, c.eps, row_scale);
    } else {
      hipLaunchKernelGGL(lm_norm_u_kernel, dim3((unsigned)T), dim3(256), 0, sp, pooled32, pssq, chunks,
                         P, c.eps, h->u_down, row_scale, (_Float16*)u16);
    }
    LM_HIP(hipGetLastError());
    }
  } else {
    PoolerProb<Cp> p;
    if (F16) p.pooled32 = pooled32;
    p.x = xp;
    p.lda = xp_ld;
    p.w = (const Et*)Wpool;
    p.gamma = w.pool_gamma;
    p.pooled = pooled;
    p.ssq = pssq;
    p.T = (int)T;
    p.H = H;
    p.P = P;
    p.mt = ceil_div(T, Cp::BM);
    p.nt = pnt;
    LM_HIP(launch(p, (int64_t)p.mt * p.nt, sp));
    LM_MARK(5);
    if (F16 && !MXA) {
      if constexpr (F16)
        hipLaunchKernelGGL(lm_norm_u_kernel, dim3((unsigned)T), dim3(256), 0, sp, pooled32, pssq, pnt,
                           P, c.eps, h->u_down, row_scale, u16);
    } else {
      hipLaunchKernelGGL(lm_rowscale_kernel, dim3(ceil_div(T, 256)), dim3(256), 0, sp, pssq, pnt,
                         (int)T, P, c.eps, row_scale);
    }
    LM_HIP(hipGetLastError());
  }
  if constexpr (MXA) {  // u = r * gamma_p * h MX-quantised for the expert GEMMs
    const int64_t nthr = T * (int64_t)(P / 32) * 8;
    hipLaunchKernelGGL(lm_quant_u_kernel<AB>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, sp,
                       pooled32, row_scale, (int)T, P, (uint8_t*)(ws + L.uq),
                       (uint8_t*)(ws + L.us));
    LM_HIP(hipGetLastError());
  }
  if (fork) {
    LM_HIP(hipEventRecord(h->join, sp));
    LM_HIP(hipStreamWaitEvent(s, h->join, 0));
  }
  LM_MARK(6);
  const int64_t max_tiles = ceil_div(npairs, kBmGroup) + (npairs < E ? npairs : E);
  // 5. gate/up + SwiGLU
  if constexpr (MXA) {
    GateUpMxaProb<Cw, AB> p;
    p.sg = h->pk_sgate;
    p.su = h->pk_sup;
    p.pooled = (const Et*)pooled32;
    p.wg = (const Et*)Wgate;
    p.wu = (const Et*)Wup;
    p.row_scale = row_scale;
    p.perm_token = perm_token;
    p.counts = counts;
    p.offsets = offsets;
    p.tile_off = tile_off;
    p.act = (Et*)act;
    p.P = P;
    p.I = I;
    p.Ex = E;
    p.nt = I / GateUpMxaProb<Cw, AB>::kCols;
    p.uq = (const uint8_t*)(ws + L.uq);
    p.us = (const uint8_t*)(ws + L.us);
    p.aq = (uint8_t*)act;
    p.as = (uint8_t*)(ws + L.acts);
    LM_HIP(launch_mxa(p, max_tiles * p.nt, s));
  } else {
    GateUpProb<Ce, MX> p;
    if constexpr (MX) {
      p.sg = h->pk_sgate;
      p.su = h->pk_sup;
    }
    if constexpr (F16) {
      p.dsg = h->ds_gate;
      p.dsu = h->ds_up;
      p.u_up = 1.0f / h->u_down;  // exact: a power of two
      p.a_down = h->a_down;
      p.pooled = u16;
    } else {
      p.pooled = (const Eh*)pooled;
    }
    p.wg = (const Eh*)Wgate;
    p.wu = (const Eh*)Wup;
    p.row_scale = row_scale;
    p.perm_token = perm_token;
    p.counts = counts;
    p.offsets = offsets;
    p.tile_off = tile_off;
    p.act = act;
    p.P = P;
    p.I = I;
    p.Ex = E;
    p.nt = I / GateUpProb<Ce, MX>::kCols;
    LM_HIP(launch(p, max_tiles * p.nt, s));
  }
  LM_MARK(7);
  // 6. down + per-row sum of squares partials
  const int dnt = ceil_div(P, MXA ? Cx::BN : Ce::BN);
  if constexpr (MXA) {
    DownMxaProb<Cx, AB> p;
    p.sd = h->pk_sdown;
    p.act = (const Et*)act;
    p.wd = (const Et*)Wdown;
    p.counts = counts;
    p.offsets = offsets;
    p.tile_off = tile_off;
    p.out = O;
    if (LM_O_F16) {
      p.out16 = (_Float16*)O;
      p.o_down = h->o_down;
      p.gamma = w.expert_gamma;
    }
    p.ssq = ossq;
    p.P = P;
    p.I = I;
    p.Ex = E;
    p.nt = dnt;
    p.aq = (const uint8_t*)act;
    p.as = (const uint8_t*)(ws + L.acts);
    LM_HIP(launch_mxa(p, max_tiles * p.nt, s));
  } else {
    DownProb<Ce, MX> p;
    if constexpr (MX) p.sd = h->pk_sdown;
    if constexpr (F16) p.dsd = h->ds_down;
    p.act = act;
    p.wd = (const Eh*)Wdown;
    p.counts = counts;
    p.offsets = offsets;
    p.tile_off = tile_off;
    p.out = O;
    if constexpr (F16 && LM_O_F16) {
      p.out16 = (_Float16*)O;
      p.o_down = h->o_down;
      p.gamma = w.expert_gamma;
    }
    p.ssq = ossq;
    p.P = P;
    p.I = I;
    p.Ex = E;
    p.nt = dnt;
    LM_HIP(launch(p, max_tiles * p.nt, s));
  }
  LM_MARK(8);
  // 7. per-expert norm, routing weight, FP32 sum
  constexpr bool kO16 = F16 && LM_O_F16;
  using OT = std::conditional_t<kO16, _Float16, float>;
  hipLaunchKernelGGL((lm_combine_kernel<OT, Eh>), dim3((unsigned)T), dim3(256), 0, s, (const OT*)O, ossq, dnt,
                     pair_row, ids, wts, w.expert_gamma, kO16 ? h->o_up : nullptr, k, P, c.eps,
                     F16 ? h->y_down : 1.0f, y);
  LM_HIP(hipGetLastError());
  LM_MARK(9);
  // 8. unpooler (BF16 layers: FP16 y against the per-row scaled FP16 copy of W)
  int usplits = 1, ukt = 0;
  if (packed) dense_split(T, H, P, Ch::BM, Ch::BN, usplits, ukt);  // the split kernel's tiles, as the layout
  if (usplits > 1) {
    if constexpr (F16) {
    DenseSplitProb<Ch> p;
    p.a = y;
    p.w = (const Eh*)Wunpool;
    p.ds = h->ds_unpooler;
    p.a_up = 1.0f / h->y_down;
    p.part = (float*)(ws + L.kpart);
    p.T = (int)T;
    p.N = H;
    p.K = P;
    p.mt = ceil_div(T, Ch::BM);
    p.nt = ceil_div(H, Ch::BN);
    p.splits = usplits;
    p.kt_per = ukt;
    LM_HIP(launch(p, (int64_t)p.mt * p.nt * usplits, s));
    const int64_t n = T * (int64_t)H;
    hipLaunchKernelGGL(lm_unpool_finish_kernel, dim3((unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192)),
                       dim3(256), 0, s, (const float*)(ws + L.kpart), usplits, n, out);
    LM_HIP(hipGetLastError());
    }
  } else {
    UnpoolerProb<Ce> p;
    p.y = y;
    p.w = (const Eh*)Wunpool;
    if constexpr (F16) {
      p.ds = h->ds_unpooler;
      p.y_up = 1.0f / h->y_down;
    }
    p.out = out;
    p.T = (int)T;
    p.H = H;
    p.P = P;
    p.mt = ceil_div(T, Ce::BM);
    p.nt = ceil_div(H, Ce::BN);
    LM_HIP(launch(p, (int64_t)p.mt * p.nt, s));
  }
  LM_MARK(10);
  if (h->prof) h->prof_valid = true;
  return LMOE_OK;
}

}  // namespace

extern "C" {

const char* latent_moe_last_error(void) { return g_err.c_str(); }

int latent_moe_workspace_bytes(const latent_moe_config* cfg, size_t* bytes) {
  g_err.clear();
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(LMOE_ERR_INVALID_ARG, "bytes is NULL");
  size_t pf;
  *bytes = make_layout(*cfg, &pf).total;
  return LMOE_OK;
}

int latent_moe_create(latent_moe_t** out, const latent_moe_config* cfg, const latent_moe_weights* w,
                      void* stream) {
  g_err.clear();
  if (!out) return fail(LMOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (!w) return fail(LMOE_ERR_INVALID_ARG, "weights is NULL");
  const void* req[] = {w->router, w->pooler, w->pool_gamma, w->w_gate, w->w_up,
                       w->w_down, w->expert_gamma, w->unpooler};
  const char* names[] = {"router", "pooler", "pool_gamma", "w_gate", "w_up",
                         "w_down", "expert_gamma", "unpooler"};
  for (int i = 0; i < 8; ++i) {
    if (!req[i]) return fail(LMOE_ERR_INVALID_ARG, "weight %s is NULL", names[i]);
    if (!aligned16(req[i])) return fail(LMOE_ERR_INVALID_ARG, "weight %s is not 16-byte aligned", names[i]);
  }
  if (w->router_bias && !aligned16(w->router_bias))
    return fail(LMOE_ERR_INVALID_ARG, "router_bias is not 16-byte aligned");
  if (cfg->input_norm && !w->input_gamma)
    return fail(LMOE_ERR_INVALID_ARG, "input_norm needs input_gamma");
  if (cfg->input_norm && !aligned16(w->input_gamma))
    return fail(LMOE_ERR_INVALID_ARG, "input_gamma is not 16-byte aligned");
  if (cfg->expert_dtype == LMOE_MXFP4) {
    const void* sc[] = {w->s_gate, w->s_up, w->s_down};
    const char* sn[] = {"s_gate", "s_up", "s_down"};
    for (int i = 0; i < 3; ++i) {
      if (!sc[i]) return fail(LMOE_ERR_INVALID_ARG, "MXFP4 scale array %s is NULL", sn[i]);
      if (!aligned16(sc[i])) return fail(LMOE_ERR_INVALID_ARG, "scale array %s is not 16-byte aligned", sn[i]);
    }
  }

  int ndev = 0;
  hipError_t he = hipGetDeviceCount(&ndev);
  if (he != hipSuccess || ndev == 0)
    return fail(LMOE_ERR_HIP, "no HIP device available (%s)", hipGetErrorString(he));
  int dev = 0;
  LM_HIP(hipGetDevice(&dev));
  const hipStream_t s = (hipStream_t)stream;

  latent_moe* h = new (std::nothrow) latent_moe();
  if (!h) return fail(LMOE_ERR_OOM, "host allocation failed");
  h->cfg = *cfg;
  h->device = dev;
  h->lay = make_layout(*cfg, &h->part_floats);
  h->poison = debug_poison();
  AllocCtl actl = alloc_ctl_from_env();
  // Every failure below releases what was made so far: the handle, its two
  // device allocations, the routing stream and its events.
  auto cleanup = [&](int code, const char* what, hipError_t e) {
    (void)hipGetLastError();
    if (h->ws || h->owned) (void)hipStreamSynchronize(s);  // no kernel of this call still reads them
    if (h->join) (void)hipEventDestroy(h->join);
    if (h->fork) (void)hipEventDestroy(h->fork);
    if (h->side) (void)hipStreamDestroy(h->side);
    if (h->ws) (void)hipFree(h->ws);
    if (h->owned) (void)hipFree(h->owned);
    delete h;
    return fail(code, "%s: %s", what, hipGetErrorString(e));
  };

  // 1. workspace (sized by max_tokens), plus the guard words in poison mode
  const size_t ws_bytes = h->lay.total + (h->poison ? kGuardBytes : 0);
  he = lm_malloc(actl, (void**)&h->ws, ws_bytes);
  if (he != hipSuccess) {
    h->ws = nullptr;
    char what[96];
    snprintf(what, sizeof what, "device allocation of %zu workspace bytes failed", ws_bytes);
    return cleanup(LMOE_ERR_OOM, what, he);
  }

  // 2. one allocation for the library's own copies of everything forward
  // reads: gammas, bias, and the weights (FP32 layers: as given; BF16 layers:
  // the router split and the packed matrix-core copies with their scales)
  const size_t E = cfg->experts, H = cfg->hidden, P = cfg->pooled, I = cfg->intermediate;
  const bool bf16 = cfg->act_dtype == LMOE_BF16;
  const bool mx = cfg->expert_dtype == LMOE_MXFP4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  const size_t o_bias = take(w->router_bias ? E * 4 : 0), o_gp = take(P * 4), o_ge = take(E * P * 4),
               o_gin = take(cfg->input_norm ? H * 4 : 0);
  // FP32 layers
  const size_t o_r = take(bf16 ? 0 : E * H * 4), o_p = take(bf16 ? 0 : P * H * 4),
               o_g = take(bf16 ? 0 : E * I * P * 4), o_u = take(bf16 ? 0 : E * I * P * 4),
               o_d = take(bf16 ? 0 : E * P * I * 4), o_un = take(bf16 ? 0 : H * P * 4);
  // BF16 layers
  const size_t sz_pool = bf16 ? H * P * 2 : 0, sz_exp = !bf16 ? 0 : mx ? E * I * P / 2 : E * I * P * 2;
  const size_t sz_sc = bf16 && mx ? E * I * P / 32 : 0;
  // per weight row 2^-s: gate, up [E*I], down [E*P], unpooler [H] (FP32); the SwiGLU
  // output's block shifts c (int) and 2^-c (FP32), [E, I/32] each; row norms of the
  // gate and up weights [2*E*I] (create-time scratch); largest |gamma_p|, |gamma_e|
  const size_t n_ds = bf16 ? 2 * E * I + E * P + H : 0, n_ab = bf16 ? E * I / 32 : 0;
  const size_t o_wr3 = take(bf16 ? E * 3 * H * 2 : 0), o_pp = take(sz_pool), o_pu = take(sz_pool),
               o_pg = take(sz_exp), o_pup = take(sz_exp), o_pd = take(sz_exp), o_sg = take(sz_sc),
               o_su = take(sz_sc), o_sd = take(sz_sc), o_ds = take(n_ds * 4), o_ash = take(n_ab * 4),
               o_ad = take(n_ab * 4), o_norm = take(bf16 ? (2 * E * I + E * P) * 4 : 0), o_gmax = take(bf16 ? 8 : 0),
               o_od = take(bf16 ? 2 * E * 4 : 0);
  h->owned_bytes = o;
  he = lm_malloc(actl, (void**)&h->owned, h->owned_bytes);
  if (he != hipSuccess) {
    h->owned = nullptr;
    char what[96];
    snprintf(what, sizeof what, "device allocation of %zu bytes for the weight copies failed", h->owned_bytes);
    return cleanup(LMOE_ERR_OOM, what, he);
  }
  char* ob = h->owned;
  auto copy = [&](size_t at, const void* src, size_t bytes) {
    return bytes ? hipMemcpyAsync(ob + at, src, bytes, hipMemcpyDeviceToDevice, s) : hipSuccess;
  };
  latent_moe_weights& hw = h->w;
  hw = latent_moe_weights{};
  he = copy(o_gp, w->pool_gamma, P * 4);
  if (he == hipSuccess) he = copy(o_ge, w->expert_gamma, E * P * 4);
  if (he == hipSuccess && w->router_bias) he = copy(o_bias, w->router_bias, E * 4);
  if (he == hipSuccess && cfg->input_norm) he = copy(o_gin, w->input_gamma, H * 4);
  hw.pool_gamma = (const float*)(ob + o_gp);
  hw.expert_gamma = (const float*)(ob + o_ge);
  hw.router_bias = w->router_bias ? (const float*)(ob + o_bias) : nullptr;
  hw.input_gamma = cfg->input_norm ? (const float*)(ob + o_gin) : nullptr;
  if (he == hipSuccess && !bf16) {
    he = copy(o_r, w->router, E * H * 4);
    if (he == hipSuccess) he = copy(o_p, w->pooler, P * H * 4);
    if (he == hipSuccess) he = copy(o_g, w->w_gate, E * I * P * 4);
    if (he == hipSuccess) he = copy(o_u, w->w_up, E * I * P * 4);
    if (he == hipSuccess) he = copy(o_d, w->w_down, E * P * I * 4);
    if (he == hipSuccess) he = copy(o_un, w->unpooler, H * P * 4);
    hw.router = (const float*)(ob + o_r);
    hw.pooler = ob + o_p;
    hw.w_gate = ob + o_g;
    hw.w_up = ob + o_u;
    hw.w_down = ob + o_d;
    hw.unpooler = ob + o_un;
  }
  if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "weight copy failed", he);

  if (bf16) {
    h->wr3 = ob + o_wr3;
    h->pk_pooler = ob + o_pp;
    h->pk_unpooler = ob + o_pu;
    h->pk_gate = ob + o_pg;
    h->pk_up = ob + o_pup;
    h->pk_down = ob + o_pd;
    h->pk_sgate = ob + o_sg;
    h->pk_sup = ob + o_su;
    h->pk_sdown = ob + o_sd;
    float* ds = (float*)(ob + o_ds);
    h->ds_gate = ds;
    h->ds_up = ds + E * I;
    h->ds_down = ds + 2 * E * I;
    h->ds_unpooler = ds + 2 * E * I + E * P;
    int* a_shift = (int*)(ob + o_ash);
    float* a_down = (float*)(ob + o_ad);
    float* norms = (float*)(ob + o_norm);
    float* gmax = (float*)(ob + o_gmax);
    // Largest |gamma_p| and |gamma_e| (for the FP16 ranges of u, a and y below).
    hipLaunchKernelGGL(lm_absmax_kernel, dim3(1), dim3(256), 0, s, hw.pool_gamma, (int64_t)P, gmax);
    hipLaunchKernelGGL(lm_absmax_kernel, dim3(1), dim3(256), 0, s, hw.expert_gamma, (int64_t)(E * P), gmax + 1);
    float gm[2] = {0.0f, 0.0f};
    he = hipGetLastError();
    if (he == hipSuccess) he = hipMemcpyAsync(gm, gmax, sizeof gm, hipMemcpyDeviceToHost, s);
    if (he == hipSuccess) he = hipStreamSynchronize(s);
    // Row norms of the gate, up and down weights: the FP16 ranges of a and of
    // the expert outputs follow from them.
    const int* kc = nullptr;
    h->a_down = nullptr;
    const float u2 = (float)((double)P * (double)gm[0] * (double)gm[0]);
    if (he == hipSuccess) {
      const unsigned nb = (unsigned)((E * I + 3) / 4 < 65536 ? (E * I + 3) / 4 : 65536);
      const unsigned nbd = (unsigned)((E * P + 3) / 4 < 65536 ? (E * P + 3) / 4 : 65536);
      if (mx) {
        hipLaunchKernelGGL(lm_row_norm_mx_kernel, dim3(nb), dim3(256), 0, s, (const uint8_t*)w->w_gate,
                           (const uint8_t*)w->s_gate, (int64_t)(E * I), (int)P, norms);
        hipLaunchKernelGGL(lm_row_norm_mx_kernel, dim3(nb), dim3(256), 0, s, (const uint8_t*)w->w_up,
                           (const uint8_t*)w->s_up, (int64_t)(E * I), (int)P, norms + E * I);
        hipLaunchKernelGGL(lm_row_norm_mx_kernel, dim3(nbd), dim3(256), 0, s, (const uint8_t*)w->w_down,
                           (const uint8_t*)w->s_down, (int64_t)(E * P), (int)I, norms + 2 * E * I);
      } else {
        hipLaunchKernelGGL(lm_row_norm_bf16_kernel, dim3(nb), dim3(256), 0, s, (const uint16_t*)w->w_gate,
                           (int64_t)(E * I), (int)P, norms);
        hipLaunchKernelGGL(lm_row_norm_bf16_kernel, dim3(nb), dim3(256), 0, s, (const uint16_t*)w->w_up,
                           (int64_t)(E * I), (int)P, norms + E * I);
        hipLaunchKernelGGL(lm_row_norm_bf16_kernel, dim3(nbd), dim3(256), 0, s, (const uint16_t*)w->w_down,
                           (int64_t)(E * P), (int)I, norms + 2 * E * I);
      }
      // FP16 expert outputs: one power of two per expert (lm_o_shift_kernel);
      // an MX-quantised a may exceed silu(g) v by up to a factor 1.5
      float* od = (float*)(ob + o_od);
      hipLaunchKernelGGL(lm_o_shift_kernel, dim3((unsigned)E), dim3(256), 0, s, norms, norms + E * I,
                         norms + 2 * E * I, hw.expert_gamma, (int)I, (int)P, u2, cfg->expert_act ? 2.0f : 1.0f,
                         od, od + E);
      h->o_down = od;
      h->o_up = od + E;
      // FP16 a (expert inputs in FP16 only; MX inputs quantise a per block): per
      // expert and block of 32 intermediate columns, the shift from the norms of
      // the gate and up rows (lm_a_shift_kernel); the down weights carry it.
      if (cfg->expert_act == 0) {
        hipLaunchKernelGGL(lm_a_shift_kernel, dim3((unsigned)((n_ab + 255) / 256)), dim3(256), 0, s, norms,
                           norms + E * I, (int64_t)n_ab, u2, a_shift, a_down);
        kc = a_shift;
        h->a_down = a_down;
      }
      he = hipGetLastError();
    }
    if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "weight range analysis failed", he);
    // The pooler stays BF16 (x is BF16). The unpooler and BF16 experts become
    // FP16 copies scaled per row by 2^s; MXFP4 experts keep their codes and
    // get the per-row 2^s applied when they are decoded.
    struct Job { const void* src; const void* src_s; const void* dst; const void* dst_s; int64_t rows; int K;
                 bool mx; const float* ds; const int* kc; int64_t rows_per_set; };
    const Job jobs[] = {
        {w->pooler, nullptr, h->pk_pooler, nullptr, (int64_t)P, (int)H, false, nullptr, nullptr, 1},
        {w->unpooler, nullptr, h->pk_unpooler, nullptr, (int64_t)H, (int)P, false, h->ds_unpooler, nullptr, 1},
        {w->w_gate, w->s_gate, h->pk_gate, h->pk_sgate, (int64_t)(E * I), (int)P, mx, h->ds_gate, nullptr, 1},
        {w->w_up, w->s_up, h->pk_up, h->pk_sup, (int64_t)(E * I), (int)P, mx, h->ds_up, nullptr, 1},
        {w->w_down, w->s_down, h->pk_down, h->pk_sdown, (int64_t)(E * P), (int)I, mx, h->ds_down, kc,
         (int64_t)P}};
    for (const Job& j : jobs) {
      if (j.mx) {
        hipLaunchKernelGGL(lm_row_descale_mx_kernel, dim3((unsigned)((j.rows + 255) / 256)), dim3(256), 0, s,
                           (const uint8_t*)j.src_s, j.rows, j.K, (float*)j.ds, j.kc, j.rows_per_set);
        hipLaunchKernelGGL(lm_pack_mx_kernel, dim3(65536), dim3(256), 0, s, (const lm_u32x4*)j.src,
                           (const uint8_t*)j.src_s, (lm_u32x4*)j.dst, (uint8_t*)j.dst_s, j.rows, j.K, j.kc,
                           j.rows_per_set);
      } else {
        if (j.ds)
          hipLaunchKernelGGL(lm_row_descale_bf16_kernel, dim3((unsigned)((j.rows + 3) / 4 < 65536 ? (j.rows + 3) / 4 : 65536)),
                             dim3(256), 0, s, (const uint16_t*)j.src, j.rows, j.K, (float*)j.ds, j.kc,
                             j.rows_per_set);
        hipLaunchKernelGGL(lm_pack_mfma_kernel, dim3(65536), dim3(256), 0, s, (const lm_u32x4*)j.src,
                           (lm_u32x4*)j.dst, j.rows, j.K, j.ds, j.kc, j.rows_per_set);
      }
    }
    const size_t n = E * H;
    unsigned blocks = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
    hipLaunchKernelGGL(lm_split_router_kernel, dim3(blocks), dim3(256), 0, s, w->router, (uint16_t*)h->wr3,
                       (int)E, (int)H);
    he = hipGetLastError();
    if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "weight repack failed", he);
    // FP16 u and y: |u| <= sqrt(P) max|gamma_p| and |y| <= sqrt(P) max|gamma_e| (an
    // RMS-normed row has no element above sqrt(P) times its gamma, and the routing
    // weights sum to one); each is stored times a power of two that keeps its bound
    // within 2^15, undone exactly in FP32 after the product (1 for ordinary gammas).
    auto down_for = [&](float g) {
      const double bound = std::sqrt((double)P) * (double)g;
      if (!(bound > 32768.0) || !std::isfinite(bound)) return 1.0f;
      int e = 0;
      std::frexp(bound / 32768.0, &e);  // bound / 2^15 <= 2^e
      return std::ldexp(1.0f, -(e < 100 ? e : 100));
    };
    h->u_down = down_for(gm[0]);
    h->y_down = down_for(gm[1]);
  }
  if (h->poison) {  // workspace all 0xFF bytes (NaN floats, -1 ints), guard words after it
    he = lm_fill_launch(h->ws, h->lay.total, 0xFFFFFFFFu, s);
    if (he == hipSuccess) he = lm_fill_launch(h->ws + h->lay.total, kGuardBytes, kGuardWord, s);
    if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "workspace poison failed", he);
  }
  // side stream for the pooler steps (default priority) and its fork / join events
  he = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
  if (he == hipSuccess) he = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
  if (he == hipSuccess) he = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
  if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "stream / event creation failed", he);
  h->side_ok = true;
  // the copies are complete before create returns: the caller may free its tensors
  he = hipStreamSynchronize(s);
  if (he != hipSuccess) return cleanup(LMOE_ERR_HIP, "create", he);
  *out = h;
  return LMOE_OK;
}

int latent_moe_forward(latent_moe_t* h, const void* x, int64_t T, float* out, int32_t* topk_ids,
                       float* topk_weights, void* stream) {
  g_err.clear();
  if (!h) return fail(LMOE_ERR_INVALID_ARG, "handle is NULL");
  if (T < 0) return fail(LMOE_ERR_INVALID_ARG, "T must be >= 0");
  if (T > h->cfg.max_tokens)
    return fail(LMOE_ERR_TOO_MANY_TOKENS, "T=%lld exceeds max_tokens=%lld", (long long)T,
                (long long)h->cfg.max_tokens);
  if (T == 0) return LMOE_OK;
  if (!x || !out) return fail(LMOE_ERR_INVALID_ARG, "x and out must be non-NULL");
  if (!aligned16(x) || !aligned16(out) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_weights && !aligned16(topk_weights)))
    return fail(LMOE_ERR_INVALID_ARG, "x, out, topk_ids and topk_weights must be 16-byte aligned");
  int cur = -1;
  LM_HIP(hipGetDevice(&cur));
  if (cur != h->device) LM_HIP(hipSetDevice(h->device));
  hipStream_t s = (hipStream_t)stream;
  int rc;
  const bool nar = narrow_for(h->cfg, T);
  if (h->cfg.act_dtype == LMOE_F32)
    rc = nar ? forward_impl<float, CfgNarrow, CfgRouterNarrow>(h, x, T, out, s)
             : forward_impl<float, CfgWide, CfgRouterWide>(h, x, T, out, s);
  else if (h->cfg.expert_dtype == LMOE_MXFP4 && h->cfg.expert_act == LMOE_MXFP8)
    rc = nar ? forward_impl<uint16_t, CfgNarrow, CfgRouterNarrow, true, 8>(h, x, T, out, s)
             : forward_impl<uint16_t, CfgWide, CfgRouterWide, true, 8>(h, x, T, out, s);
  else if (h->cfg.expert_dtype == LMOE_MXFP4 && h->cfg.expert_act == LMOE_MXFP4)
    rc = nar ? forward_impl<uint16_t, CfgNarrow, CfgRouterNarrow, true, 4>(h, x, T, out, s)
             : forward_impl<uint16_t, CfgWide, CfgRouterWide, true, 4>(h, x, T, out, s);
  else if (h->cfg.expert_dtype == LMOE_MXFP4)
    rc = nar ? forward_impl<uint16_t, CfgNarrow, CfgRouterNarrow, true>(h, x, T, out, s)
             : forward_impl<uint16_t, CfgWide, CfgRouterWide, true>(h, x, T, out, s);
  else
    rc = nar ? forward_impl<uint16_t, CfgNarrow, CfgRouterNarrow>(h, x, T, out, s)
             : forward_impl<uint16_t, CfgWide, CfgRouterWide>(h, x, T, out, s);
  if (rc == LMOE_OK) {
    const size_t nk = (size_t)T * h->cfg.top_k;
    if (topk_ids)
      rc = hipMemcpyAsync(topk_ids, h->ws + h->lay.ids, nk * 4, hipMemcpyDeviceToDevice, s) == hipSuccess
               ? LMOE_OK : fail(LMOE_ERR_HIP, "copy of topk_ids failed");
    if (rc == LMOE_OK && topk_weights)
      rc = hipMemcpyAsync(topk_weights, h->ws + h->lay.wts, nk * 4, hipMemcpyDeviceToDevice, s) == hipSuccess
               ? LMOE_OK : fail(LMOE_ERR_HIP, "copy of topk_weights failed");
  }
  if (cur != h->device) (void)hipSetDevice(cur);
  return rc;
}

// ------------------------------------------------------------ no allocation
// latent_moe_forward_static: the FP32 layer's forward with its workspace in a
// file-scope device array instead of a handle's allocation. In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// comes from hipGetSymbolAddress, once per device (each device holds its own
// copy), and only that address is handed to kernels.
}  // extern "C"

static __device__ __align__(256) char scratch[LMOE_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of this device's scratch array (the current device).
int scratch_address(int dev, char** p) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LMOE_ERR_HIP, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* q = nullptr;
    const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q)
      return fail(LMOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_dev[dev] = q;
  }
  *p = (char*)g_scratch_dev[dev];
  return LMOE_OK;
}
}  // namespace

extern "C" {

int latent_moe_forward_static(const latent_moe_config* cfg, const latent_moe_weights* w, const void* x,
                              int64_t T, float* out, int32_t* topk_ids, float* topk_weights, void* stream) {
  g_err.clear();
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (cfg->act_dtype != LMOE_F32)
    return fail(LMOE_ERR_UNSUPPORTED, "the static-workspace forward runs FP32 layers only (BF16 layers use "
                                      "weight copies made by latent_moe_create)");
  if (!w) return fail(LMOE_ERR_INVALID_ARG, "weights is NULL");
  const void* req[] = {w->router, w->pooler, w->pool_gamma, w->w_gate, w->w_up,
                       w->w_down, w->expert_gamma, w->unpooler};
  for (int i = 0; i < 8; ++i)
    if (!req[i] || !aligned16(req[i])) return fail(LMOE_ERR_INVALID_ARG, "a weight is NULL or misaligned");
  if ((w->router_bias && !aligned16(w->router_bias)) ||
      (cfg->input_norm && (!w->input_gamma || !aligned16(w->input_gamma))))
    return fail(LMOE_ERR_INVALID_ARG, "router_bias or input_gamma misaligned or missing");
  if (T < 0) return fail(LMOE_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return LMOE_OK;
  if (!x || !out) return fail(LMOE_ERR_INVALID_ARG, "x and out must be non-NULL");
  if (!aligned16(x) || !aligned16(out) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_weights && !aligned16(topk_weights)))
    return fail(LMOE_ERR_INVALID_ARG, "x, out, topk_ids and topk_weights must be 16-byte aligned");
  latent_moe hs{};
  hs.cfg = *cfg;
  hs.cfg.max_tokens = T;
  if (T * cfg->top_k > (1 << 28)) return fail(LMOE_ERR_TOO_MANY_TOKENS, "T too large");
  hs.lay = make_layout(hs.cfg, &hs.part_floats);
  if (hs.lay.total > (size_t)LMOE_STATIC_SCRATCH_BYTES)
    return fail(LMOE_ERR_TOO_MANY_TOKENS, "T=%lld needs %zu workspace bytes, above the static scratch of %zu",
                (long long)T, hs.lay.total, (size_t)LMOE_STATIC_SCRATCH_BYTES);
  int dev = 0;
  LM_HIP(hipGetDevice(&dev));
  rc = scratch_address(dev, &hs.ws);
  if (rc) return rc;
  hs.w = *w;  // read in place for the duration of the call
  hs.device = dev;
  const hipStream_t s = (hipStream_t)stream;
  rc = narrow_for(hs.cfg, T) ? forward_impl<float, CfgNarrow, CfgRouterNarrow>(&hs, x, T, out, s)
                             : forward_impl<float, CfgWide, CfgRouterWide>(&hs, x, T, out, s);
  if (rc == LMOE_OK) {
    const size_t nk = (size_t)T * cfg->top_k;
    if (topk_ids && hipMemcpyAsync(topk_ids, hs.ws + hs.lay.ids, nk * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return fail(LMOE_ERR_HIP, "copy of topk_ids failed");
    if (topk_weights && hipMemcpyAsync(topk_weights, hs.ws + hs.lay.wts, nk * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return fail(LMOE_ERR_HIP, "copy of topk_weights failed");
  }
  return rc;
}

int latent_moe_debug_views(const latent_moe_t* h, latent_moe_views* v) {
  g_err.clear();
  if (!h || !v) return fail(LMOE_ERR_INVALID_ARG, "handle and views must be non-NULL");
  char* ws = h->ws;
  const Layout& L = h->lay;
  v->logits = (const float*)(ws + L.logits);
  v->ids = (const int32_t*)(ws + L.ids);
  v->weights = (const float*)(ws + L.wts);
  v->counts = (const int32_t*)(ws + L.counts);
  v->offsets = (const int32_t*)(ws + L.offsets);
  v->perm_token = (const int32_t*)(ws + L.perm_token);
  v->pair_row = (const int32_t*)(ws + L.pair_row);
  v->pooled = ws + L.pooled;
  v->row_scale = (const float*)(ws + L.row_scale);
  v->act = ws + L.act;
  v->expert_out = (const void*)(ws + L.O);
  v->combined = ws + L.y;
  const bool mxa = h->cfg.expert_act != 0;
  v->expert_in = mxa ? (const uint8_t*)(ws + L.uq)
                 : h->cfg.act_dtype == LMOE_BF16 ? (const uint8_t*)(ws + L.u16) : nullptr;
  v->expert_in_scales = mxa ? (const uint8_t*)(ws + L.us) : nullptr;
  v->act_scales = mxa ? (const uint8_t*)(ws + L.acts) : nullptr;
  v->x_norm = !h->cfg.input_norm ? nullptr
              : h->cfg.act_dtype == LMOE_F32 ? (const void*)(ws + L.xn) : (const void*)(ws + L.xna);
  v->expert_in_scale = mxa || h->cfg.act_dtype == LMOE_F32 ? 1.0f : h->u_down;
  v->combined_scale = h->cfg.act_dtype == LMOE_F32 ? 1.0f : h->y_down;
  v->act_down = h->cfg.act_dtype == LMOE_F32 ? nullptr : h->a_down;
  v->expert_out_down = h->cfg.act_dtype == LMOE_F32 ? nullptr : h->o_down;
  return LMOE_OK;
}

int latent_moe_set_profiling(latent_moe_t* h, int enable) {
  g_err.clear();
  if (!h) return fail(LMOE_ERR_INVALID_ARG, "handle is NULL");
  if (enable && !h->ev[0]) {
    for (int i = 0; i <= kStages; ++i) {
      hipError_t e = hipEventCreate(&h->ev[i]);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) {
          (void)hipEventDestroy(h->ev[j]);
          h->ev[j] = nullptr;
        }
        return fail(LMOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
      }
    }
  }
  h->prof = enable != 0;
  h->prof_valid = false;
  return LMOE_OK;
}

int latent_moe_stage_times(latent_moe_t* h, float* ms, int n) {
  g_err.clear();
  if (!h || !ms || n < kStages) return fail(LMOE_ERR_INVALID_ARG, "need a handle and %d floats", kStages);
  if (!h->prof || !h->prof_valid)
    return fail(LMOE_ERR_INVALID_ARG, "no profiled forward since profiling was enabled");
  LM_HIP(hipEventSynchronize(h->ev[kStages]));
  for (int i = 0; i < kStages; ++i) LM_HIP(hipEventElapsedTime(&ms[i], h->ev[i], h->ev[i + 1]));
  return LMOE_OK;
}

int latent_moe_destroy(latent_moe_t* h) {
  g_err.clear();
  if (!h) return fail(LMOE_ERR_INVALID_ARG, "handle is NULL");
  int cur = -1;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(h->device);
  hipError_t e1 = hipDeviceSynchronize();
  size_t bad = 0;
  if (h->poison && e1 == hipSuccess) {  // guard words after the workspace
    uint32_t* g = (uint32_t*)malloc(kGuardBytes);
    if (g && hipMemcpy(g, h->ws + h->lay.total, kGuardBytes, hipMemcpyDeviceToHost) == hipSuccess)
      for (size_t i = 0; i < kGuardBytes / 4; ++i) bad += g[i] != kGuardWord;
    free(g);
  }
  hipError_t e2 = hipFree(h->ws);
  if (h->owned) {
    hipError_t e3 = hipFree(h->owned);
    if (e2 == hipSuccess) e2 = e3;
  }
  for (int i = 0; i <= kStages; ++i)
    if (h->ev[i]) (void)hipEventDestroy(h->ev[i]);
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
  delete h;
  if (e1 != hipSuccess || e2 != hipSuccess)
    return fail(LMOE_ERR_HIP, "destroy: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  if (bad) return fail(LMOE_ERR_CORRUPT, "destroy: %zu guard words after the workspace were overwritten", bad);
  return LMOE_OK;
}

}  // extern "C"
