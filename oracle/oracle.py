"""FP64 oracle of the latent-MoE layer forward (test infrastructure only).

What the layer computes, for each token t (all arithmetic in FP64 on the exact
input values; BF16/FP32 inputs widen exactly, MXFP4 weights decode exactly):

0. Optional boundary norm, when an input gamma is given ([vllm] "三明治归一化":
   a block sees the normalised residual, x + post_norm(F(norm(x))); [vllm]
   "硬件后端 / Nvidia": the router GEMM is driven by the norm's FP32 output;
   [lmsys] "Fuse normalization and remove routing conversions": the boundary
   kernel normalises each row in registers): the input is then the pre-norm
   residual r_t and x_t = r_t / sqrt(mean(r_t^2) + eps) * gamma_in, held in
   FP32 (nearest). The router reads that FP32 value; the pooler reads it in
   the activation format (BF16 nearest-even for BF16 inputs, else FP32).

1. Router on the full-width token ([lmsys] "MoE with Pooler, Unpooler and
   Per-Expert Normalization": the router reads the full-width representation;
   [vllm] "硬件后端 / Nvidia": the router GEMM is driven by the norm's FP32
   output):  l_t = Wr x_t + b.
2. Top-k selection. The router works in FP32, so the selection is decided on
   the FP32 rounding of l_t: experts ordered by (logit descending, index
   ascending), the first k kept, slot j holding the j-th largest.
3. Routing weights: softmax over the k selected (FP64) logits.
4. Pooler and pre-expert RMSNorm ([lmsys] same section: the pooler compresses
   the width, and the pooled expert input is normalised before the experts;
   [vllm] "潜空间 MoE": an 8192x4096 pooler shared by all 256 experts):
   h_t = Wp x_t,  u_t = h_t / sqrt(mean(h_t^2) + eps) * gamma_p.
5. Each selected SwiGLU expert e ([lmsys] same section, "routed SwiGLU experts"):
   g = Wg_e u_t, v = Wu_e u_t, a = silu(g) * v with silu(z) = z / (1 + e^-z),
   o = Wd_e a. Optional MX activations (act_quant="mxfp8"; the "fp8 x fp4" MMA
   kind of [lmsys] "NVFP4 as a third MMA kind", with the pre-expert norm folded
   into the quantiser as in [lmsys] "Fuse normalization and remove routing
   conversions"): the expert GEMMs read u and a MX-quantised to FP8 E4M3 in
   blocks of 32 along their reduction axis (oracle/mx.py).
6. Per-expert RMSNorm before the routing weight ([lmsys] same section, and
   "The Fused Post-per-expert Norm"):  o^ = o / sqrt(mean(o^2) + eps) * gamma_e.
7. Routing-weighted sum ([lmsys] "Trainable Muse Spark Open Backend": each
   expert output normalised independently, then summed with its routing
   weight in FP32; here in FP64, slot order j = 1..k): y_t = sum_j w_tj o^_tj.
8. Unpooler back to the model width ([lmsys] same MoE section; [vllm]
   "潜空间 MoE"): out_t = Wun y_t.

Emulation mode (emulate="f16"): the same steps with the layer's own rounding
points applied, so that a kernel can be checked far tighter than the FP64
bound. With BF16 activations the expert and unpooler products run on FP16
operands that the layer forms itself: u (step 4), the SwiGLU output a (step 5)
and the combined y (step 7) are each rounded to FP16 (nearest even,
saturating at 65504) after multiplication by a power of two fixed at create,
and divided by it again after the product (the products themselves are exact
in FP16 x FP16 -> FP32 up to FP32 accumulation). The powers of two follow
bounds on each value: |u_i| <= sqrt(P) max|gamma_p| and |y_i| <= sqrt(P)
max|gamma_e| (no element of an RMS-normed row exceeds sqrt(P) times its
gamma; routing weights sum to one), and per expert and block of 32 SwiGLU
outputs |a_i| <= ||Wg_i|| ||Wu_i|| P max(gamma_p)^2 (Cauchy-Schwarz, |silu(g)|
<= |g|); each value is stored times the largest power of two that keeps its
bound within 2^15 (1 when the bound already is). The expert output, times
its expert's gamma (step 6's gamma_e * o), is stored in FP16 too, one power of
two per expert from |o_p gamma_p| <= ||Wd_p|| ||a|| max|gamma_e| <= max_p
||Wd_p|| P max(gamma_p)^2 sqrt(sum_i (||Wg_i|| ||Wu_i||)^2) max|gamma_e|
(twice that with MX activations: a code may exceed its value by up to a
factor 1.5); the per-expert RMS (step 6) is that of the unrounded o. With MX
activations (act_quant) u and a are the MX codes instead and only gamma_e * o
and y are FP16.

Readings where the pages are silent (each listed in the design notes): without
an input gamma, x is already the normed token (the sandwich norm sits outside
the layer, [vllm] "三明治归一化"); gammas multiply directly; one eps for all
norms; no biases
in any linear except an optional router bias, which is part of the logits;
per-expert gamma has shape [E, P].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

from .mx import quantize_mx, to_f64

NEAR_TIE = 1e-6


@dataclass
class OracleResult:
    out: np.ndarray  # [T, H] f64
    ids: np.ndarray  # [T, k] int64, slot order
    w: np.ndarray  # [T, k] f64
    logits: np.ndarray  # [T, E] f64
    gaps: np.ndarray  # [T, k] f64: sorted-logit gaps l(j) - l(j+1), j = 1..k
    h: np.ndarray  # [T, P] pooled, before the norm
    u: np.ndarray  # [T, P] pooled and normed expert input
    a: np.ndarray | None  # [T, k, I] SwiGLU output per slot
    o: np.ndarray | None  # [T, k, P] expert output per slot before its norm (emulation: gamma_e * o as stored)
    ohat: np.ndarray | None  # [T, k, P] normed expert output per slot
    # a, o and ohat hold the rows of all tokens, or (keep_pairs given as token
    # indices) of those tokens only, in the order given
    y: np.ndarray  # [T, P] combined
    near_tie: np.ndarray  # [T] bool: some gap j <= k below NEAR_TIE
    xn: np.ndarray | None = None  # [T, H] FP32 boundary-norm output (input gamma given)
    u_pre: np.ndarray | None = None  # [T, P] MX activations: u before its quantisation


def rms_norm(v: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * gamma over the last axis."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * gamma


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def router_logits(x: np.ndarray, router: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    lg = x @ router.T
    if bias is not None:
        lg = lg + bias
    return lg


def select_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k ids decided on the FP32-rounded logits, ties to the lowest index.

    Returns (ids [T, k], gaps [T, k]); gaps come from the FP64 logits sorted
    descending (index ascending on equal values)."""
    T, E = logits.shape
    l32 = logits.astype(np.float32)
    idx = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> (-l32) primary, index secondary
    order = np.lexsort((idx, -l32.astype(np.float64)), axis=-1)
    ids = order[:, :k].astype(np.int64)
    order64 = np.lexsort((idx, -logits), axis=-1)
    srt = np.take_along_axis(logits, order64, axis=-1)
    kk = min(k + 1, E)
    g = srt[:, : kk - 1] - srt[:, 1:kk]
    if kk - 1 < k:  # k == E: no (k+1)-th logit; last gap is infinite
        g = np.concatenate([g, np.full((T, k - (kk - 1)), np.inf)], axis=1)
    return ids, g


def softmax_selected(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(logits, ids, axis=-1)
    m = sel.max(axis=-1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=-1, keepdims=True)


ExpertFn = Callable[[int], tuple[np.ndarray, np.ndarray, np.ndarray]]


def experts_from_arrays(w_gate, w_up, w_down) -> ExpertFn:
    """Expert accessor over stored arrays ([E, N, K] float32 / BF16 bits, or
    MXFP4 (packed, scales) pairs); returns FP64 (Wg [I,P], Wu [I,P], Wd [P,I])."""

    def pick(a, e):
        return (a[0][e], a[1][e]) if isinstance(a, tuple) else a[e]

    def fn(e: int):
        return to_f64(pick(w_gate, e)), to_f64(pick(w_up, e)), to_f64(pick(w_down, e))

    return fn


def forward(x, router, router_bias, pooler, pool_gamma, experts: ExpertFn, expert_gamma,
            unpooler, k: int, eps: float, *, force_ids: dict | None = None,
            order: str = "norm_then_sum", keep_pairs: bool = True,
            emulate=None, input_gamma=None,
            act_quant: str | None = None, force_u: dict | None = None):
    """Layer forward on tokens x [T, H] (any stored dtype).

    force_ids: {token: ids sequence} replaces the selection for those tokens
      (weights recomputed from this oracle's own FP64 logits).
    order: "norm_then_sum" is the layer; "sum_then_norm" normalises the
      combined vector instead (used only to show that the two differ).
    emulate: None (the exact definition) or "f16": u, a and y rounded to FP16
      at the layer's declared points with their power-of-two range scalings
      (module docstring; f16_scales). A tuple of these returns a list of
      results, one per mode, computed in one pass over the experts (each
      expert's weights fetched once).
    input_gamma: [H] gamma of the boundary norm (step 0); x is then the
      pre-norm residual.
    act_quant: None, "mxfp8" or "mxfp4": the expert GEMMs read u and a
      MX-quantised.
    force_u: {token: quantised u row} replaces the quantised u of those tokens
      (an element whose value sits on the midpoint between two codes may be
      rounded either way by a kernel that forms it in lower precision; the
      caller checks that the rows differ from this oracle's only there).
    keep_pairs: True keeps the per-slot a, o and ohat of every token; False
      none; a sequence of token indices keeps those tokens' rows only (in
      that order). The output is the same in every case.
    """
    modes = tuple(emulate) if isinstance(emulate, (tuple, list)) else (emulate,)
    for m in modes:
        if m not in (None, "f16"):
            raise ValueError(f"unknown emulation {m!r}")
    act_bf16 = np.asarray(x).dtype == np.uint16
    x = to_f64(x)
    xn = None
    x_router = x
    if input_gamma is not None:
        xn = rms_norm(x, to_f64(input_gamma), eps).astype(np.float32).astype(np.float64)
        x_router = xn
        x = _bf16_round(xn) if act_bf16 else xn
    Wr = to_f64(router)
    b = None if router_bias is None else to_f64(router_bias)
    Wp = to_f64(pooler)
    gp = to_f64(pool_gamma)
    ge = to_f64(expert_gamma)
    Wun = to_f64(unpooler)
    T = x.shape[0]
    P = Wp.shape[0]

    logits = router_logits(x_router, Wr, b)
    ids, gaps = select_topk(logits, k)
    if force_ids:
        ids = ids.copy()
        for t, seq in force_ids.items():
            ids[t] = np.asarray(seq, dtype=np.int64)
    w = softmax_selected(logits, ids)
    near = (gaps < NEAR_TIE).any(axis=-1)

    h = x @ Wp.T
    u_exact = rms_norm(h, gp, eps)
    sc = f16_scales(gp, ge, P) if "f16" in modes else None
    u_pre = None
    if act_quant:
        u_pre = u_exact
        uq = quantize_mx(u_exact, act_quant)[0]
        if force_u:
            uq = uq.copy()
            for t, row in force_u.items():
                uq[t] = row

    # tokens whose per-slot rows are kept, and each token's row among them (-1: not kept)
    if keep_pairs is True:
        kept = np.arange(T)
    elif keep_pairs is False or keep_pairs is None:
        kept = np.zeros(0, dtype=np.int64)
    else:
        kept = np.asarray(keep_pairs, dtype=np.int64)
    slot_row = np.full(T, -1, dtype=np.int64)
    slot_row[kept] = np.arange(len(kept))
    keep = keep_pairs is not False and keep_pairs is not None

    # per mode: the expert input u and the per-slot results
    st = []
    for m in modes:
        u = uq if act_quant else (f16_round(u_exact, sc["u"]) if m == "f16" else u_exact)
        st.append(dict(u=u, ohat=np.zeros((T, k, P)), o=np.zeros((len(kept), k, P)) if keep else None, a=None,
                       ohat_kept=np.zeros((len(kept), k, P)) if keep else None))

    for e in np.unique(ids):
        tt, jj = np.nonzero(ids == e)
        Wg, Wu, Wd = experts(int(e))
        asc = osc = None
        if "f16" in modes:
            asc, osc = expert_scales(Wg, Wu, Wd, P, gp, 2.0 if act_quant else 1.0, float(np.max(np.abs(ge[e]))))
            asc = None if act_quant else np.repeat(asc, 32)
        kr = slot_row[tt]
        ks = kr >= 0
        for m, S in zip(modes, st):
            U = S["u"][tt]
            g = U @ Wg.T
            v = U @ Wu.T
            a = silu(g) * v
            if m == "f16" and not act_quant:
                a = f16_round(a, asc)
            if act_quant:
                a = quantize_mx(a, act_quant)[0]
            o = a @ Wd.T
            # emulation: gamma_e * o as stored; its norm uses o
            o_st = f16_round(o * ge[e], osc) if m == "f16" else o
            if order == "norm_then_sum":
                inv = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
                S["ohat"][tt, jj] = o_st * inv if m == "f16" else o_st * inv * ge[e]
            else:
                S["ohat"][tt, jj] = o_st
            if keep:
                if S["a"] is None:
                    S["a"] = np.zeros((len(kept), k, Wg.shape[0]))
                S["a"][kr[ks], jj[ks]] = a[ks]
                S["o"][kr[ks], jj[ks]] = o_st[ks]
                S["ohat_kept"][kr[ks], jj[ks]] = S["ohat"][tt[ks], jj[ks]]

    # a token kept at several positions: its rows were written at the last of them
    src = slot_row[kept]
    dup = src != np.arange(len(kept))
    if keep and dup.any():
        for S in st:
            for name in ("a", "o", "ohat_kept"):
                if S[name] is not None:
                    S[name][dup] = S[name][src[dup]]

    res = []
    for m, S in zip(modes, st):
        y = np.zeros((T, P))
        for j in range(k):  # slot order
            y = y + w[:, j : j + 1] * S["ohat"][:, j]
        if order == "sum_then_norm":
            y = rms_norm(y, np.ones(P), eps)
        if m == "f16":
            y = f16_round(y, sc["y"])
        out = y @ Wun.T
        res.append(OracleResult(out=out, ids=ids, w=w, logits=logits, gaps=gaps, h=h, u=S["u"], a=S["a"],
                                o=S["o"], ohat=S["ohat_kept"], y=y, near_tie=near, xn=xn,
                                u_pre=u_pre))
    return res if isinstance(emulate, (tuple, list)) else res[0]


def f16_round(v: np.ndarray, scale) -> np.ndarray:
    """v stored as FP16 times `scale` (a power of two): nearest even, saturating
    at the largest finite FP16 value, then divided by the scale again."""
    z = np.clip(np.asarray(v, np.float64) * scale, -65504.0, 65504.0)
    return z.astype(np.float16).astype(np.float64) / scale


def pow2_down(bound: float, cap: int) -> float:
    """The largest power of two 2^-c (0 <= c <= cap) with bound * 2^-c <= 2^15;
    2^-cap for an infinite or NaN bound."""
    if not np.isfinite(bound):
        return 2.0 ** -cap
    c = 0
    while bound * 2.0 ** -c > 32768.0 and c < cap:
        c += 1
    return 2.0 ** -c


def f16_scales(pool_gamma, expert_gamma, P: int) -> dict:
    """Powers of two u and y are stored with in FP16 (module docstring): from
    the bounds sqrt(P) max|gamma_p| and sqrt(P) max|gamma_e|."""
    return {"u": pow2_down(np.sqrt(P) * float(np.max(np.abs(pool_gamma))), 100),
            "y": pow2_down(np.sqrt(P) * float(np.max(np.abs(expert_gamma))), 100)}


def row_norms(W: np.ndarray) -> np.ndarray:
    """Euclidean norm of each row of W."""
    return np.sqrt(np.einsum("ij,ij->i", W, W))


def scales_from_norms(ng, nu, nd, P: int, pool_gamma, amp: float = 1.0, ge_max: float = 1.0):
    """The FP16 range scalings of one expert from the row norms of its gate,
    up and down weights (ng, nu [I], nd [P]): the SwiGLU outputs' powers of
    two per block of 32 outputs [I/32], from max over the block of
    ||Wg_i|| ||Wu_i|| times P max(gamma_p)^2, and the outputs' power of two,
    from max_p ||Wd_p|| P max(gamma_p)^2 sqrt(sum_i (||Wg_i|| ||Wu_i||)^2)
    times amp and the largest |gamma_e| of the expert (module docstring)."""
    gp = float(np.max(np.abs(pool_gamma)))
    gu = ng * nu
    m = gu.reshape(-1, 32).max(axis=1)
    asc = np.array([pow2_down(b * P * gp * gp, 60) for b in m])
    osc = pow2_down(float(nd.max()) * P * gp * gp * float(np.sqrt(np.sum(gu * gu))) * amp * ge_max, 100)
    return asc, osc


def expert_scales(Wg, Wu, Wd, P: int, pool_gamma, amp: float = 1.0, ge_max: float = 1.0):
    """scales_from_norms of one expert's weights."""
    return scales_from_norms(row_norms(Wg), row_norms(Wu), row_norms(Wd), P, pool_gamma, amp, ge_max)


def a_scales(Wg, Wu, P: int, pool_gamma) -> np.ndarray:
    """Powers of two one expert's SwiGLU outputs are stored with in FP16, per
    block of 32 outputs [I/32] (scales_from_norms)."""
    return scales_from_norms(row_norms(Wg), row_norms(Wu), np.zeros(1), P, pool_gamma)[0]


def o_scale(Wg, Wu, Wd, P: int, pool_gamma, amp: float = 1.0, ge_max: float = 1.0) -> float:
    """Power of two one expert's outputs are stored with in FP16 (scales_from_norms)."""
    return expert_scales(Wg, Wu, Wd, P, pool_gamma, amp, ge_max)[1]


def _bf16_round(v: np.ndarray) -> np.ndarray:
    """FP64 -> FP32 (nearest) -> BF16 (nearest even) -> FP64 (the boundary
    norm's BF16 output)."""
    f = v.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def forward_inputs(inp: dict, k: int, eps: float, **kw) -> OracleResult:
    """Convenience: inputs as a dict of stored arrays (names as the layer's
    weights: x, router, router_bias, pooler, pool_gamma, w_gate, w_up, w_down,
    expert_gamma, unpooler)."""
    ex = inp.get("experts") or experts_from_arrays(inp["w_gate"], inp["w_up"], inp["w_down"])
    if inp.get("input_gamma") is not None:
        kw.setdefault("input_gamma", inp["input_gamma"])
    return forward(inp["x"], inp["router"], inp.get("router_bias"), inp["pooler"], inp["pool_gamma"],
                   ex, inp["expert_gamma"], inp["unpooler"], k, eps, **kw)
