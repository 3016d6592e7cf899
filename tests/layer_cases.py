"""Shared helpers for the layer's tests: seeded inputs on both sides, the
oracle on chosen tokens, and the parity comparisons."""
from __future__ import annotations

import numpy as np

import synth
from oracle import oracle as orc
from oracle.mx import to_f64

NON_EXPERT = ("router", "router_bias", "pooler", "pool_gamma", "expert_gamma", "unpooler")


class HostLayer:
    """Host copies of a layer's non-expert tensors; experts generated on demand."""

    def __init__(self, spec: synth.LayerSpec):
        self.spec = spec
        self.w = {n: synth.host(spec, n) for n in NON_EXPERT}
        self._cache = {}

    def expert(self, e: int):
        if e not in self._cache:
            if len(self._cache) > 8:
                self._cache.clear()
            s = self.spec
            self._cache[e] = tuple(
                to_f64(_first(synth.host(s, n, experts=(e, e + 1)))) for n in ("w_gate", "w_up", "w_down"))
        return self._cache[e]

    def x(self, chunk: int = 0):
        return synth.host(self.spec, "x", chunk=chunk)

    def oracle(self, x_rows, **kw) -> orc.OracleResult:
        s = self.spec
        return orc.forward(x_rows, self.w["router"], self.w["router_bias"], self.w["pooler"],
                           self.w["pool_gamma"], self.expert, self.w["expert_gamma"],
                           self.w["unpooler"], s.k, s.eps, **kw)

    def logits(self, x_rows) -> np.ndarray:
        return orc.router_logits(to_f64(x_rows), to_f64(self.w["router"]),
                                 None if self.w["router_bias"] is None else to_f64(self.w["router_bias"]))


def _first(a):
    """Strip the leading length-1 expert axis of an array or (packed, scales) pair."""
    if isinstance(a, tuple):
        return (a[0][0], a[1][0])
    return a[0]


def device_weights(spec: synth.LayerSpec, tables) -> dict:
    return {n: synth.device_tensor(spec, n, tables) for n in synth.WEIGHT_NAMES}


def make_layer(spec: synth.LayerSpec, weights: dict, max_tokens: int):
    from latent_moe_layer_fp32_amd import LatentMoE

    return LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                     eps=spec.eps, act_dtype=spec.act_dtype, expert_dtype=spec.expert_format,
                     max_tokens=max_tokens, weights=weights, expert_act=spec.expert_act)


def check_routing(gpu_ids: np.ndarray, gpu_w: np.ndarray, logits64: np.ndarray, k: int,
                  w_tol: float = 1e-6):
    """Selected ids must equal the oracle's, except where the oracle's FP64
    logits of the two choices are within 1e-6 slot by slot (near-ties, which
    are reported). Returns (near_tie_tokens, oracle_ids)."""
    ids, gaps = orc.select_topk(logits64, k)
    diff = np.nonzero((gpu_ids != ids).any(axis=1))[0]
    near = []
    for t in diff:
        g = gpu_ids[t].astype(np.int64)
        assert len(set(g.tolist())) == k, f"token {t}: repeated expert in {g}"
        dl = np.abs(logits64[t, g] - logits64[t, ids[t]])
        assert (dl < orc.NEAR_TIE).all(), (
            f"token {t}: ids {g.tolist()} vs oracle {ids[t].tolist()}, logit gaps {dl.tolist()}")
        near.append(int(t))
    # weights: softmax of the oracle's FP64 logits at the GPU's ids
    sel = np.take_along_axis(logits64, gpu_ids.astype(np.int64), axis=1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    err = np.abs(gpu_w.astype(np.float64) - ref).max()
    assert err <= w_tol, f"routing weight error {err:.3g} > {w_tol}"
    return near, ids


def check_output(gpu: np.ndarray, ref: np.ndarray, c: float, what: str = "out"):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    assert err <= c * rms, f"{what}: max-abs error {err:.4g} > {c} x RMS {rms:.4g} ({err / rms:.3g} x RMS)"
    return err / rms


def check_rel_l2(gpu: np.ndarray, ref: np.ndarray, c: float, what: str):
    """Relative L2 error of an intermediate stage: BF16 rounding gives ~1e-3,
    a wrong index, operand or scale gives O(1)."""
    err = float(np.linalg.norm(gpu.astype(np.float64) - ref) / np.linalg.norm(ref))
    assert err <= c, f"{what}: relative L2 error {err:.3g} > {c}"
    return err


def bf16_to_f64(a):
    return to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def check_expert_input(v: dict, rows, ref_u: np.ndarray) -> float:
    """BF16 layers: the pooler's FP32 gamma_p * h times the row scale equals
    the oracle's u to FP32 accumulation error, and the FP16 u the expert
    GEMMs read is its nearest FP16 value (relative error <= 2^-11, plus the
    same absolute slack). Returns the largest relative error of the FP16 u."""
    u32 = v["pooled"][rows].astype(np.float64) * v["row_scale"][rows, None]
    d32 = np.abs(u32 - ref_u)
    assert np.all(d32 <= 2.0 ** -20 * np.abs(ref_u) + 2e-5), f"pooled * row_scale: max abs error {d32.max():.3g}"
    u16 = v["expert_in"][rows].astype(np.float64)
    d16 = np.abs(u16 - ref_u)
    assert np.all(d16 <= 2.0 ** -10 * np.abs(ref_u) + 2e-5), f"FP16 u: max abs error {d16.max():.3g}"
    return float((d16 / (np.abs(ref_u) + 1e-30)).max())


def mx_rounding_ties(uq_gpu: np.ndarray, r, fmt: str, rel: float = 1e-4) -> dict:
    """MX-quantised u from the kernel against the oracle's: where they differ,
    check that the oracle's unquantised value lies on the midpoint between the
    two codes (within rel of the block scale: the kernel forms u in FP32, the
    oracle in FP64, so exactly there either rounding is right), or that the
    block maximum lies on a power of two (the scale itself a tie). Returns
    {token: kernel row} to pass to the oracle as force_u."""
    from oracle import mx

    diff = uq_gpu != r.u
    if not diff.any():
        return {}
    _, e = mx.quantize_mx(r.u_pre, fmt)
    X = np.repeat(np.ldexp(1.0, e.astype(np.int64)), 32, axis=-1)
    amax = np.repeat(np.abs(r.u_pre).reshape(r.u_pre.shape[0], -1, 32).max(-1), 32, axis=-1)
    scale_tie = np.abs(np.log2(amax) - np.round(np.log2(amax))) <= rel
    q, g, o = r.u_pre / X, uq_gpu / X, r.u / X
    code_tie = np.abs(q - 0.5 * (g + o)) <= rel * np.maximum(np.abs(q), 1.0)
    bad = diff & ~(code_tie | scale_tie)
    assert not bad.any(), f"u differs from the oracle away from a rounding tie at {np.argwhere(bad)[:5]}"
    return {int(t): uq_gpu[t] for t in np.unique(np.nonzero(diff)[0])}
