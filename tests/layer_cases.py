"""Shared helpers for the layer's tests: seeded inputs on both sides, the
oracle on chosen tokens, and the parity comparisons."""
from __future__ import annotations

import numpy as np

import synth
from oracle import oracle as orc
from oracle.mx import to_f64

NON_EXPERT = ("router", "router_bias", "pooler", "pool_gamma", "expert_gamma", "unpooler")


class HostLayer:
    """Host copies of a layer's non-expert tensors; experts fetched on demand,
    from the layer's device tensors when given (`dev`: the weights dict the
    layer was created from; equal to the host generator's output bit for bit,
    test_device_generator_matches_host, and ten times faster to fetch), else
    generated on the host."""

    def __init__(self, spec: synth.LayerSpec, dev: dict | None = None):
        self.spec = spec
        self.w = {n: synth.host(spec, n) for n in NON_EXPERT}
        self.dev = dev
        self._cache = {}
        self._norms = {}

    def expert(self, e: int):
        if e not in self._cache:
            if len(self._cache) > 8:
                self._cache.clear()
            s = self.spec
            names = ("w_gate", "w_up", "w_down")
            if self.dev is not None:
                self._cache[e] = tuple(fast_f64(_device_rows(self.dev[n], e)) for n in names)
            else:
                self._cache[e] = tuple(to_f64(_first(synth.host(s, n, experts=(e, e + 1)))) for n in names)
        return self._cache[e]

    def norms(self, e: int):
        """Row norms of expert e's gate, up and down weights (kept for the
        layer's lifetime: three short vectors per expert)."""
        if e not in self._norms:
            self._norms[e] = tuple(orc.row_norms(W) for W in self.expert(e))
        return self._norms[e]

    def scales(self, e: int, amp: float = 1.0):
        """Expert e's FP16 range scalings (a per block of 32, gamma_e o), as
        the oracle derives them."""
        ng, nu, nd = self.norms(e)
        ge = float(np.max(np.abs(self.w["expert_gamma"][e].astype(np.float64))))
        return orc.scales_from_norms(ng, nu, nd, self.spec.P, self.w["pool_gamma"].astype(np.float64), amp, ge)

    def gamma_o(self, ids) -> np.ndarray:
        """The expert gammas of the selected experts [..., P] (the BF16-activation
        layer stores gamma_e * o as its expert outputs)."""
        return to_f64(self.w["expert_gamma"])[np.asarray(ids)]

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


def fast_f64(a) -> np.ndarray:
    """The same values as oracle.mx.to_f64 for BF16 bits (uint16) and MXFP4
    (codes, scales) pairs, converted with torch's multithreaded CPU kernels
    (a real-shape expert matrix in ~0.02 s instead of ~0.1-0.2 s); anything
    else goes to to_f64. Pinned to to_f64 by test_fast_f64_equals_to_f64."""
    import torch

    from oracle import mx

    if isinstance(a, tuple):
        codes, scales = (torch.from_numpy(np.ascontiguousarray(x)) for x in a)
        tab = torch.from_numpy(mx.E2M1)
        lo = tab[(codes & 0x0F).long()]
        hi = tab[(codes >> 4).long()]
        el = torch.stack([lo, hi], dim=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
        sc = torch.from_numpy(mx.e8m0_to_f64(a[1]))
        K = el.shape[-1]
        return (el.reshape(el.shape[:-1] + (K // 32, 32)) * sc[..., None]).reshape(el.shape).numpy()
    if isinstance(a, np.ndarray) and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return to_f64(a)


def _device_rows(t, e):
    """Expert e of a device expert tensor (BF16 as its bits, or an MXFP4
    (codes, scales) pair) as host arrays."""
    import torch

    if isinstance(t, tuple):
        return (t[0][e].cpu().numpy(), t[1][e].cpu().numpy())
    if t.dtype == torch.bfloat16:
        return t[e].view(torch.int16).cpu().numpy().view(np.uint16)
    return t[e].cpu().numpy()


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


def check_output(gpu: np.ndarray, ref: np.ndarray, c: float, what: str = "out", rms: float | None = None):
    """max-abs error <= c x RMS, the RMS of `ref` unless given (the batch RMS
    when `ref` holds only sampled rows of a batch whose full output is known)."""
    if rms is None:
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


# FP32 formation error of u = r * (gamma_p * h): h accumulates H BF16 products
# in FP32; a bound of 2^-20 relative plus 2e-5 absolute holds with a wide
# margin for H up to 8192 (typical FP32 chain error ~ sqrt(H) 2^-24 ~ 5e-6 at
# unit-scale rows) and is what the pooler stage is checked against.
U_FORM_REL, U_FORM_ABS = 2.0 ** -20, 2e-5


def mx_u_ties(v: dict, rows, uq_gpu: np.ndarray, r, fmt: str):
    """MX-quantised u from the kernel against the oracle's quantisation of the
    exact u. The kernel quantises its own FP32 u = fl32(pooled * row_scale)
    (both in the views); that value must lie within the FP32 formation bound
    of the exact u, and the kernel's codes must be exactly the MX quantisation
    of it (nearest even, the same scale rule). Where the two quantisations then
    differ, the exact u and the kernel's FP32 u lie on either side of a
    rounding midpoint (or of a power of two deciding the block scale), so
    either code is a correct rounding: the oracle is given the kernel's codes
    for those tokens (force_u). Returns ({token: row}, differing elements)."""
    from oracle import mx

    u32 = (v["pooled"][rows].astype(np.float32) * v["row_scale"][rows, None].astype(np.float32))
    u32 = u32.astype(np.float64)
    d = np.abs(u32 - r.u_pre)
    assert np.all(d <= U_FORM_REL * np.abs(r.u_pre) + U_FORM_ABS), f"FP32 u: max |error| {d.max():.3g}"
    q32 = mx.quantize_mx(u32, fmt)[0]
    bad = q32 != uq_gpu
    assert not bad.any(), f"u codes are not the MX rounding of the kernel's FP32 u at {np.argwhere(bad)[:5]}"
    diff = uq_gpu != r.u
    return {int(t): uq_gpu[t] for t in np.unique(np.nonzero(diff)[0])}, int(diff.sum())


# ------------------------------------------------------- stage-chained checks
# Each stage of the BF16-activation layer checked against the FP64 evaluation
# of its declared rounding applied to the GPU's own inputs of that stage, so
# no rounding difference upstream cascades into it:
#   u  = FP16(r * (gamma_p * h)) from the GPU's FP32 gamma_p * h and row
#        scale: bit for bit (the same FP32 product rounded to FP16)
#   a  = FP16(silu(Wg u16) * (Wu u16))            from the GPU's FP16 u
#   o  = FP16(gamma_e (Wd a16)) (FP32 accumulation) from the GPU's FP16 a
#   y  = FP16(sum_j w_j o16_j / rms(o_j))          from the GPU's FP16 gamma_e o,
#        the RMS of the unrounded o (the GPU's FP32 sums of squares)
#   out = Wun y16 (FP32 accumulation)             from the GPU's FP16 y
# FP16 stages a, o and y: within one FP16 unit in the last place of the
# reference plus the FP32 error of the value the GPU rounds (the GPU rounds
# its FP32 value, the reference its FP64 value; they differ only where a
# rounding midpoint lies between the two), and such flips are a small
# fraction. FP32-accumulated products: |err| <= 2^-15 sum |x w| (a 4096- or
# 8192-term MFMA chain in FP32 adds at most ~300 roundings of 2^-24 relative
# to the sum of magnitudes).
ACC_REL = 2.0 ** -15


def _f16_ulp(v: np.ndarray) -> np.ndarray:
    """One FP16 unit in the last place at |v| (subnormal spacing 2^-24 below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _check_f16(gpu, ref, scale, slack, what):
    """gpu and ref hold values stored as FP16 times `scale`: at most one FP16
    ulp (of the scaled value) plus `slack` (the FP32 error of the value the GPU
    rounded) apart. Returns the fraction that differ."""
    d = np.abs(gpu - ref) * scale
    lim = _f16_ulp(ref * scale) * (1 + 1e-9) + slack * scale
    assert np.all(d <= lim), f"{what}: max |diff| / (ulp + slack) = {(d / lim).max():.3g}"
    return float((d > 0).mean())


def _check_acc(gpu, ref, mag, what):
    err = np.abs(gpu - ref)
    assert np.all(err <= ACC_REL * mag), f"{what}: max err / (2^-15 sum|x w|) = {(err / (ACC_REL * mag)).max():.3g}"
    return float((err / np.maximum(mag, 1e-300)).max())


def gather_rows(v: dict, rows, k: int, out: np.ndarray) -> dict:
    """The stage values of the tokens `rows` of the last forward (views `v`
    and its output `out`), as host arrays per token: expert_in, pooled and
    row_scale [n, ...], act and expert_out per slot [n, k, ...], combined,
    and out. Rows of several forwards concatenate (concat_rows)."""
    rows = np.asarray(rows)
    pr = v["pair_row"].reshape(-1, k)[rows]
    return dict(expert_in=v["expert_in"][rows].astype(np.float64), pooled=v["pooled"][rows].astype(np.float32),
                row_scale=v["row_scale"][rows].astype(np.float32), act=v["act"][pr].astype(np.float64),
                expert_out=v["expert_out"][pr].astype(np.float64),
                combined=v["combined"][rows].astype(np.float64), out=out[rows].astype(np.float64))


def concat_rows(parts) -> dict:
    return {n: np.concatenate([p[n] for p in parts]) for n in parts[0]}


def check_stage_chain(g: dict, ids_rows, w_rows, host: HostLayer, u_exact: np.ndarray) -> dict:
    """Chained stage checks (above) on gathered rows `g` (gather_rows) of a
    BF16-activation layer whose expert inputs are FP16; ids_rows, w_rows: the
    GPU's selection and weights of those rows; u_exact: the oracle's u of
    those rows. The FP32 accumulation slack of a product x W^T is taken as
    2^-15 ||x|| ||W_row|| (Cauchy-Schwarz bound on sum |x w|). Returns the flip
    fractions and the largest accumulation error of out."""
    spec = host.spec
    P, k = spec.P, spec.k
    hw = host.w
    gp, ge = to_f64(hw["pool_gamma"]), to_f64(hw["expert_gamma"])
    sc = orc.f16_scales(gp, ge, P)
    res = {}
    u16 = g["expert_in"]
    rd = (g["row_scale"] * np.float32(sc["u"]))[:, None]
    u32 = g["pooled"] * rd  # the kernel's FP32 product
    ref_u = np.clip(u32, -65504, 65504).astype(np.float16).astype(np.float64) / sc["u"]
    assert np.array_equal(u16, ref_u), "u: not the FP16 rounding of the kernel's FP32 u"
    res["u_flips"] = float((u16 != orc.f16_round(u_exact, sc["u"])).mean())  # against the exact u
    n = len(u16)
    fa, eo = [], []
    ohat = np.zeros((n, k, P))
    for e in np.unique(ids_rows):
        tt, jj = np.nonzero(ids_rows == e)
        Wg, Wu, Wd = host.expert(int(e))
        ng, nu, nd = host.norms(int(e))
        asc, osc = host.scales(int(e))
        asc = np.repeat(asc, 32)
        U = u16[tt]
        nU = orc.row_norms(U)[:, None]
        g_, vv = U @ Wg.T, U @ Wu.T
        a_ref = orc.silu(g_) * vv
        # FP32 error of the kernel's silu(g) v: from g and v (FP32 sums) and the
        # FP32 evaluation of silu (exp and reciprocal, a few ulp)
        dg, dv = ACC_REL * nU * ng[None, :], ACC_REL * nU * nu[None, :]
        slack = 1.1 * (dg * np.abs(vv) + np.abs(g_) * dv) + 2.0 ** -20 * np.abs(a_ref)
        a16 = g["act"][tt, jj]
        fa.append(_check_f16(a16, orc.f16_round(a_ref, asc), asc, slack, f"act, expert {e}"))
        o16 = g["expert_out"][tt, jj]  # gamma_e o as stored
        o_ref = a16 @ Wd.T
        go = o_ref * ge[e]
        # FP32 accumulation of o, times |gamma|, plus the FP32 rounding of the product
        slack_o = ACC_REL * orc.row_norms(a16)[:, None] * (nd * np.abs(ge[e]))[None, :] + 2.0 ** -23 * np.abs(go)
        eo.append(_check_f16(o16, orc.f16_round(go, osc), osc, slack_o, f"expert out, expert {e}"))
        ohat[tt, jj] = o16 / np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + spec.eps)
    res["a_flips"] = float(np.mean(fa))
    res["o_flips"] = float(np.mean(eo))
    wr = w_rows.astype(np.float64)
    y_ref = np.einsum("tj,tjp->tp", wr, ohat)
    y_slack = 2.0 ** -17 * np.einsum("tj,tjp->tp", np.abs(wr), np.abs(ohat))  # FP32 sums of squares, norm, k-term sum
    y16 = g["combined"]
    res["y_flips"] = _check_f16(y16, orc.f16_round(y_ref, sc["y"]), sc["y"], y_slack, "y")
    Wun = to_f64(hw["unpooler"])
    mag = orc.row_norms(y16)[:, None] * orc.row_norms(Wun)[None, :]
    res["out_acc"] = _check_acc(g["out"], y16 @ Wun.T, mag, "out")
    return res
