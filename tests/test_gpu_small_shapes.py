"""Full-token parity of the BF16 and MXFP4 paths at small shapes.

The real-shape tests sample tokens; here every token and every output element
is compared with the FP64 oracle, at shapes that still span several tiles
(H = 1024, P = I = 512, E = 16..24) with ragged token counts, for both tile
families (decode-sized narrow tiles: T*k < 64*E; prefill-sized wide tiles),
top-1 and top-8 routing, a non-power-of-two expert count, MXFP4 experts and the
boundary norm. Bounds as for the real shapes: routing ids bit-exact except
reported near-ties, weights within 1e-6, output max-abs <= 2e-2 x RMS (BF16)
and 5e-2 x RMS (MXFP4 against the identically decoded weights).
"""
import sys

import numpy as np
import pytest

import synth
from layer_cases import (HostLayer, bf16_to_f64, check_output, check_rel_l2, check_routing, check_stage_chain,
                         device_weights, gather_rows, mx_u_ties)

pytestmark = pytest.mark.gpu

SMALL = dict(H=1024, P=512, I=512)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch


@pytest.fixture(scope="module")
def tables(torch_dev):
    return synth.DeviceTables("cuda:0")


CASES = [
    # name, spec overrides, T
    ("bf16 wide", dict(E=16, k=4), 300),
    ("bf16 narrow", dict(E=16, k=4), 100),
    ("bf16 top-1", dict(E=16, k=1), 257),
    ("bf16 top-8 E=24", dict(E=24, k=8), 199),
    ("mxfp4 wide", dict(E=16, k=4, expert_format="mxfp4"), 300),
    ("mxfp4 narrow", dict(E=16, k=4, expert_format="mxfp4"), 37),
    ("bf16 boundary norm", dict(E=16, k=4, input_norm=True), 300),
]


@pytest.mark.parametrize("name,over,T", CASES, ids=[c[0] for c in CASES])
def test_small_full_parity(torch_dev, tables, name, over, T):
    torch = torch_dev
    from latent_moe_layer_fp32_amd import LatentMoE

    spec = synth.CONFIGS["decode"].with_(name="small", T=T, **SMALL, **over)
    say(f"case: {name}, T={T}, E={spec.E}, k={spec.k}")
    wts = device_weights(spec, tables)
    gin = None
    if spec.input_norm:
        wts["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
        gin = synth.host(spec, "input_gamma")
    layer = LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                      eps=spec.eps, act_dtype=spec.act_dtype, expert_dtype=spec.expert_format,
                      max_tokens=512, weights=wts, input_norm=spec.input_norm)
    try:
        x = synth.device_tensor(spec, "x", tables)
        ids_d = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
        w_d = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids_d, topk_weights=w_d)
        torch.cuda.synchronize()
        out, ids, w = out.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
        v = layer.views(T)
        # run to run, bit for bit (fixed reduction orders, no atomics)
        assert np.array_equal(layer.forward(x).cpu().numpy(), out), "second forward differs"
        host = HostLayer(spec)
        xh = host.x()
        r, re_ = host.oracle(xh, input_gamma=gin, emulate=(None, "f16"))
        near, _ = check_routing(ids, w, r.logits, spec.k)
        force = {int(t): ids[t] for t in near}
        if near:
            say(f"{name}: near-ties at tokens {near}")
            r, re_ = host.oracle(xh, input_gamma=gin, force_ids=force, emulate=(None, "f16"))
        assert np.array_equal(ids, r.ids)
        order = np.argsort(ids.ravel(), kind="stable")
        assert np.array_equal(v["perm_token"], order // spec.k)
        assert np.array_equal(v["counts"], np.bincount(ids.ravel(), minlength=spec.E))
        pr = v["pair_row"].reshape(T, spec.k)
        check_rel_l2(bf16_to_f64(v["act"][pr]), r.a, 1e-2, "act")
        check_rel_l2(v["expert_out"][pr], r.o * host.gamma_o(ids), 1e-2, "expert out")
        tol = 5e-2 if spec.expert_format == "mxfp4" else 2e-2
        e = check_output(out, r.out, tol)
        # each stage against its declared FP16 rounding of the GPU's own inputs (to one
        # FP16 ulp, or an FP32 accumulation bound), and end to end against the oracle
        # emulating the FP16 rounding points
        ch = check_stage_chain(gather_rows(v, np.arange(T), spec.k, out), ids, w, host, r.u)
        rms = float(np.sqrt(np.mean(r.out ** 2)))
        d = out.astype(np.float64) - re_.out
        em = (float(np.abs(d).max() / rms), float(np.sqrt(np.mean(d * d)) / rms))
        say(f"{name}: out max-abs {e:.3g} x RMS over all {T} tokens; vs emulation max {em[0]:.3g} rms {em[1]:.3g}; "
            f"stage flips u {ch['u_flips']:.2g} a {ch['a_flips']:.2g} y {ch['y_flips']:.2g}, "
            f"o {ch['o_flips']:.2g}, FP32 acc out {ch['out_acc']:.2g}")
        assert em[0] <= 4e-3 and em[1] <= 6e-4, f"vs FP16 emulation: max {em[0]:.3g}, rms {em[1]:.3g}"
    finally:
        layer.close()


# ------------------- MX FP8 / FP4 activations (fp8 x fp4, mxfp4 x mxfp4 MMA)

MXA_CASES = [("mxfp8 wide", "mxfp8", 300, False), ("mxfp8 narrow", "mxfp8", 37, False),
             ("mxfp4 wide", "mxfp4", 300, False), ("mxfp4 narrow", "mxfp4", 37, False),
             ("mxfp8 boundary norm", "mxfp8", 64, True), ("mxfp4 boundary norm", "mxfp4", 300, True)]


def _decode_mx(codes, scales, fmt):
    from oracle import mx

    if fmt == "mxfp4":
        return mx.mxfp4_to_f64(codes, scales)
    v = mx.E4M3[codes.astype(np.int64)]
    s = mx.e8m0_to_f64(scales)
    K = codes.shape[-1]
    return (v.reshape(codes.shape[:-1] + (K // 32, 32)) * s[..., None]).reshape(codes.shape)


@pytest.mark.parametrize("name,fmt,T,norm", MXA_CASES, ids=[c[0] for c in MXA_CASES])
def test_small_mx_activations_parity(torch_dev, tables, name, fmt, T, norm):
    """Against the oracle with u and a MX-quantised (FP8 or FP4) at the same
    points: quantised u equal code for code except rare rounding-boundary flips
    to a neighbouring code (the GPU forms u in FP32, the oracle in FP64),
    output max-abs <= 5e-2 x RMS."""
    torch = torch_dev
    from latent_moe_layer_fp32_amd import LatentMoE

    spec = synth.CONFIGS["decode"].with_(name="small", T=T, E=16, k=4, expert_format="mxfp4",
                                         input_norm=norm, **SMALL)
    say(f"case: {name}, T={T}")
    wts = device_weights(spec, tables)
    gin = None
    if norm:  # x is the pre-norm residual
        wts["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
        gin = synth.host(spec, "input_gamma")
    layer = LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                      eps=spec.eps, act_dtype=spec.act_dtype, expert_dtype=spec.expert_format,
                      max_tokens=512, weights=wts, expert_act=fmt, input_norm=norm)
    try:
        x = synth.device_tensor(spec, "x", tables)
        ids_d = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
        w_d = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids_d, topk_weights=w_d)
        torch.cuda.synchronize()
        out, ids, w = out.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
        v = layer.views(T)
        assert np.array_equal(layer.forward(x).cpu().numpy(), out), "second forward differs"
        host = HostLayer(spec)
        xh = host.x()
        r0 = host.oracle(xh, keep_pairs=False, act_quant=fmt, input_gamma=gin)
        near, _ = check_routing(ids, w, r0.logits, spec.k)
        force = {int(t): ids[t] for t in near}
        r = host.oracle(xh, act_quant=fmt, input_gamma=gin, force_ids=force or None)
        assert np.array_equal(ids, r.ids)
        # the quantised expert input: the kernel's codes are the exact MX rounding of
        # its own FP32 u; where they differ from the rounding of the exact u, the two
        # lie on either side of a rounding midpoint (mx_u_ties)
        uq = _decode_mx(v["expert_in"], v["expert_in_scales"], fmt)
        ties, nel = mx_u_ties(v, np.arange(T), uq, r, fmt)
        assert nel <= 1e-3 * uq.size, f"u: {nel} of {uq.size} elements differ"
        if ties:  # the oracle takes the kernel's rounding where u sits on a midpoint
            say(f"{name}: u rounding ties at {nel} elements of tokens {sorted(ties)}")
            r = host.oracle(xh, act_quant=fmt, input_gamma=gin, force_ids=force or None, force_u=ties)
        frac = nel / uq.size
        pr = v["pair_row"].reshape(T, spec.k)
        aq = _decode_mx(v["act"], v["act_scales"], fmt)[pr]
        check_rel_l2(aq, r.a, 1e-2, f"act ({fmt})")
        check_rel_l2(v["expert_out"][pr], r.o * host.gamma_o(ids), 1e-2, "expert out")
        e = check_output(out, r.out, 5e-2)
        say(f"{name}: u flips {frac:.2e}; out max-abs {e:.3g} x RMS over all {T} tokens")
    finally:
        layer.close()


# ------------------------------- weight rows of very different magnitudes

ROW_CASES = [("bf16 wide", "bf16", 300), ("bf16 narrow", "bf16", 100), ("mxfp4 wide", "mxfp4", 300)]


@pytest.mark.parametrize("name,fmt,T", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_small_row_magnitudes(torch_dev, tables, name, fmt, T):
    """Every weight row of the expert and unpooler matrices scaled by its own
    power of two 2^k (gate/up rows k in [-8, 3], down rows [-10, 10], unpooler
    rows [-30, 30]; exact in BF16 and, for MXFP4, an offset of the row's E8M0
    codes). The FP16 copies take each row's own 2^s, so the layer matches the
    oracle on the scaled weights: routing exact, every output element within
    2e-2 x RMS after dividing each unpooler column by its 2^k (so the rows of
    2^-30 are checked as tightly as those of 2^30). Gate/up rows stay at most
    2^3 up: the SwiGLU output a is an FP16 operand and saturates at 65504
    (here |a| stays below ~2e3)."""
    torch = torch_dev
    from latent_moe_layer_fp32_amd import LatentMoE
    from oracle import oracle as orc
    from oracle.mx import to_f64

    spec = synth.CONFIGS["decode"].with_(name="small", T=T, E=16, k=4, expert_format=fmt, **SMALL)
    E, H, P, I = spec.E, spec.H, spec.P, spec.I
    say(f"case: row magnitudes, {name}, T={T}")
    rng = np.random.default_rng(21)
    kexp = {"w_gate": rng.integers(-8, 4, size=(E, I)), "w_up": rng.integers(-8, 4, size=(E, I)),
            "w_down": rng.integers(-10, 11, size=(E, P))}
    kun = rng.integers(-30, 31, size=H)
    wts = device_weights(spec, tables)
    dev = wts["pooler"].device
    for n, k in kexp.items():
        if fmt == "mxfp4":  # 2^k on a row = k added to each of its E8M0 scale codes
            codes, sc = wts[n]
            wts[n] = (codes, (sc.int() + torch.from_numpy(k).to(dev)[..., None].int()).to(torch.uint8))
        else:
            f = torch.from_numpy(np.ldexp(1.0, k).astype(np.float32)).to(dev)
            wts[n] = (wts[n].float() * f[..., None]).to(torch.bfloat16)
    fu = torch.from_numpy(np.ldexp(1.0, kun).astype(np.float32)).to(dev)
    wts["unpooler"] = (wts["unpooler"].float() * fu[:, None]).to(torch.bfloat16)
    layer = LatentMoE(hidden=H, pooled=P, experts=E, intermediate=I, top_k=spec.k, eps=spec.eps,
                      act_dtype=spec.act_dtype, expert_dtype=fmt, max_tokens=512, weights=wts)
    try:
        x = synth.device_tensor(spec, "x", tables)
        ids_d = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
        w_d = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids_d, topk_weights=w_d)
        torch.cuda.synchronize()
        out, ids, w = out.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
    finally:
        layer.close()
    host = HostLayer(spec)

    def expert(e):
        return tuple(to_f64(_first(synth.host(spec, n, experts=(e, e + 1)))) * np.ldexp(1.0, kexp[n][e])[:, None]
                     for n in ("w_gate", "w_up", "w_down"))

    xh = host.x()
    hw = host.w
    near, _ = check_routing(ids, w, host.logits(xh), spec.k)
    force = {int(t): ids[t] for t in near}
    r = orc.forward(xh, hw["router"], None, hw["pooler"], hw["pool_gamma"], expert, hw["expert_gamma"],
                    hw["unpooler"], spec.k, spec.eps, force_ids=force or None, keep_pairs=False)
    assert np.array_equal(ids, r.ids)
    e = check_output(np.ldexp(out.astype(np.float64), -kun[None, :]), r.out, 2e-2)
    say(f"row magnitudes, {name}: out max-abs {e:.3g} x RMS over all {T} tokens (columns divided by 2^k)")


def _first(a):
    return (a[0][0], a[1][0]) if isinstance(a, tuple) else a[0]


# ------------------------------------------------------ large norm gammas

@pytest.mark.parametrize("fmt,T", [("bf16", 300), ("bf16", 100), ("mxfp4", 300)])
def test_small_large_gammas(torch_dev, tables, fmt, T):
    """Norm gammas 2^14 (gamma_p) and 2^15 (gamma_e) times larger, the gate/up
    weights 2^14 times smaller so that g and v keep their size: u and y then
    reach ~9e4, beyond FP16's 65504, and are stored times a power of two
    chosen at create from sqrt(P) max|gamma|, undone after their products.
    Every output element within 2e-2 x RMS of the oracle on the same inputs."""
    torch = torch_dev
    from latent_moe_layer_fp32_amd import LatentMoE
    from oracle import oracle as orc
    from oracle.mx import to_f64

    spec = synth.CONFIGS["decode"].with_(name="small", T=T, E=16, k=4, expert_format=fmt, **SMALL)
    E, H, P, I = spec.E, spec.H, spec.P, spec.I
    say(f"case: large gammas, {fmt}, T={T}")
    big, bige = 2.0 ** 14, 2.0 ** 15
    wts = device_weights(spec, tables)
    wts["pool_gamma"] = wts["pool_gamma"] * big
    wts["expert_gamma"] = wts["expert_gamma"] * bige
    for n in ("w_gate", "w_up"):
        if fmt == "mxfp4":  # 2^-14 on every block = -14 on each E8M0 code
            codes, sc = wts[n]
            wts[n] = (codes, (sc.int() - 14).to(torch.uint8))
        else:
            wts[n] = (wts[n].float() / big).to(torch.bfloat16)
    layer = LatentMoE(hidden=H, pooled=P, experts=E, intermediate=I, top_k=spec.k, eps=spec.eps,
                      act_dtype=spec.act_dtype, expert_dtype=fmt, max_tokens=512, weights=wts)
    try:
        x = synth.device_tensor(spec, "x", tables)
        ids_d = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
        w_d = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids_d, topk_weights=w_d)
        torch.cuda.synchronize()
        out, ids, w = out.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
        v = layer.views(T, names=("expert_in", "combined"))
    finally:
        layer.close()
    host = HostLayer(spec)
    hw = host.w
    scale = {"w_gate": 1.0 / big, "w_up": 1.0 / big, "w_down": 1.0}

    def expert(e):
        return tuple(to_f64(_first(synth.host(spec, n, experts=(e, e + 1)))) * scale[n]
                     for n in ("w_gate", "w_up", "w_down"))

    xh = host.x()
    near, _ = check_routing(ids, w, host.logits(xh), spec.k)
    force = {int(t): ids[t] for t in near}
    r = orc.forward(xh, hw["router"], None, hw["pooler"], to_f64(hw["pool_gamma"]) * big, expert,
                    to_f64(hw["expert_gamma"]) * bige, hw["unpooler"], spec.k, spec.eps,
                    force_ids=force or None, keep_pairs=False)
    assert np.array_equal(ids, r.ids)
    assert np.abs(r.u).max() > 65504 and np.abs(r.y).max() > 65504, "inputs do not exceed FP16's range"
    e = check_output(out, r.out, 2e-2)
    if fmt == "bf16":
        eu = float((np.abs(v["expert_in"] - r.u) / np.abs(r.u).max()).max())
        assert eu < 1e-3, f"u (stored scaled): max error {eu:.3g} of max|u|"
    ey = float((np.abs(v["combined"] - r.y) / np.abs(r.y).max()).max())
    assert ey < 1e-2, f"y (stored scaled): max error {ey:.3g} of max|y|"
    say(f"large gammas, {fmt}: max|u| {np.abs(r.u).max():.3g}, max|y| {np.abs(r.y).max():.3g}; "
        f"out max-abs {e:.3g} x RMS over all {T} tokens")


# ------------------------------------------------- large SwiGLU outputs

@pytest.mark.parametrize("fmt,T", [("bf16", 300), ("bf16", 100), ("mxfp4", 300)])
def test_small_large_swiglu_output(torch_dev, tables, fmt, T):
    """Gate and up weights 2^7 times larger: a = silu(g) v reaches ~2e5, beyond
    FP16's 65504. Per expert and block of 32 intermediate columns, create picks
    a power of two from the bound ||Wg_i|| ||Wu_i|| P max|gamma_p|^2 that keeps a
    within 2^15 (the down weights' copies carry its inverse): every output
    element within 2e-2 x RMS of the oracle, a itself within 1e-2 (relative L2)."""
    torch = torch_dev
    from latent_moe_layer_fp32_amd import LatentMoE
    from oracle import oracle as orc
    from oracle.mx import to_f64

    spec = synth.CONFIGS["decode"].with_(name="small", T=T, E=16, k=4, expert_format=fmt, **SMALL)
    E, H, P, I = spec.E, spec.H, spec.P, spec.I
    say(f"case: large SwiGLU output, {fmt}, T={T}")
    big = 2.0 ** 7
    wts = device_weights(spec, tables)
    for n in ("w_gate", "w_up"):
        if fmt == "mxfp4":  # 2^7 on every block = +7 on each E8M0 code
            codes, sc = wts[n]
            wts[n] = (codes, (sc.int() + 7).to(torch.uint8))
        else:
            wts[n] = (wts[n].float() * big).to(torch.bfloat16)
    layer = LatentMoE(hidden=H, pooled=P, experts=E, intermediate=I, top_k=spec.k, eps=spec.eps,
                      act_dtype=spec.act_dtype, expert_dtype=fmt, max_tokens=512, weights=wts)
    try:
        x = synth.device_tensor(spec, "x", tables)
        ids_d = torch.empty((T, spec.k), dtype=torch.int32, device=x.device)
        w_d = torch.empty((T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids_d, topk_weights=w_d)
        torch.cuda.synchronize()
        out, ids, w = out.cpu().numpy(), ids_d.cpu().numpy(), w_d.cpu().numpy()
        v = layer.views(T, names=("act", "pair_row"))
    finally:
        layer.close()
    host = HostLayer(spec)
    hw = host.w
    scale = {"w_gate": big, "w_up": big, "w_down": 1.0}

    def expert(e):
        return tuple(to_f64(_first(synth.host(spec, n, experts=(e, e + 1)))) * scale[n]
                     for n in ("w_gate", "w_up", "w_down"))

    xh = host.x()
    near, _ = check_routing(ids, w, host.logits(xh), spec.k)
    force = {int(t): ids[t] for t in near}
    r = orc.forward(xh, hw["router"], None, hw["pooler"], hw["pool_gamma"], expert, hw["expert_gamma"],
                    hw["unpooler"], spec.k, spec.eps, force_ids=force or None)
    assert np.array_equal(ids, r.ids)
    assert np.abs(r.a).max() > 65504, "a does not exceed FP16's range"
    pr = v["pair_row"].reshape(T, spec.k)
    ea = check_rel_l2(v["act"][pr], r.a, 1e-2, "act")
    e = check_output(out, r.out, 2e-2)
    say(f"large SwiGLU output, {fmt}: max|a| {np.abs(r.a).max():.3g}; rel L2 act {ea:.3g}; "
        f"out max-abs {e:.3g} x RMS over all {T} tokens")
