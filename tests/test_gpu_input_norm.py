"""Parity of the optional boundary norm (x given as the pre-norm residual)
against the FP64 oracle, through the C ABI.

The residual is 4x the seeded token (exact in FP32 and BF16). The norm's FP32
output must equal the oracle's (FP64 norm rounded once to FP32) to one unit
in the last place; routing, stages and outputs use the same bounds as the
plain layer (routing ids bit-exact except reported near-ties, weights within
1e-6, outputs 1e-4 x RMS for FP32 and 2e-2 x RMS for BF16).
"""
import sys

import numpy as np
import pytest

import synth
from layer_cases import (HostLayer, check_expert_input, check_output, check_rel_l2, check_routing, check_stage_chain,
                         concat_rows, device_weights, gather_rows)
from oracle import oracle as orc
from oracle.mx import to_f64

pytestmark = pytest.mark.gpu

SCALE = 4.0


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


def residual_host(spec, chunk=0):
    """4 x the seeded token, in the spec's stored format (exact)."""
    x = synth.host(spec, "x", chunk=chunk)
    if x.dtype == np.uint16:
        f = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(SCALE)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return (x * np.float32(SCALE)).astype(np.float32)


def make_norm_layer(spec, weights, max_tokens):
    from latent_moe_layer_fp32_amd import LatentMoE

    return LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                     eps=spec.eps, act_dtype=spec.act_dtype, expert_dtype=spec.expert_format,
                     max_tokens=max_tokens, weights=weights, input_norm=True)


def run(torch, layer, r):
    T = r.shape[0]
    ids = torch.empty((T, layer.top_k), dtype=torch.int32, device=r.device)
    w = torch.empty((T, layer.top_k), dtype=torch.float32, device=r.device)
    out = layer.forward(r, topk_ids=ids, topk_weights=w)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def oracle_xn(host, r_rows, gin):
    """The oracle's boundary norm of residual rows (FP32 values as FP64)."""
    return orc.rms_norm(to_f64(r_rows), to_f64(gin), host.spec.eps).astype(np.float32).astype(np.float64)


def check_xn(gpu_xn, ref_xn):
    """Equal, or one FP32 ulp apart (FP64 sums in another order)."""
    ulp = np.spacing(np.abs(ref_xn).astype(np.float32)).astype(np.float64)
    d = np.abs(gpu_xn.astype(np.float64) - ref_xn)
    assert np.all(d <= ulp), f"x_norm: max |diff| / ulp = {(d / ulp).max():.3g}"
    return int((d > 0).sum())


def test_tiny_input_norm_full_parity(torch_dev, tables):
    torch = torch_dev
    spec = synth.CONFIGS["tiny"]
    say("case: tiny FP32 with boundary norm, T=64")
    wts = device_weights(spec, tables)
    wts["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
    layer = make_norm_layer(spec, wts, spec.T)
    try:
        r_dev = synth.device_tensor(spec, "x", tables) * SCALE
        out, ids, w = run(torch, layer, r_dev)
        v = layer.views(spec.T)
        host = HostLayer(spec)
        rh = residual_host(spec)
        gin = synth.host(spec, "input_gamma")
        ref = host.oracle(rh, input_gamma=gin)
        nd = check_xn(v["x_norm"], ref.xn)
        near, _ = check_routing(ids, w, ref.logits, spec.k)
        assert not near
        assert np.abs(v["logits"] - ref.logits).max() < 1e-5
        u = v["pooled"].astype(np.float64) * v["row_scale"][:, None]
        check_output(u, ref.u, 1e-5, "u")
        e = check_output(out, ref.out, 1e-4)
        say(f"tiny norm: x_norm {nd} elements 1 ulp off; out max-abs/RMS = {e:.3g}")
        # the same layer without the norm, fed the oracle's normed tokens, agrees
        from latent_moe_layer_fp32_amd import LatentMoE

        plain = LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                          eps=spec.eps, act_dtype="f32", expert_dtype="f32", max_tokens=spec.T,
                          weights=wts)
        try:
            o2, i2, w2 = run(torch, plain, torch.from_numpy(v["x_norm"]).to(r_dev.device))
            assert np.array_equal(i2, ids)
            check_output(o2, out.astype(np.float64), 1e-6, "plain vs normed")
        finally:
            plain.close()
    finally:
        layer.close()


@pytest.fixture(scope="module")
def real_norm(torch_dev, tables):
    spec = synth.CONFIGS["prefill"]
    say("generating real-shape BF16 weights on the device")
    wts = device_weights(spec, tables)
    wts["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
    torch_dev.cuda.synchronize()
    layer = make_norm_layer(spec, wts, spec.T)
    host = HostLayer(spec, wts)
    yield spec, layer, host, synth.host(spec, "input_gamma")
    layer.close()


def _sample(T, n, seed):
    if n >= T:
        return np.arange(T)
    s = np.sort(np.random.default_rng(seed).choice(T, n, replace=False))
    s[-1] = T - 1
    return np.unique(s)


def test_real_input_norm_parity(torch_dev, tables, real_norm):
    """Decode (64 tokens), 4097 and 16384 tokens with the boundary norm: the
    norm's FP32 output on every token (one ulp), its BF16 rounding, logits and
    routing on every token; outputs against the exact oracle (2e-2 x RMS) and
    the FP16 emulation, stages and the stage chain on all 64 decode tokens and
    256 tokens of each prefill batch (one oracle pass over the 576 tokens)."""
    torch = torch_dev
    spec, layer, host, gin = real_norm
    k = spec.k
    r_all = (synth.device_tensor(spec, "x", tables) * SCALE).contiguous()
    rh_all = residual_host(spec)
    cases = []
    for T, n in ((64, 64), (4097, 256), (16384, 256)):
        say(f"case: BF16 with boundary norm, T={T}")
        out, ids, w = run(torch, layer, r_all[:T].contiguous())
        v = layer.views(T)
        xn_ref = oracle_xn(host, rh_all[:T], gin)
        nd = check_xn(v["x_norm"], xn_ref)
        # the split's first piece is the BF16 rounding (nearest even) of the FP32 norm
        f = v["x_norm"].view(np.uint32).astype(np.uint64)
        rne = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
        assert np.array_equal(v["x_norm_split"][:, :spec.H], rne)
        logits64 = orc.router_logits(xn_ref, to_f64(host.w["router"]), None)
        near, _ = check_routing(ids, w, logits64, k)
        dl = np.abs(v["logits"].astype(np.float64) - logits64)
        assert np.all(dl <= 2.0 ** -24 * np.abs(logits64) + 2.5e-7), f"logit error {dl.max():.3g}"
        sample = _sample(T, n, T)
        say(f"T={T}: x_norm {nd} elements 1 ulp off (all tokens); max |logit err| {dl.max():.3g}; near-ties {near}")
        cases.append(dict(T=T, rh=rh_all[sample], out=out[sample], ids=ids[sample], w=w[sample],
                          near=np.isin(sample, near), g=gather_rows(v, sample, k, out)))
    X = np.concatenate([c["rh"] for c in cases])
    IDS = np.concatenate([c["ids"] for c in cases])
    force = {int(i): IDS[i] for i in np.nonzero(np.concatenate([c["near"] for c in cases]))[0]}
    ref, em = host.oracle(X, input_gamma=gin, force_ids=force or None, emulate=(None, "f16"), keep_pairs=True)
    assert np.array_equal(IDS, ref.ids)
    G = concat_rows([c["g"] for c in cases])
    n0 = 0
    for c in cases:
        sl = slice(n0, n0 + len(c["out"]))
        n0 += len(c["out"])
        rms = float(np.sqrt(np.mean(ref.out[sl] ** 2)))
        e = check_output(c["out"], ref.out[sl], 2e-2, rms=rms)
        d = c["out"].astype(np.float64) - em.out[sl]
        ee = (float(np.abs(d).max() / rms), float(np.sqrt(np.mean(d * d)) / rms))
        say(f"T={c['T']}: out max-abs {e:.3g} x RMS on {len(c['out'])} tokens, vs emulation max {ee[0]:.3g} "
            f"rms {ee[1]:.3g}")
        assert ee[0] <= 4e-3 and ee[1] <= 6e-4, f"T={c['T']} vs FP16 emulation: max {ee[0]:.3g}, rms {ee[1]:.3g}"
    n = len(X)
    check_expert_input(G, np.arange(n), ref.u)
    check_rel_l2(G["act"], ref.a, 1e-2, "act")
    ch = check_stage_chain(G, IDS, np.concatenate([c["w"] for c in cases]), host, ref.u)
    say(f"boundary norm, {n} tokens: stage flips u {ch['u_flips']:.2g} a {ch['a_flips']:.2g} "
        f"o {ch['o_flips']:.2g} y {ch['y_flips']:.2g}, FP32 acc out {ch['out_acc']:.2g}")
