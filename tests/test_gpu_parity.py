"""Parity of the HIP path against the FP64 oracle, through the C ABI.

Tiny FP32 layer: every token, every stage. Real shapes (H=8192, P=4096,
E=256, I=4096, k=8, BF16): routing on every token; outputs and stage
intermediates on every token of the 64-token decode batches and on sampled
tokens of the prefill batches (the layer is token-local, so the oracle on a
token subset is exact for those rows), and once every token of the 16384-token
batch.

MXFP4 expert weights: the same real shapes, compared with the oracle run on
the identically decoded weights.

Tolerances: routing ids bit-exact except reported near-ties (< 1e-6 apart in
the FP64 logits), routing weights within 1e-6; outputs max-abs <= 2e-2 x RMS
(BF16), <= 5e-2 x RMS (MXFP4), <= 1e-4 x RMS for the FP32 layer (its expected
error is ~1e-6). Besides these bounds against the exact definition, the BF16
and MXFP4-weight outputs are checked against the oracle's emulation of the
layer's own rounding points (u, a and y in FP16 with their power-of-two range
scalings): max-abs <= 1e-3 x RMS, which leaves only FP32 accumulation order
and the rare FP16 rounding-boundary flip it causes.
"""
import sys

import numpy as np
import pytest

import synth
from layer_cases import (HostLayer, bf16_to_f64, check_expert_input, check_output, check_rel_l2,
                         check_routing, check_stage_chain, device_weights, make_layer, mx_u_ties)
from oracle import mx as mx_mod
from oracle import oracle as orc
from oracle.mx import to_f64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
# against the oracle emulating the FP16 rounding points end to end: largest
# per-element error and RMS of the error, both relative to the output RMS. The
# GPU and the emulation round the same FP16 points from FP32 and FP64 values,
# so single elements flip by one FP16 ulp where a midpoint lies between them,
# and the flips of u, a and y cascade (each stage's flips perturb the next
# stage's inputs); each stage on its own is checked to one ulp by
# check_stage_chain.
TOL_EMUL = 4e-3
TOL_EMUL_RMS = 6e-4
STAGE_L2 = 1e-2  # relative L2 bound for FP16 intermediates (expected ~1e-4)


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


def run_layer(torch, layer, x):
    T = x.shape[0]
    k = layer.top_k
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    out = layer.forward(x, topk_ids=ids, topk_weights=w)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


# --------------------------------------------------------------- tiny FP32


@pytest.fixture(scope="module")
def tiny(torch_dev, tables):
    spec = synth.CONFIGS["tiny"]
    wts = device_weights(spec, tables)
    layer = make_layer(spec, wts, max_tokens=spec.T)
    host = HostLayer(spec)
    yield spec, wts, layer, host
    layer.close()


def test_device_generator_matches_host(torch_dev, tables):
    spec = synth.CONFIGS["tiny"]
    for name in ("x", "router", "w_down", "expert_gamma"):
        d = synth.device_tensor(spec, name, tables).cpu().numpy()
        assert np.array_equal(d, synth.host(spec, name)), name
    s2 = synth.CONFIGS["decode"].with_(E=2, I=128, P=256, H=512)
    d = synth.device_tensor(s2, "w_gate", tables).view(torch_dev.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(d, synth.host(s2, "w_gate"))
    s3 = s2.with_(expert_format="mxfp4")
    dp, ds = synth.device_tensor(s3, "w_up", tables)
    hp, hs = synth.host(s3, "w_up")
    assert np.array_equal(dp.cpu().numpy(), hp) and np.array_equal(ds.cpu().numpy(), hs)


def test_tiny_full_parity(torch_dev, tiny):
    torch = torch_dev
    spec, _, layer, host = tiny
    say("case: tiny FP32, T=64")
    x = synth.device_tensor(spec, "x", synth.DeviceTables("cuda:0"))
    out, ids, w = run_layer(torch, layer, x)
    v = layer.views(spec.T)
    xh = host.x()
    r = host.oracle(xh)
    # routing
    near, _ = check_routing(ids, w, r.logits, spec.k)
    assert not near
    assert np.abs(v["logits"] - r.logits).max() < 1e-5
    # grouping: stable by expert
    order = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(v["perm_token"], order // spec.k)
    assert np.array_equal(v["pair_row"][order], np.arange(spec.T * spec.k))
    assert np.array_equal(v["counts"], np.bincount(ids.ravel(), minlength=spec.E))
    # stages
    u = v["pooled"].astype(np.float64) * v["row_scale"][:, None]
    check_output(u, r.u, 1e-5, "u")
    pr = v["pair_row"].reshape(spec.T, spec.k)
    check_output(v["act"][pr], r.a, 1e-5, "act")
    check_output(v["expert_out"][pr], r.o, 1e-5, "expert out")
    check_output(v["combined"], r.y, 1e-5, "y")
    e = check_output(out, r.out, TOL_F32)
    say(f"tiny: max-abs/RMS = {e:.3g}")


@pytest.mark.parametrize("T", [1, 3, 33, 63])
def test_tiny_ragged_token_counts(torch_dev, tiny, T):
    torch = torch_dev
    spec, _, layer, host = tiny
    say(f"case: tiny FP32 ragged T={T}")
    x = synth.device_tensor(spec, "x", synth.DeviceTables("cuda:0"))[:T].contiguous()
    out, ids, w = run_layer(torch, layer, x)
    r = host.oracle(host.x()[:T])
    check_routing(ids, w, r.logits, spec.k)
    check_output(out, r.out, TOL_F32)


def test_tiny_empty_and_errors(torch_dev, tiny):
    torch = torch_dev
    from latent_moe_layer_fp32_amd import binding as B

    spec, _, layer, _ = tiny
    x = torch.zeros((0, spec.H), dtype=torch.float32, device="cuda:0")
    out = layer.forward(x)
    assert out.shape == (0, spec.H)
    xb = torch.zeros((spec.T + 1, spec.H), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.LatentMoEError) as ei:
        layer.forward(xb)
    assert ei.value.code == B.LMOE_ERR_TOO_MANY_TOKENS
    buf = torch.zeros((spec.T * spec.H + 4,), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.LatentMoEError) as ei:
        B.latent_moe_forward(layer.handle, buf.data_ptr(), 4, buf.data_ptr() + 4, None, None, None)
    assert ei.value.code == B.LMOE_ERR_INVALID_ARG


def test_tiny_determinism_and_token_equivariance(torch_dev, tiny):
    torch = torch_dev
    spec, _, layer, _ = tiny
    say("case: tiny determinism / permutation")
    x = synth.device_tensor(spec, "x", synth.DeviceTables("cuda:0"))
    o1, i1, w1 = run_layer(torch, layer, x)
    o2, i2, w2 = run_layer(torch, layer, x)
    assert np.array_equal(o1, o2) and np.array_equal(i1, i2) and np.array_equal(w1, w2)
    perm = np.random.default_rng(3).permutation(spec.T)
    xp = x[torch.from_numpy(perm).to(x.device)].contiguous()
    op, ip, wp = run_layer(torch, layer, xp)
    assert np.array_equal(ip, i1[perm])
    assert np.array_equal(wp, w1[perm])
    assert np.array_equal(op, o1[perm])


def test_tiny_caller_stream_and_profiled_order(torch_dev, tiny):
    """Routing forks onto the handle's own stream and joins back: results on a
    caller-created stream, and with stage profiling (everything in order on
    the caller's stream), equal the default-stream results bit for bit."""
    torch = torch_dev
    from latent_moe_layer_fp32_amd import binding as B

    spec, _, layer, _ = tiny
    say("case: tiny, caller stream and profiled order")
    x = synth.device_tensor(spec, "x", synth.DeviceTables("cuda:0"))
    o1, i1, w1 = run_layer(torch, layer, x)
    st = torch.cuda.Stream()  # default priority
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device=x.device)
        w = torch.empty((spec.T, spec.k), dtype=torch.float32, device=x.device)
        out = layer.forward(x, topk_ids=ids, topk_weights=w, stream=st)
    st.synchronize()
    assert np.array_equal(out.cpu().numpy(), o1)
    assert np.array_equal(ids.cpu().numpy(), i1) and np.array_equal(w.cpu().numpy(), w1)
    B.latent_moe_set_profiling(layer.handle, True)
    try:
        o3, i3, w3 = run_layer(torch, layer, x)
        times = B.latent_moe_stage_times(layer.handle)
    finally:
        B.latent_moe_set_profiling(layer.handle, False)
    assert np.array_equal(o3, o1) and np.array_equal(i3, i1) and np.array_equal(w3, w1)
    assert len(times) == len(B.STAGES) and all(v >= 0.0 for v in times.values())


def test_tiny_zero_input(torch_dev, tiny):
    torch = torch_dev
    spec, _, layer, _ = tiny
    x = torch.zeros((5, spec.H), dtype=torch.float32, device="cuda:0")
    out, ids, w = run_layer(torch, layer, x)
    assert (ids == np.arange(spec.k)).all()
    assert np.allclose(w, 1.0 / spec.k, atol=1e-7)
    assert np.all(out == 0)


# ------------------------------------------------------------ real shapes


@pytest.fixture(scope="module")
def real(torch_dev, tables):
    spec = synth.CONFIGS["prefill"]
    say("generating real-shape BF16 weights on the device")
    wts = device_weights(spec, tables)
    torch_dev.cuda.synchronize()
    layer = make_layer(spec, wts, max_tokens=spec.T)
    host = HostLayer(spec, wts)
    yield spec, wts, layer, host
    layer.close()


def _sampled_parity(torch, spec, layer, host, x_dev, xh, sample, tol, chunk_label, emul=False, rms=None):
    """Routing on every token; stages and outputs on the sampled tokens
    against the exact oracle (bound tol) and, with emul, against the oracle
    emulating the FP16 rounding points (bound TOL_EMUL). rms: the batch output
    RMS, where known (else the RMS over the sampled rows)."""
    out, ids, w = run_layer(torch, layer, x_dev)
    T = x_dev.shape[0]
    logits64 = host.logits(xh)
    near, _ = check_routing(ids, w, logits64, spec.k)
    if near:
        say(f"{chunk_label}: near-ties at tokens {near}")
    v = layer.views(T)
    # FP32 logits: half an ulp of rounding plus a small accumulation error
    dl = np.abs(v["logits"].astype(np.float64) - logits64)
    gl = dl.max()
    say(f"{chunk_label}: max |logit error| = {gl:.3g}")
    assert np.all(dl <= 2.0 ** -24 * np.abs(logits64) + 2.5e-7)
    order = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(v["perm_token"], order // spec.k)
    assert np.array_equal(v["counts"], np.bincount(ids.ravel(), minlength=spec.E))
    force = {i: ids[t] for i, t in enumerate(sample) if t in near}
    if emul:
        r, re_ = host.oracle(xh[sample], force_ids=force or None, emulate=(None, "f16"))
    else:
        r = host.oracle(xh[sample], force_ids=force or None)
    assert np.array_equal(ids[sample], r.ids)
    pr = v["pair_row"].reshape(T, spec.k)[sample]
    eu = check_expert_input(v, sample, r.u)
    ea = check_rel_l2(bf16_to_f64(v["act"][pr]), r.a, STAGE_L2, "act")
    eo = check_rel_l2(v["expert_out"][pr], r.o, STAGE_L2, "expert out")
    ey = check_rel_l2(bf16_to_f64(v["combined"][sample]), r.y, STAGE_L2, "y")
    if rms is None:
        rms = float(np.sqrt(np.mean(r.out ** 2)))
    e = check_output(out[sample], r.out, tol, rms=rms)
    msg = (f"{chunk_label}: u max rel {eu:.3g}; rel L2 act {ea:.3g} o {eo:.3g} y {ey:.3g}; "
           f"out max-abs {e:.3g} x RMS on {len(sample)} tokens")
    if emul:
        em = emul_stats(out[sample], re_.out, rms)
        v["out"] = out
        ch = check_stage_chain(v, sample, ids[sample], w[sample], host, r.u)
        msg += (f"; vs emulation max {em[0]:.3g} rms {em[1]:.3g} x RMS; stage chain: flips u {ch['u_flips']:.2g} "
                f"a {ch['a_flips']:.2g} y {ch['y_flips']:.2g}, o {ch['o_flips']:.2g}, FP32 acc out {ch['out_acc']:.2g}")
    say(msg)
    if emul:
        assert em[0] <= TOL_EMUL and em[1] <= TOL_EMUL_RMS, f"vs FP16 emulation: max {em[0]:.3g}, rms {em[1]:.3g}"
    return out, ids


def emul_stats(out, ref, rms):
    """Largest and RMS difference between the GPU output and the emulating
    oracle's, over the output RMS."""
    d = out.astype(np.float64) - ref
    return float(np.abs(d).max() / rms), float(np.sqrt(np.mean(d * d)) / rms)


def test_decode_parity(torch_dev, tables, real):
    torch = torch_dev
    spec, _, layer, host = real
    dspec = synth.CONFIGS["decode"]
    say("case: decode BF16, T=64, every token")
    x = synth.device_tensor(dspec, "x", tables)
    xh = synth.host(dspec, "x")
    _sampled_parity(torch, dspec, layer, host, x, xh, np.arange(dspec.T), TOL_BF16, "decode", emul=True)


def test_single_token_parity(torch_dev, tables, real, mx):
    """T = 1 at real shapes: split-K projections over one row, eight experts of
    one row each (every expert tile ragged), BF16 and MXFP4 experts."""
    torch = torch_dev
    for fx, wl, tol in ((real, "decode", TOL_BF16), (mx, "mxfp4_decode", TOL_MXFP4)):
        spec, _, layer, host = fx
        dspec = synth.CONFIGS[wl]
        say(f"case: {wl}, T=1")
        x = synth.device_tensor(dspec, "x", tables)[5:6].contiguous()
        xh = synth.host(dspec, "x")[5:6]
        _sampled_parity(torch, dspec, layer, host, x, xh, np.arange(1), tol, f"{wl} T=1", emul=True)


@pytest.mark.parametrize("T", [16384, 4097, 1000])
def test_prefill_parity(torch_dev, tables, real, T):
    torch = torch_dev
    spec, _, layer, host = real
    say(f"case: prefill BF16, T={T}")
    x = synth.device_tensor(spec, "x", tables)[:T].contiguous()
    xh = synth.host(spec, "x")[:T]
    sample = np.sort(np.random.default_rng(T).choice(T, 64, replace=False))
    sample[-1] = T - 1  # ragged tail
    _sampled_parity(torch, spec, layer, host, x, xh, sample, TOL_BF16, f"prefill T={T}", emul=True)


def _every_token(torch, spec, wts, layer, host, x, xh, tol, label):
    """The whole batch against the oracle, every token and output element:
    against the exact definition (bound tol) and against the emulation of the
    FP16 rounding points (TOL_EMUL), both relative to the batch output RMS.
    The oracle reads the seeded expert weights from their device copies,
    which equal the host generator's bit for bit
    (test_device_generator_matches_host)."""
    out, ids, w = run_layer(torch, layer, x)
    near, _ = check_routing(ids, w, host.logits(xh), spec.k)

    def expert(e):  # BF16 bits or MXFP4 (codes, scales), decoded exactly
        return host.expert(e)

    force = {int(t): ids[t] for t in near}
    hw = host.w
    r, re_ = orc.forward(xh, hw["router"], hw["router_bias"], hw["pooler"], hw["pool_gamma"], expert,
                         hw["expert_gamma"], hw["unpooler"], spec.k, spec.eps, force_ids=force or None,
                         keep_pairs=False, emulate=(None, "f16"))
    assert np.array_equal(ids, r.ids)
    rms = float(np.sqrt(np.mean(r.out ** 2)))
    res = {m: np.abs(out.astype(np.float64) - q.out).max(axis=1) / rms for m, q in ((None, r), ("f16", re_))}
    em = emul_stats(out, re_.out, rms)
    # each stage against its declared rounding of the GPU's own inputs, on 512 tokens
    sub = np.sort(np.random.default_rng(1).choice(spec.T, 512, replace=False))
    v = layer.views(spec.T)
    v["out"] = out
    ch = check_stage_chain(v, sub, ids[sub], w[sub], host, r.u[sub])
    del r, re_
    per_tok, per_em = res[None], res["f16"]
    q = np.quantile(per_tok, [0.5, 0.99, 0.999])
    say(f"{label} every token: per-token max-abs / RMS median {q[0]:.3g}, p99 {q[1]:.3g}, "
        f"p99.9 {q[2]:.3g}, max {per_tok.max():.3g} (token {int(per_tok.argmax())}); against the FP16 "
        f"emulation: per-token median {np.median(per_em):.3g}, max {em[0]:.3g}, rms {em[1]:.3g}; near-ties {near}; "
        f"stage chain on 512 tokens: flips u {ch['u_flips']:.2g} a {ch['a_flips']:.2g} y {ch['y_flips']:.2g}, "
        f"o {ch['o_flips']:.2g}, FP32 acc out {ch['out_acc']:.2g}")
    assert per_tok.max() <= tol
    assert em[0] <= TOL_EMUL and em[1] <= TOL_EMUL_RMS


def test_prefill_every_token(torch_dev, tables, real):
    """The whole 16384-token BF16 batch: exact bound 2e-2 x RMS (the largest is
    expected near 4e-3) and 1e-3 x RMS against the FP16 emulation."""
    torch = torch_dev
    spec, wts, layer, host = real
    say(f"case: prefill BF16, T={spec.T}, every token")
    x = synth.device_tensor(spec, "x", tables)
    _every_token(torch, spec, wts, layer, host, x, synth.host(spec, "x"), TOL_BF16, "prefill BF16")


def test_skewed_prompt_parity(torch_dev, tables, real):
    """The skewed long prompt (five 16384-token chunks, Zipf router bias):
    routing on every token of every chunk, outputs on 64 tokens per chunk
    (exact and emulated bounds)."""
    torch = torch_dev
    spec, wts, _, _ = real
    sspec = synth.CONFIGS["skew"]
    w2 = dict(wts)
    w2["router_bias"] = synth.device_tensor(sspec, "router_bias", tables)
    layer = make_layer(sspec, w2, max_tokens=sspec.T)
    host = HostLayer(sspec, w2)
    try:
        for c in range(sspec.chunks):
            say(f"case: skewed prompt, chunk {c} of {sspec.chunks}")
            x = synth.device_tensor(sspec, "x", tables, chunk=c)
            xh = synth.host(sspec, "x", chunk=c)
            sample = np.sort(np.random.default_rng(5 + c).choice(sspec.T, 64, replace=False))
            _, ids = _sampled_parity(torch, sspec, layer, host, x, xh, sample, TOL_BF16, f"skew chunk {c}",
                                     emul=True)
            counts = np.bincount(ids.ravel(), minlength=sspec.E)
            say(f"skew chunk {c}: max expert load {counts.max()} (mean {counts.mean():.0f}), "
                f"idle experts {(counts == 0).sum()}")
            assert counts.max() > 10 * counts.mean()
    finally:
        layer.close()


# ------------------------------------------------------ MXFP4 expert weights

TOL_MXFP4 = 5e-2  # against the oracle on the identically decoded weights


@pytest.fixture(scope="module")
def mx(torch_dev, tables):
    spec = synth.CONFIGS["mxfp4"]
    say("generating real-shape MXFP4 expert weights on the device")
    wts = device_weights(spec, tables)
    torch_dev.cuda.synchronize()
    layer = make_layer(spec, wts, max_tokens=spec.T)
    host = HostLayer(spec, wts)
    yield spec, wts, layer, host
    layer.close()


def test_mxfp4_decode_parity(torch_dev, tables, mx):
    torch = torch_dev
    spec, _, layer, host = mx
    dspec = synth.CONFIGS["mxfp4_decode"]
    say("case: decode, MXFP4 experts, T=64, every token")
    x = synth.device_tensor(dspec, "x", tables)
    xh = synth.host(dspec, "x")
    _sampled_parity(torch, dspec, layer, host, x, xh, np.arange(dspec.T), TOL_MXFP4, "mxfp4 decode", emul=True)


def test_mxfp4_prefill_every_token(torch_dev, tables, mx):
    """The whole 16384-token batch with MXFP4 expert weights: 5e-2 x RMS against
    the oracle on the identically decoded weights, 1e-3 x RMS against its FP16
    emulation."""
    torch = torch_dev
    spec, wts, layer, host = mx
    say(f"case: prefill, MXFP4 experts, T={spec.T}, every token")
    x = synth.device_tensor(spec, "x", tables)
    _every_token(torch, spec, wts, layer, host, x, synth.host(spec, "x"), TOL_MXFP4, "prefill MXFP4")


def test_mxfp4_prefill_ragged(torch_dev, tables, mx):
    torch = torch_dev
    spec, _, layer, host = mx
    T = 777
    say(f"case: prefill, MXFP4 experts, T={T}")
    x = synth.device_tensor(spec, "x", tables)[:T].contiguous()
    xh = synth.host(spec, "x")[:T]
    sample = np.sort(np.random.default_rng(T + 1).choice(T, 64, replace=False))
    sample[-1] = T - 1
    _sampled_parity(torch, spec, layer, host, x, xh, sample, TOL_MXFP4, f"mxfp4 prefill T={T}", emul=True)


# ------------------------------ MX FP8 / FP4 activations against MXFP4 weights


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_activations_real_shapes(torch_dev, tables, mx, fmt):
    """The MXFP4 layer with the expert GEMMs on MX FP8 or FP4 activations
    (scaled matrix cores), against the oracle quantising u and a identically:
    every token of the decode batch and sampled tokens of the 16384-token
    batch, output max-abs <= 5e-2 x RMS."""
    torch = torch_dev
    spec, wts, _, _ = mx
    pre = "mxfp8" if fmt == "mxfp8" else "mxfp4act"
    for wl, T in ((pre + "_decode", 64), (pre, 16384)):
        s8 = synth.CONFIGS[wl]
        say(f"case: {wl}, T={T}")
        layer = make_layer(s8, wts, max_tokens=T)
        host = HostLayer(s8, wts)
        try:
            x = synth.device_tensor(s8, "x", tables)
            xh = synth.host(s8, "x")
            out, ids, w = run_layer(torch, layer, x)
            near, _ = check_routing(ids, w, host.logits(xh), s8.k)
            sample = np.arange(T) if T <= 64 else np.sort(np.random.default_rng(8).choice(T, 256, replace=False))
            force = {i: ids[t] for i, t in enumerate(sample) if t in near}
            r = host.oracle(xh[sample], act_quant=fmt, force_ids=force or None)
            assert np.array_equal(ids[sample], r.ids)
            v = layer.views(T, names=("expert_in", "expert_in_scales", "pooled", "row_scale"))
            uq = (mx_mod.mxfp4_to_f64(v["expert_in"][sample], v["expert_in_scales"][sample]) if fmt == "mxfp4"
                  else mx_mod.E4M3[v["expert_in"][sample].astype(np.int64)].reshape(len(sample), -1, 32)
                  * mx_mod.e8m0_to_f64(v["expert_in_scales"][sample])[..., None]).reshape(len(sample), -1)
            ties, nel = mx_u_ties(v, sample, uq, r, fmt)
            say(f"{wl}: u differs from the exact quantisation at {nel} of {uq.size} elements "
                f"({len(ties)} of {len(sample)} tokens), each a rounding tie of the kernel's FP32 u")
            assert nel <= 1e-3 * uq.size
            if ties:  # the oracle takes the kernel's rounding where u sits on a midpoint
                r = host.oracle(xh[sample], act_quant=fmt, force_ids=force or None, force_u=ties)
            e = check_output(out[sample], r.out, 5e-2)
            say(f"{wl}: out max-abs {e:.3g} x RMS on {len(sample)} tokens")
        finally:
            layer.close()
