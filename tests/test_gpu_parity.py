"""Parity of the HIP path against the FP64 oracle, through the C ABI.

Tiny FP32 layer: every token, every stage. Real shapes (H=8192, P=4096,
E=256, I=4096, k=8; BF16 experts, and MXFP4 experts compared with the oracle
on the identically decoded weights): one oracle pass over all 16384 tokens of
the prefill batch per weight set serves the decode batch (its first 64
tokens), a single token and the prefill batches (prefixes), so every token
and output element of each run is compared; stage intermediates on chosen
tokens. The skewed prompt and the MX-activation layers: routing on every
token, outputs and stages on sampled tokens (the layer is token-local, so
the oracle on a token subset is exact for those rows).

Tolerances: routing ids bit-exact except reported near-ties (< 1e-6 apart in
the FP64 logits), routing weights within 1e-6; outputs max-abs <= 2e-2 x RMS
(BF16), <= 5e-2 x RMS (MXFP4), <= 1e-4 x RMS for the FP32 layer (its expected
error is ~1e-6). Besides these bounds against the exact definition, the BF16
and MXFP4-weight outputs are checked against the oracle's emulation of the
layer's own rounding points (u, a, o and y in FP16 with their power-of-two
range scalings), and each stage on its own against its declared rounding of
the GPU's own inputs (check_stage_chain).
"""
import sys
import time
import types

import numpy as np
import pytest

import synth
from layer_cases import (HostLayer, bf16_to_f64, check_expert_input, check_output, check_rel_l2,
                         check_routing, check_stage_chain, concat_rows, device_weights, gather_rows, make_layer,
                         mx_u_ties)
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


def test_tiny_wide_tiles(torch_dev, tables):
    """The FP32 layer at 1024 tokens (256 routed rows per expert: the
    prefill-sized FP32 tiles, 128 x 128 per workgroup of 2 x 2 waves), every
    token and stage against the FP64 oracle."""
    torch = torch_dev
    spec = synth.CONFIGS["tiny"].with_(T=1024)
    say("case: tiny FP32, T=1024 (wide tiles)")
    layer = make_layer(spec, device_weights(spec, tables), max_tokens=spec.T)
    try:
        x = synth.device_tensor(spec, "x", tables)
        out, ids, w = run_layer(torch, layer, x)
        v = layer.views(spec.T)
    finally:
        layer.close()
    host = HostLayer(spec)
    r = host.oracle(host.x())
    near, _ = check_routing(ids, w, r.logits, spec.k)
    force = {int(t): ids[t] for t in near}
    if near:
        r = host.oracle(host.x(), force_ids=force)
    assert np.array_equal(ids, r.ids)
    pr = v["pair_row"].reshape(spec.T, spec.k)
    check_output(v["act"][pr], r.a, 1e-5, "act")
    check_output(v["expert_out"][pr], r.o, 1e-5, "expert out")
    check_output(v["combined"], r.y, 1e-5, "y")
    e = check_output(out, r.out, TOL_F32)
    say(f"tiny wide: max-abs/RMS = {e:.3g}, near-ties {near}")


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
# One oracle pass per weight set serves every real-shape batch: all 16384
# tokens of the prefill batch, exact and emulating the FP16 rounding points,
# keeping the per-slot rows of the tokens whose stages are checked. The decode
# batch is the first 64 of these tokens (the same seeded draws) and each
# smaller prefill batch a prefix, so every test compares every token of its
# output. A token where the GPU took the other side of a near-tie is
# recomputed with the GPU's selection.


def _sample(T, n, seed):
    """About n distinct sorted tokens of T (all when n >= T), T - 1 included."""
    if n >= T:
        return np.arange(T)
    s = np.sort(np.random.default_rng(seed).choice(T, n, replace=False))
    s[-1] = T - 1
    return np.unique(s)


# run -> (tokens of the batch the GPU runs, stage rows among them, stage chain)
BF16_RUNS = {
    "decode": (np.arange(64), np.arange(64), True),
    "T=1": (np.array([5]), np.arange(1), True),
    "T=1000": (np.arange(1000), _sample(1000, 32, 1000), False),
    "T=4097": (np.arange(4097), _sample(4097, 32, 4097), False),
    "T=16384": (np.arange(16384), _sample(16384, 128, 1), True),
}
MX_RUNS = {
    "decode": (np.arange(64), np.arange(64), True),
    "T=1": (np.array([5]), np.arange(1), True),
    "T=777": (np.arange(777), _sample(777, 32, 778), False),
    "T=16384": (np.arange(16384), _sample(16384, 64, 2), True),
}


class BatchRef:
    """The oracle on every token of a layer's 16384-token batch (exact: r,
    FP16-emulating: re), with the per-slot rows of the runs' stage tokens."""

    def __init__(self, host, x_dev, runs):
        self.host, self.x_dev, self.runs = host, x_dev, runs
        self.xh = synth.host(host.spec, "x")
        keep = np.unique(np.concatenate([tok[rows] for tok, rows, _ in runs.values()]))
        self.pos = np.full(len(self.xh), -1)
        self.pos[keep] = np.arange(len(keep))
        t0 = time.perf_counter()
        self.r, self.re = host.oracle(self.xh, keep_pairs=keep, emulate=(None, "f16"))
        say(f"oracle on all {len(self.xh)} tokens, exact and FP16-emulating: {time.perf_counter() - t0:.0f} s")


def check_batch(torch, layer, ref, name, tol, repeat=False):
    """Run the GPU on the batch of run `name` and compare: routing on every
    token (ids exact but for near-ties, weights 1e-6, logits to FP32 rounding,
    grouping), every output element against the exact oracle (tol x RMS) and
    its FP16 emulation (TOL_EMUL, TOL_EMUL_RMS), the stages of the run's stage
    rows (relative L2) and, where marked, their stage chain."""
    tok, stage, chain = ref.runs[name]
    spec = ref.host.spec
    k = spec.k
    say(f"case: {spec.expert_format} experts, {name}")
    x = ref.x_dev[int(tok[0]):int(tok[-1]) + 1]  # the runs' batches are contiguous token ranges
    assert x.shape[0] == len(tok)
    out, ids, w = run_layer(torch, layer, x.contiguous())
    if repeat:  # run to run, bit for bit (fixed reduction orders, no atomics on values)
        out2, ids2, w2 = run_layer(torch, layer, x.contiguous())
        assert np.array_equal(out2, out) and np.array_equal(ids2, ids) and np.array_equal(w2, w), "second run differs"
    T = len(tok)
    r, re_ = ref.r, ref.re
    logits64 = r.logits[tok]
    near, _ = check_routing(ids, w, logits64, k)
    v = layer.views(T)
    dl = np.abs(v["logits"].astype(np.float64) - logits64)
    assert np.all(dl <= 2.0 ** -24 * np.abs(logits64) + 2.5e-7), f"logit error {dl.max():.3g}"
    order = np.argsort(ids.ravel(), kind="stable")
    assert np.array_equal(v["perm_token"], order // k)
    assert np.array_equal(v["counts"], np.bincount(ids.ravel(), minlength=spec.E))
    ro, reo = r.out[tok], re_.out[tok]
    redo = np.nonzero((ids != r.ids[tok]).any(axis=1))[0]
    if len(redo):
        say(f"{name}: near-ties taken the other way at tokens {tok[redo].tolist()}: oracle with the GPU's selection")
        f = {j: ids[i] for j, i in enumerate(redo)}
        a, b = ref.host.oracle(ref.xh[tok[redo]], force_ids=f, emulate=(None, "f16"), keep_pairs=False)
        ro[redo], reo[redo] = a.out, b.out
    rms = float(np.sqrt(np.mean(ro ** 2)))
    per_tok = np.abs(out.astype(np.float64) - ro).max(axis=1) / rms
    em = emul_stats(out, reo, rms)
    msg = (f"{name}: every token, per-token max-abs / RMS median {np.median(per_tok):.3g}, max {per_tok.max():.3g} "
           f"(token {int(tok[per_tok.argmax()])}); vs FP16 emulation max {em[0]:.3g} rms {em[1]:.3g}")
    stage = np.setdiff1d(stage, redo)
    if len(stage):
        tk = tok[stage]
        kr = ref.pos[tk]
        pr = v["pair_row"].reshape(T, k)[stage]
        eu = check_expert_input(v, stage, r.u[tk])
        ea = check_rel_l2(bf16_to_f64(v["act"][pr]), r.a[kr], STAGE_L2, "act")
        eo = check_rel_l2(v["expert_out"][pr], r.o[kr] * ref.host.gamma_o(ids[stage]), STAGE_L2, "expert out")
        ey = check_rel_l2(bf16_to_f64(v["combined"][stage]), r.y[tk], STAGE_L2, "y")
        msg += f"; stages on {len(stage)} tokens: u max rel {eu:.3g}, rel L2 act {ea:.3g} o {eo:.3g} y {ey:.3g}"
        if chain:
            ch = check_stage_chain(gather_rows(v, stage, k, out), ids[stage], w[stage], ref.host, r.u[tk])
            msg += (f"; stage chain flips u {ch['u_flips']:.2g} a {ch['a_flips']:.2g} o {ch['o_flips']:.2g} "
                    f"y {ch['y_flips']:.2g}, FP32 acc out {ch['out_acc']:.2g}")
    say(msg)
    assert per_tok.max() <= tol, f"{name}: max-abs error {per_tok.max():.3g} x RMS > {tol}"
    assert em[0] <= TOL_EMUL and em[1] <= TOL_EMUL_RMS, f"vs FP16 emulation: max {em[0]:.3g}, rms {em[1]:.3g}"
    return out, ids, w


def emul_stats(out, ref, rms):
    """Largest and RMS difference between the GPU output and the emulating
    oracle's, over the output RMS."""
    d = out.astype(np.float64) - ref
    return float(np.abs(d).max() / rms), float(np.sqrt(np.mean(d * d)) / rms)


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


@pytest.fixture(scope="module")
def real_ref(tables, real):
    spec, _, _, host = real
    return BatchRef(host, synth.device_tensor(spec, "x", tables), BF16_RUNS)


def test_decode_parity(torch_dev, real, real_ref):
    check_batch(torch_dev, real[2], real_ref, "decode", TOL_BF16)


def test_single_token_parity(torch_dev, real, real_ref):
    """T = 1 at real shapes: split-K projections over one row, eight experts
    of one row each (every expert tile ragged)."""
    check_batch(torch_dev, real[2], real_ref, "T=1", TOL_BF16)


@pytest.mark.parametrize("T", [4097, 1000])
def test_prefill_parity(torch_dev, real, real_ref, T):
    check_batch(torch_dev, real[2], real_ref, f"T={T}", TOL_BF16)


def test_prefill_every_token(torch_dev, real, real_ref):
    """The whole 16384-token BF16 batch: every output element within 2e-2 x
    RMS of the exact oracle (the largest is expected near 4e-3) and within the
    emulation bounds of the FP16-emulating oracle; stage chain on 128 tokens;
    a second forward bit for bit equal to the first."""
    check_batch(torch_dev, real[2], real_ref, "T=16384", TOL_BF16, repeat=True)


def test_skewed_prompt_parity(torch_dev, tables, real):
    """The skewed long prompt (five 16384-token chunks, Zipf router bias):
    routing on every token of every chunk; outputs, stages and the stage chain
    on 64 tokens per chunk (one oracle pass over the 320 tokens)."""
    torch = torch_dev
    spec, wts, _, _ = real
    sspec = synth.CONFIGS["skew"]
    k = sspec.k
    w2 = dict(wts)
    w2["router_bias"] = synth.device_tensor(sspec, "router_bias", tables)
    layer = make_layer(sspec, w2, max_tokens=sspec.T)
    host = HostLayer(sspec, w2)
    xs, outs, idss, ws, gath, nears = [], [], [], [], [], []
    try:
        for c in range(sspec.chunks):
            say(f"case: skewed prompt, chunk {c} of {sspec.chunks}")
            x = synth.device_tensor(sspec, "x", tables, chunk=c)
            xh = synth.host(sspec, "x", chunk=c)
            out, ids, w = run_layer(torch, layer, x)
            logits64 = host.logits(xh)
            near, _ = check_routing(ids, w, logits64, k)
            v = layer.views(sspec.T)
            dl = np.abs(v["logits"].astype(np.float64) - logits64)
            assert np.all(dl <= 2.0 ** -24 * np.abs(logits64) + 2.5e-7), f"logit error {dl.max():.3g}"
            order = np.argsort(ids.ravel(), kind="stable")
            assert np.array_equal(v["perm_token"], order // k)
            counts = np.bincount(ids.ravel(), minlength=sspec.E)
            assert np.array_equal(v["counts"], counts)
            say(f"skew chunk {c}: max expert load {counts.max()} (mean {counts.mean():.0f}), "
                f"idle experts {(counts == 0).sum()}, near-ties {near}")
            assert counts.max() > 10 * counts.mean()
            sample = _sample(sspec.T, 64, 5 + c)
            xs.append(xh[sample])
            outs.append(out[sample])
            idss.append(ids[sample])
            ws.append(w[sample])
            gath.append(gather_rows(v, sample, k, out))
            nears.append(np.isin(sample, near))
    finally:
        layer.close()
    X, IDS, W = np.concatenate(xs), np.concatenate(idss), np.concatenate(ws)
    force = {int(i): IDS[i] for i in np.nonzero(np.concatenate(nears))[0]}
    r, re_ = host.oracle(X, force_ids=force or None, emulate=(None, "f16"), keep_pairs=True)
    assert np.array_equal(IDS, r.ids)
    G = concat_rows(gath)
    n0 = 0
    for c, o in enumerate(outs):
        sl = slice(n0, n0 + len(o))
        n0 += len(o)
        rms = float(np.sqrt(np.mean(r.out[sl] ** 2)))
        e = check_output(o, r.out[sl], TOL_BF16, rms=rms)
        em = emul_stats(o, re_.out[sl], rms)
        say(f"skew chunk {c}: out max-abs {e:.3g} x RMS on {len(o)} tokens, vs emulation max {em[0]:.3g} "
            f"rms {em[1]:.3g}")
        assert em[0] <= TOL_EMUL and em[1] <= TOL_EMUL_RMS, f"chunk {c} vs FP16 emulation: {em}"
    n = len(X)
    eu = check_expert_input(G, np.arange(n), r.u)
    ea = check_rel_l2(G["act"], r.a, STAGE_L2, "act")
    eo = check_rel_l2(G["expert_out"], r.o * host.gamma_o(IDS), STAGE_L2, "expert out")
    ey = check_rel_l2(G["combined"], r.y, STAGE_L2, "y")
    ch = check_stage_chain(G, IDS, W, host, r.u)
    say(f"skew, {n} tokens: u max rel {eu:.3g}, rel L2 act {ea:.3g} o {eo:.3g} y {ey:.3g}; stage chain flips "
        f"u {ch['u_flips']:.2g} a {ch['a_flips']:.2g} o {ch['o_flips']:.2g} y {ch['y_flips']:.2g}, "
        f"FP32 acc out {ch['out_acc']:.2g}")


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


@pytest.fixture(scope="module")
def mx_ref(tables, mx):
    spec, _, _, host = mx
    return BatchRef(host, synth.device_tensor(spec, "x", tables), MX_RUNS)


def test_mxfp4_decode_parity(torch_dev, mx, mx_ref):
    check_batch(torch_dev, mx[2], mx_ref, "decode", TOL_MXFP4)


def test_mxfp4_single_token_parity(torch_dev, mx, mx_ref):
    check_batch(torch_dev, mx[2], mx_ref, "T=1", TOL_MXFP4)


def test_mxfp4_prefill_ragged(torch_dev, mx, mx_ref):
    check_batch(torch_dev, mx[2], mx_ref, "T=777", TOL_MXFP4)


def test_mxfp4_prefill_every_token(torch_dev, mx, mx_ref):
    """The whole 16384-token batch with MXFP4 expert weights: 5e-2 x RMS
    against the oracle on the identically decoded weights, and the emulation
    bounds against its FP16 emulation; a second forward bit for bit equal."""
    check_batch(torch_dev, mx[2], mx_ref, "T=16384", TOL_MXFP4, repeat=True)


# ------------------------------ MX FP8 / FP4 activations against MXFP4 weights


def _mx_codes(v, rows, fmt):
    if fmt == "mxfp4":
        return mx_mod.mxfp4_to_f64(v["expert_in"][rows], v["expert_in_scales"][rows])
    n = len(rows)
    return (mx_mod.E4M3[v["expert_in"][rows].astype(np.int64)].reshape(n, -1, 32)
            * mx_mod.e8m0_to_f64(v["expert_in_scales"][rows])[..., None]).reshape(n, -1)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_activations_real_shapes(torch_dev, tables, mx, fmt):
    """The MXFP4 layer with the expert GEMMs on MX FP8 or FP4 activations
    (scaled matrix cores), against the oracle quantising u and a identically:
    every token of the decode batch and 256 tokens of the 16384-token batch
    (one oracle pass over both), output max-abs <= 5e-2 x RMS."""
    torch = torch_dev
    spec, wts, _, _ = mx
    pre = "mxfp8" if fmt == "mxfp8" else "mxfp4act"
    runs = []
    host = HostLayer(synth.CONFIGS[pre], wts)
    for wl, T in ((pre + "_decode", 64), (pre, 16384)):
        s8 = synth.CONFIGS[wl]
        say(f"case: {wl}, T={T}")
        layer = make_layer(s8, wts, max_tokens=T)
        try:
            x = synth.device_tensor(s8, "x", tables)
            xh = synth.host(s8, "x")
            out, ids, w = run_layer(torch, layer, x)
            near, _ = check_routing(ids, w, host.logits(xh), s8.k)
            sample = np.arange(T) if T <= 64 else _sample(T, 256, 8)
            v = layer.views(T, names=("expert_in", "expert_in_scales", "pooled", "row_scale"))
            sub = {n: v[n][sample] for n in ("pooled", "row_scale")}
            runs.append(dict(wl=wl, xh=xh[sample], out=out[sample], ids=ids[sample], near=np.isin(sample, near),
                             uq=_mx_codes(v, sample, fmt), v=sub))
        finally:
            layer.close()
    X = np.concatenate([q["xh"] for q in runs])
    IDS = np.concatenate([q["ids"] for q in runs])
    force = {int(i): IDS[i] for i in np.nonzero(np.concatenate([q["near"] for q in runs]))[0]}
    r = host.oracle(X, act_quant=fmt, force_ids=force or None, keep_pairs=False)
    assert np.array_equal(IDS, r.ids)
    ref_out = r.out.copy()
    n0 = 0
    for q in runs:
        n = len(q["xh"])
        sl = slice(n0, n0 + n)
        rr = types.SimpleNamespace(u_pre=r.u_pre[sl], u=r.u[sl])
        ties, nel = mx_u_ties(q["v"], np.arange(n), q["uq"], rr, fmt)
        say(f"{q['wl']}: u differs from the exact quantisation at {nel} of {q['uq'].size} elements "
            f"({len(ties)} of {n} tokens), each a rounding tie of the kernel's FP32 u")
        assert nel <= 1e-3 * q["uq"].size
        if ties:  # the oracle takes the kernel's rounding where u sits on a midpoint
            tt = np.array(sorted(ties))
            f = {j: q["ids"][t] for j, t in enumerate(tt)}
            rt = host.oracle(q["xh"][tt], act_quant=fmt, force_ids=f, keep_pairs=False,
                             force_u={j: ties[t] for j, t in enumerate(tt)})
            ref_out[n0 + tt] = rt.out
        e = check_output(q["out"], ref_out[sl], 5e-2)
        say(f"{q['wl']}: out max-abs {e:.3g} x RMS on {n} tokens")
        n0 += n
