"""The create/forward/destroy contract on the device, through the C ABI.

- weights are borrowed for create only: freeing and overwriting the caller's
  tensors right after create leaves the forward's output bit for bit the same;
- create runs on the caller's stream, and two handles forwarding on two
  streams at once give the results of running them in turn;
- a device allocation that fails inside create (LATENT_MOE_FAULT=alloc:N)
  returns OOM, names the size, and leaves the device's free memory where it
  was (nothing leaked);
- the poison debug mode (workspace refilled with 0xFF bytes before each
  forward, guard words after it) gives bitwise the same outputs, so no stage
  reads workspace that an earlier stage of the same forward did not write,
  and no stage writes past the workspace;
- top-k up to 32 and up to 1024 experts against the FP64 oracle, every token.
"""
import os
import sys

import numpy as np
import pytest

import synth
from layer_cases import HostLayer, check_output, check_routing, device_weights

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


def small(**over):
    return synth.CONFIGS["decode"].with_(**{"name": "small", "T": 300, "E": 16, "k": 4, **SMALL, **over})


SPECS = {
    "tiny f32": synth.CONFIGS["tiny"],
    "bf16": small(),
    "mxfp4": small(expert_format="mxfp4"),
    "bf16 boundary norm": small(input_norm=True),
    "mxfp4 + mxfp8 inputs": small(expert_format="mxfp4", expert_act="mxfp8"),
}


def make(spec, wts, max_tokens=None):
    from latent_moe_layer_fp32_amd import LatentMoE

    return LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I, top_k=spec.k,
                     eps=spec.eps, act_dtype=spec.act_dtype, expert_dtype=spec.expert_format,
                     max_tokens=max_tokens or spec.T, weights=wts, input_norm=spec.input_norm,
                     expert_act=spec.expert_act)


def build(spec, tables, max_tokens=None):
    wts = device_weights(spec, tables)
    if spec.input_norm:
        wts["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
    return make(spec, wts, max_tokens), wts


def run(torch, layer, x):
    ids = torch.empty((x.shape[0], layer.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((x.shape[0], layer.top_k), dtype=torch.float32, device=x.device)
    out = layer.forward(x, topk_ids=ids, topk_weights=w)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name", list(SPECS))
def test_weights_borrowed_for_create_only(torch_dev, tables, name):
    torch = torch_dev
    spec = SPECS[name]
    say(f"case: {name}, weights freed after create")
    keep, wk = build(spec, tables)
    free, wf = build(spec, tables)
    x = synth.device_tensor(spec, "x", tables)
    try:
        ref = run(torch, keep, x)
        # drop the caller's copies and reuse their memory for garbage
        wf.clear()
        torch.cuda.synchronize()
        junk = [torch.full((1 << 22,), float("nan"), device="cuda:0") for _ in range(64)]
        torch.cuda.synchronize()
        got = run(torch, free, x)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
        del junk
    finally:
        keep.close()
        free.close()


def test_create_on_caller_stream(torch_dev, tables):
    torch = torch_dev
    spec = SPECS["bf16"]
    say("case: create and forward on a caller-created stream")
    a, _ = build(spec, tables)
    x = synth.device_tensor(spec, "x", tables)
    ref = run(torch, a, x)
    a.close()
    st = torch.cuda.Stream()  # default priority
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        b, _ = build(spec, tables)
        got = run(torch, b, x)
    torch.cuda.synchronize()
    b.close()
    for u, v in zip(ref, got):
        assert np.array_equal(u, v)


def test_handles_on_concurrent_streams(torch_dev, tables):
    """Two handles forwarding at the same time on two caller streams (each
    handle also forks its pooler steps onto its own side stream) give bit for bit
    the results of running them one after the other: handles share no device
    state."""
    torch = torch_dev
    s1, s2 = SPECS["bf16"], SPECS["mxfp4"]
    say("case: bf16 and mxfp4 handles on two concurrent streams")
    a, _ = build(s1, tables)
    b, _ = build(s2, tables)
    xa = synth.device_tensor(s1, "x", tables)
    xb = synth.device_tensor(s2, "x", tables)
    try:
        ref_a, ref_b = run(torch, a, xa), run(torch, b, xb)
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
        outs = []
        for _ in range(3):
            sa.wait_stream(torch.cuda.current_stream())
            sb.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(sa):
                oa = a.forward(xa)
            with torch.cuda.stream(sb):
                ob = b.forward(xb)
            outs.append((oa, ob))
        torch.cuda.synchronize()
        for oa, ob in outs:
            assert np.array_equal(oa.cpu().numpy(), ref_a[0])
            assert np.array_equal(ob.cpu().numpy(), ref_b[0])
    finally:
        a.close()
        b.close()


def _free_bytes(torch):
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


@pytest.mark.parametrize("name", ["tiny f32", "bf16", "mxfp4"])
def test_failed_allocation_leaks_nothing(torch_dev, tables, name):
    torch = torch_dev
    from latent_moe_layer_fp32_amd import binding as B

    spec = SPECS[name]
    say(f"case: {name}, injected allocation failures")
    wts = device_weights(spec, tables)
    # warm the runtime (code object load, stream pools) with one full cycle
    make(spec, wts).close()
    base = _free_bytes(torch)
    for n, where in ((1, "workspace"), (2, "weight copies")):
        os.environ["LATENT_MOE_FAULT"] = f"alloc:{n}"
        try:
            with pytest.raises(B.LatentMoEError) as ei:
                make(spec, wts)
        finally:
            del os.environ["LATENT_MOE_FAULT"]
        assert ei.value.code == B.LMOE_ERR_OOM
        msg = str(ei.value)
        assert where in msg and "bytes" in msg, msg
        say(f"  alloc:{n} -> {msg}")
        assert _free_bytes(torch) == base, "device memory leaked by a failed create"
    os.environ["LATENT_MOE_FAULT"] = "alloc:3"  # no third allocation: create succeeds
    try:
        layer = make(spec, wts)
    finally:
        del os.environ["LATENT_MOE_FAULT"]
    layer.close()
    assert _free_bytes(torch) == base
    del wts


@pytest.mark.parametrize("name", list(SPECS))
def test_poison_mode_bitwise(torch_dev, tables, name):
    torch = torch_dev
    spec = SPECS[name]
    say(f"case: {name}, poisoned workspace")
    x = synth.device_tensor(spec, "x", tables)
    ref_layer, _ = build(spec, tables, max_tokens=512)
    ref = run(torch, ref_layer, x)
    ref_small = run(torch, ref_layer, x[:37].contiguous())
    ref_layer.close()
    os.environ["LATENT_MOE_DEBUG"] = "poison"
    try:
        layer, _ = build(spec, tables, max_tokens=512)
    finally:
        del os.environ["LATENT_MOE_DEBUG"]
    got = run(torch, layer, x)
    got_small = run(torch, layer, x[:37].contiguous())
    for a, b in zip(ref + ref_small, got + got_small):
        assert np.array_equal(a, b)
    assert np.isfinite(got[0]).all()
    layer.close()  # raises LMOE_ERR_CORRUPT if a guard word was overwritten


@pytest.mark.parametrize("E,k,T", [(40, 32, 130), (24, 17, 300), (1024, 8, 200), (300, 16, 150)])
def test_top_k_beyond_16(torch_dev, tables, E, k, T):
    """Top-k up to 32 and expert counts up to the largest the library takes
    (1024; 300 and 1024 run the selection kernel's wider per-lane layouts),
    every token against the FP64 oracle."""
    torch = torch_dev
    spec = small(E=E, k=k, T=T)
    say(f"case: bf16, E={E}, top-{k}, T={T}, every token")
    layer, _ = build(spec, tables, max_tokens=T)
    try:
        x = synth.device_tensor(spec, "x", tables)
        out, ids, w = run(torch, layer, x)
    finally:
        layer.close()
    host = HostLayer(spec)
    xh = host.x()
    r0 = host.oracle(xh, keep_pairs=False)
    near, _ = check_routing(ids, w, r0.logits, spec.k)
    r = host.oracle(xh, force_ids={int(t): ids[t] for t in near} or None, keep_pairs=False)
    assert np.array_equal(ids, r.ids)
    e = check_output(out, r.out, 2e-2)
    say(f"top-{k}: out max-abs {e:.3g} x RMS over all {T} tokens; near-ties {near}")
