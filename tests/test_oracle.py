"""Pins of the FP64 oracle against things other than itself.

Each test checks the oracle against brute force, a closed form, an invariant
or a library routine, chosen so that a dropped term, a wrong sign or index or
a transposed operand anywhere in the oracle fails at least one of them.
"""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import synth
from oracle import brute
from oracle import oracle as orc


def rand_layer(rng, T=5, H=8, P=4, E=6, I=4, k=2, bias=False, dtype=np.float32):
    def nrm(*s, fan=1):
        return (rng.standard_normal(s) / np.sqrt(fan)).astype(dtype)

    d = dict(
        x=nrm(T, H),
        router=nrm(E, H, fan=H),
        router_bias=nrm(E) if bias else None,
        pooler=nrm(P, H, fan=H),
        pool_gamma=(1 + 0.1 * rng.standard_normal(P)).astype(dtype),
        w_gate=nrm(E, I, P, fan=P),
        w_up=nrm(E, I, P, fan=P),
        w_down=nrm(E, P, I, fan=I),
        expert_gamma=(1 + 0.1 * rng.standard_normal((E, P))).astype(dtype),
        unpooler=nrm(H, P, fan=P),
    )
    return d


def run(d, k, eps=1e-6, **kw):
    return orc.forward_inputs(d, k, eps, **kw)


def run_brute(d, k, eps=1e-6):
    f = lambda a: None if a is None else np.asarray(a, np.float64).tolist()
    return brute.forward(f(d["x"]), f(d["router"]), f(d["router_bias"]), f(d["pooler"]),
                         f(d["pool_gamma"]), f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]),
                         f(d["expert_gamma"]), f(d["unpooler"]), k, eps)


@pytest.mark.parametrize("seed,k,bias,shape", [
    (0, 2, False, dict(T=5, H=8, P=4, E=6, I=4)),
    (1, 3, True, dict(T=4, H=6, P=5, E=7, I=3)),
    (2, 1, False, dict(T=3, H=4, P=4, E=4, I=2)),
    (3, 4, True, dict(T=3, H=5, P=3, E=4, I=6)),  # k == E
])
def test_oracle_matches_brute_force(seed, k, bias, shape):
    rng = np.random.default_rng(seed)
    d = rand_layer(rng, k=k, bias=bias, **shape)
    r = run(d, k)
    out, ids, w = run_brute(d, k)
    assert np.array_equal(r.ids, np.array(ids))
    np.testing.assert_allclose(r.w, np.array(w), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.out, np.array(out), rtol=0, atol=1e-12)


def test_exact_ties_go_to_lowest_index():
    rng = np.random.default_rng(5)
    d = rand_layer(rng, T=4, E=6, k=3)
    d["router"][4] = d["router"][1]  # experts 1 and 4 always tie
    d["router"][5] = d["router"][1]
    d["router"][1] *= 1  # keep
    # make the tied experts the largest for token 0
    d["x"][0] = d["router"][1] * 10
    r = run(d, 3)
    assert list(r.ids[0]) == [1, 4, 5]
    np.testing.assert_allclose(r.w[0], [1 / 3] * 3, atol=1e-15)
    out, ids, _ = run_brute(d, 3)
    assert ids[0] == [1, 4, 5]
    assert np.array_equal(r.ids, np.array(ids))


def test_selection_uses_fp32_rounded_logits_and_flags_near_ties():
    # two logits differing below FP32 resolution: FP32 sees a tie -> lower index first
    T, H, E = 1, 2, 3
    lg = np.array([[1.0, 1.0 + 2.0 ** -30, 0.5]])
    ids, gaps = orc.select_topk(lg, 2)
    assert list(ids[0]) == [0, 1]
    assert gaps[0, 0] == pytest.approx(2.0 ** -30)
    assert orc.forward(np.zeros((1, H)), np.zeros((E, H)), lg[0], np.eye(2), np.ones(2),
                       lambda e: (np.ones((2, 2)), np.ones((2, 2)), np.ones((2, 2))),
                       np.ones((E, 2)), np.eye(2), 2, 1e-6).near_tie[0]


def test_routing_weights_closed_forms():
    rng = np.random.default_rng(7)
    d = rand_layer(rng, T=16, E=8, k=3, bias=True)
    r = run(d, 3)
    np.testing.assert_allclose(r.w.sum(-1), 1.0, atol=1e-15)
    # slot order is logit-descending
    sel = np.take_along_axis(r.logits, r.ids, -1)
    assert (np.diff(sel, axis=-1) <= 0).all()
    # weights are the library softmax of the selected logits
    np.testing.assert_allclose(r.w, scipy.special.softmax(sel, axis=-1), atol=1e-15)
    # ids are the library top-k of the logits (no ties here)
    ref = np.argsort(-r.logits, axis=-1, kind="stable")[:, :3]
    assert np.array_equal(r.ids, ref)
    # k = 1 -> weight exactly 1
    assert np.all(run(d, 1).w == 1.0)
    # zero router, zero bias -> all logits equal -> experts 0..k-1, w = 1/k
    d0 = dict(d, router=np.zeros_like(d["router"]), router_bias=None)
    r0 = run(d0, 3)
    assert (r0.ids == np.arange(3)).all()
    np.testing.assert_allclose(r0.w, 1 / 3, atol=1e-15)
    # bias enters the logits: a huge bias on expert 5 makes it slot 0 everywhere
    db = dict(d, router_bias=np.where(np.arange(8) == 5, 100.0, 0.0).astype(np.float32))
    assert (run(db, 3).ids[:, 0] == 5).all()


def test_pooled_norm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(8)
    d = rand_layer(rng, T=6, H=10, P=7, E=5, I=4, k=2)
    eps = 1e-3
    r = run(d, 2, eps=eps)
    ms = (r.h ** 2).mean(-1)
    rms = np.sqrt(((r.u / d["pool_gamma"]) ** 2).mean(-1))
    np.testing.assert_allclose(rms, np.sqrt(ms / (ms + eps)), rtol=1e-13)
    np.testing.assert_allclose(r.h, d["x"].astype(np.float64) @ d["pooler"].astype(np.float64).T,
                               rtol=1e-13)
    # with eps = 0 the output is invariant under Wp -> c Wp (c > 0)
    r1 = run(d, 2, eps=0.0)
    r2 = run(dict(d, pooler=d["pooler"].astype(np.float64) * 3.7), 2, eps=0.0)
    np.testing.assert_allclose(r2.out, r1.out, rtol=1e-12, atol=1e-13)


def test_per_expert_norm_closed_form_gamma_scale_and_invariance():
    rng = np.random.default_rng(9)
    d = rand_layer(rng, T=6, H=8, P=6, E=4, I=5, k=2)
    eps = 1e-4
    r = run(d, 2, eps=eps)
    g = d["expert_gamma"].astype(np.float64)[r.ids]  # [T,k,P]
    ms = (r.o ** 2).mean(-1)
    rms = np.sqrt(((r.ohat / g) ** 2).mean(-1))
    np.testing.assert_allclose(rms, np.sqrt(ms / (ms + eps)), rtol=1e-12)
    # gamma_e = c * 1 -> RMS(o^) = |c| sqrt(ms/(ms+eps))  (eps=0: exactly |c|)
    c = np.array([0.5, 2.0, 1.0, 3.0])
    dc = dict(d, expert_gamma=np.repeat(c[:, None], 6, axis=1))
    rc = run(dc, 2, eps=0.0)
    np.testing.assert_allclose(np.sqrt((rc.ohat ** 2).mean(-1)), c[rc.ids], rtol=1e-13)
    # eps = 0: scaling one expert's down projection leaves the output unchanged,
    # which holds only if the norm is applied to each expert separately
    wd = d["w_down"].astype(np.float64).copy()
    wd[2] *= 5.0
    r1 = run(d, 2, eps=0.0)
    r2 = run(dict(d, w_down=wd), 2, eps=0.0)
    np.testing.assert_allclose(r2.out, r1.out, rtol=1e-12, atol=1e-13)
    r3 = run(dict(d, w_down=wd), 2, eps=0.0, order="sum_then_norm")
    r4 = run(d, 2, eps=0.0, order="sum_then_norm")
    assert np.abs(r3.out - r4.out).max() > 1e-3


def test_reduces_to_textbook_block_with_identity_projections():
    """k=1, H=P, Wp=Wun=I: out = gamma_e * RMSNorm(SwiGLU-FFN_e(RMSNorm(x) * gamma_p)),
    checked against torch's own rms_norm and silu in float64."""
    rng = np.random.default_rng(10)
    P = 12
    d = rand_layer(rng, T=7, H=P, P=P, E=5, I=9, k=1)
    d["pooler"] = np.eye(P, dtype=np.float32)
    d["unpooler"] = np.eye(P, dtype=np.float32)
    eps = 1e-6
    r = run(d, 1, eps=eps)
    x = torch.tensor(d["x"], dtype=torch.float64)
    gp = torch.tensor(d["pool_gamma"], dtype=torch.float64)
    u = F.rms_norm(x, (P,), weight=gp, eps=eps)
    for t in range(7):
        e = int(r.ids[t, 0])
        Wg = torch.tensor(d["w_gate"][e], dtype=torch.float64)
        Wu = torch.tensor(d["w_up"][e], dtype=torch.float64)
        Wd = torch.tensor(d["w_down"][e], dtype=torch.float64)
        ge = torch.tensor(d["expert_gamma"][e], dtype=torch.float64)
        o = F.linear(F.silu(F.linear(u[t], Wg)) * F.linear(u[t], Wu), Wd)
        ref = F.rms_norm(o, (P,), weight=ge, eps=eps).numpy()
        np.testing.assert_allclose(r.out[t], ref, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(11)
    d = rand_layer(rng, T=9, E=6, k=3, bias=True)
    r = run(d, 3)
    perm = rng.permutation(9)
    rp = run(dict(d, x=d["x"][perm]), 3)
    assert np.array_equal(rp.ids, r.ids[perm])
    np.testing.assert_allclose(rp.w, r.w[perm], atol=1e-15)
    np.testing.assert_allclose(rp.out, r.out[perm], atol=1e-13)


def test_norm_each_then_sum_differs_from_sum_then_norm():
    spec = synth.CONFIGS["tiny"]
    d = {n: synth.host(spec, n) for n in ["x", "router", "pooler", "pool_gamma", "w_gate", "w_up",
                                          "w_down", "expert_gamma", "unpooler"]}
    d["router_bias"] = None
    a = run(d, spec.k, spec.eps)
    b = run(d, spec.k, spec.eps, order="sum_then_norm")
    rms = np.sqrt((a.out ** 2).mean())
    assert np.abs(a.out - b.out).max() > 100 * 1e-4 * rms
    # and the layer is the former: its y is the weighted sum of separately normed outputs
    ref_y = sum(a.w[:, j:j + 1] * a.ohat[:, j] for j in range(spec.k))
    np.testing.assert_allclose(a.y, ref_y, atol=1e-14)


def test_zero_input():
    rng = np.random.default_rng(12)
    d = rand_layer(rng, T=3, E=5, k=2)
    r = run(dict(d, x=np.zeros_like(d["x"])), 2)
    assert (r.ids == np.arange(2)).all()
    np.testing.assert_allclose(r.w, 0.5, atol=1e-15)
    assert np.all(r.out == 0.0)


def test_single_width_expert_closed_form():
    rng = np.random.default_rng(13)
    d = rand_layer(rng, T=5, H=6, P=1, E=4, I=3, k=2)
    eps = 1e-6
    r = run(d, 2, eps=eps)
    ge = d["expert_gamma"].astype(np.float64)[r.ids][..., 0]
    o = r.o[..., 0]
    np.testing.assert_allclose(r.ohat[..., 0], ge * o / np.sqrt(o * o + eps), rtol=1e-13)
    np.testing.assert_allclose(r.ohat[..., 0], ge * np.sign(o), rtol=1e-3)


def test_sampled_tokens_equal_full_run():
    """The layer is token-local: running a subset of tokens gives those rows."""
    spec = synth.CONFIGS["tiny"]
    d = {n: synth.host(spec, n) for n in ["x", "router", "pooler", "pool_gamma", "w_gate", "w_up",
                                          "w_down", "expert_gamma", "unpooler"]}
    d["router_bias"] = None
    full = run(d, spec.k, spec.eps)
    sel = np.array([3, 17, 40, 63])
    part = run(dict(d, x=d["x"][sel]), spec.k, spec.eps)
    np.testing.assert_allclose(part.out, full.out[sel], atol=1e-13)
    assert np.array_equal(part.ids, full.ids[sel])


def test_force_ids_recomputes_weights_from_own_logits():
    rng = np.random.default_rng(14)
    d = rand_layer(rng, T=4, E=6, k=2)
    r = run(d, 2, force_ids={1: [5, 0]})
    assert list(r.ids[1]) == [5, 0]
    lg = r.logits[1, [5, 0]]
    np.testing.assert_allclose(r.w[1], scipy.special.softmax(lg), atol=1e-15)


# ------------------------------------------------------- boundary norm (step 0)


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bits, nearest even (test-local)."""
    u = a32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("bf16_acts", [False, True])
@pytest.mark.parametrize("seed,k,shape", [
    (10, 2, dict(T=4, H=8, P=4, E=6, I=4)),
    (11, 3, dict(T=3, H=6, P=5, E=5, I=3)),
])
def test_boundary_norm_matches_brute_force(seed, k, shape, bf16_acts):
    rng = np.random.default_rng(seed)
    d = rand_layer(rng, k=k, **shape)
    d["x"] = (3.0 * d["x"] + 0.5).astype(np.float32)  # a residual stream, not unit-RMS
    gin = (1 + 0.2 * rng.standard_normal(shape["H"])).astype(np.float32)
    xs = _to_bf16_bits(d["x"]) if bf16_acts else d["x"]
    r = orc.forward(xs, d["router"], None, d["pooler"], d["pool_gamma"],
                    orc.experts_from_arrays(d["w_gate"], d["w_up"], d["w_down"]), d["expert_gamma"],
                    d["unpooler"], k, 1e-6, input_gamma=gin)
    f = lambda a: np.asarray(a, np.float64).tolist()
    xin = (xs.astype(np.uint32) << 16).view(np.float32) if bf16_acts else xs
    out, ids, w = brute.forward(f(xin), f(d["router"]), None, f(d["pooler"]), f(d["pool_gamma"]),
                                f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]), f(d["expert_gamma"]),
                                f(d["unpooler"]), k, 1e-6, input_gamma=f(gin), bf16_acts=bf16_acts)
    assert np.array_equal(r.ids, np.array(ids))
    np.testing.assert_allclose(r.w, np.array(w), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.out, np.array(out), rtol=0, atol=1e-12)


def test_boundary_norm_closed_forms_and_invariance():
    rng = np.random.default_rng(12)
    k = 2
    d = rand_layer(rng, T=6, H=16, P=8, E=5, I=4, k=k)
    res = (2.5 * d["x"] - 1.0).astype(np.float32)
    ex = orc.experts_from_arrays(d["w_gate"], d["w_up"], d["w_down"])

    def go(x, gin, eps=0.0):
        return orc.forward(x, d["router"], None, d["pooler"], d["pool_gamma"], ex, d["expert_gamma"],
                           d["unpooler"], k, eps, input_gamma=gin)

    ones = np.ones(16, np.float32)
    r1 = go(res, ones)
    # unit gamma, eps = 0: every normed row has RMS 1 (to FP32 rounding); gamma c: RMS c
    np.testing.assert_allclose(np.sqrt((r1.xn ** 2).mean(-1)), 1.0, rtol=2e-7)
    r3 = go(res, 3 * ones)
    np.testing.assert_allclose(np.sqrt((r3.xn ** 2).mean(-1)), 3.0, rtol=2e-7)
    # per-column gamma multiplies column-wise
    g = np.linspace(0.5, 2.0, 16).astype(np.float32)
    np.testing.assert_allclose(go(res, g).xn, r1.xn * g, rtol=2e-7)
    # scale invariance (power-of-two scale, eps = 0: bit-identical)
    r8 = go((8 * res).astype(np.float32), ones)
    assert np.array_equal(r8.xn, r1.xn) and np.array_equal(r8.out, r1.out)
    # FP32 activations: the layer on the residual equals the layer on its FP32 norm
    plain = orc.forward(r1.xn.astype(np.float32), d["router"], None, d["pooler"], d["pool_gamma"], ex,
                        d["expert_gamma"], d["unpooler"], k, 0.0)
    assert np.array_equal(plain.ids, r1.ids)
    np.testing.assert_allclose(plain.out, r1.out, rtol=0, atol=1e-15)
    # BF16 activations: the router reads the FP32 norm, the pooler its BF16 rounding
    rb = go(_to_bf16_bits(res), ones)
    resb = (_to_bf16_bits(res).astype(np.uint32) << 16).view(np.float32)
    xn_b = go(resb, ones).xn
    np.testing.assert_allclose(rb.logits, xn_b @ d["router"].astype(np.float64).T, rtol=1e-13, atol=1e-15)
    xb = (_to_bf16_bits(xn_b.astype(np.float32)).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert not np.array_equal(xb, xn_b)  # the rounding is visible at these values
    np.testing.assert_allclose(rb.h, xb @ d["pooler"].astype(np.float64).T, rtol=1e-13, atol=1e-15)
