"""Pins of the oracle's emulation mode (emulate="f16": u, a and y stored in
FP16 times their power-of-two range scalings, as the layer with BF16
activations declares) against the brute-force scalar oracle, which rounds
with Python's own half-precision packing and derives the scalings from the
bounds with its own loops."""
import numpy as np
import pytest

from oracle import brute
from oracle import oracle as orc
from test_oracle import rand_layer


def run_brute(d, k, eps=1e-6, **kw):
    f = lambda a: None if a is None else np.asarray(a, np.float64).tolist()
    return brute.forward(f(d["x"]), f(d["router"]), f(d["router_bias"]), f(d["pooler"]),
                         f(d["pool_gamma"]), f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]),
                         f(d["expert_gamma"]), f(d["unpooler"]), k, eps, **kw)


def close(a, b, rel=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    np.testing.assert_allclose(a, b, rtol=0, atol=rel * max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("seed,k,bias,shape,gp,ge,wgu", [
    (0, 2, False, dict(T=5, H=8, P=6, E=5, I=32), 1.0, 1.0, 1.0),
    (1, 3, True, dict(T=4, H=6, P=9, E=6, I=64), 1.0, 1.0, 1.0),
    # gammas 2^14 times larger: u and y exceed FP16's range before their scaling
    (2, 2, False, dict(T=3, H=8, P=16, E=4, I=32), 2.0 ** 14, 2.0 ** 14 * 3, 1.0),
    # gate and up weights 2^7 times larger: a needs its per-block scaling
    (3, 1, False, dict(T=4, H=5, P=8, E=3, I=64), 8.0, 1.0, 2.0 ** 7),
])
def test_emulation_matches_brute_force(seed, k, bias, shape, gp, ge, wgu):
    rng = np.random.default_rng(seed)
    d = rand_layer(rng, k=k, bias=bias, **shape)
    d["pool_gamma"] = (d["pool_gamma"] * gp).astype(np.float32)
    d["expert_gamma"] = (d["expert_gamma"] * ge).astype(np.float32)
    d["w_gate"] = (d["w_gate"] * wgu).astype(np.float32)
    d["w_up"] = (d["w_up"] * wgu).astype(np.float32)
    r = orc.forward_inputs(d, k, 1e-6, emulate="f16")
    out, ids, w = run_brute(d, k, f16_points=True)
    assert np.array_equal(r.ids, np.array(ids))
    np.testing.assert_allclose(r.w, np.array(w), rtol=0, atol=1e-14)
    close(r.out, out)
    # and it is not the exact definition (the rounding points are applied)
    ex = orc.forward_inputs(d, k, 1e-6)
    assert np.abs(r.out - ex.out).max() > 1e-6 * np.abs(ex.out).max()


def test_emulated_points_are_fp16_values():
    rng = np.random.default_rng(7)
    d = rand_layer(rng, T=6, H=8, P=16, E=4, I=32, k=2)
    d["pool_gamma"] = (d["pool_gamma"] * 2.0 ** 14).astype(np.float32)  # u scaled by 2^-c, c > 0
    r = orc.forward_inputs(d, 2, 1e-6, emulate="f16")
    ex = orc.forward_inputs(d, 2, 1e-6)
    sc = orc.f16_scales(d["pool_gamma"], d["expert_gamma"], 16)
    assert sc["u"] < 1.0 and sc["y"] == 1.0
    for v, s in ((r.u, sc["u"]), (r.y, sc["y"])):
        z = v * s
        assert np.array_equal(z, z.astype(np.float16).astype(np.float64))
        assert np.abs(z).max() <= 32768.0
    # each rounding is within half an FP16 ulp (relative 2^-11) of the value it rounds
    rel = np.abs(r.u - ex.u) / np.maximum(np.abs(ex.u), 2.0 ** -14 / sc["u"])
    assert rel.max() <= 2.0 ** -11 * (1 + 1e-12)
    # a, per expert and block of 32 outputs, times its own power of two (here < 1:
    # its bound grows with max(gamma_p)^2)
    for t in range(6):
        for j in range(2):
            e = r.ids[t, j]
            Wg, Wu = d["w_gate"][e].astype(np.float64), d["w_up"][e].astype(np.float64)
            s = np.repeat(orc.a_scales(Wg, Wu, 16, d["pool_gamma"]), 32)
            assert np.all(s < 1.0)
            z = r.a[t, j] * s
            assert np.array_equal(z, z.astype(np.float16).astype(np.float64))
            assert np.abs(z).max() <= 32768.0


def test_f16_round_saturates_and_scales_exactly():
    assert orc.f16_round(np.array([1e6, -1e6]), 1.0).tolist() == [65504.0, -65504.0]
    v = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11])  # midpoints: ties to even
    assert orc.f16_round(v, 1.0).tolist() == [1.0, 1.0 + 2.0 ** -9]
    assert orc.f16_round(v * 2.0 ** 20, 2.0 ** -20).tolist() == [2.0 ** 20, (1.0 + 2.0 ** -9) * 2.0 ** 20]
    assert orc.pow2_down(32768.0, 100) == 1.0
    assert orc.pow2_down(32769.0, 100) == 0.5
    assert orc.pow2_down(float("inf"), 60) == 2.0 ** -60


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_emulation_with_mx_activations_matches_brute_force(fmt):
    rng = np.random.default_rng(11)
    d = rand_layer(rng, T=4, H=8, P=64, E=4, I=64, k=2)
    r = orc.forward_inputs(d, 2, 1e-6, act_quant=fmt, emulate="f16")
    out, ids, _ = run_brute(d, 2, f16_points=True, **{fmt + "_acts": True})
    assert np.array_equal(r.ids, np.array(ids))
    close(r.out, out, 1e-11)


def test_kept_rows_are_the_full_rows():
    """keep_pairs given as token indices keeps exactly those tokens' per-slot
    rows (in the order given, repeats allowed), for both modes in one pass,
    and changes no output."""
    rng = np.random.default_rng(12)
    d = rand_layer(rng, T=9, H=8, P=32, E=5, I=64, k=2)
    full = orc.forward_inputs(d, 2, 1e-6, emulate=(None, "f16"))
    rows = [7, 0, 3, 7]
    part = orc.forward_inputs(d, 2, 1e-6, emulate=(None, "f16"), keep_pairs=rows)
    none = orc.forward_inputs(d, 2, 1e-6, emulate=(None, "f16"), keep_pairs=False)
    for f, p, n in zip(full, part, none):
        assert np.array_equal(f.out, p.out) and np.array_equal(f.out, n.out)
        for name in ("a", "o", "ohat"):
            assert np.array_equal(getattr(f, name)[rows], getattr(p, name))
        assert n.a is None and n.o is None and n.ohat is None


def test_scales_from_row_norms_match_the_bounds():
    """The range scalings follow their bounds: every stored value of the
    emulation lies within 2^15 after its scaling, and halving the scaling
    (the next power of two down) is never needed: the bound itself times the
    scaling lies in (2^14, 2^15] unless the scaling is 1."""
    rng = np.random.default_rng(13)
    P, I = 16, 64
    Wg, Wu = rng.standard_normal((I, P)) * 40, rng.standard_normal((I, P))
    Wd = rng.standard_normal((P, I)) * 30
    gp = np.full(P, 3.0)
    asc, osc = orc.expert_scales(Wg, Wu, Wd, P, gp)
    ng, nu, nd = (np.sqrt((W * W).sum(1)) for W in (Wg, Wu, Wd))
    ba = (ng * nu).reshape(-1, 32).max(1) * P * 9.0
    bo = nd.max() * P * 9.0 * np.sqrt(((ng * nu) ** 2).sum())
    for b, s in list(zip(ba, asc)) + [(bo, osc)]:
        assert b * s <= 32768.0 and (s == 1.0 or b * s > 16384.0)
    assert np.array_equal(asc, orc.a_scales(Wg, Wu, P, gp)) and osc == orc.o_scale(Wg, Wu, Wd, P, gp)
