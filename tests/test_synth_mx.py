"""The seeded input generator and the oracle's MXFP4 decoder, pinned to the
OCP Microscaling v1.0 definitions and to their own invariants."""
import numpy as np
import pytest
import torch

import synth
from oracle import mx


def test_e2m1_table_is_the_ocp_grid():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(mx.E2M1[:8]) == grid
    assert list(mx.E2M1[8:]) == [-v for v in grid]
    assert np.signbit(mx.E2M1[8])  # code 8 is -0


def test_e8m0_decode():
    v = mx.e8m0_to_f64(np.array([0, 1, 126, 127, 128, 254, 255], np.uint8))
    assert v[3] == 1.0 and v[2] == 0.5 and v[4] == 2.0
    assert v[0] == 2.0 ** -127 and v[5] == 2.0 ** 127
    assert np.isnan(v[6])


def test_bf16_decode_exact():
    f = np.array([1.0, -2.5, 3.140625, 0.0], np.float32)
    u16 = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert list(mx.bf16_to_f64(u16)) == [1.0, -2.5, 3.140625, 0.0]


def _rne_bf16(f32):
    u = f32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_generator_determinism_slices_and_threads():
    s = synth.CONFIGS["decode"].with_(E=4, I=64, P=128, H=256)
    a = synth.host(s, "w_gate", nthreads=1)
    b = synth.host(s, "w_gate", nthreads=7)
    assert np.array_equal(a, b)
    c = synth.host(s, "w_gate", experts=(1, 3))
    assert np.array_equal(c, a[1:3])
    # different tensors / seeds / chunks differ
    assert not np.array_equal(a, synth.host(s, "w_up"))
    assert not np.array_equal(a, synth.host(s.with_(seed=1), "w_gate"))
    x0 = synth.host(s, "x", chunk=0)
    x1 = synth.host(s, "x", chunk=1)
    assert not np.array_equal(x0, x1)


def test_generator_distributions():
    s = synth.CONFIGS["decode"].with_(E=8, I=256, P=512, H=1024)
    f = synth.host(s.with_(expert_format="f32"), "w_down")
    assert abs(f.mean()) < 2e-3 / np.sqrt(s.I)
    assert abs(f.std() * np.sqrt(s.I) - 1) < 2e-3
    # standardised 4th moment of a normal is 3
    z = f.astype(np.float64) * np.sqrt(s.I)
    assert abs((z ** 4).mean() - 3) < 0.03
    g = synth.host(s, "expert_gamma").astype(np.float64)
    assert abs(g.mean() - 1) < 1e-3 and abs(g.std() - 0.1) < 1e-3
    x = synth.host(synth.CONFIGS["tiny"], "x").astype(np.float64)
    assert abs(x.std() - 1) < 0.02


def test_generator_tails():
    """The normal variate reaches into the tails: 16.8M draws land beyond
    4.5 sigma about 2 * Q(4.5) * n = 114 times (Poisson), beyond 4.17 sigma
    (the two end segments, probability 2^-15) about 512 times; a table that
    stopped at the end segments' inner knots would give none beyond 4.5."""
    from scipy.special import ndtr

    s = synth.CONFIGS["decode"].with_(E=1, P=4096, I=4096, expert_format="f32")
    w = synth.host(s, "w_gate").astype(np.float64).ravel()
    z = w / float(np.float32(1.0 / np.sqrt(s.P)))
    n = z.size
    for thr in (4.17, 4.5, 5.0):
        expect = 2 * ndtr(-thr) * n
        got = int((np.abs(z) > thr).sum())
        assert abs(got - expect) < 5 * np.sqrt(expect) + 1, (thr, got, expect)
    assert np.abs(z).max() <= 6.37
    # symmetric tails
    assert abs(int((z > 4.17).sum()) - int((z < -4.17).sum())) < 5 * np.sqrt(256) + 1


def test_bf16_tensors_are_rne_of_the_fp32_draw():
    s = synth.CONFIGS["decode"].with_(E=3, I=64, P=96, H=160)
    f = synth.host(s.with_(expert_format="f32"), "w_up")
    b = synth.host(s, "w_up")
    assert np.array_equal(b, _rne_bf16(f))
    fx = synth.host(s.with_(act_dtype="f32"), "pooler")
    assert np.array_equal(synth.host(s, "pooler"), _rne_bf16(fx))


def test_mxfp4_quantiser_matches_ocp_definition():
    s = synth.CONFIGS["mxfp4"].with_(E=2, I=64, P=128, H=256)
    f = synth.host(s.with_(expert_format="f32"), "w_gate").astype(np.float64)
    packed, scales = synth.host(s, "w_gate")
    deq = mx.mxfp4_to_f64(packed, scales)
    blocks = f.reshape(-1, 32)
    dq = deq.reshape(-1, 32)
    sc = mx.e8m0_to_f64(scales.reshape(-1))
    amax = np.abs(blocks).max(-1)
    # scale = 2^(floor(log2 amax) - 2)
    np.testing.assert_array_equal(sc, 2.0 ** (np.floor(np.log2(amax)) - 2))
    # each element is a nearest grid point (ties: either neighbour is nearest)
    grid = np.unique(np.abs(mx.E2M1))
    v = np.abs(blocks) / sc[:, None]
    best = np.abs(v[..., None] - grid).min(-1)
    got = np.abs(np.abs(dq) / sc[:, None] - v)
    np.testing.assert_allclose(got, best, atol=1e-12)
    # sign preserved for non-zero codes
    nz = dq != 0
    assert (np.sign(dq[nz]) == np.sign(blocks[nz])).all()
    # the block maximum lands on 4 or 6 times the scale
    big = np.abs(dq).max(-1) / sc
    assert set(np.unique(big)) <= {4.0, 6.0}


def test_mxfp4_round_trip_and_ties_to_even():
    # quantising already-representable values reproduces their codes exactly
    s = synth.CONFIGS["mxfp4"].with_(E=1, I=32, P=64, H=64)
    packed, scales = synth.host(s, "w_down")
    deq = mx.mxfp4_to_f64(packed, scales)
    # re-encode with the OCP nearest-even rule, written from the grid table
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(deq.shape)
    sc = mx.e8m0_to_f64(scales)
    v = (deq.reshape(-1, 32) / sc.reshape(-1, 1)).reshape(deq.shape)
    re = np.array([np.argmin(np.abs(mx.E2M1[:8] - abs(t))) + (8 if (t < 0 or (t == 0 and c >= 8)) else 0)
                   for t, c in zip(v.ravel(), codes.ravel())]).reshape(codes.shape)
    assert np.array_equal(re, codes)


def test_zipf_bias():
    s = synth.CONFIGS["skew"]
    b = synth.router_bias(s).astype(np.float64)
    assert b.shape == (256,)
    w = np.exp(b)
    assert abs(w.sum() - 1) < 1e-5
    r = np.sort(w)[::-1]
    ranks = np.arange(1, 257)
    np.testing.assert_allclose(r / r[0], ranks ** -1.1, rtol=1e-5)


# ------------------------------------------------------------ MXFP8 activations


def test_e4m3_table_matches_ocp_definition():
    t = mx.E4M3
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x00] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()
    # the same values as torch's float8_e4m3fn (finite OCP E4M3) for every finite code
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(t)
    np.testing.assert_array_equal(tv[fin], t[fin])


def test_mx_quantiser_reproduces_generated_mxfp4_weights():
    # the generator (synth, C) and the oracle's quantiser (numpy) share no code
    s = synth.CONFIGS["mxfp4"].with_(E=2, I=64, P=128, H=256)
    f = synth.host(s.with_(expert_format="f32"), "w_up").astype(np.float64)
    packed, scales = synth.host(s, "w_up")
    q, e = mx.quantize_mx(f, "mxfp4")
    np.testing.assert_array_equal(q, mx.mxfp4_to_f64(packed, scales))
    np.testing.assert_array_equal(e, scales.astype(np.int64) - 127)


def test_mxfp8_quantiser_definition_ties_saturation_and_library_rounding():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-6, 6, (64, 1)))
    q, e = mx.quantize_mx(v, "mxfp8")
    b = v.reshape(-1, 32)
    amax = np.abs(b).max(-1)
    np.testing.assert_array_equal(e.reshape(-1), np.floor(np.log2(amax)) - 8)
    X = 2.0 ** e.reshape(-1, 1)
    r = b / X
    # in range (|r| <= 448), element rounding equals torch's FP8 E4M3 cast (nearest even)
    ok = np.abs(r) <= 448
    tq = torch.from_numpy(r[ok]).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    # the FP32 step is exact here: r has at most 53-bit significands but torch needs FP32 input,
    # so only compare values that FP32 holds exactly
    exact32 = r[ok].astype(np.float32).astype(np.float64) == r[ok]
    np.testing.assert_array_equal((q.reshape(-1, 32) / X)[ok][exact32], tq[exact32])
    # saturation above 448, ties to even, power-of-two equivariance, idempotence
    sat, _ = mx.quantize_mx(np.array([[480.0, 500.0, -511.0] + [1.0] * 29]), "mxfp8")
    assert sat[0, 0] == 448.0 and sat[0, 1] == 448.0 and sat[0, 2] == -448.0
    tie, _ = mx.quantize_mx(np.array([[256.0, 1.0625, 1.1875, 3 * 2.0 ** -10] + [0.0] * 28]), "mxfp8")
    assert tie[0, 1] == 1.0 and tie[0, 2] == 1.25 and tie[0, 3] == 2.0 ** -8
    q2, _ = mx.quantize_mx(v * 2.0 ** 5, "mxfp8")
    np.testing.assert_array_equal(q2, q * 2.0 ** 5)
    q3, _ = mx.quantize_mx(q, "mxfp8")
    np.testing.assert_array_equal(q3, q)
    z, ez = mx.quantize_mx(np.zeros((1, 32)), "mxfp8")
    assert not z.any() and ez[0, 0] == -127


def test_oracle_mxfp8_activations_match_brute_force():
    from oracle import brute
    from oracle import oracle as orc

    rng = np.random.default_rng(21)
    T, H, P, E, I, k = 3, 8, 32, 4, 32, 2

    def nrm(*shape, fan=1):
        return (rng.standard_normal(shape) / np.sqrt(fan)).astype(np.float32)

    d = dict(x=nrm(T, H), router=nrm(E, H, fan=H), pooler=nrm(P, H, fan=H),
             pool_gamma=(1 + 0.1 * rng.standard_normal(P)).astype(np.float32),
             w_gate=nrm(E, I, P, fan=P), w_up=nrm(E, I, P, fan=P), w_down=nrm(E, P, I, fan=I),
             expert_gamma=(1 + 0.1 * rng.standard_normal((E, P))).astype(np.float32),
             unpooler=nrm(H, P, fan=P))
    r = orc.forward_inputs(d, k, 1e-6, act_quant="mxfp8")
    plain = orc.forward_inputs(d, k, 1e-6)
    f = lambda a: np.asarray(a, np.float64).tolist()
    out, ids, w = brute.forward(f(d["x"]), f(d["router"]), None, f(d["pooler"]), f(d["pool_gamma"]),
                                f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]), f(d["expert_gamma"]),
                                f(d["unpooler"]), k, 1e-6, mxfp8_acts=True)
    assert np.array_equal(r.ids, np.array(ids))
    np.testing.assert_allclose(r.out, np.array(out), rtol=0, atol=1e-12)
    # the quantisation is visible, and of the size FP8 predicts (a few percent)
    rel = np.abs(r.out - plain.out).max() / np.sqrt(np.mean(plain.out ** 2))
    assert 1e-3 < rel < 0.2


def test_mxfp4_quantiser_ties_saturation_and_scale():
    # amax 7 -> scale 2^(floor(log2 7) - 2) = 1, so the block shows the element rule directly:
    # midpoints 0.25, 1.25, 2.5, 5 go down to the even code, 0.75, 1.75, 3.5 up; 7 saturates to 6
    blk = [7.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, 0.3, -6.5, 0.2]
    q, e = mx.quantize_mx(np.array([blk + [0.0] * (32 - len(blk))]), "mxfp4")
    assert e[0, 0] == 0
    np.testing.assert_array_equal(q[0, :len(blk)],
                                  [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -1.0, 0.5, -6.0, 0.0])
    # power-of-two equivariance and idempotence on random data
    rng = np.random.default_rng(3)
    v = rng.standard_normal((16, 64)) * np.exp(rng.uniform(-4, 4, (16, 1)))
    q1, _ = mx.quantize_mx(v, "mxfp4")
    q2, _ = mx.quantize_mx(v * 2.0 ** -7, "mxfp4")
    np.testing.assert_array_equal(q2, q1 * 2.0 ** -7)
    np.testing.assert_array_equal(mx.quantize_mx(q1, "mxfp4")[0], q1)


def test_oracle_mxfp4_activations_match_brute_force():
    from oracle import brute
    from oracle import oracle as orc

    rng = np.random.default_rng(22)
    T, H, P, E, I, k = 3, 8, 32, 4, 32, 2

    def nrm(*shape, fan=1):
        return (rng.standard_normal(shape) / np.sqrt(fan)).astype(np.float32)

    d = dict(x=nrm(T, H), router=nrm(E, H, fan=H), pooler=nrm(P, H, fan=H),
             pool_gamma=(1 + 0.1 * rng.standard_normal(P)).astype(np.float32),
             w_gate=nrm(E, I, P, fan=P), w_up=nrm(E, I, P, fan=P), w_down=nrm(E, P, I, fan=I),
             expert_gamma=(1 + 0.1 * rng.standard_normal((E, P))).astype(np.float32),
             unpooler=nrm(H, P, fan=P))
    r = orc.forward_inputs(d, k, 1e-6, act_quant="mxfp4")
    plain = orc.forward_inputs(d, k, 1e-6)
    f = lambda a: np.asarray(a, np.float64).tolist()
    out, ids, w = brute.forward(f(d["x"]), f(d["router"]), None, f(d["pooler"]), f(d["pool_gamma"]),
                                f(d["w_gate"]), f(d["w_up"]), f(d["w_down"]), f(d["expert_gamma"]),
                                f(d["unpooler"]), k, 1e-6, mxfp4_acts=True)
    assert np.array_equal(r.ids, np.array(ids))
    np.testing.assert_allclose(r.out, np.array(out), rtol=0, atol=1e-12)
    # FP4 activations move the output by far more than FP8 ones (one mantissa bit)
    rel = np.abs(r.out - plain.out).max() / np.sqrt(np.mean(plain.out ** 2))
    assert 2e-2 < rel < 1.0


def test_fast_f64_equals_to_f64():
    """The tests' fast weight decoder (torch CPU kernels) gives the oracle's
    decoded values exactly, for BF16 bits and MXFP4 (codes, scales)."""
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from layer_cases import fast_f64
    from oracle.mx import to_f64

    rng = np.random.default_rng(3)
    bf = rng.integers(0, 1 << 16, size=(64, 256), dtype=np.uint16)
    bf = bf[(bf & 0x7F80) != 0x7F80].reshape(-1)[:4096].reshape(16, 256)  # no inf / NaN patterns
    assert np.array_equal(fast_f64(bf), to_f64(bf))
    codes = rng.integers(0, 256, size=(3, 8, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(3, 8, 4), dtype=np.uint8)
    assert np.array_equal(fast_f64((codes, scales)), to_f64((codes, scales)))
