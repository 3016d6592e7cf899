"""The bounds the FP16 datapath scales u, a and y by, checked on the FP64 oracle.

The BF16 layer stores the normed expert input u, the SwiGLU output a and the
combined vector y in FP16, each times a power of two chosen at create from a
bound that holds for every token:
  |u_i| <= sqrt(P) max|gamma_p|              (an RMS-normed row: sum u^2 <= P max gamma^2)
  |y_i| <= sqrt(P) max|gamma_e|              (normed expert rows, weights summing to one)
  |a_i| <= ||Wg_i|| ||Wu_i|| P max|gamma_p|^2 (|silu(g)| <= |g|, Cauchy-Schwarz, ||u||^2 bound)
and the expert output times its expert's gamma in FP16, one power of two per expert:
  |o_p gamma_p| <= ||Wd_p|| ||a|| max|gamma_e| <= max_p ||Wd_p|| P max|gamma_p|^2
                   sqrt(sum_i (||Wg_i|| ||Wu_i||)^2) max|gamma_e|
These tests check the bounds on random layers of several scales and on inputs
that attain the u bound (a one-hot pooled row).
"""
import numpy as np
import pytest

from oracle import oracle as orc


def layer(rng, T=40, H=32, P=16, E=6, I=12, k=3, scale=1.0):
    def nrm(*s, fan=1):
        return rng.standard_normal(s) / np.sqrt(fan)

    return dict(
        x=nrm(T, H) * scale,
        router=nrm(E, H, fan=H),
        router_bias=None,
        pooler=nrm(P, H, fan=H) * scale,
        pool_gamma=1 + rng.standard_normal(P) * scale,
        w_gate=nrm(E, I, P, fan=P) * scale,
        w_up=nrm(E, I, P, fan=P) / scale,
        w_down=nrm(E, P, I, fan=I),
        expert_gamma=1 + rng.standard_normal((E, P)) * scale,
        unpooler=nrm(H, P, fan=P),
    ), k


def bounds(d):
    P = d["pooler"].shape[0]
    gp, ge = np.abs(d["pool_gamma"]).max(), np.abs(d["expert_gamma"]).max()
    ng = np.linalg.norm(d["w_gate"], axis=-1)  # [E, I]
    nu = np.linalg.norm(d["w_up"], axis=-1)
    return np.sqrt(P) * gp, np.sqrt(P) * ge, ng * nu * P * gp * gp


def o_bound(d):
    """Per expert: max_p ||Wd_p|| times the bound on ||a|| times max|gamma_e|."""
    P = d["pooler"].shape[0]
    gp = np.abs(d["pool_gamma"]).max()
    ng = np.linalg.norm(d["w_gate"], axis=-1)
    nu = np.linalg.norm(d["w_up"], axis=-1)
    nd = np.linalg.norm(d["w_down"], axis=-1).max(axis=-1)  # [E]
    gm = np.abs(d["expert_gamma"]).max(axis=-1)  # [E]
    return nd * P * gp * gp * np.sqrt(((ng * nu) ** 2).sum(axis=-1)) * gm


@pytest.mark.parametrize("seed,scale", [(0, 1.0), (1, 0.1), (2, 10.0), (3, 3.0)])
def test_bounds_hold_on_random_layers(seed, scale):
    d, k = layer(np.random.default_rng(seed), scale=scale)
    r = orc.forward_inputs(d, k, 1e-6)
    bu, by, ba = bounds(d)
    assert np.abs(r.u).max() <= bu * (1 + 1e-12)
    assert np.abs(r.y).max() <= by * (1 + 1e-12)
    bo = o_bound(d)
    T = d["x"].shape[0]
    for t in range(T):
        for j in range(k):
            e = r.ids[t, j]
            assert np.all(np.abs(r.a[t, j]) <= ba[e] * (1 + 1e-12))
            assert np.all(np.abs(r.o[t, j] * d["expert_gamma"][e]) <= bo[e] * (1 + 1e-12))


def test_u_bound_is_attained_by_a_one_hot_row():
    # pooler output h = (c, 0, ..., 0): RMSNorm gives sqrt(P) gamma_0 at element 0 (eps -> 0)
    rng = np.random.default_rng(5)
    d, k = layer(rng, T=1, H=16, P=16)
    d["x"] = np.eye(1, 16) * 3.0
    d["pooler"] = np.eye(16)
    d["pool_gamma"] = np.full(16, 2.0)
    r = orc.forward_inputs(d, k, 0.0)
    bu, _, _ = bounds(d)
    assert np.isclose(np.abs(r.u).max(), bu, rtol=1e-12)
    # and y reaches its bound when every selected expert puts its output on one element
    d["w_down"] = np.zeros_like(d["w_down"])
    d["w_down"][:, 0, :] = 1.0
    d["expert_gamma"] = np.full_like(d["expert_gamma"], 0.5)
    r = orc.forward_inputs(d, k, 0.0)
    _, by, _ = bounds(d)
    assert np.isclose(np.abs(r.y).max(), by, rtol=1e-12)
