"""Brute-force scalar version of the layer forward (test infrastructure only).

Pure-Python loops over Python floats (IEEE double), for tiny shapes. It follows
the same steps as ``oracle.forward`` (see that module's docstring for the
passages each step follows) but shares none of its code, so that a slip in
the vectorised oracle (an index, an axis, a transposed operand) shows up as a
disagreement. Inputs are nested lists or numpy arrays already decoded to
float; experts are given as full [E][N][K] nested arrays.
"""
from __future__ import annotations

import math
import struct


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16(v: float) -> float:
    """FP32 value -> bfloat16, round to nearest, ties to even."""
    bits = struct.unpack("<I", struct.pack("<f", v))[0]
    lower = bits & 0xFFFF
    upper = bits >> 16
    if lower > 0x8000 or (lower == 0x8000 and (upper & 1)):
        upper += 1
    return struct.unpack("<f", struct.pack("<I", (upper & 0xFFFF) << 16))[0]


def _e4m3_value(code: int) -> float:
    e, m = (code >> 3) & 15, code & 7
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if code & 0x80 else mag


def _mxfp8(v):
    """MX FP8 (E4M3) quantisation of a list, blocks of 32: scale 2^(floor(log2
    amax) - 8), each element the nearest finite E4M3 value (ties to the even
    code), saturating at 448. Returns the dequantised list."""
    out = []
    for b0 in range(0, len(v), 32):
        blk = v[b0:b0 + 32]
        amax = max(abs(z) for z in blk)
        if amax == 0.0:
            out.extend(0.0 for _ in blk)
            continue
        m, ex = math.frexp(amax)  # amax = m * 2^ex, 0.5 <= m < 1
        scale = 2.0 ** (ex - 1 - 8)
        for z in blk:
            q = min(abs(z) / scale, 448.0)
            best, best_d = 0, None
            for code in range(0x7F):  # +0 .. 448
                d = abs(_e4m3_value(code) - q)
                if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
                    best, best_d = code, d
            out.append(math.copysign(_e4m3_value(best) * scale, z) if best else 0.0)
    return out


_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mxfp4(v):
    """MX FP4 (E2M1) quantisation of a list, blocks of 32: scale 2^(floor(log2
    amax) - 2), each element the nearest of the eight E2M1 magnitudes (ties to
    the even code), saturating at 6. Returns the dequantised list."""
    out = []
    for b0 in range(0, len(v), 32):
        blk = v[b0:b0 + 32]
        amax = max(abs(z) for z in blk)
        if amax == 0.0:
            out.extend(0.0 for _ in blk)
            continue
        m, ex = math.frexp(amax)
        scale = 2.0 ** (ex - 1 - 2)
        for z in blk:
            q = min(abs(z) / scale, 6.0)
            best, best_d = 0, None
            for code, val in enumerate(_E2M1):
                d = abs(val - q)
                if best_d is None or d < best_d or (d == best_d and code % 2 == 0):
                    best, best_d = code, d
            out.append(math.copysign(_E2M1[best] * scale, z) if best else 0.0)
    return out


def _f16(v: float, scale: float) -> float:
    """v times scale (a power of two) stored in IEEE half precision (nearest,
    ties to even, by Python's own half-precision packing), saturating at
    +-65504, then divided by the scale again."""
    z = max(-65504.0, min(65504.0, v * scale))
    return struct.unpack("<e", struct.pack("<e", z))[0] / scale


def _down(bound: float, cap: int) -> float:
    """2^-c for the smallest c in [0, cap] with bound * 2^-c <= 2^15."""
    if bound != bound or bound == math.inf:
        return 2.0 ** -cap
    c = 0
    while c < cap and bound > 32768.0 * 2.0 ** c:
        c += 1
    return 2.0 ** -c


def _silu(z: float) -> float:
    """z * sigma(z); for z below -700, e^-z overflows a double and z e^z is used."""
    return z / (1.0 + math.exp(-z)) if z >= -700.0 else z * math.exp(z)


def _matvec(W, v):
    return [math.fsum(W[r][c] * v[c] for c in range(len(v))) for r in range(len(W))]


def _rmsnorm(v, gamma, eps):
    ms = math.fsum(z * z for z in v) / len(v)
    d = math.sqrt(ms + eps)
    return [v[i] / d * gamma[i] for i in range(len(v))]


def forward(x, router, bias, pooler, pool_gamma, w_gate, w_up, w_down, expert_gamma,
            unpooler, k, eps, input_gamma=None, bf16_acts=False, mxfp8_acts=False,
            mxfp4_acts=False, f16_points=False):
    """Returns (out [T][H], ids [T][k], w [T][k]) as Python lists.

    input_gamma: x is the pre-norm residual; the router reads its RMSNorm
    (times input_gamma) rounded to FP32, the pooler the same value rounded
    on to BF16 when bf16_acts, else the FP32 value. mxfp8_acts / mxfp4_acts:
    the expert GEMMs read u and a MX-quantised to FP8 E4M3 / FP4 E2M1.
    f16_points: u, a (unless MX-quantised), the expert output times its
    expert's gamma (gamma_e o) and y are stored in FP16 times a power of two
    each, as the layer with BF16 activations stores them: the largest 2^-c
    keeping a bound within 2^15 -- u: sqrt(P) max|gamma_p|, y: sqrt(P)
    max|gamma_e|, a (per expert, 32 outputs at a time): the largest ||Wg row||
    ||Wu row|| of the block times P max(gamma_p)^2, gamma_e o (per expert):
    see o_scale; the per-expert norm takes the RMS of the unrounded o."""
    T, E = len(x), len(router)
    if f16_points:
        P0 = len(pooler)
        gpm = max(abs(float(g)) for g in pool_gamma)
        gem = max(abs(float(g)) for row in expert_gamma for g in row)
        su = _down(math.sqrt(P0) * gpm, 100)
        sy = _down(math.sqrt(P0) * gem, 100)

        def o_scale(e):
            """2^-c keeping max_p ||Wd row p|| P max(gamma_p)^2 sqrt(sum_i (||Wg row i||
            ||Wu row i||)^2) max|gamma_e| (twice that with MX activations) within 2^15."""
            nd = max(math.sqrt(math.fsum(float(z) * float(z) for z in row)) for row in w_down[e])
            s2 = math.fsum((math.sqrt(math.fsum(float(z) * float(z) for z in w_gate[e][i]))
                            * math.sqrt(math.fsum(float(z) * float(z) for z in w_up[e][i]))) ** 2
                           for i in range(len(w_gate[e])))
            amp = 2.0 if (mxfp8_acts or mxfp4_acts) else 1.0
            gmx = max(abs(float(g)) for g in expert_gamma[e])
            return _down(nd * P0 * gpm * gpm * math.sqrt(s2) * amp * gmx, 100)

        def a_scale(e, i):
            b0 = i - i % 32
            m = 0.0
            for r in range(b0, b0 + 32):
                ng = math.sqrt(math.fsum(float(z) * float(z) for z in w_gate[e][r]))
                nu = math.sqrt(math.fsum(float(z) * float(z) for z in w_up[e][r]))
                m = max(m, ng * nu)
            return _down(m * P0 * gpm * gpm, 60)
    outs, all_ids, all_w = [], [], []
    for t in range(T):
        xt = [float(v) for v in x[t]]
        xr = xt
        if input_gamma is not None:
            xr = [_f32(z) for z in _rmsnorm(xt, [float(g) for g in input_gamma], eps)]
            xt = [_bf16(z) for z in xr] if bf16_acts else xr
        logit = _matvec(router, xr)
        if bias is not None:
            logit = [logit[e] + float(bias[e]) for e in range(E)]
        # selection on FP32-rounded logits; ties go to the lower expert index
        chosen = []
        remaining = list(range(E))
        for _ in range(k):
            best = remaining[0]
            for e in remaining[1:]:
                if _f32(logit[e]) > _f32(logit[best]):
                    best = e
            chosen.append(best)
            remaining.remove(best)
        mx = max(logit[e] for e in chosen)
        ex = [math.exp(logit[e] - mx) for e in chosen]
        s = math.fsum(ex)
        wt = [v / s for v in ex]

        u = _rmsnorm(_matvec(pooler, xt), pool_gamma, eps)
        if f16_points and not (mxfp8_acts or mxfp4_acts):
            u = [_f16(z, su) for z in u]
        if mxfp8_acts:
            u = _mxfp8(u)
        if mxfp4_acts:
            u = _mxfp4(u)
        P = len(u)
        y = [0.0] * P
        for j, e in enumerate(chosen):
            g = _matvec(w_gate[e], u)
            v = _matvec(w_up[e], u)
            a = [_silu(g[i]) * v[i] for i in range(len(g))]
            if f16_points and not (mxfp8_acts or mxfp4_acts):
                a = [_f16(a[i], a_scale(e, i)) for i in range(len(a))]
            if mxfp8_acts:
                a = _mxfp8(a)
            if mxfp4_acts:
                a = _mxfp4(a)
            o = _matvec(w_down[e], a)
            oh = _rmsnorm(o, expert_gamma[e], eps)
            if f16_points:  # gamma_e o stored in FP16 times its expert's power of two; the norm of o itself
                so = o_scale(e)
                ms = math.fsum(z * z for z in o) / len(o)
                d = math.sqrt(ms + eps)
                oh = [_f16(o[i] * float(expert_gamma[e][i]), so) / d for i in range(len(o))]
            y = [y[p] + wt[j] * oh[p] for p in range(P)]
        if f16_points:
            y = [_f16(z, sy) for z in y]
        outs.append(_matvec(unpooler, y))
        all_ids.append(chosen)
        all_w.append(wt)
    return outs, all_ids, all_w
