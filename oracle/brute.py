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


def _matvec(W, v):
    return [math.fsum(W[r][c] * v[c] for c in range(len(v))) for r in range(len(W))]


def _rmsnorm(v, gamma, eps):
    ms = math.fsum(z * z for z in v) / len(v)
    d = math.sqrt(ms + eps)
    return [v[i] / d * gamma[i] for i in range(len(v))]


def forward(x, router, bias, pooler, pool_gamma, w_gate, w_up, w_down, expert_gamma,
            unpooler, k, eps, input_gamma=None, bf16_acts=False, mxfp8_acts=False,
            mxfp4_acts=False):
    """Returns (out [T][H], ids [T][k], w [T][k]) as Python lists.

    input_gamma: x is the pre-norm residual; the router reads its RMSNorm
    (times input_gamma) rounded to FP32, the pooler the same value rounded
    on to BF16 when bf16_acts, else the FP32 value. mxfp8_acts / mxfp4_acts:
    the expert GEMMs read u and a MX-quantised to FP8 E4M3 / FP4 E2M1."""
    T, E = len(x), len(router)
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
        if mxfp8_acts:
            u = _mxfp8(u)
        if mxfp4_acts:
            u = _mxfp4(u)
        P = len(u)
        y = [0.0] * P
        for j, e in enumerate(chosen):
            g = _matvec(w_gate[e], u)
            v = _matvec(w_up[e], u)
            a = [g[i] / (1.0 + math.exp(-g[i])) * v[i] for i in range(len(g))]
            if mxfp8_acts:
                a = _mxfp8(a)
            if mxfp4_acts:
                a = _mxfp4(a)
            o = _matvec(w_down[e], a)
            oh = _rmsnorm(o, expert_gamma[e], eps)
            y = [y[p] + wt[j] * oh[p] for p in range(P)]
        outs.append(_matvec(unpooler, y))
        all_ids.append(chosen)
        all_w.append(wt)
    return outs, all_ids, all_w
