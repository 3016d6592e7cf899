"""Seeded synthetic inputs for the latent-MoE layer.

This package is the only code shared by the CPU oracle and the GPU path, and it
holds none of the layer's arithmetic: it draws numbers. Every tensor is a
counter-based stream (SplitMix64 over the element index, see ``synth.hip``), so
any slice of any tensor can be produced independently on host cores
(``host``) or directly in device memory (``fill_device``), with identical bytes.

Workloads (one per layer configuration the method is exercised on):

* ``tiny``     T=64,  H=256,  P=128,  E=8,   I=128,  k=2, everything FP32
* ``decode``   T=64,  H=8192, P=4096, E=256, I=4096, k=8, BF16 x/projections/experts
* ``prefill``  T=16384, shapes as ``decode``
* ``mxfp4``    ``prefill`` with the expert weights quantised to MXFP4
* ``mxfp4_decode`` ``decode`` with the same MXFP4 expert weights
* ``mxfp8``, ``mxfp8_decode``: the MXFP4 layer with the expert GEMMs reading
  MX FP8 activations (quantised inside the layer; no extra input)
* ``mxfp4act``, ``mxfp4act_decode``: the same with MX FP4 activations
* ``decode_norm``, ``prefill_norm``: ``decode`` / ``prefill`` with x taken as the
  pre-norm residual (the layer applies its boundary norm, gamma ``input_gamma``)
* ``skew``     5 chunks of 16384 tokens, BF16, with a Zipf(s=1.1) router bias

Value distributions: x ~ N(0,1); every weight ~ N(0, 1/fan_in); RMSNorm gammas
1 + 0.1 N(0,1); router weights and gammas stay FP32; BF16 tensors are the
round-to-nearest-even of the same FP32 draw; MXFP4 tensors quantise that FP32
draw per OCP MX v1.0 (block 32 along the contiguous input axis).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, replace
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
SRC_PATH = os.path.join(_HERE, "synth.hip")

KIND_F32, KIND_BF16, KIND_MXFP4 = 0, 1, 2
MODE_SCALED, MODE_GAMMA = 0, 1


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    H: int
    P: int
    E: int
    I: int
    k: int
    eps: float = 1e-6
    act_dtype: str = "bf16"  # x, pooler and unpooler: 'f32' or 'bf16'
    expert_format: str = "bf16"  # 'f32' | 'bf16' | 'mxfp4'
    router_bias: str = "none"  # 'none' | 'zipf'
    zipf_s: float = 1.1
    chunks: int = 1
    seed: int = 0
    input_norm: bool = False  # x is the pre-norm residual; the layer applies its boundary norm
    expert_act: str | None = None  # None: BF16 activations into the experts; 'mxfp8' / 'mxfp4': MX

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


_REAL = dict(H=8192, P=4096, E=256, I=4096, k=8)
CONFIGS = {
    "tiny": LayerSpec("tiny", T=64, H=256, P=128, E=8, I=128, k=2, act_dtype="f32", expert_format="f32"),
    "decode": LayerSpec("decode", T=64, **_REAL),
    "prefill": LayerSpec("prefill", T=16384, **_REAL),
    "mxfp4": LayerSpec("mxfp4", T=16384, expert_format="mxfp4", **_REAL),
    "mxfp4_decode": LayerSpec("mxfp4_decode", T=64, expert_format="mxfp4", **_REAL),
    "mxfp8": LayerSpec("mxfp8", T=16384, expert_format="mxfp4", expert_act="mxfp8", **_REAL),
    "mxfp8_decode": LayerSpec("mxfp8_decode", T=64, expert_format="mxfp4", expert_act="mxfp8", **_REAL),
    "mxfp4act": LayerSpec("mxfp4act", T=16384, expert_format="mxfp4", expert_act="mxfp4", **_REAL),
    "mxfp4act_decode": LayerSpec("mxfp4act_decode", T=64, expert_format="mxfp4", expert_act="mxfp4",
                                 **_REAL),
    "decode_norm": LayerSpec("decode_norm", T=64, input_norm=True, **_REAL),
    "prefill_norm": LayerSpec("prefill_norm", T=16384, input_norm=True, **_REAL),
    "skew": LayerSpec("skew", T=16384, router_bias="zipf", chunks=5, **_REAL),
}

# tensor name -> (tensor id, mode)
_TENSOR_IDS = {
    "x": 0,
    "router": 1,
    "pooler": 3,
    "pool_gamma": 4,
    "w_gate": 5,
    "w_up": 6,
    "w_down": 7,
    "expert_gamma": 8,
    "unpooler": 9,
    "input_gamma": 10,
}


def shape(spec: LayerSpec, name: str) -> tuple:
    H, P, E, I, T = spec.H, spec.P, spec.E, spec.I, spec.T
    return {
        "x": (T, H),
        "router": (E, H),
        "router_bias": (E,),
        "pooler": (P, H),
        "pool_gamma": (P,),
        "w_gate": (E, I, P),
        "w_up": (E, I, P),
        "w_down": (E, P, I),
        "expert_gamma": (E, P),
        "unpooler": (H, P),
        "input_gamma": (H,),
    }[name]


def _fan_in(spec: LayerSpec, name: str) -> int:
    return {"router": spec.H, "pooler": spec.H, "w_gate": spec.P, "w_up": spec.P,
            "w_down": spec.I, "unpooler": spec.P}.get(name, 1)


def _mode(name: str) -> int:
    return MODE_GAMMA if name in ("pool_gamma", "expert_gamma", "input_gamma") else MODE_SCALED


def kind(spec: LayerSpec, name: str) -> int:
    if name in ("router", "router_bias", "pool_gamma", "expert_gamma", "input_gamma"):
        return KIND_F32
    if name in ("x", "pooler", "unpooler"):
        return KIND_F32 if spec.act_dtype == "f32" else KIND_BF16
    return {"f32": KIND_F32, "bf16": KIND_BF16, "mxfp4": KIND_MXFP4}[spec.expert_format]


def _scale(spec: LayerSpec, name: str) -> float:
    # rounded once to FP32; both generator sides multiply by this same float
    return float(np.float32(1.0 / math.sqrt(_fan_in(spec, name))))


@lru_cache(maxsize=1)
def knot_tables() -> tuple[np.ndarray, np.ndarray]:
    """Piecewise-linear inverse normal CDF, 2 x 65536 entries (see synth.hip):
    [s] for the interior segments s = 1 .. 65534 between the quantiles s/2^16
    and (s+1)/2^16, [65536 + t] for the lower tail's sub-segments between the
    quantiles t/2^32 and (t+1)/2^32, the first starting at 2^-33 (ndtri(0) is
    -inf). Entries 0 and 65535 are unused (the end segments use the tail
    table)."""
    from scipy.special import ndtri

    qi = ndtri(np.arange(65537, dtype=np.float64) / 65536.0)  # -inf, ..., +inf
    qt = ndtri(np.arange(65537, dtype=np.float64) / 2.0 ** 32)
    qt[0] = ndtri(2.0 ** -33)
    knots = np.zeros(131072, dtype=np.float32)
    slopes = np.zeros(131072, dtype=np.float32)
    knots[1:65535] = qi[1:65535]
    slopes[1:65535] = qi[2:65536] - qi[1:65535]
    knots[65536:] = qt[:-1]
    slopes[65536:] = qt[1:] - qt[:-1]
    return np.ascontiguousarray(knots), np.ascontiguousarray(slopes)


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           SRC_PATH, "-o", LIB_PATH + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("synth build failed:\n" + r.stdout + r.stderr)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if verbose:
        print(" ".join(cmd))
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        # bind to torch's HIP runtime when torch drives the device memory
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        args = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p]
        L.synth_fill_cpu.argtypes = args + [ctypes.c_int]
        L.synth_fill_cpu.restype = ctypes.c_int
        L.synth_fill_gpu.argtypes = args + [ctypes.c_void_p]
        L.synth_fill_gpu.restype = ctypes.c_int
        _lib = L
    return _lib


def router_bias(spec: LayerSpec) -> np.ndarray | None:
    """Zipf(s) log-weights at a seeded rank permutation, FP32 ``[E]`` (or None)."""
    if spec.router_bias == "none":
        return None
    rng = np.random.default_rng(np.random.SeedSequence(spec.seed, spawn_key=(2,)))
    rank = rng.permutation(spec.E) + 1  # rank[e] in 1..E
    w = rank.astype(np.float64) ** (-spec.zipf_s)
    return np.log(w / w.sum()).astype(np.float32)


def _slice(spec: LayerSpec, name: str, experts):
    """(start element, count, leading shape) for a whole tensor or an expert range."""
    shp = shape(spec, name)
    per = int(np.prod(shp[1:])) if len(shp) > 1 else 1
    if experts is None:
        return 0, int(np.prod(shp)), shp
    lo, hi = experts
    assert name in ("w_gate", "w_up", "w_down", "expert_gamma") and 0 <= lo <= hi <= spec.E
    return lo * per, (hi - lo) * per, (hi - lo,) + tuple(shp[1:])


def host(spec: LayerSpec, name: str, chunk: int = 0, experts=None, nthreads: int = 0):
    """Generate a tensor (or experts [lo, hi) of an expert tensor) in host memory.

    Returns float32 / uint16 (BF16 bits) arrays, or for MXFP4 a pair
    (packed uint8 [..., K/2], scale codes uint8 [..., K/32]).
    """
    if name == "router_bias":
        return router_bias(spec)
    start, count, shp = _slice(spec, name, experts)
    knots, slopes = knot_tables()
    kd = kind(spec, name)
    scales = None
    if kd == KIND_F32:
        out = np.empty(shp, np.float32)
    elif kd == KIND_BF16:
        out = np.empty(shp, np.uint16)
    else:
        out = np.empty(shp[:-1] + (shp[-1] // 2,), np.uint8)
        scales = np.empty(shp[:-1] + (shp[-1] // 32,), np.uint8)
    rc = lib().synth_fill_cpu(spec.seed, _TENSOR_IDS[name], chunk, kd, _mode(name), _scale(spec, name),
                              start, count, knots.ctypes.data, slopes.ctypes.data, out.ctypes.data,
                              None if scales is None else scales.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError(f"synth_fill_cpu({name}) failed: {rc}")
    return out if scales is None else (out, scales)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- device side


class DeviceTables:
    """Device copies of the knot tables (needs torch with a GPU)."""

    def __init__(self, device):
        import torch

        k, s = knot_tables()
        self.knots = torch.from_numpy(k).to(device)
        self.slopes = torch.from_numpy(s).to(device)


def device_tensor(spec: LayerSpec, name: str, tables: DeviceTables, chunk: int = 0, stream=None):
    """Allocate and fill a tensor in device memory; returns a torch tensor
    (float32 / bfloat16) or for MXFP4 a pair of uint8 tensors."""
    import torch

    dev = tables.knots.device
    if name == "router_bias":
        b = router_bias(spec)
        return None if b is None else torch.from_numpy(b).to(dev)
    shp = shape(spec, name)
    kd = kind(spec, name)
    scales = None
    if kd == KIND_F32:
        out = torch.empty(shp, dtype=torch.float32, device=dev)
    elif kd == KIND_BF16:
        out = torch.empty(shp, dtype=torch.bfloat16, device=dev)
    else:
        out = torch.empty(shp[:-1] + (shp[-1] // 2,), dtype=torch.uint8, device=dev)
        scales = torch.empty(shp[:-1] + (shp[-1] // 32,), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = lib().synth_fill_gpu(spec.seed, _TENSOR_IDS[name], chunk, kd, _mode(name), _scale(spec, name),
                              0, out.numel() * (2 if kd == KIND_MXFP4 else 1),
                              tables.knots.data_ptr(), tables.slopes.data_ptr(), out.data_ptr(),
                              None if scales is None else scales.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_gpu({name}) failed: {rc}")
    return out if scales is None else (out, scales)


WEIGHT_NAMES = ("router", "router_bias", "pooler", "pool_gamma", "w_gate", "w_up", "w_down",
                "expert_gamma", "unpooler")
