"""ctypes binding of liblatent_moe.so (C ABI in include/latent_moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch is used for device memory (tensor data pointers) and streams.
The functions below carry the C names; ``LatentMoE`` wraps them for torch
callers. If the shared library is missing this module raises on import of
``lib()``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.environ.get("LATENT_MOE_LIB") or os.path.join(HERE, "liblatent_moe.so")
HEADER = os.path.join(ROOT, "include", "latent_moe.h")

LMOE_OK = 0
LMOE_ERR_INVALID_ARG = -1
LMOE_ERR_UNSUPPORTED = -2
LMOE_ERR_OOM = -3
LMOE_ERR_HIP = -4
LMOE_ERR_TOO_MANY_TOKENS = -5
LMOE_ERR_CORRUPT = -6
LMOE_F32, LMOE_BF16, LMOE_MXFP4, LMOE_MXFP8 = 0, 1, 2, 3
DTYPE_CODES = {"f32": LMOE_F32, "bf16": LMOE_BF16, "mxfp4": LMOE_MXFP4, "mxfp8": LMOE_MXFP8}


class LatentMoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"latent_moe error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int64),
        ("pooled", ctypes.c_int64),
        ("experts", ctypes.c_int64),
        ("intermediate", ctypes.c_int64),
        ("top_k", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("act_dtype", ctypes.c_int32),
        ("expert_dtype", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
        ("input_norm", ctypes.c_int32),
        ("expert_act", ctypes.c_int32),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router", "router_bias", "pooler", "pool_gamma", "w_gate", "w_up", "w_down",
        "s_gate", "s_up", "s_down", "expert_gamma", "unpooler", "input_gamma")]


class Views(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "ids", "weights", "counts", "offsets", "perm_token", "pair_row", "pooled",
        "row_scale", "act", "expert_out", "combined", "expert_in", "expert_in_scales", "act_scales",
        "x_norm")] + [("expert_in_scale", ctypes.c_float), ("combined_scale", ctypes.c_float),
                      ("act_down", ctypes.c_void_p), ("expert_out_down", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime and puts it in the global symbol
        # scope; importing it first makes this library bind to that same
        # runtime, so torch tensors, streams and our kernels share one.
        import torch  # noqa: F401

        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.latent_moe_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(Config),
                                        ctypes.POINTER(Weights), ctypes.c_void_p]
        L.latent_moe_create.restype = ctypes.c_int
        L.latent_moe_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
        L.latent_moe_workspace_bytes.restype = ctypes.c_int
        L.latent_moe_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.latent_moe_forward.restype = ctypes.c_int
        L.latent_moe_forward_static.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]
        L.latent_moe_forward_static.restype = ctypes.c_int
        L.latent_moe_debug_views.argtypes = [ctypes.c_void_p, ctypes.POINTER(Views)]
        L.latent_moe_debug_views.restype = ctypes.c_int
        L.latent_moe_set_profiling.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.latent_moe_set_profiling.restype = ctypes.c_int
        L.latent_moe_stage_times.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.latent_moe_stage_times.restype = ctypes.c_int
        L.latent_moe_destroy.argtypes = [ctypes.c_void_p]
        L.latent_moe_destroy.restype = ctypes.c_int
        L.latent_moe_last_error.argtypes = []
        L.latent_moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Entry points declared in include/latent_moe.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(latent_moe_\w+)\s*\(", txt, re.M)))


def latent_moe_last_error() -> str:
    return lib().latent_moe_last_error().decode()


def _check(rc: int):
    if rc != LMOE_OK:
        raise LatentMoEError(rc, latent_moe_last_error())


def make_config(hidden, pooled, experts, intermediate, top_k, eps, act_dtype, expert_dtype,
                max_tokens, input_norm=False, expert_act=0) -> Config:
    return Config(hidden, pooled, experts, intermediate, top_k, eps,
                  DTYPE_CODES.get(act_dtype, act_dtype), DTYPE_CODES.get(expert_dtype, expert_dtype),
                  max_tokens, int(input_norm), DTYPE_CODES.get(expert_act, expert_act) if expert_act else 0)


def latent_moe_workspace_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().latent_moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def latent_moe_create(cfg: Config, w: Weights, stream: int | None = None) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), stream))
    return h.value


def latent_moe_forward(h: int, x: int, T: int, out: int, topk_ids: int | None,
                       topk_weights: int | None, stream: int | None) -> None:
    _check(lib().latent_moe_forward(h, x, T, out, topk_ids, topk_weights, stream))


def latent_moe_forward_static(cfg: Config, w: Weights, x: int, T: int, out: int, topk_ids: int | None,
                              topk_weights: int | None, stream: int | None) -> None:
    _check(lib().latent_moe_forward_static(ctypes.byref(cfg), ctypes.byref(w), x, T, out, topk_ids, topk_weights,
                                           stream))


def latent_moe_debug_views(h: int) -> Views:
    v = Views()
    _check(lib().latent_moe_debug_views(h, ctypes.byref(v)))
    return v


STAGES = ("input_norm", "router", "topk", "group", "pooler", "rowscale", "gate_up", "down", "combine",
          "unpooler")


def latent_moe_set_profiling(h: int, enable: bool) -> None:
    _check(lib().latent_moe_set_profiling(h, 1 if enable else 0))


def latent_moe_stage_times(h: int) -> dict:
    a = (ctypes.c_float * len(STAGES))()
    _check(lib().latent_moe_stage_times(h, a, len(STAGES)))
    return dict(zip(STAGES, [float(v) for v in a]))


def latent_moe_destroy(h: int) -> None:
    _check(lib().latent_moe_destroy(h))


# ------------------------------------------------------------- torch wrapper


def _ptr(t):
    return None if t is None else t.data_ptr()


def weight_specs(hidden, pooled, experts, intermediate, act_dtype, expert_dtype, input_norm=False,
                 router_bias=False) -> dict:
    """Expected (shape, torch dtype name) of each weight tensor; MXFP4 expert
    tensors are (packed codes, scales) pairs, given as a pair of specs."""
    H, P, E, I = hidden, pooled, experts, intermediate
    act = {"f32": "float32", "bf16": "bfloat16"}[act_dtype]
    spec = {"router": ((E, H), "float32"), "pooler": ((P, H), act), "pool_gamma": ((P,), "float32"),
            "expert_gamma": ((E, P), "float32"), "unpooler": ((H, P), act)}
    if router_bias:
        spec["router_bias"] = ((E,), "float32")
    if input_norm:
        spec["input_gamma"] = ((H,), "float32")
    for name, n, k in (("w_gate", I, P), ("w_up", I, P), ("w_down", P, I)):
        if expert_dtype == "mxfp4":
            spec[name] = (((E, n, k // 2), "uint8"), ((E, n, k // 32), "uint8"))
        else:
            spec[name] = ((E, n, k), {"f32": "float32", "bf16": "bfloat16"}[expert_dtype])
    return spec


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if str(t.dtype).replace("torch.", "") not in (dtype, "int16" if dtype == "bfloat16" else dtype):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def validate_weights(weights: dict, specs: dict, device) -> None:
    """Shape, dtype (BF16 may come as its int16 bits), device and contiguity of
    every weight; ValueError names the first mismatch."""
    # input_gamma is ignored without input_norm (as the C ABI ignores it); any
    # other name the layer does not take is an error
    extra = set(k for k, v in weights.items() if v is not None) - set(specs) - {"input_gamma"}
    if extra:
        raise ValueError(f"unexpected weights {sorted(extra)}")
    for name, sp in specs.items():
        v = weights.get(name)
        if isinstance(sp[0][0], tuple):  # MXFP4 pair
            if not isinstance(v, tuple) or len(v) != 2:
                raise ValueError(f"{name} must be a (codes, scales) pair for MXFP4 experts")
            _check_tensor(name + " codes", v[0], sp[0][0], sp[0][1], device)
            _check_tensor(name + " scales", v[1], sp[1][0], sp[1][1], device)
        else:
            _check_tensor(name, v, sp[0], sp[1], device)


def validate_forward(x, out, topk_ids, topk_weights, hidden, top_k, act_dtype, device) -> None:
    """x [T, hidden] in the activation dtype; out F32 [T, hidden]; optional
    topk_ids int32 and topk_weights F32 [T, top_k]; all contiguous on device."""
    if x.dim() != 2 or x.shape[1] != hidden:
        raise ValueError(f"x must be [T, {hidden}], got {tuple(x.shape)}")
    T = x.shape[0]
    act = {"f32": "float32", "bf16": "bfloat16"}[act_dtype]
    _check_tensor("x", x, (T, hidden), act, device)
    if out is not None:
        _check_tensor("out", out, (T, hidden), "float32", device)
    if topk_ids is not None:
        _check_tensor("topk_ids", topk_ids, (T, top_k), "int32", device)
    if topk_weights is not None:
        _check_tensor("topk_weights", topk_weights, (T, top_k), "float32", device)


class LatentMoE:
    """A layer handle created from torch device tensors.

    weights: dict with router, router_bias (or None), pooler, pool_gamma,
    w_gate, w_up, w_down (MXFP4: (packed, scales) pairs), expert_gamma,
    unpooler, and input_gamma when input_norm (x is then the pre-norm
    residual). expert_act="mxfp8" or "mxfp4" runs the expert GEMMs on MX FP8 or
    MX FP4 activations (MXFP4 experts only). Shapes, dtypes and devices are
    checked here; the library copies what it needs during create (on the
    current stream), so the tensors need not outlive the constructor.
    """

    def __init__(self, *, hidden, pooled, experts, intermediate, top_k, eps, act_dtype,
                 expert_dtype, max_tokens, weights: dict, input_norm: bool = False,
                 expert_act=None):
        import torch

        self.cfg = make_config(hidden, pooled, experts, intermediate, top_k, eps, act_dtype,
                               expert_dtype, max_tokens, input_norm, expert_act or 0)
        self.input_norm = bool(input_norm)
        self.expert_act = expert_act
        self.top_k, self.hidden, self.pooled, self.experts = top_k, hidden, pooled, experts
        self.intermediate = intermediate
        self.act_dtype, self.expert_dtype = act_dtype, expert_dtype
        self.device = torch.device("cuda", torch.cuda.current_device())
        specs = weight_specs(hidden, pooled, experts, intermediate, act_dtype, expert_dtype, input_norm,
                             weights.get("router_bias") is not None)
        validate_weights(weights, specs, self.device)
        w = Weights()
        for name in ("router", "router_bias", "pooler", "pool_gamma", "expert_gamma", "unpooler",
                     "input_gamma"):
            setattr(w, name, _ptr(weights.get(name)))
        for name, sname in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
            v = weights[name]
            if isinstance(v, tuple):
                setattr(w, name, _ptr(v[0]))
                setattr(w, sname, _ptr(v[1]))
            else:
                setattr(w, name, _ptr(v))
        self.handle = latent_moe_create(self.cfg, w, torch.cuda.current_stream(self.device).cuda_stream)

    def forward(self, x, out=None, topk_ids=None, topk_weights=None, stream=None):
        import torch

        validate_forward(x, out, topk_ids, topk_weights, self.hidden, self.top_k, self.act_dtype, self.device)
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.hidden), dtype=torch.float32, device=x.device)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        latent_moe_forward(self.handle, x.data_ptr(), T, out.data_ptr(), _ptr(topk_ids),
                           _ptr(topk_weights), stream.cuda_stream)
        return out

    __call__ = forward

    def views(self, T: int, names=None) -> dict:
        """Host copies (numpy) of the last forward's intermediates for T tokens
        (all of them, or only those in ``names``)."""
        import numpy as np
        import torch

        torch.cuda.synchronize(self.device)
        v = latent_moe_debug_views(self.handle)
        k, E, P, I = self.top_k, self.experts, self.pooled, self.intermediate
        mxa = self.expert_act in ("mxfp8", "mxfp4")
        cb = 2 if self.expert_act == "mxfp4" else 1  # elements per code byte
        f32 = self.act_dtype == "f32"
        exp_np = np.float32 if f32 else (np.uint8 if mxa else np.float16)
        spec = {
            "logits": (v.logits, (T, E), np.float32),
            "ids": (v.ids, (T, k), np.int32),
            "weights": (v.weights, (T, k), np.float32),
            "counts": (v.counts, (E,), np.int32),
            "offsets": (v.offsets, (E + 1,), np.int32),
            "perm_token": (v.perm_token, (T * k,), np.int32),
            "pair_row": (v.pair_row, (T * k,), np.int32),
            "pooled": (v.pooled, (T, P), np.float32),
            "row_scale": (v.row_scale, (T,), np.float32),
            "act": (v.act, (T * k, I // cb), exp_np),
            "expert_out": (v.expert_out, (T * k, P), np.float32 if f32 else np.float16),
            "combined": (v.combined, (T, P), np.float32 if f32 else np.float16),
        }
        if not f32 and not mxa:  # the FP16 u the expert GEMMs read
            spec["expert_in"] = (v.expert_in, (T, P), np.float16)
        if mxa:  # MX codes (FP4: two per byte) and E8M0 scales, as stored
            spec["expert_in"] = (v.expert_in, (T, P // cb), np.uint8)
            spec["expert_in_scales"] = (v.expert_in_scales, (T, P // 32), np.uint8)
            spec["act_scales"] = (v.act_scales, (T * k, I // 32), np.uint8)
        split_norm = bool(v.x_norm) and self.act_dtype != "f32"
        if v.x_norm:
            spec["x_norm"] = ((v.x_norm, (T, 3 * self.hidden), np.uint16) if split_norm
                              else (v.x_norm, (T, self.hidden), np.float32))
        res = {}
        for name, (ptr, shape, dt) in spec.items():
            if names is not None and name not in names:
                continue
            a = np.empty(shape, dt)
            _memcpy_d2h(a.ctypes.data, ptr, a.nbytes)
            res[name] = a
        # FP16 u and y are stored times a power of two (1 for ordinary gammas): the
        # views hold their values (exact in FP32)
        if not f32 and not mxa and "expert_in" in res:
            res["expert_in"] = res["expert_in"].astype(np.float32) / np.float32(v.expert_in_scale)
        if not f32 and "combined" in res:
            res["combined"] = res["combined"].astype(np.float32) / np.float32(v.combined_scale)
        if not f32 and (("act" in res and not mxa and v.act_down) or "expert_out" in res):
            offs = np.empty((E + 1,), np.int32)
            _memcpy_d2h(offs.ctypes.data, v.offsets, offs.nbytes)
            expert_of_row = np.searchsorted(offs[1:], np.arange(T * k), side="right")
            if "act" in res and not mxa and v.act_down:  # FP16 a times act_down[e][i/32]
                ad = np.empty((E, I // 32), np.float32)
                _memcpy_d2h(ad.ctypes.data, v.act_down, ad.nbytes)
                res["act"] = res["act"].astype(np.float32) / np.repeat(ad[expert_of_row], 32, axis=1)
            if "expert_out" in res:  # FP16 gamma_e * o times expert_out_down[e]
                od = np.empty((E,), np.float32)
                _memcpy_d2h(od.ctypes.data, v.expert_out_down, od.nbytes)
                res["expert_out"] = res["expert_out"].astype(np.float32) / od[expert_of_row][:, None]
        if split_norm and "x_norm" in res:  # FP32 value = sum of the three BF16 pieces (exact)
            H = self.hidden
            pcs = (res["x_norm"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            res["x_norm_split"] = res["x_norm"]
            res["x_norm"] = (pcs[:, :H] + pcs[:, H:2 * H] + pcs[:, 2 * H:]).astype(np.float32)
        return res

    def close(self):
        if getattr(self, "handle", None):
            latent_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_hip = None


def _memcpy_d2h(dst: int, src: int, nbytes: int):
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (same runtime as the library, see lib())

        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    rc = _hip.hipMemcpy(dst, src, nbytes, 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise LatentMoEError(LMOE_ERR_HIP, f"hipMemcpy failed ({rc})")
