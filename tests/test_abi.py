"""C ABI surface: the library loads, exports what the header declares, and
rejects bad arguments on the host before touching a device."""
import ctypes

import pytest

from latent_moe_layer_fp32_amd import binding as B


def _has_device() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


def real_cfg(**kw):
    d = dict(hidden=8192, pooled=4096, experts=256, intermediate=4096, top_k=8, eps=1e-6,
             act_dtype="bf16", expert_dtype="bf16", max_tokens=16384, input_norm=0, expert_act=0)
    d.update(kw)
    return B.make_config(**d)


def test_library_exports_every_header_symbol():
    syms = B.header_symbols()
    assert {"latent_moe_create", "latent_moe_forward", "latent_moe_destroy",
            "latent_moe_last_error"} <= set(syms)
    L = B.lib()
    for s in syms:
        assert hasattr(L, s), s


def test_workspace_bytes_real_shapes():
    n = B.latent_moe_workspace_bytes(real_cfg())
    # act FP16 [T*k, I], expert out FP16 [T*k, P], pooled FP32 [T, P], u and y FP16 [T, P] ...
    T, k, P, I = 16384, 8, 4096, 4096
    floor = T * k * I * 2 + T * k * P * 2 + T * P * (4 + 2 + 2)
    assert floor <= n <= floor * 1.2


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), B.LMOE_ERR_INVALID_ARG),
    (dict(intermediate=192), B.LMOE_ERR_INVALID_ARG),
    (dict(pooled=0), B.LMOE_ERR_INVALID_ARG),
    (dict(experts=0), B.LMOE_ERR_INVALID_ARG),
    (dict(experts=2000), B.LMOE_ERR_INVALID_ARG),
    (dict(top_k=0), B.LMOE_ERR_INVALID_ARG),
    (dict(top_k=33), B.LMOE_ERR_INVALID_ARG),
    (dict(experts=4, top_k=5), B.LMOE_ERR_INVALID_ARG),
    (dict(eps=float("nan")), B.LMOE_ERR_INVALID_ARG),
    (dict(eps=-1.0), B.LMOE_ERR_INVALID_ARG),
    (dict(max_tokens=0), B.LMOE_ERR_INVALID_ARG),
    (dict(act_dtype=7), B.LMOE_ERR_INVALID_ARG),
    (dict(act_dtype="f32", expert_dtype="bf16"), B.LMOE_ERR_UNSUPPORTED),
    (dict(act_dtype="f32", expert_dtype="mxfp4"), B.LMOE_ERR_UNSUPPORTED),
    (dict(intermediate=4096 + 256), B.LMOE_ERR_UNSUPPORTED),  # valid, BF16 built for multiples of 512
    (dict(expert_dtype="mxfp4", pooled=4096 + 256), B.LMOE_ERR_UNSUPPORTED),
    (dict(intermediate=4096 + 64), B.LMOE_ERR_INVALID_ARG),  # not a multiple of 128
    (dict(input_norm=2), B.LMOE_ERR_INVALID_ARG),
    (dict(expert_act=5), B.LMOE_ERR_INVALID_ARG),
    (dict(expert_act="mxfp8"), B.LMOE_ERR_UNSUPPORTED),  # BF16 experts
    (dict(expert_act="mxfp8", expert_dtype="mxfp4", act_dtype="f32"), B.LMOE_ERR_UNSUPPORTED),
    (dict(expert_act="mxfp4"), B.LMOE_ERR_UNSUPPORTED),  # BF16 experts
    (dict(expert_act="mxfp4", expert_dtype="mxfp4", act_dtype="f32"), B.LMOE_ERR_UNSUPPORTED),
])
def test_bad_configs_rejected(kw, code):
    with pytest.raises(B.LatentMoEError) as ei:
        B.latent_moe_workspace_bytes(real_cfg(**kw))
    assert ei.value.code == code
    assert B.latent_moe_last_error()


def test_create_rejects_null_and_misaligned_weights():
    L = B.lib()
    cfg = real_cfg()
    h = ctypes.c_void_p(123)
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), None, None) == B.LMOE_ERR_INVALID_ARG
    assert h.value is None  # *out cleared on failure
    w = B.Weights()
    for n in ("router", "pooler", "pool_gamma", "w_gate", "w_up", "w_down", "expert_gamma", "unpooler"):
        setattr(w, n, 4096)
    w.pooler = None
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "pooler" in B.latent_moe_last_error()
    w.pooler = 4096 + 8
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "aligned" in B.latent_moe_last_error()
    assert L.latent_moe_create(None, ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG


def test_top_k_up_to_32_accepted():
    for k in (16, 17, 32):
        assert B.latent_moe_workspace_bytes(real_cfg(top_k=k)) > 0


def test_mx_activations_accepted_with_mxfp4_experts():
    base = B.latent_moe_workspace_bytes(real_cfg(expert_dtype="mxfp4"))
    f8 = B.latent_moe_workspace_bytes(real_cfg(expert_dtype="mxfp4", expert_act="mxfp8"))
    T, P, I, k = 16384, 4096, 4096, 8
    # FP8 u codes and the E8M0 scales of u and act in place of the FP16 u
    assert f8 == base - T * P * 2 + T * P + T * P // 32 + T * k * I // 32
    f4 = B.latent_moe_workspace_bytes(real_cfg(expert_dtype="mxfp4", expert_act="mxfp4"))
    # FP4 u codes are half the size of FP8 ones
    assert f4 == base - T * P * 2 + T * P // 2 + T * P // 32 + T * k * I // 32


def test_input_norm_needs_gamma_and_sizes_workspace():
    base = B.latent_moe_workspace_bytes(real_cfg())
    withn = B.latent_moe_workspace_bytes(real_cfg(input_norm=1))
    T, H = 16384, 8192
    assert withn >= base + T * H * (4 + 2)  # FP32 norm output + its BF16 copy
    L = B.lib()
    cfg = real_cfg(input_norm=1)
    h = ctypes.c_void_p(0)
    w = B.Weights()
    for n in ("router", "pooler", "pool_gamma", "w_gate", "w_up", "w_down", "expert_gamma", "unpooler"):
        setattr(w, n, 4096)
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "input_gamma" in B.latent_moe_last_error()
    w.input_gamma = 4096 + 4
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "aligned" in B.latent_moe_last_error()


def test_mxfp4_accepted_and_scales_required():
    assert B.latent_moe_workspace_bytes(real_cfg(expert_dtype="mxfp4")) == \
        B.latent_moe_workspace_bytes(real_cfg())
    L = B.lib()
    cfg = real_cfg(expert_dtype="mxfp4")
    h = ctypes.c_void_p(0)
    w = B.Weights()
    for n in ("router", "pooler", "pool_gamma", "w_gate", "w_up", "w_down", "expert_gamma", "unpooler",
              "s_gate", "s_up"):
        setattr(w, n, 4096)
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "s_down" in B.latent_moe_last_error()
    w.s_down = 4096 + 4
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_INVALID_ARG
    assert "aligned" in B.latent_moe_last_error()


@pytest.mark.skipif(_has_device(), reason="checks the no-device error path")
def test_create_without_device_reports_hip_error():
    L = B.lib()
    cfg = real_cfg()
    w = B.Weights()
    for n in ("router", "pooler", "pool_gamma", "w_gate", "w_up", "w_down", "expert_gamma", "unpooler"):
        setattr(w, n, 4096)
    h = ctypes.c_void_p(0)
    assert L.latent_moe_create(ctypes.byref(h), ctypes.byref(cfg), ctypes.byref(w), None) == B.LMOE_ERR_HIP
    assert "device" in B.latent_moe_last_error()


def test_null_handle_calls():
    L = B.lib()
    assert L.latent_moe_forward(None, None, 1, None, None, None, None) == B.LMOE_ERR_INVALID_ARG
    assert L.latent_moe_destroy(None) == B.LMOE_ERR_INVALID_ARG
    v = B.Views()
    assert L.latent_moe_debug_views(None, ctypes.byref(v)) == B.LMOE_ERR_INVALID_ARG
    assert B.latent_moe_last_error()
