"""The no-allocation forward (latent_moe_forward_static, through the C ABI)
against the handle's forward on the same tiny FP32 layer: bitwise equal
outputs, ids and weights on two calls in a row, the second with fewer tokens
(the static workspace keeps the first call's contents), plus its errors."""
import ctypes

import numpy as np
import pytest

import synth
from layer_cases import device_weights, make_layer

pytestmark = pytest.mark.gpu


def test_static_forward_matches_handle_forward():
    import torch

    from latent_moe_layer_fp32_amd import binding as B

    assert torch.cuda.is_available(), "GPU tests need a device"
    tables = synth.DeviceTables("cuda:0")
    spec = synth.CONFIGS["tiny"]
    wts = device_weights(spec, tables)
    x = synth.device_tensor(spec, "x", tables)
    layer = make_layer(spec, wts, max_tokens=spec.T)
    cfg = B.make_config(spec.H, spec.P, spec.E, spec.I, spec.k, spec.eps, "f32", "f32", 1)
    w = B.Weights()
    for n in ("router", "pooler", "pool_gamma", "w_gate", "w_up", "w_down", "expert_gamma", "unpooler"):
        setattr(w, n, wts[n].data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    try:
        for T in (spec.T, 37):
            xt = x[:T].contiguous()
            ref_ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda:0")
            ref_w = torch.empty((T, spec.k), dtype=torch.float32, device="cuda:0")
            ref = layer.forward(xt, topk_ids=ref_ids, topk_weights=ref_w)
            out = torch.full((T, spec.H), float("nan"), device="cuda:0")
            ids = torch.full((T, spec.k), -1, dtype=torch.int32, device="cuda:0")
            wt = torch.full((T, spec.k), float("nan"), device="cuda:0")
            B.latent_moe_forward_static(cfg, w, xt.data_ptr(), T, out.data_ptr(), ids.data_ptr(), wt.data_ptr(),
                                        stream)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref.cpu().numpy()), f"T={T}: outputs differ"
            assert np.array_equal(ids.cpu().numpy(), ref_ids.cpu().numpy()), f"T={T}: ids differ"
            assert np.array_equal(wt.cpu().numpy(), ref_w.cpu().numpy()), f"T={T}: weights differ"
        # errors: beyond the static workspace, BF16 layers, bad arguments
        L = B.lib()
        big = B.make_config(spec.H, spec.P, spec.E, spec.I, spec.k, spec.eps, "f32", "f32", 1)
        rc = L.latent_moe_forward_static(ctypes.byref(big), ctypes.byref(w), x.data_ptr(), 1 << 20,
                                         out.data_ptr(), None, None, stream)
        assert rc == B.LMOE_ERR_TOO_MANY_TOKENS and "static scratch" in B.latent_moe_last_error()
        bf = B.make_config(1024, 512, 16, 512, 4, 1e-6, "bf16", "bf16", 1)
        rc = L.latent_moe_forward_static(ctypes.byref(bf), ctypes.byref(w), x.data_ptr(), 4, out.data_ptr(),
                                         None, None, stream)
        assert rc == B.LMOE_ERR_UNSUPPORTED
        rc = L.latent_moe_forward_static(ctypes.byref(cfg), None, x.data_ptr(), 4, out.data_ptr(), None, None, stream)
        assert rc == B.LMOE_ERR_INVALID_ARG
        assert L.latent_moe_forward_static(ctypes.byref(cfg), ctypes.byref(w), x.data_ptr(), 0, None, None, None,
                                           stream) == B.LMOE_OK
    finally:
        layer.close()
