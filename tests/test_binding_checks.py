"""Argument checks of the Python binding (CPU tensors stand in for device
ones: the checks compare shapes, dtypes and devices before any library call)."""
import pytest
import torch

from latent_moe_layer_fp32_amd import binding as B

CPU = torch.device("cpu")
DIMS = dict(hidden=256, pooled=128, experts=8, intermediate=128)


def weights(act="f32", exp="f32", **over):
    H, P, E, I = 256, 128, 8, 128
    adt = torch.float32 if act == "f32" else torch.bfloat16
    edt = torch.float32 if exp == "f32" else torch.bfloat16

    def ex(n, k):
        if exp == "mxfp4":
            return (torch.zeros(E, n, k // 2, dtype=torch.uint8), torch.zeros(E, n, k // 32, dtype=torch.uint8))
        return torch.zeros(E, n, k, dtype=edt)

    w = dict(router=torch.zeros(E, H), router_bias=None, pooler=torch.zeros(P, H, dtype=adt),
             pool_gamma=torch.ones(P), w_gate=ex(I, P), w_up=ex(I, P), w_down=ex(P, I),
             expert_gamma=torch.ones(E, P), unpooler=torch.zeros(H, P, dtype=adt))
    w.update(over)
    return w


def check(w, act="f32", exp="f32", **kw):
    specs = B.weight_specs(act_dtype=act, expert_dtype=exp, router_bias=w.get("router_bias") is not None,
                           **DIMS, **kw)
    B.validate_weights(w, specs, CPU)


@pytest.mark.parametrize("act,exp", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "mxfp4")])
def test_good_weights_pass(act, exp):
    check(weights(act, exp), act, exp)
    check(weights(act, exp, router_bias=torch.zeros(8)), act, exp)
    check(weights(act, exp, input_gamma=torch.ones(256)), act, exp, input_norm=True)


@pytest.mark.parametrize("name,bad,msg", [
    ("router", torch.zeros(8, 255), "shape"),
    ("router", torch.zeros(8, 256, dtype=torch.bfloat16), "dtype"),  # the router stays FP32
    ("pooler", torch.zeros(128, 256, dtype=torch.bfloat16), "dtype"),  # FP32 layer
    ("w_down", torch.zeros(8, 128, 129), "shape"),
    ("expert_gamma", torch.ones(128), "shape"),
    ("unpooler", torch.zeros(128, 256), "shape"),  # transposed
    ("router_bias", torch.zeros(9), "shape"),
    ("w_gate", torch.zeros(8, 128, 128).transpose(1, 2), "contiguous"),
])
def test_bad_weight_rejected(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        check(weights(**{name: bad}))


def test_missing_extra_and_mx_pairs():
    w = weights()
    del w["pool_gamma"]
    with pytest.raises(ValueError, match="pool_gamma"):
        check(w)
    with pytest.raises(ValueError, match="unexpected"):
        check(weights(w_gates=torch.ones(256)))  # not a weight of the layer
    check(weights(input_gamma=torch.ones(256)))  # ignored without input_norm, as by the C ABI
    w = weights("bf16", "mxfp4")
    w["w_up"] = w["w_up"][0]
    with pytest.raises(ValueError, match="pair"):
        check(w, "bf16", "mxfp4")
    w = weights("bf16", "mxfp4")
    w["w_up"] = (w["w_up"][0], torch.zeros(8, 128, 5, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales"):
        check(w, "bf16", "mxfp4")


def test_device_mismatch_rejected():
    w = weights()
    specs = B.weight_specs(act_dtype="f32", expert_dtype="f32", **DIMS)
    with pytest.raises(ValueError, match="expected cuda"):
        B.validate_weights(w, specs, torch.device("cuda", 0))


def test_forward_arguments():
    T = 5
    x = torch.zeros(T, 256)
    B.validate_forward(x, torch.zeros(T, 256), torch.zeros(T, 2, dtype=torch.int32), torch.zeros(T, 2),
                       256, 2, "f32", CPU)
    bad = [
        (torch.zeros(T, 256, dtype=torch.bfloat16), None, None, None, "dtype"),  # FP32 layer, BF16 x
        (torch.zeros(T, 255), None, None, None, "x must be"),
        (x, torch.zeros(T, 256, dtype=torch.bfloat16), None, None, "out"),
        (x, torch.zeros(T - 1, 256), None, None, "out"),
        (x, None, torch.zeros(T, 2, dtype=torch.int64), None, "topk_ids"),
        (x, None, torch.zeros(T, 3, dtype=torch.int32), None, "topk_ids"),
        (x, None, None, torch.zeros(T, 2, dtype=torch.float64), "topk_weights"),
        (torch.zeros(256, T).t(), None, None, None, "contiguous"),
    ]
    for xx, out, ids, wts, msg in bad:
        with pytest.raises(ValueError, match=msg):
            B.validate_forward(xx, out, ids, wts, 256, 2, "f32", CPU)
    with pytest.raises(ValueError, match="dtype"):  # BF16 layer, FP32 x
        B.validate_forward(x, None, None, None, 256, 2, "bf16", CPU)
