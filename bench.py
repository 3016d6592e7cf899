#!/usr/bin/env python3
"""Throughput of the latent-MoE layer forward on one MI355X.

One step = one forward of the whole layer (router, top-k, grouping, pooler,
pre-expert norm, gate/up, down, per-expert norm + weighted sum, unpooler) over
one batch of seeded synthetic tokens already resident in HBM. Default
workload: 64-token decode at the real layer shapes (H=8192, P=4096, E=256,
I=4096, k=8, BF16); the 16384-token prefill chunk on the same weights, the
skewed long prompt (five 16384-token chunks, Zipf router bias; one step runs
all five), and the 64-token decode and 16384-token prefill with MXFP4 expert
weights are measured in the same run and reported under their workload names.

Prints one JSON line with tokens/s, the roofline of the dominant kernel (the
gate/up grouped GEMM: HBM-bound at decode, MFMA-bound at prefill; its time
comes from HIP events recorded on the forward's stream) and the FP64 CPU
oracle timed on a bounded token sample on this host's cores (the first 48
decode tokens, and a seeded 2048-token subset of the prefill batch).

Timing: every timed step is preceded by writing a 1 GiB buffer and then
reading another 1 GiB buffer, which evicts the layer's weights and
activations from L2 and the 256 MB MALL, and is timed alone with HIP events;
`value` and `ms_per_step` come from the median of these cold steps (p10 and
p90 reported beside it). The read leaves the caches holding clean lines of
unrelated data: after the write alone, up to 256 MB of the buffer's dirty
lines are still in the MALL and their write-back to HBM lands inside the
timed step; the median of such steps is reported beside the cold one as
`cold_after_write_p50`. A warm-cache mean (steps back to back) is reported
separately and labelled as such. The tiny FP32 layer is reported in
microseconds per forward.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 (and FP16) matrix peak
# dense matrix peaks of the scaled (MX) instructions: an fp8 x fp4 product runs at the
# FP8 rate, fp4 x fp4 at the FP4 rate
MX_PEAK_TFLOPS = {"mxfp8": 5000.0, "mxfp4": 10100.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    """sha256 (first 16 hex digits) of the kernel sources and the C header."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "latent_moe_layer_fp32_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "*.hip"))
                   + [os.path.join(ROOT, "include", "latent_moe.h")])
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k] = v
    if kv.get("source_sha256") != source_hash():
        return None
    return int(float(kv["traffic_bytes"]))


def layer_bytes(spec, counts, T):
    """Algorithmic HBM bytes of one forward: touched expert weights once, the
    projections and router once, x in, out (FP32) out."""
    import numpy as np

    ew = 2 if spec.expert_format == "bf16" else (0.5 + 1 / 32)
    touched = int((np.asarray(counts) > 0).sum())
    experts = touched * 3 * spec.P * spec.I * ew
    proj = 2 * spec.H * spec.P * 2 + spec.E * spec.H * 4
    return experts + proj + T * spec.H * 2 + T * spec.H * 4, touched


def gate_up_bytes(spec, counts, T):
    import numpy as np

    ew = 2 if spec.expert_format == "bf16" else (0.5 + 1 / 32)
    touched = int((np.asarray(counts) > 0).sum())
    pairs = T * spec.k
    return touched * 2 * spec.I * spec.P * ew + pairs * spec.P * 2 + pairs * spec.I * 2


def layer_flops(spec, T):
    k, H, P, I = spec.k, spec.H, spec.P, spec.I
    return T * (2 * H * P * 2 + k * 2 * P * 2 * I + k * 2 * I * P)


FLUSH_BYTES = 1 << 30  # evicting buffers: larger than L2 (8 x 4 MB) plus the 256 MB MALL


def measure(spec, layer, xs, steps, warmup, torch):
    """One step = one forward per chunk in xs (a single batch, or the chunks
    of a long prompt in order). Cold steps: before each, a 1 GiB buffer is
    written and another 1 GiB buffer read (evicting the layer's weights and
    activations from L2 and the MALL, and leaving no dirty line of the write
    behind) and the step is timed alone with HIP events on the forward's
    stream. The same steps after the write alone are timed too: then the
    write-back of the MALL's dirty lines falls inside the step. Warm steps:
    back to back, caches as the previous step left them. Returns the per-step
    cold times (ms), the per-step times after the write alone (ms), the warm
    mean (ms), the wall time of the cold loop, per-stage ms (summed over the
    chunks of a step) and the last chunk's expert counts."""
    from latent_moe_layer_fp32_amd import binding as B

    stream = torch.cuda.current_stream()
    T = xs[0].shape[0]
    out = torch.empty((T, spec.H), dtype=torch.float32, device=xs[0].device)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=xs[0].device)
    clean = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=xs[0].device)  # only ever read

    def step():
        for x in xs:
            layer.forward(x, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        scratch.fill_(1.0)  # a fill kernel on the same stream, outside the timed events
        clean.sum()  # a reduction reading 1 GiB: the MALL's dirty lines are written back here
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cold = [a.elapsed_time(b) for a, b in evs]
    for a, b in evs:
        scratch.fill_(1.0)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    dirty = [a.elapsed_time(b) for a, b in evs]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    warm = start.elapsed_time(end) / steps
    del scratch, clean
    # per-stage HIP events on the same stream, over the same number of (warm) steps
    B.latent_moe_set_profiling(layer.handle, True)
    acc = None
    for _ in range(steps):
        for x in xs:
            layer.forward(x, out=out)
            st = B.latent_moe_stage_times(layer.handle)
            acc = st if acc is None else {k: acc[k] + v for k, v in st.items()}
    B.latent_moe_set_profiling(layer.handle, False)
    stages = {k: v / steps for k, v in acc.items()}
    return cold, dirty, warm, wall, stages, layer.views(T, names=("counts",))["counts"]


def host_info() -> dict:
    """CPU model and the BLAS numpy calls (for the CPU baseline's record)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        libs = [f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)"
                for d in threadpool_info() if d.get("user_api") == "blas"]
        blas = "; ".join(libs) or blas
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_baseline(spec, xs, experts=None):
    """The FP64 oracle on tokens xs of the workload (a bounded sample). Expert
    weights are fetched by `experts` (e -> host arrays as stored) or generated
    on the host; only the oracle's own work is timed (its conversions of the
    stored weights included), not the fetch."""
    import numpy as np

    from oracle import oracle as orc
    from oracle.mx import to_f64
    import synth

    host = {n: synth.host(spec, n) for n in ("router", "router_bias", "pooler", "pool_gamma",
                                            "expert_gamma", "unpooler")}
    gin = synth.host(spec, "input_gamma") if spec.input_norm else None
    fetch_s = [0.0]

    def first(a):
        return (a[0][0], a[1][0]) if isinstance(a, tuple) else a[0]

    def expert(e):
        t = time.perf_counter()
        raw = (experts(e) if experts is not None else
               tuple(first(synth.host(spec, n, experts=(e, e + 1))) for n in ("w_gate", "w_up", "w_down")))
        fetch_s[0] += time.perf_counter() - t
        return tuple(to_f64(a) for a in raw)

    t0 = time.perf_counter()
    r = orc.forward(xs, host["router"], host["router_bias"], host["pooler"], host["pool_gamma"], expert,
                    host["expert_gamma"], host["unpooler"], spec.k, spec.eps, keep_pairs=False, input_gamma=gin,
                    act_quant=spec.expert_act)
    dt = time.perf_counter() - t0 - fetch_s[0]
    return len(xs) / dt, dt, len(np.unique(r.ids))


def pct(v, q):
    import numpy as np

    return float(np.percentile(np.asarray(v), q))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed steps of the main workload (default: 100, the 64-token decode)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "mxfp4", "mxfp4_decode", "mxfp8", "mxfp8_decode",
                             "mxfp4act", "mxfp4act_decode", "decode_norm", "prefill_norm"])
    # skew: five 16384-token chunks of one long prompt (81920 tokens per step)
    ap.add_argument("--also", default="tiny,prefill,skew,decode_norm,prefill_norm,mxfp4_decode,mxfp4,mxfp8_decode,"
                                      "mxfp8,mxfp4act_decode,mxfp4act",
                    help="extra workloads measured in the same run (comma list)")
    ap.add_argument("--cpu-tokens", type=int, default=48,
                    help="token sample for the CPU oracle on the main workload (0: skip all CPU baselines)")
    ap.add_argument("--cpu-prefill-tokens", type=int, default=2048,
                    help="seeded token subset for the CPU oracle on the 16384-token prefill (0: skip)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time torch's BF16 batched GEMM (hipBLASLt) on the gate/up shape, for reference")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run a plain device copy of this many bytes (calibrates profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs unsharded on a single MI355X "
              "(sharding across GPUs is designed, not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from latent_moe_layer_fp32_amd import LatentMoE

    def make_layer(spec, w, max_tokens):
        return LatentMoE(hidden=spec.H, pooled=spec.P, experts=spec.E, intermediate=spec.I,
                         top_k=spec.k, eps=spec.eps, act_dtype=spec.act_dtype,
                         expert_dtype=spec.expert_format, max_tokens=max_tokens, weights=w,
                         input_norm=spec.input_norm, expert_act=spec.expert_act)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tables = synth.DeviceTables("cuda:0")
    wcache = {}

    def weights_for(spec):
        """Weights of the real layer shapes in the spec's expert format (one
        format resident at a time)."""
        fmt = spec.expert_format
        if fmt not in wcache:
            wcache.clear()
            torch.cuda.empty_cache()
            base = synth.CONFIGS["prefill"].with_(expert_format=fmt)
            log(f"generating {fmt} weights on the device")
            wcache[fmt] = {n: synth.device_tensor(base, n, tables) for n in synth.WEIGHT_NAMES}
            torch.cuda.synchronize()
        return wcache[fmt]

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_bytes} bytes")
        del src, dst

    def expert_fetch(w):
        """Expert e of the device weights as host arrays, as stored (BF16 bits,
        or MXFP4 codes and scales); the device copies equal the host
        generator's output bit for bit."""
        def fetch(e):
            out = []
            for n in ("w_gate", "w_up", "w_down"):
                t = w[n]
                if isinstance(t, tuple):
                    out.append((t[0][e].cpu().numpy(), t[1][e].cpu().numpy()))
                elif t.dtype == torch.bfloat16:
                    out.append(t[e].view(torch.int16).cpu().numpy().view(np.uint16))
                else:
                    out.append(t[e].cpu().numpy())
            return tuple(out)
        return fetch

    hinfo = host_info()
    cores = len(os.sched_getaffinity(0))
    results = {}
    for wl in [args.workload] + [w for w in args.also.split(",") if w and w != args.workload]:
        spec = synth.CONFIGS[wl]
        if spec.act_dtype == "f32":  # the tiny all-FP32 layer: its own weights
            w = {n: synth.device_tensor(spec, n, tables) for n in synth.WEIGHT_NAMES}
        else:
            w = dict(weights_for(spec))
        if spec.input_norm:
            w["input_gamma"] = synth.device_tensor(spec, "input_gamma", tables)
        if spec.router_bias != "none":
            w["router_bias"] = synth.device_tensor(spec, "router_bias", tables)
        layer = make_layer(spec, w, max_tokens=spec.T)
        xs = [synth.device_tensor(spec, "x", tables, chunk=c) for c in range(spec.chunks)]
        prefill_sized = spec.T * spec.k >= 64 * spec.E
        if wl == args.workload:
            steps, warm = args.steps, args.warmup
        elif args.steps < 20:  # a short run (profiling): as many steps as the main workload
            steps = min(5, args.steps) if spec.chunks > 1 else args.steps
            warm = max(2, args.warmup // 2)
        else:  # 100 timed steps at decode sizes, 20 at prefill sizes, 5 of the five-chunk prompt
            steps = 5 if spec.chunks > 1 else (20 if prefill_sized else max(100, args.steps))
            warm = max(2, args.warmup // 2)
        log(f"{wl}: T={spec.T} x {spec.chunks} chunk(s), {warm} warmup + {steps} timed steps")
        cold, dirty, warm_ms, wall, stages, counts = measure(spec, layer, xs, steps, warm, torch)
        ms = pct(cold, 50)
        lb, touched = layer_bytes(spec, counts, spec.T)
        r = dict(spec=spec, ms=ms, wall=wall, stages=stages, touched=touched, layer_bytes=lb,
                 tokens_per_s=spec.T * spec.chunks / (ms / 1e3), steps=steps, warmup=warm,
                 cold={"p10": round(pct(cold, 10), 4), "p50": round(ms, 4), "p90": round(pct(cold, 90), 4)},
                 cold_after_write_p50=round(pct(dirty, 50), 4), warm_ms=round(warm_ms, 4))
        gu = stages["gate_up"] / 1e3
        if spec.act_dtype == "f32":
            r["roofline"] = None  # launch-latency bound (21 MFLOP): reported in microseconds
            r["us_per_forward"] = {"cold_p50": round(ms * 1e3, 1), "warm": round(warm_ms * 1e3, 1)}
            r["layer_frac"] = None
        elif not prefill_sized:  # decode-sized: the expert weights stream once
            ach = gate_up_bytes(spec, counts, spec.T) / gu / 1e9
            r["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic(wl, "gate_up"),
                             "kernel": "gate_up grouped GEMM + SwiGLU",
                             "kernel_ms": round(stages["gate_up"], 4)}
            r["layer_frac"] = round(lb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            fl = 2 * spec.T * spec.chunks * spec.k * spec.P * 2 * spec.I
            ach = fl / gu / 1e12
            peak = MX_PEAK_TFLOPS.get(spec.expert_act, BF16_PEAK_TFLOPS)
            r["roofline"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                             "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                             "peak_dtype": spec.expert_act or "f16",
                             "traffic": measured_traffic(wl, "gate_up"),
                             "kernel": "gate_up grouped GEMM + SwiGLU",
                             "kernel_ms": round(stages["gate_up"], 4)}
            r["layer_frac"] = round(layer_flops(spec, spec.T * spec.chunks) / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        log(f"{wl}: cold {ms:.3f} ms/step (p10 {r['cold']['p10']:.3f}, p90 {r['cold']['p90']:.3f}), "
            f"after write alone {r['cold_after_write_p50']:.3f}, "
            f"warm {warm_ms:.3f}, {r['tokens_per_s']:.0f} tok/s, stages "
            + ", ".join(f"{k} {v:.3f}" for k, v in stages.items()))
        cpu_n = 0
        if args.cpu_tokens > 0 and wl == args.workload:
            cpu_n, sample_desc = args.cpu_tokens, f"first {args.cpu_tokens} tokens of the {wl} batch"
            idx = np.arange(cpu_n)
        elif args.cpu_tokens > 0 and wl == "prefill" and args.cpu_prefill_tokens > 0:
            cpu_n = args.cpu_prefill_tokens
            idx = np.sort(np.random.default_rng(0).choice(spec.T, cpu_n, replace=False))
            sample_desc = f"seeded subset of {cpu_n} of the {spec.T} prefill tokens (exact: the layer is token-local)"
        if cpu_n:
            log(f"{wl}: cpu oracle on {cpu_n} tokens")
            xh = synth.host(spec, "x")[idx]
            v, dt, ne = cpu_baseline(spec, xh, expert_fetch(w) if spec.act_dtype != "f32" else None)
            r["cpu_baseline"] = {"value": round(v, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                                 "sample": f"{sample_desc} ({ne} experts), FP64 numpy, {dt:.1f} s",
                                 **hinfo}
        results[wl] = r
        layer.close()
        del xs

    main_r = results[args.workload]
    spec = main_r["spec"]
    line = {
        "metric": "latent-MoE layer tokens/s (16K prefill, 64-tok decode); % of MFMA/HBM peak",
        "value": round(main_r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": main_r["steps"],
        "warmup": main_r["warmup"],
        "ms_per_step": round(main_r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f16",
        "data": "synthetic (seeded counter-based N(0,1) inputs, N(0,1/fan_in) weights)",
        "config": {"workload": f"{args.workload}: " + (f"{spec.chunks} x " if spec.chunks > 1 else "") + f"{spec.T} tokens, H={spec.H}, P={spec.P}, E={spec.E}, "
                               f"I={spec.I}, top-{spec.k}, {spec.expert_format.upper()} experts"
                               + (f", {spec.expert_act.upper()} expert inputs" if spec.expert_act else "")
                               + ", FP32 router",
                   "global_batch": spec.T * spec.chunks, "parallelism": "none (one GPU)"},
        "roofline": main_r["roofline"],
        "layer_frac": main_r["layer_frac"],
        "timing": {"value_from": "median of cold steps (before each, 1 GiB written, then another 1 GiB "
                                 "read; HIP events per step)",
                   "cold_ms": main_r["cold"], "cold_after_write_p50": main_r["cold_after_write_p50"],
                   "warm_ms": main_r["warm_ms"],
                   "warm_tokens_per_s": round(spec.T * spec.chunks / (main_r["warm_ms"] / 1e3), 1)},
        "stages_ms": {k: round(v, 4) for k, v in main_r["stages"].items()},
        "experts_touched": main_r["touched"],
    }
    for wl, r in results.items():
        if wl == args.workload:
            continue
        sub = {"value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "ms_per_step": round(r["ms"], 4),
               "tokens_per_step": r["spec"].T * r["spec"].chunks, "steps": r["steps"],
               "cold_ms": r["cold"], "cold_after_write_p50": r["cold_after_write_p50"],
               "warm_ms": r["warm_ms"], "roofline": r["roofline"],
               "layer_frac": r["layer_frac"], "stages_ms": {k: round(v, 4) for k, v in r["stages"].items()}}
        for key in ("us_per_forward", "cpu_baseline"):
            if key in r:
                sub[key] = r[key]
        line[wl] = sub
    if args.vendor_gemm:
        # 256 experts x 512 rows (uniform routing), K = P, N = 2I; contiguous operands, no gather
        E_, M_, K_, N_ = 256, 512, 4096, 8192
        a = torch.randn(E_, M_, K_, device="cuda:0", dtype=torch.bfloat16)
        b = torch.randn(E_, K_, N_, device="cuda:0", dtype=torch.bfloat16)
        torch.bmm(a, b)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(10):
            torch.bmm(a, b)
        ev1.record()
        torch.cuda.synchronize()
        vms = ev0.elapsed_time(ev1) / 10
        line["vendor_bf16_gemm"] = {"shape": f"bmm {E_} x [{M_} x {K_}] x [{K_} x {N_}]", "ms": round(vms, 4),
                                    "TFLOP/s": round(2 * E_ * M_ * K_ * N_ / vms / 1e9, 1)}
        del a, b
    if "cpu_baseline" in main_r:
        line["cpu_baseline"] = main_r["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
