"""Benchmark of one sparse MoE FFN layer forward on one MI355X.

Default workload: the Mixtral-8x7B-shaped layer (H=4096, F=14336, E=8, k=2,
bf16 weights and activations, fp32 accumulation) on a prefill batch of
T=4096 tokens; one step = one full layer forward (router, top-k + softmax,
dispatch, gate/up + SiLU, down, combine) over the batch, inputs resident in
HBM.  Then decode batches T = 1, 4, 16, 64 on the same layer shape (HIP-graph
replays over four copies of the weights) and the 32-layer stacked decode, each
with bf16 experts and again with uint8 experts (one affine map per matrix,
quantised on the device from the same bf16 weights).

Prints ONE JSON line.  `roofline` describes the dominant kernel (the
gate/up launch of the step: the grouped GEMM for the Mixtral-shaped prefill
and the 128-expert workload, the weight-streaming kernel for the 64-expert
one), timed with HIP events recorded by the library on the launch stream
around that kernel in every timed step; its bound is MFMA above the ridge
(312.5 flop/B) and HBM below, from the launch's algorithmic flops and bytes.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of tokens of the
same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (decode T=1..64, prefill T=4096); % HBM / bf16-MFMA peak"
PROFILE = os.path.join(ROOT, "profiles", "grouped_gemm_mixtral_prefill_T4096.md")
LAYERS_PROFILE = os.path.join(ROOT, "profiles", "layers_qwen_deepseek_shapes.md")
CSRC = os.path.join(ROOT, "mixture_experts_amd", "csrc")


def measured_traffic(profile=PROFILE, key="traffic_bytes_per_launch",
                     src="expert_grouped.hip"):
    """HBM bytes per launch of the kernel a committed rocprofv3 counter summary
    covers (`key`), or None when that kernel's source (`src`) changed since the
    counters were taken."""
    import hashlib
    try:
        text = open(profile).read()
        digest = hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith(("source_sha256", "traffic_bytes_per_launch")) and ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get(f"source_sha256 {src}", fields.get("source_sha256")) != digest:
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill",
                    choices=["mixtral_prefill", "qwen", "deepseek"])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 32-layer stacked decode (90 GB of experts)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 64-expert and 128-expert layers")
    ap.add_argument("--decode-batches", default="1,4,16,64",
                    help="decode / stacked-decode batch sizes to run (comma-separated, "
                         "from 1,4,16,64; a subset isolates one batch size in a kernel trace)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (reference "
                         "for the HBM traffic counters)")
    return ap.parse_args()


def expert_blob(shape, n_blocks, u8, layer_of=lambda b: 0):
    """Device buffer of n_blocks layers' experts (block b generated as layer
    layer_of(b)); with u8, quantised on the device from the bf16 weights.
    Returns (buffer, bytes per expert)."""
    import torch

    import gen
    import mixture_experts_amd as moe
    st = torch.cuda.current_stream()
    if not u8:
        blob = torch.empty(n_blocks * shape.E * shape.stride, dtype=torch.uint8, device="cuda")
        for b in range(n_blocks):
            gen.experts_device(shape, blob.data_ptr() + b * shape.E * shape.stride,
                               layer=layer_of(b), stream=st.cuda_stream)
        return blob, shape.stride
    ust = moe.u8_stride(shape.H, shape.F)
    blob = torch.empty(n_blocks * shape.E * ust, dtype=torch.uint8, device="cuda")
    tmp = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
    for b in range(n_blocks):
        gen.experts_device(shape, tmp.data_ptr(), layer=layer_of(b), stream=st.cuda_stream)
        moe.moe_quantize_experts_u8(tmp, shape.stride, shape.E, shape.H, shape.F,
                                    blob.data_ptr() + b * shape.E * ust, ust, st)
    torch.cuda.synchronize()
    del tmp
    return blob, ust


def stage_times(layer, x, y, T, steps, warm):
    """Per-stage device times (ms) of eager forwards, from the library's events."""
    import torch

    import mixture_experts_amd as moe
    st = torch.cuda.current_stream()
    nst = moe.MOE_NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record(st)
    for _ in range(warm):
        moe.moe_forward(layer.handle, x, T, y, st)
    for i in range(steps):
        moe.moe_forward_ev(layer.handle, x, T, y, st, [e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    return [sum(evs[i][s].elapsed_time(evs[i][s + 1]) for i in range(steps)) / steps
            for s in range(nst)]


def routing_stats(shape, x_h, wr_h, b_h, counts):
    """Per-config routing report: the experts' token loads (from the GPU's own
    dispatch) and the near ties, tokens whose k-th and (k+1)-th largest logit
    differ by less than 1e-3 (logits in float64 from the stored bf16 values;
    a statistic of the inputs, not a step of the path)."""
    import numpy as np

    import gen
    c = np.asarray(counts, dtype=np.int64)
    out = {"experts_touched": int((c > 0).sum()), "load_min": int(c.min()),
           "load_median": float(np.median(c)), "load_max": int(c.max())}
    if shape.k < shape.E:
        xs = gen.bf16_bits_to_f32(x_h).astype(np.float64)
        ws = gen.bf16_bits_to_f32(wr_h).astype(np.float64)
        lg = xs @ ws
        if b_h is not None:
            lg += b_h.astype(np.float64)[None, :]
        srt = -np.sort(-lg, axis=1)
        out["near_ties"] = int((srt[:, shape.k - 1] - srt[:, shape.k] < 1e-3).sum())
    return out


def time_layer(layer, x, y, T, steps, warm, stream):
    """Wall time of `steps` forwards (after `warm`), and the mean per-stage and
    whole-step device times (ms) from the library's per-stage HIP events."""
    import torch

    import mixture_experts_amd as moe
    nst = moe.MOE_NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    for row in evs:  # materialise the event handles
        for e in row:
            e.record(stream)
    for _ in range(warm):
        moe.moe_forward(layer.handle, x, T, y, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_forward_ev(layer.handle, x, T, y, stream, [e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = [sum(evs[i][s].elapsed_time(evs[i][s + 1]) for i in range(steps)) / steps
                for s in range(nst)]
    per_step = [evs[i][0].elapsed_time(evs[i][nst]) for i in range(steps)]
    return wall, stage_ms, sum(per_step) / steps, per_step


def percentiles(ms):
    """p10 / p50 / p90 of per-step times (ms)."""
    import numpy as np
    return [round(float(np.percentile(np.asarray(ms), q)), 4) for q in (10, 50, 90)]


def replay_times(g, K, stream, scale=1.0):
    """Device times (ms, times `scale`) of K single replays of graph g, each
    bracketed by HIP events on the launch stream (a pass of its own, after the
    timed one)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evs[0].record(stream)
    for i in range(K):
        g.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) * scale for i in range(K)]


def graph_step(layer, x, y, T, K, W, stream):
    """One forward captured in a HIP graph (after one eager call on the
    capture stream) and replayed W times untimed, then K times between two
    HIP events: mean device ms per replay, and p10/p50/p90 of single replays.
    The replay has no host launch gaps between the layer's kernels."""
    import torch

    import mixture_experts_amd as moe
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        moe.moe_forward(layer.handle, x, T, y, side)
    stream.wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(layer.handle, x, T, y, torch.cuda.current_stream())
    for _ in range(W):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / K
    pct = percentiles(replay_times(g, K, stream))
    del g
    return mean, pct


def gate_up_roofline(shape, T, touched, t_gu_s):
    """Roofline of the gate/up launch: algorithmic flops 4*T*k*H*F and bytes
    (touched experts' gate and up weights once, token rows in, activation
    out); bound MFMA above the ridge (2.5 PF / 8 TB/s = 312.5 flop/B), else
    HBM; the other fraction is reported beside it."""
    S = T * shape.k
    flops = 4.0 * S * shape.H * shape.F
    byts = touched * 2.0 * shape.H * shape.F * 2 + T * shape.H * 2.0 + S * shape.F * 2.0
    tf = flops / t_gu_s / 1e12
    gbs = byts / t_gu_s / 1e9
    if flops / byts >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_workload(name, shape, T, K, W):
    """One layer of another shape (the 64-expert and the Zipf-skewed
    128-expert layers): tokens/s, stage times, the gate/up roofline and the
    layer's fractions of both peaks over its algorithmic work."""
    import numpy as np
    import torch

    import gen
    import mixture_experts_amd as moe
    st = torch.cuda.current_stream()
    x_h, wr_h, b_h = gen.gen_x(shape, T), gen.gen_router(shape), gen.gen_bias(shape)
    x = torch.from_numpy(x_h.view(np.int16)).cuda()
    wr = torch.from_numpy(wr_h.view(np.int16)).cuda()
    bias = None if b_h is None else torch.from_numpy(b_h).cuda()
    ex = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
    gen.experts_device(shape, ex.data_ptr(), stream=st.cuda_stream)
    layer = moe.MoELayer(shape.H, shape.F, shape.E, shape.k, T, moe.MOE_BF16, wr, ex,
                         shape.stride, bias)
    y = torch.empty((T, shape.H), dtype=torch.float32, device="cuda")
    wall, stage_ms, dev_ms, per_step = time_layer(layer, x, y, T, K, W, st)
    r = layer.route(x, T)
    torch.cuda.synchronize()
    counts = r["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    S = T * shape.k
    streaming = S <= 32 * shape.E  # the library's path choice
    src = "expert_stream.hip" if streaming else "expert_grouped.hip"
    flops = 6.0 * S * shape.H * shape.F + 2.0 * T * shape.H * shape.E
    byts = touched * 3.0 * shape.H * shape.F * 2 + shape.H * shape.E * 2.0 + T * shape.H * (2 + 4)
    dev_s = dev_ms * 1e-3
    res = {"tokens": T, "hidden": shape.H, "ffn": shape.F, "experts": shape.E,
           "top_k": shape.k, "router_bias": shape.bias,
           "tokens_per_s": round(T * K / wall, 1), "ms_per_step": round(wall / K * 1e3, 4),
           "step_device_ms": round(dev_ms, 4),
           "step_device_ms_p10_p50_p90": percentiles(per_step),
           "stages_ms": {n: round(v, 4) for n, v in zip(moe.STAGE_NAMES, stage_ms)},
           "roofline": dict(gate_up_roofline(shape, T, touched,
                                             stage_ms[moe.MOE_STAGE_GATE_UP] * 1e-3),
                            kernel=("streaming" if streaming else "grouped GEMM")
                            + " gate/up + SiLU",
                            traffic=measured_traffic(LAYERS_PROFILE,
                                                     "traffic_bytes_per_launch_" + name, src)),
           "layer_hbm_frac": round(byts / dev_s / 1e9 / PEAK_HBM_GBS, 4),
           "layer_mfma_frac": round(flops / dev_s / 1e12 / PEAK_BF16_TFLOPS, 4),
           "routing": routing_stats(shape, x_h, wr_h, b_h, counts)}
    g_ms, g_pct = graph_step(layer, x, y, T, K, W, st)
    g_s = g_ms * 1e-3
    res["graph_replay"] = {"device_ms": round(g_ms, 4), "device_ms_p10_p50_p90": g_pct,
                           "tokens_per_s": round(T / g_s, 1),
                           "layer_hbm_frac": round(byts / g_s / 1e9 / PEAK_HBM_GBS, 4),
                           "layer_mfma_frac": round(flops / g_s / 1e12 / PEAK_BF16_TFLOPS, 4)}
    layer.close()
    del ex
    torch.cuda.empty_cache()
    return res


DECODE_BATCHES = (1, 4, 16, 64)


def bench_decode(shape, x, y, K, W, u8=False, batches=DECODE_BATCHES):
    """The Mixtral-shaped layer on decode batches T = 1, 4, 16, 64.  Four
    copies of the layer's experts (4 x 2.8 GB bf16 or 4 x 1.4 GB uint8, far
    beyond the 256 MB of Infinity Cache) are visited in turn, one HIP-graph
    replay = one forward of each copy, so no repeat is served from a cache;
    the step time is the replay time / 4.  Stage times come from a separate
    eager pass with the library's per-stage events (they include the event
    overhead)."""
    import numpy as np
    import torch

    import gen
    import mixture_experts_amd as moe
    NCOPY = 4
    st = torch.cuda.current_stream()
    blob, stride = expert_blob(shape, NCOPY, u8)
    wr = torch.from_numpy(gen.gen_router(shape).view(np.int16)).cuda()
    fmt = moe.MOE_EXPERT_U8 if u8 else moe.MOE_EXPERT_DTYPE
    layers = [moe.MoELayer(shape.H, shape.F, shape.E, shape.k, 64, moe.MOE_BF16, wr,
                           blob.data_ptr() + c * shape.E * stride, stride, expert_format=fmt)
              for c in range(NCOPY)]
    torch.cuda.synchronize()
    wbytes = 1 if u8 else 2  # per weight
    eb = 3 * shape.H * shape.F * wbytes + (64 if u8 else 0)
    res = {"weight_copies": NCOPY, "expert_weights": "uint8 (affine per matrix)" if u8 else "bf16"}
    for Td in batches:
        xd, yd = x[:Td], y[:Td]
        r = layers[0].route(xd, Td)
        torch.cuda.synchronize()
        touched = int((r["counts"] > 0).sum().item())
        st_d = stage_times(layers[0], xd, yd, Td, 20, W)
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            for L in layers:
                moe.moe_forward(L.handle, xd, Td, yd, side)
        st.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for L in layers:
                moe.moe_forward(L.handle, xd, Td, yd, cs)
        for _ in range(W):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(K):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / (K * NCOPY)
        dev_s = e0.elapsed_time(e1) * 1e-3 / (K * NCOPY)
        pct = percentiles(replay_times(g, K, st, 1.0 / NCOPY))
        bytes_step = touched * eb + shape.H * shape.E * 2 + Td * shape.H * (2 + 4)
        gu_bytes = touched * 2 * shape.H * shape.F * wbytes
        res[f"T{Td}"] = {
            "tokens_per_s": round(Td / wall, 1),
            "ms_per_step": round(wall * 1e3, 4),
            "device_ms": round(dev_s * 1e3, 4),
            "device_ms_p10_p50_p90": pct,
            "experts_touched": touched,
            "hbm_frac_step": round(bytes_step / dev_s / 1e9 / PEAK_HBM_GBS, 4),
            "gate_up_GBs": round(gu_bytes / (st_d[moe.MOE_STAGE_GATE_UP] * 1e-3) / 1e9, 1),
            "stages_ms_eager": {n: round(v, 4) for n, v in zip(moe.STAGE_NAMES, st_d)},
        }
        del g
    for L in layers:
        L.close()
    del blob
    torch.cuda.empty_cache()
    return res


def bench_stack(K, W, u8=False, batches=DECODE_BATCHES):
    """32 Mixtral-shaped layers, experts in one contiguous buffer (layer l,
    expert e at blob + (l*E + e)*stride), residual stream h <- h + MoE(norm(h));
    one step = all 32 layers on a decode batch, replayed as one HIP graph."""
    import numpy as np
    import torch

    import gen
    import mixture_experts_amd as moe
    shape, NL = gen.MIXTRAL, 32
    st = torch.cuda.current_stream()
    blob, stride = expert_blob(shape, NL, u8, layer_of=lambda b: b)
    fmt = moe.MOE_EXPERT_U8 if u8 else moe.MOE_EXPERT_DTYPE
    layers, keep = [], []
    for l in range(NL):
        base = blob.data_ptr() + l * shape.E * stride
        wr = torch.from_numpy(gen.gen_router(shape, layer=l).view(np.int16)).cuda()
        keep.append(wr)
        layers.append(moe.MoELayer(shape.H, shape.F, shape.E, shape.k, 64, moe.MOE_BF16, wr,
                                   base, stride, flags=moe.MOE_FLAG_RESIDUAL_PRENORM,
                                   expert_format=fmt))
    torch.cuda.synchronize()
    eb = 3 * shape.H * shape.F * (1 if u8 else 2) + (64 if u8 else 0)
    res = {"layers": NL, "expert_buffer_GB": round(blob.numel() / 1e9, 2),
           "expert_weights": "uint8 (affine per matrix)" if u8 else "bf16"}
    for T in batches:
        x0 = torch.from_numpy(gen.normal(0, 0, gen.T_X, T * shape.H, 1.0, "f32")).cuda()
        x0 = x0.view(T, shape.H)
        h = torch.empty_like(x0)
        h.copy_(x0)
        touched = 0
        for L in layers:  # eager pass: experts each layer touches (same routing as the graph)
            r = L.route(h, T)
            touched += int((r["counts"] > 0).sum().item())
            moe.moe_forward(L.handle, h, T, h, st)
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            for _ in range(2):
                h.copy_(x0)
                for L in layers:
                    moe.moe_forward(L.handle, h, T, h, side)
        st.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            h.copy_(x0)
            for L in layers:
                moe.moe_forward(L.handle, h, T, h, cs)
        for _ in range(W):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(K):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / K
        dev_s = e0.elapsed_time(e1) / K * 1e-3
        pct = percentiles(replay_times(g, K, st))
        byts = touched * eb
        res[f"T{T}"] = {"tokens_per_s": round(T / wall, 1), "ms_per_step": round(wall * 1e3, 4),
                        "device_ms": round(dev_s * 1e3, 4),
                        "device_ms_p10_p50_p90": pct,
                        "experts_touched_per_layer": round(touched / NL, 3),
                        "hbm_frac": round(byts / dev_s / 1e9 / PEAK_HBM_GBS, 4)}
        del g
    for L in layers:
        L.close()
    del blob
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)
    batches = tuple(int(b) for b in args.decode_batches.split(","))
    if not set(batches) <= set(DECODE_BATCHES):
        print(f"--decode-batches: choose from {DECODE_BATCHES}", file=sys.stderr, flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import gen
    import mixture_experts_amd as moe

    torch.cuda.set_device(0)
    shape, T = {"mixtral_prefill": (gen.MIXTRAL, 4096), "qwen": (gen.QWEN, 512),
                "deepseek": (gen.DEEPSEEK, 8192)}[args.workload]
    print(f"[bench] generating inputs for {shape.name} T={T}", file=sys.stderr, flush=True)
    x_h = gen.gen_x(shape, T)
    wr_h, b_h = gen.gen_router(shape), gen.gen_bias(shape)

    def dev(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()

    x, wr = dev(x_h), dev(wr_h)
    if args.no_cpu_baseline:  # the host copy of the experts only feeds the oracle
        ex_h = None
        ex = torch.empty(shape.E * shape.stride, dtype=torch.uint8, device="cuda")
        gen.experts_device(shape, ex.data_ptr(), stream=torch.cuda.current_stream().cuda_stream)
    else:
        ex_h = gen.gen_experts(shape)
        ex = dev(ex_h)
    bias = None if b_h is None else dev(b_h)
    layer = moe.MoELayer(shape.H, shape.F, shape.E, shape.k, T, moe.MOE_BF16, wr, ex,
                         shape.stride, bias)
    y = torch.empty((T, shape.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup

    print(f"[bench] prefill: {W} warmup + {K} timed steps", file=sys.stderr, flush=True)
    wall, stage_ms, dev_ms, per_step = time_layer(layer, x, y, T, K, W, stream)
    tok_s = T * K / wall
    S = T * shape.k
    step_flops = 6.0 * S * shape.H * shape.F + 2.0 * T * shape.H * shape.E
    r = layer.route(x, T)
    counts = r["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    streaming = S <= 32 * shape.E  # the library's path choice
    roof = gate_up_roofline(shape, T, touched, stage_ms[moe.MOE_STAGE_GATE_UP] * 1e-3)
    roof["kernel"] = ("streaming" if streaming else "grouped GEMM") + " gate/up + SiLU"
    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) tokens, N(0,0.02) weights (random init)",
        "config": {"workload": f"{shape.name}_prefill", "tokens": T, "hidden": shape.H,
                   "ffn": shape.F, "experts": shape.E, "top_k": shape.k,
                   "router_bias": shape.bias},
        # the committed counters cover the Mixtral-shaped launch only
        "roofline": dict(roof, traffic=measured_traffic()
                         if args.workload == "mixtral_prefill" else None),
        "stages_ms": {n: round(v, 4) for n, v in zip(moe.STAGE_NAMES, stage_ms)},
        "step_device_ms": round(dev_ms, 4),
        "step_device_ms_p10_p50_p90": percentiles(per_step),
        "step_tflops": round(step_flops / (dev_ms * 1e-3) / 1e12, 2),
        "step_mfma_frac": round(step_flops / (dev_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "routing": routing_stats(shape, x_h, wr_h, b_h, counts),
    }
    g_ms, g_pct = graph_step(layer, x, y, T, K, W, stream)
    out["graph_replay"] = {"device_ms": round(g_ms, 4), "device_ms_p10_p50_p90": g_pct,
                           "tokens_per_s": round(T / (g_ms * 1e-3), 1)}

    if not args.no_workloads and args.workload == "mixtral_prefill":
        print("[bench] 64-expert and 128-expert layers", file=sys.stderr, flush=True)
        out["workloads"] = {n: bench_workload(n, sh, t, K, W) for n, sh, t in
                            (("qwen2_moe_layer_T512", gen.QWEN, 512),
                             ("deepseek_moe_layer_T8192", gen.DEEPSEEK, 8192))}

    if not args.no_decode and args.workload == "mixtral_prefill":
        print("[bench] decode batches, bf16 and uint8 experts", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(shape, x, y, max(K, 50), W, batches=batches)
        out["decode_u8"] = bench_decode(shape, x, y, max(K, 50), W, u8=True, batches=batches)

    if not args.no_stack and args.workload == "mixtral_prefill":
        print("[bench] 32-layer stacked decode, bf16 and uint8 experts", file=sys.stderr,
              flush=True)
        out["stack_decode"] = bench_stack(max(K, 20), W, batches=batches)
        out["stack_decode_u8"] = bench_stack(max(K, 20), W, u8=True, batches=batches)

    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.layer_from_gen(shape, wr_h, b_h, ex_h)

        def sample_rate(seconds):
            """Tokens/s of the oracle over an evenly spread sample of tokens,
            grown until it takes about `seconds` / 4 or more."""
            n, el = 1, 0.0
            while True:
                toks = np.arange(n, dtype=np.int32) * (T // n)
                t0 = time.perf_counter()
                orc.tokens(x_h, toks)
                el = time.perf_counter() - t0
                if el >= seconds / 4 or n >= 1024:
                    return n, el
                n = min(1024, max(n * 2, int(n * seconds / 2 / max(el, 1e-3))))

        threads = oracle.num_threads()
        n, el = sample_rate(args.cpu_seconds)
        oracle.set_num_threads(1)
        n1, el1 = sample_rate(args.cpu_seconds / 2)
        oracle.set_num_threads(threads)
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
        except OSError:
            pass
        what = f"full layer per token (router, top-k, {shape.k} experts, combine), fp64"
        out["cpu_baseline"] = {"value": round(n / el, 3), "unit": "tokens/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{n} of the {T} tokens, {what}",
                               "seconds": round(el, 2), "cpu_model": model,
                               "single_thread": {"value": round(n1 / el1, 3),
                                                 "unit": "tokens/s", "cores": 1,
                                                 "sample": f"{n1} of the {T} tokens, {what}",
                                                 "seconds": round(el1, 2)}}
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = n
    layer.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
