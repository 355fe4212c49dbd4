#!/usr/bin/env python3
"""Benchmark of the Lightning Attention mixer library on one MI355X.

One step is one ``lightning_prefill`` call over the 512K-token Qwen3-1.7B-shaped RNN layer
(B = 1, H = 16, T = 524288, d = 128, bf16 activations, fp32 state): the segment pre-pass, the
segment scan and the main chunk-loop kernel, i.e. every prefill step of the mixer (prologue,
decayed intra-chunk scores, inter-chunk term, state update, gated output norm).  Inputs are
drawn on the device from a seeded generator and are resident in HBM before timing starts.

Printed (one JSON line): prefill tokens/s/layer (``value``), the main kernel's roofline
(algorithmic HBM bytes per launch / its average duration, timed with HIP events recorded by the
library around that kernel on the launch stream), its MFMA rate, the batched decode step
(B = 64, H = 16, d = 128) in microseconds with its HBM roofline, and the fp64 CPU oracle timed on
a bounded sample of the same prefill workload on this host's cores.  ``decode.batch_1``: the
same step with one sequence (16 workgroups), timed as a captured HIP graph's replay because a
step takes less time than its launch.  Under ``other_configs``: the prefill of the 32K-token
layer and of the Qwen3-8B-shaped one (B = 4, H = 32, T = 128K, nonzero initial state), each with
its roofline.  Under ``layer``: the whole RNN layer around the mixer (QKVZ projection GEMM,
mixer, output projection GEMM; d_model = 2048) at the same 512K tokens with per-stage times and
the QKVZ GEMM's MFMA roofline, its B = 64 and B = 1 decode steps, and the layer oracle timed on
a bounded sample.  Under ``attention``: the hybrid's
HyPE softmax-attention layer (NoPE, s_t = log_a(t + a) logits scale, 16 query / 8 key-value
heads) at 512K tokens with the flash kernel's MFMA roofline, and its oracle on sampled rows.
Under ``time_dependent_decay``: the same prefill with a per-token decay alpha_t (the
data-dependent variant of the same kernels) and its cost relative to the fixed decay.
"""
from __future__ import annotations

import argparse
import ctypes as ct
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_qwen17_512k.md")
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "prefill tokens/s/layer at T=512K (MFMA %) ; decode step µs at B=64 (HBM %)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen17_512k",
                    choices=["qwen17_512k", "qwen17_32k", "qwen8_128k"])
    ap.add_argument("--segments", type=int, default=0, help="0 = library default")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per chunk: 0 (= 32) or 64")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--decode-buffers", type=int, default=8,
                    help="rotating state buffers (64 MiB each) so the step cannot run from MALL")
    ap.add_argument("--cpu-sample-tokens", type=int, default=524288)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 32K and Qwen3-8B-shaped prefill legs")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the whole-layer legs (projections + mixer + output projection)")
    ap.add_argument("--layer-steps", type=int, default=5)
    ap.add_argument("--cpu-layer-tokens", type=int, default=65536)
    ap.add_argument("--no-attn", action="store_true", help="skip the HyPE attention leg")
    ap.add_argument("--no-time-dep", action="store_true",
                    help="skip the data-dependent decay variant")
    ap.add_argument("--attn-steps", type=int, default=2)
    ap.add_argument("--attn-warmup", type=int, default=1)
    ap.add_argument("--cpu-attn-rows", type=int, default=32)
    ap.add_argument("--attn-decode-steps", type=int, default=50)
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill-backward leg")
    ap.add_argument("--bwd-steps", type=int, default=5)
    ap.add_argument("--cpu-bwd-slices", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed runs, copy this many MiB device to device three times "
                         "(a plain copy of known size that calibrates HBM byte counters)")
    return ap.parse_args()


def copy_calibration(torch, mib):
    """Three device-to-device copies of `mib` MiB: each reads and writes exactly mib MiB."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


MIXER_SOURCES = ("abi.hip", "decode.hip", "lt_device.h", "lt_internal.h", "prefill.hip")
LAYER_SOURCES = ("decode.hip", "gemm.hip", "gemm_tile.hip", "gemv.hip", "layer.hip", "lt_device.h",
                 "lt_internal.h")
LAYER_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_layer_qwen17_512k.md")
BWD_SOURCES = ("backward.hip", "lt_device.h", "lt_internal.h")
ATTN_SOURCES = ("attention.hip", "lt_device.h", "lt_internal.h")
ATTN_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_attention_qwen17_512k.md")
BWD_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_backward_qwen17_16k.md")


def source_fingerprint(sources=MIXER_SOURCES):
    """sha256 over the sources of the measured kernels and their launch configuration (the code
    the byte counters measured): the mixer's by default, the layer's GEMMs and decode step with
    LAYER_SOURCES."""
    import hashlib

    h = hashlib.sha256()
    files = [os.path.join(ROOT, "long_context_hybrid_amd", "csrc", f) for f in sources]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload, record=TRAFFIC_RECORD, sources=MIXER_SOURCES):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    record, scaled by what the same counters read for a plain copy of known size; None when no
    record exists for this workload or the kernel sources changed since it was taken."""
    try:
        with open(record) as fh:
            lines = [l for l in fh if l.startswith("traffic-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("traffic-record: "):])
    if rec.get("source_sha256") != source_fingerprint(sources):
        return None
    for k in rec.get("entries", []):
        if k["kernel"] == kernel and k["workload"] == workload:
            return int(round((k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"])
                             * 1024))
    return None


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime PyTorch already loaded (one runtime)."""

    def __init__(self):
        self.hip = ct.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ct.POINTER(ct.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ct.POINTER(ct.c_float), ct.c_void_p, ct.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ct.c_void_p]
        self.hip.hipEventRecord.argtypes = [ct.c_void_p, ct.c_void_p]

    def record(self, e, stream):
        """Record event `e` on a torch stream (the library's calls run on torch's current one)."""
        if self.hip.hipEventRecord(ct.c_void_p(e), ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ct.c_void_p()
            if self.hip.hipEventCreate(ct.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b):
        ms = ct.c_float()
        if self.hip.hipEventElapsedTime(ct.byref(ms), ct.c_void_p(a), ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ct.c_void_p(e))


def eager_step_stats(torch, step, n, group=10):
    """Median and minimum step time over n eagerly launched steps, in groups of `group` steps
    bracketed by HIP events (a step is shorter than its host-side launch plus one event record,
    so an event per step would time launch gaps).  A separate pass after the timed loop."""
    hev = HipEvents()
    ng = max(1, n // group)
    ev = hev.create(ng + 1)
    cur = torch.cuda.current_stream()
    for gi in range(ng):
        hev.record(ev[gi], cur)
        for i in range(group):
            step(gi * group + i)
    hev.record(ev[ng], cur)
    torch.cuda.synchronize()
    per = [hev.elapsed_ms(ev[i], ev[i + 1]) * 1e3 / group for i in range(ng)]
    hev.destroy(ev)
    return {"us_median": round(statistics.median(per), 3), "us_min": round(min(per), 3),
            "groups": ng, "steps_per_group": group}


def bench_prefill(args, torch, lt, synth, workload=None, steps=None):
    spec = synth.WORKLOADS[workload or args.workload]
    steps = steps or args.steps
    dev = torch.device("cuda:0")
    inp = synth.make_prefill(spec, device=dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    chunk, P, seg_len = lt.lightning_prefill_plan(B, T, H, d, spec.dtype, args.chunk, args.segments)
    y = torch.empty_like(inp["q"])
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws_bytes = lt.lightning_prefill_workspace_size(B, T, H, d, spec.dtype, args.chunk, args.segments)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    call_args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["qw"], inp["kw"], inp["lambdas"],
                 inp["rope_base"])
    kw = dict(rms_eps=inp["eps"], pos0=inp["pos0"], state_in=inp["state_in"], state_out=s_out,
              y=y, chunk=args.chunk, segments=args.segments, workspace=ws)
    for _ in range(args.warmup):
        lt.lightning_prefill(*call_args, **kw)
    torch.cuda.synchronize()

    hev = HipEvents()
    ev = hev.create(2 * steps)
    call_ev = hev.create(steps + 1)  # before each call, and after the last
    cur = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        hev.record(call_ev[i], cur)
        lt.lightning_prefill(*call_args, **kw, main_kernel_events=(ev[2 * i], ev[2 * i + 1]))
    hev.record(call_ev[steps], cur)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    main_list = [hev.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps)]
    call_list = [hev.elapsed_ms(call_ev[i], call_ev[i + 1]) for i in range(steps)]
    main_ms = sum(main_list) / steps
    hev.destroy(ev)
    hev.destroy(call_ev)

    ms_per_step = total_ms / steps
    tokens = B * T
    act_bytes = 2 if spec.dtype == torch.bfloat16 else 4
    units = B * H * T  # token-heads per launch
    per_unit = 5 * d * act_bytes  # read q, k, v, g and write y
    state_bytes = B * H * P * 2 * d * d * 4  # each segment reads its entry state, writes its end
    alg_bytes = units * per_unit + state_bytes
    achieved = alg_bytes / (main_ms * 1e-3) / 1e9
    useful_flops = units * (4 * d * d + 2 * chunk * d)
    tflops = useful_flops / (main_ms * 1e-3) / 1e12
    pre_bytes = B * H * (P - 1) * seg_len * 2 * d * act_bytes if P > 1 else 0  # k, v of segments 0 .. P-2
    return dict(
        spec=spec, inp=inp, chunk=chunk, P=P, ms_per_step=ms_per_step, main_ms=main_ms, steps=steps,
        value=tokens / (ms_per_step * 1e-3),
        step_stats={"call_ms_median": round(statistics.median(call_list), 4),
                    "call_ms_min": round(min(call_list), 4),
                    "main_ms_median": round(statistics.median(main_list), 4),
                    "main_ms_min": round(min(main_list), 4)},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": measured_traffic("main", spec.name),
                  "kernel": "chunk_kernel<ModeBF16,128,false> (main chunk loop)",
                  "alg_bytes_per_launch": alg_bytes, "bytes_per_token_head": per_unit,
                  "launch_ms": round(main_ms, 4)},
        mfma={"useful_flops_per_launch": useful_flops, "achieved_tflops": round(tflops, 1),
              "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
              "flops_per_token_head": 4 * d * d + 2 * chunk * d},
        whole_call={"ms": round(ms_per_step, 4), "prepass_alg_bytes": pre_bytes,
                    "alg_bytes": alg_bytes + pre_bytes,
                    "hbm_frac": round((alg_bytes + pre_bytes) / (ms_per_step * 1e-3) / 1e9
                                      / HBM_PEAK_GBS, 4)},
    )


def graph_replay_us(torch, step, n):
    """Mean step time of one replay of n steps captured into a HIP graph (torch.cuda.graph),
    after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for i in range(n):
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) * 1e3 / n


def bench_decode(args, torch, lt, synth, B=None):
    """The mixer's decode step over rotating state buffers (so the state cannot be served from
    MALL).  At B = 64 the steps are launched one by one; with fewer rows a step's kernel takes
    less time than the host needs to launch it, so the steps are captured once into a HIP graph
    (torch.cuda.graph) and the graph's replay is timed."""
    spec = synth.DECODE_B64
    dev = torch.device("cuda:0")
    inp = synth.make_decode(spec, device=dev, B=B)
    B, H, d = inp["B"], inp["H"], inp["d"]
    # enough buffers that the states of one pass over them exceed the 256 MB MALL
    nbuf = max(args.decode_buffers, -(-300 * 2**20 // (B * H * d * d * 4)))
    states = [inp["state_in"].clone() for _ in range(nbuf)]
    y = torch.empty_like(inp["q"])
    a = (inp["q"], inp["k"], inp["v"], inp["g"], inp["qw"], inp["kw"], inp["lambdas"],
         inp["rope_base"], inp["positions"])

    def step(i):
        lt.lightning_decode_step(*a, states[i % len(states)], y=y, rms_eps=inp["eps"])

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    graph = B < 64
    if graph:
        us = graph_replay_us(torch, step, args.decode_steps)
    else:
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(args.decode_steps):
            step(i)
        stop.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / args.decode_steps
    stats = None if graph else eager_step_stats(torch, step, args.decode_steps)
    # the same steps replayed from a captured graph (no host launch gaps), beside the eager time
    us_graph = us if graph else graph_replay_us(torch, step, args.decode_steps)
    act_bytes = 2
    per_bh = 2 * d * d * 4 + 5 * d * act_bytes
    alg = B * H * per_bh + B * 8
    gbs = alg / (us * 1e-6) / 1e9
    name = spec.name if B == spec.B else spec.name.replace("B=%d" % spec.B, "B=%d" % B)
    return {"workload": name, "us_per_step": round(us, 3),
            "timing": "HIP graph of %d steps" % args.decode_steps if graph else "eager launches",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode", name),
                         "kernel": "decode_kernel<ModeBF16,128>", "alg_bytes_per_launch": alg,
                         "bytes_per_bh": per_bh, "workgroups": B * H},
            "step_stats": stats, "us_per_step_graph": round(us_graph, 3),
            "state_buffers": len(states)}


def bench_configs(args, torch, lt, synth):
    """The other prefill configurations at their own sizes: the 32K-token Qwen3-1.7B-shaped layer
    and the Qwen3-8B-shaped one (B = 4, H = 32, T = 128K, nonzero initial state)."""
    out = {}
    for name, steps in (("qwen17_32k", max(args.steps, 20)), ("qwen8_128k", args.steps)):
        print(f"[bench] prefill {name}: warmup {args.warmup}, steps {steps}", file=sys.stderr,
              flush=True)
        r = bench_prefill(args, torch, lt, synth, workload=name, steps=steps)
        sp = r["spec"]
        out[name] = {"workload": sp.name, "B": sp.B, "T": sp.T, "H": sp.H, "d": sp.d,
                     "chunk": r["chunk"], "segments": r["P"], "steps": steps,
                     "ms_per_step": round(r["ms_per_step"], 4),
                     "value": round(r["value"], 1), "unit": "tokens/s/layer",
                     "roofline": r["roofline"], "mfma": r["mfma"], "whole_call": r["whole_call"],
                     "step_stats": r["step_stats"]}
        del r
        torch.cuda.empty_cache()
    return out


def bench_time_dependent(args, torch, lt, synth, fixed):
    """The same 512K prefill with a data-dependent decay alpha_t (log2 alpha ~ -U(0, 0.05) per
    token and head) instead of the fixed lambda_h: the time-dependent variant of the kernels, whose
    cost against the fixed decay is the contrast Fig. 7 draws between mixers.  Also its B = 64
    decode step."""
    spec = synth.QWEN17_512K
    dev = torch.device("cuda:0")
    inp = fixed["inp"]
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 7)
    lg = (-torch.rand((B, T, H), generator=gen, device=dev) * 0.05).float()
    y = torch.empty_like(inp["q"])
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(lt.lightning_prefill_dd_workspace_size(B, T, H, d, spec.dtype), 1),
                     dtype=torch.uint8, device=dev)
    call = (inp["q"], inp["k"], inp["v"], inp["g"], inp["qw"], inp["kw"], lg, inp["rope_base"])
    kw = dict(rms_eps=inp["eps"], state_out=s_out, y=y, workspace=ws)
    for _ in range(args.warmup):
        lt.lightning_prefill_dd(*call, **kw)
    torch.cuda.synchronize()
    hev = HipEvents()
    ev = hev.create(2 * args.steps)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        lt.lightning_prefill_dd(*call, **kw, main_kernel_events=(ev[2 * i], ev[2 * i + 1]))
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    main_ms = sum(hev.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(args.steps)) / args.steps
    hev.destroy(ev)
    units = B * H * T
    alg = units * (5 * d * 2 + 4) + fixed["P"] * B * H * 2 * d * d * 4  # + the per-token decay
    gbs = alg / (main_ms * 1e-3) / 1e9
    out = {"workload": spec.name + ", data-dependent decay log2(alpha) ~ -U(0, 0.05)",
           "ms_per_step": round(ms, 4), "value": round(B * T / (ms * 1e-3), 1),
           "unit": "tokens/s/layer",
           "cost_vs_fixed_decay": round(ms / fixed["ms_per_step"], 3),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("main", spec.name + ", data-dependent decay"),
                        "kernel": "chunk_kernel<ModeBF16,128,false,4,true> (main pass)",
                        "alg_bytes_per_launch": alg, "launch_ms": round(main_ms, 4)}}
    if not args.no_decode:
        dspec = synth.DECODE_B64
        dinp = synth.make_decode(dspec, device=dev)
        states = [dinp["state_in"].clone() for _ in range(args.decode_buffers)]
        dl = (-torch.rand((dinp["B"], dinp["H"]), generator=gen, device=dev) * 0.05).float()
        yd = torch.empty_like(dinp["q"])
        a = (dinp["q"], dinp["k"], dinp["v"], dinp["g"], dinp["qw"], dinp["kw"], dl,
             dinp["rope_base"], dinp["positions"])
        for i in range(3):
            lt.lightning_decode_step_dd(*a, states[i % len(states)], y=yd)
        torch.cuda.synchronize()
        start.record()
        for i in range(args.decode_steps):
            lt.lightning_decode_step_dd(*a, states[i % len(states)], y=yd)
        stop.record()
        torch.cuda.synchronize()
        out["decode_us_per_step"] = round(start.elapsed_time(stop) * 1e3 / args.decode_steps, 3)
    return out


def bench_layer(args, torch, lt, synth):
    """The whole RNN layer (QKVZ GEMM, mixer, W_o GEMM) at 512K tokens, with each stage timed by
    the HIP events the library records between the stages on the launch stream."""
    spec = synth.LAYER_QWEN17_512K
    dev = torch.device("cuda:0")
    inp = synth.make_layer(spec, device=dev)
    B, T, H, d, dm = inp["B"], inp["T"], inp["H"], inp["d"], inp["d_model"]
    out = torch.empty_like(inp["x"])
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(lt.lightning_layer_prefill_workspace_size(B, T, H, d, dm), dtype=torch.uint8,
                     device=dev)
    call = (inp["x"], inp["w_qkvz"], inp["w_o"], inp["qw"], inp["kw"], inp["lambdas"],
            inp["rope_base"], H, d)
    kw = dict(rms_eps=inp["eps"], state_out=s_out, out=out, workspace=ws)
    for _ in range(args.warmup):
        lt.lightning_layer_prefill(*call, **kw)
    torch.cuda.synchronize()
    hev = HipEvents()
    n = args.layer_steps
    ev = hev.create(4 * n)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(n):
        lt.lightning_layer_prefill(*call, **kw, stage_events=ev[4 * i:4 * i + 4])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    stage = [sum(hev.elapsed_ms(ev[4 * i + j], ev[4 * i + j + 1]) for i in range(n)) / n
             for j in range(3)]
    hev.destroy(ev)
    rows = B * T
    f1 = 2 * rows * (4 * H * d) * dm
    f2 = 2 * rows * dm * (H * d)
    t1 = f1 / (stage[0] * 1e-3) / 1e12
    t2 = f2 / (stage[2] * 1e-3) / 1e12
    del inp, out, ws
    return {"workload": spec.name, "ms_per_step": round(ms, 4),
            "value": round(rows / (ms * 1e-3), 1), "unit": "tokens/s/layer", "steps": n,
            "stages_ms": {"qkvz_gemm": round(stage[0], 4), "mixer": round(stage[1], 4),
                          "o_gemm": round(stage[2], 4)},
            "roofline": {"bound": "mfma", "achieved": round(t1, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(t1 / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("qkvz_gemm", spec.name,
                                                     LAYER_TRAFFIC_RECORD, LAYER_SOURCES),
                         "kernel": "gemm_tile_kernel: x [W_q|W_k|W_v|W_z] (M=%d N=%d K=%d)"
                                   % (rows, 4 * H * d, dm),
                         "flops_per_launch": f1, "launch_ms": round(stage[0], 4),
                         "alg_bytes_per_launch": rows * dm * 2 + 4 * H * d * dm * 2
                                                 + rows * 4 * H * d * 2},
            "o_gemm": {"achieved_tflops": round(t2, 1), "frac": round(t2 / BF16_PEAK_TFLOPS, 4),
                       "flops_per_launch": f2},
            "mfma_floor_ms": round((f1 + f2) / (BF16_PEAK_TFLOPS * 1e12) * 1e3, 3)}


def bench_layer_decode(args, torch, lt, synth, B=None):
    """One layer decode step at B = 64 (or B) over rotating sets of (state, weights), so that
    neither the state nor the 40 MiB of projection weights can be served from MALL.  With fewer
    than 64 rows the steps are timed as the replay of a captured HIP graph (see bench_decode)."""
    spec = synth.LAYER_DECODE_B64
    dev = torch.device("cuda:0")
    inp = synth.make_layer(spec, device=dev, B=B)
    B, H, d, dm = inp["B"], inp["H"], inp["d"], inp["d_model"]
    nset = args.decode_buffers
    sets = [(inp["state_in"].clone(), inp["w_qkvz"].clone(), inp["w_o"].clone())
            for _ in range(nset)]
    out = torch.empty_like(inp["x"])
    ws = torch.empty(lt.lightning_layer_decode_workspace_size(B, H, d, dm), dtype=torch.uint8,
                     device=dev)

    def step(i):
        st, w, wo = sets[i % nset]
        lt.lightning_layer_decode_step(inp["x"], w, wo, inp["qw"], inp["kw"], inp["lambdas"],
                                       inp["rope_base"], H, d, inp["positions"], st,
                                       rms_eps=inp["eps"], out=out, workspace=ws)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    graph = B < 64
    if graph:
        us = graph_replay_us(torch, step, args.decode_steps)
    else:
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(args.decode_steps):
            step(i)
        stop.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(stop) * 1e3 / args.decode_steps
    stats = None if graph else eager_step_stats(torch, step, args.decode_steps)
    # the same steps replayed from a captured graph (no host launch gaps), beside the eager time
    us_graph = us if graph else graph_replay_us(torch, step, args.decode_steps)
    wbytes = (4 * H * d * dm + dm * H * d) * 2
    io = B * dm * 2 * 2 + B * (4 * H * d + H * d) * 2 * 2  # x, out; projections and y written + read
    alg = wbytes + B * H * 2 * d * d * 4 + io + B * 8
    gbs = alg / (us * 1e-6) / 1e9
    name = spec.name if B == spec.B else spec.name.replace("B=%d" % spec.B, "B=%d" % B)
    return {"workload": name, "us_per_step": round(us, 3),
            "timing": "HIP graph of %d steps" % args.decode_steps if graph else "eager launches",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("layer_decode_step", name, LAYER_TRAFFIC_RECORD,
                                                     LAYER_SOURCES),
                         "alg_bytes_per_step": alg, "weight_bytes": wbytes},
            "step_stats": stats, "us_per_step_graph": round(us_graph, 3), "rotating_sets": nset}


def bench_attn(args, torch, lt, synth):
    """HyPE softmax attention (the hybrid's attention layers) at 512K tokens: the prologue
    (QK-norm and the s_t log2(e)/sqrt(d) query scale; the normalised keys into the key cache)
    and the flash-attention kernel, timed with the HIP events the library records around the
    latter and one recorded just before each call."""
    spec = synth.ATTN_QWEN17_512K
    dev = torch.device("cuda:0")
    inp = synth.make_attn(spec, device=dev)
    B, T, Hq, Hkv, d = inp["B"], inp["T"], inp["Hq"], inp["Hkv"], inp["d"]
    y = torch.empty_like(inp["q"])
    cache = torch.empty_like(inp["k"])
    ws = torch.empty(lt.lightning_attn_prefill_workspace_size(B, T, Hq, Hkv, d, torch.bfloat16,
                                                              True, True),
                     dtype=torch.uint8, device=dev)
    call = (inp["q"], inp["k"], inp["v"], inp["g"], inp["a"])
    kw = dict(q_norm_w=inp["qw"], k_norm_w=inp["kw"], rms_eps=inp["eps"], y=y,
              key_cache_out=cache, workspace=ws)
    for _ in range(args.attn_warmup):
        lt.lightning_attn_prefill(*call, **kw)
    torch.cuda.synchronize()
    hev = HipEvents()
    n = args.attn_steps
    ev = hev.create(3 * n)
    cur = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(n):
        hev.record(ev[3 * i], cur)
        lt.lightning_attn_prefill(*call, **kw, main_kernel_events=(ev[3 * i + 1], ev[3 * i + 2]))
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    main_ms = sum(hev.elapsed_ms(ev[3 * i + 1], ev[3 * i + 2]) for i in range(n)) / n
    pro_ms = sum(hev.elapsed_ms(ev[3 * i], ev[3 * i + 1]) for i in range(n)) / n
    hev.destroy(ev)
    # prologue bytes: q read and q~ written (Hq rows), k read and k^ written to the key cache
    pro_bytes = 2 * B * T * (Hq + Hkv) * d * 2
    pro_gbs = pro_bytes / (pro_ms * 1e-3) / 1e9
    flops = 4 * d * Hq * B * T * (T + 1) // 2  # q.k and p.v over the causal triangle
    tf = flops / (main_ms * 1e-3) / 1e12
    del inp, y, cache, ws
    return {"workload": spec.name, "ms_per_step": round(ms, 3),
            "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s/layer", "steps": n,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("attn_fwd", spec.name, ATTN_TRAFFIC_RECORD,
                                                     ATTN_SOURCES),
                         "kernel": "attn_fwd_kernel<2> (flash attention)",
                         "flops_per_launch": flops, "launch_ms": round(main_ms, 3)},
            "prologue": {"ms": round(pro_ms, 4), "bound": "hbm", "achieved": round(pro_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(pro_gbs / HBM_PEAK_GBS, 4), "alg_bytes": pro_bytes,
                         "traffic": measured_traffic("attn_prologue", spec.name, ATTN_TRAFFIC_RECORD,
                                                     ATTN_SOURCES)}}


def bench_attn_decode(args, torch, lt, synth):
    """One HyPE attention decode step at B = 1 with 524287 cached tokens (Qwen3-1.7B shape):
    the step reads the whole 2 GiB key/value cache, which no cache level holds."""
    spec = synth.ATTN_QWEN17_512K
    dev = torch.device("cuda:0")
    Hq, Hkv, d, cap = spec.Hq, spec.Hkv, spec.d, spec.T
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 100)

    def rnd(*shape):
        return torch.randn(*shape, generator=gen, device=dev).to(torch.bfloat16)

    q, kn, vn, g = rnd(1, Hq, d), rnd(1, Hkv, d), rnd(1, Hkv, d), rnd(1, Hq, d)
    kc, vc = rnd(1, cap, Hkv, d), rnd(1, cap, Hkv, d)
    qw = 0.5 + torch.rand(d, generator=gen, device=dev)
    kw = 0.5 + torch.rand(d, generator=gen, device=dev)
    n = cap - 1
    y = torch.empty_like(q)
    ws = torch.empty(lt.lightning_attn_decode_workspace_size(1, Hq, Hkv, d, n), dtype=torch.uint8,
                     device=dev)

    def step():
        lt.lightning_attn_decode_step(q, kn, vn, g, kc, vc, [n], spec.a, q_norm_w=qw, k_norm_w=kw,
                                      y=y, workspace=ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.attn_decode_steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) * 1e3 / args.attn_decode_steps
    alg = 2 * (n + 1) * Hkv * d * 2 + (2 * Hq + 2 * Hkv + Hq) * d * 2
    gbs = alg / (us * 1e-6) / 1e9
    del kc, vc
    name = "HyPE attention decode step B=1, 524287 cached tokens, Hq=16 Hkv=8 d=128 bf16"
    return {"workload": name, "us_per_step": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("attn_decode_step", name, ATTN_TRAFFIC_RECORD,
                                                     ATTN_SOURCES),
                         "alg_bytes_per_step": alg}}


def bench_backward(args, torch, lt, synth):
    """The backward of the mixer prefill at the 16K training shape (B = 8, H = 16): dq, dk, dv,
    dgate, d_state_in and the three norm-weight gradients from dL/dy.  The two chunk sweeps are
    timed by HIP events on the call's stream."""
    spec = synth.BWD_QWEN17_16K
    dev = torch.device("cuda:0")
    inp = synth.make_backward(spec, device=dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    ws = torch.empty(lt.lightning_prefill_backward_workspace_size(B, T, H, d), dtype=torch.uint8,
                     device=dev)
    call = (inp["q"], inp["k"], inp["v"], inp["g"], inp["qw"], inp["kw"], inp["lambdas"],
            inp["rope_base"], inp["dy"])
    kw = dict(rms_eps=inp["eps"], workspace=ws)
    for _ in range(args.warmup):
        lt.lightning_prefill_backward(*call, **kw)
    torch.cuda.synchronize()
    hev = HipEvents()
    ev = hev.create(4 * args.bwd_steps)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.bwd_steps):
        lt.lightning_prefill_backward(*call, **kw, kernel_events=ev[4 * i:4 * i + 4])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.bwd_steps
    n = args.bwd_steps
    dq_ms = sum(hev.elapsed_ms(ev[4 * i], ev[4 * i + 1]) for i in range(n)) / n
    dkv_ms = sum(hev.elapsed_ms(ev[4 * i + 2], ev[4 * i + 3]) for i in range(n)) / n
    hev.destroy(ev)
    pl = lt.lightning_prefill_plan_cus(torch.cuda.get_device_properties(0).multi_processor_count,
                                       B, T, H, d)
    P, seg_len = pl["backward_segments"], pl["backward_segment_len"]
    units = B * T * H
    wgs = B * H * P
    st = d * d * 4
    C = 32
    act = d * 2  # one bf16 activation row of one token-head
    # The method's minimum per call: read q, k, v, gate, dy once and write dq, dk, dv, dgate once
    # (9 rows per token-head), plus recomputing the forward entry states of segments 1 .. P-1
    # (k and v of segments 0 .. P-2 read once more) and the d x d states (entry state and state
    # gradient per segment; d_state_in).
    recompute = B * H * (P - 1) * seg_len * 2 * act if P > 1 else 0
    method_min = units * 9 * act + recompute + wgs * 2 * st + B * H * st
    # What the current kernels move besides: dL/do written by the first sweep and read by the
    # second, and the two masked C x C fp32 score tiles of every chunk likewise.
    score = units * 2 * C * 4
    intermediates = 2 * units * act + 2 * score
    # Bytes each sweep moves as built (inputs, outputs and intermediates):
    # dq sweep reads q, k, v, gate, dy; writes dq, dgate, do and the score tiles; entry state in,
    # W out.  dk/dv sweep reads q, k, v, do and the score tiles; writes dk, dv; the segment's
    # end-state gradient in.
    moved_dq = units * 8 * act + score + wgs * 2 * st
    moved_dkv = units * 6 * act + score + wgs * st
    # useful MFMA flops per token-head: dq sweep 4 C d + 4 d^2 multiply-adds (scores, P V, do V^T,
    # dP K~; q~ S, do S^T, W, S update), dk/dv sweep 2 C d + 3 d^2 (P^T do, dP^T Q~; K~ dS,
    # V dS^T, dS update)
    fl_dq = units * 2 * (4 * C * d + 4 * d * d)
    fl_dkv = units * 2 * (2 * C * d + 3 * d * d)
    legs = {"dq_sweep": (dq_ms, moved_dq, fl_dq, "bwd_dq_kernel<128> (forward-in-time sweep)"),
            "dkv_sweep": (dkv_ms, moved_dkv, fl_dkv, "bwd_dkv_kernel<128> (backward-in-time sweep)")}
    dom = max(legs, key=lambda k: legs[k][0])
    traffic = measured_traffic(dom, spec.name, BWD_TRAFFIC_RECORD, BWD_SOURCES)
    # The roofline is the whole call's against the method's minimum bytes: intermediates the
    # implementation chooses to round-trip through HBM earn nothing.
    gbs = method_min / (ms * 1e-3) / 1e9
    out = {"workload": spec.name, "ms_per_step": round(ms, 4),
           "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s/layer",
           "steps": args.bwd_steps, "segments": P,
           "stages_ms": {"dq_sweep": round(dq_ms, 4), "dkv_sweep": round(dkv_ms, 4),
                         "rest": round(ms - dq_ms - dkv_ms, 4)},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": traffic, "traffic_kernel": legs[dom][3],
                        "kernel": "whole backward call (state pass, scan, both sweeps, weight sums)",
                        "alg_bytes_per_launch": method_min,
                        "bytes_per_token_head": 9 * act, "launch_ms": round(ms, 4)},
           "intermediate_bytes": intermediates,
           "sweeps": {k: {"ms": round(v[0], 4), "moved_bytes": v[1],
                          "moved_gbs": round(v[1] / (v[0] * 1e-3) / 1e9, 1),
                          "useful_tflops": round(v[2] / (v[0] * 1e-3) / 1e12, 1)}
                      for k, v in legs.items()}}
    return out


def cpu_baseline_backward(args, torch, synth):
    """The gradient oracle (fp64 numpy, token by token) on whole (b, h) slices of the 16K
    training-shape backward workload."""
    import numpy as np

    from oracle import backward as ob

    spec = synth.BWD_QWEN17_16K
    inp = synth.make_backward(spec, device="cuda:0")
    n = args.cpu_bwd_slices
    slices = [(b, 0) for b in range(n)]
    host = {k: synth.host_bits(inp[k][:n, :, :1].cpu()) for k in ("q", "k", "v", "g", "dy")}
    t0 = time.perf_counter()
    r = ob.prefill_backward(host["q"], host["k"], host["v"], host["g"], host["dy"],
                            inp["qw"][:1].cpu().numpy(), inp["kw"][:1].cpu().numpy(),
                            inp["lambdas"][:1], inp["rope_base"], eps=inp["eps"], slices=slices)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["dq"]).all()
    T, H = inp["T"], inp["H"]
    return {"value": round(n * T / dt / H, 1), "unit": "tokens/s/layer", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} whole (b, h) slices ({T} tokens, head 0) of the {spec.name} workload, "
                      f"fp64 numpy on one thread of control, {dt:.1f} s; token-heads/s divided "
                      f"by the {H} heads of a layer"}


def cpu_baseline_attn(args, torch, synth):
    """The attention oracle on evenly spaced query rows of the 512K workload (all heads): their
    mean cost is the mean over all rows, so rows / time estimates the whole prefill's rate."""
    import numpy as np

    from oracle import attention as oa

    spec = synth.ATTN_QWEN17_512K
    inp = synth.make_attn(spec, device="cuda:0")
    host = {n: synth.host_bits(inp[n].cpu()) for n in ("q", "k", "v", "g")}
    n = args.cpu_attn_rows
    T = inp["T"]
    rows = (np.arange(n) * T + T // 2) // n
    t0 = time.perf_counter()
    r = oa.attn_prefill(host["q"], host["k"], host["v"], host["g"], inp["qw"].cpu().numpy(),
                        inp["kw"].cpu().numpy(), None, a=inp["a"], eps=inp["eps"], rows=rows,
                        want_k_hat=False)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["y"]).all()
    return {"value": round(n / dt, 3), "unit": "tokens/s/layer", "cores": 1, "kind": "oracle",
            "sample": f"{n} evenly spaced query rows (all {inp['Hq']} heads) of the {spec.name} "
                      f"workload, fp64 numpy on one thread of control, {dt:.1f} s"}


def cpu_baseline_layer(args, torch, synth):
    """The layer oracle (fp64 projections through numpy, the fp64 recurrence in C threads) on the
    first tokens of the 512K layer workload."""
    import numpy as np

    from oracle import layer as ol

    spec = synth.LAYER_QWEN17_512K
    Ts = args.cpu_layer_tokens
    inp = synth.make_layer(spec, device="cpu", T=Ts)
    cores = len(os.sched_getaffinity(0))
    args_h = (synth.host_bits(inp["x"]), synth.host_bits(inp["w_qkvz"]),
              synth.host_bits(inp["w_o"]), inp["qw"].numpy(), inp["kw"].numpy(), inp["lambdas"],
              inp["rope_base"], inp["H"], inp["d"])
    t0 = time.perf_counter()
    r = ol.layer_prefill(*args_h, eps=inp["eps"], nthreads=cores)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["out"]).all()
    return {"value": round(Ts / dt, 1), "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"first {Ts} tokens of the {spec.name} workload (same generator, same "
                      f"shapes), fp64: numpy matmuls for the projections, the token-by-token "
                      f"recurrence on {r['threads']} threads, {dt:.1f} s"}


def cpu_baseline(args, torch, synth, pre):
    import numpy as np

    import oracle

    inp = pre["inp"]
    Ts = min(args.cpu_sample_tokens, inp["T"])
    B, H = inp["B"], inp["H"]
    host = {n: synth.host_bits(inp[n][:, :Ts]) for n in ("q", "k", "v", "g")}
    s0 = None if inp["state_in"] is None else inp["state_in"].cpu().numpy()
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    out = oracle.prefill(host["q"], host["k"], host["v"], host["g"], inp["qw"].cpu().numpy(),
                         inp["kw"].cpu().numpy(), inp["lambdas"], inp["rope_base"],
                         eps=inp["eps"], pos0=inp["pos0"], state_in=s0, want_o=False,
                         want_state=False, nthreads=cores)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["y"]).all()
    return {"value": round(B * Ts / dt, 1), "unit": "tokens/s/layer", "cores": out["threads"],
            "kind": "oracle",
            "sample": f"first {Ts} tokens of the {pre['spec'].name} workload, all {B * H} "
                      f"(b, h) slices, fp64 token-by-token recurrence, {dt:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this mixer build runs on a single MI355X and has "
              f"no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE={world}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_hybrid_amd.lightning as lt
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    print(f"[bench] prefill {args.workload}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    pre = bench_prefill(args, torch, lt, synth)
    dec = None
    if not args.no_decode:
        print(f"[bench] decode B=64: steps {args.decode_steps}", file=sys.stderr, flush=True)
        dec = bench_decode(args, torch, lt, synth)
        print(f"[bench] decode B=1: steps {args.decode_steps}", file=sys.stderr, flush=True)
        dec["batch_1"] = bench_decode(args, torch, lt, synth, B=1)
    configs = None
    if not args.no_configs:
        configs = bench_configs(args, torch, lt, synth)
    td = None
    if not args.no_time_dep:
        print("[bench] data-dependent decay variant, prefill 512K", file=sys.stderr, flush=True)
        td = bench_time_dependent(args, torch, lt, synth, pre)
    layer = None
    if not args.no_layer:
        print(f"[bench] layer prefill 512K: warmup {args.warmup}, steps {args.layer_steps}",
              file=sys.stderr, flush=True)
        layer = bench_layer(args, torch, lt, synth)
        if not args.no_decode:
            print(f"[bench] layer decode B=64: steps {args.decode_steps}", file=sys.stderr,
                  flush=True)
            layer["decode"] = bench_layer_decode(args, torch, lt, synth)
            print(f"[bench] layer decode B=1: steps {args.decode_steps}", file=sys.stderr,
                  flush=True)
            layer["decode"]["batch_1"] = bench_layer_decode(args, torch, lt, synth, B=1)
    attn = None
    if not args.no_attn:
        print(f"[bench] attention prefill 512K: warmup {args.attn_warmup}, steps {args.attn_steps}",
              file=sys.stderr, flush=True)
        attn = bench_attn(args, torch, lt, synth)
        if not args.no_decode:
            print(f"[bench] attention decode at 512K context: steps {args.attn_decode_steps}",
                  file=sys.stderr, flush=True)
            attn["decode"] = bench_attn_decode(args, torch, lt, synth)
    bwd = None
    if not args.no_backward:
        print(f"[bench] prefill backward at the 16K training shape: steps {args.bwd_steps}",
              file=sys.stderr, flush=True)
        bwd = bench_backward(args, torch, lt, synth)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args, torch, synth, pre)
        if layer is not None:
            print("[bench] cpu baseline of the layer (oracle)", file=sys.stderr, flush=True)
            layer["cpu_baseline"] = cpu_baseline_layer(args, torch, synth)
        if attn is not None:
            print("[bench] cpu baseline of the attention (oracle)", file=sys.stderr, flush=True)
            attn["cpu_baseline"] = cpu_baseline_attn(args, torch, synth)
        if bwd is not None:
            print("[bench] cpu baseline of the backward (oracle)", file=sys.stderr, flush=True)
            bwd["cpu_baseline"] = cpu_baseline_backward(args, torch, synth)
    if args.copy_mib > 0:
        print(f"[bench] calibration copy of {args.copy_mib} MiB", file=sys.stderr, flush=True)
        copy_calibration(torch, args.copy_mib)
    spec = pre["spec"]
    line = {
        "metric": METRIC,
        "value": round(pre["value"], 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "T": spec.T, "H": spec.H, "d": spec.d,
                   "chunk": pre["chunk"], "segments": pre["P"], "state": "fp32"},
        "roofline": pre["roofline"],
        "mfma": pre["mfma"],
        "step_stats": pre["step_stats"],
        "whole_call": pre["whole_call"],
        "decode": dec,
        "other_configs": configs,
        "time_dependent_decay": td,
        "layer": layer,
        "attention": attn,
        "backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
