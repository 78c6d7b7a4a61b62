#!/usr/bin/env python3
"""Throughput of the MoE FFN layer forward on one MI355X.

A step is one full layer forward (router top-k, regroup, int4 gate/up GEMM
with SwiGLU, down GEMM, combine) over one batch of the workload.  Prints ONE
JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--config mixtral_decode] [--sub-configs auto|none|a,b]

Inputs are seeded synthetic layers (synth package) resident in HBM before
timing starts.  The steps run as replays of one HIP graph that holds several
consecutive layers back to back, as a model's decode-step graph would, each
layer with its own copy of the weight pool, so that a step never finds the
previous step's weights in the 256 MB MALL (a model's successive layers have
different weights).  The graph's length divides K, so the timed region is
exactly K layer steps; the W warm-up steps are whole replays plus single
layers.  The headline `value` is the --config workload; the line's `configs`
holds the same record for each of the five BASELINE workloads.

Extra modes for counter runs:
    --copy-calibration   time a plain 1 GiB device copy (scale for FETCH/WRITE_SIZE)
    --refill             time expert uploads into pool slots, alone and beside the steps
    --summarize-pmc DIR  fold a rocprofv3 --pmc output directory into a JSON summary
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; HBM GB/s (T=16 decode), MFMA util (T=2048 prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
DECODE_BOUND = {"mixtral_decode": "hbm", "phi35_skew": "hbm", "fine_decode": "hbm", "tiny": "hbm",
                "fine_tiny": "hbm", "mixtral_prefill": "mfma", "fine_prefill": "mfma",
                "shared_decode": "hbm", "shared_prefill": "mfma", "shared_tiny": "hbm", "fine_shared_tiny": "hbm",
                "mixtral_decode_q4g128": "hbm", "mixtral_decode_q8g128": "hbm", "phi35_skew_q8": "hbm",
                "mixtral_prefill_q4g128": "mfma", "mixtral_prefill_q8g128": "mfma"}
CSRC = os.path.join(ROOT, "expert_ffn_layer_router_amd", "csrc")
STREAM_MAX_TOKENS = 64   # the library's decode (weight-streaming) family runs up to this T
FUSED_COMBINE_MAX_T = 8  # up to this T its down kernel's last blocks also run the combine


def dense_decode(shape) -> bool:
    """Whether the library runs dense tiles for this shape (the rule of its
    plan): per-row int4 weights, at most 16 tokens, and an expert left without
    routed rows rare -- (1 - k/E)^T <= 0.02 over the routed experts -- and
    T E <= 1024.  The router then runs in the gate/up launch."""
    T, E, k = shape.T, shape.num_experts, shape.top_k
    return (shape.bits == 4 and not shape.group and 0 < T <= 16 and (1.0 - k / E) ** T <= 0.02
            and T * E <= 1024)


def kernel_of_stage(stage, T, dense=False):
    """Name prefix of the kernel that runs a GEMM stage for T tokens."""
    if T <= STREAM_MAX_TOKENS:
        if dense and stage == "gate_up":
            return "stream_gemm_router_kernel"
        return {"gate_up": "stream_gemm_kernel<true", "down": "stream_gemm_kernel<false"}[stage]
    return {"gate_up": "prefill_gemm_kernel<true", "down": "prefill_gemm_kernel<false"}[stage]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha() -> str:
    """Hash of all kernel sources."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as fh:
                h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


# Sources that decide what a GEMM family's kernels read and write: the kernel
# file, its headers, the plan (splits, tile sizes) and the row tiles it is given.
GEMM_FAMILY_SOURCES = {
    family: [os.path.join(CSRC, f) for f in (f"{family}.hip", "device_common.h", "plan.h", "regroup.h", "moe_api.hip")
             + extra]
    + [os.path.join(ROOT, "include", "moe.h")]
    for family, extra in (("stream_gemm", ("router_small.h",)), ("prefill_gemm", ()))
}


def family_sha(family: str) -> str:
    """Hash of one GEMM family's sources: its counter summaries stay valid while it is unchanged."""
    h = hashlib.sha256()
    for path in GEMM_FAMILY_SOURCES[family]:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------- work accounting
def algorithmic_work(shape, counts):
    """Bytes and FLOPs the method itself must move / compute for one forward,
    per kernel and for the layer (active experts only; no tile padding).
    Shared experts count as experts with T rows each; `counts` covers them."""
    d, f, T, ns = shape.d_model, shape.d_ff, shape.T, shape.num_shared
    k, E = shape.top_k + ns, shape.num_experts          # rows per token; routed experts
    R = T * k
    active = int(sum(1 for c in counts if c > 0))
    bits, G = shape.bits, shape.group
    gu_groups = d // G if G else 1                      # (s, z) per output row and group
    dn_groups = f // G if G else 1
    gate_up_w = active * (2 * f * d * bits // 8 + 2 * 2 * 2 * f * gu_groups)   # gate+up codes + fp16 s,z of both
    down_w = active * (d * f * bits // 8 + 2 * 2 * d * dn_groups)              # down codes + fp16 s,z
    gate_up_bytes = gate_up_w + 2 * T * d + 2 * R * f   # + x rows read, h written (bf16)
    down_bytes = down_w + 2 * R * f + 2 * R * d         # + h read, y written (bf16-equivalent)
    layer_bytes = gate_up_w + down_w + 2 * T * d + 2 * T * d + 4 * E * d + 4 * E + 4 * (E + ns)
    if dense_decode(shape):  # the router's inputs are read by the same launch
        gate_up_bytes += 4 * E * d + 4 * E + 4 * (E + ns)
    return dict(active=active, R=R,
                gate_up=dict(bytes=gate_up_bytes, flops=4 * R * d * f),
                down=dict(bytes=down_bytes, flops=2 * R * d * f),
                layer=dict(bytes=layer_bytes, flops=6 * R * d * f))


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(case, budget_s=15.0):
    """The oracle (fp32 BLAS, routing in fp64) as it stands, timed on the host."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        available = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        available = os.cpu_count() or 1
    shape, w = case.shape, case.weights
    kw = {a: getattr(w, a) for a in w.ARRAYS}
    n_tok = min(shape.T, 64)
    tokens = None if n_tok == shape.T else np.arange(n_tok)
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.forward(case.hidden, top_k=shape.top_k, precision="f32", tokens=tokens,
                       num_shared=shape.num_shared, bits=shape.bits, group=shape.group, **kw)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 5:
            break
    med = statistics.median(times)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.forward(case.hidden, top_k=shape.top_k, precision="f32", tokens=tokens,
                           num_shared=shape.num_shared, bits=shape.bits, group=shape.group, **kw)
            single = time.perf_counter() - t0
    except Exception:  # pragma: no cover
        single = None
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    sample = (f"{n_tok} of {shape.T} tokens of the same workload, full forward incl. dequant of the "
              f"experts they use, median of {len(times)} runs; BLAS on {threads} threads of the "
              f"{available} cores in the process's affinity mask; host CPU: {cpu}")
    res = {"value": n_tok / med, "unit": "tokens/s", "cores": threads, "host_cores_available": available,
           "kind": "oracle", "sample": sample, "seconds_per_run": med}
    if single is not None:
        res["single_thread"] = {"value": n_tok / single, "unit": "tokens/s", "seconds_per_run": single}
    return res


# --------------------------------------------------------------------------- PMC summaries
def _pmc_rows(directory):
    import csv
    per = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection*.csv"), recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                try:
                    val = float(row.get("Counter_Value", "nan"))
                except ValueError:
                    continue
                key = (row.get("Kernel_Name", ""), row.get("Counter_Name", ""))
                disp = row.get("Dispatch_Id", "")
                per.setdefault(key, {}).setdefault(disp, 0.0)
                per[key][disp] += val
    return per


def summarize_pmc(dirs, out_path, copy_dirs=(), copy_bytes=1 << 30, workload=""):
    """Mean FETCH_SIZE / WRITE_SIZE per dispatch (KiB) of every kernel in the
    rocprofv3 --pmc output directories `dirs`, and the scale that makes the
    same counters read `copy_bytes` for a plain device copy of that size."""
    kernels = {}
    for d in dirs:
        for (name, ctr), disp in _pmc_rows(d).items():
            kernels.setdefault(name, {})[ctr] = statistics.mean(disp.values())
    scale = {}
    for d in copy_dirs:
        for (name, ctr), disp in _pmc_rows(d).items():
            if "copybuffer" in name.lower():  # the runtime's device-to-device copy kernel
                v = max(disp.values())
                if v > 0:
                    # a copy reads copy_bytes and writes copy_bytes
                    scale[ctr] = copy_bytes / (v * 1024.0)
    res = {"workload": workload, "source_sha": source_sha(),
           "family_sha": {f: family_sha(f) for f in GEMM_FAMILY_SOURCES}, "copy_bytes": copy_bytes,
           "scale": scale, "kernels": kernels}
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
    return res


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from committed counter summaries, if they
    were taken on the current sources of its GEMM family; else None."""
    family = "stream_gemm" if kernel.startswith("stream_gemm") else "prefill_gemm"
    sha = family_sha(family)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_pmc.json"))):
        with open(path) as fh:
            data = json.load(fh)
        if data.get("family_sha", {}).get(family) != sha:
            continue
        sc = data.get("scale", {})
        for name, ctr in data.get("kernels", {}).items():
            if kernel in name and "FETCH_SIZE" in ctr and "WRITE_SIZE" in ctr:
                return (ctr["FETCH_SIZE"] * sc.get("FETCH_SIZE", 1.0) +
                        ctr["WRITE_SIZE"] * sc.get("WRITE_SIZE", 1.0)) * 1024.0
    return None


def copy_calibration(gib=1.0, reps=5):
    import torch
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x {reps}")


# --------------------------------------------------------------------------- main bench
def achievable_peaks(shape, torch, reps=10):
    """What simple code reaches on this GPU, a second yardstick next to the
    vendor peaks: a read-only stream of 4 GiB through the library's read probe
    (the best of three grid sizes; bytes read / time), and a dense bf16 GEMM
    shaped like the gate/up product of the workload's rows (hipBLASLt through
    torch.matmul)."""
    from expert_ffn_layer_router_amd import hbm_read_probe
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    read_gbs, best_blocks = 0.0, 0
    for blocks in (1024, 2048, 4096):
        hbm_read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            hbm_read_probe(buf, sink, blocks)
        ev1.record()
        torch.cuda.synchronize()
        gbs = n * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
        if gbs > read_gbs:
            read_gbs, best_blocks = gbs, blocks
    del buf, sink
    M = max(256, -(-shape.T * (shape.top_k + shape.num_shared) // 256) * 256)
    N, K = 2 * shape.d_ff, shape.d_model
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    ev1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * M * N * K * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e12
    return {"hbm_read_gbs": read_gbs, "hbm_read_blocks": best_blocks, "bf16_gemm_tflops": gemm_tflops,
            "bf16_gemm_shape": [M, N, K],
            "how": "4 GiB read-only stream (moe_hbm_read_probe, 256-thread blocks, best grid); "
                   "torch.matmul bf16 (hipBLASLt) of the gate/up shape"}


def step_percentiles(step, stream, torch, n=60):
    """p10 / p50 / p90 of single steps, each between its own pair of events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    with torch.cuda.stream(stream):
        for i, (e0, e1) in enumerate(evs):
            e0.record(stream)
            step(i)
            e1.record(stream)
    stream.synchronize()
    ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    return {"p10": ts[n // 10], "p50": ts[n // 2], "p90": ts[(9 * n) // 10], "n": n}


def graph_length(steps: int, max_layers: int = 32) -> int:
    """Layers per replayed graph: a divisor of `steps`, so that the timed
    region is whole replays of one graph, with at least two replays when that
    leaves graphs of 4 or more layers."""
    if steps <= 3:
        return max(1, steps)
    cap = min(max_layers, steps // 2)
    n = max(d for d in range(1, cap + 1) if steps % d == 0)
    if n < 4 and steps <= max_layers:
        n = steps
    return n


def build_layer_graph(layers, pools, outs, x, rw, rb, st, ws, stream, torch):
    """One HIP graph holding len(layers) layer forwards back to back: layer i
    with its own handle, weight pool pools[i % len(pools)] and output outs[i],
    all reading the same hidden state and sharing one workspace -- a model's
    decode-step graph, each layer with its own weights.  The handles run once
    eagerly first (outside the capture), after the work already queued on the
    current stream (the workspace's zero fill, pool copies): the library needs
    the workspace's control words at zero before its first use."""
    stream.wait_stream(torch.cuda.current_stream())

    def run_all():
        for i, L in enumerate(layers):
            L.forward(x, rw, rb, st, pools[i % len(pools)], out=outs[i], workspace=ws, stream=stream)
    run_all()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        run_all()
    stream.synchronize()
    return g


# BASELINE targets at layer level: decode shapes >= 70 % of HBM peak, prefill >= 50 % of bf16 peak
LAYER_TARGET_FRAC = {"hbm": 0.70, "mfma": 0.50}
HEADLINE_CONFIGS = ("mixtral_decode", "mixtral_prefill", "phi35_skew", "fine_decode", "fine_prefill")


def run_workload(name, steps, warmup, torch, *, mode="layers", model_layers=32, stage_timing=True,
                 pool_budget=60e9, log_prefix=""):
    """Times `steps` layer steps (after `warmup` untimed ones) of workload
    `name` and returns its record plus the objects the other bench legs reuse."""
    import synth
    from expert_ffn_layer_router_amd import DeviceWeights, MoeLayer, to_device

    case = synth.make_case(name)
    shape, w = case.shape, case.weights
    T = shape.T
    log(f"{log_prefix}workload {name}: T={T} d={shape.d_model} d_ff={shape.d_ff} E={shape.num_experts} "
        f"k={shape.top_k} shared={shape.num_shared} slots={shape.num_slots}")
    x = to_device(case.hidden).view(torch.bfloat16)
    rw = to_device(w.router_w)
    rb = None if w.router_b is None else to_device(w.router_b)
    st = to_device(w.slot_table)

    def new_layer():
        return MoeLayer(shape.d_model, shape.d_ff, shape.num_experts, shape.top_k, shape.num_slots, T,
                        num_shared=shape.num_shared, weight_bits=shape.bits, group_size=shape.group)

    probe = new_layer()
    ws = probe.new_workspace(T)
    pools = [DeviceWeights.upload(w)]
    out0 = torch.empty((T, shape.d_model), dtype=torch.bfloat16, device="cuda")
    probe.forward(x, rw, rb, st, pools[0], out=out0, workspace=ws)
    torch.cuda.synchronize()
    counts = probe.routing(ws, T)["counts"].cpu().numpy()
    work = algorithmic_work(shape, counts)
    plan_fused = T <= STREAM_MAX_TOKENS
    dense = dense_decode(shape)

    nlay = graph_length(steps, model_layers) if mode == "layers" else 1
    pool_bytes = w.nbytes()
    rot = max(1, min(nlay if mode == "layers" else model_layers, int(pool_budget // max(1, pool_bytes))))
    if rot < 2:
        log(f"{log_prefix}only one weight-pool copy fits: steps may find weights in the MALL")
    while len(pools) < rot:
        pools.append(pools[0].clone())
    log(f"{log_prefix}{work['active']} active experts, {work['layer']['bytes'] / 1e6:.1f} MB algorithmic per "
        f"step, {rot} weight-pool copies of {pool_bytes / 1e6:.1f} MB")
    stream = torch.cuda.Stream()

    if mode == "layers":
        layers = [new_layer() for _ in range(nlay)]
        outs = [torch.empty((T, shape.d_model), dtype=torch.bfloat16, device="cuda") for _ in range(nlay)]
        graph = build_layer_graph(layers, pools, outs, x, rw, rb, st, ws, stream, torch)
        with torch.cuda.stream(stream):
            graph.replay()  # set-up: the graph's first launch uploads it
        stream.synchronize()
    else:
        layers = [probe]
        outs = [out0]
        graph = None

    def eager(i):
        L = layers[i % len(layers)]
        L.forward(x, rw, rb, st, pools[i % rot], out=outs[i % len(outs)], workspace=ws, stream=stream)

    # warm-up: exactly `warmup` layer steps (whole replays, then single layers)
    with torch.cuda.stream(stream):
        if mode == "layers":
            for _ in range(warmup // nlay):
                graph.replay()
            for i in range(warmup % nlay):
                eager(i)
        else:
            for i in range(warmup):
                eager(i)
    stream.synchronize()
    torch.cuda.synchronize()

    # timed region: exactly `steps` layer steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if mode == "layers":
            for _ in range(steps // nlay):
                graph.replay()
        else:
            for i in range(steps):
                eager(i)
        ev1.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    us_per_step = 1e6 * wall / steps
    log(f"{log_prefix}{mode}: {us_per_step:.1f} us/step wall, {ev_ms / steps * 1e3:.1f} us/step events "
        f"({steps} steps, {'graphs of %d layers' % nlay if mode == 'layers' else 'eager'})")

    # kernel time: HIP events the library records between its stages, on the
    # kernels' own stream, over `steps` eager layer steps of the same layers
    stage_us = {}
    if stage_timing:
        for L in layers:
            L.set_stage_timing(-(-steps // len(layers)))
        with torch.cuda.stream(stream):
            for i in range(steps):
                eager(i)
        stream.synchronize()
        stage_sum, n_fw = {}, 0
        for L in layers:
            ms, n = L.stage_times()
            n_fw += n
            for key, v in ms.items():
                stage_sum[key] = stage_sum.get(key, 0.0) + v
            L.set_stage_timing(0)
        # few tokens: the regroup runs inside the router kernel (and up to
        # FUSED_COMBINE_MAX_T tokens the combine inside the down kernel) -- no
        # kernel of their own to time; dense tiles: the router runs inside the
        # gate/up launch
        fused = ("regroup",) if plan_fused else ()
        if T <= FUSED_COMBINE_MAX_T:
            fused += ("combine",)
        if dense:
            fused += ("router",)
        stage_us = {key: 1e3 * v / max(1, n_fw) for key, v in stage_sum.items() if key not in fused}
        log(f"{log_prefix}stage us: " + ", ".join(f"{key} {v:.1f}" for key, v in stage_us.items()))

    bound = DECODE_BOUND.get(name, "hbm")
    layer_s = us_per_step * 1e-6
    lay = work["layer"]
    rec = {"T": T, "tokens_per_s": T * steps / wall, "us_per_step": us_per_step, "steps": steps,
           "warmup": warmup, "bound": bound,
           "timing": (f"{steps // nlay} replays of a HIP graph of {nlay} layers (own weights each)"
                      if mode == "layers" else "eager launches"),
           "weight_pool_copies": rot, "active_experts": work["active"],
           "layer": {"algorithmic_bytes": lay["bytes"], "algorithmic_flops": lay["flops"],
                     "hbm_gbs": lay["bytes"] / layer_s / 1e9, "hbm_frac": lay["bytes"] / layer_s / 1e9 / HBM_PEAK_GBS,
                     "mfma_tflops": lay["flops"] / layer_s / 1e12,
                     "mfma_frac": lay["flops"] / layer_s / 1e12 / BF16_PEAK_TFLOPS},
           "stage_us": stage_us}
    rec["layer"]["frac"] = rec["layer"]["hbm_frac" if bound == "hbm" else "mfma_frac"]
    rec["layer"]["target_frac"] = LAYER_TARGET_FRAC[bound]
    rec["layer"]["meets_target"] = rec["layer"]["frac"] >= LAYER_TARGET_FRAC[bound]
    if stage_us:
        dom = max(("gate_up", "down"), key=lambda s_: stage_us[s_])
        dur_s = stage_us[dom] * 1e-6
        if bound == "hbm":
            achieved = work[dom]["bytes"] / dur_s / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS}
        else:
            achieved = work[dom]["flops"] / dur_s / 1e12
            roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS}
        roof["traffic"] = load_traffic(name, kernel_of_stage(dom, T, dense))
        roof.update({"kernel": kernel_of_stage(dom, T, dense), "kernel_us": stage_us[dom],
                     "algorithmic_bytes": work[dom]["bytes"], "algorithmic_flops": work[dom]["flops"]})
        rec["roofline"] = roof
    ctx = dict(case=case, shape=shape, layers=layers, pools=pools, stream=stream, eager=eager, graph=graph,
               nlay=nlay, ev_ms=ev_ms)
    return rec, ctx


def run_refill(args, shape, w, pools, layer, step, stream, torch):
    """Slot-pool refill: one expert's weights copied from page-locked host
    memory into a pool slot on a copy stream (moe_expert_upload), timed alone,
    and beside the layer steps on the compute stream.  The copies rewrite
    slots 0 and 1 with the experts they already hold, so the steps compute
    the same layer.  Prints one JSON line."""
    from expert_ffn_layer_router_amd import HostExpert
    d, f = shape.d_model, shape.d_ff
    expert_bytes = 3 * d * f // 2 + 2 * (4 * f + 2 * d)
    host = [HostExpert.from_pool(w, e) for e in (0, 1)]
    copy = torch.cuda.Stream()
    n_up = 8

    def uploads(n):
        for i in range(n):
            layer.upload_expert(pools[0], i % 2, host[i % 2], stream=copy)

    uploads(2)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(copy)
    uploads(n_up)
    c1.record(copy)
    torch.cuda.synchronize()
    up_alone = c0.elapsed_time(c1) / n_up
    log(f"refill: one expert ({expert_bytes / 1e6:.1f} MB) uploads in {up_alone * 1e3:.0f} us alone")

    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        s0.record(stream)
        for i in range(args.steps):
            step(i)
        s1.record(stream)
    torch.cuda.synchronize()
    step_alone = s0.elapsed_time(s1) / args.steps
    # beside the steps: enough uploads to cover the steps
    n_bg = max(2, int(step_alone * args.steps / max(up_alone, 1e-3)) + 1)
    c0.record(copy)
    uploads(n_bg)
    c1.record(copy)
    with torch.cuda.stream(stream):
        s0.record(stream)
        for i in range(args.steps):
            step(i)
        s1.record(stream)
    torch.cuda.synchronize()
    step_beside = s0.elapsed_time(s1) / args.steps
    up_beside = c0.elapsed_time(c1) / n_bg
    log(f"refill: step {step_alone * 1e3:.1f} us alone, {step_beside * 1e3:.1f} us beside uploads; "
        f"upload {up_beside * 1e3:.0f} us beside steps")
    print(json.dumps({
        "metric": "expert refill (host -> pool slot) beside layer steps", "config": {"workload": args.config},
        "expert_bytes": expert_bytes, "upload_us_alone": up_alone * 1e3,
        "upload_gbs_alone": expert_bytes / (up_alone * 1e-3) / 1e9,
        "upload_us_beside_steps": up_beside * 1e3, "upload_gbs_beside_steps": expert_bytes / (up_beside * 1e-3) / 1e9,
        "step_us_alone": step_alone * 1e3, "step_us_beside_uploads": step_beside * 1e3,
        "steps": args.steps, "uploads_beside": n_bg}))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="mixtral_decode", help="the workload of the headline value")
    ap.add_argument("--sub-configs", default="auto",
                    help="comma-separated workloads also measured into the line's `configs` ('auto': the five "
                         "BASELINE workloads; 'none': only --config)")
    ap.add_argument("--sub-steps", type=int, default=64, help="timed layer steps per sub-workload")
    ap.add_argument("--mode", choices=["layers", "eager"], default="layers",
                    help="layers: HIP graphs of consecutive layers (own weights each) replayed, as a model's "
                         "decode-step graph; eager: plain launches")
    ap.add_argument("--model-layers", type=int, default=32,
                    help="most layers per graph (Mixtral-8x7B has 32 MoE layers), each with its own weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the read-stream / library-GEMM yardsticks")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--refill", action="store_true",
                    help="time expert uploads (host -> slot) alone and beside the layer steps")
    ap.add_argument("--summarize-pmc", metavar="DIR", nargs="+", help="rocprofv3 --pmc output directories")
    ap.add_argument("--copy-pmc", metavar="DIR", nargs="*", default=[], help="--pmc runs of --copy-calibration")
    ap.add_argument("--pmc-out", metavar="JSON")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        res = summarize_pmc(args.summarize_pmc, args.pmc_out or "pmc_summary.json", args.copy_pmc,
                            workload=args.config)
        print(json.dumps(res))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              f"(--gpus {args.gpus} / WORLD_SIZE {world} is not supported)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    torch.cuda.set_device(0)
    rec, ctx = run_workload(args.config, args.steps, args.warmup, torch, mode=args.mode,
                            model_layers=args.model_layers)
    shape, stream = ctx["shape"], ctx["stream"]
    if args.refill:
        return run_refill(args, shape, ctx["case"].weights, ctx["pools"], ctx["layers"][0], ctx["eager"], stream,
                          torch)

    # single-step latency spread (one layer per replay of a one-layer graph would
    # add a graph launch per step, so these are eager single layers)
    per = step_percentiles(ctx["eager"], stream, torch)
    peaks = None
    roof = dict(rec["roofline"])
    if not args.no_peaks:
        peaks = achievable_peaks(shape, torch)
        ref = peaks["hbm_read_gbs"] if roof["bound"] == "hbm" else peaks["bf16_gemm_tflops"]
        roof["frac_of_achievable"] = roof["achieved"] / ref
        log(f"achievable: read {peaks['hbm_read_gbs']:.0f} GB/s, bf16 GEMM {peaks['bf16_gemm_tflops']:.0f} TFLOP/s")

    configs = {args.config: rec}
    subs = [c for c in (HEADLINE_CONFIGS if args.sub_configs == "auto" else
                        ([] if args.sub_configs == "none" else args.sub_configs.split(","))) if c and c != args.config]
    del ctx
    for name in subs:
        torch.cuda.empty_cache()
        sub, sctx = run_workload(name, args.sub_steps, graph_length(args.sub_steps, args.model_layers), torch,
                                 mode=args.mode, model_layers=args.model_layers, log_prefix="  ")
        del sctx
        configs[name] = sub

    result = {
        "metric": METRIC, "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["us_per_step"] * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.config, "T": shape.T, "d_model": shape.d_model, "d_ff": shape.d_ff,
                   "num_experts": shape.num_experts, "top_k": shape.top_k, "num_shared": shape.num_shared,
                   "num_slots": shape.num_slots,
                   "weights": (f"{'int4' if shape.bits == 4 else '8-bit'} codes + fp16 scale/zero-point per "
                               + ("output row" if not shape.group else f"output row and {shape.group}-input group")),
                   "timing": rec["timing"], "weight_pool_copies": rec["weight_pool_copies"],
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": dict(rec["layer"], active_experts=rec["active_experts"], stage_us=rec["stage_us"]),
        "configs": configs,
        "step_us": per,
        "achievable": peaks,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        import synth
        result["cpu_baseline"] = cpu_baseline(synth.make_case(args.config), args.cpu_budget_s)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
