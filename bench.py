#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer on one MI355X.

Headline workload: the gpt-oss-20b-shaped layer in the decode regime (hidden
2880, 32 experts, top-4, expert width 2880, bf16 weights ~N(0, 0.02), 16
tokens x ~N(0, 1)).  One step = one whole layer (route, permute, gate/up +
SwiGLU, down, combine) over that batch, with every input already in HBM.  The
expert weights rotate over several device copies so the 256 MB Infinity
Cache cannot serve them from one step to the next.

Prints ONE JSON line.  Besides the headline fields it carries:
  roofline      the dominant kernel (gate/up + SwiGLU) against the HBM peak:
                algorithmic bytes per launch (weights of the experts the
                routing touched) / its mean duration from HIP events on the
                launch stream; frac_of_copy relates it to hbm_copy_gbs, the
                bandwidth a plain 1 GiB copy kernel achieves on this GPU;
  ms_per_step_hip_graph  the same step replayed from a captured HIP graph;
  cpu_baseline  the CPU oracle timed on this host on the whole 16-token layer;
  secondary     the other workloads (prefill bf16 with Zipf routing, MXFP4
                decode and prefill, the 120b token sweep): us per layer,
                tokens/s and their roofline fractions; and the MXFP4
                quantiser / fake quantiser on the 20b gate/up tensor (GB/s
                against the HBM peak); and the layer backward on the 20b
                prefill config (TFLOP/s against the bf16 MFMA peak); and MXFP4
                decode with the expert weights in pinned host memory (GB/s
                against the host link).
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]

Traffic measurement (two rocprofv3 counter runs, then a summary):
  rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run -- python3 bench.py --no-secondary --no-cpu --copy-probe
  rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run -- python3 bench.py --no-secondary --no-cpu --copy-probe
  python3 bench.py --write-traffic DIR_F DIR_W OUT.json
--copy-probe adds launches of a plain elementwise copy (torch.neg on a 1 GiB
bf16 tensor: 1 GiB read, 1 GiB written) whose counter readings calibrate
the kernel's: HBM bytes = counter KiB x 1024 x (known bytes / copy's reading).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0   # dense MXFP4 MFMA
# The MX path multiplies every product twice (E2M1 weights by the hi and the lo
# E2M3 term of the activations, both at the fp4/fp6 rate), so the layer's own
# FLOPs can run at most at half the fp4 peak: the fp8 rate.
MX_TWO_TERM_PEAK_TFLOPS = FP4_PEAK_TFLOPS / 2
METRIC = "MoE-layer tokens/s + % HBM peak (decode, 16 tok) and % MFMA peak (prefill)"
MALL_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"gate_up_skinny": "mixture_experts_ffn_05_amd/csrc/ffn_skinny.hip",
                  "gate_up_skinny4": "mixture_experts_ffn_05_amd/csrc/ffn_skinny.hip",
                  "gate_up_tiled": "mixture_experts_ffn_05_amd/csrc/ffn_tiled.hip",
                  "mxfp4_quantize": "mixture_experts_ffn_05_amd/csrc/quant.hip"}
TRAFFIC_FILES = {"gate_up_skinny": "skinny_gate_up_bf16_20b_decode_traffic.json",
                 "gate_up_skinny4": "skinny4_gate_up_mxfp4_packed_20b_decode_traffic.json",
                 "mxfp4_quantize": "mxfp4_quantize_20b_gate_up_traffic.json"}
# per counter summary: kernel-name pattern, workload, and the bench arguments of the counter runs
TRAFFIC_RUNS = {
    "gate_up_skinny": ("skinny_kernel<0, true>", "20b decode, 16 tokens, bf16",
                       "--steps 20 --warmup 3 --no-secondary --no-cpu --copy-probe"),
    "gate_up_skinny4": ("skinny4_kernel<2, true>", "20b MXFP4 decode, 16 tokens, weights in the packed order",
                        "--only 20b_mxfp4_decode+packed --steps 20 --warmup 3 --copy-probe"),
    "mxfp4_quantize": ("mxfp4_quant_kernel<false>", "MXFP4 quantiser on the 20b gate/up tensor [184320][2880] bf16",
                       "--only mxfp4_quantize --steps 20 --copy-probe"),
}


def source_digest(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


CSRC = "mixture_experts_ffn_05_amd/csrc"
HEADLINE_TRACE = "bench_20b_decode_kernel_stats.txt"


def sources_digest() -> str:
    """One digest over every kernel source file (a trace summary is current
    only while this matches the one it was taken on)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, CSRC)
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def summarize_trace(run_dir: str, out_path: str, title: str, command: str):
    """Text summary of a `rocprofv3 --kernel-trace --stats` run directory:
    per-kernel calls and average/min/max duration, with the command that made
    it and the digest of the kernel sources it ran."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [title, "", "command (repo root, MI355X):", "  " + command,
             f"kernel sources digest: {sources_digest()}", "",
             f"{'kernel':<72}{'calls':>8}{'avg us':>10}{'min us':>10}{'max us':>10}{'% time':>8}"]
    for r in rows:
        lines.append(f"{r['Name'][:70]:<72}{int(r['Calls']):>8}{float(r['AverageNs']) / 1e3:>10.2f}"
                     f"{float(r['MinNs']) / 1e3:>10.2f}{float(r['MaxNs']) / 1e3:>10.2f}{float(r['Percentage']):>8.2f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_mean_us(pattern: str, summary: str = HEADLINE_TRACE):
    """Average duration (us) of the kernel matching `pattern` in a committed
    trace summary, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILE_DIR, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    if f"kernel sources digest: {sources_digest()}" not in text:
        return None
    for ln in text:
        if pattern in ln:
            parts = ln[72:].split()
            return float(parts[1])
    return None


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current source of the kernel (else None)."""
    path = os.path.join(PROFILE_DIR, TRAFFIC_FILES[kernel])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


PATHS = {"auto": 0, "skinny": 1, "tiled": 2, "tiled_dequant": 3, "tiled_mx": 4}


def device_layer(layer, packed: bool = False, weights_dev=None, path: int = 0):
    """The package's DeviceLayer for a synthetic layer (synth.Layer)."""
    from mixture_experts_ffn_05_amd.layer import DeviceLayer
    c, w = layer.cfg, layer.weights
    host = {} if weights_dev is not None else dict(gate_up=w.gate_up, down=w.down, gate_up_scale=w.gate_up_scale,
                                                   down_scale=w.down_scale)
    return DeviceLayer(c.T, c.H, c.E, c.k, c.I, c.wfmt, layer.x, layer.w_router, packed=packed,
                       weights_dev=weights_dev, path=path, **host)


class Timed:
    """One workload on the device, with rotated weight copies."""

    def __init__(self, layer, n_copies: int, packed: bool = False, weights_dev=None, path: int = 0):
        import torch

        import mixture_experts_ffn_05_amd as moe
        self.torch, self.moe = torch, moe
        self.g = device_layer(layer, packed=packed, weights_dev=weights_dev, path=path)
        c = layer.cfg
        g = self.g
        self.copies = [(g.gate_up, g.down, g.gate_up_scale, g.down_scale)]
        for _ in range(n_copies - 1):
            self.copies.append(tuple(t.clone() if t is not None else None for t in self.copies[0]))
        self.weights = [moe.expert_weights(gu, dn, gus, dns) for gu, dn, gus, dns in self.copies]
        self.cfg = c
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(4096)]

    def step(self, i: int, ev=None):
        g, moe = self.g, self.moe
        w = self.weights[i % len(self.weights)]
        rec = (lambda j: ev[j].record()) if ev is not None else (lambda j: None)
        rec(0)
        moe.moe_route(g.dims, g.x, g.w_router, g.topk_idx, g.topk_w, g.ws, g.ws_bytes)
        rec(1)
        moe.moe_permute(g.dims, g.topk_idx, g.offsets, g.sorted_pairs, g.pair_rank, g.ws, g.ws_bytes)
        rec(2)
        moe.moe_gate_up(g.dims, g.x, g.offsets, g.sorted_pairs, w, g.h, g.ws, g.ws_bytes)
        rec(3)
        moe.moe_down(g.dims, g.h, g.offsets, w, g.y_sorted, g.ws, g.ws_bytes)
        rec(4)
        moe.moe_combine(g.dims, g.y_sorted, g.pair_rank, g.topk_w, g.y)
        rec(5)

    def forward(self, i: int):
        """One whole layer through the single fused entry point."""
        g = self.g
        self.moe.moe_forward(g.dims, g.x, g.w_router, self.weights[i % len(self.weights)], g.y, None, None, g.ws,
                             g.ws_bytes)

    def capture(self):
        """One HIP graph per weight copy, each holding one moe_forward."""
        torch = self.torch
        self.forward(0)
        torch.cuda.synchronize()
        self.graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        for i in range(len(self.weights)):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(gr, stream=s):
                    self.forward(i)
            self.graphs.append(gr)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def run(self, steps: int, warmup: int, graph: bool = False, repeats: int = 1):
        """Seconds per layer step (moe_forward, eager launches or a HIP graph
        replay of the same launches), inputs resident in HBM: `warmup` untimed
        steps, then `repeats` windows of exactly `steps` steps, each
        bracketed by device synchronisations; the median window.  The
        per-window figures are kept in self.windows."""
        import statistics
        torch = self.torch
        if graph:
            self.capture()
            go = lambda i: self.graphs[i % len(self.graphs)].replay()  # noqa: E731
        else:
            go = self.forward
        for i in range(warmup):
            go(i)
        self.windows = []
        for _ in range(repeats):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                go(i)
            torch.cuda.synchronize()
            self.windows.append((time.perf_counter() - t0) / steps)
        return statistics.median(self.windows)

    def stages(self, steps: int, warmup: int = 3):
        """Mean microseconds of each stage entry point, from HIP events
        recorded on the stream the kernels are launched on (torch's current
        stream, which the binding passes to the library)."""
        for i in range(warmup):
            self.step(i)
        n = min(steps, len(self.ev))
        for i in range(n):
            self.step(i, self.ev[i])
        self.torch.cuda.synchronize()
        sums = [0.0] * 5
        for i in range(n):
            e = self.ev[i]
            for j in range(5):
                sums[j] += e[j].elapsed_time(e[j + 1])
        return {name: 1000.0 * s / n for name, s in zip(("route", "permute", "gate_up", "down", "combine"), sums)}

    def touched_experts(self) -> int:
        off = self.g.offsets.cpu().numpy()
        return int(((off[1:] - off[:-1]) > 0).sum())


def steady_steps(step_s: float, warm_s: float = 0.06, timed_s: float = 0.06, lo: int = 3, hi: int = 100):
    """(timed steps, warmup steps) for a workload whose step takes about
    step_s seconds: the untimed warmup lasts about warm_s, so that the GPU's
    clock has settled under the load before the window opens, and the timed
    window about timed_s (a few milliseconds of prefill work is too short for
    either)."""
    n = max(lo, min(hi, math.ceil(timed_s / step_s)))
    w = max(2, min(hi, math.ceil(warm_s / step_s)))
    return n, w


def layer_bytes(cfg, touched: int):
    """Algorithmic HBM bytes of one layer step and of the gate/up kernel:
    the weights of the experts the routing touched (each read once), the
    router, and x in / y out."""
    if cfg.wfmt == 0:
        per_w = 2.0
    else:
        per_w = 0.5 + 1.0 / 32.0  # E2M1 nibble + one E8M0 byte per 32
    gate_up = touched * 2 * cfg.I * cfg.H * per_w
    down = touched * cfg.H * cfg.I * per_w
    rest = cfg.E * cfg.H * 2 + 2 * cfg.T * cfg.H * 2
    return gate_up + down + rest, gate_up


def layer_flops(cfg):
    """Algorithmic FLOPs: 2*P*3*H*I for the experts + 2*T*E*H for the router."""
    P = cfg.T * cfg.k
    return 2.0 * P * 3 * cfg.H * cfg.I + 2.0 * cfg.T * cfg.E * cfg.H, 2.0 * P * 2 * cfg.I * cfg.H


def prefill_record(cfg, sec, stages, mx: bool):
    """A prefill line: tokens/s, us, TFLOP/s of the layer's own FLOPs, and the
    fractions of the peaks that bound it (bf16 MFMA; for the MX kernel also
    the fp4 peak and its two-term ceiling, half of it)."""
    fl, fl_gu = layer_flops(cfg)
    tf = fl / sec / 1e12
    rec = {"kernel": ("MX matrix cores, E2M1 weights x two E2M3 activation terms" if mx
                      else "bf16 MFMA" + (" (E2M1 decoded to bf16 in LDS)" if cfg.wfmt else "")),
           "tokens_per_s": round(cfg.T / sec, 1), "us_per_layer": round(sec * 1e6, 1), "tflops": round(tf, 2),
           "mfma_bf16_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    if cfg.wfmt:
        rec["mfma_fp4_frac"] = round(tf / FP4_PEAK_TFLOPS, 4)
    if mx:
        rec["mx_two_term_frac"] = round(tf / MX_TWO_TERM_PEAK_TFLOPS, 4)
    rec["gate_up_tflops"] = round(fl_gu / (stages["gate_up"] * 1e-6) / 1e12, 2)
    rec["stages_us"] = {k: round(v, 1) for k, v in stages.items()}
    return rec


def n_copies_for(cfg, touched_bytes):
    return max(4, min(16, int(4 * MALL_BYTES // max(touched_bytes, 1)) + 1))


def bench_decode(layer, steps, warmup, graph=False, packed=False, weights_dev=None, repeats=1):
    import torch
    probe = Timed(layer, 1, packed, weights_dev)
    probe.step(0)
    torch.cuda.synchronize()
    touched = probe.touched_experts()
    total_b, gu_b = layer_bytes(layer.cfg, touched)
    del probe
    tm = Timed(layer, n_copies_for(layer.cfg, total_b), packed, weights_dev)
    sec = tm.run(steps, warmup, graph, repeats)
    stages = tm.stages(steps)
    return tm, sec, stages, touched, total_b, gu_b


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown CPU")
    except OSError:
        return "unknown CPU"


def _time_oracle(fn, min_seconds: float, max_runs: int = 20):
    """Runs fn until min_seconds have passed (at least once); (runs, seconds)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or runs >= max_runs:
            return runs, el


def cpu_baseline(layer, min_seconds: float = 8.0, prefill_tokens: int = 64):
    """The fp64 C oracle, as it stands, on this host's cores:
      - the whole decode layer (headline workload) on all the cores the oracle's
        OpenMP runtime uses, and on one core;
      - the two prefill configs (8192-token Zipf bf16, 32768-token MXFP4): the
        router over all tokens, then the expert FFN and combine of a seeded
        sample of `prefill_tokens` tokens (every token's output depends on that
        token alone), extrapolated to the whole batch (labelled as such)."""
    import numpy as np

    import oracle
    import synth
    orc = oracle.get()
    cores = orc.max_threads()
    c = layer.cfg
    tokens = np.arange(c.T, dtype=np.int32)
    fwd = lambda thr: orc.forward_tokens(layer.x, layer.w_router, layer.weights, c.k, c.I, tokens,  # noqa: E731
                                         threads=thr)
    runs, el = _time_oracle(lambda: fwd(cores), min_seconds)
    runs1, el1 = _time_oracle(lambda: fwd(1), 0.0, 1)
    out = {"value": round(runs * c.T / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": f"the whole {c.T}-token decode layer ({c.T * c.k} expert pairs), fp64 C oracle, {runs} run(s) "
                     f"on {cores} threads, {el:.1f} s",
           "single_core": {"value": round(runs1 * c.T / el1, 3), "unit": "tokens/s", "cores": 1,
                           "sample": f"the same layer on one thread, {runs1} run(s), {el1:.1f} s"}}
    for name in ("20b_prefill_zipf", "20b_mxfp4_prefill"):
        pl = synth.make_layer(name)
        pc = pl.cfg
        t0 = time.perf_counter()
        orc.route(pl.x, pl.w_router, pc.k, threads=cores)
        t_route = time.perf_counter() - t0
        sub = synth.sample_tokens(pc.T, prefill_tokens, pc.seed + 1)
        t0 = time.perf_counter()
        orc.forward_tokens(pl.x, pl.w_router, pl.weights, pc.k, pc.I, sub, threads=cores)
        t_sub = time.perf_counter() - t0
        per_tok = t_sub / len(sub)
        out[name] = {"route_all_tokens_s": round(t_route, 2), "subset_tokens": len(sub), "subset_s": round(t_sub, 2),
                     "us_per_token": round(per_tok * 1e6, 1),
                     "extrapolated_tokens_per_s": round(1.0 / per_tok, 3),
                     "extrapolated_us_per_layer": round(per_tok * pc.T * 1e6 + t_route * 1e6, 0),
                     "cores": cores, "note": "expert FFN time extrapolated from the sample to all "
                                             f"{pc.T} tokens; router timed on all tokens"}
        del pl
    return out


COPY_PROBE_BYTES = 1 << 30
COPY_KERNEL_KEY = "neg"


def copy_probe(reps: int = 5):
    """Launches of a plain copy kernel of known size, for counter calibration."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def copy_bandwidth(reps: int = 10) -> float:
    """Achievable HBM bandwidth (GB/s) of a plain elementwise copy kernel
    (torch.neg over a 1 GiB bf16 tensor: 1 GiB read + 1 GiB written), timed
    with HIP events: the measured counterpart of the datasheet peak."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * COPY_PROBE_BYTES / sec / 1e9, 1)


def _counter_means(run_dir: str, counter: str):
    """Mean per-dispatch value of one counter for each kernel name in a
    rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {k: sum(v) / len(v) for k, v in out.items()}


DOMINANT_KERNEL = "skinny_kernel<0, true>"  # gate/up + SwiGLU, bf16 weights, skinny regime


def write_traffic(fetch_dir: str, write_dir: str, out_path: str, kernel: str = "gate_up_skinny"):
    """HBM bytes per launch of a kernel (the dominant one by default) from
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the factor
    that maps the copy kernel's reading onto its known bytes."""
    pattern, workload, run_args = TRAFFIC_RUNS[kernel]
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        means = _counter_means(d, counter)
        copy = [v for k, v in means.items() if COPY_KERNEL_KEY in k]
        kern = [v for k, v in means.items() if pattern in k]
        if not copy or not kern:
            raise SystemExit(f"{counter}: kernels not found in {d}: {sorted(means)}")
        factor = COPY_PROBE_BYTES / (copy[0] * 1024.0)
        res[counter] = {"kernel_kib_per_dispatch": kern[0], "copy_kib_per_dispatch": copy[0],
                        "copy_known_bytes": COPY_PROBE_BYTES, "scale": factor,
                        "bytes_per_launch": kern[0] * 1024.0 * factor}
    rec = {"kernel": "moe::" + pattern, "workload": workload,
           "source": KERNEL_SOURCES[kernel], "source_sha256_16": source_digest(KERNEL_SOURCES[kernel]),
           "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d FETCH_DIR -o run -- python3 bench.py "
                        f"{run_args}",
                        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d WRITE_DIR -o run -- python3 bench.py "
                        f"{run_args}",
                        f"python3 bench.py --write-traffic FETCH_DIR WRITE_DIR OUT.json --traffic-kernel {kernel}"],
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "hbm_bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def bench_quantize(steps: int):
    """MXFP4 quantiser and fake quantiser on the 20b gate/up tensor
    ([32*5760][2880] bf16 ~N(0, 0.02), drawn on the device from a seeded
    generator; 1.06 GB, beyond the Infinity Cache).  Algorithmic bytes per
    element: 2 read + 1/2 + 1/32 written (quantise), 2 + 2 (fake quantise)."""
    import torch

    import mixture_experts_ffn_05_amd as moe
    rows, cols = 32 * 5760, 2880
    n = rows * cols
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    w = (torch.randn((rows, cols), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    fq = torch.empty_like(w)
    calls = {"quantize": (lambda: moe.moe_mxfp4_quantize(rows, cols, w, packed, scales), n * (2 + 0.5 + 1 / 32)),
             "fakequant": (lambda: moe.moe_mxfp4_fakequant(rows, cols, w, fq), n * 4.0)}
    out = {"tensor": f"[{rows}][{cols}] bf16"}
    reps = max(10, steps // 10)
    for name, (fn, nbytes) in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        out[name] = {"us": round(sec * 1e6, 1), "gbs": round(nbytes / sec / 1e9, 1),
                     "hbm_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(nbytes)}
    del w, packed, scales, fq
    torch.cuda.empty_cache()
    return out


def bench_backward(steps: int, name: str = "20b_prefill_zipf"):
    """moe_backward (forward recompute + all gradients) on a prefill config,
    dy ~ N(0, 1) bf16.  FLOP count: the six expert GEMMs, 18 * P * H * I
    (forward recompute 6, data gradients 6, weight gradients 6)."""
    import numpy as np
    import torch

    import mixture_experts_ffn_05_amd as moe
    import synth
    from mixture_experts_ffn_05_amd.layer import to_dev
    layer = synth.make_layer(name)
    c = layer.cfg
    P = c.T * c.k
    d = moe.dims(c.T, c.H, c.E, c.k, c.I)
    nbytes = moe.moe_backward_workspace_size(d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x, wr = to_dev(layer.x), to_dev(layer.w_router)
    gu, dn = to_dev(layer.weights.gate_up), to_dev(layer.weights.down)
    W = moe.expert_weights(gu, dn)
    dy = to_dev(synth.bf16_from_f32(np.random.default_rng(c.seed + 9).standard_normal((c.T, c.H))
                                    .astype(np.float32)))
    dx = torch.empty((c.T, c.H), dtype=torch.int16, device="cuda")
    dwr = torch.empty((c.E, c.H), dtype=torch.float32, device="cuda")
    dgu = torch.empty((c.E, 2 * c.I, c.H), dtype=torch.float32, device="cuda")
    ddn = torch.empty((c.E, c.H, c.I), dtype=torch.float32, device="cuda")
    call = lambda: moe.moe_backward(d, x, wr, W, dy, dx, dwr, dgu, ddn, ws, nbytes)  # noqa: E731
    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    reps, warm = steady_steps(time.perf_counter() - t0)
    for _ in range(warm):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    fl = 18.0 * P * c.H * c.I
    out = {"workload": name, "tokens": c.T, "us_per_backward": round(sec * 1e6, 1),
           "tokens_per_s": round(c.T / sec, 1), "tflops": round(fl / sec / 1e12, 2),
           "mfma_bf16_frac": round(fl / sec / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del ws, x, wr, gu, dn, dy, dx, dwr, dgu, ddn
    torch.cuda.empty_cache()
    return out


HOST_LINK_GBS = 64.0  # PCIe Gen5 x16, one direction


def bench_host_weights(name: str = "20b_mxfp4_decode", reps: int = 5, packed: bool = False):
    """Decode with the expert weights in pinned host memory (mapped; the skinny
    kernels read only the touched experts' rows over the host link): us per
    layer and GB/s of touched weight bytes against the link's peak.  packed:
    MXFP4 weights in the packed order (reordered on the device, then copied to
    the host)."""
    import torch

    import mixture_experts_ffn_05_amd as moe
    import synth
    from mixture_experts_ffn_05_amd.host_weights import pinned_weights
    layer = synth.make_layer(name)
    g = device_layer(layer, packed=packed)
    host = [t.cpu().numpy() for t in (g.gate_up, g.down)]  # the device's (possibly packed) bytes
    if g.gate_up_scale is not None:
        host += [g.gate_up_scale.cpu().numpy(), g.down_scale.cpu().numpy()]
    parts = pinned_weights(*host)
    if parts is None:
        return {"workload": name, "skipped": "pinned host memory not mapped"}
    ptrs = [p.dev for p in parts] + [None, None]
    g.weights = moe.expert_weights(ptrs[0], ptrs[1], ptrs[2], ptrs[3])
    g.forward()
    torch.cuda.synchronize()
    touched = int(torch.unique(g.topk_idx).numel())  # moe_forward writes the routing when asked
    total_b, gu_b = layer_bytes(layer.cfg, touched)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.forward()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del g, parts
    torch.cuda.empty_cache()
    return {"workload": name + (" (packed order)" if packed else ""), "us_per_layer": round(sec * 1e6, 1),
            "touched_experts": touched,
            "gbs": round(total_b / sec / 1e9, 2), "link_peak_gbs": HOST_LINK_GBS,
            "link_frac": round(total_b / sec / 1e9 / HOST_LINK_GBS, 4), "gate_up_bytes": int(gu_b)}


def library_gemm_tflops(M: int = 32768, K: int = 2880, N: int = 5760, reps: int = 10) -> float:
    """Dense bf16 GEMM of the library torch dispatches to (hipBLASLt/rocBLAS)
    on random N(0, 1) data with the grouped gate/up's FLOP count (all pairs x
    one expert's 2I x H): the achievable-MFMA reference point."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((K, N), generator=g, device="cuda").to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.mm(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b, c
    torch.cuda.empty_cache()
    return round(2.0 * M * K * N / sec / 1e12, 2)


def library_mxfp8_gemm_tflops(M: int = 32768, K: int = 2944, N: int = 5760, reps: int = 10):
    """The library's block-scaled GEMM on MX operands, as the reference point
    for the MX kernel: torch's scaled matmul (hipBLASLt) with E4M3 x E4M3 and
    one E8M0 scale per 32 along K, on random N(0, 1) data, at the grouped
    gate/up's shape with K rounded up to the multiple of 128 it requires
    (2880 -> 2944).  MXFP8 issues at the fp8 rate, the same as one product of
    the MX kernel's two fp6 x fp4 terms.  This torch has no MXFP4 (E2M1 with
    E8M0 per 32) scaled matmul.  Returns (TFLOP/s or None, note)."""
    import torch
    try:
        g = torch.Generator(device="cuda")
        g.manual_seed(12)
        a = torch.randn((M, K), generator=g, device="cuda").to(torch.float8_e4m3fn)
        b = torch.randn((N, K), generator=g, device="cuda").to(torch.float8_e4m3fn)
        kb = (K // 32 + 3) // 4 * 4  # scale columns, padded as the library's blocked layout wants
        sa = torch.full((M * kb,), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
        sb = torch.full((N * kb,), 127, dtype=torch.uint8, device="cuda").view(torch.float8_e8m0fnu)
        fn = lambda: torch._scaled_mm(a, b.t(), sa, sb, out_dtype=torch.bfloat16)
        for _ in range(3):
            c = fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        del a, b, c, sa, sb
        torch.cuda.empty_cache()
        return round(2.0 * M * K * N / sec / 1e12, 2), f"[{M}x{K}]x[{K}x{N}] MXFP8, scales all 1"
    except Exception as e:  # an older library without block-scaled MX support
        return None, f"not available: {type(e).__name__}: {str(e)[:200]}"


def progress(what: str):
    """One line on stderr as each part of a long run starts (the JSON line
    stays alone on stdout)."""
    print(f"[bench] {what}", file=sys.stderr, flush=True)


def secondary(steps, graph=False):
    import synth
    out = {}
    progress("secondary: library dense GEMM")
    out["library_dense_gemm_bf16_tflops"] = library_gemm_tflops()
    out["library_dense_gemm_mxfp8_tflops"], out["library_dense_gemm_mxfp8_note"] = library_mxfp8_gemm_tflops()
    # prefill regimes: MFMA-bound.  MXFP4 runs on the MX kernel (the default
    # tiled path) and, as "+dequant", on the bf16-decode kernel.
    import mixture_experts_ffn_05_amd as moe
    for name in ("20b_prefill_zipf", "20b_mxfp4_prefill", "20b_mxfp4_prefill+packed"):
        progress(f"secondary: {name}")
        layer = synth.make_layer(name.split("+")[0])
        mx = layer.cfg.wfmt != 0
        for suffix, path in ([("", moe.MOE_PATH_AUTO), ("+dequant", moe.MOE_PATH_TILED_DEQUANT)] if mx
                             else [("", moe.MOE_PATH_AUTO)]):
            tm = Timed(layer, 1, name.endswith("+packed"), path=path)
            n, w = steady_steps(tm.run(1, 1))
            sec = tm.run(n, w)
            stages = tm.stages(n, w)
            out[name + suffix] = prefill_record(layer.cfg, sec, stages, mx and not suffix)
            del tm
        del layer
    # decode regimes: HBM-bound
    # MXFP4 decode in the row-major order and in the packed order (moe_mxfp4_pack)
    for packed in (False, True):
        progress("secondary: 20b_mxfp4_decode" + ("+packed" if packed else ""))
        layer = synth.make_layer("20b_mxfp4_decode")
        # the headline's protocol: median of 5 windows of `steps` steps (one short window read 2-6% high
        # right after the prefill lines)
        tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, steps, 20, graph, packed, repeats=5)
        rec = {"tokens_per_s": round(layer.cfg.T / sec, 1), "us_per_layer": round(sec * 1e6, 1),
               "touched_experts": touched, "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
               "stages_us": {k: round(v, 1) for k, v in stages.items()}}
        if packed:  # the gate/up kernel's measured HBM traffic against its algorithmic bytes
            rec["gate_up_algorithmic_bytes"] = int(gu_b)
            rec["gate_up_traffic_bytes"] = measured_traffic("gate_up_skinny4")
        out["20b_mxfp4_decode" + ("+packed" if packed else "")] = rec
        del tm, layer
    progress("secondary: 120b sweep")
    base = synth.CONFIGS["120b_sweep"]
    w120 = synth.make_weights(base)
    sweep = {}
    for T in synth.SWEEP_120B:
        cfg = base.with_T(T)
        layer = synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg), w120)
        tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, steps, 20, graph, repeats=3)
        sweep[str(T)] = {"us_per_layer": round(sec * 1e6, 1), "touched_experts": touched,
                         "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
                         "gate_up_us": round(stages["gate_up"], 1)}
        del tm, layer
    out["120b_sweep"] = sweep
    del w120
    # the 120b shape with MXFP4 expert weights in the packed order (the pages' 120b is MXFP4)
    import torch
    progress("secondary: 120b MXFP4 sweep")
    cfg4 = synth.CONFIGS["120b_mxfp4_sweep"]
    w4 = synth.make_weights(cfg4)
    sweep = {}
    for T in synth.SWEEP_120B:
        cfg = cfg4.with_T(T)
        layer = synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg), w4)
        tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, steps, 20, graph, True, repeats=3)
        sweep[str(T)] = {"us_per_layer": round(sec * 1e6, 1), "touched_experts": touched,
                         "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
                         "gate_up_us": round(stages["gate_up"], 1)}
        del tm, layer
    del w4
    torch.cuda.empty_cache()
    out["120b_mxfp4_packed_sweep"] = sweep
    progress("secondary: MXFP4 quantiser")
    out["mxfp4_quantize_20b_gate_up"] = bench_quantize(steps)
    out["backward_20b_prefill_zipf"] = bench_backward(steps)
    progress("secondary: host-resident weights")
    out["host_weights_20b_mxfp4_decode"] = bench_host_weights("20b_mxfp4_decode")
    out["host_weights_20b_mxfp4_decode+packed"] = bench_host_weights("20b_mxfp4_decode", packed=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed windows of --steps steps each; the headline is their median")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help="also launch a copy kernel of known size")
    ap.add_argument("--graph", action="store_true", help="replay each layer step as a captured HIP graph")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"))
    ap.add_argument("--summarize-trace", nargs=4, metavar=("RUN_DIR", "OUT_TXT", "TITLE", "COMMAND"),
                    help="write a text summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--traffic-kernel", default="gate_up_skinny", choices=sorted(TRAFFIC_RUNS),
                    help="which kernel --write-traffic summarises")
    ap.add_argument("--path", default="auto", choices=sorted(PATHS),
                    help="expert-FFN schedule for --only (auto, skinny, tiled, tiled_dequant, tiled_mx)")
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="time just this synthetic workload (e.g. 20b_prefill_zipf) for --steps layer steps and "
                         "print its line; for profiling one regime")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic, kernel=args.traffic_kernel)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_05_amd as moe
    import synth
    moe.library()
    torch.cuda.set_device(0)

    if args.only == "host_weights":
        print(json.dumps([bench_host_weights("20b_mxfp4_decode"), bench_host_weights("20b_decode")]))
        return
    if args.only == "backward":
        print(json.dumps(bench_backward(args.steps)))
        return
    if args.only == "mxfp4_quantize":
        rec = {"workload": args.only, **bench_quantize(args.steps)}
        rec["traffic_bytes_per_launch"] = measured_traffic("mxfp4_quantize")
        if args.copy_probe:
            copy_probe()
        print(json.dumps(rec))
        return
    if args.only:  # "<config>" or "<config>+packed" (MXFP4 weights in the packed order)
        layer = synth.make_layer(args.only.split("+")[0])
        packed = args.only.endswith("+packed")
        if layer.cfg.T <= 64:  # decode: rotated weight copies, as in the decode lines of the full run
            tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, args.steps, args.warmup, False, packed,
                                                                   repeats=args.repeats)
            if args.copy_probe:
                copy_probe()
            print(json.dumps({"workload": args.only, "tokens": layer.cfg.T, "steps": args.steps,
                              "us_per_layer": round(sec * 1e6, 1), "tokens_per_s": round(layer.cfg.T / sec, 1),
                              "touched_experts": touched, "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
                              "stages_us": {k: round(v, 1) for k, v in stages.items()}}))
            return
        tm = Timed(layer, 1, packed, path=PATHS[args.path])
        sec = tm.run(args.steps, args.warmup)
        stages = tm.stages(args.steps, 1)
        mx = layer.cfg.wfmt != 0 and args.path in ("auto", "tiled", "tiled_mx")
        print(json.dumps({"workload": args.only, "path": args.path, "tokens": layer.cfg.T, "steps": args.steps,
                          **prefill_record(layer.cfg, sec, stages, mx)}))
        return

    layer = synth.make_layer("20b_decode")
    c = layer.cfg
    tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, args.steps, args.warmup, args.graph,
                                                           repeats=args.repeats)
    windows = [round(w * 1e3, 4) for w in tm.windows]
    gu_us = stages["gate_up"]
    achieved = gu_b / (gu_us * 1e-6) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(c.T / sec, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "ms_per_step_windows": windows,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) random-init weights; no checkpoint)",
        "config": {"workload": "gpt-oss-20b-shaped MoE layer, decode: hidden 2880, 32 experts, top-4, expert width "
                               "2880, 16 tokens, bf16 weights",
                   "tokens": c.T, "hidden": c.H, "experts": c.E, "top_k": c.k, "expert_width": c.I,
                   "touched_experts": touched, "weight_copies_rotated": len(tm.weights), "parallelism": "none (1 GPU)",
                   "launch": "hip_graph" if args.graph else "eager"},
        "hbm_frac_layer": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
        "layer_gbs": round(total_b / sec / 1e9, 1),
        "stages_us": {k: round(v, 2) for k, v in stages.items()},
        "roofline": {"kernel": "moe::" + DOMINANT_KERNEL + " (gate/up + SwiGLU)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gate_up_skinny"),
                     "algorithmic_bytes_per_launch": gu_b, "mean_launch_us": round(gu_us, 2),
                     "mean_launch_us_source": "HIP events around the launch on its stream, this run",
                     "mean_launch_us_trace": trace_mean_us(DOMINANT_KERNEL),
                     "trace_summary": "profiles/" + HEADLINE_TRACE},
    }
    # the same layer step replayed from a captured HIP graph, for reference (eager launches are the headline)
    sec_other = tm.run(args.steps, args.warmup, graph=not args.graph)
    rec["ms_per_step_" + ("eager" if args.graph else "hip_graph")] = round(sec_other * 1e3, 4)
    rec["hbm_copy_gbs"] = copy_bandwidth()
    rec["roofline"]["frac_of_copy"] = round(achieved / rec["hbm_copy_gbs"], 4)
    if not args.no_secondary:
        tm = None
        torch.cuda.empty_cache()
        rec["secondary"] = secondary(args.steps, args.graph)
    if not args.no_cpu:
        progress("cpu baseline (the oracle on the host cores)")
        rec["cpu_baseline"] = cpu_baseline(layer)
    if args.copy_probe:
        tm = None
        copy_probe()
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
