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
                launch stream;
  cpu_baseline  the CPU oracle timed on this host on the whole 16-token layer;
  secondary     the other workloads (prefill bf16 with Zipf routing, MXFP4
                decode and prefill, the 120b token sweep): us per layer,
                tokens/s and their roofline fractions.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0   # dense MXFP4 MFMA
METRIC = "MoE-layer tokens/s + % HBM peak (decode, 16 tok) and % MFMA peak (prefill)"
MALL_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"gate_up_skinny": "mixture_experts_ffn_05_amd/csrc/ffn_skinny.hip",
                  "gate_up_tiled": "mixture_experts_ffn_05_amd/csrc/ffn_tiled.hip"}


def source_digest(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current source of the kernel (else None)."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


class Timed:
    """One workload on the device, with rotated weight copies."""

    def __init__(self, layer, n_copies: int):
        import torch

        import mixture_experts_ffn_05_amd as moe
        from tests.gpu_layer import GpuLayer
        self.torch, self.moe = torch, moe
        self.g = GpuLayer(layer)
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

    def run(self, steps: int, warmup: int, stage_events: bool = True):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, self.ev[i % len(self.ev)] if stage_events else None)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stages = None
        if stage_events:
            n = min(steps, len(self.ev))
            sums = [0.0] * 5
            for i in range(n):
                e = self.ev[i]
                for j in range(5):
                    sums[j] += e[j].elapsed_time(e[j + 1])
            stages = {name: 1000.0 * s / n for name, s in
                      zip(("route", "permute", "gate_up", "down", "combine"), sums)}
        return wall / steps, stages

    def touched_experts(self) -> int:
        off = self.g.offsets.cpu().numpy()
        return int(((off[1:] - off[:-1]) > 0).sum())


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


def n_copies_for(cfg, touched_bytes):
    return max(4, min(16, int(4 * MALL_BYTES // max(touched_bytes, 1)) + 1))


def bench_decode(layer, steps, warmup):
    import torch
    probe = Timed(layer, 1)
    probe.step(0)
    torch.cuda.synchronize()
    touched = probe.touched_experts()
    total_b, gu_b = layer_bytes(layer.cfg, touched)
    del probe
    tm = Timed(layer, n_copies_for(layer.cfg, total_b))
    sec, stages = tm.run(steps, warmup)
    return tm, sec, stages, touched, total_b, gu_b


def cpu_baseline(layer, min_seconds=10.0):
    import numpy as np

    import oracle
    orc = oracle.get()
    c = layer.cfg
    tokens = np.arange(c.T, dtype=np.int32)
    runs, t0 = 0, time.perf_counter()
    while True:
        orc.forward_tokens(layer.x, layer.w_router, layer.weights, c.k, c.I, tokens)
        runs += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or runs >= 20:
            break
    return {"value": round(runs * c.T / el, 3), "unit": "tokens/s", "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"the whole {c.T}-token layer ({c.T * c.k} expert pairs), fp64 C oracle, {runs} run(s), "
                      f"{el:.1f} s"}


def secondary(steps):
    import synth
    out = {}
    # prefill regimes: MFMA-bound
    for name in ("20b_prefill_zipf", "20b_mxfp4_prefill"):
        layer = synth.make_layer(name)
        tm = Timed(layer, 1)
        sec, stages = tm.run(max(3, steps // 10), 2)
        fl, fl_gu = layer_flops(layer.cfg)
        peak = BF16_PEAK_TFLOPS  # the kernels issue bf16 MFMA (MXFP4 decoded to bf16 in LDS)
        out[name] = {"tokens_per_s": round(layer.cfg.T / sec, 1), "us_per_layer": round(sec * 1e6, 1),
                     "tflops": round(fl / sec / 1e12, 2), "mfma_bf16_frac": round(fl / sec / 1e12 / peak, 4),
                     "mfma_fp4_frac": round(fl / sec / 1e12 / FP4_PEAK_TFLOPS, 4),
                     "gate_up_tflops": round(fl_gu / (stages["gate_up"] * 1e-6) / 1e12, 2),
                     "stages_us": {k: round(v, 1) for k, v in stages.items()}}
        del tm, layer
    # decode regimes: HBM-bound
    layer = synth.make_layer("20b_mxfp4_decode")
    tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, steps, 10)
    out["20b_mxfp4_decode"] = {"tokens_per_s": round(layer.cfg.T / sec, 1), "us_per_layer": round(sec * 1e6, 1),
                               "touched_experts": touched, "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
                               "stages_us": {k: round(v, 1) for k, v in stages.items()}}
    del tm, layer
    base = synth.CONFIGS["120b_sweep"]
    w120 = synth.make_weights(base)
    sweep = {}
    for T in synth.SWEEP_120B:
        cfg = base.with_T(T)
        layer = synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg), w120)
        tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, steps, 10)
        sweep[str(T)] = {"us_per_layer": round(sec * 1e6, 1), "touched_experts": touched,
                         "hbm_frac": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
                         "gate_up_us": round(stages["gate_up"], 1)}
        del tm, layer
    out["120b_sweep"] = sweep
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_05_amd as moe
    import synth
    moe.library()
    torch.cuda.set_device(0)

    layer = synth.make_layer("20b_decode")
    c = layer.cfg
    tm, sec, stages, touched, total_b, gu_b = bench_decode(layer, args.steps, args.warmup)
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) random-init weights; no checkpoint)",
        "config": {"workload": "gpt-oss-20b-shaped MoE layer, decode: hidden 2880, 32 experts, top-4, expert width "
                               "2880, 16 tokens, bf16 weights",
                   "tokens": c.T, "hidden": c.H, "experts": c.E, "top_k": c.k, "expert_width": c.I,
                   "touched_experts": touched, "weight_copies_rotated": len(tm.weights), "parallelism": "none (1 GPU)"},
        "hbm_frac_layer": round(total_b / sec / 1e9 / HBM_PEAK_GBS, 4),
        "layer_gbs": round(total_b / sec / 1e9, 1),
        "stages_us": {k: round(v, 2) for k, v in stages.items()},
        "roofline": {"kernel": "gate_up_skinny_kernel<0> (gate/up + SwiGLU)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("gate_up_skinny"),
                     "algorithmic_bytes_per_launch": gu_b, "mean_launch_us": round(gu_us, 2)},
    }
    if not args.no_secondary:
        del tm
        torch.cuda.empty_cache()
        rec["secondary"] = secondary(args.steps)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(layer)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
