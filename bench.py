#!/usr/bin/env python3
"""Throughput of the MXFP4 sparse-MoE block on one MI355X.

One step = one pass of the whole block (moe_forward: route -> permute -> expert
FFN -> combine) over one batch of T tokens whose inputs are already resident in
HBM. The headline workload is the decode-shaped gpt-oss-20b layer (T=16,
d=F=2880, E=32, top-4), bound by streaming the MXFP4 weights from HBM. Every
other workload gets a line beside it: tiny (T=128, d=F=512), prefill-20b
(T=8192, against the MXFP4 matrix-core peak), wide-120b (T=4096, E=128, skewed
router) and the 24-block pre-norm stack (T=2048 per block).

Timing protocol, per workload:
  * the weights rotate over R identical copies (R * layer bytes >= 1.5 GB) so
    the 256 MB last-level cache cannot hold them (the stack's 24 layers already
    exceed it; the tiny layer is cache-resident by nature);
  * W untimed warmup steps, then `repeats` runs of exactly K timed steps, each
    bracketed by torch.cuda.synchronize(); the line reports the median run
    (and the best), eager calls on torch's current stream;
  * beside it the same steps captured once as a HIP graph and replayed;
  * one timed step's output is checked against the CPU oracle (tiny and
    decode-20b; the larger workloads are checked element by element in the
    GPU tests).
The roofline object is the dominant kernel's, the decode gate/up GEMM
(moe_expert_ffn_mxfp4_stage 1), whose average launch duration comes from HIP
events on its launch stream around a loop of back-to-back launches over the
weight copies. The oracle is timed on the host cores as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats 5]
                       [--workloads 1,0,2,3,4] [--no-cpu-baseline]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4/MXFP6 matrix throughput, published
METRIC = "MoE layer tokens/s; % HBM peak (T=16) and % MXFP4 MFMA peak (T=8192)"


# the sources of the expert-FFN call's kernels, hashed into the traffic summary
TRAFFIC_SOURCES = ("ffn.hip", "ffn_dev.hpp", "mx6.hpp", "layout.hpp", "common.hpp")


def traffic_sources_hash(read=None) -> str:
    """First 16 hex digits of the sha256 of TRAFFIC_SOURCES concatenated, each
    with its comments removed and every run of white space made one blank, so
    that an edit of comments alone does not void a counter summary. `read`
    (file name -> text) defaults to the working tree."""
    import hashlib
    import re
    if read is None:
        def read(f):
            return open(os.path.join(ROOT, "sparse_moe_transformer_gemm_amd", "csrc", f)).read()
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        t = re.sub(r"/\*.*?\*/", " ", read(f), flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name: str, key: str = "traffic_bytes_per_launch"):
    """HBM bytes per launch (of the gate/up GEMM, or with key
    traffic_bytes_per_call of the whole expert-FFN call) from the committed
    rocprofv3 counter summary for this workload, or None when there is none or
    when the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_expert_ffn_{name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            name_, _, val = line.strip().partition(":")
            fields[name_.strip()] = val.strip()
    if traffic_sources_hash() != fields.get("sources_sha256_16") or key not in fields:
        return None
    return int(fields[key])


def gateup_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert in the gate/up GEMM: the gate and up
    MXFP4 matrices (0.5 B per element + 1 B per 32) and their bf16 biases."""
    return 2 * (d * F // 2 + d * F // 32) + 2 * 2 * F


def down_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert in the down GEMM: W_down and its bias."""
    return (d * F // 2 + d * F // 32) + 2 * d


def expert_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert: 3 MXFP4 matrices and its bf16 biases."""
    return gateup_bytes(d, F) + down_bytes(d, F)


def layer_alg(T, d, F, E, k, U, has_bias) -> tuple:
    """The layer's algorithmic bytes (touched experts' weights and biases, the
    router weight and bias, x in, out back) and flops (the three expert
    contractions); traffic the implementation adds is not credited."""
    b = U * expert_bytes(d, F) + 4 * d * E + (4 * E if has_bias else 0) + 2 * T * d + 2 * T * d
    return b, 2.0 * T * k * 3 * d * F


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5)
    ap.add_argument("--workloads", default="1,0,2,3,4",
                    help="comma list; the first is the headline (default: decode-20b)")
    ap.add_argument("--fp8", default="1,2", help="workloads also run with FP8 expert weights ('' for none)")
    ap.add_argument("--attention", default="attn-decode,attn-prefill",
                    help="attention-with-sinks workloads to time ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timings")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 passes of the library's streaming residual-add kernel "
                         "over MIB MiB per operand (reads 2 x MIB, writes MIB: a known byte "
                         "count to calibrate a profiler's HBM byte counters) and exit")
    return ap.parse_args()


def clocks() -> dict:
    """Current GPU clocks as rocm-smi reports them (not locked)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [l.strip() for l in r.stdout.splitlines() if "sclk" in l or "mclk" in l]
        return {"rocm_smi": lines[:4]}
    except Exception as e:  # rocm-smi missing or failing: say so
        return {"rocm_smi": f"unavailable ({type(e).__name__})"}


def _dev_inputs(L, dev):
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    return moe.load_expert_weights(
        w_router=torch.from_numpy(L.w_router).to(dev),
        b_router=None if L.b_router is None else torch.from_numpy(L.b_router).to(dev),
        gate_codes=u8(L.gate.codes), gate_scales=u8(L.gate.scales),
        up_codes=u8(L.up.codes), up_scales=u8(L.up.scales),
        down_codes=u8(L.down.codes), down_scales=u8(L.down.scales),
        b_gate=bf16(L.b_gate), b_up=bf16(L.b_up), b_down=bf16(L.b_down)), bf16


def xcd_tiles(counts: np.ndarray, d: int, F: int) -> dict:
    """Tiles per XCD of the two persistent prefill GEMMs for these expert row
    counts: ceil(rows / 128) row tiles per expert times the column tiles (192
    h-columns per gate/up tile, 320 output columns per down tile), the list cut
    into eight equal ranges, one per XCD, as the kernels schedule it."""
    rt = int(sum((int(c) + 127) // 128 for c in counts))
    out = {}
    for name, ntn in (("gate_up", F // 192), ("down", d // 320)):
        g = rt * ntn
        out[name] = [g // 8 + (1 if x < g % 8 else 0) for x in range(8)]
    return out


def timed_runs(step, steps, warmup, repeats) -> list:
    """ms per step of `repeats` runs of exactly `steps` calls of step(i), each
    run between torch.cuda.synchronize() calls, after `warmup` untimed calls."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3 / steps)
    return out


def graph_runs(step, per_graph, steps, repeats) -> list:
    """The same steps captured once as a HIP graph of `per_graph` calls
    (step(0) .. step(per_graph - 1)) and replayed: ms per step of `repeats` runs
    of steps // per_graph replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per_graph):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step(i)
    n = max(1, steps // per_graph)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            g.replay()
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3 / (n * per_graph))
    del g
    return out


def stage_ms(moe, x, perm, copies, k, ws, y, stage, steps, warmup) -> float:
    """Average launch duration of one expert-FFN stage launched back to back over
    the weight copies, from HIP events on the launching stream around the loop
    (each launch rewrites the same h or y from what the earlier stages left)."""
    import torch
    R = len(copies)
    for i in range(warmup):
        moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], copies[i % R], k, ws, y, stage)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record()
    for i in range(steps):
        moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], copies[i % R], k, ws, y, stage)
    g1.record()
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / steps


def run_layer(cfg: int, steps: int, warmup: int, repeats: int, graph: bool, log) -> dict:
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    w = synth.workload(cfg)
    L = w.layers[0]
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    layer_bytes = E * expert_bytes(d, F) + 4 * d * E
    R = 1 if cfg == 0 else max(1, int(np.ceil(1.5e9 / layer_bytes)))
    log(f"[bench] {w.name}: T={T} d={d} F={F} E={E} k={k}; {R} weight copies")
    copies = []
    for _ in range(R):
        wt, bf16 = _dev_inputs(L, dev)
        copies.append(wt)
    x = bf16(w.x)
    ws = torch.empty(moe.workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
    bufs = moe._outputs(T, d, E, k, x.device, None)

    def step(i):
        moe.forward(x, copies[i % R], k, ws, bufs)

    eager = timed_runs(step, steps, warmup, repeats)
    per_graph = max(R, min(steps, 8 * R))
    gr = graph_runs(step, per_graph, steps, repeats) if graph else None

    # the GEMM stages back to back, on what the earlier stages left in ws
    wt0 = copies[0]
    idx, _ = moe.route(x, wt0.w_router, wt0.b_router, k, ws, bufs["topk_idx"], bufs["topk_w"])
    perm = moe.permute(idx, E, ws, bufs["perm"])
    moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], wt0, k, ws, bufs["y_sorted"], 0)
    kst = max(10, steps // 4)
    gu_ms = stage_ms(moe, x, perm, copies, k, ws, bufs["y_sorted"], 1, kst, max(3, warmup // 4))
    dn_ms = stage_ms(moe, x, perm, copies, k, ws, bufs["y_sorted"], 2, kst, max(3, warmup // 4))

    step(0)
    torch.cuda.synchronize()
    counts = bufs["perm"][0].cpu().numpy()
    U = int((counts > 0).sum())
    out_bits = bufs["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    idx_gpu = bufs["topk_idx"].cpu().numpy()
    ms = float(np.median(eager))
    b_alg, f_alg = layer_alg(T, d, F, E, k, U, L.b_router is not None)
    gu_b, dn_b = U * gateup_bytes(d, F), U * down_bytes(d, F)
    gu_f = 2.0 * T * k * 2 * d * F
    res = dict(
        workload=w.name, T=T, d=d, F=F, E=E, k=k, seed=w.seed, weight_copies=R, experts_touched=U,
        rows_per_expert=[int(counts.min()), int(counts.max())],
        tiles_per_xcd=xcd_tiles(counts, d, F) if T > 64 else None,
        ms_per_step=ms, ms_per_step_best=float(min(eager)), ms_per_step_runs=eager,
        ms_per_step_graph=None if gr is None else float(np.median(gr)),
        ms_per_step_graph_best=None if gr is None else float(min(gr)),
        tokens_per_s=T / (ms / 1e3),
        alg_bytes=b_alg, alg_flops=f_alg,
        frac_hbm_peak=b_alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        frac_mxfp4_peak=f_alg / (ms / 1e3) / 1e12 / MXFP4_PEAK_TFLOPS,
        gate_up_gemm=dict(avg_launch_ms=gu_ms, alg_bytes=gu_b, flops=gu_f,
                          gbs=gu_b / (gu_ms / 1e3) / 1e9, tflops=gu_f / (gu_ms / 1e3) / 1e12),
        down_gemm=dict(avg_launch_ms=dn_ms, alg_bytes=dn_b, flops=gu_f / 2,
                       gbs=dn_b / (dn_ms / 1e3) / 1e9, tflops=gu_f / 2 / (dn_ms / 1e3) / 1e12),
        _out_bits=out_bits, _idx=idx_gpu, _workload=w)
    log(f"[bench] {w.name}: {ms * 1e3:.1f} us/step median of {repeats} (best {min(eager) * 1e3:.1f}"
        + ("" if gr is None else f", graph {np.median(gr) * 1e3:.1f}") + f"), {res['tokens_per_s']:.4g} tok/s, "
        f"{100 * res['frac_hbm_peak']:.1f}% HBM / {100 * res['frac_mxfp4_peak']:.1f}% MXFP4; "
        f"gate/up {gu_ms * 1e3:.1f} us, down {dn_ms * 1e3:.1f} us, U={U}")
    del copies, ws, bufs
    torch.cuda.empty_cache()
    return res


FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix throughput, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix throughput, published


def fp8_expert_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert in FP8: 3 matrices of 1 B per element, their
    float32 128x128 block scales, and the bf16 biases."""
    nb = lambda n: (n + 127) // 128
    return 3 * d * F + 4 * 3 * nb(d) * nb(F) + 2 * (2 * F + d)


def run_fp8(cfg: int, steps: int, warmup: int, repeats: int, log) -> dict:
    """The same layer with its experts converted once to FP8 with 128x128 block
    scales (moe_convert_mxfp4_to_fp8), run as the four calls moe_route,
    moe_permute, moe_expert_ffn_fp8 and moe_combine."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    w = synth.workload(cfg)
    L = w.layers[0]
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    R = max(1, int(np.ceil(1.5e9 / (E * fp8_expert_bytes(d, F)))))
    log(f"[bench] {w.name} fp8: T={T} d={d} F={F} E={E} k={k}; {R} weight copies")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    copies = [moe.fp8_from_mxfp4(
        w_router=u8(L.w_router), b_router=None if L.b_router is None else u8(L.b_router),
        gate_codes=u8(L.gate.codes), gate_scales=u8(L.gate.scales), up_codes=u8(L.up.codes),
        up_scales=u8(L.up.scales), down_codes=u8(L.down.codes), down_scales=u8(L.down.scales),
        b_gate=bf16(L.b_gate), b_up=bf16(L.b_up), b_down=bf16(L.b_down)) for _ in range(R)]
    x = bf16(w.x)
    ws = torch.empty(moe.workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
    b = moe._outputs(T, d, E, k, x.device, None)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def step(i):
        wt = copies[i % R]
        idx, tw = moe.route(x, wt.w_router, wt.b_router, k, ws, b["topk_idx"], b["topk_w"])
        perm = moe.permute(idx, E, ws, b["perm"])
        if i < steps:
            ev[i][0].record()
        y = moe.expert_ffn_fp8(x, perm[2], perm[1], wt, k, ws, b["y_sorted"])
        if i < steps:
            ev[i][1].record()
        moe.combine(y, perm[3], tw, b["out"])

    runs = timed_runs(step, steps, warmup, repeats)
    ffn_ms = float(np.median([a.elapsed_time(c) for a, c in ev]))
    ms = float(np.median(runs))
    U = int((b["perm"][0].cpu().numpy() > 0).sum())
    ffn_bytes = U * fp8_expert_bytes(d, F) + 2 * T * d
    lay_bytes = ffn_bytes + 4 * d * E + 2 * T * d
    flops = 2.0 * T * k * 3 * d * F
    res = dict(workload=f"{w.name}-fp8", T=T, weight_copies=R, experts_touched=U, ms_per_step=ms,
               ms_per_step_best=float(min(runs)), tokens_per_s=T / (ms / 1e3),
               frac_hbm_peak=lay_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
               frac_fp8_peak=flops / (ms / 1e3) / 1e12 / FP8_PEAK_TFLOPS,
               ffn_call=dict(avg_ms=ffn_ms, alg_bytes=ffn_bytes,
                             gbs=ffn_bytes / (ffn_ms / 1e3) / 1e9,
                             tflops=flops / (ffn_ms / 1e3) / 1e12),
               note="four calls (route, permute, FP8 expert FFN, combine); weights converted once "
                    "from the MXFP4 layer, exactly")
    log(f"[bench] {w.name} fp8: {ms * 1e3:.1f} us/step, {res['tokens_per_s']:.4g} tok/s, "
        f"{100 * res['frac_hbm_peak']:.1f}% HBM / {100 * res['frac_fp8_peak']:.1f}% FP8; "
        f"ffn {ffn_ms * 1e3:.1f} us = {res['ffn_call']['gbs']:.0f} GB/s")
    del copies, ws, b
    torch.cuda.empty_cache()
    return res


def attention_alg(B, Tq, S, Hq, Hkv, D, window) -> tuple:
    """(flops, bytes) of one attention call: 4 D flops per visible (query, key)
    pair (the score and the value product); K and V read once, q read and out
    written once, in bf16."""
    qpos = np.arange(Tq) + (S - Tq)
    lo = np.zeros(Tq, np.int64) if window <= 0 else np.maximum(qpos - window + 1, 0)
    pairs = int((qpos - lo + 1).sum())
    flops = 4.0 * D * pairs * B * Hq
    byts = 2 * B * S * Hkv * D * 2 + 2 * B * Tq * Hq * D * 2
    return flops, byts


def run_attention(name: str, steps: int, warmup: int, repeats: int, log) -> dict:
    """moe_attention_sink on a gpt-oss-20b-shaped attention (64 query heads over
    8 KV heads of size 64, per-head sinks): a causal prefill (bound by the bf16
    matrix cores) or batched decode against long caches (bound by HBM; the caches
    rotate over copies larger than the last-level cache)."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    c = synth.ATTN_WORKLOADS[name]
    B, Tq, S, Hq, Hkv, D, win = c["B"], c["Tq"], c["S"], c["Hq"], c["Hkv"], c["D"], c["window"]
    q, k, v, sk = synth.attention_inputs(c["seed"], B, Tq, S, Hq, Hkv, D)
    bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    flops, byts = attention_alg(B, Tq, S, Hq, Hkv, D, win)
    decode = Tq <= 64
    R = max(1, int(np.ceil(1.5e9 / byts))) if decode else 1
    qd, sd = bf(q), torch.from_numpy(sk).to(dev)
    kv = [(bf(k), bf(v)) for _ in range(R)]
    out = torch.empty_like(qd)
    n = moe.attention_workspace_bytes(B, Tq, S, Hq, Hkv, D, win)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    log(f"[bench] {name}: B={B} Tq={Tq} S={S} Hq={Hq} Hkv={Hkv} D={D}; {R} cache copies; "
        f"workspace {n} B")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def step(i):
        kk, vv = kv[i % R]
        if i < steps:
            ev[i][0].record()
        moe.attention_sink(qd, kk, vv, sd, 0.125, win, out, ws)
        if i < steps:
            ev[i][1].record()

    def call(i):
        kk, vv = kv[i % R]
        moe.attention_sink(qd, kk, vv, sd, 0.125, win, out, ws)

    runs = timed_runs(step, steps, warmup, repeats)
    eager_ms = float(np.median(runs))
    call_ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # graph replay: the launches back to back without the host's per-call work,
    # which would otherwise set the pace of a call this short
    per_graph = 2 * R if decode else 2
    graph = graph_runs(call, per_graph, steps, repeats)
    ms = float(np.median(graph))
    res = dict(workload=name, B=B, Tq=Tq, S=S, Hq=Hq, Hkv=Hkv, D=D, window=win, cache_copies=R,
               ms_per_call=ms, ms_per_call_best=float(min(graph)), eager_ms_per_call=eager_ms,
               eager_event_ms=call_ms, timing=f"median of {repeats} runs of HIP graph replays of "
               f"{per_graph} calls (caches rotating); eager launches beside it",
               alg_flops=flops, alg_bytes=byts,
               tflops=flops / (ms / 1e3) / 1e12, gbs=byts / (ms / 1e3) / 1e9)
    if decode:
        res.update(bound="hbm", frac=res["gbs"] / HBM_PEAK_GBS)
    else:
        res.update(bound="mfma", frac=res["tflops"] / BF16_PEAK_TFLOPS)
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call (graph; eager {eager_ms * 1e3:.1f}), "
        f"{res['tflops']:.1f} TFLOP/s, {res['gbs']:.0f} GB/s ({100 * res['frac']:.1f}% of the {res['bound']} peak)")
    del kv, ws, out
    torch.cuda.empty_cache()
    return res


def run_stack(cfg: int, steps: int, warmup: int, repeats: int, log) -> dict:
    """The pre-norm stack workload: per step, every block does
    x <- x + MoE(RMSNorm(x)) through the C ABI, all layers' weights resident."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    w = synth.workload(cfg, with_layers=False)
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    layers = []
    for l in range(w.n_layers):
        L = synth.stack_layer(cfg, l)
        wt, bf16 = _dev_inputs(L, dev)
        layers.append((bf16(L.gain), wt))
    log(f"[bench] {w.name}: T={T} d={d} F={F} E={E} k={k}, {w.n_layers} blocks")
    x0 = bf16(w.x)
    xa = x0.clone()
    nrm = torch.empty_like(x0)
    ws = torch.empty(moe.workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
    bufs = moe._outputs(T, d, E, k, x0.device, None, store_out=False)

    def stack_pass(i):
        # the first block's pre-norm alone; after that each block ends with its
        # combine, residual add and the next block's pre-norm in one pass (the
        # block output itself is not stored), in place on xa and nrm
        xa.copy_(x0)
        moe.rmsnorm(xa, layers[0][0], w.eps, nrm)
        for l, (_, wt) in enumerate(layers):
            gain = layers[l + 1][0] if l + 1 < len(layers) else None
            moe.forward_residual_rmsnorm(nrm, wt, k, ws, xa, gain, w.eps, resid_out=xa, n_out=nrm,
                                         bufs=bufs)

    runs = timed_runs(stack_pass, steps, warmup, repeats)
    ms = float(np.median(runs))
    U = int((bufs["perm"][0].cpu().numpy() > 0).sum())
    b, f = layer_alg(T, d, F, E, k, U, False)
    # per block the glue reads and writes the residual stream and writes the next
    # pre-norm; the block output m (counted as written by layer_alg) stays on chip
    b += 6 * T * d
    res = dict(workload=w.name, T=T, blocks=w.n_layers, ms_per_step=ms, ms_per_step_best=float(min(runs)),
               ms_per_step_runs=runs, ms_per_block=ms / w.n_layers, tokens_per_s=T / (ms / 1e3),
               frac_hbm_peak=w.n_layers * b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
               frac_mxfp4_peak=w.n_layers * f / (ms / 1e3) / 1e12 / MXFP4_PEAK_TFLOPS,
               note="one step = one pass of all 24 blocks; x copied in at its start (0.02%)")
    log(f"[bench] {w.name}: {ms:.2f} ms per {w.n_layers}-block pass ({ms / w.n_layers * 1e3:.0f} us per block), "
        f"{res['tokens_per_s']:.4g} tok/s")
    del layers, ws, bufs
    torch.cuda.empty_cache()
    return res


def oracle_check(res: dict, log) -> dict:
    """Compare the timed run's output with the CPU oracle (the parity tests' bars)."""
    import oracle
    w = res["_workload"]
    L = w.layers[0]
    t0 = time.perf_counter()
    ref = oracle.moe_layer(w.x, L, w.k)
    dt = time.perf_counter() - t0
    out = oracle.bf16_to_f64(res["_out_bits"])
    err = np.abs(out - ref["out"])
    rms = float(np.sqrt(np.mean(ref["out"] ** 2)))
    _, e2 = np.frexp(np.abs(ref["out"]))
    excess = float(np.maximum(err - np.ldexp(1.0, e2 - 9), 0).max() / rms)
    mean_rel = float(err.sum() / np.abs(ref["out"]).sum())
    same = bool(np.array_equal(res["_idx"], ref["idx"]))
    ok = bool(same and excess <= 2e-2 and mean_rel <= 5e-3)
    log(f"[bench] oracle check {w.name}: routing equal {same}, excess {excess:.3g}, "
        f"mean rel {mean_rel:.3g} -> {'ok' if ok else 'FAIL'}")
    return dict(ok=ok, excess_over_rms=excess, mean_rel=mean_rel,
                literal_over_rms=float(err.max() / rms), oracle_seconds=dt)


def cpu_baseline(res: dict, seconds: float, log) -> dict:
    """The oracle as it stands, on the host cores, on a bounded sample: whole
    layer passes over the same workload's tokens until `seconds` have elapsed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible CPUs
        threads = os.cpu_count() or 1
    w = res["_workload"]
    L = w.layers[0]
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(w.x, L, w.k)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    v = n * w.T / dt
    log(f"[bench] cpu oracle: {n} passes of {w.T} tokens in {dt:.1f} s -> {v:.3g} tok/s on {threads} threads")
    return dict(value=v, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{n} full passes of the {w.name} workload ({w.T} tokens each), numpy float64")


def _public(r: dict) -> dict:
    return {k: v for k, v in r.items() if not k.startswith("_")}


def main():
    args = parse()
    log = lambda s: print(s, file=sys.stderr, flush=True)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        import sparse_moe_transformer_gemm_amd as moe
        n = args.copy_calibration << 20
        rows = n // (2 * 2880)
        a = torch.ones((rows, 2880), dtype=torch.bfloat16, device="cuda:0")
        b = torch.ones_like(a)
        c = torch.empty_like(a)
        for _ in range(3):
            moe.residual_add(a, b, c)
        torch.cuda.synchronize()
        log(f"[bench] residual add over {a.numel() * 2} bytes per operand, 3 times "
            f"(read {2 * a.numel() * 2} B, write {a.numel() * 2} B per pass)")
        return

    clk0 = clocks()
    order = [int(c) for c in args.workloads.split(",") if c.strip()]
    results, checks = {}, {}
    for cfg in order:
        if synth.WORKLOADS[cfg]["n_layers"] > 1:
            results[cfg] = run_stack(cfg, max(3, args.steps // 40), max(2, args.warmup // 10),
                                     max(3, args.repeats), log)
        else:
            # the prefill-sized layers take ~1 ms per step: fewer steps
            big = synth.WORKLOADS[cfg]["T"] > 1024
            st = max(20, args.steps // 5) if big else args.steps
            results[cfg] = run_layer(cfg, st, args.warmup, args.repeats, not args.no_graph, log)
            if cfg in (0, 1):
                checks[cfg] = oracle_check(results[cfg], log)
    fp8 = {}
    for cfg in [int(c) for c in args.fp8.split(",") if c.strip()]:
        big = synth.WORKLOADS[cfg]["T"] > 1024
        r8 = run_fp8(cfg, max(20, args.steps // 5) if big else args.steps, args.warmup, args.repeats, log)
        fp8[r8["workload"]] = r8
    attn = {}
    for name in [a.strip() for a in args.attention.split(",") if a.strip()]:
        big = synth.ATTN_WORKLOADS[name]["Tq"] > 64
        attn[name] = run_attention(name, max(10, args.steps // 10) if big else args.steps,
                                   max(2, args.warmup // 2) if big else args.warmup, args.repeats, log)
    head = results[order[0]]
    cpu = None
    if not args.no_cpu_baseline and "_workload" in head:
        cpu = cpu_baseline(head, args.cpu_seconds, log)
    clk1 = clocks()

    # value and config are the first workload's; the roofline object describes the
    # gate/up GEMM of the first single-layer workload (none if only the stack ran)
    r = next((results[c] for c in order if "gate_up_gemm" in results[c]), None)
    gu = r.get("gate_up_gemm", {}) if r else {}
    decode = r is not None and r["T"] <= 64
    if r is None:
        roof = None
    elif decode:
        roof = {"bound": "hbm", "achieved": gu["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gu["gbs"] / HBM_PEAK_GBS,
                "traffic": measured_traffic(f"{r['workload']}_T{r['T']}"),
                "kernel": "grouped_decode<true, 6>: the gate/up GEMM with SwiGLU "
                          "(moe_expert_ffn_mxfp4 stage 1)",
                "alg_bytes_per_launch": gu["alg_bytes"], "avg_launch_ms": gu["avg_launch_ms"],
                "units": f"{r['experts_touched']} touched experts x {gateup_bytes(r['d'], r['F'])} B "
                         f"(gate and up MXFP4 codes, E8M0 scales, bf16 biases)"}
    else:
        roof = {"bound": "mfma", "achieved": gu["tflops"], "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": gu["tflops"] / MXFP4_PEAK_TFLOPS,
                "traffic": measured_traffic(f"{r['workload']}_T{r['T']}"),
                "kernel": "grouped_prefill<6, true>: the gate/up GEMM with SwiGLU (stage 1)",
                "flops_per_launch": gu["flops"], "avg_launch_ms": gu["avg_launch_ms"]}
    if roof is not None:
        roof["timing"] = ("stage launched back to back over the rotating weight copies, HIP events "
                          "on the launch stream around the timed launches")
        roof["layer_frac"] = r["frac_hbm_peak"] if decode else r["frac_mxfp4_peak"]
    r = head
    line = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 weights x 2-term mxfp6 activations, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{r['workload']}: " + (f"T={r['T']} d={r['d']} F={r['F']} E={r['E']} "
                                                         f"top-{r['k']}, seed {r['seed']}" if "d" in r else
                                                         f"T={r['T']} per block, {r.get('blocks')} blocks"),
                   "global_batch": r["T"], "weight_copies": r.get("weight_copies"),
                   "experts_touched": r.get("experts_touched")},
        "timing": f"median of {args.repeats} runs of {args.steps} eager moe_forward steps after "
                  f"{args.warmup} warmup steps; graph replay and best run beside it",
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": {("tiny" if c == 0 else "decode-20b"): v for c, v in checks.items()},
        "workloads": {results[c]["workload"]: _public(results[c]) for c in order},
        "fp8_weights": fp8,
        "attention_sink": attn,
        "clocks": {"before": clk0, "after": clk1},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
