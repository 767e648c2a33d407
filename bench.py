#!/usr/bin/env python3
"""Throughput of the MXFP4 sparse-MoE block on one MI355X.

One step = one pass of the whole block (moe_forward: route -> permute ->
expert FFN -> combine) over one batch of T tokens whose inputs are already
resident in HBM. The headline workload is the decode-shaped gpt-oss-20b
layer (T=16, d=F=2880, E=32, top-4), which is bound by streaming the MXFP4
weights from HBM; the prefill-shaped layer (T=8192) is reported beside it
against the MXFP4 matrix-core peak, and the 24-block pre-norm stack (T=2048 per
block) as tokens/s of the whole stack.

Timing: W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize(); the weights rotate over R identical copies (R * layer
bytes >= 1.5 GB) so the 256 MB last-level cache cannot hold them. A second timed
loop runs the same steps as the four separate calls (moe_route, moe_permute,
moe_expert_ffn_mxfp4, moe_combine) with HIP events on the launch stream around
the expert-FFN call. The roofline figure is the dominant kernel's, the gate/up
GEMM (moe_expert_ffn_mxfp4_stage 1), whose average launch duration comes from
a third loop that launches it back to back over the weight copies with events
around the loop; the whole expert-FFN call's figure is reported beside it. The timed output is checked against the CPU oracle in the same run, and the
oracle is timed on the host cores as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
                       [--no-stack] [--no-cpu-baseline] [--workload 1]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
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


def enc_bytes(rows: int, K: int) -> int:
    """Bytes of `rows` activation rows encoded for the matrix cores (208 per
    128-deep step)."""
    return rows * ((K + 127) // 128) * 208


def gateup_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert in the gate/up GEMM: the gate and up
    MXFP4 matrices and their bf16 biases."""
    return 2 * (d * F // 2 + d * F // 32) + 2 * 2 * F


def expert_bytes(d: int, F: int) -> int:
    """Algorithmic bytes of one expert: 3 MXFP4 matrices (0.5 B/elt + 1 B per 32)
    and its bf16 biases (2F + d)."""
    return 3 * (d * F // 2 + d * F // 32) + 2 * (2 * F + d)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--secondary", type=int, default=2, help="second workload (-1: none)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-stack", action="store_true", help="skip the 24-block stack workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 passes of the library's streaming residual-add kernel "
                         "over MIB MiB per operand (reads 2 x MIB, writes MIB: a known byte "
                         "count to calibrate a profiler's HBM byte counters) and exit")
    return ap.parse_args()


def run_gpu(cfg: int, steps: int, warmup: int, log) -> dict:
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    w = synth.workload(cfg)
    L = w.layers[0]
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k
    layer_bytes = E * expert_bytes(d, F) + 4 * d * E
    R = max(1, int(np.ceil(1.5e9 / layer_bytes)))
    log(f"[bench] workload {w.name}: T={T} d={d} F={F} E={E} k={k}; {R} weight copies")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    copies = []
    for _ in range(R):
        copies.append(moe.load_expert_weights(
            w_router=torch.from_numpy(L.w_router).to(dev),
            b_router=None if L.b_router is None else torch.from_numpy(L.b_router).to(dev),
            gate_codes=u8(L.gate.codes), gate_scales=u8(L.gate.scales),
            up_codes=u8(L.up.codes), up_scales=u8(L.up.scales),
            down_codes=u8(L.down.codes), down_scales=u8(L.down.scales),
            b_gate=bf16(L.b_gate), b_up=bf16(L.b_up), b_down=bf16(L.b_down)))
    x = bf16(w.x)
    ws = torch.empty(moe.workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
    P = T * k
    bufs = dict(
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        perm=(torch.empty(E, dtype=torch.int32, device=dev),
              torch.empty(E + 1, dtype=torch.int32, device=dev),
              torch.empty(P, dtype=torch.int32, device=dev),
              torch.empty(P, dtype=torch.int32, device=dev)),
        y_sorted=torch.empty((P, d), dtype=torch.float32, device=dev),
        out=torch.empty((T, d), dtype=torch.bfloat16, device=dev))

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]

    def step(i):
        moe.forward(x, copies[i % R], k, ws, bufs)

    def step_calls(i):
        # the same block as the four separate calls, with HIP events on the
        # launch stream around the expert-FFN call
        wt = copies[i % R]
        idx, tw = moe.route(x, wt.w_router, wt.b_router, k, ws, bufs["topk_idx"], bufs["topk_w"])
        perm = moe.permute(idx, E, ws, bufs["perm"])
        ev[i][0].record()
        y = moe.expert_ffn_mxfp4(x, perm[2], perm[1], wt, k, ws, bufs["y_sorted"])
        ev[i][1].record()
        moe.combine(y, perm[3], tw, bufs["out"])

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_step = timed(step)                 # the headline: whole-block calls
    ms_step_calls = timed(step_calls)     # the FFN call's duration
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # The GEMMs' average launch durations: the gate/up GEMM (stage 1, the
    # dominant kernel) and then the down GEMM (stage 2) launched back to back
    # over the rotating weight copies, on what the earlier stages left in the
    # workspace (every launch rewrites the same h or y), one event pair around
    # each timed run.
    wt0 = copies[0]
    idx, _ = moe.route(x, wt0.w_router, wt0.b_router, k, ws, bufs["topk_idx"], bufs["topk_w"])
    perm = moe.permute(idx, E, ws, bufs["perm"])
    moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], wt0, k, ws, bufs["y_sorted"], 0)

    def stage_ms(stage):
        for i in range(warmup):
            moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], copies[i % R], k, ws, bufs["y_sorted"], stage)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record()
        for i in range(steps):
            moe.expert_ffn_mxfp4_stage(x, perm[2], perm[1], copies[i % R], k, ws, bufs["y_sorted"], stage)
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / steps

    gu_ms = stage_ms(1)
    dn_ms = stage_ms(2)
    # the checked output is the whole-block call's
    step(0)
    torch.cuda.synchronize()
    counts = bufs["perm"][0].cpu().numpy()
    U = int((counts > 0).sum())
    out_bits = bufs["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    idx_gpu = bufs["topk_idx"].cpu().numpy()

    ffn_bytes = U * expert_bytes(d, F) + 2 * T * d
    # gate/up GEMM: its weights and biases, the encoded x it reads, the encoded h it writes
    gu_bytes = U * gateup_bytes(d, F) + enc_bytes(T, d) + enc_bytes(T * k, F)
    gu_flops = 2.0 * T * k * 2 * d * F
    layer_alg_bytes = ffn_bytes + 4 * d * E + (4 * E if L.b_router is not None else 0) + 2 * T * d
    flops = 2.0 * T * k * 3 * d * F
    res = dict(
        workload=w.name, T=T, d=d, F=F, E=E, k=k, seed=w.seed, weight_copies=R,
        experts_touched=U, ms_per_step=ms_step, ms_per_step_calls=ms_step_calls,
        tokens_per_s=T / (ms_step / 1e3),
        ffn_ms=ffn_ms, ffn_alg_bytes=ffn_bytes, layer_alg_bytes=layer_alg_bytes,
        gu_ms=gu_ms, dn_ms=dn_ms, gu_alg_bytes=gu_bytes, gu_flops=gu_flops,
        gu_gbs=gu_bytes / (gu_ms / 1e3) / 1e9, gu_tflops=gu_flops / (gu_ms / 1e3) / 1e12,
        ffn_gbs=ffn_bytes / (ffn_ms / 1e3) / 1e9, ffn_tflops=flops / (ffn_ms / 1e3) / 1e12,
        layer_gbs=layer_alg_bytes / (ms_step / 1e3) / 1e9,
        layer_tflops=flops / (ms_step / 1e3) / 1e12, flops=flops,
        _out_bits=out_bits, _idx=idx_gpu, _workload=w)
    log(f"[bench] {w.name}: {ms_step * 1e3:.1f} us/step ({ms_step_calls * 1e3:.1f} as four calls), "
        f"ffn {ffn_ms * 1e3:.1f} us (back to back: gate/up {gu_ms * 1e3:.1f}, down {dn_ms * 1e3:.1f}), "
        f"{res['tokens_per_s']:.4g} tok/s, ffn {res['ffn_gbs']:.0f} GB/s / {res['ffn_tflops']:.0f} TFLOP/s, "
        f"gate/up {res['gu_gbs']:.0f} GB/s / {res['gu_tflops']:.0f} TFLOP/s")
    del copies, ws, bufs
    torch.cuda.empty_cache()
    return res


def run_stack(cfg: int, steps: int, warmup: int, log) -> dict:
    """The pre-norm stack workload: per step, every block does
    x <- x + MoE(RMSNorm(x)) through the C ABI, all layers' weights resident."""
    import torch

    import sparse_moe_transformer_gemm_amd as moe

    dev = "cuda:0"
    w = synth.workload(cfg, with_layers=False)
    T, d, F, E, k = w.T, w.d, w.F, w.E, w.k

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    layers = []
    for l in range(w.n_layers):
        L = synth.stack_layer(cfg, l)
        layers.append((bf16(L.gain), moe.load_expert_weights(
            w_router=torch.from_numpy(L.w_router).to(dev), b_router=None,
            gate_codes=u8(L.gate.codes), gate_scales=u8(L.gate.scales),
            up_codes=u8(L.up.codes), up_scales=u8(L.up.scales),
            down_codes=u8(L.down.codes), down_scales=u8(L.down.scales),
            b_gate=bf16(L.b_gate), b_up=bf16(L.b_up), b_down=bf16(L.b_down))))
    log(f"[bench] workload {w.name}: T={T} d={d} F={F} E={E} k={k}, {w.n_layers} blocks")
    x0 = bf16(w.x)
    xa, xb = x0.clone(), torch.empty_like(x0)
    nrm = torch.empty_like(x0)
    ws = torch.empty(moe.workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
    P = T * k
    bufs = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                perm=(torch.empty(E, dtype=torch.int32, device=dev),
                      torch.empty(E + 1, dtype=torch.int32, device=dev),
                      torch.empty(P, dtype=torch.int32, device=dev),
                      torch.empty(P, dtype=torch.int32, device=dev)),
                y_sorted=torch.empty((P, d), dtype=torch.float32, device=dev),
                out=torch.empty((T, d), dtype=torch.bfloat16, device=dev))
    touched = []

    def stack_pass():
        xa.copy_(x0)
        cur, nxt = xa, xb
        for gain, wt in layers:
            moe.rmsnorm(cur, gain, w.eps, nrm)
            r = moe.forward(nrm, wt, k, ws, bufs)
            moe.residual_add(cur, r["out"], nxt)
            cur, nxt = nxt, cur

    for _ in range(warmup):
        stack_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack_pass()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # experts touched by the last block (every block touches all 32 at T=2048)
    U = int((bufs["perm"][0].cpu().numpy() > 0).sum())
    per_layer_bytes = U * expert_bytes(d, F) + 4 * d * E + 4 * T * d + 10 * T * d
    flops = w.n_layers * 2.0 * T * k * 3 * d * F
    res = dict(workload=w.name, T=T, blocks=w.n_layers, ms_per_step=ms, tokens_per_s=T / (ms / 1e3),
               frac_hbm_peak=w.n_layers * per_layer_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
               frac_mxfp4_peak=flops / (ms / 1e3) / 1e12 / MXFP4_PEAK_TFLOPS,
               note="x copied in at the start of every step (0.02% of the step)")
    log(f"[bench] {w.name}: {ms:.2f} ms per {w.n_layers}-block pass, {res['tokens_per_s']:.4g} tok/s")
    del layers, ws, bufs
    torch.cuda.empty_cache()
    return res


def oracle_check(res: dict, log) -> dict:
    """Compare the timed run's output with the CPU oracle (tolerance of the parity tests)."""
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
    ok = bool(np.array_equal(res["_idx"], ref["idx"]) and excess <= 2e-2 and mean_rel <= 5e-3)
    log(f"[bench] oracle check: routing equal {np.array_equal(res['_idx'], ref['idx'])}, "
        f"excess {excess:.3g}, mean rel {mean_rel:.3g} -> {'ok' if ok else 'FAIL'}")
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

    main_res = run_gpu(args.workload, args.steps, args.warmup, log)
    check = oracle_check(main_res, log) if args.workload in (0, 1) else None
    sec = None
    if not args.no_secondary and args.secondary >= 0:
        s = run_gpu(args.secondary, max(10, args.steps // 4), max(3, args.warmup // 4), log)
        sec = {
            "workload": s["workload"], "T": s["T"], "tokens_per_s": s["tokens_per_s"],
            "ms_per_step": s["ms_per_step"], "experts_touched": s["experts_touched"],
            "roofline": {"bound": "mfma", "kernel": "grouped_prefill<6, true>: the gate/up GEMM with "
                                                     "SwiGLU (moe_expert_ffn_mxfp4 stage 1)",
                         "achieved": s["gu_tflops"], "peak": MXFP4_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": s["gu_tflops"] / MXFP4_PEAK_TFLOPS,
                         "traffic": measured_traffic(f"{s['workload']}_T{s['T']}"),
                         "flops_per_launch": s["gu_flops"], "avg_launch_ms": s["gu_ms"],
                         "down_gemm_ms": s["dn_ms"],
                         "ffn_call": {"achieved": s["ffn_tflops"], "frac": s["ffn_tflops"] / MXFP4_PEAK_TFLOPS,
                                      "avg_ms": s["ffn_ms"], "flops": s["flops"],
                                      "traffic": measured_traffic(f"{s['workload']}_T{s['T']}",
                                                                  "traffic_bytes_per_call")}},
            "layer_frac_mxfp4_peak": s["layer_tflops"] / MXFP4_PEAK_TFLOPS,
            "ffn_ms": s["ffn_ms"],
        }
    stack = None
    if not args.no_stack:
        stack = run_stack(4, 3, 1, log)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(main_res, args.cpu_seconds, log)

    r = main_res
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
        "config": {"workload": f"{r['workload']}: T={r['T']} d={r['d']} F={r['F']} E={r['E']} "
                               f"top-{r['k']}, seed {r['seed']}",
                   "global_batch": r["T"], "weight_copies": r["weight_copies"],
                   "experts_touched": r["experts_touched"]},
        "roofline": {"bound": "hbm", "kernel": "grouped_decode<true, 6>: the gate/up GEMM with SwiGLU "
                                               "(moe_expert_ffn_mxfp4 stage 1)",
                     "achieved": r["gu_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["gu_gbs"] / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"{r['workload']}_T{r['T']}"),
                     "alg_bytes_per_launch": r["gu_alg_bytes"], "avg_launch_ms": r["gu_ms"],
                     "timing": "gate/up GEMM (moe_expert_ffn_mxfp4_stage 1) launched back to back "
                               "over the rotating weight copies, HIP events on the launch stream "
                               "around the timed launches",
                     "down_gemm_ms": r["dn_ms"],
                     "ffn_call": {"kernels": "encode + gate/up GEMM + down GEMM",
                                  "achieved": r["ffn_gbs"], "frac": r["ffn_gbs"] / HBM_PEAK_GBS,
                                  "avg_ms": r["ffn_ms"], "alg_bytes": r["ffn_alg_bytes"],
                                  "timing": "HIP events around moe_expert_ffn_mxfp4 in a second "
                                            "timed loop of the same steps run as the four "
                                            "separate calls",
                                  "traffic": measured_traffic(f"{r['workload']}_T{r['T']}",
                                                              "traffic_bytes_per_call")}},
        "ms_per_step_four_calls": r["ms_per_step_calls"],
        "layer_frac_hbm_peak": r["layer_gbs"] / HBM_PEAK_GBS,
        "cpu_baseline": cpu,
        "parity": check,
        "secondary": sec,
        "stack": stack,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
