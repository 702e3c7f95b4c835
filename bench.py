#!/usr/bin/env python3
"""Benchmark of the Skiparse-2D attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 720p_5s]

A step is one token-wise layer followed by one group-wise layer (the pattern
alternation of the method) over the workload's Q, K, V, already resident in
HBM.  Printed as ONE JSON line: TFLOP/s counting only computed (real x real,
same subsequence) pairs, ms per step, the roofline of the attention kernel
(average launch duration from HIP events on the launch stream), the oracle's
CPU baseline on a bounded sample, and extras: ms per layer, the same kernel at
k = 1 (full attention), the fp8 path, a training step (forward with the
log-sum-exp, backward), Skiparse-1D, the fp8 block's projection GEMM, rotary
quantizer and whole block, and the other bf16 workloads (768P-5s unpadded,
480P with its k = 1 layer).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HBM_GBS = 8000.0
COPY_BYTES = 1 << 30          # calibration copy of the traffic run
PROFILE_PMC = os.path.join(ROOT, "profiles", "attn_fwd_bf16_720p_5s_pmc.md")
KERNEL_SOURCES = ["fixed_pattern_sparse_amd/csrc/attn_bf16.hip", "fixed_pattern_sparse_amd/csrc/attn_common.h",
                  "fixed_pattern_sparse_amd/csrc/geom.h", "fixed_pattern_sparse_amd/csrc/internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch recorded from rocprofv3 counters, if they were taken
    on the current kernel source (else None)."""
    if workload != "720p_5s" or not os.path.exists(PROFILE_PMC):
        return None
    text = open(PROFILE_PMC).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(workload, cpu_inputs, budget_s=20.0):
    """The oracle's fp32 numpy/BLAS algorithm on a bounded sample of units
    (b = 0, heads 0.., every subsequence of both patterns), scaled by pairs."""
    from oracle import cpu_baseline as cb
    B, T, H, W, nh, d = workload.shape
    N = T * H * W
    q, k, v = (t.float().numpy().reshape(B, N, nh, d) for t in cpu_inputs)
    secs = 0.0
    pairs = 0
    units = 0
    heads_done = 0
    for h in range(nh):
        for mode in (0, 1):
            us = [(0, h, s) for s in range(workload.k * workload.k)]
            dt, pr = cb.time_sample(q, k, v, T, H, W, workload.k, mode, us)
            secs += dt
            pairs += pr
            units += len(us)
        heads_done += 1
        if secs > budget_s:
            break
    tflops = 4 * d * pairs / secs / 1e12
    return {
        "value": round(tflops, 6),
        "unit": "TFLOP/s",
        "cores": cb.blas_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{units} (batch, head, subsequence) units = heads 0-{heads_done - 1} of batch 0, all "
                   f"{workload.k * workload.k} subsequences of both patterns; {pairs:.4g} pairs in "
                   f"{secs:.1f} s, fp32 numpy/BLAS; TFLOP/s scales exactly by pair count"),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_layers(sk, stream, plans, q, k, v, out, reps):
    """ms of one pass over ``plans`` (bf16 forward layers back to back),
    averaged over ``reps`` passes after one untimed pass."""
    import torch
    for pl in plans:
        sk.skiparse_attn_fwd(pl, sk.BF16, q, k, v, out, stream=stream)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(reps):
        for pl in plans:
            sk.skiparse_attn_fwd(pl, sk.BF16, q, k, v, out, stream=stream)
    e[1].record(stream)
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) / reps


def other_workloads(sk, stream, ref_rate):
    """The other bf16 forward configurations, each timed on its own inputs:
    768P-5s (B = 2, no padding) token-wise and group-wise layers separately
    and back to back, and 480P with both patterns and its k = 1 layer.  Inputs
    are N(0,1) from torch's device generator with a fixed seed, rounded to
    bf16.  ``ref_rate`` is the padded 720P-5s layer rate of the same run, for
    the padded / unpadded per-pair comparison."""
    import torch
    import workloads as wl
    res = {}
    for name, reps in (("768p_5s", 3), ("480p", 10)):
        w = wl.WORKLOADS[name]
        B, T, H, W, nh, d = w.shape
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed)
        q, k, v = (torch.randn(w.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(3))
        out = torch.empty_like(q)
        p_tok = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_TOKEN)
        p_grp = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_GROUP)
        r = {"shape": list(w.shape), "k": w.k, "padded": [p_tok.Hp, p_tok.Wp] != [H, W]}
        for tag, plans in (("token", [p_tok]), ("group", [p_grp]), ("token_then_group", [p_tok, p_grp])):
            ms = time_layers(sk, stream, plans, q, k, v, out, reps)
            fl = sum(pl.flops for pl in plans)
            r[tag] = {"ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                      "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
        if name == "480p":
            p1 = sk.skiparse_plan_init(B, T, H, W, nh, d, 1, sk.MODE_TOKEN)
            ms = time_layers(sk, stream, [p1], q, k, v, out, reps)
            r["k1_full"] = {"ms": round(ms, 3), "tflops": round(p1.flops / (ms * 1e-3) / 1e12, 2)}
            r["speedup_vs_k1"] = round(ms / r["token"]["ms"], 3)
        else:
            r["per_pair_rate_vs_720p_padded"] = round(r["token_then_group"]["tflops"] / ref_rate, 4)
        res[name] = r
        del q, k, v, out
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p_5s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--traffic-run", action="store_true",
                    help="for rocprofv3 --pmc: one 1 GiB copy kernel (calibration), then one token-wise and "
                         "one group-wise layer, no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no multi-GPU path; "
              "a rank would run its share of the subsequences through sub_begin / sub_count", file=sys.stderr)
        sys.exit(2)

    import torch
    import fixed_pattern_sparse_amd as sk
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("the timed step uses a bf16 workload")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    t0 = time.time()
    cpu = wl.make_inputs(w)
    q, k, v = (t.to("cuda") for t in cpu)
    o_tok = torch.empty_like(q)
    o_grp = torch.empty_like(q)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    B, T, H, W, nh, d = w.shape
    if args.traffic_run:
        # a plain elementwise copy of known size: reads and writes COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        for mode in (sk.MODE_TOKEN, sk.MODE_GROUP):
            plan = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, mode)
            sk.skiparse_attn_fwd(plan, sk.BF16, q, k, v, o_tok, stream=stream)
        torch.cuda.synchronize()
        print("# traffic run done", file=sys.stderr, flush=True)
        return
    p_tok = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_TOKEN)
    p_grp = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_GROUP)
    flops_step = p_tok.flops + p_grp.flops

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sk.skiparse_attn_fwd(p_tok, sk.BF16, q, k, v, o_tok, stream=stream)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)
        sk.skiparse_attn_fwd(p_grp, sk.BF16, q, k, v, o_grp, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    launch_ms = []
    for ev in events:
        launch_ms.append(ev[0].elapsed_time(ev[1]))
        launch_ms.append(ev[2].elapsed_time(ev[3]))
    avg_launch_ms = float(np.mean(launch_ms))
    achieved = (flops_step / 2) / (avg_launch_ms * 1e-3) / 1e12
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step, kernel avg {avg_launch_ms:.3f} ms/launch",
          file=sys.stderr, flush=True)

    traffic = recorded_traffic(args.workload)
    result = {
        "metric": "Skiparse-2D attn fwd TFLOP/s + ms/layer, 720P-5s shape, 1 MI355X",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "T": T, "H": H, "W": W, "heads": nh, "d": d, "k": w.k,
                   "padded_H": p_tok.Hp, "padded_W": p_tok.Wp, "outlier_channels": w.outliers,
                   "step": "token-wise layer + group-wise layer", "flop_per_step": flops_step},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic, "kernel": "attn_fwd_bf16_kernel<128, 2>",
                     "avg_launch_ms": round(avg_launch_ms, 4)},
    }
    extras = {"ms_per_layer": round(ms_step / 2, 4)}

    if not args.no_extras:
        t_x = time.time()

        def progress(name):
            print(f"# extras: {name} done at {time.time() - t_x:.1f} s", file=sys.stderr, flush=True)

        # same kernel at k = 1 (full attention, the hybrid model's full layers)
        p1 = sk.skiparse_plan_init(B, T, H, W, nh, d, 1, sk.MODE_TOKEN)
        o1 = torch.empty_like(q)
        sk.skiparse_attn_fwd(p1, sk.BF16, q, k, v, o1, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(3):
            sk.skiparse_attn_fwd(p1, sk.BF16, q, k, v, o1, stream=stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        k1_ms = e[0].elapsed_time(e[1]) / 3
        extras["k1_ms_per_layer"] = round(k1_ms, 3)
        extras["k1_tflops"] = round(p1.flops / (k1_ms * 1e-3) / 1e12, 3)
        extras["speedup_vs_k1"] = round(k1_ms / avg_launch_ms, 3)
        progress("k = 1 layer")
        del o1
        # fp8 path on the same shape: per-tensor e4m3 quantization of Q, K, V
        # (scale = 448 / (amax + 1e-12)) then the e4m3 kernel, k = 2 and k = 4
        scales = torch.empty((3, 2), dtype=torch.float32, device="cuda")
        codes = [sk.quantize_fp8(t, scale_out=scales[i])[0] for i, t in enumerate((q, k, v))]
        o8 = torch.empty_like(q)
        fp8 = {}
        for kf in (2, 4):
            for mode, name in ((sk.MODE_TOKEN, "token"), (sk.MODE_GROUP, "group")):
                pl = sk.skiparse_plan_init(B, T, H, W, nh, d, kf, mode)
                sk.skiparse_attn_fwd(pl, sk.FP8_E4M3, *codes, o8, descale_qkv=scales, stream=stream)
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
                for _ in range(5):
                    sk.skiparse_attn_fwd(pl, sk.FP8_E4M3, *codes, o8, descale_qkv=scales, stream=stream)
                e[1].record(stream)
                torch.cuda.synchronize()
                ms = e[0].elapsed_time(e[1]) / 5
                fp8[f"k{kf}_{name}"] = {"ms": round(ms, 3), "tflops": round(pl.flops / (ms * 1e-3) / 1e12, 2),
                                        "frac_fp8_peak": round(pl.flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4)}
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(3):
            for i, t in enumerate((q, k, v)):
                sk.quantize_fp8(t, scale_out=scales[i])
        e[1].record(stream)
        torch.cuda.synchronize()
        qms = e[0].elapsed_time(e[1]) / 3
        # algorithmic HBM bytes of quantizing the three tensors: amax pass reads
        # 2 B/elt, the cast reads 2 B/elt and writes 1 B/elt
        qbytes = 3 * q.numel() * 5
        fp8["quantize_qkv"] = {"ms": round(qms, 3), "GBps": round(qbytes / (qms * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(qbytes / (qms * 1e-3) / 1e9 / HBM_GBS, 4)}
        extras["fp8_e4m3"] = fp8
        progress("e4m3 forward")
        del o8, codes
        # training step of one layer: forward keeping the log-sum-exp, then the
        # backward pass for a synthetic upstream gradient.  Backward FLOPs are
        # counted as 2.5x the forward's (five n x n x d products: the S
        # recompute, dP, dV, dQ, dK), whatever the kernels recompute beyond.
        do_ = torch.from_numpy(wl.normal_tensor(w.shape, w.seed, 3)).to(torch.bfloat16).cuda()
        train = {}
        for mode, name in ((sk.MODE_TOKEN, "token"), (sk.MODE_GROUP, "group")):
            pl = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, mode)
            ot = torch.empty_like(q)
            lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device="cuda")
            grads = [torch.empty_like(q) for _ in range(3)]
            ws = torch.empty(sk.skiparse_attn_bwd_workspace_bytes(pl), dtype=torch.uint8, device="cuda")
            sk.skiparse_attn_fwd_lse(pl, sk.BF16, q, k, v, ot, lse, stream=stream)
            sk.skiparse_attn_bwd(pl, sk.BF16, q, k, v, ot, do_, lse, *grads, workspace=ws, stream=stream)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            for _ in range(3):
                sk.skiparse_attn_fwd_lse(pl, sk.BF16, q, k, v, ot, lse, stream=stream)
            e[1].record(stream)
            for _ in range(3):
                sk.skiparse_attn_bwd(pl, sk.BF16, q, k, v, ot, do_, lse, *grads, workspace=ws, stream=stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            fms, bms = e[0].elapsed_time(e[1]) / 3, e[1].elapsed_time(e[2]) / 3
            train[name] = {"fwd_lse_ms": round(fms, 3), "bwd_ms": round(bms, 3),
                           "bwd_tflops": round(2.5 * pl.flops / (bms * 1e-3) / 1e12, 2),
                           "bwd_frac_bf16_peak": round(2.5 * pl.flops / (bms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
            del ot, lse, grads, ws
        extras["training_bf16"] = train
        progress("bf16 training step")
        # the 8-bit training step (token-wise): Q, K, V and dO quantized per
        # tensor on the device, the e4m3 forward keeping the log-sum-exp, then
        # the backward on the codes; quantization of dO is timed with the
        # backward, that of Q, K, V with the forward
        pl = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_TOKEN)
        sc8 = torch.empty((3, 2), dtype=torch.float32, device="cuda")
        dsc8 = torch.empty(2, dtype=torch.float32, device="cuda")
        c8 = [torch.empty(q.shape, dtype=torch.uint8, device="cuda") for _ in range(4)]
        qws = torch.empty(sk.skiparse_quant_fp8_workspace_bytes(q.numel()), dtype=torch.uint8, device="cuda")
        ot = torch.empty_like(q)
        lse = torch.empty((B, T * H * W, nh), dtype=torch.float32, device="cuda")
        grads = [torch.empty_like(q) for _ in range(3)]
        ws = torch.empty(sk.skiparse_attn_bwd_workspace_bytes(pl), dtype=torch.uint8, device="cuda")

        def fwd8():
            for i, t in enumerate((q, k, v)):
                sk.skiparse_quant_fp8(t, c8[i], sc8[i], workspace=qws, stream=stream)
            sk.skiparse_attn_fwd_lse_fp8(pl, c8[0], c8[1], c8[2], sc8, ot, lse, stream=stream)

        def bwd8():
            sk.skiparse_quant_fp8(do_, c8[3], dsc8, workspace=qws, stream=stream)
            sk.skiparse_attn_bwd_fp8(pl, c8[0], c8[1], c8[2], sc8, ot, c8[3], dsc8, lse, *grads, workspace=ws,
                                     stream=stream)

        fwd8()
        bwd8()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for _ in range(3):
            fwd8()
        e[1].record(stream)
        for _ in range(3):
            bwd8()
        e[2].record(stream)
        torch.cuda.synchronize()
        fms, bms = e[0].elapsed_time(e[1]) / 3, e[1].elapsed_time(e[2]) / 3
        extras["training_fp8_token"] = {
            "fwd_lse_ms": round(fms, 3), "bwd_ms": round(bms, 3),
            "bwd_tflops": round(2.5 * pl.flops / (bms * 1e-3) / 1e12, 2),
            "note": "e4m3 tensors, quantization included; S and dP on the e4m3 matrix core, dV, dK, dQ on bf16 MFMA"}
        del sc8, dsc8, c8, qws, ot, lse, grads, ws
        del do_
        progress("8-bit training step")
        # Skiparse-1D on the same shape (the 1D rule on each frame's flattened
        # (h, w), stride k*k: the variant the 2D pattern is compared with)
        one_d = {}
        o1d = torch.empty_like(q)
        for mode, name in ((sk.MODE_TOKEN_1D, "token"), (sk.MODE_GROUP_1D, "group")):
            pl = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, mode)
            sk.skiparse_attn_fwd(pl, sk.BF16, q, k, v, o1d, stream=stream)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(3):
                sk.skiparse_attn_fwd(pl, sk.BF16, q, k, v, o1d, stream=stream)
            e[1].record(stream)
            torch.cuda.synchronize()
            ms = e[0].elapsed_time(e[1]) / 3
            one_d[name] = {"ms": round(ms, 3), "tflops": round(pl.flops / (ms * 1e-3) / 1e12, 2), "pairs": int(pl.pairs)}
        extras["skiparse_1d_bf16"] = one_d
        progress("Skiparse-1D")
        del o1d
        # pieces of the fp8 attention block at C = heads * d channels: the
        # e4m3 projection GEMM (2 * tokens * C * C FLOPs) and the rotary
        # embedding fused with per-tensor quantization (reads bf16 twice,
        # writes e4m3 once: 5 bytes per element)
        C = nh * d
        M = B * T * H * W
        xq = sk.quantize_fp8(q.reshape(M, C))[0]
        wv = torch.from_numpy(wl.normal_tensor((C, C), w.seed, 5) * np.float32(1.0 / np.sqrt(C))).cuda()
        wq, wsc = sk.quantize_fp8(wv)
        del wv
        ysc = torch.ones(2, dtype=torch.float32, device="cuda")
        yg = torch.empty((M, C), dtype=torch.bfloat16, device="cuda")
        sk.skiparse_gemm_fp8(xq, wq, ysc[0:1], wsc[1:2], yg, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(5):
            sk.skiparse_gemm_fp8(xq, wq, ysc[0:1], wsc[1:2], yg, stream=stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        gms = e[0].elapsed_time(e[1]) / 5
        gfl = 2.0 * M * C * C
        block = {"projection_gemm": {"M": M, "N": C, "K": C, "ms": round(gms, 3),
                                     "tflops": round(gfl / (gms * 1e-3) / 1e12, 1),
                                     "frac_fp8_peak": round(gfl / (gms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4)}}
        del xq, wq, yg
        pl = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, sk.MODE_TOKEN)
        codes_r = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
        rsc = torch.empty(2, dtype=torch.float32, device="cuda")
        rws = torch.empty(sk.skiparse_rope_fp8_workspace_bytes(pl), dtype=torch.uint8, device="cuda")
        sk.skiparse_rope_fp8(pl, q, codes_r, rsc, workspace=rws, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(5):
            sk.skiparse_rope_fp8(pl, q, codes_r, rsc, workspace=rws, stream=stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        rms_ = e[0].elapsed_time(e[1]) / 5
        rbytes = q.numel() * 5
        block["rope_quant"] = {"ms": round(rms_, 3), "GBps": round(rbytes / (rms_ * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(rbytes / (rms_ * 1e-3) / 1e9 / HBM_GBS, 4)}
        del codes_r, rws
        # the whole fp8 block at the 480p workload shape (21 x 32 x 52 tokens,
        # 12 heads, C = 1536): projections, rotary quantizer, attention
        w4 = wl.WORKLOADS["480p"]
        B4, T4, H4, W4, nh4, d4 = w4.shape
        C4, M4 = nh4 * d4, B4 * T4 * H4 * W4
        x4 = torch.from_numpy(wl.normal_tensor((B4, T4, H4, W4, C4), w4.seed, 4)).to(torch.bfloat16).cuda()
        wts = [torch.from_numpy(wl.normal_tensor((C4, C4), w4.seed, 5 + i) * np.float32(1.0 / np.sqrt(C4))).cuda()
               for i in range(4)]
        w_codes, w_scales = sk.quantize_weights(*wts)
        del wts
        for mode, name in ((sk.MODE_TOKEN, "token"), (sk.MODE_GROUP, "group")):
            pl = sk.skiparse_plan_init(B4, T4, H4, W4, nh4, d4, w4.k, mode)
            bf = sk.BlockFP8(w_codes, w_scales, nh4, w4.k, mode)
            y4 = bf(x4)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(5):
                bf(x4, out=y4)
            e[1].record(stream)
            torch.cuda.synchronize()
            ms = e[0].elapsed_time(e[1]) / 5
            flops = pl.flops + 4 * 2 * M4 * C4 * C4
            block[f"block_480p_{name}"] = {"ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                                           "attention_tflop": round(pl.flops / 1e12, 3),
                                           "projection_tflop": round(4 * 2 * M4 * C4 * C4 / 1e12, 3)}
            del y4, bf
        del x4
        # the same block (C = 1536) on the 720P-5s token grid, token-wise
        T7, H7, W7 = 21, 45, 80
        M7 = T7 * H7 * W7
        x7 = torch.from_numpy(wl.normal_tensor((1, T7, H7, W7, C4), w4.seed, 9)).to(torch.bfloat16).cuda()
        pl = sk.skiparse_plan_init(1, T7, H7, W7, nh4, d4, 2, sk.MODE_TOKEN)
        bf = sk.BlockFP8(w_codes, w_scales, nh4, 2, sk.MODE_TOKEN)
        y7 = bf(x7)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(5):
            bf(x7, out=y7)
        e[1].record(stream)
        torch.cuda.synchronize()
        ms = e[0].elapsed_time(e[1]) / 5
        flops = pl.flops + 4 * 2 * M7 * C4 * C4
        block["block_720p_grid_12_heads_token"] = {"ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                                                   "attention_tflop": round(pl.flops / 1e12, 3),
                                                   "projection_tflop": round(4 * 2 * M7 * C4 * C4 / 1e12, 3)}
        del x7, y7, bf
        # the block at its real shape: 720P-5s with all 40 heads (C = 5120);
        # x and the weights are N(0,1) from torch's device generator with a
        # fixed seed (weights scaled by 1/sqrt(C)), rounded to bf16 / e4m3
        Cf = nh * d
        gb = torch.Generator(device="cuda")
        gb.manual_seed(w.seed + 7)
        xf = torch.randn((B, T, H, W, Cf), generator=gb, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        wf = [torch.randn((Cf, Cf), generator=gb, device="cuda", dtype=torch.float32) * (1.0 / np.sqrt(Cf))
              for _ in range(4)]
        wf_codes, wf_scales = sk.quantize_weights(*wf)
        del wf
        for mode, name in ((sk.MODE_TOKEN, "token"), (sk.MODE_GROUP, "group")):
            pl = sk.skiparse_plan_init(B, T, H, W, nh, d, w.k, mode)
            bf = sk.BlockFP8(wf_codes, wf_scales, nh, w.k, mode)
            yf = bf(xf)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(3):
                bf(xf, out=yf)
            e[1].record(stream)
            torch.cuda.synchronize()
            ms = e[0].elapsed_time(e[1]) / 3
            flops = pl.flops + 4 * 2 * M * Cf * Cf
            block[f"block_720p_5s_40_heads_{name}"] = {
                "ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                "attention_tflop": round(pl.flops / 1e12, 3), "projection_tflop": round(4 * 2 * M * Cf * Cf / 1e12, 3)}
            del yf, bf
        del xf, wf_codes, wf_scales
        torch.cuda.empty_cache()
        extras["block_fp8"] = block
        progress("fp8 block")
        del w_codes, w_scales
        del k, v, o_tok, o_grp
        torch.cuda.empty_cache()
        extras["bf16_other_workloads"] = other_workloads(sk, stream, tflops)
        progress("768P-5s and 480P layers")
    result["extras"] = extras

    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
