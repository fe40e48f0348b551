"""Benchmark of the retention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunkwise forward of the 6.7B-shaped training workload (B=2, H=16,
N=8192, d_k=256, d_v=512, chunk 256, bf16 q/k/v/gate, GroupNorm + swish gate, bf16
output, float32 final state) with inputs resident in HBM. The line also carries the
decode step time of the 6.7B-shaped decode workload (batch 128, 16 heads, float32
state updated in place; 1024 sequential steps timed back to back), and secondary records
for the chunkwise backward, the same forward with one decay per (head, coordinate pair),
the gated multi-scale layer around it (projections and output projection) and the
parallel form.

Prints one JSON line. `roofline` describes the fused chunkwise kernel: its average
duration is measured with HIP events recorded on the stream it runs on; achieved
bandwidth = compulsory HBM bytes / duration; `traffic` is the HBM bytes per launch
from the committed rocprofv3 counter summary, reported only while the kernel sources
match the ones it was taken on. `cpu_baseline` times the fp64 oracle on the same
workload (every head, repeated to at least 10 s of CPU time) on this host's cores.

The default warm-up (50 steps, about 35 ms of the headline kernel) lets the GPU clock
reach its steady state before the timed steps: after 5 steps the same kernel reads about
4 % slower.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


CHUNKWISE_PROFILE = os.path.join(ROOT, "profiles", "chunkwise_fused_6p7b_training.md")
CHUNKWISE_SOURCES = ("linear_recurrent_sequence_rn_amd/csrc/chunkwise_mfma.hip",
                     "linear_recurrent_sequence_rn_amd/csrc/rn_device.h")


def chunkwise_source_hash() -> str:
    """sha256 over the fused chunkwise kernel's sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for rel in CHUNKWISE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic():
    """HBM bytes per launch of the fused chunkwise kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary was taken on other kernel
    sources than the ones built now."""
    try:
        with open(CHUNKWISE_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    src, traffic = None, None
    for line in text.splitlines():
        line = line.strip().strip("`")
        if line.startswith("kernel source sha256:"):
            src = line.split(":", 1)[1].strip()
        elif line.startswith("traffic bytes per launch:"):
            traffic = int(line.split(":", 1)[1].strip())
    if src is None or traffic is None or src != chunkwise_source_hash():
        return None
    return traffic


def chunkwise_work(B, H, N, dk, dv, C, gate=True):
    """Algorithmic flops and compulsory HBM bytes of one chunkwise forward with
    GroupNorm (+ gate): causal intra-chunk pairs (C+1)(dk+dv) per token, cross term and
    state carry 2*dk*dv each per token; bytes: q, k, v (and gate) read, out written
    (bf16), final state written (fp32)."""
    th = B * H * N
    flops = th * ((C + 1) * (dk + dv) + 4 * dk * dv)
    bytes_ = th * 2 * (dk + dk + dv + (dv if gate else 0) + dv) + B * H * dk * dv * 4
    return flops, bytes_


def parallel_work(B, H, N, dk, dv):
    """Causal pairs only: N(N+1)/2 (q.k and p.v) per head; bytes: q, k, v read and out
    written once (bf16)."""
    flops = B * H * N * (N + 1) * (dk + dv)
    bytes_ = B * H * N * 2 * (dk + dk + dv + dv)
    return flops, bytes_


def decode_work(B, H, dk, dv):
    flops = 5 * B * H * dk * dv
    bytes_ = B * H * dk * dv * 4 * 2 + B * H * (dk + dk + dv) * 2 + B * H * dv * 4
    return flops, bytes_


def warm_up(fn, min_ms=60.0, max_calls=400):
    """Calls fn until at least min_ms of GPU time has passed (the clock needs tens of ms
    to reach its steady state after an idle spell, such as the host-side input
    generation before each secondary record), so that every record is timed at steady
    clocks like the headline."""
    import torch
    total, calls = 0.0, 0
    while total < min_ms and calls < max_calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            fn()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
        calls += 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-parallel", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-pair", action="store_true")
    ap.add_argument("--no-schedules", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the chunkwise kernel's source hash (as recorded in its profile) and exit")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--only", choices=["chunkwise", "decode", "parallel", "backward", "pair", "layer",
                                       "long", "copy"],
                    default=None,
                    help="run one workload only (for profiling); 'copy' times a plain 1 GiB "
                         "device copy, the reference for the HBM byte counters")
    args = ap.parse_args()
    if args.source_hash:
        print(chunkwise_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the retention heads shard over GPUs without communication, so the "
              "whole-job figure is N times the one-GPU figure, which is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_recurrent_sequence_rn_amd as rn
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "copy":
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "copy_GBs": 2 * src.numel() * 4 / dt / 1e9}))
        return
    if args.only in ("decode", "parallel", "backward", "pair", "layer", "long"):
        args.no_cpu_baseline = True
    w = W.WORKLOADS["chunkwise_6p7b"]
    x = W.make_inputs(w)
    q, k, v, gate = (x[n].to(dev) for n in ("q", "k", "v", "gate"))
    gamma, theta = x["gamma"], x["theta"]
    out = torch.empty_like(v)
    S_out = torch.empty(w.B, w.H, w.d_k, w.d_v, dtype=torch.float32, device=dev)
    nws = rn.rn_chunkwise_workspace_bytes(q, v, gamma, theta, w.chunk, gn=True, gate=gate)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step():
        rn.rn_retention_chunkwise(q, k, v, gamma, theta, w.chunk, gate=gate, gn=True,
                                  gn_eps=w.gn_eps, state_out=S_out, out=out, workspace=ws)

    if args.only in ("decode", "parallel", "backward", "pair", "layer", "long"):
        args.steps = args.warmup = 1
    if args.only is not None and args.only != "long":
        args.no_long = True
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    kern_s = float(np.mean(durs_ms)) / 1e3
    tokens = w.B * w.N
    value = tokens * args.steps / wall
    flops, bytes_ = chunkwise_work(w.B, w.H, w.N, w.d_k, w.d_v, w.chunk)
    gbs = bytes_ / kern_s / 1e9
    tfl = flops / kern_s / 1e12

    rec = {
        "metric": "retention tokens/s (chunkwise fwd N=8192) + decode step us; % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the type the matrix products compute in: bf16 inputs are rounded to IEEE half
        # for every MFMA operand (3 more significand bits than bf16), fp32 accumulation
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "chunkwise_6p7b: B=2 H=16 N=8192 d_k=256 d_v=512 chunk=256, "
                               "bf16 in/out, GroupNorm+swish gate, fp32 final state",
                   "global_batch": w.B, "seq_len": w.N, "heads": w.H, "d_k": w.d_k, "d_v": w.d_v,
                   "chunk": w.chunk, "io_dtype": "bf16", "mfma_operands": "f16",
                   "accumulate": "fp32"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": profiled_traffic(),
                     "kernel": "chunkwise_fused", "kernel_ms": kern_s * 1e3,
                     "algorithmic_bytes": bytes_, "algorithmic_flops": flops,
                     "effective_tflops": tfl, "effective_mfma_frac": tfl / BF16_PEAK_TFLOPS},
    }

    # ---- the other chunkwise schedules on the same workload (secondary record) ------------
    # Same inputs and outputs, same result: the segmented schedule (segment-local states,
    # scan, outputs) and the chunk-parallel pair (state snapshots, outputs).
    if args.only is not None:
        args.no_schedules = True
    if not args.no_schedules:
        sched = {"workload": "chunkwise_6p7b, the headline call with another schedule flag",
                 "sequential_ms": kern_s * 1e3}
        for name, kw in (("segmented", dict(segmented=True)), ("pair", dict(chunk_parallel=True))):
            wss = torch.empty(rn.rn_chunkwise_workspace_bytes(q, v, gamma, theta, w.chunk, gn=True, gate=gate, **kw),
                              dtype=torch.uint8, device=dev)

            def sstep():
                rn.rn_retention_chunkwise(q, k, v, gamma, theta, w.chunk, gate=gate, gn=True,
                                          gn_eps=w.gn_eps, state_out=S_out, out=out, workspace=wss, **kw)

            warm_up(sstep)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                sstep()
            e1.record(stream)
            torch.cuda.synchronize()
            sched[name + "_ms"] = e0.elapsed_time(e1) / reps
            del wss
        rec["schedules"] = sched

    # ---- chunkwise backward on the same workload (secondary record) ------------------
    # Gradients of q, k, v and the gate through GroupNorm + gate, given a random dout; the
    # tile products on matrix cores (f16 operands), the state scans in float32.
    # Algorithmic flops: twice the forward's (each product of the forward has two gradient
    # products of the same size).
    if args.only in ("chunkwise", "decode", "parallel", "pair", "layer", "long"):
        args.no_backward = True
    if not args.no_backward:
        dout = torch.randn(v.shape, generator=torch.Generator(device=dev).manual_seed(5),
                           device=dev).to(torch.bfloat16)
        wsb = torch.empty(rn.rn_chunkwise_backward_workspace_bytes(q, v, gamma, theta, w.chunk, gn=True, gate=gate),
                          dtype=torch.uint8, device=dev)

        def bstep():
            rn.rn_retention_chunkwise_backward(q, k, v, gamma, theta, w.chunk, dout, gate=gate, gn=True,
                                               workspace=wsb)

        warm_up(bstep)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bs = e0.elapsed_time(e1) / reps / 1e3
        bfl = 2 * flops
        rec["backward"] = {"workload": "chunkwise_6p7b backward: dq, dk, dv, dgate through GroupNorm + gate",
                           "ms": bs * 1e3, "tokens_per_s": tokens / bs,
                           "algorithmic_flops": bfl, "tflops": bfl / bs / 1e12,
                           "bound": "mfma", "mfma_frac": bfl / bs / 1e12 / BF16_PEAK_TFLOPS,
                           "workspace_bytes": wsb.numel()}
        del dout, wsb
    if args.only == "backward":
        args.no_parallel = True
        args.no_decode = True
        args.no_pair = True
        args.no_layer = True

    # ---- the same forward with one decay per (head, coordinate pair) -------------------
    # Chunk-parallel pair of kernels (state snapshots, then outputs) with the decays
    # folded into the operands per coordinate; same algorithmic bytes and flops as the
    # per-head-decay forward.
    if args.only in ("chunkwise", "decode", "parallel", "layer", "long"):
        args.no_pair = True
    if args.only == "pair":
        args.no_parallel = True
        args.no_decode = True
        args.no_layer = True
    if not args.no_pair:
        wv = W.WORKLOADS["chunkwise_6p7b_pair"]
        xv = W.make_inputs(wv)
        qv, kv, vv, gv = (xv[n].to(dev) for n in ("q", "k", "v", "gate"))
        gpair = torch.from_numpy(xv["gamma"]).to(dev)
        outv = torch.empty_like(vv)
        Sv = torch.empty(wv.B, wv.H, wv.d_k, wv.d_v, dtype=torch.float32, device=dev)
        wsv = torch.empty(rn.rn_chunkwise_workspace_bytes(qv, vv, gpair, xv["theta"], wv.chunk, gn=True,
                                                          gate=gv), dtype=torch.uint8, device=dev)

        def vstep():
            rn.rn_retention_chunkwise(qv, kv, vv, gpair, xv["theta"], wv.chunk, gate=gv, gn=True,
                                      gn_eps=wv.gn_eps, state_out=Sv, out=outv, workspace=wsv)

        warm_up(vstep)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            vstep()
        e1.record(stream)
        torch.cuda.synchronize()
        vs = e0.elapsed_time(e1) / reps / 1e3
        vfl, vby = chunkwise_work(wv.B, wv.H, wv.N, wv.d_k, wv.d_v, wv.chunk)
        rec["pair_decay"] = {"workload": "chunkwise_6p7b_pair: the chunkwise_6p7b shape with one decay "
                                         "per (head, coordinate pair), 1 - 2^-(5 + 4h/16 + 4j/127)",
                             "ms": vs * 1e3, "tokens_per_s": wv.B * wv.N / vs,
                             "bound": "hbm", "achieved_GBs": vby / vs / 1e9,
                             "hbm_frac": vby / vs / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": vby, "algorithmic_flops": vfl,
                             "mfma_tflops": vfl / vs / 1e12, "kernels": "cp_states + cp_outputs"}
        del xv, qv, kv, vv, gv, outv, Sv, wsv

    # ---- the gated multi-scale layer around the same retention ---------------------------
    # x [2, 8192, 4096] -> projections (rocBLAS bf16 GEMMs) -> fused chunkwise retention
    # with GroupNorm + gate -> heads regrouped by token -> W_O. Algorithmic flops: the five
    # projections plus the retention's.
    if args.only in ("chunkwise", "decode", "parallel", "long"):
        args.no_layer = True
    if args.only == "layer":
        args.no_parallel = True
        args.no_decode = True
    if not args.no_layer:
        D = W.LAYER_D_MODEL
        xl = W.make_layer_inputs(w, D)
        lt = {n: xl[n].to(dev) for n in ("x", "w_q", "w_k", "w_v", "w_g", "w_o")}
        outl = torch.empty(w.B, w.N, D, dtype=torch.bfloat16, device=dev)
        wsl = torch.empty(rn.rn_msr_layer_workspace_bytes(lt["x"], w.H, w.d_k, w.d_v, xl["gamma"],
                                                          xl["theta"], w.chunk), dtype=torch.uint8,
                          device=dev)

        def lstep():
            rn.rn_msr_layer_forward(lt["x"], lt["w_q"], lt["w_k"], lt["w_v"], lt["w_g"], lt["w_o"],
                                    xl["gamma"], xl["theta"], w.H, w.d_k, w.d_v, w.chunk,
                                    out=outl, workspace=wsl)

        warm_up(lstep)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            lstep()
        e1.record(stream)
        torch.cuda.synchronize()
        ls = e0.elapsed_time(e1) / reps / 1e3
        tok = w.B * w.N
        gemm_fl = 2 * tok * D * (2 * w.H * w.d_k + 2 * w.H * w.d_v) + 2 * tok * w.H * w.d_v * D
        lfl = gemm_fl + flops
        rec["layer"] = {"workload": f"gated multi-scale layer on chunkwise_6p7b: x [2, 8192, {D}] bf16, "
                                    "W_Q/W_K [4096, 4096], W_V/W_G [4096, 8192], W_O [8192, 4096], "
                                    "GroupNorm + swish gate, bf16 out",
                        "ms": ls * 1e3, "tokens_per_s": tok / ls, "bound": "mfma",
                        "algorithmic_flops": lfl, "gemm_flops": gemm_fl, "tflops": lfl / ls / 1e12,
                        "mfma_frac": lfl / ls / 1e12 / BF16_PEAK_TFLOPS,
                        "workspace_bytes": wsl.numel()}
        del xl, lt, outl, wsl

    # ---- parallel form, 1.3B shape (secondary record) --------------------------------
    if args.only in ("chunkwise", "decode", "long"):
        args.no_parallel = True
    if args.only == "parallel":
        args.no_decode = True
    if not args.no_parallel:
        del q, k, v, gate, out, ws
        wp = W.WORKLOADS["parallel_1p3b"]
        xp = W.make_inputs(wp)
        qp, kp, vp = (xp[n].to(dev) for n in ("q", "k", "v"))
        outp = torch.empty_like(vp)
        wsp = torch.empty(rn.rn_parallel_workspace_bytes(qp, vp, xp["gamma"], xp["theta"], norm_d=True,
                                                         norm_r=True, gn=True), dtype=torch.uint8, device=dev)

        def pstep():
            rn.rn_retention_parallel(qp, kp, vp, xp["gamma"], xp["theta"], out=outp, workspace=wsp,
                                     qk_scale=wp.qk_scale, norm_d=True, norm_r=True, gn=True)

        warm_up(pstep)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            pstep()
        e1.record(stream)
        torch.cuda.synchronize()
        ps = e0.elapsed_time(e1) / reps / 1e3
        pfl, pby = parallel_work(wp.B, wp.H, wp.N, wp.d_k, wp.d_v)
        rec["parallel"] = {"workload": "parallel_1p3b: B=8 H=8 N=2048 d_k=256 d_v=512, alpha=1/16, "
                                       "D and R row normalisation, GroupNorm, bf16 in/out",
                           "ms": ps * 1e3, "tokens_per_s": wp.B * wp.N / ps,
                           "mfma_tflops": pfl / ps / 1e12, "mfma_frac": pfl / ps / 1e12 / BF16_PEAK_TFLOPS,
                           "algorithmic_flops": pfl, "algorithmic_bytes": pby,
                           "hbm_frac": pby / ps / 1e9 / HBM_PEAK_GBS}
        del xp, qp, kp, vp, outp, wsp

    # ---- long sequences (secondary record) ---------------------------------------------
    # B=1, H=16, chunk 512, GroupNorm, bf16 in/out, fp32 final state, default schedule, at
    # N = 16K, 32K and 64K tokens: time per call, roofline fractions and the peak device
    # memory of the call's tensors (inputs, output, state and workspace; the workspace
    # does not grow with N).
    if not args.no_long:
        if args.only == "long":
            del q, k, v, gate, out, ws
        wl_ = W.WORKLOADS["chunkwise_long"]
        long_rec = {"workload": "chunkwise_long: B=1 H=16 d_k=256 d_v=512 chunk=512, bf16 in/out, "
                                "GroupNorm, fp32 final state, default (sequential) schedule",
                    "by_N": {}}
        for Nl in (16384, 32768, 65536):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            xl_ = W.make_inputs(wl_, N=Nl)
            ql, kl, vl = (xl_[n].to(dev) for n in ("q", "k", "v"))
            outl_ = torch.empty_like(vl)
            Sl = torch.empty(wl_.B, wl_.H, wl_.d_k, wl_.d_v, dtype=torch.float32, device=dev)
            wsl_ = torch.empty(rn.rn_chunkwise_workspace_bytes(ql, vl, xl_["gamma"], xl_["theta"], wl_.chunk,
                                                               gn=True), dtype=torch.uint8, device=dev)

            def lgstep():
                rn.rn_retention_chunkwise(ql, kl, vl, xl_["gamma"], xl_["theta"], wl_.chunk, gn=True,
                                          gn_eps=wl_.gn_eps, state_out=Sl, out=outl_, workspace=wsl_)

            warm_up(lgstep)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                lgstep()
            e1.record(stream)
            torch.cuda.synchronize()
            ts = e0.elapsed_time(e1) / reps / 1e3
            lfl, lby = chunkwise_work(wl_.B, wl_.H, Nl, wl_.d_k, wl_.d_v, wl_.chunk, gate=False)
            long_rec["by_N"][str(Nl)] = {
                "ms": ts * 1e3, "tokens_per_s": wl_.B * Nl / ts,
                "achieved_GBs": lby / ts / 1e9, "hbm_frac": lby / ts / 1e9 / HBM_PEAK_GBS,
                "effective_tflops": lfl / ts / 1e12,
                "effective_mfma_frac": lfl / ts / 1e12 / BF16_PEAK_TFLOPS,
                "algorithmic_bytes": lby, "algorithmic_flops": lfl,
                "workspace_bytes": wsl_.numel(),
                "max_memory_allocated_bytes": torch.cuda.max_memory_allocated(dev) - base}
            del xl_, ql, kl, vl, outl_, Sl, wsl_
        rec["long"] = long_rec

    # ---- decode step ---------------------------------------------------------------
    if args.only in ("chunkwise", "parallel", "long"):
        args.no_decode = True
    if not args.no_decode:
        wd = W.WORKLOADS["decode_6p7b"]
        state = W.initial_state(wd).to(dev)
        n_in = 32
        ins = [W.make_decode_step_inputs(wd, i) for i in range(n_in)]
        ins = [{kk: t.to(dev) for kk, t in d.items()} for d in ins]
        dout = torch.empty(wd.B, wd.H, 1, wd.d_v, dtype=torch.float32, device=dev)
        g_d, th_d = wd.gamma(), wd.theta()
        wi = [0]

        def dstep():
            d = ins[wi[0] % n_in]
            rn.rn_retention_recurrent_step(d["q"], d["k"], d["v"], g_d, th_d, state, wi[0], out=dout,
                                           out_dtype=torch.float32)
            wi[0] += 1

        warm_up(dstep)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            d = ins[i % n_in]
            rn.rn_retention_recurrent_step(d["q"], d["k"], d["v"], g_d, th_d, state, i, out=dout,
                                           out_dtype=torch.float32)
        e1.record(stream)
        torch.cuda.synchronize()
        step_us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        dfl, dby = decode_work(wd.B, wd.H, wd.d_k, wd.d_v)
        rec["decode_step_us"] = step_us
        rec["decode"] = {"workload": "decode_6p7b: batch 128, H=16, d_k=256, d_v=512, fp32 state in place, "
                                     f"{args.decode_steps} sequential steps",
                         "tokens_per_s": wd.B / (step_us * 1e-6),
                         "achieved_GBs": dby / (step_us * 1e-6) / 1e9,
                         "hbm_frac": dby / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": dby}
        del state

    # ---- CPU baseline: the fp64 oracle on the same workload ---------------------------
    # The whole workload (every head, full length, GroupNorm + gate) is run through the
    # oracle, repeated until at least 10 s of CPU time have been spent (at most 3 passes).
    if not args.no_cpu_baseline:
        import oracle as O
        cores = cpu_cores()
        heads = w.B * w.H
        passes, t_total = 0, 0.0
        while passes < 3 and (passes == 0 or t_total < 10.0):
            t0 = time.perf_counter()
            for b in range(w.B):
                for hh in range(w.H):
                    sl = (slice(b, b + 1), slice(hh, hh + 1))
                    raw, _ = O.chunkwise(x["q"][sl], x["k"][sl], x["v"][sl], gamma[hh:hh + 1], theta, w.chunk)
                    O.groupnorm_gate(raw, x["gate"][sl], w.gn_eps)
            t_total += time.perf_counter() - t0
            passes += 1
        t_pass = t_total / passes
        rec["cpu_baseline"] = {"value": tokens / t_pass, "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"the whole chunkwise_6p7b workload ({heads} heads x N={w.N}, "
                                         f"chunk {w.chunk}, GroupNorm+gate) in fp64, {passes} pass(es), "
                                         f"{t_pass:.2f} s per pass"}
        secondary_cpu_baselines(rec, args, O, W, cores)
    print(json.dumps(rec))
    teardown()


def cpu_cores() -> int:
    """Threads the oracle's numpy calls use on this host."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def secondary_cpu_baselines(rec, args, O, W, cores):
    """The fp64 oracle on bounded samples of the secondary workloads (about 10 s each)."""
    if "parallel" in rec:
        wp = W.WORKLOADS["parallel_1p3b"]
        xp = W.make_inputs(wp)
        t0 = time.perf_counter()
        for b in range(wp.B):
            for hh in range(wp.H):
                sl = (slice(b, b + 1), slice(hh, hh + 1))
                raw = O.parallel(xp["q"][sl], xp["k"][sl], xp["v"][sl], xp["gamma"][hh:hh + 1],
                                 xp["theta"], 0, wp.qk_scale, True, True)
                O.group_norm(raw, wp.gn_eps)
        t = time.perf_counter() - t0
        rec["parallel"]["cpu_baseline"] = {
            "value": wp.B * wp.N / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole parallel_1p3b workload ({wp.B * wp.H} heads x N={wp.N}, D and R "
                      f"normalisation, GroupNorm) in fp64, {t:.2f} s"}
    if "decode" in rec:
        wd = W.WORKLOADS["decode_6p7b"]
        S0 = W.initial_state(wd)
        nsteps, nb = 4, 16
        states = [S0[b0:b0 + nb] for b0 in range(0, wd.B, nb)]
        g_d, th_d = wd.gamma(), wd.theta()
        t = 0.0
        for i in range(nsteps):
            d = W.make_decode_step_inputs(wd, i)
            t0 = time.perf_counter()
            for j, b0 in enumerate(range(0, wd.B, nb)):
                sl = (slice(b0, b0 + nb),)
                _, states[j] = O.recurrent_step(d["q"][sl], d["k"][sl], d["v"][sl], g_d, th_d, i, 1.0,
                                                states[j])
            t += time.perf_counter() - t0
        rec["decode"]["cpu_baseline"] = {
            "value": wd.B * nsteps / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "step_us": t / nsteps * 1e6,
            "sample": f"{nsteps} decode steps of the whole decode_6p7b batch ({wd.B} x {wd.H} heads, "
                      f"256 x 512 states) in fp64, {t:.2f} s"}
    if "long" in rec:
        wl_ = W.WORKLOADS["chunkwise_long"]
        heads = [0, 5, 11, 15]
        x = W.make_inputs(wl_)
        t0 = time.perf_counter()
        for hh in heads:
            sl = (slice(0, 1), slice(hh, hh + 1))
            raw, _ = O.chunkwise(x["q"][sl], x["k"][sl], x["v"][sl], x["gamma"][hh:hh + 1], x["theta"],
                                 wl_.chunk)
            O.group_norm(raw, wl_.gn_eps)
        t = (time.perf_counter() - t0) * wl_.H / len(heads)
        rec["long"]["cpu_baseline"] = {
            "value": wl_.B * wl_.N / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(heads)} of the {wl_.H} heads of chunkwise_long at N={wl_.N} (chunk "
                      f"{wl_.chunk}, GroupNorm) in fp64, time scaled by {wl_.H // len(heads)} to the "
                      f"whole workload: {t:.2f} s"}


def teardown():
    """Ends the run with every launch finished and every tensor released before the
    interpreter exits (so nothing of the library's or torch's GPU state is freed while a
    profiler that wraps the process finalises)."""
    import gc

    import torch
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
