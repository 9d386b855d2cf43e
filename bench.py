#!/usr/bin/env python3
"""Benchmark of the KDA operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D] [--no-cpu]

A step is one kda_chunk_fwd over the T=8192, H=96, d=128 bf16 prefill
(S0 = 0, final state returned); the headline value is prefill tokens/s
(8192 tokens per step, all 96 heads).  The same run measures the decode
step on B=256 requests x H=96 heads with a 1.6 GB fp32 state chained over
D steps and reports the state GB/s (state read + write per step / step
time).  Inputs are seeded synthetic data resident in HBM before the timed
regions; timing uses HIP events on the stream the kernels run on.

Order of the run: W + K launches of the headline prefill on the idle GPU
(reported as its cold launch time), the informational paths (1M-token
prefill, packed varlen prefill, multi-token decode, layer steps, backward),
the decode step, then the headline prefill: --settle-seconds (0.3) of
untimed launches, W warm-up launches and K timed ones.  The GPU raises its
clocks only after tens of milliseconds of sustained load, and a serving
deployment runs at those clocks; the cold figure is reported beside it.

Prints one JSON line (rank 0) with the metric, a roofline object for the
prefill kernel (mean, median and minimum launch times; the roofline uses the
mean), one for the decode kernel under "decode", and the fp64 CPU oracle
timed on a bounded sample of the same workload.
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

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
KDA_BWD_WINDOW = 2048           # the backward's default window (include/kda.h)
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix
PEAK_F32_TFLOPS = 157.3         # MI355X dense fp32 matrix
N_XCD = 8                       # MI355X accelerator complex dies
N_SIMD = 1024                   # 256 compute units x 4 SIMDs
# Backward pass, algorithmic flops per token and head: the forward pass it
# repeats (131072) plus its own products per 32-token chunk (P, M: 2 x
# 2*32*32*128; the state-gradient walk: K_end dS, Q+^T dO, Kb^T W at
# 2*32*128*128 and M^T dO, T^T dU at 2*32*32*128; the gradient kernel: dO S^T,
# W S^T, U Sn^T at 2*32*128*128 and dM, dA', dM Y, dPm Y, dM^T Qr, dPm^T X at
# 2*32*32*128), 8912896 per chunk = 278528 per token.
BWD_FLOPS_PER_TOKEN_HEAD = 131072 + 278528
PREFILL_BYTES_PER_TOKEN_HEAD = 1796      # q,k,v bf16 768 + log alpha 512 + beta 4 + o fp32 512
PREFILL_FLOPS_PER_TOKEN_HEAD = 131072    # chunkwise algorithm, 64-token chunks, d = 128
STATE_BYTES = 128 * 128 * 4
DECODE_INPUT_BYTES_PER_STATE = 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4   # q,k,v + log alpha + beta + o
DECODE_FLOPS_PER_STATE = 7 * 128 * 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run one path only (for profiler runs); prints no JSON line")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed launches of the headline kernel before its warm-up steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the repeated oracle runs")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the informational 1M-token prefill and multi-token decode runs")
    return ap.parse_args()


def long_context(torch, kda, W, dev, reps=3):
    """The T=1,048,576, H=16 prefill (for information): few (sequence, head)
    pairs, so kda_chunk_fwd takes its sequence-parallel path.  Inputs are drawn
    on the device with torch's seeded generator in the workload's
    distributions (generating 1M tokens x 16 heads on the host would dominate
    the run)."""
    w = W.workload(3)
    T, H = w.T, w.H
    g = torch.Generator(device=dev).manual_seed(2026)
    shp = (1, T, H, 128)
    nrm = torch.nn.functional.normalize
    q = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    k = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.randn(shp, device=dev, generator=g).to(torch.bfloat16)
    la = -5.0 * torch.sigmoid(torch.randn(shp, device=dev, generator=g))
    b = torch.sigmoid(torch.randn((1, T, H), device=dev, generator=g))
    o = torch.empty(shp, dtype=torch.float32, device=dev)
    st = torch.empty((1, H, 128, 128), dtype=torch.float32, device=dev)
    ws_bytes = kda.chunk_fwd_workspace_bytes(1, T, H, varlen=False)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, sp in (("sequence_parallel", True), ("sequential", False)):
        n = reps if sp else 1
        kda.chunk_fwd(q, k, v, la, b, None, None, o=o, S_T=st, workspace=ws if sp else None,
                      sequence_parallel=sp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            kda.chunk_fwd(q, k, v, la, b, None, None, o=o, S_T=st, workspace=ws if sp else None,
                          sequence_parallel=sp)
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / n
    del q, k, v, la, b, o, st, ws
    torch.cuda.empty_cache()
    ms = out["sequence_parallel"]
    return {"workload": f"KDA prefill B=1 T={T} H={H} d=128 bf16, S0=0 (device-drawn inputs)",
            "tokens_per_s": T / (ms * 1e-3), "ms": ms,
            "sequential_path_ms": out["sequential"],
            "path": "sequence-parallel: the first segment from S0 beside the middle segments from zero and from the identity, merge, the middle segments rerun beside the last one",
            "workspace_bytes": ws_bytes}


def multi_token_decode(torch, kda, W, dev, T=8, reps=5):
    """Recurrent decode of T tokens per request on the decode workload's state
    (B=256, H=96; for information), and one speculative step: replay of the
    accepted prefix of 4 earlier drafts, then 4 new drafts without commit.
    Inputs are drawn on the device (torch's seeded generator, the workload's
    distributions)."""
    wd = W.workload(4)
    B, H = wd.B, wd.H
    g = torch.Generator(device=dev).manual_seed(7)
    S = torch.from_numpy(W.decode_state(wd)).to(dev)
    nrm = torch.nn.functional.normalize

    def toks(n):
        shp = (B, n, H, 128)
        return (nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16),
                nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16),
                torch.randn(shp, device=dev, generator=g).to(torch.bfloat16),
                -5.0 * torch.sigmoid(torch.randn(shp, device=dev, generator=g)),
                torch.sigmoid(torch.randn((B, n, H), device=dev, generator=g)))

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    new = toks(T)
    o = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)
    ms = timed(lambda: kda.recurrent_fwd(*new, S, o=o))
    rep, drafts = toks(4), toks(4)
    n_acc = torch.randint(0, 5, (B,), device=dev, generator=g, dtype=torch.int32)
    o4 = torch.empty((B, 4, H, 128), dtype=torch.float32, device=dev)
    ms_spec = timed(lambda: kda.recurrent_fwd(*drafts, S, replay=rep, n_replay=n_acc,
                                              commit=False, o=o4))
    del S, new, rep, drafts, o, o4
    torch.cuda.empty_cache()
    # algorithmic bytes: the fp32 state read and written once, and per token
    # q, k, v (bf16), log alpha, o (fp32) and beta
    nbytes = B * H * (2 * 128 * 128 * 4 + T * (3 * 128 * 2 + 2 * 128 * 4 + 4))
    return {"workload": f"KDA recurrent decode B={B} H={H} d=128, {T} tokens per request, "
                        "fp32 state in place (device-drawn inputs)",
            "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "ms_per_token": ms / T,
            "hbm_bytes_algorithmic": nbytes,
            "hbm_frac": nbytes / (ms * 1e-3) / (PEAK_HBM_GBPS * 1e9),
            "speculative_step_ms": ms_spec,
            "speculative_step": "replay of up to 4 accepted drafts + 4 new drafts, commit after replay"}


def layer_steps(torch, kda, W, dev, reps=10):
    """The layer prologue and epilogue around the headline prefill shape
    (T=8192, H=96; for information): both stream HBM once, so they are
    reported against the HBM roofline with their algorithmic bytes."""
    w = W.workload(1)
    T, H = w.T, w.H
    g = torch.Generator(device=dev).manual_seed(11)
    shp = (1, T, H, 128)
    raw = [torch.randn(shp, device=dev, generator=g).to(torch.bfloat16) for _ in range(3)]
    conv_w = 0.5 * torch.randn((3, H, 128, 4), device=dev, generator=g)
    a = torch.randn(shp, device=dev, generator=g)
    b = torch.randn((1, T, H), device=dev, generator=g)
    cache = torch.randn((1, 3, 3, H, 128), device=dev, generator=g)
    o = torch.randn(shp, device=dev, generator=g)
    gate = torch.randn(shp, device=dev, generator=g)
    wn = 1.0 + 0.1 * torch.randn(128, device=dev, generator=g)
    out = torch.empty_like(o)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_p = timed(lambda: kda.prologue(*raw, conv_w, a, b, cache))
    ms_e = timed(lambda: kda.epilogue(o, gate, wn, out=out))
    th = T * H
    bytes_p = th * (3 * 256 + 512 + 4 + 3 * 256 + 512 + 4)   # raw q,k,v + a + b in; q,k,v + log_alpha + beta out
    bytes_e = th * 3 * 512                                     # o, g in; out
    del raw, a, b, cache, o, gate, out
    torch.cuda.empty_cache()
    return {"workload": f"layer prologue / epilogue at T={T} H={H} d=128 (bf16 raw q,k,v; device-drawn)",
            "prologue_ms": ms_p, "prologue_gbps": bytes_p / (ms_p * 1e-3) / 1e9,
            "prologue_hbm_frac": bytes_p / (ms_p * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "epilogue_ms": ms_e, "epilogue_gbps": bytes_e / (ms_e * 1e-3) / 1e9,
            "epilogue_hbm_frac": bytes_e / (ms_e * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "bytes_per_token_head": {"prologue": bytes_p // th, "epilogue": bytes_e // th}}


def backward_step(torch, kda, W, dev, reps=5):
    """kda_chunk_bwd on the headline prefill shape (T=8192, H=96, bf16) with
    an upstream gradient on o and on the final state (for information)."""
    w = W.workload(1)
    T, H = w.T, w.H
    g = torch.Generator(device=dev).manual_seed(13)
    shp = (1, T, H, 128)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)
    q = unit(torch.randn(shp, device=dev, generator=g)).to(torch.bfloat16)
    k = unit(torch.randn(shp, device=dev, generator=g)).to(torch.bfloat16)
    v = torch.randn(shp, device=dev, generator=g).to(torch.bfloat16)
    la = -5.0 * torch.sigmoid(torch.randn(shp, device=dev, generator=g))
    beta = torch.sigmoid(torch.randn((1, T, H), device=dev, generator=g))
    go = torch.randn(shp, device=dev, generator=g)
    gst = torch.randn((1, H, 128, 128), device=dev, generator=g)
    stream = torch.cuda.current_stream(dev)

    def timed(ws):
        kda.chunk_bwd(q, k, v, la, beta, None, go, gst, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            kda.chunk_bwd(q, k, v, la, beta, None, go, gst, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the default workspace (2048-token windows), then one window per sequence
    ws_default = kda.chunk_bwd_workspace_bytes(1, T, H)
    ws_one = kda.chunk_bwd_workspace_bytes(1, T, H, window_tokens=T)
    ws = torch.empty(ws_default, dtype=torch.uint8, device=dev)
    ms = timed(ws)
    del ws
    ws = torch.empty(ws_one, dtype=torch.uint8, device=dev)
    ms_one = timed(ws)
    flops = BWD_FLOPS_PER_TOKEN_HEAD * T * H
    del q, k, v, la, beta, go, gst, ws
    torch.cuda.empty_cache()
    return {"workload": f"KDA backward B=1 T={T} H={H} d=128, bf16 q/k/v, fp32 gates, "
                        "dL/do and dL/dS_T ~ N(0,1) (device-drawn)",
            "ms": ms, "tokens_per_s": T / (ms * 1e-3),
            "workspace_bytes": ws_default,
            "algorithmic_flops": flops, "tflops_algorithmic": flops / (ms * 1e-3) / 1e12,
            "mfma_f32_peak_tflops": PEAK_F32_TFLOPS,
            "frac_f32_peak": flops / (ms * 1e-3) / 1e12 / PEAK_F32_TFLOPS,
            "single_window": {"ms": ms_one, "workspace_bytes": ws_one},
            "passes": "forward keeping chunk states, V - K+S and U; chunk matrices; "
                      "reverse state-gradient walk; per-chunk gradients; equal lengths run in "
                      f"windows of {KDA_BWD_WINDOW} tokens, last first (the states at window starts "
                      "from a forward pass without per-chunk outputs)"}


def varlen_prefill(torch, kda, W, dev, reps=3):
    """The packed-batch prefill (for information): 32 sequences with seeded
    lengths in [512, 16384] (the varlen workload's own lengths), H=96, with
    per-sequence initial states.  Inputs are drawn on the device with torch's
    seeded generator in the workload's distributions."""
    w = W.workload(2)
    cu = W.cu_seqlens(w)
    T, H, N = int(cu[-1]), w.H, len(cu) - 1
    g = torch.Generator(device=dev).manual_seed(2027)
    shp = (T, H, 128)
    nrm = torch.nn.functional.normalize
    q = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    k = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.randn(shp, device=dev, generator=g).to(torch.bfloat16)
    la = -5.0 * torch.sigmoid(torch.randn(shp, device=dev, generator=g))
    b = torch.sigmoid(torch.randn((T, H), device=dev, generator=g))
    S0 = 0.02 * torch.randn((N, H, 128, 128), device=dev, generator=g)
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(dev)
    o = torch.empty(shp, dtype=torch.float32, device=dev)
    st = torch.empty((N, H, 128, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(N, T, H, varlen=True), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: kda.chunk_fwd(q, k, v, la, b, S0, cu_d, o=o, S_T=st, workspace=ws)
    run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del q, k, v, la, b, S0, o, st, ws
    torch.cuda.empty_cache()
    med = float(np.median(ms))
    lens = np.diff(cu)
    return {"workload": f"KDA packed prefill, {N} sequences of {int(lens.min())}..{int(lens.max())} "
                        f"tokens (total {T}), H={H} d=128 bf16, S0 ~ N(0, 0.02^2) (device-drawn inputs)",
            "tokens_per_s": T / (med * 1e-3), "ms_median": med, "ms_min": float(np.min(ms)),
            "launches": reps,
            "hbm_bytes_algorithmic": T * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * N * H * STATE_BYTES,
            "hbm_frac": (T * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * N * H * STATE_BYTES)
                        / (med * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def run_decode_only(args, torch, kda, W, dev):
    wd = W.workload(4)
    S = torch.from_numpy(W.decode_state(wd)).to(dev)
    x = W.decode_inputs(wd, 0)
    e = {n: torch.from_numpy(x[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v")}
    e["log_alpha"] = torch.from_numpy(x["log_alpha"]).to(dev)
    e["beta"] = torch.from_numpy(x["beta"]).to(dev)
    od = torch.empty((wd.B, wd.H, 128), dtype=torch.float32, device=dev)
    for _ in range(args.warmup + args.steps):
        kda.decode_step(e["q"], e["k"], e["v"], e["log_alpha"], e["beta"], S, o=od)
    torch.cuda.synchronize()
    print(f"decode only: {args.warmup + args.steps} launches", flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 "
                                   "(every (sequence, head) chain is independent, so more GPUs "
                                   "would shard heads with no communication; that path is not "
                                   "implemented)"}))
        sys.exit(2)

    import torch
    import gated_delta_rule_amd as kda
    from gated_delta_rule_amd import workloads as W
    from gated_delta_rule_amd.traffic import measured as measured_traffic, measured_mfma, measured_phases

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = W.workload(1)
    if args.only == "decode":
        run_decode_only(args, torch, kda, W, dev)
        return
    stream = torch.cuda.current_stream(dev)

    # The headline prefill's inputs, generated on the host before any timing
    # and kept resident, so that no host-side work separates the timed runs
    # below from the GPU work before them.
    a = W.prefill_inputs(w)
    B, T, H = w.B, w.T, w.H
    shp = (B, T, H, 128)
    d = {n: torch.from_numpy(a[n]).to(dev, torch.bfloat16).view(shp) for n in ("q", "k", "v")}
    d["log_alpha"] = torch.from_numpy(a["log_alpha"]).to(dev).view(shp)
    d["beta"] = torch.from_numpy(a["beta"]).to(dev).view(B, T, H)
    del a
    o = torch.empty(shp, dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, 128, 128), dtype=torch.float32, device=dev)

    def prefill():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, None, o=o, S_T=S_T)

    def launch_times(n):
        ev = []
        for _ in range(n):
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e_a.record(stream)
            prefill()
            e_b.record(stream)
            ev.append((e_a, e_b))
        torch.cuda.synchronize()
        return [x.elapsed_time(y) for x, y in ev]

    # The first launches of the process, on a GPU that has been idle (for
    # information: its clocks are still low).
    cold_ms = launch_times(args.warmup + args.steps)

    if args.only is None:   # the decode step's state and per-step inputs, likewise
        wd = W.workload(4)
        Bd, Hd = wd.B, wd.H
        S = torch.from_numpy(W.decode_state(wd)).to(dev)
        steps_d = max(1, args.decode_steps)
        ins = []
        for s_ in range(steps_d):
            x = W.decode_inputs(wd, s_)
            e = {n: torch.from_numpy(x[n]).to(dev, torch.bfloat16) for n in ("q", "k", "v")}
            e["log_alpha"] = torch.from_numpy(x["log_alpha"]).to(dev)
            e["beta"] = torch.from_numpy(x["beta"]).to(dev)
            ins.append(e)
        od = torch.empty((Bd, Hd, 128), dtype=torch.float32, device=dev)

    # -------------------------------------- informational paths (run first,
    # so the headline prefill below is timed on a GPU at its working clocks)
    long_ctx = multi_tok = layer = bwd = varlen = None
    if not args.no_long and args.only is None:
        long_ctx = long_context(torch, kda, W, dev)
        varlen = varlen_prefill(torch, kda, W, dev)
        multi_tok = multi_token_decode(torch, kda, W, dev)
        layer = layer_steps(torch, kda, W, dev)
        bwd = backward_step(torch, kda, W, dev)

    # ------------------------------------------------------------- decode
    dec = None
    if args.only is None:

        def dstep(e):
            kda.decode_step(e["q"], e["k"], e["v"], e["log_alpha"], e["beta"], S, o=od)

        for i in range(min(args.warmup, steps_d)):
            dstep(ins[i])
        torch.cuda.synchronize()
        per_d = []
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for e in ins:
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e_a.record(stream)
            dstep(e)
            e_b.record(stream)
            per_d.append((e_a, e_b))
        ev1.record(stream)
        torch.cuda.synchronize()
        dec_total_ms = ev0.elapsed_time(ev1)
        dec_launch = [x.elapsed_time(y) for x, y in per_d]
        dec_kernel_ms = float(np.mean(dec_launch))
        n_states = Bd * Hd
        state_gbps = 2 * n_states * STATE_BYTES / (dec_kernel_ms * 1e-3) / 1e9
        dec_bytes = n_states * (2 * STATE_BYTES + DECODE_INPUT_BYTES_PER_STATE)
        dec_gbps_all = dec_bytes / (dec_kernel_ms * 1e-3) / 1e9
        dec = {
            "metric": "decode-step state GB/s", "value": state_gbps, "unit": "GB/s",
            "ms_per_step": dec_total_ms / steps_d, "steps": steps_d,
            "kernel_ms_median": float(np.median(dec_launch)),
            "kernel_ms_min": float(np.min(dec_launch)),
            "config": {"workload": "KDA decode B=256 H=96 d=128, bf16 q/k/v, fp32 gates, "
                                   "fp32 state [256,96,128,128] ~N(0,0.02^2), chained steps"},
            "roofline": {"bound": "hbm", "achieved": dec_gbps_all, "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": dec_gbps_all / PEAK_HBM_GBPS,
                         "traffic": measured_traffic("decode"), "kernel": "recurrent_kernel",
                         "kernel_ms": dec_kernel_ms, "algorithmic_bytes": dec_bytes,
                         "algorithmic_flops": n_states * DECODE_FLOPS_PER_STATE},
        }
        del S, ins
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ prefill
    # Clock settle: the GPU raises its clocks only after tens of milliseconds
    # of sustained load, so the headline kernel runs untimed for
    # --settle-seconds first; then the W warm-up launches and the K timed ones.
    n_settle, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(10):
            prefill()
        torch.cuda.synchronize()
        n_settle += 10
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record(stream)
        prefill()
        e_b.record(stream)
        per.append((e_a, e_b))
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = ev0.elapsed_time(ev1)
    launch_ms = [x.elapsed_time(y) for x, y in per]
    pf_ms = total_ms / args.steps
    pf_kernel_ms = float(np.mean(launch_ms))
    tokens_per_s = B * T / (pf_ms * 1e-3)
    pf_bytes = B * T * H * PREFILL_BYTES_PER_TOKEN_HEAD + B * H * STATE_BYTES
    pf_flops = B * T * H * PREFILL_FLOPS_PER_TOKEN_HEAD
    pf_gbps = pf_bytes / (pf_kernel_ms * 1e-3) / 1e9
    pf_tflops = pf_flops / (pf_kernel_ms * 1e-3) / 1e12
    traffic = measured_traffic("prefill")
    mfma = measured_mfma()
    mfma_counters = None
    if mfma is not None:
        # matrix-core flops the counters saw per launch (MOPS x 512), over the
        # live launch time; busy = MFMA busy cycles summed over the SIMDs over
        # (GPU active cycles of one XCD x 1024 SIMDs)
        hw = sum(mfma["hw_flops_per_launch_from_counters"].values())
        c = mfma["counters"]
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"]["per_dispatch"] / (
            c["GRBM_GUI_ACTIVE"]["per_dispatch"] / N_XCD * N_SIMD)
        mfma_counters = {"hw_flops_per_launch": hw,
                         "hw_tflops": hw / (pf_kernel_ms * 1e-3) / 1e12,
                         "hw_frac_of_bf16_peak": hw / (pf_kernel_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "mfma_busy_frac": busy,
                         "source": "profiles/chunk_fwd_workload1_mfma.json"}
    # the contraction phases alone (the phase probe's rocprof record)
    ph = measured_phases()
    phases = None if ph is None else {
        name: {"frac_of_16bit_peak": m["frac_of_16bit_peak"], "mfma_busy_frac": m["mfma_busy_frac"],
               "lds_bank_conflict_frac": m.get("lds_bank_conflict_frac")}
        for name, m in ph["modes"].items()}
    if phases is not None:
        phases["source"] = "profiles/contraction_phases_probe.json"
    del d, o, S_T
    torch.cuda.empty_cache()
    if args.only == "prefill":
        print(f"prefill only: {pf_kernel_ms:.4f} ms per launch, {tokens_per_s:.4g} tokens/s", flush=True)
        return

    # ------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        threads = oracle.max_threads()
        # the whole workload's heads, repeated until --cpu-seconds of wall time
        a = W.prefill_inputs(w)
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 50:
            t0 = time.perf_counter()
            oracle.forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], None, a["cu_seqlens"])
            t_cpu += time.perf_counter() - t0
            reps += 1
        n_heads = H
        t_cpu /= reps
        cpu = {"value": T * (n_heads / H) / t_cpu, "unit": "tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"fp64 token-by-token recurrence (C, OpenMP over heads) on all {n_heads} "
                         f"heads x {T} tokens of the same workload, {reps} runs, {t_cpu:.2f} s wall each; "
                         f"tokens/s counts a token once across all {H} heads; "
                         f"{cores} cores in the affinity mask"}
        # the decode step on a sixteenth of the decode workload's states, for
        # the decode metric's unit (fp32-equivalent state bytes read + written)
        wdc = W.workload(4).shrink(B=16)
        xs = W.decode_inputs(wdc, 0)
        Sd = W.decode_state(wdc)
        oracle.decode_step(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["beta"], Sd)   # first touch
        dreps, t_dec = 0, 0.0
        while dreps < 5 and t_dec < 2.0:
            t0 = time.perf_counter()
            oracle.decode_step(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["beta"], Sd)
            t_dec += time.perf_counter() - t0
            dreps += 1
        t_dec /= dreps
        dbytes = 2 * Sd.size * 4
        cpu["decode"] = {"value": dbytes / t_dec / 1e9, "unit": "GB/s",
                         "sample": f"fp64 decode step (C, OpenMP over states) on {wdc.B} x {wdc.H} "
                                   f"states of the decode workload, {dreps} runs, {t_dec:.3f} s each "
                                   "(fp32-equivalent state bytes read + written)"}

    out = {
        "metric": "KDA prefill tokens/s (H=96,d=128,T=8K) + decode-step state GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "token_heads_per_s": tokens_per_s * H,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "log_alpha=-5*sigmoid(N(0,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "KDA prefill B=1 T=8192 H=96 d=128, bf16 q/k/v, fp32 gates, "
                               "S0=0, fp32 o and final state",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": 128},
        "roofline": {"bound": "hbm", "achieved": pf_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": pf_gbps / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": "chunk_fwd_pipe_kernel", "kernel_ms": pf_kernel_ms,
                     "kernel_ms_median": float(np.median(launch_ms)),
                     "kernel_ms_min": float(np.min(launch_ms)),
                     "kernel_ms_cold_median": float(np.median(cold_ms[args.warmup:] or cold_ms)),
                     "clock_settle": {"seconds": t_settle, "launches": n_settle,
                                      "note": "untimed launches of the same kernel before the W "
                                              "warm-up steps; kernel_ms_cold_median is the first "
                                              "launches of the process on an idle GPU"},
                     "algorithmic_bytes": pf_bytes, "algorithmic_flops": pf_flops,
                     "mfma_tflops_algorithmic": pf_tflops,
                     "mfma_frac_algorithmic": pf_tflops / PEAK_BF16_TFLOPS,
                     "mfma_counters": mfma_counters,
                     "contraction_phases": phases},
        "decode": dec,
        "cpu_baseline": cpu,
        "long_context_prefill": long_ctx,
        "varlen_prefill": varlen,
        "multi_token_decode": multi_tok,
        "layer_prologue_epilogue": layer,
        "backward": bwd,
        "wall_s_timed_prefill": t_wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
