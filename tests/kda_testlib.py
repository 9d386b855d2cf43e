"""Helpers shared by the GPU parity tests (not collected by pytest).

Inputs come from gated_delta_rule_amd.workloads (seeded, per head); expected
values come only from the fp64 oracle.  The error measure is the one the
operator's target is stated in: max |x - y| / max |y| over the compared
elements, per output tensor, in fp64.
"""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from gated_delta_rule_amd import workloads as W

TOL_BF16 = 2e-3   # bf16 inputs, fp32 accumulation
TOL_F32 = 1e-5    # fp32 inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def torch_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_dev(arrs: dict, w, device="cuda"):
    """numpy inputs (float32 holding exact input-dtype values) -> device tensors."""
    import torch
    dt = torch_dtype(w)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.from_numpy(np.ascontiguousarray(arrs[name])).to(device=device, dtype=dt)
    for name in ("log_alpha", "beta"):
        out[name] = torch.from_numpy(np.ascontiguousarray(arrs[name])).to(device)
    if arrs.get("S0") is not None:
        out["S0"] = torch.from_numpy(np.ascontiguousarray(arrs["S0"])).to(device)
    else:
        out["S0"] = None
    if "cu_seqlens" in arrs and arrs["cu_seqlens"] is not None:
        out["cu_seqlens"] = torch.from_numpy(arrs["cu_seqlens"].astype(np.int32)).to(device)
    return out


def device_prefill_inputs(w, device="cuda", threads=None):
    """Allocate the whole prefill input on the device, generating it on the host
    one head at a time (bounded host memory).  Returns a dict of tensors laid
    out [T_total, H, d] plus cu_seqlens (int32, device) and S0 or None."""
    import torch
    cu = W.cu_seqlens(w)
    T = int(cu[-1])
    N = len(cu) - 1
    if threads is None:   # about 6 fp64 temporaries of [T, 128] per head in flight
        threads = int(max(1, min(16, 40e9 // max(1, T * 128 * 8 * 6))))
    dt = torch_dtype(w)
    dev = {n: torch.empty((T, w.H, w.dk), dtype=dt, device=device) for n in ("q", "k")}
    dev["v"] = torch.empty((T, w.H, w.dv), dtype=dt, device=device)
    dev["log_alpha"] = torch.empty((T, w.H, w.dk), dtype=torch.float32, device=device)
    dev["beta"] = torch.empty((T, w.H), dtype=torch.float32, device=device)
    dev["S0"] = (torch.empty((N, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
                 if w.s0_std else None)

    def gen(h):
        s = W.head_stream(w, h, T)
        s0 = W.initial_state_head(w, h, N)
        return h, s, s0

    with ThreadPoolExecutor(threads) as ex:
        for h, s, s0 in ex.map(gen, range(w.H)):
            for name in ("q", "k", "v"):
                dev[name][:, h, :] = torch.from_numpy(s[name]).to(device=device, dtype=dt)
            dev["log_alpha"][:, h, :] = torch.from_numpy(s["log_alpha"]).to(device)
            dev["beta"][:, h] = torch.from_numpy(s["beta"]).to(device)
            if s0 is not None:
                dev["S0"][:, h] = torch.from_numpy(s0).to(device)
    dev["cu_seqlens"] = torch.from_numpy(cu.astype(np.int32)).to(device)
    return dev, cu


def oracle_head(w, h, cu, *, cols=None, seqs=None):
    """fp64 oracle for one head (all sequences, or the listed ones), inputs
    regenerated from the seeds.  Returns (o [T, dv] fp64, S_T [N, dk, dv])."""
    import oracle
    T = int(cu[-1])
    s = W.head_stream(w, h, T)
    s0 = W.initial_state_head(w, h, len(cu) - 1)
    N = len(cu) - 1
    units = None if seqs is None else [(n, 0) for n in seqs]
    o, st = oracle.forward(s["q"][:, None], s["k"][:, None], s["v"][:, None],
                           s["log_alpha"][:, None], s["beta"][:, None],
                           None if s0 is None else s0[:, None], cu, cols=cols, units=units)
    return o[:, 0], st[:, 0]
