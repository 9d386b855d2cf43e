"""Seeded synthetic inputs for the KDA operator (numpy only).

This module draws inputs; it holds none of the operator's arithmetic, and
both the HIP path's callers and the fp64 oracle's callers take their inputs
from here.  Every array is generated per head from
``numpy.random.SeedSequence([2026, workload_id, tensor_id, head, ...])`` with
PCG64, so any head (or any sequence of a packed batch) can be regenerated on
its own without materialising the rest.

Distributions (the operator's input contract on the pages: q, k L2-normalised
per token after the short convolution, "把注意力换成一块「会遗忘的内存」"
section "层的实现"; per-channel log-decay bounded in (-5, 0) by a scaled
sigmoid, "Kimi K3 技术报告解读" section 3.5; beta a sigmoid write strength):

  q, k       ~ N(0, 1) per element, then L2-normalised over d_k per (token, head)
  v          ~ N(0, 1)
  log_alpha  = -5 * sigmoid(N(0, 1)) per channel          (in (-5, 0))
  beta       = sigmoid(N(0, 1)) per (token, head)          (in (0, 1))
  S0 / state ~ N(0, 0.02^2)                                 (fp32)

Values are drawn in fp64 and rounded once to the workload's input dtype
(bf16 by round-to-nearest-even, or fp32).  Arrays are returned as float32
numpy arrays whose values are exactly representable in that dtype, laid out
token-major: [T, H, d] (prefill) or [B, H, d] (decode).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

SEED_ROOT = 2026
T_Q, T_K, T_V, T_LOGA, T_BETA, T_S0, T_LEN = range(7)
# layer prologue / epilogue inputs
T_RAW_Q, T_RAW_K, T_RAW_V, T_CONV_W, T_GATE_A, T_GATE_B, T_GATE_O, T_NORM_W, T_CACHE = range(7, 16)
LAYER_WID = 100
# upstream gradients for the backward pass
T_GRAD_O, T_GRAD_S = 16, 17


@dataclass(frozen=True)
class Workload:
    wid: int                 # seed namespace
    name: str
    kind: str                # "prefill" | "decode"
    H: int
    dk: int = 128
    dv: int = 128
    dtype: str = "bf16"      # q/k/v input dtype: "bf16" | "f32"
    B: int = 1               # equal-length sequences (prefill) / requests (decode)
    T: int = 0               # tokens per sequence (prefill, equal length)
    n_varlen: int = 0        # >0: packed varlen batch of this many sequences
    len_lo: int = 0
    len_hi: int = 0
    s0_std: float = 0.0      # 0 => S0 = zeros (prefill)
    steps: int = 1           # decode steps chained on the state
    chunk: int = 64          # chunk length quoted for the workload (internal)

    @property
    def varlen(self) -> bool:
        return self.n_varlen > 0

    def shrink(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads the operator is measured and checked on.
WORKLOADS = {
    0: Workload(0, "single head fp32 T=256", "prefill", H=1, dtype="f32", T=256),
    1: Workload(1, "prefill T=8192 H=96 bf16", "prefill", H=96, T=8192),
    2: Workload(2, "varlen prefill 32 seqs in [512,16384] H=96 bf16, S0~N(0,0.02)",
                "prefill", H=96, n_varlen=32, len_lo=512, len_hi=16384, s0_std=0.02),
    3: Workload(3, "long-context prefill T=1048576 H=16 bf16", "prefill", H=16, T=1048576),
    4: Workload(4, "decode B=256 H=96 bf16, state~N(0,0.02), 64 chained steps",
                "decode", H=96, B=256, s0_std=0.02, steps=64),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, *key])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _to_dtype(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x64.astype(np.float32))
    if dtype == "f32":
        return x64.astype(np.float32)
    raise ValueError(dtype)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def cu_seqlens(w: Workload) -> np.ndarray:
    """int64 [N+1] sequence offsets of the packed token axis."""
    if w.varlen:
        lens = _rng(w.wid, T_LEN).integers(w.len_lo, w.len_hi, size=w.n_varlen,
                                           endpoint=True)
    else:
        lens = np.full(w.B, w.T, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def n_sequences(w: Workload) -> int:
    return w.n_varlen if w.varlen else w.B


def total_tokens(w: Workload) -> int:
    return int(cu_seqlens(w)[-1])


def _unit_rows(g: np.random.Generator, n: int, d: int) -> np.ndarray:
    x = g.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def head_stream(w: Workload, head: int, n_tokens: int, step: int | None = None) -> dict:
    """All per-token inputs of one head over `n_tokens` tokens (the packed
    token axis of a prefill, or the B requests of decode step `step`).
    Returns float32 arrays q, k, log_alpha [n, dk]; v [n, dv]; beta [n]."""
    key = (head,) if step is None else (head, step)
    dt = w.dtype
    q = _to_dtype(_unit_rows(_rng(w.wid, T_Q, *key), n_tokens, w.dk), dt)
    k = _to_dtype(_unit_rows(_rng(w.wid, T_K, *key), n_tokens, w.dk), dt)
    v = _to_dtype(_rng(w.wid, T_V, *key).standard_normal((n_tokens, w.dv)), dt)
    la = (-5.0 * _sigmoid(_rng(w.wid, T_LOGA, *key).standard_normal((n_tokens, w.dk))))
    beta = _sigmoid(_rng(w.wid, T_BETA, *key).standard_normal(n_tokens))
    return dict(q=q, k=k, v=v, log_alpha=la.astype(np.float32),
                beta=beta.astype(np.float32))


def initial_state_head(w: Workload, head: int, n_seq: int) -> np.ndarray | None:
    """S0 for one head of all sequences / requests: float32 [n_seq, dk, dv]."""
    if w.s0_std == 0.0:
        return None
    g = _rng(w.wid, T_S0, head)
    return (w.s0_std * g.standard_normal((n_seq, w.dk, w.dv))).astype(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def prefill_inputs(w: Workload, heads=None) -> dict:
    """Full token-major arrays for a prefill workload (only for sizes that fit
    in host memory).  heads: optional subset of head indices; the returned
    arrays then have len(heads) heads, in that order."""
    assert w.kind == "prefill"
    heads = list(range(w.H)) if heads is None else list(heads)
    cu = cu_seqlens(w)
    T = int(cu[-1])
    N = len(cu) - 1
    Hs = len(heads)
    out = dict(q=np.empty((T, Hs, w.dk), np.float32), k=np.empty((T, Hs, w.dk), np.float32),
               v=np.empty((T, Hs, w.dv), np.float32),
               log_alpha=np.empty((T, Hs, w.dk), np.float32),
               beta=np.empty((T, Hs), np.float32))
    S0 = np.zeros((N, Hs, w.dk, w.dv), np.float32) if w.s0_std else None

    def fill(i_h):
        i, h = i_h
        s = head_stream(w, h, T)
        for name in ("q", "k", "v", "log_alpha"):
            out[name][:, i, :] = s[name]
        out["beta"][:, i] = s["beta"]
        if S0 is not None:
            S0[:, i] = initial_state_head(w, h, N)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, enumerate(heads)))
    out["S0"] = S0
    out["cu_seqlens"] = cu
    return out


def decode_inputs(w: Workload, step: int, heads=None) -> dict:
    """Inputs of decode step `step`: q, k, log_alpha [B, H, dk]; v [B, H, dv];
    beta [B, H] (float32 arrays)."""
    assert w.kind == "decode"
    heads = list(range(w.H)) if heads is None else list(heads)
    B, Hs = w.B, len(heads)
    out = dict(q=np.empty((B, Hs, w.dk), np.float32), k=np.empty((B, Hs, w.dk), np.float32),
               v=np.empty((B, Hs, w.dv), np.float32),
               log_alpha=np.empty((B, Hs, w.dk), np.float32),
               beta=np.empty((B, Hs), np.float32))
    for i, h in enumerate(heads):
        s = head_stream(w, h, B, step=step)
        for name in ("q", "k", "v", "log_alpha"):
            out[name][:, i, :] = s[name]
        out["beta"][:, i] = s["beta"]
    return out


def decode_state(w: Workload, heads=None) -> np.ndarray:
    """Initial decode state float32 [B, H, dk, dv]."""
    assert w.kind == "decode"
    heads = list(range(w.H)) if heads is None else list(heads)
    S = np.empty((w.B, len(heads), w.dk, w.dv), np.float32)

    def fill(i_h):
        i, h = i_h
        S[:, i] = initial_state_head(w, h, w.B)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, enumerate(heads)))
    return S


def layer_inputs(lens, H: int, dtype: str = "bf16", seed: int = 0, with_cache: bool = True,
                 d: int = 128) -> dict:
    """Inputs of the layer prologue / epilogue for packed sequences of the
    given lengths (synthetic weights; the pages give no trained values):
      q_raw, k_raw, v_raw ~ N(0, 1)  [T, H, d]   (pre-convolution projections)
      conv_w ~ N(0, 0.5^2)           [3, H, d, 4] (q, k, v; tap 0 on t-3)
      a ~ N(0, 1) [T, H, d], b ~ N(0, 1) [T, H]   (decay / write pre-activations)
      g ~ N(0, 1) [T, H, d], w_norm = 1 + 0.1 N(0, 1) [d]   (output gate, norm weight)
      cache ~ N(0, 1) [N, 3, 3, H, d] or None     (previous raw inputs)
    Raw inputs and cache are rounded to `dtype`; everything else is float32."""
    lens = np.asarray(lens, np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N = int(cu[-1]), len(lens)
    key = (LAYER_WID + seed,)
    raw = {n: _to_dtype(_rng(*key, t).standard_normal((T, H, d)), dtype)
           for n, t in (("q_raw", T_RAW_Q), ("k_raw", T_RAW_K), ("v_raw", T_RAW_V))}
    out = dict(raw)
    out["conv_w"] = (0.5 * _rng(*key, T_CONV_W).standard_normal((3, H, d, 4))).astype(np.float32)
    out["a"] = _rng(*key, T_GATE_A).standard_normal((T, H, d)).astype(np.float32)
    out["b"] = _rng(*key, T_GATE_B).standard_normal((T, H)).astype(np.float32)
    out["g"] = _rng(*key, T_GATE_O).standard_normal((T, H, d)).astype(np.float32)
    out["w_norm"] = (1.0 + 0.1 * _rng(*key, T_NORM_W).standard_normal(d)).astype(np.float32)
    out["cache"] = (_to_dtype(_rng(*key, T_CACHE).standard_normal((N, 3, 3, H, d)), dtype)
                    if with_cache else None)
    out["cu_seqlens"] = cu
    return out


def grad_head(w: Workload, head: int, n_tokens: int, n_seq: int, s_std: float = 1.0):
    """Upstream gradients for one head: dO ~ N(0, 1) float32 [n_tokens, dv]
    (the loss gradient at every output) and dS_T ~ N(0, s_std^2) float32
    [n_seq, dk, dv] (at every final state), or None when s_std is 0."""
    dO = _rng(w.wid, T_GRAD_O, head).standard_normal((n_tokens, w.dv)).astype(np.float32)
    dS = (None if s_std == 0.0 else
          (s_std * _rng(w.wid, T_GRAD_S, head).standard_normal((n_seq, w.dk, w.dv)))
          .astype(np.float32))
    return dO, dS


def grad_inputs(w: Workload, T: int, N: int, s_std: float = 1.0, heads=None):
    """dO [T, H, dv] and dS_T [N, H, dk, dv] (or None) for all (or the listed)
    heads, from grad_head."""
    heads = list(range(w.H)) if heads is None else list(heads)
    dO = np.empty((T, len(heads), w.dv), np.float32)
    dS = None if s_std == 0.0 else np.empty((N, len(heads), w.dk, w.dv), np.float32)
    for i, h in enumerate(heads):
        a, b = grad_head(w, h, T, N, s_std)
        dO[:, i] = a
        if dS is not None:
            dS[:, i] = b
    return dO, dS
