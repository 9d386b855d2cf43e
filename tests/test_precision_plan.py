"""CPU model of the bf16 prefill's rounding plan, checked against the oracle.

The HIP prefill evaluates each 32-token chunk as
    X = k e^{g-E0}, QX = q e^{g-E0}, Y = k e^{E0-g}        (E0: decay after 16 tokens)
    L = StrictTril(B_beta X Y^T),  M = Tril(QX Y^T),  T = (I + L)^{-1}
    R = V - X (e^{E0} S),  U = T B_beta R,  O = QX (e^{E0} S) + M U
    S <- e^{E1-E0} (e^{E0} S + Y^T U)
with matrix products on bf16 matrix cores.  This test re-evaluates the same
algebra in fp64 numpy, rounding to bf16 exactly the operands the kernel
rounds ("plain": once; "split": hi + lo pair), and checks that
  * the kernel's plan stays well inside the 2e-3 max-norm budget, and
  * rounding every operand once would not (so the splits are needed).
It models the kernel; it does not run it, and shares no code with it.

The pipelined bf16 kernel rounds differently where the state meets a chunk's
operands: K+ S = X (e^{E0} S) with the state's bf16 hi part only, and
Q+ S = (q e^{g}) S with both operands rounded once to fp16 (`model_pipe`).
"""
import numpy as np
import pytest

import oracle
from gated_delta_rule_amd import workloads as W


def bf(x):
    return W.round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def split(x):
    x = np.asarray(x, np.float64)
    hi = bf(x)
    return hi + bf(x - hi)


ROUND = {"plain": bf, "split": split}

KERNEL_PLAN = dict(X="plain", QX="split", Y="split", Xc="plain", QXc="plain", S="split",
                   T="plain", R="split", M="split", U="split", Yu="split", Uu="split")
ALL_PLAIN = {k: "plain" for k in KERNEL_PLAN}


def model(q, k, v, la, beta, S0, plan, C=32):
    f = lambda n: ROUND[plan[n]]
    T_, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T_, dv))
    for c0 in range(0, T_, C):
        n = min(C, T_ - c0)
        pad = lambda a, w: np.concatenate([a[c0:c0 + n], np.zeros((C - n,) + a.shape[1:])])
        Q, K, V, b, LA = pad(q, 0), pad(k, 0), pad(v, 0), pad(beta, 0), pad(la, 0)
        G = np.cumsum(LA, 0)
        E0, E1 = G[15], G[31]
        X, QX, Y = K * np.exp(G - E0), Q * np.exp(G - E0), K * np.exp(E0 - G)
        L = np.tril(b[:, None] * (f("X")(X) @ f("Y")(Y).T), -1)
        M = np.tril(f("QX")(QX) @ f("Y")(Y).T)
        Tm = np.linalg.inv(np.eye(C) + L)
        St = np.exp(E0)[:, None] * S
        R = V - f("Xc")(X) @ f("S")(St)
        U = f("T")(Tm) @ f("R")(b[:, None] * R)
        O = f("QXc")(QX) @ f("S")(St) + f("M")(M) @ f("U")(U)
        o[c0:c0 + n] = O[:n]
        S = np.exp(E1 - E0)[:, None] * (St + f("Yu")(Y).T @ f("Uu")(U))
    return o, S


def fp16(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def model_pipe(q, k, v, la, beta, S0, C=32):
    """The pipelined kernel's plan: L from X, Y rounded once; M from split QX,
    Y; the block substitution with T rounded once and its right-hand sides
    split; K+ S with the scaled state's hi part; Q+ S in fp16; the update
    Y^T U with both split."""
    T_, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T_, dv))
    for c0 in range(0, T_, C):
        n = min(C, T_ - c0)
        pad = lambda a: np.concatenate([a[c0:c0 + n], np.zeros((C - n,) + a.shape[1:])])
        Q, K, V, b, LA = pad(q), pad(k), pad(v), pad(beta), pad(la)
        G = np.cumsum(LA, 0)
        E0, E1 = G[15], G[31]
        X, QX, Y = K * np.exp(G - E0), Q * np.exp(G - E0), K * np.exp(E0 - G)
        L = np.tril(b[:, None] * (bf(X) @ bf(Y).T), -1)
        M = np.tril(split(QX) @ split(Y).T)
        IL = np.eye(C) + L
        T00, T11 = np.linalg.inv(IL[:16, :16]), np.linalg.inv(IL[16:, 16:])
        St = np.exp(E0)[:, None] * S
        Rp = b[:, None] * (V - bf(X) @ bf(St))
        U0 = bf(T00) @ split(Rp[:16])
        U1 = bf(T11) @ split(Rp[16:] - bf(L[16:, :16]) @ split(U0))
        U = np.concatenate([U0, U1])
        O = fp16(Q * np.exp(G)) @ fp16(S) + split(M) @ split(U)
        o[c0:c0 + n] = O[:n]
        S = np.exp(E1 - E0)[:, None] * (St + split(Y).T @ split(U))
    return o, S


def worst_pipe(T=256, heads=3, wid=1):
    w = W.workload(wid).shrink(T=T, H=heads, s0_std=0.02)
    a = W.prefill_inputs(w)
    ro, rs = oracle.forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["S0"],
                            a["cu_seqlens"])
    eo = es = 0.0
    for h in range(heads):
        o, s = model_pipe(*(a[x][:, h].astype(np.float64) for x in ("q", "k", "v", "log_alpha", "beta")),
                          a["S0"][0, h])
        eo = max(eo, np.abs(o - ro[:, h]).max() / np.abs(ro[:, h]).max())
        es = max(es, np.abs(s - rs[0, h]).max() / np.abs(rs[0, h]).max())
    return eo, es


def worst(plan, T=256, heads=3, wid=1):
    w = W.workload(wid).shrink(T=T, H=heads, s0_std=0.02)
    a = W.prefill_inputs(w)
    ro, rs = oracle.forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["S0"],
                            a["cu_seqlens"])
    eo = es = 0.0
    for h in range(heads):
        o, s = model(*(a[x][:, h].astype(np.float64) for x in ("q", "k", "v", "log_alpha", "beta")),
                     a["S0"][0, h], plan)
        eo = max(eo, np.abs(o - ro[:, h]).max() / np.abs(ro[:, h]).max())
        es = max(es, np.abs(s - rs[0, h]).max() / np.abs(rs[0, h]).max())
    return eo, es


def test_exact_model_equals_oracle():
    exact = {k: "split" for k in KERNEL_PLAN}
    ROUND_SAVE = dict(ROUND)
    try:
        ROUND["split"] = lambda x: np.asarray(x, np.float64)
        eo, es = worst(exact, T=100, heads=1)
    finally:
        ROUND.update(ROUND_SAVE)
    assert eo < 1e-12 and es < 1e-12


def test_kernel_plan_within_budget():
    eo, es = worst(KERNEL_PLAN)
    assert eo < 6e-4 and es < 2e-4, (eo, es)


def test_single_rounding_everywhere_exceeds_budget():
    eo, es = worst(ALL_PLAIN)
    assert max(eo, es) > 2e-3, (eo, es)


def test_pipelined_plan_within_budget():
    eo, es = worst_pipe()
    assert eo < 2e-4 and es < 2e-4, (eo, es)
    ek, _ = worst(KERNEL_PLAN)
    assert eo < ek, (eo, ek)   # fp16 Q+ S is the more accurate of the two
