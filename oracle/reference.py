"""Special cases and alternative forms of the KDA recurrence, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  These are the textbook
forms the pages place KDA among; the tests use them to pin the C oracle to
facts other than its own formula.  All arrays are for ONE (sequence, head):
q, k, log_alpha [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv].

Sources (page title, section / equation):
  * linear attention S_t = S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, and its
    attention form o_t = sum_{j<=t} (q_t . k_j) v_j: "把注意力换成一块「会遗忘的
    内存」" (jokeuncle.github.io), section "第一步"; "Kimi K3 技术报告解读"
    (marsggbo.github.io), section 3.1.
  * DeltaNet S_t = (I - beta k k^T) S_{t-1} + beta k v^T: jokeuncle page,
    section "第二步"; "Kimi K3 核心算子拆解" (devpress.csdn.net), section 2.1.
  * Gated DeltaNet S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T with a
    scalar alpha_t: jokeuncle page, section "第三步".
  * naive DPLR product: form the d_k x d_k transition (I - beta k k^T)
    Diag(alpha) and multiply, "Kimi K3 核心算子拆解" section 2.3 (cost table)
    and eq. (3) of "尝试对Kimi KDA的数学推导&算子实现分析" (hjcheng0602.cn).
  * unrolled product s_t = (D_t..D_1) s_0 + sum_j (D_t..D_{j+1}) C_j with
    D_t = (I - beta_t k_t k_t^T) Diag(alpha_t), C_t = beta_t k_t v_t^T:
    hjcheng0602.cn page, eqs. (4)-(6).
"""
from __future__ import annotations

import numpy as np


def linear_attention_parallel(q, k, v):
    """Un-normalised causal linear attention in its attention (non-recurrent)
    form: o_t = sum_{j<=t} (q_t . k_j) v_j."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    scores = np.tril(q @ k.T)          # [T, T], entry (t, j) = q_t . k_j, j <= t
    return scores @ v


def deltanet(q, k, v, beta, S0=None):
    """DeltaNet: S <- (I - beta k k^T) S + beta k v^T, o = S^T q."""
    q, k, v, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        S = (eye - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def gated_deltanet(q, k, v, alpha, beta, S0=None):
    """Gated DeltaNet with a scalar gate alpha_t per token:
    S <- alpha_t (I - beta k k^T) S + beta k v^T, o = S^T q."""
    q, k, v, alpha, beta = (np.asarray(a, dtype=np.float64)
                            for a in (q, k, v, alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        S = alpha[t] * ((eye - beta[t] * np.outer(k[t], k[t])) @ S) \
            + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def transition(k_t, log_alpha_t, beta_t):
    """The explicit d_k x d_k KDA transition D_t = (I - beta k k^T) Diag(alpha)."""
    k_t = np.asarray(k_t, dtype=np.float64)
    dk = k_t.shape[0]
    return (np.eye(dk) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.exp(log_alpha_t))


def naive_dplr(q, k, v, log_alpha, beta, S0=None):
    """KDA by forming the full transition matrix each step (O(dk^2 dv))."""
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64)
                         for a in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = transition(k[t], la[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def unrolled_product(q, k, v, log_alpha, beta, S0=None):
    """Brute-force closed form s_t = (D_t..D_1) s_0 + sum_{j<=t} (D_t..D_{j+1}) C_j,
    evaluated from scratch for every t (cubic in T; tiny inputs only)."""
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64)
                         for a in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    s0 = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    D = [transition(k[t], la[t], beta[t]) for t in range(T)]
    C = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    o = np.zeros((T, dv))
    S = s0
    for t in range(T):
        prod = np.eye(dk)
        for r in range(t, -1, -1):          # D_t D_{t-1} ... D_0
            prod = prod @ D[r]
        S = prod @ s0
        for j in range(t + 1):
            pj = np.eye(dk)
            for r in range(t, j, -1):       # D_t ... D_{j+1}
                pj = pj @ D[r]
            S = S + pj @ C[j]
        o[t] = S.T @ q[t]
    return o, S


def decay_only(q, log_alpha, S0):
    """beta == 0: nothing is written or erased, so S_t = Diag(exp(sum_{r<=t}
    log_alpha_r)) S0 in closed form and o_t = S_t^T q_t."""
    q = np.asarray(q, dtype=np.float64)
    G = np.cumsum(np.asarray(log_alpha, dtype=np.float64), axis=0)   # [T, dk]
    S0 = np.asarray(S0, dtype=np.float64)
    o = np.einsum("tk,tk,kv->tv", q, np.exp(G), S0)
    S_T = np.exp(G[-1])[:, None] * S0
    return o, S_T
