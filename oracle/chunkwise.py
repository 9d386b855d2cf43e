"""CPU chunkwise form of KDA, fp64, written from the pages' derivation.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  It reaches the same
result as the token-by-token recurrence by a different route, so the tests
compare the two (it pins the oracle and checks the algebra the GPU path is
built on).  One (sequence, head) at a time; q, k, log_alpha [T, dk],
v [T, dv], beta [T], S0 [dk, dv].

The steps follow "尝试对Kimi KDA的数学推导&算子实现分析" (hjcheng0602.cn),
in its row-vector notation (o_t = q_t s_t):

  * per chunk, g_t = sum_{r<=t} log alpha_r restarted at the chunk start,
    P_t = Diag(e^{g_t}), P_0 = I                              eqs. (8)-(10)
  * k+ = k e^{g}, k- = k e^{-g}, q+ = q e^{g}           eqs. (15), (16), (54)
  * L = StrictTril(B_beta K+ (K-)^T)                          eqs. (51), (56)
  * U = (I + L)^{-1} B_beta (V - K+ S)                        eqs. (52), (60)
    (solved by forward substitution; the page's identity (26) is not used)
  * O = Q+ S + Tril(Q+ (K-)^T) U                         eqs. (36), (57), (63)
  * S_next = P_C S + (K_end)^T U, k_end_j = k_j e^{g_C - g_j}  eqs. (64)-(66)

`sub_tile`, when given, evaluates every e^{g_t - g_j} product with the
references restarted every `sub_tile` tokens (k e^{g - r} and k e^{r - g}
with r the cumulative decay at the start / end of a sub-tile) instead of
e^{+-g} from the chunk start; the lower-bounded decay (log alpha >= -5,
"Kimi K3 技术报告解读" section 3.5) keeps every factor of a 16-token
sub-tile within e^{+-80}.  Both evaluations are the same numbers in exact
arithmetic.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _pair_decay_products(X, K, G, sub_tile):
    """Return P[t, j] = sum_i X[t,i] K[j,i] e^{G[t,i] - G[j,i]} for j <= t
    (entries with j > t are left at 0)."""
    C = X.shape[0]
    P = np.zeros((C, C))
    if sub_tile is None:
        P = (X * np.exp(G)) @ (K * np.exp(-G)).T
        return np.tril(P)
    for b0 in range(0, C, sub_tile):                 # row sub-tile (t)
        b1 = min(b0 + sub_tile, C)
        for a0 in range(0, b1, sub_tile):            # column sub-tile (j), a <= b
            a1 = min(a0 + sub_tile, C)
            r = G[a1 - 1]                            # decay at the end of sub-tile a
            left = X[b0:b1] * np.exp(G[b0:b1] - r)   # <= e^80 on the diagonal tile
            right = K[a0:a1] * np.exp(r - G[a0:a1])  # <= 1
            P[b0:b1, a0:a1] = left @ right.T
    return np.tril(P)


def chunkwise(q, k, v, log_alpha, beta, S0=None, chunk=64, sub_tile=None):
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64)
                         for a in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        Q, K, V, b = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        G = np.cumsum(la[c0:c1], axis=0)             # g_t within the chunk
        Kp = K * np.exp(G)                           # k+
        Qp = Q * np.exp(G)                           # q+
        KK = _pair_decay_products(K, K, G, sub_tile)  # k+_t . k-_j, j <= t
        QK = _pair_decay_products(Q, K, G, sub_tile)  # q+_t . k-_j, j <= t
        L = np.tril(b[:, None] * KK, k=-1)           # StrictTril(B_beta K+ K-^T)
        rhs = b[:, None] * (V - Kp @ S)              # B_beta (V - K+ S)
        U = solve_triangular(np.eye(c1 - c0) + L, rhs, lower=True, unit_diagonal=True)
        o[c0:c1] = Qp @ S + QK @ U                   # QK is already Tril(...)
        Kend = K * np.exp(G[-1] - G)                 # k_end = k e^{g_C - g_j}
        S = np.exp(G[-1])[:, None] * S + Kend.T @ U
    return o, S
