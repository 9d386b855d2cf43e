"""Pins of the oracle's backward pass (oracle.backward, the reverse-mode
derivative of the fp64 token loop) to facts other than its own formulas:
central finite differences of the forward oracle, automatic differentiation
of the explicit d_k x d_k transition product, exact identities of the
recurrence (linearity in (v, S0), linearity of o_t in q_t, the invariance of
every state under (k, beta, v) -> (s k, beta / s^2, s v)), the closed form
without writes (beta = 0), and continuation across a split (CPU only)."""
import numpy as np
import pytest

import oracle


def _inputs(lens, H, dk, dv, seed, s0=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk)) * 0.5
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = len(lens)
    S0 = 0.3 * rng.standard_normal((N, H, dk, dv)) if s0 else None
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    return dict(q=q, k=k, v=v, la=la, beta=beta, cu=cu, S0=S0, dO=dO, dST=dST)


def _loss(x, **over):
    a = dict(x, **over)
    o, st = oracle.forward(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S0"], a["cu"])
    return float(np.sum(a["dO"] * o) + np.sum(a["dST"] * st))


def _grads(x):
    return oracle.backward(x["q"], x["k"], x["v"], x["la"], x["beta"], x["S0"], x["dO"],
                           x["dST"], x["cu"])


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_finite_differences_every_input():
    """Every element of every gradient against a central difference of the
    forward oracle's loss (step 1e-6: truncation ~1e-12, rounding ~1e-10)."""
    x = _inputs([5, 3, 1], H=2, dk=4, dv=3, seed=0)
    dq, dk, dv, dla, db, dS0 = _grads(x)
    names = [("q", dq), ("k", dk), ("v", dv), ("la", dla), ("beta", db), ("S0", dS0)]
    for name, g in names:
        base = x[name]
        fd = np.zeros_like(base)
        h = 1e-6
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += h
            m[idx] -= h
            fd[idx] = (_loss(x, **{name: p}) - _loss(x, **{name: m})) / (2 * h)
        assert _rel(g, fd) < 1e-7, (name, _rel(g, fd))


def _dplr_loss_torch(x):
    """The same loss through the explicit transition (I - beta k k^T) Diag(alpha)
    applied as a d_k x d_k matrix, differentiated by torch autograd (fp64)."""
    torch = pytest.importorskip("torch")
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True)
         for n in ("q", "k", "v", "la", "beta", "S0")}
    dO = torch.tensor(x["dO"])
    dST = torch.tensor(x["dST"])
    cu = x["cu"]
    H, dk = x["q"].shape[1], x["q"].shape[2]
    eye = torch.eye(dk, dtype=torch.float64)
    L = torch.zeros((), dtype=torch.float64)
    for n in range(len(cu) - 1):
        for h in range(H):
            S = t["S0"][n, h]
            for i in range(cu[n], cu[n + 1]):
                kk, b = t["k"][i, h], t["beta"][i, h]
                trans = (eye - b * torch.outer(kk, kk)) @ torch.diag(torch.exp(t["la"][i, h]))
                S = trans @ S + b * torch.outer(kk, t["v"][i, h])
                L = L + dO[i, h] @ (S.T @ t["q"][i, h])
            L = L + torch.sum(dST[n, h] * S)
    L.backward()
    return {n: t[n].grad.numpy() for n in t}


def test_autograd_of_explicit_transition_product():
    x = _inputs([6, 4], H=2, dk=5, dv=3, seed=1)
    ref = _dplr_loss_torch(x)
    dq, dk, dv, dla, db, dS0 = _grads(x)
    for name, g in (("q", dq), ("k", dk), ("v", dv), ("la", dla), ("beta", db), ("S0", dS0)):
        assert _rel(g, ref[name]) < 1e-12, (name, _rel(g, ref[name]))


def test_adjoint_identity_in_v_and_S0():
    """(v, S0) -> (o, S_T) is linear for fixed q, k, alpha, beta, so
    <dO, o> + <dS_T, S_T> = <dv, v> + <dS0, S0> exactly."""
    x = _inputs([40, 70, 1], H=2, dk=128, dv=128, seed=2)
    L = _loss(x)
    _, _, dv, _, _, dS0 = _grads(x)
    rhs = float(np.sum(dv * x["v"]) + np.sum(dS0 * x["S0"]))
    assert abs(L - rhs) <= 1e-11 * max(abs(L), 1.0), (L, rhs)


def test_per_token_identities_q_and_scaling():
    """o_t is linear in q_t (and S_t does not depend on q_t):
    q_t . dq_t = dO_t . o_t for every token and head.  The map
    (k_t, beta_t, v_t) -> (s k_t, beta_t / s^2, s v_t) leaves every state
    unchanged, so k_t . dk_t - 2 beta_t dbeta_t + v_t . dv_t = 0."""
    x = _inputs([33, 20], H=3, dk=128, dv=128, seed=3)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["la"], x["beta"], x["S0"], x["cu"])
    dq, dk, dv, dla, db, dS0 = _grads(x)
    lhs = np.sum(x["q"] * dq, axis=-1)
    rhs = np.sum(x["dO"] * o, axis=-1)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    inv = np.sum(x["k"] * dk, -1) - 2 * x["beta"] * db + np.sum(x["v"] * dv, -1)
    scale = np.max(np.abs(np.sum(x["v"] * dv, -1)))
    assert np.max(np.abs(inv)) <= 1e-12 * scale


def test_no_writes_closed_form():
    """beta = 0: S_t = Diag(e^{g_t}) S0 with g_t the running sum of
    log_alpha, o_t = S0^T (e^{g_t} * q_t).  Then dq_t = e^{g_t} * (S0 dO_t),
    dk = dv = 0, dS0 = sum_t (e^{g_t} * q_t) dO_t^T + Diag(e^{g_T}) dS_T,
    dlog_alpha_r = sum_{t>=r} e^{g_t} q_t (S0 dO_t) + e^{g_T} rowsum(dS_T S0),
    dbeta_t = k_t^T G_t (v_t - S'_t^T k_t) with G_t the state gradient."""
    x = _inputs([9], H=1, dk=6, dv=4, seed=4)
    x["beta"] = np.zeros_like(x["beta"])
    dq, dk, dv, dla, db, dS0 = _grads(x)
    q, k, v, la = x["q"][:, 0], x["k"][:, 0], x["v"][:, 0], x["la"][:, 0]
    S0, dO, dST = x["S0"][0, 0], x["dO"][:, 0], x["dST"][0, 0]
    T = q.shape[0]
    e = np.exp(np.cumsum(la, axis=0))                      # e^{g_t}
    assert np.allclose(dq[:, 0], e * (dO @ S0.T), atol=1e-14)
    assert np.all(dk == 0) and np.all(dv == 0)
    ref_dS0 = (e * q).T @ dO + e[-1][:, None] * dST
    assert np.allclose(dS0[0, 0], ref_dS0, atol=1e-13)
    per_t = e * q * (dO @ S0.T)                            # [T, dk]
    ref_dla = np.cumsum(per_t[::-1], axis=0)[::-1] + e[-1] * np.sum(dST * S0, axis=1)
    assert np.allclose(dla[:, 0], ref_dla, atol=1e-13)
    for t in range(T):
        G = (e[-1] / e[t])[:, None] * dST
        for s in range(t, T):
            G = G + (e[s] / e[t])[:, None] * np.outer(q[s], dO[s])
        Sd = e[t][:, None] * S0
        assert np.isclose(db[t, 0], k[t] @ G @ (v[t] - Sd.T @ k[t]), atol=1e-13)


def test_continuation_across_a_split():
    """Backward over [0, T1) with dS_T = the dS0 of the backward over
    [T1, T) started from S_{T1} gives the gradients of the whole run."""
    x = _inputs([50], H=2, dk=16, dv=8, seed=5)
    T1 = 21
    full = _grads(x)
    _, s1 = oracle.forward(x["q"][:T1], x["k"][:T1], x["v"][:T1], x["la"][:T1],
                           x["beta"][:T1], x["S0"])
    second = oracle.backward(x["q"][T1:], x["k"][T1:], x["v"][T1:], x["la"][T1:],
                             x["beta"][T1:], s1, x["dO"][T1:], x["dST"])
    first = oracle.backward(x["q"][:T1], x["k"][:T1], x["v"][:T1], x["la"][:T1],
                            x["beta"][:T1], x["S0"], x["dO"][:T1], second[5])
    for i in range(5):
        assert _rel(np.concatenate([first[i], second[i]]), full[i]) < 1e-12
    assert _rel(first[5], full[5]) < 1e-12


def test_units_subset_and_empty_sequence():
    x = _inputs([7, 0, 5], H=3, dk=8, dv=8, seed=6)
    full = _grads(x)
    part = oracle.backward(x["q"], x["k"], x["v"], x["la"], x["beta"], x["S0"], x["dO"],
                           x["dST"], x["cu"], units=[(2, 1), (1, 0)])
    rows = slice(7, 12)
    assert np.array_equal(part[0][rows, 1], full[0][rows, 1])
    assert np.all(part[0][rows, 0] == 0)
    # an empty sequence passes its state gradient straight through
    assert np.array_equal(full[5][1], x["dST"][1])
    assert np.array_equal(part[5][1, 0], x["dST"][1, 0])
