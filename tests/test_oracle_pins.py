"""Pins of the fp64 oracle to facts other than its own formula (CPU only).

Each test names the fact it checks and where the pages state it.  A plausible
mistake in the oracle -- reading o before the update, applying the decay
after the correction, a transposed state, a wrong sign on the erase term, an
off-by-one in the gate -- fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref
from oracle.chunkwise import chunkwise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-300))


def run1(q, k, v, la, beta, S0=None):
    """Oracle on one (sequence, head): inputs [T, d] -> (o [T, dv], S_T [dk, dv])."""
    T, dk = q.shape
    dv = v.shape[1]
    o, st = oracle.forward(q[:, None], k[:, None], v[:, None], la[:, None],
                           beta[:, None], None if S0 is None else S0[None, None])
    return o[:, 0], st[0, 0]


def rand_inputs(rng, T, dk, dv, la_lo=-5.0, normalise=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if normalise:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = la_lo / (1.0 + np.exp(-rng.standard_normal((T, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    return q, k, v, la, beta


def test_golden_hand_example():
    """Two tokens worked by hand with the three-step method (fixture cites it)."""
    g = json.load(open(os.path.join(GOLDEN, "kda_hand_example.json")))
    q, k, v = (np.array(g[n]) for n in ("q", "k", "v"))
    la = np.log(np.array(g["alpha"]))
    beta = np.array(g["beta"])
    o, st = run1(q, k, v, la, beta)
    np.testing.assert_allclose(o, np.array(g["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st, np.array(g["S_T"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("dk,dv,T", [(8, 8, 20), (16, 4, 9), (128, 128, 12)])
def test_p1_three_step_equals_naive_dplr(dk, dv, T):
    """The O(dk dv) three-step update equals the explicit (I - b k k^T) Diag(a)
    product (devpress page section 2.3 table; hjcheng0602.cn eq. (3))."""
    rng = np.random.default_rng(1)
    q, k, v, la, beta = rand_inputs(rng, T, dk, dv)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    o, st = run1(q, k, v, la, beta, S0)
    o2, st2 = ref.naive_dplr(q, k, v, la, beta, S0)
    assert rel(o, o2) < 1e-12 and rel(st, st2) < 1e-12


def test_p2_alpha_one_is_deltanet():
    """log alpha == 0 reduces KDA to DeltaNet (jokeuncle page, '第二步')."""
    rng = np.random.default_rng(2)
    q, k, v, _, beta = rand_inputs(rng, 40, 32, 24)
    S0 = 0.1 * rng.standard_normal((32, 24))
    o, st = run1(q, k, v, np.zeros((40, 32)), beta, S0)
    o2, st2 = ref.deltanet(q, k, v, beta, S0)
    assert rel(o, o2) < 1e-12 and rel(st, st2) < 1e-12


def test_p3_scalar_gate_is_gated_deltanet():
    """A gate equal on all channels reduces KDA to Gated DeltaNet, since a
    scalar Diag commutes with (I - b k k^T) (jokeuncle page, '第三步')."""
    rng = np.random.default_rng(3)
    q, k, v, _, beta = rand_inputs(rng, 40, 32, 24)
    a = -5.0 / (1.0 + np.exp(-rng.standard_normal(40)))
    la = np.repeat(a[:, None], 32, axis=1)
    S0 = 0.1 * rng.standard_normal((32, 24))
    o, st = run1(q, k, v, la, beta, S0)
    o2, st2 = ref.gated_deltanet(q, k, v, np.exp(a), beta, S0)
    assert rel(o, o2) < 1e-12 and rel(st, st2) < 1e-12


def test_p4_beta_zero_is_pure_decay():
    """beta == 0 writes and erases nothing: S_t = Diag(e^{sum log a}) S0; with
    alpha == 1 as well the state is frozen, o_t = S0^T q_t and S_T = S0."""
    rng = np.random.default_rng(4)
    q, k, v, la, _ = rand_inputs(rng, 30, 16, 8)
    S0 = rng.standard_normal((16, 8))
    o, st = run1(q, k, v, la, np.zeros(30), S0)
    o2, st2 = ref.decay_only(q, la, S0)
    assert rel(o, o2) < 1e-12 and rel(st, st2) < 1e-12
    o, st = run1(q, k, v, np.zeros((30, 16)), np.zeros(30), S0)
    assert rel(o, q @ S0) < 1e-14 and rel(st, S0) == 0.0


def test_p5_orthonormal_keys_give_linear_attention():
    """alpha == 1, beta == 1, S0 = 0 and mutually orthogonal unit keys: every
    erase term k_t^T S_{t-1} vanishes and KDA equals un-normalised causal
    linear attention o_t = sum_{j<=t} (q_t . k_j) v_j, evaluated here in its
    attention form (jokeuncle page, '第一步')."""
    rng = np.random.default_rng(5)
    dk, dv, T = 64, 48, 64
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T]                                        # orthonormal rows
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    o, st = run1(q, k, v, np.zeros((T, dk)), np.ones(T))
    assert rel(o, ref.linear_attention_parallel(q, k, v)) < 1e-12
    assert rel(st, k.T @ v) < 1e-12


@pytest.mark.parametrize("seed", [6, 7])
def test_p6_exact_recall(seed):
    """With beta_t = 1/|k_t|^2 the update is an exact reconstruction step:
    S_t^T k_t = v_t for ANY decay and any S0, so q_t = k_t gives o_t = v_t
    (delta rule as a reconstruction loss step, jokeuncle page '第二步')."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 50, 32, 16
    q, k, v, la, _ = rand_inputs(rng, T, dk, dv, normalise=False)
    beta = 1.0 / np.sum(k * k, axis=1)
    S0 = rng.standard_normal((dk, dv))
    o, _ = run1(k, k, v, la, beta, S0)
    assert rel(o, v) < 1e-12


@pytest.mark.parametrize("T,d,C,sub", [(37, 8, 16, None), (37, 8, 16, 4),
                                       (200, 128, 64, None), (200, 128, 64, 16),
                                       (100, 128, 32, 16)])
def test_p7_chunkwise_derivation_matches_recurrence(T, d, C, sub):
    """The chunkwise algebra (k+/k-, (I+L)^{-1}, O, state hand-off; hjcheng0602.cn
    eqs. (8)-(66)) reproduces the recurrence, with and without sub-tile
    references, including a partial last chunk."""
    rng = np.random.default_rng(8)
    q, k, v, la, beta = rand_inputs(rng, T, d, d)
    S0 = 0.02 * rng.standard_normal((d, d))
    o, st = run1(q, k, v, la, beta, S0)
    o2, st2 = chunkwise(q, k, v, la, beta, S0, chunk=C, sub_tile=sub)
    assert rel(o2, o) < 1e-10 and rel(st2, st) < 1e-10


def test_p8_linear_in_values_and_state():
    """For fixed q, k, alpha, beta the map (V, S0) -> (O, S_T) is linear."""
    rng = np.random.default_rng(9)
    q, k, v1, la, beta = rand_inputs(rng, 25, 16, 12)
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = rng.standard_normal((2, 16, 12))
    a, b = 0.7, -1.3
    o1, t1 = run1(q, k, v1, la, beta, s1)
    o2, t2 = run1(q, k, v2, la, beta, s2)
    o3, t3 = run1(q, k, a * v1 + b * v2, la, beta, a * s1 + b * s2)
    assert rel(o3, a * o1 + b * o2) < 1e-12 and rel(t3, a * t1 + b * t2) < 1e-12


def test_p9_continuation():
    """Running x[:T1] then x[T1:] from the carried state equals one run."""
    rng = np.random.default_rng(10)
    q, k, v, la, beta = rand_inputs(rng, 60, 16, 16)
    S0 = rng.standard_normal((16, 16))
    o, st = run1(q, k, v, la, beta, S0)
    oa, sa = run1(q[:23], k[:23], v[:23], la[:23], beta[:23], S0)
    ob, sb = run1(q[23:], k[23:], v[23:], la[23:], beta[23:], sa)
    assert rel(np.concatenate([oa, ob]), o) == 0.0 and rel(sb, st) == 0.0


def test_p10_varlen_packing_equals_separate_runs():
    rng = np.random.default_rng(11)
    lens = [5, 1, 17, 9]
    H, d = 3, 8
    T = sum(lens)
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    la = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, d))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = rng.standard_normal((len(lens), H, d, d))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, st = oracle.forward(q, k, v, la, beta, S0, cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        for h in range(H):
            o1, s1 = run1(q[sl, h], k[sl, h], v[sl, h], la[sl, h], beta[sl, h], S0[n, h])
            assert rel(o[sl, h], o1) == 0.0 and rel(st[n, h], s1) == 0.0


def test_p11_decode_chain_equals_prefill():
    """T chained decode steps equal one prefill over the same T tokens."""
    rng = np.random.default_rng(12)
    B, H, d, T = 3, 2, 16, 7
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    la = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, d))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = rng.standard_normal((B, H, d, d))
    o, st = oracle.forward(q, k, v, la, beta, S0)
    S = S0.copy()
    for t in range(T):
        ot, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], beta[:, t], S)
        assert rel(ot, o[:, t]) == 0.0
    assert rel(S, st) == 0.0


def test_p13_extreme_decay_forgets():
    """log alpha == -5 on every channel: the state keeps e^{-5} per step of the
    past, so o_t matches the one-token readout up to that order (lower-bounded
    decay, 'Kimi K3 技术报告解读' section 3.5)."""
    rng = np.random.default_rng(13)
    q, k, v, _, beta = rand_inputs(rng, 40, 16, 16)
    la = np.full((40, 16), -5.0)
    o, st = run1(q, k, v, la, beta)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    last = beta[:, None] * (q * k).sum(1, keepdims=True) * v   # S_t ~ b k v^T
    assert np.max(np.abs(o - last)) < 0.05 * np.max(np.abs(o))


def test_p14_unrolled_product_brute_force():
    """Tiny inputs against the unrolled closed form (hjcheng0602.cn eq. (6))."""
    rng = np.random.default_rng(14)
    for dk, dv, T in [(2, 3, 4), (3, 2, 5), (4, 4, 3)]:
        q, k, v, la, beta = rand_inputs(rng, T, dk, dv)
        S0 = rng.standard_normal((dk, dv))
        o, st = run1(q, k, v, la, beta, S0)
        o2, st2 = ref.unrolled_product(q, k, v, la, beta, S0)
        assert rel(o, o2) < 1e-12 and rel(st, st2) < 1e-12


def test_column_subset_equals_full_run():
    """Computing only some value columns gives those columns of the full run
    (the transition acts on S from the left)."""
    rng = np.random.default_rng(15)
    q, k, v, la, beta = rand_inputs(rng, 33, 16, 16)
    S0 = rng.standard_normal((1, 1, 16, 16))
    o, st = oracle.forward(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None], S0)
    o2, st2 = oracle.forward(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None],
                             S0, cols=(5, 11))
    assert np.array_equal(o[..., 5:11], o2[..., 5:11]) and np.all(o2[..., :5] == 0)
    assert np.array_equal(st[..., 5:11], st2[..., 5:11])


def test_unit_subset_equals_full_run():
    rng = np.random.default_rng(16)
    T, H, d = 12, 4, 8
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    la = -rng.random((T, H, d))
    beta = rng.random((T, H))
    cu = np.array([0, 5, 12])
    o, st = oracle.forward(q, k, v, la, beta, None, cu)
    o2, st2 = oracle.forward(q, k, v, la, beta, None, cu, units=[(1, 2), (0, 3)])
    assert np.array_equal(o2[5:, 2], o[5:, 2]) and np.array_equal(o2[:5, 3], o[:5, 3])
    assert np.array_equal(st2[1, 2], st[1, 2]) and np.all(st2[0, 0] == 0)
