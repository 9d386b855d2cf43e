"""GPU cases that reach every kernel instantiation the ABI can choose, the
integer work of the packed-batch ordering, and the degenerate gate beta = 0.

* The prefill runs two value slices per head (pipelined bf16 kernel, or the
  16-column fp32 kernel) when there are fewer than 256 (sequence, head)
  pairs, and one 32-column slice per head otherwise; the cases below with
  N * H >= 256 take the one-slice kernels in fp32 and bf16, with packed
  sequences of 0, 1, 31, 33 tokens, and through the backward's forward pass.
* P0: the packed-batch order written into the caller's workspace is a stable
  longest-first sort of the sequence lengths (ties keep index order, empty
  sequences last); above 4096 sequences no order is used (the workspace
  query returns 0) and every sequence still gets its own result.
* beta == 0 removes every write: S_t = Diag(exp(sum log alpha)) S0 and
  o_t = S_t^T q_t ("Kimi K3 核心算子拆解" section 2.2: beta is the write
  strength of the rank-1 update).
"""
import numpy as np
import pytest

from gated_delta_rule_amd import workloads as W
from kda_testlib import TOL_BF16, TOL_F32, rel_err, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_amd as kda  # noqa: E402
import oracle  # noqa: E402


def packed(lens, H, dtype="bf16", s0=0.02, seed=0):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    w = W.workload(0 if dtype == "f32" else 2).shrink(n_varlen=0, B=1, T=T, H=H, dtype=dtype,
                                                      s0_std=0.0)
    a = W.prefill_inputs(w)
    rng = np.random.default_rng(seed)
    S0 = (s0 * rng.standard_normal((len(lens), H, 128, 128))).astype(np.float32) if s0 else None
    arrs = {n: a[n] for n in ("q", "k", "v", "log_alpha", "beta")}
    arrs["S0"] = S0
    return w, arrs, cu


def run_and_compare(w, arrs, cu, tol, label, workspace=None):
    d = to_dev(arrs, w)
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    say(f"[coverage] {label}: GPU")
    o, st = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], cu_dev,
                          workspace=workspace)
    torch.cuda.synchronize()
    say(f"[coverage] {label}: oracle")
    ro, rs = oracle.forward(arrs["q"], arrs["k"], arrs["v"], arrs["log_alpha"], arrs["beta"],
                            arrs["S0"], cu)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(st.cpu().numpy(), rs)
    say(f"[coverage] {label}: rel err o {eo:.3e}  S_T {es:.3e}  (tol {tol})")
    assert eo <= tol and es <= tol, (eo, es)
    return o, st


# ---------------------------------------------------------------- P0 order
def test_order_workspace_is_stable_longest_first():
    lens = [5, 0, 33, 5, 64, 0, 1, 33, 200, 64, 5, 31]
    H = 2
    w, arrs, cu = packed(lens, H)
    n = len(lens)
    assert kda.chunk_fwd_workspace_bytes(n, int(cu[-1]), H, varlen=True) == 4 * n
    ws = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    run_and_compare(w, arrs, cu, TOL_BF16, f"order lens={lens}", workspace=ws)
    got = ws.cpu().numpy()
    want = np.argsort(-np.asarray(lens), kind="stable")
    say(f"[coverage] order {got.tolist()}")
    assert np.array_equal(got, want)


def test_order_random_lengths_with_many_ties():
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 6, size=300).tolist()      # 300 sequences, lengths 0..5
    w, arrs, cu = packed(lens, 1, s0=0.0)
    ws = torch.empty((len(lens),), dtype=torch.int32, device="cuda")
    run_and_compare(w, arrs, cu, TOL_BF16, "order 300 short sequences, H=1", workspace=ws)
    assert np.array_equal(ws.cpu().numpy(), np.argsort(-np.asarray(lens), kind="stable"))


def test_more_than_4096_sequences_run_unsorted():
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 40, size=4100).tolist()
    lens[17] = 70                                      # one multi-chunk sequence
    H = 2
    w, arrs, cu = packed(lens, H, s0=0.0)
    assert kda.chunk_fwd_workspace_bytes(len(lens), int(cu[-1]), H, varlen=True) == 0
    run_and_compare(w, arrs, cu, TOL_BF16, "4100 packed sequences (no order), H=2")


# ------------------------------------------- one-slice kernels, N * H >= 256
def test_fp32_one_slice_equal_lengths():
    B, T, H = 3, 45, 96          # 288 (sequence, head) pairs
    w = W.workload(0).shrink(T=T, H=H, B=B, s0_std=0.02)
    a = W.prefill_inputs(w)
    r = {n: a[n].reshape((B, T) + a[n].shape[1:]) for n in ("q", "k", "v", "log_alpha", "beta")}
    d = to_dev(dict(r, S0=a["S0"]), w)
    say("[coverage] fp32 B=3 T=45 H=96: GPU")
    o, st = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    ro, rs = oracle.forward(r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], a["S0"])
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(st.cpu().numpy(), rs)
    say(f"[coverage] fp32 one slice: rel err o {eo:.3e}  S_T {es:.3e}")
    assert eo <= TOL_F32 and es <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_slice_packed_edge_lengths(dtype):
    lens = [0, 1, 31, 33, 64, 100]
    H = 48                       # 6 * 48 = 288 pairs
    w, arrs, cu = packed(lens, H, dtype=dtype)
    run_and_compare(w, arrs, cu, TOL_F32 if dtype == "f32" else TOL_BF16,
                    f"one slice {dtype} lens={lens} H={H}", workspace=None)


def test_same_sequence_in_both_slice_plans():
    """One sequence alone (2 slices per head) and inside a batch with >= 256
    (sequence, head) pairs (1 slice per head): both within the tolerance of
    the oracle, and of each other."""
    lens = [150]
    H = 96
    w, arrs, cu = packed(lens * 3, H)
    o3, s3 = run_and_compare(w, arrs, cu, TOL_BF16, "3 x 150 tokens, H=96 (one slice)")
    one = {n: (None if v is None else v[:150] if n != "S0" else v[:1]) for n, v in arrs.items()}
    o1, s1 = run_and_compare(w, one, cu[:2], TOL_BF16, "1 x 150 tokens, H=96 (two slices)")
    e = rel_err(o1.cpu().numpy(), o3[:150].cpu().numpy())
    say(f"[coverage] two-slice vs one-slice plan: o {e:.3e}")
    assert e <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_one_slice(dtype):
    """The backward's forward pass with >= 256 pairs (one slice per head,
    states stored); all six gradients against the oracle's backward."""
    lens = [0, 1, 31, 33, 70]
    H = 64                       # 5 * 64 = 320 pairs
    w, arrs, cu = packed(lens, H, dtype=dtype)
    dO, dS = W.grad_inputs(w, int(cu[-1]), len(lens), 1.0)
    d = to_dev(arrs, w)
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    say(f"[coverage] backward one slice {dtype}: GPU")
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                      torch.from_numpy(dO).cuda(), torch.from_numpy(dS).cuda(), cu_dev)
    torch.cuda.synchronize()
    say(f"[coverage] backward one slice {dtype}: oracle")
    ref = oracle.backward(arrs["q"], arrs["k"], arrs["v"], arrs["log_alpha"], arrs["beta"],
                          arrs["S0"], dO, dS, cu)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for name, x, r in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), g, ref):
        e = rel_err(x.cpu().numpy().reshape(r.shape), r)
        say(f"[coverage]   {name} {e:.2e}")
        assert e <= tol, (name, e)


# ------------------------------------------------------------- beta == 0
@pytest.mark.parametrize("H", [2, 96])
def test_prefill_beta_zero_is_pure_decay(H):
    lens = [1, 33, 100] if H == 2 else [40, 0, 70]
    w, arrs, cu = packed(lens, H)
    arrs["beta"] = np.zeros_like(arrs["beta"])
    # a mild decay (log alpha in (-0.05, 0)), so that the state after 100
    # tokens is still far from fp32's underflow
    arrs["log_alpha"] = (0.01 * arrs["log_alpha"]).astype(np.float32)
    o, st = run_and_compare(w, arrs, cu, TOL_BF16, f"beta == 0, H={H}")
    # closed form: per sequence S_T = Diag(exp(sum log alpha)) S0
    la = arrs["log_alpha"].astype(np.float64)
    for n in range(len(lens)):
        g = la[cu[n]:cu[n + 1]].sum(axis=0)                       # [H, dk]
        want = np.exp(g)[:, :, None] * arrs["S0"][n].astype(np.float64)
        assert rel_err(st[n].cpu().numpy(), want) <= TOL_BF16


def test_decode_beta_zero_is_pure_decay():
    w = W.workload(4).shrink(B=5, H=7)
    a = W.decode_inputs(w, 0)
    a["beta"] = np.zeros_like(a["beta"])
    S_h = W.decode_state(w)
    d = {n: torch.from_numpy(a[n]).cuda() for n in a}
    for n in ("q", "k", "v"):
        d[n] = d[n].to(torch.bfloat16)
    S = torch.from_numpy(S_h).cuda()
    o = kda.decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S)
    torch.cuda.synchronize()
    ro, rS = oracle.decode_step(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], S_h)
    want = np.exp(a["log_alpha"].astype(np.float64))[..., None] * S_h.astype(np.float64)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rS)
    say(f"[coverage] decode beta == 0: rel err o {eo:.3e} S {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert rel_err(S.cpu().numpy(), want) <= 1e-6


# ------------------------------------------ equal-length batches of length 0
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_length_sequences_pass_the_state_through(dtype):
    """B = 2 sequences of T = 0 tokens: the forward returns S_T = S0 and the
    backward grad_S0 = grad_S_T, exactly (no token touches either), through
    the same entry points and launches as any other equal-length batch."""
    B, H = 2, 3
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(5)
    z = lambda *s, t=torch.float32: torch.empty(s, dtype=t, device="cuda")
    q, k, v = z(B, 0, H, 128, t=dt), z(B, 0, H, 128, t=dt), z(B, 0, H, 128, t=dt)
    la, b = z(B, 0, H, 128), z(B, 0, H)
    S0 = torch.randn((B, H, 128, 128), device="cuda", generator=g)
    o, st = kda.chunk_fwd(q, k, v, la, b, S0)
    gst = torch.randn((B, H, 128, 128), device="cuda", generator=g)
    grads = kda.chunk_bwd(q, k, v, la, b, S0, z(B, 0, H, 128), gst)
    torch.cuda.synchronize()
    say(f"[coverage] T=0 {dtype}: |S_T - S0| {float((st - S0).abs().max()):.1e}, "
        f"|dS0 - dS_T| {float((grads[5] - gst).abs().max()):.1e}")
    assert o.numel() == 0 and torch.equal(st, S0)
    assert all(t.numel() == 0 for t in grads[:5]) and torch.equal(grads[5], gst)
