"""GPU parity of kda_recurrent_fwd (multi-token decode, speculative replay)
against the fp64 oracle, through the C ABI.

The expected values come from the oracle's token-by-token forward pass:
the replayed prefix of each request from its initial state, then the new
tokens from the state after the replay.
"""
import numpy as np
import pytest

from gated_delta_rule_amd import workloads as W
from kda_testlib import TOL_BF16, TOL_F32, rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_amd as kda  # noqa: E402
import oracle  # noqa: E402

NAMES = ("q", "k", "v", "log_alpha", "beta")


def tokens(B, T, H, dtype="bf16", seed=0):
    """Decode-workload token streams [B, T, H, ...] (T steps of workload 4's
    per-step generator, one step per token)."""
    w = W.workload(4).shrink(B=B, H=H, dtype=dtype)
    steps = [W.decode_inputs(w, seed * 1000 + t) for t in range(T)]
    return {n: np.stack([s[n] for s in steps], axis=1) for n in NAMES}, w


def state(B, H, seed=0):
    rng = np.random.default_rng(1234 + seed)
    return (0.02 * rng.standard_normal((B, H, 128, 128))).astype(np.float32)


def dev(arrs, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {n: torch.from_numpy(np.ascontiguousarray(arrs[n])).cuda().to(dt) for n in ("q", "k", "v")}
    for n in ("log_alpha", "beta"):
        out[n] = torch.from_numpy(np.ascontiguousarray(arrs[n])).cuda()
    return out


def oracle_run(arrs, S0, n=None):
    """Oracle over the first n[b] tokens of each request (all when None):
    returns (o [B, T, H, 128] for the full T when n is None, S after)."""
    B = S0.shape[0]
    if n is None:
        return oracle.forward(*(arrs[x] for x in NAMES), S0, None)
    S = np.empty_like(S0, dtype=np.float64)
    for b in range(B):
        if n[b] == 0:
            S[b] = S0[b]
            continue
        sub = {x: arrs[x][b:b + 1, :n[b]] for x in NAMES}
        _, s = oracle.forward(*(sub[x] for x in NAMES), S0[b:b + 1], None)
        S[b] = s[0]
    return None, S


@pytest.mark.parametrize("B,T,H,dtype", [(3, 17, 4, "bf16"), (2, 64, 3, "bf16"),
                                         (2, 5, 2, "f32"), (4, 1, 3, "bf16")])
def test_multi_token_decode_commit(B, T, H, dtype):
    arrs, _ = tokens(B, T, H, dtype)
    S0 = state(B, H)
    d = dev(arrs, dtype)
    S = torch.from_numpy(S0).cuda()
    say(f"[recurrent] B={B} T={T} H={H} {dtype}: GPU")
    o = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S)
    torch.cuda.synchronize()
    ro, rs = oracle_run(arrs, S0)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rs)
    say(f"[recurrent] B={B} T={T} H={H} {dtype}: rel err o {eo:.3e} S {es:.3e}")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("commit", [False, True])
def test_speculative_replay(commit):
    """Replay the accepted prefix of the previous drafts, then verify new
    drafts; commit=False leaves exactly the accepted tokens in the state."""
    B, H, Tr, T = 4, 3, 5, 4
    rep, _ = tokens(B, Tr, H, seed=1)
    new, _ = tokens(B, T, H, seed=2)
    S0 = state(B, H, seed=3)
    n = np.array([0, 3, 5, 1], np.int32)
    dr, dn = dev(rep, "bf16"), dev(new, "bf16")
    S = torch.from_numpy(S0).cuda()
    say(f"[recurrent] speculative replay commit={commit}: GPU")
    o = kda.recurrent_fwd(dn["q"], dn["k"], dn["v"], dn["log_alpha"], dn["beta"], S,
                          replay=tuple(dr[x] for x in NAMES),
                          n_replay=torch.from_numpy(n).cuda(), commit=commit)
    torch.cuda.synchronize()
    _, s_mid = oracle_run(rep, S0, n)
    ro, s_end = oracle_run(new, s_mid.astype(np.float64))
    eo = rel_err(o.cpu().numpy(), ro)
    es = rel_err(S.cpu().numpy(), s_end if commit else s_mid)
    say(f"[recurrent] speculative replay commit={commit}: rel err o {eo:.3e} S {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


@pytest.mark.parametrize("T,Tr", [(2, 0), (3, 0), (9, 0), (1, 1), (1, 2), (2, 1), (0, 3)])
def test_forms_around_the_threshold(T, Tr):
    """Two tokens per state (new plus replayed) run the 1024-thread form,
    three or more the 512-thread form (eight tokens per staging pass, so 9
    takes two passes): each against the oracle, with the replay count of
    every request drawn below or at Tr, committing after all tokens."""
    B, H = 6, 3
    rep, _ = tokens(B, max(Tr, 1), H, seed=7)
    new, _ = tokens(B, max(T, 1), H, seed=8)
    rep = {x: a[:, :Tr] for x, a in rep.items()}
    new = {x: a[:, :T] for x, a in new.items()}
    S0 = state(B, H, seed=9)
    n = (np.arange(B) % (Tr + 1)).astype(np.int32)
    dr, dn = dev(rep, "bf16"), dev(new, "bf16")
    S = torch.from_numpy(S0).cuda()
    say(f"[recurrent] T={T} Tr={Tr}: GPU")
    o = kda.recurrent_fwd(dn["q"], dn["k"], dn["v"], dn["log_alpha"], dn["beta"], S,
                          replay=tuple(dr[x] for x in NAMES) if Tr else None,
                          n_replay=torch.from_numpy(n).cuda() if Tr else None, commit=True)
    torch.cuda.synchronize()
    s_mid = oracle_run(rep, S0, n)[1] if Tr else S0.astype(np.float64)
    if T:
        ro, s_end = oracle_run(new, s_mid.astype(np.float64))
        eo = rel_err(o.cpu().numpy(), ro)
    else:
        s_end, eo = s_mid, 0.0
    es = rel_err(S.cpu().numpy(), s_end)
    say(f"[recurrent] T={T} Tr={Tr}: rel err o {eo:.3e} S {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_replay_all_and_state_only():
    """n_replay omitted (all replay tokens) and no new tokens: the state
    advances by the replay alone."""
    B, H, Tr = 2, 2, 20
    rep, _ = tokens(B, Tr, H, seed=4)
    S0 = state(B, H, seed=5)
    dr = dev(rep, "bf16")
    empty = {x: t[:, :0].contiguous() for x, t in dr.items()}
    S = torch.from_numpy(S0).cuda()
    kda.recurrent_fwd(empty["q"], empty["k"], empty["v"], empty["log_alpha"], empty["beta"], S,
                      replay=tuple(dr[x] for x in NAMES), commit=False)
    torch.cuda.synchronize()
    _, rs = oracle_run(rep, S0)
    es = rel_err(S.cpu().numpy(), rs)
    say(f"[recurrent] replay only: rel err S {es:.3e}")
    assert es <= TOL_BF16


def test_single_token_matches_decode_step():
    B, H = 5, 3
    arrs, _ = tokens(B, 1, H, seed=6)
    S0 = state(B, H, seed=7)
    d = dev(arrs, "bf16")
    S1 = torch.from_numpy(S0).cuda()
    S2 = S1.clone()
    o1 = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S1)
    o2 = kda.decode_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(),
                         d["v"][:, 0].contiguous(), d["log_alpha"][:, 0].contiguous(),
                         d["beta"][:, 0].contiguous(), S2)
    torch.cuda.synchronize()
    assert rel_err(o1[:, 0].cpu().numpy(), o2.cpu().numpy()) < 1e-5
    assert rel_err(S1.cpu().numpy(), S2.cpu().numpy()) < 1e-5


def test_deterministic():
    B, T, H = 3, 9, 2
    arrs, _ = tokens(B, T, H, seed=8)
    S0 = state(B, H, seed=9)
    d = dev(arrs, "bf16")
    outs = []
    for _ in range(2):
        S = torch.from_numpy(S0).cuda()
        o = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S)
        torch.cuda.synchronize()
        outs.append((o.cpu(), S.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("B,H,T,replay", [(65, 67, 5, False), (65, 67, 17, False),
                                          (67, 97, 1, False), (65, 67, 4, True)])
def test_many_states_per_workgroup(B, H, T, replay):
    """Batches of 4,096+ states, where a workgroup walks several states and
    reads the next one (and, with 2..16 tokens and no replay, its tokens)
    while the current one runs; state counts that leave a short last
    workgroup."""
    new, _ = tokens(B, T, H, seed=6)
    S0 = state(B, H, seed=7)
    dn = dev(new, "bf16")
    S = torch.from_numpy(S0).cuda()
    say(f"[recurrent] {B * H} states T={T} replay={replay}: GPU")
    if replay:
        rep, _ = tokens(B, 3, H, seed=8)
        n = np.random.default_rng(9).integers(0, 4, B).astype(np.int32)
        dr = dev(rep, "bf16")
        o = kda.recurrent_fwd(dn["q"], dn["k"], dn["v"], dn["log_alpha"], dn["beta"], S,
                              replay=tuple(dr[x] for x in NAMES),
                              n_replay=torch.from_numpy(n).cuda(), commit=False)
        torch.cuda.synchronize()
        _, s_mid = oracle_run(rep, S0, n)
        ro, _ = oracle_run(new, s_mid.astype(np.float64))
        rs = s_mid
    else:
        o = kda.recurrent_fwd(dn["q"], dn["k"], dn["v"], dn["log_alpha"], dn["beta"], S)
        torch.cuda.synchronize()
        ro, rs = oracle_run(new, S0)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rs)
    say(f"[recurrent] {B * H} states T={T} replay={replay}: rel err o {eo:.3e} S {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)
