"""GPU parity of kda_chunk_fwd against the fp64 oracle (through the C ABI).

Small and ragged cases compare every output element; the full-size
workloads compare sampled heads / sequences / value columns that the oracle
computes on its own (each value column of the state evolves independently,
so the oracle can follow a few columns of a 1M-token head exactly).
"""
import numpy as np
import pytest

from gated_delta_rule_amd import workloads as W
from kda_testlib import (TOL_BF16, TOL_F32, device_prefill_inputs, oracle_head, rel_err,
                         say, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_amd as kda  # noqa: E402
import oracle  # noqa: E402


def run_gpu(d, cu=None):
    o, st = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                          cu)
    torch.cuda.synchronize()
    return o, st


def check_full(w, arrs, cu=None, tol=TOL_BF16, label=""):
    """All outputs of a small case against the oracle."""
    d = to_dev(arrs, w)
    cu_dev = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    say(f"[prefill] {label}: GPU")
    o, st = run_gpu(d, cu_dev)
    say(f"[prefill] {label}: oracle")
    q = arrs["q"]
    if cu is None and q.ndim == 3:   # [T, H, d] single sequence
        lead = dict(q=arrs["q"][None], k=arrs["k"][None], v=arrs["v"][None],
                    log_alpha=arrs["log_alpha"][None], beta=arrs["beta"][None])
    else:
        lead = arrs
    ro, rs = oracle.forward(lead["q"], lead["k"], lead["v"], lead["log_alpha"], lead["beta"],
                            arrs.get("S0"), cu)
    eo = rel_err(o.cpu().numpy().reshape(ro.shape), ro)
    es = rel_err(st.cpu().numpy(), rs)
    say(f"[prefill] {label}: rel err o {eo:.3e}  S_T {es:.3e}  (tol {tol})")
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


def small(T, H, B=1, s0=0.0, dtype="bf16", wid=1):
    w = W.workload(wid).shrink(T=T, H=H, B=B, s0_std=s0, dtype=dtype)
    a = W.prefill_inputs(w)
    # equal-length batch layout [B, T, H, d]
    out = {n: a[n].reshape((B, T) + a[n].shape[1:]) for n in ("q", "k", "v", "log_alpha", "beta")}
    out["S0"] = a["S0"]
    return w, out


def test_workload0_fp32_full():
    """Single fp32 head, T=256, S0=0: every element, tolerance 1e-5."""
    w = W.workload(0)
    a = W.prefill_inputs(w)
    arrs = {n: a[n][None] for n in ("q", "k", "v", "log_alpha", "beta")}
    arrs["S0"] = None
    check_full(w, arrs, tol=TOL_F32, label="workload 0 (fp32, T=256)")


@pytest.mark.parametrize("T,H,B,s0", [(1, 1, 1, 0.0), (16, 1, 1, 0.02), (31, 2, 1, 0.0),
                                      (32, 1, 2, 0.02), (33, 3, 1, 0.0), (100, 2, 3, 0.02),
                                      (257, 5, 1, 0.02), (0, 2, 2, 0.02)])
def test_bf16_ragged(T, H, B, s0):
    w, arrs = small(T, H, B, s0)
    check_full(w, arrs, label=f"bf16 T={T} H={H} B={B} s0={s0}")


@pytest.mark.parametrize("T,H,B", [(1, 1, 1), (45, 2, 2), (300, 3, 1)])
def test_fp32_ragged(T, H, B):
    w, arrs = small(T, H, B, 0.02, dtype="f32", wid=0)
    check_full(w, arrs, tol=TOL_F32, label=f"fp32 T={T} H={H} B={B}")


def test_varlen_packing_with_empty_and_ragged_sequences():
    lens = [17, 0, 1, 32, 33, 200, 64, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    w = W.workload(2).shrink(n_varlen=0, B=1, T=T, H=4)
    a = W.prefill_inputs(w)
    rng = np.random.default_rng(0)
    a["S0"] = (0.02 * rng.standard_normal((len(lens), 4, 128, 128))).astype(np.float32)
    arrs = {n: a[n] for n in ("q", "k", "v", "log_alpha", "beta", "S0")}
    check_full(w, arrs, cu=cu, label=f"varlen lens={lens}")


@pytest.mark.parametrize("T", [64, 65, 96, 97, 128])
def test_bf16_pipeline_fill_and_drain(T):
    """Two to four chunks per sequence: the bf16 kernel overlaps the gate scan of
    chunk n+2, the tiles of chunk n+1 and the state update of chunk n, so short
    sequences end the pipeline before it is full."""
    w, arrs = small(T, 2, 1, 0.02)
    check_full(w, arrs, label=f"bf16 pipeline T={T}")


def test_varlen_pipeline_lengths_mixed():
    """Packed sequences of 1 to 4 chunks (and ragged tails) in one launch."""
    lens = [1, 32, 33, 64, 65, 96, 97, 0, 2, 128]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    w = W.workload(2).shrink(n_varlen=0, B=1, T=T, H=2)
    a = W.prefill_inputs(w)
    rng = np.random.default_rng(1)
    a["S0"] = (0.02 * rng.standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    arrs = {n: a[n] for n in ("q", "k", "v", "log_alpha", "beta", "S0")}
    check_full(w, arrs, cu=cu, label=f"varlen pipeline lens={lens}")


@pytest.mark.parametrize("scale", [1e-4, 3e4])
@pytest.mark.parametrize("H,B", [(2, 2), (96, 3)])
def test_value_scale_edges(scale, H, B):
    """v and S0 scaled by 1e-4 and by 3e4 (states up to about 1.4e4): with
    fewer than 256 (sequence, head) pairs Q+ S runs on fp16 matrix cores, whose
    range these scales approach from both sides; with 256 or more on bf16.
    Every element against the oracle."""
    w, arrs = small(70, H, B, 0.02)
    arrs["v"] = W.round_bf16((arrs["v"].astype(np.float64) * scale).astype(np.float32))
    arrs["S0"] = (arrs["S0"].astype(np.float64) * scale).astype(np.float32)
    check_full(w, arrs, label=f"value scale {scale:g}, H={H} B={B}")


def test_continuation_matches_single_run():
    """chunk_fwd(x[:T1]) then chunk_fwd(x[T1:], S0=S_T1) equals chunk_fwd(x)."""
    w, arrs = small(300, 2, 1, 0.02)
    d = to_dev(arrs, w)
    say("[prefill] continuation")
    o, st = run_gpu(d)
    T1 = 77
    d1 = {n: (t[:, :T1].contiguous() if n not in ("S0",) and t is not None else t)
          for n, t in d.items()}
    o1, s1 = run_gpu(d1)
    d2 = {n: (t[:, T1:].contiguous() if n not in ("S0",) and t is not None else t)
          for n, t in d.items()}
    d2["S0"] = s1
    o2, s2 = run_gpu(d2)
    oc = torch.cat([o1, o2], dim=1)
    assert rel_err(oc.cpu().numpy(), o.cpu().numpy()) < 1e-3
    assert rel_err(s2.cpu().numpy(), st.cpu().numpy()) < 1e-3


def test_exact_recall():
    """q_t = k_t and beta_t = 1/|k_t|^2 make every step an exact reconstruction,
    so o_t = v_t whatever the decay and S0 (the delta rule as a reconstruction
    step).  Checked through the kernel at the bf16 tolerance."""
    w, arrs = small(200, 2, 1, 0.02)
    k = arrs["k"].astype(np.float64)
    arrs["q"] = arrs["k"].copy()
    arrs["beta"] = (1.0 / np.sum(k * k, axis=-1)).astype(np.float32)
    d = to_dev(arrs, w)
    say("[prefill] exact recall")
    o, _ = run_gpu(d)
    e = rel_err(o.cpu().numpy(), arrs["v"])
    say(f"[prefill] exact recall rel err {e:.3e}")
    assert e <= TOL_BF16


def test_state_in_place_and_no_state():
    w, arrs = small(90, 2, 2, 0.02)
    d = to_dev(arrs, w)
    o_ref, st_ref = run_gpu(d)
    S = d["S0"].clone()
    o, st = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S, None, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, st_ref)
    o2, st2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], None,
                            output_final_state=False)
    torch.cuda.synchronize()
    assert st2 is None and torch.equal(o2, o_ref)


def test_decay_extremes():
    """log alpha == -5 (the lower bound) and == 0 (no decay) on every channel."""
    for val in (-5.0, 0.0):
        w, arrs = small(130, 2, 1, 0.02)
        arrs["log_alpha"] = np.full_like(arrs["log_alpha"], val)
        check_full(w, arrs, label=f"log_alpha == {val}")


def test_deterministic():
    w, arrs = small(200, 3, 2, 0.02)
    d = to_dev(arrs, w)
    o1, s1 = run_gpu(d)
    o2, s2 = run_gpu(d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ------------------------------------------------ sequence-parallel path
# Equal-length batches with few (sequence, head) pairs and long sequences run
# as independent segments merged through their transitions (the workspace
# query reports the path: nonzero for equal lengths means it is taken).

@pytest.mark.parametrize("T,H,B,s0,dtype", [(7000, 3, 2, 0.02, "bf16"),   # 3 segments, ragged
                                            (8192, 4, 1, 0.0, "bf16"),    # 4 segments
                                            (6144, 2, 1, 0.02, "f32")])   # fp32 inputs, 3 segments
def test_sequence_parallel_matches_oracle(T, H, B, s0, dtype):
    assert kda.chunk_fwd_workspace_bytes(B, T, H, varlen=False) > 0
    w, arrs = small(T, H, B, s0, dtype=dtype, wid=0 if dtype == "f32" else 1)
    check_full(w, arrs, tol=TOL_F32 if dtype == "f32" else TOL_BF16,
               label=f"sequence-parallel {dtype} T={T} H={H} B={B} s0={s0}")


@pytest.mark.parametrize("T,H,B,dtype", [(8192, 64, 1, "bf16"),    # 4 segments x 64 heads
                                         (8192, 32, 2, "f32")])    # 2 x 4 segments x 32 heads
def test_sequence_parallel_fused_chains_match_oracle(T, H, B, dtype):
    """64 (sequence, head) pairs cut into four segments each: segment 0 on
    two workgroups per pair beside the dual-chain pass over the 128 middle
    chains (local final states and transitions from one launch on the same
    tiles), then the rerun on 192 one-workgroup chains; every output element
    against the oracle.  Workspace: transitions and local final states of
    the middle segments, incoming states of the later ones, segment 0's final
    states."""
    assert kda.chunk_fwd_workspace_bytes(B, T, H, varlen=False) == (2 * 2 + 3 + 1) * 64 * 65536
    w, arrs = small(T, H, B, 0.02, dtype=dtype, wid=0 if dtype == "f32" else 1)
    check_full(w, arrs, tol=TOL_F32 if dtype == "f32" else TOL_BF16,
               label=f"sequence-parallel fused chains {dtype} T={T} H={H} B={B}")


def test_sequence_parallel_agrees_with_sequential_and_in_place():
    w, arrs = small(7000, 3, 2, 0.02)
    d = to_dev(arrs, w)
    say("[prefill] sequence-parallel vs sequential")
    o_p, s_p = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    o_s, s_s = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                             sequence_parallel=False)
    S = d["S0"].clone()
    o_i, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S, S_T=S)
    torch.cuda.synchronize()
    eo = rel_err(o_p.cpu().numpy(), o_s.cpu().numpy())
    es = rel_err(s_p.cpu().numpy(), s_s.cpu().numpy())
    say(f"[prefill] parallel vs sequential: o {eo:.3e}  S_T {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert torch.equal(o_i, o_p) and torch.equal(S, s_p)   # S_T may be S0


def _seq_parallel_job(T, H, B, seed_s0=0.02):
    """Device inputs, outputs and workspace of one sequence-parallel call."""
    w, arrs = small(T, H, B, seed_s0)
    d = to_dev(arrs, w)
    lib = kda.load_library()
    wsb = lib.kda_chunk_fwd_workspace_bytes(B, T, H, 128, 128, 0)
    assert wsb > 0
    return dict(d=d, B=B, T=T, H=H, wsb=wsb,
                ws=torch.empty(wsb, dtype=torch.uint8, device="cuda"),
                o=torch.empty(d["v"].shape, dtype=torch.float32, device="cuda"),
                st=torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda"))


def _seq_parallel_call(job, stream_handle, noalloc=False):
    import ctypes
    lib = kda.load_library()
    vp = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    d = job["d"]
    args = [vp(d["q"]), vp(d["k"]), vp(d["v"]), kda.KDA_BF16, vp(d["log_alpha"]), vp(d["beta"]),
            vp(d["S0"]), None, job["B"], job["T"], job["H"], 128, 128, vp(job["o"]), vp(job["st"])]
    if noalloc:
        return lib.kda_chunk_fwd_noalloc(*args, ctypes.c_void_p(stream_handle))
    return lib.kda_chunk_fwd(*args, vp(job["ws"]), job["wsb"], ctypes.c_void_p(stream_handle))


@pytest.mark.parametrize("noalloc", [False, True])
def test_sequence_parallel_graph_capture_replays_bitwise(noalloc):
    """The sequence-parallel path runs each pass as two launches, one on the
    library's second stream (forked from and joined back into the caller's
    stream by events), so a HIP graph captured on the caller's stream takes
    in both: captured once, replayed three times with eager work and
    synchronisations between the replays, every replay equals the eager
    result bitwise (with a caller's workspace, and through the entry point
    that allocates nothing)."""
    job = _seq_parallel_job(7000, 3, 2)
    say(f"[prefill] graph capture (sequence-parallel, noalloc={noalloc}): eager")
    assert _seq_parallel_call(job, torch.cuda.current_stream().cuda_stream, noalloc) == 0
    torch.cuda.synchronize()
    ref = (job["o"].clone(), job["st"].clone())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    say("[prefill] graph capture: capture")
    with torch.cuda.graph(g, stream=s):
        rc = _seq_parallel_call(job, s.cuda_stream, noalloc)
    assert rc == 0
    for rep in range(3):
        job["o"].fill_(float("nan"))
        job["st"].fill_(float("nan"))
        job["ws"].fill_(0xFF)
        torch.cuda.synchronize()
        say(f"[prefill] graph capture: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(job["o"], ref[0]) and torch.equal(job["st"], ref[1])


def test_sequence_parallel_concurrent_threads_bitwise():
    """Two host threads run sequence-parallel calls at the same time on their
    own streams, inputs, outputs and workspaces (they share the library's
    second stream and its events and enqueue under one lock): every result
    equals the same call made alone, bitwise."""
    import threading
    jobs = [_seq_parallel_job(7000, 3, 2), _seq_parallel_job(8192, 4, 1)]
    for job in jobs:
        job["stream"] = torch.cuda.Stream()
    say("[prefill] two threads: each call alone")
    ref = []
    for job in jobs:
        assert _seq_parallel_call(job, job["stream"].cuda_stream) == 0
        torch.cuda.synchronize()
        ref.append((job["o"].clone(), job["st"].clone()))
    for rep in range(3):
        for job in jobs:
            job["o"].fill_(float("nan"))
            job["st"].fill_(float("nan"))
        torch.cuda.synchronize()
        rcs = [None, None]

        def worker(i):
            rcs[i] = [_seq_parallel_call(jobs[i], jobs[i]["stream"].cuda_stream) for _ in range(2)]

        say(f"[prefill] two threads: round {rep}")
        th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        torch.cuda.synchronize()
        assert rcs == [[0, 0], [0, 0]]
        for job, (o, st) in zip(jobs, ref):
            assert torch.equal(job["o"], o) and torch.equal(job["st"], st)


def _sampled_check(w, heads, label, seqs=None, cols=None):
    say(f"[prefill] {label}: generating inputs on the device")
    d, cu = device_prefill_inputs(w)
    if not w.varlen:   # equal-length layout [B, T, H, d]
        for n in ("q", "k", "v", "log_alpha", "beta"):
            d[n] = d[n].view((w.B, w.T) + tuple(d[n].shape[1:]))
    say(f"[prefill] {label}: GPU")
    o, st = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                          d["cu_seqlens"] if w.varlen else None)
    torch.cuda.synchronize()
    c0, c1 = (0, w.dv) if cols is None else cols
    worst_o = worst_s = 0.0
    for h in heads:
        say(f"[prefill] {label}: oracle head {h}")
        ro, rs = oracle_head(w, h, cu, cols=cols, seqs=seqs)
        go = o.view(-1, w.H, w.dv)[:, h, c0:c1].cpu().numpy()
        gs = st[:, h, :, c0:c1].cpu().numpy()
        if seqs is None:
            eo, es = rel_err(go, ro[:, c0:c1]), rel_err(gs, rs[:, :, c0:c1])
        else:
            rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
            eo = rel_err(go[rows], ro[rows, c0:c1])
            es = rel_err(gs[seqs], rs[seqs][:, :, c0:c1])
        say(f"[prefill] {label}: head {h} rel err o {eo:.3e} S_T {es:.3e}")
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    del d, o, st
    torch.cuda.empty_cache()
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16, (worst_o, worst_s)


@pytest.mark.timeout(600)
def test_workload1_full_size_sampled_heads():
    """T=8192, H=96, bf16, S0=0: heads 0, 41, 95 in full."""
    _sampled_check(W.workload(1), [0, 41, 95], "workload 1 (T=8192 H=96)")


@pytest.mark.timeout(600)
def test_workload2_full_size_sampled_units():
    """32 packed sequences (lengths 512..16384), H=96, S0 ~ N(0, 0.02^2):
    the longest and shortest sequences and two others, on three heads."""
    w = W.workload(2)
    cu = W.cu_seqlens(w)
    lens = np.diff(cu)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 3, 17})
    _sampled_check(w, [5, 60], "workload 2 (varlen, H=96)", seqs=seqs)


@pytest.mark.timeout(900)
def test_workload3_full_size_sampled_columns():
    """T=1,048,576, H=16: eight value columns of two heads, every token (the
    sequence-parallel path: 16 segments per head, the first on two
    workgroups, every later one on one 512-thread workgroup per chain)."""
    _sampled_check(W.workload(3), [0, 9], "workload 3 (T=1M H=16)", cols=(40, 48))
