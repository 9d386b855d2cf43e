"""GPU parity of kda_chunk_bwd (through the C ABI) against the fp64 oracle's
backward pass (oracle.backward, the reverse-mode derivative of the token
loop).  Small and ragged cases compare every element of all six gradients;
the full-size prefill shape compares sampled heads, which the oracle follows
on their own (every (sequence, head) chain is independent)."""
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

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def inputs(w, lens, s0, ds_std, la_const=None):
    """Token-major packed inputs for sequences of the given lengths (one
    seeded stream per head, cut into the sequences)."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, N = int(cu[-1]), len(lens)
    w = w.shrink(s0_std=s0)
    a = {n: np.empty((T, w.H) + ((w.dk,) if n != "beta" else ()), np.float32)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = np.empty((N, w.H, w.dk, w.dv), np.float32) if s0 else None
    for h in range(w.H):
        s = W.head_stream(w, h, T)
        for n in a:
            a[n][:, h] = s[n]
        if S0 is not None:
            S0[:, h] = W.initial_state_head(w, h, N)
    if la_const is not None:
        a["log_alpha"][:] = la_const
    dO, dS = W.grad_inputs(w, T, N, ds_std)
    return w, a, S0, dO, dS, cu


def run(w, a, S0, dO, dS, cu, equal=None, window_tokens=None):
    """GPU backward; `equal` = (B, T) passes the equal-length layout instead
    of cu_seqlens; window_tokens sizes its workspace for that window length."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in a}
    for n in ("q", "k", "v"):
        d[n] = d[n].to(dt)
    s0 = None if S0 is None else torch.from_numpy(S0).cuda()
    go = torch.from_numpy(dO).cuda()
    gst = None if dS is None else torch.from_numpy(dS).cuda()
    cu_dev = None
    if equal is not None:
        B, T = equal
        for n in d:
            d[n] = d[n].reshape((B, T) + tuple(d[n].shape[1:]))
        go = go.reshape((B, T) + tuple(go.shape[1:]))
    else:
        cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s0, go, gst, cu_dev,
                      window_tokens=window_tokens)
    torch.cuda.synchronize()
    T = a["q"].shape[0]
    out = [t.cpu().numpy() for t in g]
    for i in range(5):
        out[i] = out[i].reshape((T,) + out[i].shape[2 if equal else 1:])
    return out


def compare(w, a, S0, dO, dS, cu, tol, label, equal=None, window_tokens=None):
    say(f"[bwd] {label}: GPU")
    got = run(w, a, S0, dO, dS, cu, equal, window_tokens)
    say(f"[bwd] {label}: oracle")
    ref = oracle.backward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], S0, dO, dS, cu)
    errs = {n: rel_err(x, r) for n, x, r in zip(NAMES, got, ref)}
    say(f"[bwd] {label}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol})")
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return got


@pytest.mark.parametrize("lens,H,s0,ds", [([100, 100], 3, 0.02, 1.0), ([1], 1, 0.0, 0.0),
                                          ([32], 2, 0.02, 1.0), ([33, 33], 1, 0.0, 1.0),
                                          ([257], 2, 0.02, 0.0)])
def test_bwd_equal_lengths_bf16(lens, H, s0, ds):
    w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=H), lens, s0, ds)
    compare(w, a, S0, dO, dS, cu, TOL_BF16, f"bf16 lens={lens} H={H} s0={s0} dS={ds}",
            equal=(len(lens), lens[0]))


def test_bwd_varlen_bf16_edges():
    """Empty, one-token, exactly-one-chunk and chunk-plus-one sequences, packed."""
    w, a, S0, dO, dS, cu = inputs(W.workload(2).shrink(H=2), [0, 1, 31, 32, 33, 70, 0, 5],
                                  0.02, 1.0)
    compare(w, a, S0, dO, dS, cu, TOL_BF16, "bf16 varlen edges")


def test_bwd_workload0_fp32():
    """Single fp32 head, T=256, S0 = 0, no state gradient."""
    w, a, S0, dO, dS, cu = inputs(W.workload(0), [256], 0.0, 0.0)
    compare(w, a, S0, dO, dS, cu, TOL_F32, "fp32 T=256", equal=(1, 256))


@pytest.mark.parametrize("la", [-5.0, 0.0])
def test_bwd_decay_extremes(la):
    """log alpha = -5 everywhere (the fastest forgetting: 16 tokens span e^-80)
    and log alpha = 0 (no decay, DeltaNet)."""
    w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=2), [70, 45], 0.02, 1.0, la_const=la)
    compare(w, a, S0, dO, dS, cu, TOL_BF16, f"bf16 log_alpha={la}")


def test_bwd_full_size_sampled_heads():
    """The full prefill shape (T=8192, H=96, bf16) on the GPU; two heads
    followed by the oracle on their own."""
    w = W.workload(1)
    T, H = w.T, w.H
    say("[bwd] full size: inputs")
    dt = torch.bfloat16
    d = {n: torch.empty((1, T, H, 128), dtype=dt, device="cuda") for n in ("q", "k", "v")}
    d["log_alpha"] = torch.empty((1, T, H, 128), device="cuda")
    d["beta"] = torch.empty((1, T, H), device="cuda")
    go = torch.empty((1, T, H, 128), device="cuda")
    gst = torch.empty((1, H, 128, 128), device="cuda")
    for h in range(H):
        s = W.head_stream(w, h, T)
        for n in ("q", "k", "v", "log_alpha"):
            d[n][0, :, h] = torch.from_numpy(s[n]).cuda().to(d[n].dtype)
        d["beta"][0, :, h] = torch.from_numpy(s["beta"]).cuda()
        a, b = W.grad_head(w, h, T, 1)
        go[0, :, h] = torch.from_numpy(a).cuda()
        gst[:, h] = torch.from_numpy(b).cuda()
    say("[bwd] full size: GPU")
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, go, gst)
    torch.cuda.synchronize()
    for h in (0, 77):
        say(f"[bwd] full size: oracle head {h}")
        s = W.head_stream(w, h, T)
        a, b = W.grad_head(w, h, T, 1)
        ref = oracle.backward(s["q"][:, None], s["k"][:, None], s["v"][:, None],
                              s["log_alpha"][:, None], s["beta"][:, None], None, a[:, None],
                              b[:, None])
        errs = {}
        for i, n in enumerate(NAMES):
            x = g[i][0, :, h].cpu().numpy() if i < 5 else g[i][:, h].cpu().numpy()
            r = ref[i][:, 0] if i < 5 else ref[i][:, 0]
            errs[n] = rel_err(x, r)
        say(f"[bwd] full size head {h}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= TOL_BF16, (h, n, e)


def test_bwd_varlen_multichunk_with_state():
    """Packed sequences of several chunks each, S0 and dL/dS_T given."""
    w, a, S0, dO, dS, cu = inputs(W.workload(2).shrink(H=3), [200, 513, 64, 1000, 31], 0.02, 1.0)
    compare(w, a, S0, dO, dS, cu, TOL_BF16, "bf16 varlen multi-chunk")


def test_bwd_deterministic_and_in_place_state_gradient():
    """Two calls give bitwise equal gradients (no atomics anywhere), and
    grad_S0 written over grad_S_T equals the separate result."""
    w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=2), [150, 77], 0.02, 1.0)
    g1 = run(w, a, S0, dO, dS, cu)
    g2 = run(w, a, S0, dO, dS, cu)
    for x, y in zip(g1, g2):
        assert np.array_equal(x, y)
    d = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in a}
    for n in ("q", "k", "v"):
        d[n] = d[n].to(torch.bfloat16)
    gst = torch.from_numpy(dS).cuda()
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    lib = kda.load_library()
    T, H = a["q"].shape[0], a["q"].shape[1]
    outs = [torch.empty_like(d["log_alpha"]) for _ in range(4)] + [torch.empty_like(d["beta"])]
    ws = torch.empty(lib.kda_chunk_bwd_workspace_bytes(len(cu) - 1, T, H, 128, 128, 1),
                     dtype=torch.uint8, device="cuda")
    import ctypes
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.kda_chunk_bwd(vp(d["q"]), vp(d["k"]), vp(d["v"]), 0, vp(d["log_alpha"]), vp(d["beta"]),
                           vp(torch.from_numpy(S0).cuda()), vp(cu_dev), len(cu) - 1, T, H, 128, 128,
                           vp(torch.from_numpy(dO).cuda()), vp(gst), *[vp(o) for o in outs], vp(gst),
                           vp(ws), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    assert np.array_equal(gst.cpu().numpy(), g1[5])


def test_bwd_full_size_varlen_lengths_sampled():
    """The packed lengths of the varlen workload (32 sequences of 512-16384
    tokens, S0 ~ N(0, 0.02^2)) on 4 heads; the oracle follows two
    (sequence, head) units on their own."""
    w = W.workload(2).shrink(H=4)
    cu = W.cu_seqlens(w)
    T, N = int(cu[-1]), len(cu) - 1
    say(f"[bwd] varlen lengths T={T}: inputs")
    a = W.prefill_inputs(w)
    dO, dS = W.grad_inputs(w, T, N)
    d = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in ("q", "k", "v", "log_alpha", "beta")}
    for n in ("q", "k", "v"):
        d[n] = d[n].to(torch.bfloat16)
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    say("[bwd] varlen lengths: GPU")
    g = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                      torch.from_numpy(a["S0"]).cuda(), torch.from_numpy(dO).cuda(),
                      torch.from_numpy(dS).cuda(), cu_dev)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in g]
    del g, d
    for n, h in ((int(np.argmax(np.diff(cu))), 1), (5, 3)):
        say(f"[bwd] varlen lengths: oracle sequence {n} head {h}")
        ref = oracle.backward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["S0"], dO, dS, cu,
                              units=[(n, h)])
        rows = slice(int(cu[n]), int(cu[n + 1]))
        errs = {}
        for i, nm in enumerate(NAMES):
            x, r = (got[i][rows, h], ref[i][rows, h]) if i < 5 else (got[i][n, h], ref[i][n, h])
            errs[nm] = rel_err(x, r)
        say(f"[bwd] varlen sequence {n} head {h}: " + "  ".join(f"{k} {e:.2e}" for k, e in errs.items()))
        for nm, e in errs.items():
            assert e <= TOL_BF16, (n, h, nm, e)


# ------------------------------------------------ equal lengths in windows
@pytest.mark.parametrize("dtype,B,T,H", [("bf16", 3, 300, 3), ("f32", 2, 200, 2),
                                         ("bf16", 3, 200, 96), ("f32", 3, 150, 96)])
def test_bwd_windows_against_oracle(dtype, B, T, H):
    """Equal-length batches run window by window (the last window first, the
    state gradient carried between windows, the states at window starts from
    a forward pass without per-chunk outputs): 2-chunk and 4-chunk windows
    with a ragged last window, S0 and dL/dS_T given, every element of all
    six gradients against the oracle; the gradients equal those of the
    single-window layout bit for bit.  B=3, H=96 runs the one-slice kernels
    (288 pairs) in both dtypes."""
    base = W.workload(1 if dtype == "bf16" else 0).shrink(H=H)
    w, a, S0, dO, dS, cu = inputs(base, [T] * B, 0.02, 1.0)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    C = -(-T // 32)
    single = run(w, a, S0, dO, dS, cu, (B, T), window_tokens=T)
    for win in (64, 128):
        n_win = -(-C // (win // 32))
        got = compare(w, a, S0, dO, dS, cu, tol, f"{dtype} B={B} T={T} H={H} windows of {win} "
                      f"tokens ({n_win} windows)", equal=(B, T), window_tokens=win)
        for n, x, y in zip(NAMES, got, single):
            assert np.array_equal(x, y), (win, n, float(np.abs(x - y).max()))


def test_bwd_window_workspace_sizes():
    """The default workspace of the T=8192, H=96 shape is the 2048-token
    window layout (under 1.6 GB, a quarter of the single-window layout), and
    a workspace one byte short of it runs 1024-token windows with the same
    gradients."""
    n = kda.chunk_bwd_workspace_bytes
    default = n(1, 8192, 96)
    one = n(1, 8192, 96, window_tokens=8192)
    say(f"[bwd] workspace T=8192 H=96: default {default / 1e9:.3f} GB, one window {one / 1e9:.3f} GB")
    assert default == n(1, 8192, 96, window_tokens=2048) and default < 1.6e9 and one > 3.5 * default
    w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=2), [700], 0.02, 1.0)
    ws_small = torch.empty(n(1, 700, 2, window_tokens=128) - 1, dtype=torch.uint8, device="cuda")
    d = {k: torch.from_numpy(np.ascontiguousarray(a[k])).cuda()[None] for k in a}
    for k in ("q", "k", "v"):
        d[k] = d[k].to(torch.bfloat16)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], torch.from_numpy(S0).cuda(),
            torch.from_numpy(dO).cuda()[None], torch.from_numpy(dS).cuda())
    g_small = kda.chunk_bwd(*args, workspace=ws_small)      # 64-token windows
    g_one = kda.chunk_bwd(*args, window_tokens=700)
    torch.cuda.synchronize()
    for nm, x, y in zip(NAMES, g_small, g_one):
        assert torch.equal(x, y), nm


def test_bwd_graph_capture_replays_bitwise():
    """kda_chunk_bwd captured into a HIP graph replays to the eager result,
    bitwise, three times with eager work and synchronisations between the
    replays.  Its chunk-matrix passes fork onto the library's second stream
    and join back, so the capture covers that stream too: an equal-length
    batch in 64-token windows (five windows per sequence, five forks) and a
    packed batch (one fork)."""
    import ctypes
    lib = kda.load_library()
    vp = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    for equal in (True, False):
        lens = [300, 300] if equal else [300, 45, 0, 130]
        w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=3), lens, 0.02, 1.0)
        T, H, N = a["q"].shape[0], a["q"].shape[1], len(lens)
        d = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in a}
        for n in ("q", "k", "v"):
            d[n] = d[n].to(torch.bfloat16)
        s0 = torch.from_numpy(S0).cuda()
        go = torch.from_numpy(dO).cuda()
        gst = torch.from_numpy(dS).cuda()
        cu_dev = None if equal else torch.from_numpy(cu.astype(np.int32)).cuda()
        Tc = 300 if equal else T   # tokens per sequence (equal) or in total (packed)
        wsb = (lib.kda_chunk_bwd_workspace_bytes_window(N, Tc, H, 128, 128, 64) if equal
               else lib.kda_chunk_bwd_workspace_bytes(N, Tc, H, 128, 128, 1))
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        outs = [torch.empty_like(d["log_alpha"]) for _ in range(4)] + [torch.empty_like(d["beta"]),
                                                                       torch.empty_like(s0)]

        def call(stream_handle):
            return lib.kda_chunk_bwd(vp(d["q"]), vp(d["k"]), vp(d["v"]), 0, vp(d["log_alpha"]),
                                     vp(d["beta"]), vp(s0), vp(cu_dev), N, Tc, H, 128, 128, vp(go),
                                     vp(gst), *[vp(o) for o in outs], vp(ws), wsb,
                                     ctypes.c_void_p(stream_handle))

        say(f"[bwd] graph capture ({'equal lengths, 5 windows' if equal else 'packed'}): eager")
        assert call(torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        say("[bwd] graph capture: capture")
        with torch.cuda.graph(g, stream=s):
            rc = call(s.cuda_stream)
        assert rc == 0
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            ws.fill_(0xFF)
            torch.cuda.synchronize()
            say(f"[bwd] graph capture: replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            for o, r in zip(outs, ref):
                assert torch.equal(o, r)


def test_bwd_concurrent_calls_from_two_threads_bitwise():
    """Two host threads call kda_chunk_bwd at the same time on two streams
    with their own inputs, outputs and workspaces (the calls share the
    library's second stream and its events, and enqueue under one lock):
    every result equals the same call made alone, bitwise."""
    import ctypes
    import threading
    lib = kda.load_library()
    vp = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    jobs = []
    for seed_h, lens in ((3, [300, 300]), (2, [200, 200, 200])):
        w, a, S0, dO, dS, cu = inputs(W.workload(1).shrink(H=seed_h), lens, 0.02, 1.0)
        T, H, N = a["q"].shape[0], a["q"].shape[1], len(lens)
        d = {n: torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in a}
        for n in ("q", "k", "v"):
            d[n] = d[n].to(torch.bfloat16)
        job = dict(d=d, s0=torch.from_numpy(S0).cuda(), go=torch.from_numpy(dO).cuda(),
                   gst=torch.from_numpy(dS).cuda(), N=N, Tc=lens[0], H=H)
        job["wsb"] = lib.kda_chunk_bwd_workspace_bytes_window(N, lens[0], H, 128, 128, 64)
        job["ws"] = torch.empty(job["wsb"], dtype=torch.uint8, device="cuda")
        job["outs"] = [torch.empty_like(d["log_alpha"]) for _ in range(4)] + [
            torch.empty_like(d["beta"]), torch.empty_like(job["s0"])]
        job["stream"] = torch.cuda.Stream()
        jobs.append(job)

    def call(job):
        d = job["d"]
        return lib.kda_chunk_bwd(vp(d["q"]), vp(d["k"]), vp(d["v"]), 0, vp(d["log_alpha"]), vp(d["beta"]),
                                 vp(job["s0"]), None, job["N"], job["Tc"], job["H"], 128, 128, vp(job["go"]),
                                 vp(job["gst"]), *[vp(o) for o in job["outs"]], vp(job["ws"]), job["wsb"],
                                 ctypes.c_void_p(job["stream"].cuda_stream))

    say("[bwd] two threads: each call alone")
    ref = []
    for job in jobs:
        assert call(job) == 0
        torch.cuda.synchronize()
        ref.append([o.clone() for o in job["outs"]])
    for rep in range(3):
        for job in jobs:
            for o in job["outs"]:
                o.fill_(float("nan"))
        torch.cuda.synchronize()
        rcs = [None, None]

        def worker(i):
            rcs[i] = [call(jobs[i]) for _ in range(2)]

        say(f"[bwd] two threads: round {rep}")
        th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        torch.cuda.synchronize()
        assert rcs == [[0, 0], [0, 0]]
        for job, r in zip(jobs, ref):
            for o, x in zip(job["outs"], r):
                assert torch.equal(o, x)
