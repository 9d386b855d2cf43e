"""kda_chunk_fwd_noalloc (the prefill entry point that allocates nothing)
against kda_chunk_fwd with a caller-supplied workspace, through the C ABI.

The two paths that use a workspace are covered, each with two calls in a
row, the second on a smaller input (the scratch array keeps the previous
call's contents): the sequence-parallel path (segment transitions, local and
incoming states in the scratch array; once with 64 (sequence, head) pairs
in four segments, then with 8 pairs in three) and the packed batch (the
longest-first order in the scratch array).  Same kernels, so the outputs
must be bitwise equal; the first call of each pair is also checked against
the fp64 oracle on sampled heads."""
import ctypes

import numpy as np
import pytest

from gated_delta_rule_amd import workloads as W
from kda_testlib import TOL_BF16, oracle_head, rel_err, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU-only container
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_amd as kda  # noqa: E402


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(d, cu, n_seqs, T, H):
    lib = kda.load_library()
    o = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    st = torch.empty((n_seqs, H, 128, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.kda_chunk_fwd_noalloc(_p(d["q"]), _p(d["k"]), _p(d["v"]), kda.KDA_BF16,
                                   _p(d["log_alpha"]), _p(d["beta"]), _p(d["S0"]), _p(cu), n_seqs,
                                   T, H, 128, 128, _p(o), _p(st), ctypes.c_void_p(stream))
    assert rc == 0, lib.kda_status_str(rc).decode()
    return o, st


def equal_lengths(T, H, s0):
    w = W.workload(1).shrink(T=T, H=H, B=1, s0_std=s0)
    a = W.prefill_inputs(w)
    arrs = {n: a[n].reshape((1, T) + a[n].shape[1:]) for n in ("q", "k", "v", "log_alpha", "beta")}
    arrs["S0"] = a["S0"]
    return w, arrs


@pytest.mark.parametrize("first,second", [((8192, 64), (6144, 8))])
def test_noalloc_sequence_parallel_two_calls(first, second):
    for i, (T, H) in enumerate((first, second)):
        assert kda.chunk_fwd_workspace_bytes(1, T, H, varlen=False) > 0
        w, arrs = equal_lengths(T, H, 0.02)
        d = to_dev(arrs, w)
        say(f"[noalloc] sequence-parallel call {i + 1}: T={T} H={H}")
        o_ref, st_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
        o, st = noalloc(d, None, 1, T, H)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
        if i == 0:
            for h in (0, H - 1):
                ro, rs = oracle_head(w, h, W.cu_seqlens(w))
                eo = rel_err(o[0, :, h].cpu().numpy(), ro)
                es = rel_err(st[0, h].cpu().numpy(), rs[0])
                say(f"[noalloc]   head {h}: rel err o {eo:.3e} S_T {es:.3e}")
                assert eo <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_packed_batch_two_calls():
    for i, (lens, H) in enumerate((([300, 0, 17, 64, 33, 300, 5, 1, 90, 90, 12, 200], 4),
                                   ([40, 3, 0, 65, 7], 2))):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(cu[-1])
        w = W.workload(2).shrink(n_varlen=0, B=1, T=T, H=H, s0_std=0.0)
        a = W.prefill_inputs(w)
        rng = np.random.default_rng(i)
        arrs = {n: a[n] for n in ("q", "k", "v", "log_alpha", "beta")}
        arrs["S0"] = (0.02 * rng.standard_normal((len(lens), H, 128, 128))).astype(np.float32)
        d = to_dev(arrs, w)
        cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
        say(f"[noalloc] packed call {i + 1}: {len(lens)} sequences, H={H}")
        o_ref, st_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                      cu_d)
        o, st = noalloc(d, cu_d, len(lens), T, H)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, st_ref)
        if i == 0:
            import oracle
            ro, rs = oracle.forward(arrs["q"], arrs["k"], arrs["v"], arrs["log_alpha"],
                                    arrs["beta"], arrs["S0"], cu)
            eo, es = rel_err(o.cpu().numpy(), ro), rel_err(st.cpu().numpy(), rs)
            say(f"[noalloc]   rel err o {eo:.3e} S_T {es:.3e}")
            assert eo <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_validation_matches_chunk_fwd():
    """Invalid arguments give kda_chunk_fwd's status codes (nothing runs)."""
    lib = kda.load_library()
    vp = ctypes.c_void_p
    assert lib.kda_chunk_fwd_noalloc(None, None, None, 0, None, None, None, None, 1, 8, 4, 64, 128,
                                     None, None, None) == 2      # KDA_ERR_BAD_SHAPE
    assert lib.kda_chunk_fwd_noalloc(None, None, None, 5, None, None, None, None, 1, 8, 4, 128, 128,
                                     None, None, None) == 3      # KDA_ERR_BAD_DTYPE
    assert lib.kda_chunk_fwd_noalloc(vp(16), vp(16), vp(16), 0, vp(16), vp(16), None, None, 0, 8, 4,
                                     128, 128, vp(16), None, None) == 0   # empty batch
