"""The seeded input generators (CPU only)."""
import numpy as np
import torch

from gated_delta_rule_amd import workloads as W


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3e38, -2.5e-38],
                                 np.float32)])
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_distributions_and_contract():
    w = W.workload(1).shrink(T=300, H=3)
    a = W.prefill_inputs(w)
    qn = np.linalg.norm(a["q"].astype(np.float64), axis=-1)
    assert np.allclose(qn, 1.0, atol=1e-2)              # unit norm up to bf16 rounding
    assert np.all(a["log_alpha"] < 0) and np.all(a["log_alpha"] > -5)
    assert np.all(a["beta"] > 0) and np.all(a["beta"] < 1)
    # log alpha = -5 sigmoid(N(0,1)): mean -2.5
    assert abs(a["log_alpha"].mean() + 2.5) < 0.05
    assert np.array_equal(W.round_bf16(a["v"]), a["v"])  # exactly bf16 values
    assert a["S0"] is None


def test_reproducible_and_per_head():
    w = W.workload(2).shrink(n_varlen=3, len_lo=20, len_hi=40, H=5)
    a = W.prefill_inputs(w)
    b = W.prefill_inputs(w, heads=[3, 1])
    for n in ("q", "k", "v", "log_alpha"):
        assert np.array_equal(a[n][:, 3], b[n][:, 0]) and np.array_equal(a[n][:, 1], b[n][:, 1])
    assert np.array_equal(a["S0"][:, 3], b["S0"][:, 0])
    c = W.prefill_inputs(w)
    assert all(np.array_equal(a[n], c[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0"))


def test_varlen_lengths():
    w = W.workload(2)
    cu = W.cu_seqlens(w)
    lens = np.diff(cu)
    assert len(lens) == 32 and lens.min() >= 512 and lens.max() <= 16384
    assert cu[0] == 0 and W.total_tokens(w) == cu[-1]


def test_decode_inputs_and_state():
    w = W.workload(4).shrink(B=5, H=3)
    s = W.decode_state(w)
    assert s.shape == (5, 3, 128, 128) and abs(s.std() - 0.02) < 0.002
    x0, x1 = W.decode_inputs(w, 0), W.decode_inputs(w, 1)
    assert x0["q"].shape == (5, 3, 128) and x0["beta"].shape == (5, 3)
    assert not np.array_equal(x0["q"], x1["q"])
