"""GPU parity of the layer prologue / epilogue (kda_prologue, kda_epilogue)
against the fp64 oracle (oracle/layer.py), and of the whole layer step
prologue -> kda_chunk_fwd -> epilogue against the oracle's composition."""
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
from oracle import layer as L  # noqa: E402


# bf16 outputs: round-to-nearest-even leaves at most half a unit in the last
# place, 2^-8 of the value (8 significant bits), plus the fp32 arithmetic
# before the rounding.
BF16_HALF_ULP = 2.0 ** -8


def bf16_err(x, ref):
    """Largest element error in units of the bound 2^-8 |ref| + 1e-5 max|ref|
    (<= 1 means every element is within correctly rounded bf16 of ref)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = BF16_HALF_ULP * np.abs(ref) + 1e-5 * np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref) / bound))


def layer_inputs(lens, H, dtype="bf16", seed=0, cache=True):
    """Packed inputs for sequences of the given lengths (see workloads.layer_inputs)."""
    return W.layer_inputs(lens, H, dtype=dtype, seed=seed, with_cache=cache)


def dev_layer(x, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(dt)
         for n in ("q_raw", "k_raw", "v_raw")}
    for n in ("conv_w", "a", "b", "g", "w_norm"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).cuda()
    d["cache"] = None if x["cache"] is None else torch.from_numpy(x["cache"].copy()).cuda()
    d["cu"] = torch.from_numpy(x["cu_seqlens"].astype(np.int32)).cuda()
    return d


def oracle_prologue(x):
    cu = x["cu_seqlens"]
    outs = {n: [] for n in ("q", "k", "v", "log_alpha", "beta")}
    caches = []
    for n in range(len(cu) - 1):
        s, e = cu[n], cu[n + 1]
        sl = {m: x[m][s:e] for m in ("q_raw", "k_raw", "v_raw", "a", "b")}
        q, k, v, la, be, c = L.prologue(sl["q_raw"], sl["k_raw"], sl["v_raw"], x["conv_w"],
                                        sl["a"], sl["b"],
                                        None if x["cache"] is None else x["cache"][n])
        for m, val in zip(("q", "k", "v", "log_alpha", "beta"), (q, k, v, la, be)):
            outs[m].append(val)
        caches.append(c)
    return {m: np.concatenate(v) for m, v in outs.items()}, np.stack(caches)


@pytest.mark.parametrize("lens,H,dtype", [([70, 70], 3, "bf16"), ([0, 1, 2, 5, 40, 3], 2, "bf16"),
                                          ([33, 9], 2, "f32")])
def test_prologue(lens, H, dtype):
    x = layer_inputs(lens, H, dtype)
    d = dev_layer(x, dtype)
    say(f"[layer] prologue lens={lens} H={H} {dtype}: GPU")
    q, k, v, la, be = kda.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_w"], d["a"],
                                   d["b"], d["cache"], d["cu"])
    torch.cuda.synchronize()
    ref, rc = oracle_prologue(x)
    if dtype == "f32":
        errs = {m: rel_err(t.cpu().numpy(), ref[m]) for m, t in (("q", q), ("k", k), ("v", v))}
    else:   # bf16 outputs: within correctly rounded bf16 of the fp64 values
        errs = {m: bf16_err(t.float().cpu().numpy(), ref[m]) for m, t in
                (("q", q), ("k", k), ("v", v))}
    errs["log_alpha"] = rel_err(la.cpu().numpy(), ref["log_alpha"])
    errs["beta"] = rel_err(be.cpu().numpy(), ref["beta"])
    say(f"[layer] prologue lens={lens}: " + "  ".join(f"{m} {e:.2e}" for m, e in errs.items()))
    for m in ("q", "k", "v"):
        assert errs[m] <= (TOL_F32 if dtype == "f32" else 1.0), (m, errs[m])
    assert errs["log_alpha"] <= TOL_F32 and errs["beta"] <= TOL_F32
    # the cache holds raw inputs: exact
    assert np.array_equal(d["cache"].cpu().numpy(), rc.astype(np.float32))


def test_prologue_equal_length_layout_and_no_cache():
    lens = [50, 50, 50]
    x = layer_inputs(lens, 2, cache=False)
    d = dev_layer(x, "bf16")
    shp = (3, 50, 2, 128)
    q, k, v, la, be = kda.prologue(d["q_raw"].view(shp), d["k_raw"].view(shp),
                                   d["v_raw"].view(shp), d["conv_w"], d["a"].view(shp),
                                   d["b"].view(3, 50, 2))
    torch.cuda.synchronize()
    ref, _ = oracle_prologue(x)
    assert bf16_err(q.float().cpu().numpy().reshape(ref["q"].shape), ref["q"]) <= 1.0
    assert bf16_err(v.float().cpu().numpy().reshape(ref["v"].shape), ref["v"]) <= 1.0
    assert rel_err(la.cpu().numpy().reshape(ref["log_alpha"].shape), ref["log_alpha"]) <= TOL_F32


def test_epilogue_and_in_place():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((37, 3, 128)).astype(np.float32) * 3
    g = rng.standard_normal((37, 3, 128)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    do, dg, dw = (torch.from_numpy(t).cuda() for t in (o, g, w))
    out = kda.epilogue(do, dg, dw)
    torch.cuda.synchronize()
    ref = L.epilogue(o, g, w)
    e = rel_err(out.cpu().numpy(), ref)
    say(f"[layer] epilogue rel err {e:.2e}")
    assert e <= TOL_F32
    kda.epilogue(do, dg, dw, out=do)
    torch.cuda.synchronize()
    assert torch.equal(do, out)


def test_layer_step_end_to_end():
    """prologue -> chunk_fwd (with S0) -> epilogue against the oracle's
    composition, packed sequences with conv caches."""
    lens = [100, 37, 64]
    H = 3
    x = layer_inputs(lens, H, seed=7)
    d = dev_layer(x, "bf16")
    rng = np.random.default_rng(8)
    S0 = (0.02 * rng.standard_normal((len(lens), H, 128, 128))).astype(np.float32)
    q, k, v, la, be = kda.prologue(d["q_raw"], d["k_raw"], d["v_raw"], d["conv_w"], d["a"],
                                   d["b"], d["cache"], d["cu"])
    o, st = kda.chunk_fwd(q, k, v, la, be, torch.from_numpy(S0).cuda(), d["cu"])
    out = kda.epilogue(o, d["g"], d["w_norm"])
    torch.cuda.synchronize()
    ref, _ = oracle_prologue(x)
    # the layer hands bf16 q, k, v to the recurrence: the oracle rounds its own
    # prologue outputs the same way
    qk = {m: W.round_bf16(ref[m].astype(np.float32)).astype(np.float64) for m in ("q", "k", "v")}
    ro, rs = oracle.forward(qk["q"], qk["k"], qk["v"], ref["log_alpha"], ref["beta"], S0,
                            x["cu_seqlens"])
    rout = L.epilogue(ro, x["g"], x["w_norm"])
    e1, e2 = rel_err(out.cpu().numpy(), rout), rel_err(st.cpu().numpy(), rs)
    say(f"[layer] end to end: out {e1:.2e}  S_T {e2:.2e}")
    assert e1 <= TOL_BF16 and e2 <= TOL_BF16


@pytest.mark.parametrize("T,B", [(1, 7), (3, 5), (9, 3)])
def test_prologue_equal_lengths_shorter_than_a_wave_block(T, B):
    """Equal-length batches whose sequences end inside one wave's block of
    rows (the position is counted on from the block's first row), with a
    cache."""
    lens = [T] * B
    x = layer_inputs(lens, 2, seed=11)
    d = dev_layer(x, "bf16")
    shp = (B, T, 2, 128)
    cache = d["cache"].clone()
    q, k, v, la, be = kda.prologue(d["q_raw"].view(shp), d["k_raw"].view(shp),
                                   d["v_raw"].view(shp), d["conv_w"], d["a"].view(shp),
                                   d["b"].view(B, T, 2), cache)
    torch.cuda.synchronize()
    ref, rc = oracle_prologue(x)
    for m, t in (("q", q), ("k", k), ("v", v)):
        assert bf16_err(t.float().cpu().numpy().reshape(ref[m].shape), ref[m]) <= 1.0, m
    assert rel_err(la.cpu().numpy().reshape(ref["log_alpha"].shape), ref["log_alpha"]) <= TOL_F32
    assert np.array_equal(cache.cpu().numpy(), rc.astype(np.float32))
