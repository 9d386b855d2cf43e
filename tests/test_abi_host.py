"""The C-ABI library on the host: it loads, exports every symbol that
include/kda.h declares, and rejects invalid arguments with the documented
status codes before touching the GPU (no call here reaches a kernel launch).
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, SHAPE, DTYPE, ALIGN, ALIAS, WS, LARGE, HIPERR = range(9)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        from gated_delta_rule_amd import build
        build.build()
    return kda.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def header_status_codes():
    text = open(HEADER).read()
    return dict((m[0], int(m[1])) for m in re.findall(r"\b(KDA_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", text))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert names == sorted(["kda_abi_version", "kda_status_str", "kda_chunk_fwd_workspace_bytes",
                            "kda_chunk_fwd", "kda_decode_step", "kda_recurrent_fwd",
                            "kda_prologue", "kda_epilogue", "kda_chunk_bwd_workspace_bytes",
                            "kda_chunk_bwd", "kda_chunk_fwd_noalloc",
                            "kda_chunk_bwd_workspace_bytes_window"])
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define KDA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.kda_abi_version() == ver
    codes = header_status_codes()
    assert codes["KDA_OK"] == OK and codes["KDA_ERR_HIP"] == HIPERR
    for name, code in codes.items():
        s = lib.kda_status_str(code).decode()
        assert s.startswith(name)
    assert lib.kda_status_str(12345).decode() == "unknown kda_status"


def test_workspace_query(lib):
    ws = lib.kda_chunk_fwd_workspace_bytes
    assert ws(32, 270000, 96, 128, 128, 1) == 32 * 4
    assert ws(32, 270000, 96, 128, 128, 0) == 0
    assert ws(5000, 10 ** 6, 16, 128, 128, 1) == 0        # beyond the sorted-order limit
    assert ws(32, 1000, 96, 64, 128, 1) == 0              # invalid head size
    assert ws(-1, 1000, 96, 128, 128, 1) == 0
    # equal lengths, few (sequence, head) pairs, long T: sequence-parallel
    # path with P >= 3 segments; per (sequence, head) 3P - 4 state-sized
    # arrays (transition and local final state of the P - 2 middle segments,
    # incoming state of the P - 1 later ones, segment 0's final state)
    assert ws(1, 1 << 20, 16, 128, 128, 0) == (3 * 16 - 4) * 16 * 65536   # P = 256 / 16
    assert ws(2, 7000, 3, 128, 128, 0) == (3 * 3 - 4) * 2 * 3 * 65536   # P limited by T / 2048
    assert ws(1, 8192, 16, 128, 128, 0) == (3 * 4 - 4) * 16 * 65536      # P = 8192 / 2048
    assert ws(1, 1 << 22, 1, 128, 128, 0) == (3 * 256 - 4) * 65536      # the largest: P = 256
    assert ws(2, 6000, 3, 128, 128, 0) == 0                              # two segments: no gain
    assert ws(1, 4095, 16, 128, 128, 0) == 0                             # too short to split
    assert ws(1, 1 << 20, 65, 128, 128, 0) == 0                          # enough pairs already


# Fake, never-dereferenced device addresses for validation-only calls.
A = 0x7F0000000000
P = {n: A + i * 0x100000000 for i, n in enumerate(["q", "k", "v", "la", "b", "s0", "o", "st", "cu", "ws"])}


def chunk(lib, **kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], dtype=0, la=P["la"], b=P["b"], s0=None, cu=None,
             n=2, T=64, H=4, dk=128, dv=128, o=P["o"], st=P["st"], ws=None, wsb=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_chunk_fwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), a["dtype"], vp(a["la"]),
                             vp(a["b"]), vp(a["s0"]), vp(a["cu"]), a["n"], a["T"], a["H"], a["dk"],
                             a["dv"], vp(a["o"]), vp(a["st"]), vp(a["ws"]), a["wsb"], None)


def decode(lib, **kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], dtype=0, la=P["la"], b=P["b"], S=P["st"], B=8, H=4,
             dk=128, dv=128, o=P["o"])
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_decode_step(vp(a["q"]), vp(a["k"]), vp(a["v"]), a["dtype"], vp(a["la"]),
                               vp(a["b"]), vp(a["S"]), a["B"], a["H"], a["dk"], a["dv"],
                               vp(a["o"]), None)


def test_chunk_fwd_validation(lib):
    assert chunk(lib, dtype=7) == DTYPE
    assert chunk(lib, dk=64) == SHAPE
    assert chunk(lib, dv=256) == SHAPE
    assert chunk(lib, H=0) == SHAPE
    assert chunk(lib, T=-1) == SHAPE
    assert chunk(lib, n=-1) == SHAPE
    assert chunk(lib, q=None) == NULLP
    assert chunk(lib, o=None) == NULLP
    assert chunk(lib, b=None) == NULLP
    assert chunk(lib, k=P["k"] + 2) == ALIGN
    assert chunk(lib, s0=P["s0"] + 8) == ALIGN
    assert chunk(lib, o=P["q"] + 64) == ALIAS          # o inside q
    assert chunk(lib, st=P["v"]) == ALIAS              # S_T on top of v
    assert chunk(lib, s0=P["s0"], st=P["s0"] + 1024) == ALIAS   # partial S0/S_T overlap
    assert chunk(lib, cu=P["cu"], ws=None) == WS       # packed batch needs the order workspace
    assert chunk(lib, cu=P["cu"], ws=P["ws"], wsb=4) == WS
    assert chunk(lib, n=2 ** 31 - 1, T=2 ** 40) == LARGE
    # equal lengths with a sequence-parallel workspace: checked like any other
    seg = dict(n=1, T=8192, H=16, wsb=3 * 4 * 16 * 65536)
    assert chunk(lib, ws=P["ws"] + 4, **seg) == ALIGN
    assert chunk(lib, ws=P["o"] + 4096, **seg) == ALIAS
    assert chunk(lib, n=0) == OK                        # empty batch: nothing to do
    assert chunk(lib, n=3, T=0, q=None, k=None, v=None, la=None, b=None, o=None,
                 st=P["st"] + 2) == ALIGN               # state pointers still checked


def test_decode_validation(lib):
    assert decode(lib, dtype=2) == DTYPE
    assert decode(lib, dk=127) == SHAPE
    assert decode(lib, H=0) == SHAPE
    assert decode(lib, B=-3) == SHAPE
    assert decode(lib, S=None) == NULLP
    assert decode(lib, la=P["la"] + 4) == ALIGN
    assert decode(lib, o=P["S"] if "S" in P else P["st"]) == ALIAS
    assert decode(lib, S=P["k"]) == ALIAS
    assert decode(lib, B=0) == OK


def recurrent(lib, **kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], dtype=0, la=P["la"], b=P["b"], rq=None, rk=None,
             rv=None, rla=None, rb=None, nr=None, S=P["st"], B=8, T=4, Tr=0, H=4, dk=128, dv=128,
             commit=1, o=P["o"])
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_recurrent_fwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), a["dtype"], vp(a["la"]),
                                 vp(a["b"]), vp(a["rq"]), vp(a["rk"]), vp(a["rv"]), vp(a["rla"]),
                                 vp(a["rb"]), vp(a["nr"]), vp(a["S"]), a["B"], a["T"], a["Tr"],
                                 a["H"], a["dk"], a["dv"], a["commit"], vp(a["o"]), None)


def test_recurrent_validation(lib):
    assert recurrent(lib, dtype=3) == DTYPE
    assert recurrent(lib, T=65) == SHAPE                 # at most 64 tokens per request
    assert recurrent(lib, Tr=65) == SHAPE
    assert recurrent(lib, T=-1) == SHAPE
    assert recurrent(lib, dv=64) == SHAPE
    assert recurrent(lib, S=None) == NULLP
    assert recurrent(lib, o=None) == NULLP
    assert recurrent(lib, Tr=3) == NULLP                 # replay tokens without their tensors
    rep = dict(Tr=3, rq=P["cu"], rk=P["cu"] + 2 ** 26, rv=P["cu"] + 2 ** 27, rla=P["ws"],
               rb=P["ws"] + 2 ** 27)
    assert recurrent(lib, nr=P["s0"] + 2, **rep) == ALIGN
    assert recurrent(lib, rq=P["cu"] + 8, **{k: v for k, v in rep.items() if k != "rq"}) == ALIGN
    assert recurrent(lib, o=P["cu"], **rep) == ALIAS     # o on top of the replay q
    assert recurrent(lib, S=P["k"]) == ALIAS
    assert recurrent(lib, B=0) == OK
    assert recurrent(lib, T=0, o=None, q=None, k=None, v=None, la=None, b=None,
                     S=P["st"] + 8) == ALIGN             # state still checked with no tokens


def prologue(lib, **kw):
    a = dict(qr=P["q"], kr=P["k"], vr=P["v"], dtype=0, w=P["ws"], cache=None, a=P["la"], b=P["b"],
             cu=None, n=2, T=64, H=4, dk=128, q=P["o"], k=P["o"] + 2 ** 24, v=P["o"] + 2 ** 25,
             la=P["st"], beta=P["st"] + 2 ** 25)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_prologue(vp(a["qr"]), vp(a["kr"]), vp(a["vr"]), a["dtype"], vp(a["w"]),
                            vp(a["cache"]), vp(a["a"]), vp(a["b"]), vp(a["cu"]), a["n"], a["T"],
                            a["H"], a["dk"], vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["la"]),
                            vp(a["beta"]), None)


def epilogue(lib, **kw):
    a = dict(o=P["o"], g=P["q"], w=P["b"], rows=64, H=4, dv=128, out=P["st"])
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_epilogue(vp(a["o"]), vp(a["g"]), vp(a["w"]), a["rows"], a["H"], a["dv"],
                            vp(a["out"]), None)


def test_layer_validation(lib):
    assert prologue(lib, dtype=5) == DTYPE
    assert prologue(lib, dk=64) == SHAPE
    assert prologue(lib, H=0) == SHAPE
    assert prologue(lib, w=None) == NULLP
    assert prologue(lib, beta=None) == NULLP
    assert prologue(lib, a=P["la"] + 4) == ALIGN
    assert prologue(lib, cache=P["s0"] + 4) == ALIGN
    assert prologue(lib, q=P["q"]) == ALIAS               # in place is refused
    assert prologue(lib, v=P["o"] + 2 ** 24) == ALIAS      # two outputs overlap
    assert prologue(lib, cache=P["la"]) == ALIAS
    assert prologue(lib, n=0) == OK
    assert epilogue(lib, dv=64) == SHAPE
    assert epilogue(lib, rows=-1) == SHAPE
    assert epilogue(lib, g=None) == NULLP
    assert epilogue(lib, out=P["st"] + 8) == ALIGN
    assert epilogue(lib, out=P["q"]) == ALIAS              # out on top of g
    assert epilogue(lib, out=P["o"] + 512) == ALIAS        # partial overlap with o
    assert epilogue(lib, rows=0) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(kda.KDAError):
        kda.load_library()


def test_bwd_workspace_query(lib):
    ws = lib.kda_chunk_bwd_workspace_bytes
    wsw = lib.kda_chunk_bwd_workspace_bytes_window
    per_slot = 2 * 128 * 128 + 3 * 32 * 32 + 3 * 128 * 32 + 128     # floats per chunk and head
    state = 128 * 128

    # packed: slots = tokens / 32 + n_seqs; per slot and head 2 states and
    # the chunk matrices, plus three fp32 rows per token and head
    def packed(tokens, n, H):
        slots = tokens // 32 + n
        return (slots * H * per_slot + 3 * tokens * H * 128) * 4

    # equal lengths, windows of W chunks: one window of every sequence, the
    # states at the starts of windows 1.., one carried gradient per unit
    def windowed(n, T, H, W):
        C = -(-T // 32)
        W = max(1, min(W, C))
        K = max(1, -(-C // W))
        extra = (K - 1) * n * H * state + (n * H * state if K > 1 else 0)
        return (n * W * H * per_slot + 3 * n * 32 * W * H * 128 + extra) * 4

    assert ws(1, 8192, 96, 128, 128, 0) == windowed(1, 8192, 96, 64)      # 2048-token windows
    assert ws(1, 8192, 96, 128, 128, 0) < 1.6e9                          # < 1.6 GB
    assert ws(3, 100, 2, 128, 128, 0) == windowed(3, 100, 2, 64)         # one window
    assert ws(32, 270000, 96, 128, 128, 1) == packed(270000, 32, 96)
    assert wsw(1, 8192, 96, 128, 128, 8192) == windowed(1, 8192, 96, 256)
    assert wsw(1, 8192, 96, 128, 128, 3000) == windowed(1, 8192, 96, 128)   # 94 chunks -> 128
    assert wsw(3, 300, 96, 128, 128, 64) == windowed(3, 300, 96, 2)
    assert wsw(3, 300, 96, 128, 128, 1) == windowed(3, 300, 96, 1)
    assert wsw(2, 0, 4, 128, 128, 2048) == windowed(2, 0, 4, 1)
    assert wsw(1, 1 << 31, 1, 128, 128, 32) == 0          # 2^26 windows: refused
    assert wsw(1, 1 << 31, 1, 128, 128, 1 << 16) > 0      # 2^15 windows
    assert wsw(2, 64, 4, 128, 128, 0) == 0
    assert ws(2, 64, 4, 64, 128, 0) == 0
    assert ws(-1, 64, 4, 128, 128, 0) == 0


def bwd(lib, **kw):
    G = {n: A + (16 + i) * 0x100000000 for i, n in enumerate(["go", "gst", "gq", "gk", "gv", "gla",
                                                              "gb", "gs0"])}
    a = dict(q=P["q"], k=P["k"], v=P["v"], dtype=0, la=P["la"], b=P["b"], s0=None, cu=None,
             n=2, T=64, H=4, dk=128, dv=128, go=G["go"], gst=None, gq=G["gq"], gk=G["gk"],
             gv=G["gv"], gla=G["gla"], gb=G["gb"], gs0=G["gs0"], ws=P["ws"], wsb=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.kda_chunk_bwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), a["dtype"], vp(a["la"]),
                             vp(a["b"]), vp(a["s0"]), vp(a["cu"]), a["n"], a["T"], a["H"], a["dk"],
                             a["dv"], vp(a["go"]), vp(a["gst"]), vp(a["gq"]), vp(a["gk"]),
                             vp(a["gv"]), vp(a["gla"]), vp(a["gb"]), vp(a["gs0"]), vp(a["ws"]),
                             a["wsb"], None)


def test_chunk_bwd_validation(lib):
    """Only error paths (they return before anything is enqueued)."""
    assert bwd(lib, dtype=9) == DTYPE
    assert bwd(lib, dk=64) == SHAPE
    assert bwd(lib, H=0) == SHAPE
    assert bwd(lib, T=-5) == SHAPE
    assert bwd(lib, go=None) == NULLP
    assert bwd(lib, gb=None) == NULLP
    assert bwd(lib, ws=None) == WS
    assert bwd(lib, wsb=1000) == WS
    assert bwd(lib, gq=P["q"] + 16) == ALIAS            # gradient on top of an input
    assert bwd(lib, gk=P["ws"] + 4096) == ALIAS         # gradient inside the workspace
    assert bwd(lib, gs0=P["st"], gst=P["st"] + 4096) == ALIAS
    assert bwd(lib, gla=P["la"] + 8) == ALIGN
    assert bwd(lib, ws=P["ws"] + 4) == ALIGN
    assert bwd(lib, n=2 ** 31 - 1, T=2 ** 40) == LARGE
    assert bwd(lib, n=0) == OK


def test_head_count_upper_bound(lib):
    """The kernels address a chunk's token rows with 32-bit byte offsets, so
    H above KDA_MAX_HEADS is refused with KDA_ERR_TOO_LARGE by every entry
    point (and the workspace queries report 0) before anything is enqueued."""
    hmax = int(re.search(r"#define KDA_MAX_HEADS (\d+)", open(HEADER).read()).group(1))
    assert hmax == 65536 and 32 * hmax * 128 * 4 <= 2 ** 31
    big = hmax + 1
    assert chunk(lib, H=big, n=1, T=1) == LARGE
    assert chunk(lib, H=big, n=1, T=1, cu=P["cu"], ws=P["ws"], wsb=4) == LARGE
    assert decode(lib, H=big, B=1) == LARGE
    assert recurrent(lib, H=big, B=1) == LARGE
    assert prologue(lib, H=big, n=1, T=1) == LARGE
    assert epilogue(lib, H=big, rows=1) == LARGE
    assert bwd(lib, H=big, n=1, T=1) == LARGE
    assert lib.kda_chunk_fwd_workspace_bytes(1, 1, big, 128, 128, 1) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(1, 1, big, 128, 128, 0) == 0
    # the bound itself is accepted (validation continues to later checks)
    assert chunk(lib, H=hmax, n=1, T=1, q=None) == NULLP
    assert lib.kda_chunk_fwd_workspace_bytes(1, 1, hmax, 128, 128, 1) == 4
